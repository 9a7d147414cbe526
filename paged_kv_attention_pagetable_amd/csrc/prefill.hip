// Packed varlen prefill attention over the paged cache, bf16 MFMA for gfx950.
//
// Work item = (kv head, sequence, block of query tokens).  The G query heads
// of the kv head are packed with the block's tokens into the MFMA column
// dimension (column = token * G + head), so each K/V tile serves all of them.
// A workgroup is 4 wave64s, each owning NT 16-column tiles.  Keys advance in
// 32-key chunks; each chunk's K rows and V^T rows are gathered from their
// physical pages into LDS (16-byte loads), then every wave computes
//
//   S^T[32 keys][16 cols] = K[32][D] . Q^T[D][16]         per column tile
//   O^T[D][16 cols]      += V^T[D][32] . P^T[32][16]
//
// with the same operand layout as the decode kernel (a lane's 8 key scores
// are directly its P^T k-slots).  Chunks entirely above a wave's causal
// diagonal, or entirely left of its sliding window, are skipped without any
// MFMA work; chunks entirely visible skip the per-element mask.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kPrefillWaves = 4;
constexpr int kChunk = 32;

template <int D>
constexpr int prefill_nt() { return D <= 128 ? 2 : 1; }

template <int D>
constexpr int k_row_stride() { return D + 8; }       // bf16 elements, +16 B pad
constexpr int kVRowStride = kChunk + 8;               // bf16 elements, +16 B pad

template <int D, int NT>
__global__ __launch_bounds__(kPrefillWaves * 64) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  bf16_t* sK = lds;                                   // [32][D+8]
  bf16_t* sV = lds + kChunk * k_row_stride<D>();      // [D][40]
  const int hk = blockIdx.x, n = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qc = lane & 15, quad = lane >> 4;
  const int G = a.G, QT = a.q_tokens;
  const int ps = a.g.page_size, log2ps = a.g.log2ps, n_pages = a.g.n_pages;
  const int a0 = a.cu_seqlens[n];
  const int len = a.cu_seqlens[n + 1] - a0;
  const int sp = a.start_pos ? a.start_pos[n] : 0;
  const int slot = a.slots[n];
  const bool idle = slot <= 0 || slot >= a.pt.max_slots || sp < 0;
  const int nblk = (len + QT - 1) / QT;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)a.g.n_kv * blk;
  const bf16_t* kbase = a.kpool + hk * blk;
  const bf16_t* vbase = a.vpool + hk * blk;
  const int32_t* trow = a.pt.table + (size_t)(idle ? 0 : slot) * a.pt.pps;
  const int cap = a.pt.pps * ps;

  for (int qb = a.n_qblocks - 1 - (int)blockIdx.z; qb < nblk; qb += a.n_qblocks) {
    const int i0 = qb * QT;
    const int nq = min(QT, len - i0);
    // ---- columns of this wave: col = (w*NT + nt)*16 + qc -> token col/G, head col%G
    int pcol[NT];
    u32x4 qreg[NT][D / 32];
    int first_col = w * NT * 16;
    int wave_lo = 0x7fffffff, wave_hi = -1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = first_col + nt * 16 + qc;
      const int i = col / G, g = col - i * G;
      const bool valid = i < nq && !idle;
      pcol[nt] = valid ? sp + i0 + i : -1;
      const bf16_t* qrow = a.q + ((size_t)(a0 + i0 + (valid ? i : 0)) * a.n_q + hk * G + g) * D +
                           8 * quad;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 v = load16(qrow + 32 * c);
        qreg[nt][c] = valid ? v : u32x4{0, 0, 0, 0};
      }
    }
    {
      const int i_lo = first_col / G;
      const int i_hi = min(nq - 1, (first_col + NT * 16 - 1) / G);
      if (!idle && i_lo < nq) {
        wave_lo = sp + i0 + i_lo;
        wave_hi = sp + i0 + i_hi;
      }
    }
    float m_run[NT], l_run[NT];
    f32x4 acc[NT][D / 16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = -INFINITY;
      l_run[nt] = 0.f;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[nt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // ---- key range of the workgroup
    int kv_hi = idle ? 0 : min(sp + i0 + nq, cap);
    int kv_lo = (a.window > 0) ? max(0, sp + i0 - a.window + 1) : 0;
    const int j_start = kv_lo & ~(kChunk - 1);

    for (int j0 = j_start; j0 < kv_hi; j0 += kChunk) {
      __syncthreads();  // the previous chunk's tiles are consumed
      // K tile: 32 rows x D/8 chunks of 16 bytes
      for (int i = tid; i < kChunk * (D / 8); i += kPrefillWaves * 64) {
        const int r = i / (D / 8), c8 = i - r * (D / 8);
        const int j = j0 + r;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (j < kv_hi) {
          const int page = trow[j >> log2ps];
          if (page >= 1 && page < n_pages)
            v = load16(kbase + (size_t)page * page_stride + (size_t)(j & (ps - 1)) * D + 8 * c8);
        }
        store16(sK + r * k_row_stride<D>() + 8 * c8, v);
      }
      // V^T tile: D rows x 4 groups of 8 keys
      for (int i = tid; i < D * (kChunk / 8); i += kPrefillWaves * 64) {
        const int d = i >> 2, tg = i & 3;
        const int j = j0 + 8 * tg;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (j < kv_hi) {
          const int page = trow[j >> log2ps];
          if (page >= 1 && page < n_pages) {
            v = load16(vbase + (size_t)page * page_stride + (size_t)d * ps + (j & (ps - 1)));
            const int nv = kv_hi - j;
            if (nv < 8) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t m = (2 * e < nv ? 0x0000ffffu : 0u) | (2 * e + 1 < nv ? 0xffff0000u : 0u);
                v[e] &= m;
              }
            }
          }
        }
        store16(sV + d * kVRowStride + 8 * tg, v);
      }
      __syncthreads();

      // ---- classification for this wave
      if (wave_hi < 0 || j0 > wave_hi) continue;                                   // above diagonal
      if (a.window > 0 && j0 + kChunk - 1 <= wave_lo - a.window) continue;          // left of window
      const bool full = (j0 + kChunk - 1 <= wave_lo) &&
                        (a.window <= 0 || wave_hi - j0 < a.window);

      // ---- S^T = K Q^T
      f32x4 S[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[nt][0] = S[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int r = 8 * (qc >> 2) + 4 * rg + (qc & 3);
        const bf16_t* kr = sK + r * k_row_stride<D>() + 8 * quad;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const u32x4 kv = load16(kr + 32 * c);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) S[nt][rg] = mfma16x16x32(kv, qreg[nt][c], S[nt][rg]);
        }
      }
      // ---- online softmax per column tile
      u32x4 pb[NT];
      float alpha[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float sc[8];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = j0 + 8 * quad + jj;
          const float v = (jj < 4 ? S[nt][0][jj] : S[nt][1][jj - 4]) * a.scale_log2;
          bool vis = true;
          if (!full) {
            const int pc = pcol[nt];
            vis = j <= pc && (a.window <= 0 || pc - j < a.window);
          }
          sc[jj] = vis ? v : -INFINITY;
          mx = fmaxf(mx, sc[jj]);
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[nt], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        alpha[nt] = fast_exp2(m_run[nt] - m_use);
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          p[jj] = fast_exp2(sc[jj] - m_use);
          psum += p[jj];
        }
        l_run[nt] = l_run[nt] * alpha[nt] + psum;
        m_run[nt] = m_new;
        pb[nt] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                       pack_bf16x2(p[6], p[7])};
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const u32x4 vv = load16(sV + (16 * dt + qc) * kVRowStride + 8 * quad);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt][dt] = acc[nt][dt] * alpha[nt];
          acc[nt][dt] = mfma16x16x32(vv, pb[nt], acc[nt][dt]);
        }
      }
    }

    // ---- normalise and store
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float l = l_run[nt];
      l += shfl_xor(l, 16);
      l += shfl_xor(l, 32);
      const int col = first_col + nt * 16 + qc;
      const int i = col / G, g = col - i * G;
      if (i >= nq) continue;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      bf16_t* orow = a.out + ((size_t)(a0 + i0 + i) * a.n_q + hk * G + g) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const f32x4 o = acc[nt][dt];
        uint2 pk;
        pk.x = pack_bf16x2(o[0] * inv, o[1] * inv);
        pk.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * quad) = pk;
      }
      if (a.lse && quad == 0)
        a.lse[(size_t)(a0 + i0 + i) * a.n_q + hk * G + g] =
            l > 0.f ? (m_run[nt] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t st) {
  constexpr int NT = prefill_nt<D>();
  const size_t lds = ((size_t)kChunk * k_row_stride<D>() + (size_t)D * kVRowStride) * sizeof(bf16_t);
  dim3 grid(a.g.n_kv, a.n_seqs, a.n_qblocks);
  hipLaunchKernelGGL((prefill_kernel<D, NT>), grid, dim3(kPrefillWaves * 64), lds, st, a);
  return hipGetLastError();
}

}  // namespace

int prefill_q_tokens(int G, int head_dim) {
  const int nt = head_dim <= 128 ? 2 : 1;
  return (kPrefillWaves * nt * 16) / G;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.head_dim) {
    case 64: return launch_prefill_d<64>(a, st);
    case 128: return launch_prefill_d<128>(a, st);
    case 256: return launch_prefill_d<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
