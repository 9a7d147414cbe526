// Packed varlen prefill attention over the paged cache, bf16 MFMA for gfx950.
//
// Work item = (kv head, sequence, block of query tokens).  The G query heads
// of the kv head are packed with the block's tokens into the MFMA column
// dimension (column = token * G + head), so each K/V tile serves all of them.
// A workgroup is 4 wave64s, each owning NT 16-column tiles.  Keys advance in
// 64-key chunks.  Each chunk's K rows and V^T rows are gathered from their
// physical pages (page ids staged in LDS once per workgroup) with 16-byte
// loads; the next chunk's loads are in flight in registers while the current
// chunk is computed from a double-buffered LDS tile, with one barrier per
// chunk.  Per 32-key half and column tile every wave computes
//
//   S^T[32 keys][16 cols] = K[32][D] . Q^T[D][16]
//   O^T[D][16 cols]      += V^T[D][32] . P^T[32][16]
//
// with the same operand layout as the decode kernel (a lane's 8 key scores
// are directly its P^T k-slots); the online softmax max/sum is updated once
// per 64 keys.  Chunks entirely above a wave's causal diagonal, or entirely
// left of its sliding window, are skipped without MFMA work; chunks entirely
// visible skip the per-element mask.  Query blocks are issued longest-first,
// and the workgroups of one (sequence, kv head) share an XCD L2 when the kv
// head count is a multiple of 8 (grid x = kv head).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 64;         // keys per pipeline step
constexpr int kStagePages = 4096;  // page ids staged in LDS (>= pages_per_slot, host-checked)

template <int D>
constexpr int prefill_nt() { return D <= 128 ? 2 : 1; }

template <int D>
constexpr int k_row() { return D + 8; }         // bf16 elements per LDS K row (+16 B pad)
constexpr int kVRow = kChunk + 8;               // bf16 elements per LDS V^T row (+16 B pad)
template <int D>
constexpr int tile_elems() { return kChunk * k_row<D>() + D * kVRow; }
template <int D>
constexpr int pieces() { return D / 32; }       // 16-byte pieces per thread per tile (K and V each)

template <int D, int NT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  __shared__ int s_pg[kStagePages];
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
    const int first_col = w * NT * 16;
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
    int wave_lo = 0x7fffffff, wave_hi = -1;
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
    const int kv_hi = idle ? 0 : min(sp + i0 + nq, cap);
    const int kv_lo = (a.window > 0) ? max(0, sp + i0 - a.window + 1) : 0;
    const int j_start = kv_lo & ~(kChunk - 1);
    const int n_chunks = kv_hi > j_start ? (kv_hi - j_start + kChunk - 1) / kChunk : 0;
    const int pg0 = j_start >> log2ps;
    const int n_pg = n_chunks ? ((kv_hi - 1) >> log2ps) - pg0 + 1 : 0;

    __syncthreads();  // previous block's tiles and page ids are consumed
    for (int i = tid; i < n_pg; i += kThreads) {
      const int pg = trow[pg0 + i];
      s_pg[i] = (pg >= 1 && pg < n_pages) ? pg : -1;
    }
    __syncthreads();
    // ---- per-thread prefetch of one chunk: K and V^T pieces.  Nothing here
    // reads the loaded registers, so the loads stay in flight during the math.
    u32x4 pk[pieces<D>()], pv[pieces<D>()];
    auto fetch = [&](int j0) {
      const bool tail = j0 + kChunk > kv_hi;  // uniform: only the last chunk is partial
#pragma unroll
      for (int p = 0; p < pieces<D>(); ++p) {
        const int i = tid + kThreads * p;
        const int r = i / (D / 8), c8 = i - r * (D / 8);
        const int j = j0 + r;
        const int page = (!tail || j < kv_hi) ? s_pg[(j >> log2ps) - pg0] : -1;
        pk[p] = page >= 0 ? load16(kbase + (size_t)page * page_stride + (size_t)(j & (ps - 1)) * D + 8 * c8)
                          : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int p = 0; p < pieces<D>(); ++p) {
        const int i = tid + kThreads * p;
        const int d = i >> 3, tg = i & 7;
        const int j = j0 + 8 * tg;
        const int page = (!tail || j < kv_hi) ? s_pg[(j >> log2ps) - pg0] : -1;
        pv[p] = page >= 0 ? load16(vbase + (size_t)page * page_stride + (size_t)d * ps + (j & (ps - 1)))
                          : u32x4{0, 0, 0, 0};
      }
    };
    // Writes the prefetched chunk at j0 to LDS buffer buf; V^T elements of keys
    // at or beyond kv_hi are zeroed here (stale page rows may hold anything,
    // and 0 * NaN would poison the P.V sum).
    auto stash = [&](int buf, int j0) {
      bf16_t* sK = lds + buf * tile_elems<D>();
      bf16_t* sV = sK + kChunk * k_row<D>();
#pragma unroll
      for (int p = 0; p < pieces<D>(); ++p) {
        const int i = tid + kThreads * p;
        const int r = i / (D / 8), c8 = i - r * (D / 8);
        store16(sK + r * k_row<D>() + 8 * c8, pk[p]);
      }
      const bool tail = j0 + kChunk > kv_hi;
#pragma unroll
      for (int p = 0; p < pieces<D>(); ++p) {
        const int i = tid + kThreads * p;
        const int d = i >> 3, tg = i & 7;
        u32x4 v = pv[p];
        if (tail) {
          const int nv = kv_hi - (j0 + 8 * tg);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t m = (2 * e < nv ? 0x0000ffffu : 0u) | (2 * e + 1 < nv ? 0xffff0000u : 0u);
            v[e] &= m;
          }
        }
        store16(sV + d * kVRow + 8 * tg, v);
      }
    };

    if (n_chunks > 0) {
      fetch(j_start);
      stash(0, j_start);
    }
    __syncthreads();
    for (int ck = 0; ck < n_chunks; ++ck) {
      const int j0 = j_start + ck * kChunk;
      if (ck + 1 < n_chunks) fetch(j0 + kChunk);  // in flight during this chunk's math
      const bf16_t* sK = lds + (ck & 1) * tile_elems<D>();
      const bf16_t* sV = sK + kChunk * k_row<D>();
      const bool skip = wave_hi < 0 || j0 > wave_hi ||
                        (a.window > 0 && j0 + kChunk - 1 <= wave_lo - a.window);
      if (!skip) {
        const bool full = (j0 + kChunk - 1 <= wave_lo) && (a.window <= 0 || wave_hi - j0 < a.window);
        // ---- S^T = K Q^T: half h, MFMA rg rows m hold keys 32h + 8*(m/4) + 4*rg + m%4
        f32x4 S[NT][2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rg = 0; rg < 2; ++rg) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[nt][h][rg] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = 32 * h + 8 * (qc >> 2) + 4 * rg + (qc & 3);
            const bf16_t* kr = sK + r * k_row<D>() + 8 * quad;
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
              const u32x4 kv = load16(kr + 32 * c);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) S[nt][h][rg] = mfma16x16x32(kv, qreg[nt][c], S[nt][h][rg]);
            }
          }
        // ---- scores in log2 units; lane holds keys j0 + 32h + 8*quad + jj
        float sc[NT][2][8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
              sc[nt][h][jj] = (jj < 4 ? S[nt][h][0][jj] : S[nt][h][1][jj - 4]) * a.scale_log2;
        if (!full) {  // wave-uniform: only chunks crossing the diagonal or the window edge
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int pc = pcol[nt];
            const int jmin = a.window > 0 ? pc - a.window + 1 : -0x7fffffff;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const int j = j0 + 32 * h + 8 * quad + jj;
                if (j > pc || j < jmin) sc[nt][h][jj] = -INFINITY;
              }
          }
        }
        // ---- online softmax over the 64 keys, per column tile
        u32x4 pb[NT][2];
        float alpha[NT];
        bool rescale = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float mx = -INFINITY;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) mx = fmaxf(mx, sc[nt][h][jj]);
          mx = fmaxf(mx, shfl_xor(mx, 16));
          mx = fmaxf(mx, shfl_xor(mx, 32));
          const float m_new = fmaxf(m_run[nt], mx);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          alpha[nt] = fast_exp2(m_run[nt] - m_use);
          rescale |= m_new != m_run[nt];
          float psum = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float p[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              p[jj] = fast_exp2(sc[nt][h][jj] - m_use);
              psum += p[jj];
            }
            pb[nt][h] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                              pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
          }
          l_run[nt] = l_run[nt] * alpha[nt] + psum;
          m_run[nt] = m_new;
        }
        // The O accumulators only need rescaling when some column's max moved
        // (alpha is exactly 1 otherwise); that is rare after the first chunks.
        if (__any(rescale)) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) acc[nt][dt] *= alpha[nt];
        }
        // ---- O^T += V^T P^T over both halves
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const u32x4 v0 = load16(sV + (16 * dt + qc) * kVRow + 8 * quad);
          const u32x4 v1 = load16(sV + (16 * dt + qc) * kVRow + 32 + 8 * quad);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[nt][dt] = mfma16x16x32(v1, pb[nt][1], mfma16x16x32(v0, pb[nt][0], acc[nt][dt]));
        }
      }
      if (ck + 1 < n_chunks) stash((ck + 1) & 1, j0 + kChunk);
      __syncthreads();
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
        uint2 pk2;
        pk2.x = pack_bf16x2(o[0] * inv, o[1] * inv);
        pk2.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * quad) = pk2;
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
  const size_t lds = 2 * (size_t)tile_elems<D>() * sizeof(bf16_t);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prefill_kernel<D, NT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  dim3 grid(a.g.n_kv, a.n_seqs, a.n_qblocks);
  hipLaunchKernelGGL((prefill_kernel<D, NT>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace

int prefill_q_tokens(int G, int head_dim) {
  const int nt = head_dim <= 128 ? 2 : 1;
  return (kWaves * nt * 16) / G;
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
