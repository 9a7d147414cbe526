// Packed varlen prefill attention over the paged cache, bf16 MFMA for gfx950.
//
// Work item = (kv head, sequence, block of query tokens).  The G query heads
// of the kv head are packed with the block's tokens into the MFMA column
// dimension (column = token * G + head), so each K/V tile serves all of them.
// A workgroup is 4 wave64s, each owning NT 16-column tiles (32 query columns
// per wave at head_dim <= 128).  Registers are capped so that two waves run
// per SIMD (two workgroups per CU): one wave's softmax overlaps the other's
// MFMAs.  (64 columns per wave halve the LDS operand traffic but need ~350
// registers, one wave per SIMD, and then the softmax serialises with the
// MFMAs -- measured slower.)
//
// Keys advance in 64-key chunks.  Each chunk's K rows and V^T rows are copied
// from their physical pages straight into LDS with gfx950's global-to-LDS
// loads (16 bytes per lane, no staging registers); the next chunk's copies are
// in flight while the current chunk is computed from the other LDS buffer,
// with one wait + barrier per chunk.  Tiles are XOR-swizzled in 16-byte units
// so that the MFMA operand reads of 16 rows hit 16 distinct bank groups.
// Page ids of the workgroup's key range are staged in LDS once.
//
// Per 32-key half and column tile every wave computes
//
//   S^T[32 keys][16 cols] = K[32][D] . Q^T[D][16]
//   O^T[D][16 cols]      += V^T[D][32] . P^T[32][16]
//
// with the same operand layout as the decode kernel (a lane's 8 key scores
// are directly its P^T k-slots).  The softmax keeps a reference max that only
// moves when the running max outgrows it by 2^8, so the O accumulators are
// rarely rescaled.  Chunks entirely above a wave's causal diagonal, or
// entirely left of its sliding window, are skipped without MFMA work; chunks
// entirely visible skip the per-element mask.  Query blocks are issued
// longest-first, and the workgroups of one (sequence, kv head) share an XCD L2
// when the kv head count is a multiple of 8 (grid x = kv head).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 64;         // keys per pipeline step
constexpr int kStagePages = 2048;  // page ids staged in LDS (>= pages_per_slot, host-checked)

// 16-column MFMA tiles per wave.
template <int D>
constexpr int prefill_nt() { return D <= 128 ? 2 : 1; }

template <int D>
constexpr int k_tile_bytes() { return kChunk * D * 2; }   // [64 keys][D] bf16
template <int D>
constexpr int tile_bytes() { return 2 * k_tile_bytes<D>(); }  // + V^T [D][64 keys]
template <int D>
constexpr int dma_per_wave() { return D / 32; }  // 1 KB copies per wave, for K and for V each

// Swizzles (16-byte slot of a row).  K row r holds chunk c (dims 8c..8c+7) at
// slot c ^ k_swz(r); V^T row d holds key group g (keys 8g..8g+7) at slot
// g ^ v_swz(d).  Both are bijections within a row; for the 16 rows one MFMA
// operand read touches they give 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 64 ? (((r >> 1) + 2 * (r >> 4)) & 7) : ((r + 4 * (r >> 4)) & 15);
}
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max of the 8 scores a lane holds for its column (two 4-row accumulators).
// Scores are finite or -inf (masked), so the NaN-propagating maximum needs no
// canonicalisation of the MFMA results.
__device__ __forceinline__ float max8(const f32x4 (&s)[2]) {
  return vmax(vmax(vmax(s[0][0], s[0][1]), vmax(s[0][2], s[0][3])),
              vmax(vmax(s[1][0], s[1][1]), vmax(s[1][2], s[1][3])));
}

// Max over the four lanes l, l^16, l^32, l^48 (the 4 key groups of a column)
// with gfx950's row-swap permutes: each swap hands every lane its partner's
// value in one of the two outputs.
__device__ __forceinline__ float quad_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = vmax(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return vmax(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
}

template <int D, int NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
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
  const float inv_c = 1.0f / a.scale_log2;  // scale > 0 (host-checked)
  // LDS byte offsets (within a tile buffer) of this lane's MFMA operand rows.
  // K row r, dims chunk c sits at kofs ^ (64 * c): the row's swizzle is folded
  // into kofs and 64*c only flips bits inside the row.  V^T rows d = 16*dt + qc
  // share one swizzle across dt, so dt is a plain 2 KB step from vofs.
  int kofs[2][2], vofs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int r = 32 * h + 8 * (qc >> 2) + 4 * rg + (qc & 3);
      kofs[h][rg] = r * (2 * D) + 16 * (quad ^ k_swz<D>(r));
    }
    vofs[h] = k_tile_bytes<D>() + qc * 128 + 16 * ((4 * h + quad) ^ v_swz(qc));
  }
  // Source byte offsets of this lane's tile copies, relative to the chunk's
  // first key in its page.  Copy k of the wave fills tile bytes m*1024 ..
  // m*1024+1023 (m = w*dpw + k), lane i the 16 bytes at +16*i.  K: tile row r
  // slot s holds dims 8*(s ^ k_swz(r)) ..  V^T: row d slot s holds keys
  // 8*(s ^ v_swz(d)) .. (V pages are d-major: element (d, key) at d*ps + key).
  uint32_t dma_k[dma_per_wave<D>()], dma_v[dma_per_wave<D>()];
#pragma unroll
  for (int k = 0; k < dma_per_wave<D>(); ++k) {
    const int o = (w * dma_per_wave<D>() + k) * 1024 + 16 * lane;
    const int r = o / (2 * D), sk = (o % (2 * D)) >> 4;
    dma_k[k] = 2 * (r * D + 8 * (sk ^ k_swz<D>(r)));
    const int d = o >> 7, sv = (o >> 4) & 7;
    dma_v[k] = 2 * (d * ps + 8 * (sv ^ v_swz(d)));
  }

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
    // m_run: reference max (log2 units), neg_m: -m_run (0 while m_run = -inf),
    // thr: raw-score threshold (m_run + 8) / c above which m_run must move.
    float m_run[NT], l_run[NT], neg_m[NT], thr[NT];
    f32x4 acc[NT][D / 16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = -INFINITY;
      neg_m[nt] = 0.f;
      thr[nt] = -INFINITY;
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

    // Copies the chunk at j0 into LDS buffer buf: this wave's share of the K
    // and V^T 1 KB blocks.  Keys past kv_hi (and unmapped pages) read page 0
    // or stay inside the chunk's page, so every address is inside the pool;
    // the scores of such keys are masked and their V^T entries zeroed after
    // the copy lands.
    auto issue = [&](int buf, int j0) {
      uint8_t* tK = lds + buf * tile_bytes<D>();
      uint8_t* tV = tK + k_tile_bytes<D>();
      if (ps >= kChunk) {
        // The chunk lies inside one page: one (scalar) page id and source base;
        // the lane offsets within the page are fixed.
        const int page = __builtin_amdgcn_readfirstlane(max(s_pg[(j0 >> log2ps) - pg0], 0));
        const size_t base = (size_t)page * page_stride;
        const int in_pg = j0 & (ps - 1);
        const uint8_t* ks = reinterpret_cast<const uint8_t*>(kbase + base + (size_t)in_pg * D);
        const uint8_t* vs = reinterpret_cast<const uint8_t*>(vbase + base + in_pg);
#pragma unroll
        for (int k = 0; k < dma_per_wave<D>(); ++k)
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const bf16_t*>(ks + dma_k[k]), (lds_void_ptr)(tK + (w * dma_per_wave<D>() + k) * 1024),
                                           16, 0, 0);
#pragma unroll
        for (int k = 0; k < dma_per_wave<D>(); ++k)
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const bf16_t*>(vs + dma_v[k]), (lds_void_ptr)(tV + (w * dma_per_wave<D>() + k) * 1024),
                                           16, 0, 0);
        return;
      }
      // Small pages: a page id per lane and copy (branch-free, so the page id
      // reads are issued together).
#pragma unroll
      for (int k = 0; k < dma_per_wave<D>(); ++k) {
        const int r = (int)dma_k[k] / (2 * D), c8 = ((int)dma_k[k] % (2 * D)) >> 1;  // row, first dim
        const int j = j0 + r;
        const int pgv = s_pg[min((j >> log2ps) - pg0, n_pg - 1)];
        const int page = j < kv_hi ? max(pgv, 0) : 0;
        const bf16_t* src = kbase + (size_t)page * page_stride + (size_t)(j & (ps - 1)) * D + c8;
        __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(tK + (w * dma_per_wave<D>() + k) * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < dma_per_wave<D>(); ++k) {
        const int o = (w * dma_per_wave<D>() + k) * 1024 + 16 * lane;
        const int d = o >> 7, g = ((o >> 4) & 7) ^ v_swz(d);
        const int j = j0 + 8 * g;
        const int pgv = s_pg[min((j >> log2ps) - pg0, n_pg - 1)];
        const int page = j < kv_hi ? max(pgv, 0) : 0;
        const bf16_t* src = vbase + (size_t)page * page_stride + (size_t)d * ps + (j & (ps - 1));
        __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(tV + (w * dma_per_wave<D>() + k) * 1024), 16, 0, 0);
      }
    };
    // After a tail chunk lands: zero the V^T entries of keys >= kv_hi (stale
    // page rows may hold anything, and 0 * NaN would poison P.V).
    auto zero_tail = [&](int buf, int j0) {
      const int nvk = kv_hi - j0;
      if (nvk >= kChunk) return;
      uint8_t* tV = lds + buf * tile_bytes<D>() + k_tile_bytes<D>();
      for (int idx = tid; idx < D * 8; idx += kThreads) {
        const int d = idx >> 3, s = idx & 7;
        const int g = s ^ v_swz(d);
        const int nv = nvk - 8 * g;
        if (nv >= 8) continue;
        u32x4* p = reinterpret_cast<u32x4*>(tV + d * 128 + 16 * s);
        u32x4 v = *p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t m = (2 * e < nv ? 0x0000ffffu : 0u) | (2 * e + 1 < nv ? 0xffff0000u : 0u);
          v[e] &= m;
        }
        *p = v;
      }
    };

    if (n_chunks > 0) issue(0, j_start);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
    __syncthreads();
    if (n_chunks > 0 && j_start + kChunk > kv_hi) {
      zero_tail(0, j_start);
      __syncthreads();
    }
    for (int ck = 0; ck < n_chunks; ++ck) {
      const int j0 = j_start + ck * kChunk;
      if (ck + 1 < n_chunks) issue((ck + 1) & 1, j0 + kChunk);  // lands during this chunk's math
      const int buf_off = (ck & 1) * tile_bytes<D>();
      const bool skip = wave_hi < 0 || j0 > wave_hi ||
                        (a.window > 0 && j0 + kChunk - 1 <= wave_lo - a.window);
      if (!skip) {
        const bool full = (j0 + kChunk - 1 <= wave_lo) && (a.window <= 0 || wave_hi - j0 < a.window);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // ---- S^T = K Q^T for keys j0 + 32h + ..: MFMA rg row m holds key 8*(m/4) + 4*rg + m%4
          f32x4 S[NT][2];
#pragma unroll
          for (int rg = 0; rg < 2; ++rg) {
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
              const u32x4 kv = *reinterpret_cast<const u32x4*>(
                  lds + ((buf_off + kofs[h][rg]) ^ (64 * c)));
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                S[nt][rg] = mfma16x16x32(kv, qreg[nt][c], c ? S[nt][rg] : f32x4{0.f, 0.f, 0.f, 0.f});
            }
          }
          // ---- element mask, only on chunks crossing the diagonal or the window edge
          if (!full) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const int pc = pcol[nt];
              const int jmin = a.window > 0 ? pc - a.window + 1 : -0x7fffffff;
#pragma unroll
              for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int j = j0 + 32 * h + 8 * quad + 4 * rg + e;
                  if (j > pc || j < jmin) S[nt][rg][e] = -INFINITY;
                }
            }
          }
          // ---- softmax against a lazily moved per-column reference max m_run:
          // p = 2^(s*c - m_run).  m_run (with O and l rescaled) only moves when
          // a score exceeds it by more than 2^8, which the common path detects
          // with a per-lane compare against the column threshold (m_run + 8) / c
          // -- no cross-lane work unless some lane of the wave crosses it.
          bool need = false;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) need |= max8(S[nt]) > thr[nt];
          if (__any(need)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const float mx = quad_max(max8(S[nt]));  // max over the column's 32 keys
              const float m_new = fmaxf(m_run[nt], mx * a.scale_log2);
              float alpha = 1.0f;
              if (m_new > m_run[nt] + 8.0f) {
                alpha = fast_exp2(m_run[nt] - m_new);  // 0 when m_run was -inf
                m_run[nt] = m_new;
                neg_m[nt] = -m_new;
                thr[nt] = (m_new + 8.0f) * inv_c;
              }
              l_run[nt] *= alpha;
#pragma unroll
              for (int dt = 0; dt < D / 16; ++dt) acc[nt][dt] *= alpha;
            }
          }
          u32x4 pb[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(S[nt][e >> 2][e & 3], a.scale_log2, neg_m[nt]));
            pb[nt] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            // fp32 row sum (summing the bf16 weights instead would cost the
            // log-sum-exp up to 2^-9 of relative accuracy)
            l_run[nt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          }
          // ---- O^T += V^T P^T for this half; lane row d = 16*dt + qc, keys group 4h + quad
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const u32x4 vv = *reinterpret_cast<const u32x4*>(lds + buf_off + vofs[h] + dt * 2048);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt][dt] = mfma16x16x32(vv, pb[nt], acc[nt][dt]);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next chunk's copies have landed
      __syncthreads();
      if (ck + 1 < n_chunks && j0 + 2 * kChunk > kv_hi) {
        zero_tail((ck + 1) & 1, j0 + kChunk);
        __syncthreads();
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
  const size_t lds = 2 * (size_t)tile_bytes<D>();
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
