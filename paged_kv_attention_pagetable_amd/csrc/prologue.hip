// Fused prefill prologue, k and v side: per token and kv head, RMSNorm of k
// over head_dim with a gain, then half-split rotary embedding; the new k and
// v (raw, or for Gemma-4 its RMSNorm without a gain) are appended to the
// pages.  (q gets the same norm and
// rotation inside the prefill attention kernel, as it loads q.)
//
// Row layout: D/8 lanes hold one head row, 8 dims (16 bytes) each.  The
// rotate_half partner of dims 8c..8c+7 lives in lane c ^ (D/16) of the same
// row group, and the mean of squares is a xor-shuffle reduction over the
// row's lanes.  All arithmetic is fp32; each output is rounded to bf16 once.
// grid = (2 n_kv, ceil(T / 32)): a workgroup handles 32 tokens of one k head
// or of one v head (the v heads stage V^T in LDS, as the append kernel does).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kProTokens = 32;  // tokens per workgroup (many small workgroups: the
                                 // per-workgroup set-up is latency, not bandwidth)
// k heads per workgroup (one: more workgroups in flight measured faster than
// sharing a token's cos / sin across heads)
template <int D>
constexpr int pro_heads() { return 1; }
constexpr int kCuStage = 512;  // sequences whose metadata is staged in LDS (n_seqs < this)

// RMSNorm without a gain of one head row (D/8 lanes, 8 dims each): the mean
// of squares is a xor-shuffle sum over the row's lanes; fp32, one bf16
// rounding (Gemma-4 v_norm).
template <int D>
__device__ __forceinline__ u32x4 norm_row(u32x4 x, float eps) {
  constexpr int LPR = D / 8;
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16lo(x[e]);
    v[2 * e + 1] = bf16hi(x[e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e] * inv, v[2 * e + 1] * inv);
  return out;
}

// cs / sn: cos and sin of the lane's 8 rotary angles (frequencies f0 .. f0+7,
// f0 = 8c mod D/2) at the row's position.
template <int D>
__device__ __forceinline__ u32x4 norm_rope_row(u32x4 x, const bf16_t* w, const float (&cs)[8],
                                               const float (&sn)[8], int c, float eps) {
  constexpr int LPR = D / 8;  // lanes per row
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16lo(x[e]);
    v[2 * e + 1] = bf16hi(x[e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  const u32x4 wv = load16(w + 8 * c);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = v[2 * e] * inv * bf16lo(wv[e]);
    v[2 * e + 1] = v[2 * e + 1] * inv * bf16hi(wv[e]);
  }
  // rotate_half partner: dims +- D/2, i.e. lane chunk c ^ (LPR/2).
  float pr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pr[j] = shfl_xor(v[j], LPR / 2);
  const bool first_half = c < LPR / 2;
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float o[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = 2 * e + k;
      const float rot = first_half ? -pr[j] : pr[j];
      o[k] = v[j] * cs[j] + rot * sn[j];
    }
    out[e] = pack_bf16x2(o[0], o[1]);
  }
  return out;
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// accesses, not for its outstanding global loads (__syncthreads() would also
// drain the row loads in flight).  The signal fences keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sequence of token t: the last n with cu[n] <= t (cu ascending, cu[0] = 0).
__device__ __forceinline__ int seq_of(const int32_t* cu, int n_seqs, int t) {
  int lo = 0, hi = n_seqs;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Shared memory of one prologue workgroup.
template <int D>
struct ProSmem {
  int cu[kCuStage];
  int slot[kCuStage];
  int sp[kCuStage];
  int page[kProTokens];
  int row[kProTokens];
  int pos[kProTokens];
  bf16_t v[kProTokens][D + 2];  // +2: odd dword stride, no bank conflicts
};

enum { kHeadK = 1, kHeadV = 2 };

// One workgroup: 64 tokens of one head of kind KIND (q: normalise + rotate in
// place; k: normalise + rotate + append; v: raw append).  Each kind (and the
// staged / global metadata form) is its own code path, so the compiler's
// waits for one path's loads never drain another's rows in flight.
template <int D, int KIND, bool STAGED>
__device__ __forceinline__ void prologue_body(const PrologueArgs& a, ProSmem<D>& sm, int h0) {
  // k workgroups take pro_heads<D>() heads of the same tokens (the cos / sin
  // of a token serve all of them); v workgroups one head.
  constexpr int LPR = D / 8;
  constexpr int ROWS = 256 / LPR;              // rows processed per pass by the workgroup
  constexpr int PASSES = kProTokens / ROWS;    // passes over the workgroup's tokens
  const int t0 = blockIdx.y * kProTokens;
  const int nt = min(kProTokens, a.T - t0);
  const int tid = threadIdx.x;
  const int n_kv = a.g.n_kv, ps = a.g.page_size;
  const int c = tid % LPR;
  const int rsub = tid / LPR;
  constexpr int HN = KIND == kHeadV ? 1 : pro_heads<D>();
  const int n_heads = n_kv;
  const int h = h0;  // first head of the workgroup
  // Sequence metadata (cu_seqlens, slots, start_pos) staged in LDS: loads
  // issued first, the row loads right after, so the set-up overlaps the rows'
  // latency (it waits for the metadata only; the barriers are LDS-only).
  // Loads are unconditional with clamped indices so the waits stay partial.
  int m_cu[kCuStage / 256], m_slot[kCuStage / 256], m_sp[kCuStage / 256];
  if (STAGED) {
#pragma unroll
    for (int j = 0; j < kCuStage / 256; ++j) {
      const int i = tid + 256 * j;
      m_cu[j] = a.cu_seqlens[min(i, a.n_seqs)];
      m_slot[j] = a.slots[min(i, a.n_seqs - 1)];
      m_sp[j] = a.start_pos ? a.start_pos[min(i, a.n_seqs - 1)] : 0;
    }
  }
  // This thread's rows.  Rows past the last token re-read token t0 (in
  // bounds) and are never stored.
  const bf16_t* src = KIND == kHeadK ? a.k_raw : a.v_raw;
  const int src_heads = n_kv;
  u32x4 x[PASSES][HN];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const int tt = rsub + k * ROWS;
    const int tr = t0 + (tt < nt ? tt : 0);
#pragma unroll
    for (int j = 0; j < HN; ++j)
      x[k][j] = load16(src + ((size_t)tr * src_heads + min(h + j, n_heads - 1)) * D + 8 * c);
  }
  if (STAGED) {
#pragma unroll
    for (int j = 0; j < kCuStage / 256; ++j) {
      const int i = tid + 256 * j;
      if (i <= a.n_seqs) sm.cu[i] = m_cu[j];
      if (i < a.n_seqs) {
        sm.slot[i] = m_slot[j];
        sm.sp[i] = m_sp[j];
      }
    }
    lds_barrier();
  }
  // k rows with staged metadata: each lane finds its rows' positions itself
  // and issues their cos / sin loads now, in flight with the page-table loads
  // below (one memory round trip instead of two).
  const int f0 = (8 * c) & (D / 2 - 1);
  int pos_k[PASSES];
  float cs[PASSES][8], sn[PASSES][8];
  auto load_cs = [&]() {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const size_t ro = (size_t)max(pos_k[k], 0) * (D / 2) + f0;
#pragma unroll
      for (int j = 0; j < 8; j += 4) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(a.cos_t + ro + j);
        const f32x4 sv = *reinterpret_cast<const f32x4*>(a.sin_t + ro + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cs[k][j + e] = cv[e];
          sn[k][j + e] = sv[e];
        }
      }
    }
  };
  if constexpr (KIND == kHeadK && STAGED) {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int tt = rsub + k * ROWS;
      pos_k[k] = -1;
      if (tt < nt) {
        const int t = t0 + tt;
        const int n = seq_of(sm.cu, a.n_seqs, t);
        const int slot = sm.slot[n], pos = sm.sp[n] + (t - sm.cu[n]);
        if (slot > 0 && slot < a.pt.max_slots && pos >= 0 && pos < a.max_pos) pos_k[k] = pos;
      }
    }
    load_cs();
  }
  if (tid < nt) {
    const int t = t0 + tid;
    int n, cu_n, slot, sp;
    if (STAGED) {
      n = seq_of(sm.cu, a.n_seqs, t);
      cu_n = sm.cu[n];
      slot = sm.slot[n];
      sp = sm.sp[n];
    } else {
      n = seq_of(a.cu_seqlens, a.n_seqs, t);
      cu_n = a.cu_seqlens[n];
      slot = a.slots[n];
      sp = a.start_pos ? a.start_pos[n] : 0;
    }
    const int pos = sp + (t - cu_n);
    int page = -1, row = 0;
    const bool ok = slot > 0 && slot < a.pt.max_slots && pos >= 0 && pos < a.max_pos;
    if (ok) {
      const int lp = pos >> a.g.log2ps;
      if (lp < a.pt.pps) {
        const int pg = a.pt.table[(size_t)slot * a.pt.pps + lp];
        if (pg >= 1 && pg < a.g.n_pages) {
          page = pg;
          row = pos & (ps - 1);
        }
      }
    }
    sm.page[tid] = page;
    sm.row[tid] = row;
    sm.pos[tid] = ok ? pos : -1;
  }
  lds_barrier();
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)n_kv * blk;
  if (KIND == kHeadV) {
    // V rows (raw, or RMSNorm without a gain) -> LDS staging, then stored
    // transposed: lanes on consecutive tokens, so tokens sharing a page and
    // key group are contiguous
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int tt = rsub + k * ROWS;
      const u32x4 y = a.v_norm ? norm_row<D>(x[k][0], a.eps) : x[k][0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.v[tt][8 * c + 2 * e] = (bf16_t)(y[e] & 0xffffu);
        sm.v[tt][8 * c + 2 * e + 1] = (bf16_t)(y[e] >> 16);
      }
    }
    lds_barrier();
    for (int i = tid; i < D * kProTokens; i += 256) {
      const int d = i / kProTokens, tt = i - d * kProTokens;
      if (tt >= nt) continue;
      const int page = sm.page[tt];
      if (page < 0 || sm.pos[tt] < 0) continue;
      a.vpool[(size_t)page * page_stride + h * blk + v_elem_offset(d, sm.row[tt], D, a.g.log2ps)] = sm.v[tt][d];
    }
    return;
  }
  if constexpr (!STAGED) {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int tt = rsub + k * ROWS;
      pos_k[k] = tt < nt ? sm.pos[tt] : -1;
    }
    load_cs();
  }
  const bf16_t* w = a.k_w;
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const int tt = rsub + k * ROWS;
    if (pos_k[k] < 0) continue;  // uniform over the row's lanes
#pragma unroll
    for (int j = 0; j < HN; ++j) {
      if (h + j >= n_heads) break;  // uniform over the workgroup
      const u32x4 y = norm_rope_row<D>(x[k][j], w, cs[k], sn[k], c, a.eps);
      if (sm.page[tt] >= 0) {
        store16(a.kpool + (size_t)sm.page[tt] * page_stride + (h + j) * blk + (size_t)sm.row[tt] * D + 8 * c, y);
      }
    }
  }
}

// grid = (nk_wg + n_kv, ceil(T / 64)): x < nk_wg takes k heads
// pro_heads*x .., then one workgroup per v head.
template <int D>
__global__ __launch_bounds__(256) void prologue_kernel(const int32_t* cu_seqlens, const int32_t* slots,
                                                       const int32_t* start_pos, const bf16_t* k_raw,
                                                       const bf16_t* v_raw, int T, int n_seqs,
                                                       PrologueArgs args) {
  // cu_seqlens .. n_seqs repeat fields of `args`: passed first, they arrive
  // preloaded in scalar registers (the library builds this file with seven
  // preloaded kernel arguments), so the first metadata and row loads issue
  // at once.  (prologue_body is inlined: the copy stays in registers.)
  PrologueArgs a = args;
  a.cu_seqlens = cu_seqlens;
  a.slots = slots;
  a.start_pos = start_pos;
  a.k_raw = k_raw;
  a.v_raw = v_raw;
  a.T = T;
  a.n_seqs = n_seqs;
  __shared__ ProSmem<D> sm;
  const int nk_wg = (a.g.n_kv + pro_heads<D>() - 1) / pro_heads<D>();
  const int x = blockIdx.x;
  if (a.n_seqs < kCuStage) {
    if (x < nk_wg) prologue_body<D, kHeadK, true>(a, sm, pro_heads<D>() * x);
    else prologue_body<D, kHeadV, true>(a, sm, x - nk_wg);
  } else {
    if (x < nk_wg) prologue_body<D, kHeadK, false>(a, sm, pro_heads<D>() * x);
    else prologue_body<D, kHeadV, false>(a, sm, x - nk_wg);
  }
}

template <int D>
hipError_t launch_prologue_d(const PrologueArgs& a, hipStream_t st) {
  // Heads vary fastest: the workgroups in flight cover all heads of a few
  // token blocks, i.e. contiguous [token][head][D] memory, not one head's
  // 256-byte pieces strided across many tokens.
  const int nk_wg = (a.g.n_kv + pro_heads<D>() - 1) / pro_heads<D>();
  dim3 grid(nk_wg + a.g.n_kv, (a.T + kProTokens - 1) / kProTokens);
  hipLaunchKernelGGL((prologue_kernel<D>), grid, dim3(256), 0, st, a.cu_seqlens, a.slots, a.start_pos,
                     a.k_raw, a.v_raw, a.T, a.n_seqs, a);
  return hipGetLastError();
}

// cos / sin of p * theta^(-2i/D) in fp64, stored as fp32.
__global__ void rope_table_kernel(float* c, float* s, int max_pos, int half, double theta,
                                  int head_dim, int n_rot) {
  const long n = (long)max_pos * half;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < n;
       idx += (long)gridDim.x * blockDim.x) {
    const int p = (int)(idx / half), i = (int)(idx - (long)p * half);
    // frequencies past n_rot are zero (partial rotary: cos 1, sin 0)
    const double inv = i < n_rot ? pow(theta, -2.0 * (double)i / (double)head_dim) : 0.0;
    const double ang = (double)p * inv;
    c[idx] = (float)cos(ang);
    s[idx] = (float)sin(ang);
  }
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  switch (a.g.head_dim) {
    case 64: return launch_prologue_d<64>(a, st);
    case 128: return launch_prologue_d<128>(a, st);
    case 256: return launch_prologue_d<256>(a, st);
    case 512: return launch_prologue_d<512>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope_table(float* c, float* s, int max_pos, int head_dim, double theta,
                             int n_rot, hipStream_t st) {
  const int half = head_dim / 2;
  const long n = (long)max_pos * half;
  if (n <= 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, st, c, s, max_pos, half,
                     theta, head_dim, n_rot);
  return hipGetLastError();
}

}  // namespace pkv
