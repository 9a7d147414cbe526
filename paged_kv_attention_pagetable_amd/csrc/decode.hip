// Split-K paged decode attention for gfx950 (one kernel per call).
//
// One query token per batch row attends to its slot's keys 0..L-1 (window:
// the last W of them).  Grid = (split, kv head, batch row); a workgroup of 4
// wave64s owns one contiguous key range of one (row, kv head).  Keys are
// processed in 32-key chunks on bf16 MFMA 16x16x32 tiles whose 16 columns are
// the G query heads of the kv head (G <= 16, unused columns are zero):
//
//   S^T[32 keys][16 q]  = K[32][D] . Q^T[D][16]
//   O^T[D][16 q]       += V^T[D][32 keys] . P^T[32][16]
//
// K rows come from the token-major K pool and V^T rows from the d-major V
// pool as 16-byte loads straight into MFMA operand registers; a lane's 8 key
// scores land exactly in its P^T k-slots, so no LDS round trip is needed for
// P.  The physical page ids of the workgroup's range are read once into LDS,
// so no page-table load sits on a chunk's critical path, and each chunk's K
// and V loads are issued together.
//
// head_dim <= 128: the 4 waves take interleaved chunks (key split inside the
// workgroup) and are merged in LDS at the end.  head_dim >= 256: the 4 waves
// split head_dim instead -- each computes a partial S over its quarter of the
// dims, the partials are summed through LDS (one barrier per chunk) and every
// wave owns a quarter of the output rows, which keeps the operand registers of
// a chunk at the head_dim-128 size.
//
// With several splits per row the partial (o, max, sum) of each workgroup
// goes to the workspace and a small merge kernel combines them in fixed split
// order (bitwise deterministic).  (A last-arriving-workgroup merge inside the
// split kernel needs an agent-scope release per workgroup, which on gfx950 is
// an L2 write-back each; measured far slower than the second launch.)
// Optionally the new token's K/V is appended first by the workgroup that owns
// the last key.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kDecodeWaves = 4;
constexpr int kThreads = kDecodeWaves * 64;
constexpr int kSegPages = 64;  // page ids staged in LDS per range segment
constexpr int kMaxGD = 2048;   // (query heads per kv head) * head_dim, checked on the host
constexpr int kMaxMergeWeights = 1024;  // splits * G of one (row, kv head)

// Masks the bf16 elements e >= nvalid (0..8) of an 8-element operand.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nvalid) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = (2 * i < nvalid ? 0x0000ffffu : 0u) | (2 * i + 1 < nvalid ? 0xffff0000u : 0u);
    r[i] = v[i] & m;
  }
  return r;
}

struct RowRange {
  int slot, L, lo, start, end, n_valid;
  bool idle;
};

__device__ __forceinline__ RowRange row_range(const DecodeArgs& a, int b, int s) {
  RowRange r;
  r.slot = a.slots[b];
  r.L = a.seq_lens[b];
  r.idle = r.slot <= 0 || r.slot >= a.pt.max_slots || r.L <= 0;
  r.lo = r.start = r.end = r.n_valid = 0;
  if (r.idle) return r;
  r.L = min(r.L, a.pt.pps * a.g.page_size);
  r.lo = a.window > 0 ? max(0, r.L - a.window) : 0;
  const int base = r.lo & ~31;
  r.n_valid = min(a.max_splits, (r.L - base + a.split_tokens - 1) / a.split_tokens);
  r.start = base + s * a.split_tokens;
  r.end = (s == a.max_splits - 1) ? r.L : min(r.L, r.start + a.split_tokens);
  return r;
}

// Fused append: the workgroup owning key L-1 writes the new token of (b, hk).
__device__ __forceinline__ void append_new_token(const DecodeArgs& a, const RowRange& r, int b,
                                                 int hk, int D) {
  const int p = r.L - 1;
  const int lp = p >> a.g.log2ps;
  const int page = a.pt.table[(size_t)r.slot * a.pt.pps + lp];
  if (page < 1 || page >= a.g.n_pages) return;
  const int ps = a.g.page_size;
  const size_t blk = (size_t)ps * D;
  const size_t dst = (size_t)page * a.g.n_kv * blk + hk * blk;
  const int row = p & (ps - 1);
  const size_t src = ((size_t)b * a.g.n_kv + hk) * D;
  for (int i = threadIdx.x; i < D / 8; i += blockDim.x)
    store16(a.kpool_w + dst + (size_t)row * D + 8 * i, load16(a.k_new + src + 8 * i));
  for (int d = threadIdx.x; d < D; d += blockDim.x) a.vpool_w[dst + (size_t)d * ps + row] = a.v_new[src + d];
}

// Stages the page ids of logical pages [p0, p0 + n) of the row into LDS.
__device__ __forceinline__ void stage_pages(const DecodeArgs& a, const int32_t* trow, int p0, int n,
                                            int* s_pg) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int pg = trow[p0 + i];
    s_pg[i] = (pg >= 1 && pg < a.g.n_pages) ? pg : -1;
  }
}

// Writes this workgroup's result: the final output (single split) or its
// unnormalised partial (o, running max in log2 units, sum) for the merge
// kernel.  o_val(g, d), Mof(g), Lof(g) give the workgroup's values.
template <int D, class OFn, class MFn, class LFn>
__device__ void finish(const DecodeArgs& a, int b, int hk, int s, OFn o_val, MFn Mof, LFn Lof) {
  const int G = a.G;
  const int tid = threadIdx.x;
  if (a.max_splits == 1) {
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
      const int g = idx / D, d = idx - g * D;
      const float l = Lof(g);
      a.out[((size_t)b * a.n_q + hk * G + g) * D + d] = f32_to_bf16(l > 0.f ? o_val(g, d) / l : 0.f);
      if (a.lse && d == 0)
        a.lse[(size_t)b * a.n_q + hk * G + g] = l > 0.f ? (Mof(g) + __log2f(l)) * kLn2 : -INFINITY;
    }
    return;
  }
  const size_t pbase = ((size_t)b * a.g.n_kv + hk) * a.max_splits + s;
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int g = idx / D, d = idx - g * D;
    a.part_o[(pbase * G + g) * D + d] = o_val(g, d);
  }
  for (int g = tid; g < G; g += blockDim.x) {
    a.part_ml[(pbase * G + g) * 2] = Mof(g);
    a.part_ml[(pbase * G + g) * 2 + 1] = Lof(g);
  }
}

// A split with nothing to do (idle row, or a split past the row's last key)
// leaves an empty partial: max -inf, sum 0.  The merge skips it.
__device__ __forceinline__ void empty_partial(const DecodeArgs& a, int b, int hk, int s) {
  if (a.max_splits == 1) return;
  const size_t pbase = ((size_t)b * a.g.n_kv + hk) * a.max_splits + s;
  for (int g = threadIdx.x; g < a.G; g += blockDim.x) {
    a.part_ml[(pbase * a.G + g) * 2] = -INFINITY;
    a.part_ml[(pbase * a.G + g) * 2 + 1] = 0.f;
  }
}

__device__ __forceinline__ void idle_output(const DecodeArgs& a, int b, int hk, int s, int D) {
  if (a.max_splits == 1) {
    for (int idx = threadIdx.x; idx < a.G * D; idx += blockDim.x) {
      const int g = idx / D, d = idx - g * D;
      a.out[((size_t)b * a.n_q + hk * a.G + g) * D + d] = 0;
      if (a.lse && d == 0) a.lse[(size_t)b * a.n_q + hk * a.G + g] = -INFINITY;
    }
  } else {
    empty_partial(a, b, hk, s);
  }
}

// Log-sum-exp merge of the split partials of one (row, kv head), in fixed
// split order.  Needs no row metadata: empty partials carry a zero sum.  One
// wave per query column reduces the split maxima and sums across its lanes.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float s_w[kMaxMergeWeights];
  const int hk = blockIdx.x, b = blockIdx.y;
  const int G = a.G, S = a.max_splits;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t pbase = ((size_t)b * a.g.n_kv + hk) * S;
  const float* ml = a.part_ml + pbase * G * 2;
  for (int g = w; g < G; g += kDecodeWaves) {
    float M = -INFINITY;
    for (int t = lane; t < S; t += 64) {
      const float2 v = *reinterpret_cast<const float2*>(ml + (t * G + g) * 2);
      if (v.y > 0.f) M = fmaxf(M, v.x);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor(M, m));
    float lsum = 0.f;
    for (int t = lane; t < S; t += 64) {
      const float2 v = *reinterpret_cast<const float2*>(ml + (t * G + g) * 2);
      const float f = v.y > 0.f ? fast_exp2(v.x - M) : 0.f;
      s_w[t * G + g] = f;
      lsum += f * v.y;
    }
    lsum = wave_sum(lsum);
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    for (int t = lane; t < S; t += 64) s_w[t * G + g] *= inv;
    if (a.lse && lane == 0)
      a.lse[(size_t)b * a.n_q + hk * G + g] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D / 4; idx += kThreads) {
    const int g = (4 * idx) / D, d = 4 * idx - g * D;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* po = a.part_o + (pbase * G + g) * D + d;
    // Loads are unconditional (an empty partial's o is never written and may
    // hold anything); the select drops them, so they can all be in flight.
#pragma unroll 8
    for (int t = 0; t < S; ++t) {
      const float wt = s_w[t * G + g];
      const f32x4 v = *reinterpret_cast<const f32x4*>(po + (size_t)t * G * D);
      o += wt != 0.f ? wt * v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint2 pk;
    pk.x = pack_bf16x2(o[0], o[1]);
    pk.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2*>(a.out + ((size_t)b * a.n_q + hk * G + g) * D + d) = pk;
  }
}

// ---------------------------------------------------------------------------
// head_dim <= 128: key split across the NW waves of the workgroup.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_keysplit_kernel(DecodeArgs a) {
  extern __shared__ float s_o[];                  // [wave][G][D] (dynamic: NW * G * D)
  __shared__ int s_pg[kSegPages];
  __shared__ float s_ml[2 * NW * 16];             // [wave][16] max, then sum
  __shared__ float s_red[NW * 16 + 32];
  const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qc = lane & 15, quad = lane >> 4;
  const int G = a.G;
  const RowRange r = row_range(a, b, s);
  if (r.idle) {
    if (s == 0 || a.max_splits > 1) idle_output(a, b, hk, s, D);
    return;
  }
  if (r.start >= r.L) {
    empty_partial(a, b, hk, s);
    return;
  }
  if (a.k_new && r.end == r.L) append_new_token(a, r, b, hk, D);

  const int ps = a.g.page_size, log2ps = a.g.log2ps;
  const int32_t* trow = a.pt.table + (size_t)r.slot * a.pt.pps;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)a.g.n_kv * blk;
  const bf16_t* kbase = a.kpool + hk * blk;
  const bf16_t* vbase = a.vpool + hk * blk;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Q^T operand; loaded after the first page staging so that no barrier
  // waits on it and it overlaps the first chunk's K/V loads.
  u32x4 qreg[D / 32];
  const bf16_t* qrow = a.q + ((size_t)b * a.n_q + hk * G + min(qc, G - 1)) * D + 8 * quad;

  const int seg_tokens = kSegPages * ps;
  for (int seg0 = r.start; seg0 < r.end; seg0 += seg_tokens) {
    const int seg1 = min(r.end, seg0 + seg_tokens);
    const int p0 = seg0 >> log2ps;
    __syncthreads();  // previous segment's page ids consumed; orders the fused append
    stage_pages(a, trow, p0, ((seg1 - 1) >> log2ps) - p0 + 1, s_pg);
    __syncthreads();
    if (seg0 == r.start) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 v = load16(qrow + 32 * c);
        qreg[c] = qc < G ? v : u32x4{0, 0, 0, 0};
      }
    }
    for (int t0 = seg0 + 32 * w; t0 < seg1; t0 += 32 * NW) {
      // ---- issue the chunk's K and V^T loads together
      u32x4 kop[2][D / 32];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int tk = t0 + 8 * (qc >> 2) + 4 * rg + (qc & 3);
        const int page = tk < seg1 ? s_pg[(tk >> log2ps) - p0] : -1;
        const bf16_t* kp = kbase + (size_t)max(page, 0) * page_stride + (size_t)(tk & (ps - 1)) * D + 8 * quad;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kop[rg][c] = page >= 0 ? load16(kp + 32 * c) : u32x4{0, 0, 0, 0};
      }
      const int tv = t0 + 8 * quad;
      const int vpage = tv < seg1 ? s_pg[(tv >> log2ps) - p0] : -1;
      const int nvalid = seg1 - tv;
      const bf16_t* vp = vbase + (size_t)max(vpage, 0) * page_stride + (size_t)qc * ps + (tv & (ps - 1));
      u32x4 vop[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        vop[dt] = vpage >= 0 ? load16(vp + (size_t)16 * dt * ps) : u32x4{0, 0, 0, 0};
        if (nvalid < 8) vop[dt] = keep_first(vop[dt], nvalid);
      }
      // ---- S^T = K Q^T; MFMA rg row m holds key 8*(m/4) + 4*rg + m%4
      f32x4 S[2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) sacc = mfma16x16x32(kop[rg][c], qreg[c], sacc);
        S[rg] = sacc;
      }
      // ---- online softmax; lane holds keys t0 + 8*quad + j
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = tv + j;
        const float v = (j < 4 ? S[0][j] : S[1][j - 4]) * a.scale_log2;
        sc[j] = (tk >= r.lo && tk < seg1) ? v : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(sc[j] - m_use);
        psum += p[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const u32x4 pb = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma16x16x32(vop[dt], pb, acc[dt] * alpha);
    }
  }
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);

  // ---- merge the 4 waves in LDS
  if (qc < G) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[(w * G + qc) * D + 16 * dt + 4 * quad + i] = acc[dt][i];
  }
  if (quad == 0) {
    s_ml[w * 16 + qc] = m_run;
    s_ml[NW * 16 + w * 16 + qc] = l_run;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, s_ml[w2 * 16 + g]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float lsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const float f = fast_exp2(s_ml[w2 * 16 + g] - Mu);
      s_red[w2 * 16 + g] = f;
      lsum += f * s_ml[NW * 16 + w2 * 16 + g];
    }
    s_red[NW * 16 + g] = M;
    s_red[NW * 16 + 16 + g] = lsum;
  }
  __syncthreads();
  auto o_val = [&](int g, int d) {
    float o = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) o += s_red[w2 * 16 + g] * s_o[(w2 * G + g) * D + d];
    return o;
  };
  auto Mof = [&](int g) { return s_red[NW * 16 + g]; };
  auto Lof = [&](int g) { return s_red[NW * 16 + 16 + g]; };
  finish<D>(a, b, hk, s, o_val, Mof, Lof);
}

// ---------------------------------------------------------------------------
// head_dim >= 256: the 4 waves split head_dim; all walk the same chunks.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_dimsplit_kernel(DecodeArgs a) {
  constexpr int DW = D / kDecodeWaves;  // dims per wave
  __shared__ int s_pg[kSegPages];
  __shared__ f32x4 s_part[2][kDecodeWaves][2][64];  // [buffer][wave][rg][lane]
  __shared__ float s_o[kMaxGD];                     // [G][D] final unnormalised output
  __shared__ float s_ml[32];
  const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qc = lane & 15, quad = lane >> 4;
  const int G = a.G;
  const RowRange r = row_range(a, b, s);
  if (r.idle) {
    if (s == 0 || a.max_splits > 1) idle_output(a, b, hk, s, D);
    return;
  }
  if (r.start >= r.L) {
    empty_partial(a, b, hk, s);
    return;
  }
  if (a.k_new && r.end == r.L) append_new_token(a, r, b, hk, D);

  const int dw0 = w * DW;
  u32x4 qreg[DW / 32];  // loaded after the first page staging (see the key-split kernel)
  const bf16_t* qrow = a.q + ((size_t)b * a.n_q + hk * G + min(qc, G - 1)) * D + dw0 + 8 * quad;
  const int ps = a.g.page_size, log2ps = a.g.log2ps;
  const int32_t* trow = a.pt.table + (size_t)r.slot * a.pt.pps;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)a.g.n_kv * blk;
  const bf16_t* kbase = a.kpool + hk * blk + dw0;
  const bf16_t* vbase = a.vpool + hk * blk + (size_t)dw0 * ps;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[DW / 16];
#pragma unroll
  for (int i = 0; i < DW / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  int it = 0;
  const int seg_tokens = kSegPages * ps;
  for (int seg0 = r.start; seg0 < r.end; seg0 += seg_tokens) {
    const int seg1 = min(r.end, seg0 + seg_tokens);
    const int p0 = seg0 >> log2ps;
    __syncthreads();
    stage_pages(a, trow, p0, ((seg1 - 1) >> log2ps) - p0 + 1, s_pg);
    __syncthreads();
    if (seg0 == r.start) {
#pragma unroll
      for (int c = 0; c < DW / 32; ++c) {
        const u32x4 v = load16(qrow + 32 * c);
        qreg[c] = qc < G ? v : u32x4{0, 0, 0, 0};
      }
    }
    for (int t0 = seg0; t0 < seg1; t0 += 32, ++it) {
      u32x4 kop[2][DW / 32];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int tk = t0 + 8 * (qc >> 2) + 4 * rg + (qc & 3);
        const int page = tk < seg1 ? s_pg[(tk >> log2ps) - p0] : -1;
        const bf16_t* kp = kbase + (size_t)max(page, 0) * page_stride + (size_t)(tk & (ps - 1)) * D + 8 * quad;
#pragma unroll
        for (int c = 0; c < DW / 32; ++c) kop[rg][c] = page >= 0 ? load16(kp + 32 * c) : u32x4{0, 0, 0, 0};
      }
      const int tv = t0 + 8 * quad;
      const int vpage = tv < seg1 ? s_pg[(tv >> log2ps) - p0] : -1;
      const int nvalid = seg1 - tv;
      const bf16_t* vp = vbase + (size_t)max(vpage, 0) * page_stride + (size_t)qc * ps + (tv & (ps - 1));
      u32x4 vop[DW / 16];
#pragma unroll
      for (int dt = 0; dt < DW / 16; ++dt) {
        vop[dt] = vpage >= 0 ? load16(vp + (size_t)16 * dt * ps) : u32x4{0, 0, 0, 0};
        if (nvalid < 8) vop[dt] = keep_first(vop[dt], nvalid);
      }
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DW / 32; ++c) sacc = mfma16x16x32(kop[rg][c], qreg[c], sacc);
        s_part[it & 1][w][rg][lane] = sacc;
      }
      __syncthreads();
      f32x4 S[2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        f32x4 t = s_part[it & 1][0][rg][lane];
#pragma unroll
        for (int w2 = 1; w2 < kDecodeWaves; ++w2) t += s_part[it & 1][w2][rg][lane];
        S[rg] = t;
      }
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = tv + j;
        const float v = (j < 4 ? S[0][j] : S[1][j - 4]) * a.scale_log2;
        sc[j] = (tk >= r.lo && tk < seg1) ? v : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(sc[j] - m_use);
        psum += p[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const u32x4 pb = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
      for (int dt = 0; dt < DW / 16; ++dt) acc[dt] = mfma16x16x32(vop[dt], pb, acc[dt] * alpha);
    }
  }
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  // every wave holds the same (m, l); wave w owns output dims [dw0, dw0 + DW)
  if (qc < G) {
#pragma unroll
    for (int dt = 0; dt < DW / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[qc * D + dw0 + 16 * dt + 4 * quad + i] = acc[dt][i];
  }
  if (w == 0 && quad == 0) {
    s_ml[qc] = m_run;
    s_ml[16 + qc] = l_run;
  }
  __syncthreads();
  auto o_val = [&](int g, int d) { return s_o[g * D + d]; };
  auto Mof = [&](int g) { return s_ml[g]; };
  auto Lof = [&](int g) { return s_ml[16 + g]; };
  finish<D>(a, b, hk, s, o_val, Mof, Lof);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.max_splits, a.g.n_kv, a.B);
  if constexpr (D <= 128) {
    if (a.waves == 8)
      hipLaunchKernelGGL((decode_keysplit_kernel<D, 8>), grid, dim3(8 * 64),
                         (size_t)8 * a.G * D * sizeof(float), st, a);
    else
      hipLaunchKernelGGL((decode_keysplit_kernel<D, kDecodeWaves>), grid, dim3(kThreads),
                         (size_t)kDecodeWaves * a.G * D * sizeof(float), st, a);
  } else
    hipLaunchKernelGGL((decode_dimsplit_kernel<D>), grid, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.g.n_kv, a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int B, int n_q, int n_kv, int head_dim, int max_seq_len_hint,
                       int window) {
  DecodePlan p;
  const int G = n_q / n_kv;
  long range = max_seq_len_hint;
  if (window > 0 && (long)window + 31 < range) range = (long)window + 31;
  if (range < 1) range = 1;
  const long pairs = (long)B * n_kv;
  long split = 32 * kDecodeWaves;
  // About 2048 workgroups over the key ranges (8 per CU): enough to cover the
  // 256 CUs several times, few enough that the partials written and merged
  // stay small next to the K/V bytes.  The split count is also capped so the
  // merge weights of a (row, kv head) fit the 1024-float LDS buffer.
  while ((pairs * ((range + split - 1) / split) > 2048 ||
          ((range + split - 1) / split) * G > kMaxMergeWeights) &&
         split < (1 << 24))
    split *= 2;
  p.split_tokens = (int)split;
  p.max_splits = (int)((range + split - 1) / split);
  p.waves = kDecodeWaves;
  // (One 8-wave workgroup per pair without a split was measured slower than
  // split + merge even for 8 rows: 64 CUs stream ~16 GB/s each with
  // sequential chunks.  The 8-wave variant stays available to the launcher.)
  if (p.max_splits <= 1) {
    p.max_splits = 1;
    p.ws_bytes = 0;
    p.part_o_floats = 0;
    return p;
  }
  const size_t units = (size_t)B * n_kv * p.max_splits * G;
  p.part_o_floats = (units * head_dim + 63) & ~(size_t)63;
  p.ws_bytes = (p.part_o_floats + units * 2) * sizeof(float);
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.g.head_dim) {
    case 64: return launch_decode_d<64>(a, st);
    case 128: return launch_decode_d<128>(a, st);
    case 256: return launch_decode_d<256>(a, st);
    case 512: return launch_decode_d<512>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
