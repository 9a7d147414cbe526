// Split-K paged decode attention for gfx950.
//
// One query token per batch row attends to its slot's keys 0..L-1 (window:
// the last W of them).  Grid = (split, kv head, batch row).  A workgroup of
// NW wave64s takes one contiguous key range of one (row, kv head); each wave
// walks 32-key chunks of it.  Per chunk the G query heads of the kv head are
// the 16 columns of bf16 MFMA tiles (G <= 16, unused columns are zero):
//
//   S^T[32 keys][16 q]  = K[32][D] . Q^T[D][16]        (2 x D/32 MFMA 16x16x32)
//   O^T[D][16 q]       += V^T[D][32 keys] . P^T[32][16] (D/16 MFMA 16x16x32)
//
// K rows come from the token-major K pool and V^T rows from the d-major V
// pool, both as 16-byte loads straight into the MFMA operand registers: the
// scores of a lane's 8 keys land exactly where the P.V product wants them, so
// no LDS round trip is needed inside the loop.  The online softmax keeps one
// running max / sum per query column (max reduced across the four lane
// groups with two xor shuffles).  Waves are merged in LDS, then either the
// final bf16 output is written (single split) or the unnormalised partial
// (o, max, sum) goes to the workspace for the log-sum-exp merge kernel.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kDecodeWaves = 4;

// Masks the bf16 elements e >= nvalid (0..8) of an 8-element operand.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nvalid) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t m = (2 * i < nvalid ? 0x0000ffffu : 0u) | (2 * i + 1 < nvalid ? 0xffff0000u : 0u);
    r[i] = v[i] & m;
  }
  return r;
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qc = lane & 15, quad = lane >> 4;
  const int G = a.G;
  const int ps = a.g.page_size;
  const int slot = a.slots[b];
  int L = a.seq_lens[b];
  const int cap = a.pt.pps * ps;
  const bool idle = slot <= 0 || slot >= a.pt.max_slots || L <= 0;
  if (idle) {
    if (a.max_splits == 1 && s == 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int g = idx / D, d = idx - g * D;
        a.out[((size_t)b * a.n_q + hk * G + g) * D + d] = 0;
        if (a.lse && d == 0) a.lse[(size_t)b * a.n_q + hk * G + g] = -INFINITY;
      }
    }
    return;
  }
  L = min(L, cap);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int base = lo & ~31;
  const int start = base + s * a.split_tokens;
  if (start >= L) return;
  const int end = (s == a.max_splits - 1) ? L : min(L, start + a.split_tokens);

  // Q^T operand: column qc = query head hk*G + qc, k-slots = 8 dims per lane group.
  u32x4 qreg[D / 32];
  {
    const bf16_t* qrow = a.q + ((size_t)b * a.n_q + hk * G + min(qc, G - 1)) * D + 8 * quad;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 v = load16(qrow + 32 * c);
      qreg[c] = qc < G ? v : u32x4{0, 0, 0, 0};
    }
  }

  const int32_t* trow = a.pt.table + (size_t)slot * a.pt.pps;
  const size_t blk = (size_t)ps * D;                  // one (page, head) block
  const size_t page_stride = (size_t)a.g.n_kv * blk;  // one page, all heads
  const bf16_t* kbase = a.kpool + hk * blk;
  const bf16_t* vbase = a.vpool + hk * blk;
  const int n_pages = a.g.n_pages, log2ps = a.g.log2ps;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = start + 32 * w; t0 < end; t0 += 32 * NW) {
    // ---- S^T = K Q^T for 32 keys: MFMA rg covers keys 8*(r/4) + 4*rg + r%4.
    f32x4 S[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int tk = t0 + 8 * (qc >> 2) + 4 * rg + (qc & 3);
      int page = -1;
      if (tk < end) page = trow[tk >> log2ps];
      const bool ok = page >= 1 && page < n_pages;
      const bf16_t* kp = kbase + (size_t)(ok ? page : 0) * page_stride +
                         (size_t)(tk & (ps - 1)) * D + 8 * quad;
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        u32x4 kv = ok ? load16(kp + 32 * c) : u32x4{0, 0, 0, 0};
        sacc = mfma16x16x32(kv, qreg[c], sacc);
      }
      S[rg] = sacc;
    }
    // ---- masked online softmax; lane holds keys t0 + 8*quad + j, j = 0..7.
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tk = t0 + 8 * quad + j;
      const float v = (j < 4 ? S[0][j] : S[1][j - 4]) * a.scale_log2;
      sc[j] = (tk >= lo && tk < end) ? v : -INFINITY;
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
    // ---- O^T += V^T P^T; lane reads V^T row d = 16*dt + qc, keys tv..tv+7.
    const int tv = t0 + 8 * quad;
    int vpage = -1;
    if (tv < end) vpage = trow[tv >> log2ps];
    const bool vok = vpage >= 1 && vpage < n_pages;
    const int nvalid = end - tv;
    const bf16_t* vp = vbase + (size_t)(vok ? vpage : 0) * page_stride + (size_t)qc * ps +
                       (tv & (ps - 1));
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      u32x4 vv = vok ? load16(vp + (size_t)16 * dt * ps) : u32x4{0, 0, 0, 0};
      if (nvalid < 8) vv = keep_first(vv, nvalid);
      acc[dt] = acc[dt] * alpha;
      acc[dt] = mfma16x16x32(vv, pb, acc[dt]);
    }
  }
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);

  // ---- merge the NW waves of this workgroup in LDS.
  float* sm_o = smem;                     // [NW][G][D]
  float* sm_m = smem + (size_t)NW * G * D;  // [NW][16]
  float* sm_l = sm_m + NW * 16;           // [NW][16]
  if (qc < G) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[((size_t)w * G + qc) * D + 16 * dt + 4 * quad + r] = acc[dt][r];
  }
  if (quad == 0) {
    sm_m[w * 16 + qc] = m_run;
    sm_l[w * 16 + qc] = l_run;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D, d = idx - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, sm_m[w2 * 16 + g]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const float f = fast_exp2(sm_m[w2 * 16 + g] - Mu);
      lsum += f * sm_l[w2 * 16 + g];
      o += f * sm_o[((size_t)w2 * G + g) * D + d];
    }
    if (a.max_splits == 1) {
      a.out[((size_t)b * a.n_q + hk * G + g) * D + d] = f32_to_bf16(lsum > 0.f ? o / lsum : 0.f);
      if (a.lse && d == 0)
        a.lse[(size_t)b * a.n_q + hk * G + g] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
    } else {
      const size_t pidx = (((size_t)b * a.g.n_kv + hk) * a.max_splits + s) * G + g;
      a.part_o[pidx * D + d] = o;
      if (d == 0) {
        a.part_ml[pidx * 2] = M;
        a.part_ml[pidx * 2 + 1] = lsum;
      }
    }
  }
}

// Log-sum-exp merge of the split partials of one (row, kv head).
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int hk = blockIdx.x, b = blockIdx.y;
  const int G = a.G;
  const int slot = a.slots[b];
  int L = a.seq_lens[b];
  const int cap = a.pt.pps * a.g.page_size;
  const bool idle = slot <= 0 || slot >= a.pt.max_slots || L <= 0;
  int n_valid = 0;
  if (!idle) {
    L = min(L, cap);
    const int lo = a.window > 0 ? max(0, L - a.window) : 0;
    const int base = lo & ~31;
    n_valid = min(a.max_splits, (L - base + a.split_tokens - 1) / a.split_tokens);
  }
  const size_t pbase = ((size_t)b * a.g.n_kv + hk) * a.max_splits;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D, d = idx - g * D;
    float M = -INFINITY;
    for (int s = 0; s < n_valid; ++s) M = fmaxf(M, a.part_ml[((pbase + s) * G + g) * 2]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float lsum = 0.f, o = 0.f;
    for (int s = 0; s < n_valid; ++s) {
      const size_t pi = (pbase + s) * G + g;
      const float f = fast_exp2(a.part_ml[pi * 2] - Mu);
      lsum += f * a.part_ml[pi * 2 + 1];
      o += f * a.part_o[pi * D + d];
    }
    a.out[((size_t)b * a.n_q + hk * G + g) * D + d] = f32_to_bf16(lsum > 0.f ? o / lsum : 0.f);
    if (a.lse && d == 0)
      a.lse[(size_t)b * a.n_q + hk * G + g] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  constexpr int NW = kDecodeWaves;
  const size_t lds = ((size_t)NW * a.G * D + 2 * NW * 16) * sizeof(float);
  dim3 grid(a.max_splits, a.g.n_kv, a.B);
  hipLaunchKernelGGL((decode_split_kernel<D, NW>), grid, dim3(NW * 64), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.g.n_kv, a.B), dim3(256), 0, st, a);
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
  // Aim for about 2048 workgroups over the key ranges (8 per CU): enough to
  // cover 256 CUs with several waves each, few enough to keep the partials
  // (written and re-read by the merge) small next to the K/V bytes.
  while (pairs * ((range + split - 1) / split) > 2048 && split < (1 << 20)) split *= 2;
  p.split_tokens = (int)split;
  p.max_splits = (int)((range + split - 1) / split);
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
