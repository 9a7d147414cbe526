// Fused Qwen3 prefill prologue: per token and head, RMSNorm over head_dim
// with a gain, then half-split rotary embedding; q is rewritten in place, the
// new k and the raw v are appended to the pages.
//
// Row layout: D/8 lanes hold one head row, 8 dims (16 bytes) each.  The
// rotate_half partner of dims 8c..8c+7 lives in lane c ^ (D/16) of the same
// row group, and the mean of squares is a xor-shuffle reduction over the
// row's lanes.  All arithmetic is fp32; each output is rounded to bf16 once.
// grid = (ceil(T / 64), n_q + n_kv); y < n_q handles q head y, otherwise kv
// head y - n_q (k rows and the V^T staging / store, as in the append kernel).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kProTokens = 64;

template <int D>
__device__ __forceinline__ u32x4 norm_rope_row(u32x4 x, const bf16_t* w, const float* cos_row,
                                               const float* sin_row, int c, float eps) {
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
  const int f0 = (8 * c) & (D / 2 - 1);
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float o[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = 2 * e + k;
      const float rot = first_half ? -pr[j] : pr[j];
      o[k] = v[j] * cos_row[f0 + j] + rot * sin_row[f0 + j];
    }
    out[e] = pack_bf16x2(o[0], o[1]);
  }
  return out;
}

template <int D>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  constexpr int LPR = D / 8;
  constexpr int ROWS = 256 / LPR;  // rows processed per pass by the workgroup
  __shared__ int s_page[kProTokens];
  __shared__ int s_row[kProTokens];
  __shared__ int s_pos[kProTokens];
  __shared__ bf16_t s_v[kProTokens][D + 2];
  const int t0 = blockIdx.x * kProTokens;
  const int hh = blockIdx.y;
  const int nt = min(kProTokens, a.T - t0);
  const int tid = threadIdx.x;
  const int n_kv = a.g.n_kv, ps = a.g.page_size;
  if (tid < nt) {
    const int t = t0 + tid;
    // sequence of token t: last n with cu_seqlens[n] <= t
    int lo = 0, hi = a.n_seqs;  // invariant: cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
    }
    const int slot = a.slots[lo];
    const int pos = (a.start_pos ? a.start_pos[lo] : 0) + (t - a.cu_seqlens[lo]);
    int page = -1, row = 0;
    bool ok = slot > 0 && slot < a.pt.max_slots && pos >= 0 && pos < a.max_pos;
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
    s_page[tid] = page;
    s_row[tid] = row;
    s_pos[tid] = ok ? pos : -1;
  }
  __syncthreads();
  const int c = tid % LPR;
  const int rsub = tid / LPR;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)n_kv * blk;
  if (hh < a.n_q) {
    for (int tt = rsub; tt < nt; tt += ROWS) {
      const int pos = s_pos[tt];
      if (pos < 0) continue;  // uniform over the row's lanes
      bf16_t* row = a.q + ((size_t)(t0 + tt) * a.n_q + hh) * D;
      const u32x4 x = load16(row + 8 * c);
      const u32x4 y = norm_rope_row<D>(x, a.q_w, a.cos_t + (size_t)pos * (D / 2),
                                       a.sin_t + (size_t)pos * (D / 2), c, a.eps);
      store16(row + 8 * c, y);
    }
    return;
  }
  const int h = hh - a.n_q;
  for (int tt = rsub; tt < nt; tt += ROWS) {
    const int pos = s_pos[tt];
    const int page = s_page[tt];
    const size_t src = ((size_t)(t0 + tt) * n_kv + h) * D + 8 * c;
    if (pos >= 0 && page >= 0) {
      const u32x4 x = load16(a.k_raw + src);
      const u32x4 y = norm_rope_row<D>(x, a.k_w, a.cos_t + (size_t)pos * (D / 2),
                                       a.sin_t + (size_t)pos * (D / 2), c, a.eps);
      store16(a.kpool + (size_t)page * page_stride + h * blk + (size_t)s_row[tt] * D + 8 * c, y);
    }
    const u32x4 vv = load16(a.v_raw + src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_v[tt][8 * c + 2 * e] = (bf16_t)(vv[e] & 0xffffu);
      s_v[tt][8 * c + 2 * e + 1] = (bf16_t)(vv[e] >> 16);
    }
  }
  __syncthreads();
  for (int i = tid; i < D * kProTokens; i += 256) {
    const int d = i / kProTokens, tt = i - d * kProTokens;
    if (tt >= nt) continue;
    const int page = s_page[tt];
    if (page < 0 || s_pos[tt] < 0) continue;
    a.vpool[(size_t)page * page_stride + h * blk + v_elem_offset(d, s_row[tt], D, a.g.log2ps)] = s_v[tt][d];
  }
}

template <int D>
hipError_t launch_prologue_d(const PrologueArgs& a, hipStream_t st) {
  dim3 grid((a.T + kProTokens - 1) / kProTokens, a.n_q + a.g.n_kv);
  hipLaunchKernelGGL((prologue_kernel<D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// cos / sin of p * theta^(-2i/D) in fp64, stored as fp32.
__global__ void rope_table_kernel(float* c, float* s, int max_pos, int half, double theta,
                                  int head_dim) {
  const long n = (long)max_pos * half;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < n;
       idx += (long)gridDim.x * blockDim.x) {
    const int p = (int)(idx / half), i = (int)(idx - (long)p * half);
    const double inv = pow(theta, -2.0 * (double)i / (double)head_dim);
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
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope_table(float* c, float* s, int max_pos, int head_dim, double theta,
                             hipStream_t st) {
  const int half = head_dim / 2;
  const long n = (long)max_pos * half;
  if (n <= 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, st, c, s, max_pos, half,
                     theta, head_dim);
  return hipGetLastError();
}

}  // namespace pkv
