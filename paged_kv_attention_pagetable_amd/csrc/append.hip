// Append kernel: scatter new K/V rows into the paged pools (bit copy).
//
// K goes to the token-major K pool with one 16-byte store per 8 dims.  V goes
// to the V pool, d-major within 32-key groups: a workgroup stages 64
// consecutive tokens of one kv head in LDS and writes each V^T row segment
// with lanes on consecutive tokens, so runs of tokens that share a page (and
// a key group) become contiguous stores.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// Tokens staged per workgroup (keeps the V staging tile at <= 33 KB of LDS).
template <int D>
constexpr int append_tokens() { return D >= 512 ? 32 : 64; }

// Resolves the destination of token t: physical page and row, or -1.
__device__ __forceinline__ int dest_page(const AppendArgs& a, int t, int* row) {
  const int s = a.slot[t];
  const int p = a.pos[t];
  *row = 0;
  if (s <= 0 || s >= a.pt.max_slots || p < 0) return -1;
  const int lp = p >> a.g.log2ps;
  if (lp >= a.pt.pps) return -1;
  const int page = a.pt.table[(size_t)s * a.pt.pps + lp];
  if (page < 1 || page >= a.g.n_pages) return -1;
  *row = p & (a.g.page_size - 1);
  return page;
}

// grid = (ceil(T / NT), n_kv); block = 256.
template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int kAppendTokens = append_tokens<D>();
  __shared__ int s_page[kAppendTokens];
  __shared__ int s_row[kAppendTokens];
  __shared__ bf16_t s_v[kAppendTokens][D + 2];  // +2: odd dword stride, no bank conflicts
  const int t0 = blockIdx.x * kAppendTokens;
  const int h = blockIdx.y;
  const int nt = min(kAppendTokens, a.T - t0);
  const int tid = threadIdx.x;
  if (tid < nt) {
    int row;
    s_page[tid] = dest_page(a, t0 + tid, &row);
    s_row[tid] = row;
  }
  __syncthreads();
  const int n_kv = a.g.n_kv, ps = a.g.page_size;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)n_kv * blk;
  // K rows and V staging: 16 bytes per thread step.
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int i = tid; i < nt * CH; i += 256) {
    const int tt = i / CH, c = i - tt * CH;
    const size_t src = ((size_t)(t0 + tt) * n_kv + h) * D + 8 * c;
    const int page = s_page[tt];
    if (page >= 0) {
      const u32x4 kv = load16(a.k_new + src);
      store16(a.kpool + (size_t)page * page_stride + h * blk + (size_t)s_row[tt] * D + 8 * c, kv);
    }
    const u32x4 vv = load16(a.v_new + src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_v[tt][8 * c + 2 * e] = (bf16_t)(vv[e] & 0xffffu);
      s_v[tt][8 * c + 2 * e + 1] = (bf16_t)(vv[e] >> 16);
    }
  }
  __syncthreads();
  // V^T rows: thread -> (d, token); consecutive lanes take consecutive tokens.
  for (int i = tid; i < D * kAppendTokens; i += 256) {
    const int d = i / kAppendTokens, tt = i - d * kAppendTokens;
    if (tt >= nt) continue;
    const int page = s_page[tt];
    if (page < 0) continue;
    a.vpool[(size_t)page * page_stride + h * blk + v_elem_offset(d, s_row[tt], D, a.g.log2ps)] = s_v[tt][d];
  }
}

template <int D>
hipError_t launch_append_d(const AppendArgs& a, hipStream_t st) {
  constexpr int NT = append_tokens<D>();
  dim3 grid((a.T + NT - 1) / NT, a.g.n_kv);
  hipLaunchKernelGGL((append_kernel<D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  switch (a.g.head_dim) {
    case 64: return launch_append_d<64>(a, st);
    case 128: return launch_append_d<128>(a, st);
    case 256: return launch_append_d<256>(a, st);
    case 512: return launch_append_d<512>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
