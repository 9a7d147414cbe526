// Validation mode: device-side checks of the metadata a call is about to use
// (slots, positions, page-table entries), enqueued before the call's kernels.
// Findings are OR-ed into a per-device flag word that the host reads back
// with pkv_validation_flags.  The calls themselves run unchanged: the kernels
// already treat such inputs as absent keys / skipped tokens, in bounds.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

__device__ uint32_t g_validate_flags;  // zero at load

// Pages [0, n_tok / ps) (rounded up) of `slot` must be mapped.
__device__ __forceinline__ uint32_t check_pages(const TableRef& pt, const PoolGeom& g, int slot,
                                                long n_tok) {
  const long cap = (long)pt.pps * g.page_size;
  uint32_t f = 0;
  if (n_tok > cap) {
    f |= kValidatePos;
    n_tok = cap;
  }
  const int np = (int)((n_tok + g.page_size - 1) >> g.log2ps);
  const int32_t* row = pt.table + (size_t)slot * pt.pps;
  for (int p = 0; p < np; ++p) {
    const int pg = row[p];
    if (pg < 1 || pg >= g.n_pages) {
      f |= kValidatePage;
      break;
    }
  }
  return f;
}

__device__ __forceinline__ void report(uint32_t f) {
  if (f) atomicOr(&g_validate_flags, f);
}

// One thread per batch row (decode) or per sequence (prefill): keys
// 0 .. len-1 of the row's slot.
__global__ void validate_rows_kernel(TableRef pt, PoolGeom g, const int32_t* slots,
                                     const int32_t* seq_lens, const int32_t* cu_seqlens,
                                     const int32_t* start_pos, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int slot = slots[i];
  long len;
  uint32_t f = 0;
  if (seq_lens) {
    len = seq_lens[i];
    if (len < 0) f |= kValidatePos;
  } else {
    const long sp = start_pos ? start_pos[i] : 0;
    const long q = (long)cu_seqlens[i + 1] - cu_seqlens[i];
    if (sp < 0 || q < 0) f |= kValidatePos;
    len = sp + q;
  }
  if (slot == 0 || len <= 0) {  // padding / idle row: nothing is used
    report(f);
    return;
  }
  if (slot < 0 || slot >= pt.max_slots) {
    report(f | kValidateSlot);
    return;
  }
  report(f | check_pages(pt, g, slot, len));
}

// One thread per appended token: its (slot, pos) must address a mapped page.
__global__ void validate_tokens_kernel(TableRef pt, PoolGeom g, const int32_t* slot,
                                       const int32_t* pos, int T) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int s = slot[t];
  if (s == 0) return;  // the reserved no-op slot
  if (s < 0 || s >= pt.max_slots) {
    report(kValidateSlot);
    return;
  }
  const int p = pos[t];
  if (p < 0 || (long)p >= (long)pt.pps * g.page_size) {
    report(kValidatePos);
    return;
  }
  const int pg = pt.table[(size_t)s * pt.pps + (p >> g.log2ps)];
  if (pg < 1 || pg >= g.n_pages) report(kValidatePage);
}

__global__ void validate_clear_kernel() {
  if (threadIdx.x == 0) atomicAnd(&g_validate_flags, 0u);
}

}  // namespace

hipError_t launch_validate_rows(const TableRef& pt, const PoolGeom& g, const int32_t* slots,
                                const int32_t* seq_lens, const int32_t* cu_seqlens,
                                const int32_t* start_pos, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(validate_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, st, pt, g, slots,
                     seq_lens, cu_seqlens, start_pos, n);
  return hipGetLastError();
}

hipError_t launch_validate_tokens(const TableRef& pt, const PoolGeom& g, const int32_t* slot,
                                  const int32_t* pos, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(validate_tokens_kernel, dim3((T + 255) / 256), dim3(256), 0, st, pt, g, slot,
                     pos, T);
  return hipGetLastError();
}

// Copies the flag word to host memory once the stream's earlier work is done
// (synchronises the stream), then optionally enqueues its clearing.
hipError_t read_validate_flags(uint32_t* host_out, int clear, hipStream_t st) {
  hipError_t e = hipMemcpyFromSymbolAsync(host_out, HIP_SYMBOL(g_validate_flags), sizeof(uint32_t), 0,
                                          hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && clear) {
    hipLaunchKernelGGL(validate_clear_kernel, dim3(1), dim3(64), 0, st);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
