// Device-side batch reserve: the pages' PageTable.reserve
// ([continuous-batching compare] flex_paged_attention.py) applied to B rows
// in order on the device, so a decode step can grow its slots without a host
// round trip.  Row b needs k_b = ceil((len_b - cap_b) / page_size) pages and,
// served in order from the top of the free stack, takes entries
// [fc - incl_b, fc - incl_b + k_b) (incl_b = k_0 + .. + k_b, fc = the stack's
// length before the tile) as its next logical pages: an inclusive scan of the
// k_b gives every row its range at once.  When a tile's rows do not all fit,
// one thread serves them one by one instead, so that a row that does not fit
// is skipped and later smaller rows still proceed, as successive host calls
// would.  One workgroup; each tile of 256 rows sees the previous tiles'
// grants.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kResThreads = 256;

__global__ __launch_bounds__(kResThreads) void reserve_kernel(ReserveArgs a) {
  __shared__ int s_scan[kResThreads];
  __shared__ int s_slot[kResThreads], s_cap[kResThreads], s_need[kResThreads];
  __shared__ int s_fc;
  const int tid = threadIdx.x;
  const int ps = a.page_size;
  int fc = min(max(*a.free_count, 0), a.n_pages);
  for (int t0 = 0; t0 < a.B; t0 += kResThreads) {
    const int b = t0 + tid;
    int slot = -1, cap = 0, need = 0;
    uint32_t flag = 0;
    if (b < a.B) {
      const int sl = a.slots[b], len = a.seq_lens[b];
      if (sl >= 1 && sl < a.max_slots) {
        const int c = a.capacity[sl];
        if (c < 0 || c % ps != 0 || c / ps > a.pps) {
          flag = kReserveBadState;
        } else if (len > c) {
          const long k = ((long)len - c + ps - 1) / ps;
          if (c / ps + k > a.pps) {
            flag = kReserveTooLong;
          } else {
            slot = sl;
            cap = c;
            need = (int)k;
          }
        }
      }
    }
    // inclusive scan of the tile's page needs
    s_scan[tid] = need;
    __syncthreads();
    for (int off = 1; off < kResThreads; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int incl = s_scan[tid], total = s_scan[kResThreads - 1];
    if (total <= fc) {
      for (int i = 0; i < need; ++i) a.table[(size_t)slot * a.pps + cap / ps + i] = a.free_pages[fc - incl + i];
      if (need > 0) a.capacity[slot] = cap + need * ps;
      fc -= total;
    } else {
      s_slot[tid] = slot;
      s_cap[tid] = cap;
      s_need[tid] = need;
      __syncthreads();
      if (tid == 0) {
        uint32_t f0 = 0;
        for (int r = 0; r < kResThreads; ++r) {
          const int k = s_need[r];
          if (k == 0) continue;
          if (k > fc) {
            f0 |= kReserveNoPages;
            continue;
          }
          const int sl = s_slot[r], c = s_cap[r];
          for (int i = 0; i < k; ++i) a.table[(size_t)sl * a.pps + c / ps + i] = a.free_pages[fc - k + i];
          a.capacity[sl] = c + k * ps;
          fc -= k;
        }
        s_fc = fc;
        if (f0) atomicOr(a.status, f0);
      }
      __syncthreads();
      fc = s_fc;
    }
    if (flag) atomicOr(a.status, flag);
    __syncthreads();  // s_scan and the row arrays are reused by the next tile
  }
  if (tid == 0) *a.free_count = fc;
}

}  // namespace

hipError_t launch_reserve(const ReserveArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(reserve_kernel, dim3(1), dim3(kResThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
