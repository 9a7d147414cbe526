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
//
// Device-side batch erase: the pages' PageTable.erase applied to B rows in
// order.  Row b's slot owns n_b = capacity / page_size pages (its first n_b
// table entries); they go back on the free stack in reverse logical order,
// after the pages of rows 0 .. b-1, so an exclusive scan of the n_b places
// every row at once.  The slot's capacity becomes 0 and its row -1, the reset
// the host allocate would do, so the host may hand the slot out again with no
// further device call.  Scans run in 64 bits: 256 rows of up to 2^30 pages
// would overflow 32.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kResThreads = 256;

__global__ __launch_bounds__(kResThreads) void reserve_kernel(ReserveArgs a) {
  __shared__ long long s_scan[kResThreads];
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
      const long long v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const long long incl = s_scan[tid], total = s_scan[kResThreads - 1];
    if (total <= fc) {
      const int first = fc - (int)incl;  // 0 <= first and first + need <= fc
      for (int i = 0; i < need; ++i) a.table[(size_t)slot * a.pps + cap / ps + i] = a.free_pages[first + i];
      if (need > 0) a.capacity[slot] = cap + need * ps;
      fc -= (int)total;
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

__global__ __launch_bounds__(kResThreads) void erase_kernel(ReserveArgs a) {
  __shared__ long long s_scan[kResThreads];
  __shared__ int s_slot[kResThreads], s_n[kResThreads];
  __shared__ int s_fc;
  const int tid = threadIdx.x;
  const int ps = a.page_size;
  int fc = min(max(*a.free_count, 0), a.n_pages);
  for (int t0 = 0; t0 < a.B; t0 += kResThreads) {
    const int b = t0 + tid;
    int slot = -1, n = 0;
    uint32_t flag = 0;
    if (b < a.B) {
      const int sl = a.slots[b];
      if (sl >= 1 && sl < a.max_slots) {
        const int c = a.capacity[sl];
        if (c < 0 || c % ps != 0 || c / ps > a.pps) {
          flag = kReserveBadState;
        } else {
          slot = sl;
          n = c / ps;
        }
      }
    }
    s_scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < kResThreads; off <<= 1) {
      const long long v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const long long incl = s_scan[tid], total = s_scan[kResThreads - 1];
    if (fc + total <= a.n_pages) {
      // the stack has room for every row's pages: each thread pushes its own
      const int first = fc + (int)(incl - n);
      const int* row = a.table + (size_t)(slot > 0 ? slot : 0) * a.pps;
      for (int i = 0; i < n; ++i) a.free_pages[first + i] = row[n - 1 - i];
      fc += (int)total;
      s_slot[tid] = slot;
    } else {
      // more pages than the stack can hold (an inconsistent state): serve the
      // rows one by one and skip, with a flag, those that do not fit
      s_slot[tid] = slot;
      s_n[tid] = n;
      __syncthreads();
      if (tid == 0) {
        uint32_t f0 = 0;
        for (int r = 0; r < kResThreads; ++r) {
          const int sl = s_slot[r], k = s_n[r];
          if (sl < 1) continue;
          if (fc + k > a.n_pages) {
            f0 |= kReserveBadState;
            s_slot[r] = -1;
            continue;
          }
          const int* row = a.table + (size_t)sl * a.pps;
          for (int i = 0; i < k; ++i) a.free_pages[fc + i] = row[k - 1 - i];
          fc += k;
        }
        s_fc = fc;
        if (f0) atomicOr(a.status, f0);
      }
      __syncthreads();
      fc = s_fc;
    }
    if (flag) atomicOr(a.status, flag);
    __syncthreads();  // every page id has been read before rows are reset
    const int rows = min(kResThreads, a.B - t0);
    for (int r = 0; r < rows; ++r) {
      const int sl = s_slot[r];
      if (sl < 1) continue;
      for (int j = tid; j < a.pps; j += kResThreads) a.table[(size_t)sl * a.pps + j] = -1;
      if (tid == 0) a.capacity[sl] = 0;
    }
    __syncthreads();  // s_scan and s_slot are reused by the next tile
  }
  if (tid == 0) *a.free_count = fc;
}

}  // namespace

hipError_t launch_erase(const ReserveArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(erase_kernel, dim3(1), dim3(kResThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_reserve(const ReserveArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(reserve_kernel, dim3(1), dim3(kResThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
