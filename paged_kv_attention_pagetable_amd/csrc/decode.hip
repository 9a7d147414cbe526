// Split-K paged decode attention for gfx950 (one kernel per call).
//
// One query token per batch row attends to its slot's keys 0..L-1 (window:
// the last W of them).  Grid = (kv head, batch row, split); a workgroup of 4
// wave64s owns one contiguous key range of one (row, kv head).  Keys are
// processed in 32-key chunks on bf16 MFMA 16x16x32 tiles whose 16 columns are
// the G query heads of the kv head (G <= 16, unused columns are zero):
//
//   S^T[32 keys][16 q]  = K[32][D] . Q^T[D][16]
//   O^T[D][16 q]       += V^T[D][32 keys] . P^T[32][16]
//
// V^T rows come from the V pool (d-major within 32-key groups, so one wave's
// 32 keys of V are one contiguous block) as 16-byte loads straight into MFMA
// operand registers; a lane's 8 key scores land exactly in its P^T k-slots, so
// no LDS round trip is needed for P.  An MFMA operand load of K would touch 16
// key rows at 64 bytes each; instead (head_dim <= 128) each wave copies its 32
// K rows -- one contiguous block of the token-major K pool -- into its own LDS
// slice with global-to-LDS loads of 1 KB each, XOR-swizzled so that the
// operand reads from LDS are free of bank conflicts (measured 9 % less time
// for the loads alone on the ragged Llama batch).  The physical page ids of the workgroup's range are read once into LDS,
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
// goes to the workspace and the last workgroup of the (row, kv head) to
// arrive merges them, in fixed split order (bitwise deterministic whichever
// workgroup merges).  The arrival counters live in the caller's workspace
// too (its last bytes), so calls with separate workspaces never share
// state.  The partials are written and read with device-scope relaxed atomic
// accesses (sc1: coherent across the XCDs' L2s), each writer waits for its
// stores to complete before it counts itself in, and the counter wraps to
// zero on the last arrival -- no release fence, which on gfx950 would write
// back the whole L2 per workgroup (see finish).  Optionally the new token's
// K/V is appended first by the workgroup that owns the last key.
#include <algorithm>
#include <mutex>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kDecodeWaves = 4;
constexpr int kThreads = kDecodeWaves * 64;
constexpr int kSegPages = 64;  // page ids staged in LDS per range segment
constexpr int kMaxGD = 2048;   // (query heads per kv head) * head_dim, checked on the host
constexpr int kMaxMergeUnits = 1024;  // cap on splits * G of one (row, kv head): bounds one merge

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

typedef __attribute__((address_space(3))) void* lds_void_ptr;
// Cache-policy operand of the global-to-LDS copies: non-temporal (K and V
// are read once per call).
constexpr int kNtAux = 2;

// K stage of a wave (head_dim <= 128): 32 key rows of D bf16.  Row r keeps
// its 16-byte unit u at slot u ^ kst_swz(r); for the 16 rows of one MFMA
// operand read (keys 8*(m/4) + 4*rg + m%4) the slots land in 16 distinct
// 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kst_swz(int r) {
  return D == 64 ? (((r >> 1) & 1) | (((r >> 3) & 3) << 1)) : ((r & 3) | (((r >> 3) & 3) << 2));
}

struct RowRange {
  int slot, L, lo, start, end, n_valid;
  int L_in;  // seq_lens[b] as given (L is clamped to the slot's table capacity)
  bool idle;
};

__device__ __forceinline__ RowRange row_range(const DecodeArgs& a, int b, int s,
                                               const int32_t* slots, const int32_t* seq_lens) {
  RowRange r;
  r.slot = slots[b];
  r.L = seq_lens[b];
  r.L_in = r.L;
  r.idle = r.slot <= 0 || r.slot >= a.pt.max_slots || r.L <= 0;
  r.lo = r.start = r.end = r.n_valid = 0;
  if (r.idle) return r;
  r.L = min(r.L, a.pt.pps * a.g.page_size);
  r.lo = a.window > 0 ? max(0, r.L - a.window) : 0;
  const int base = r.lo & ~31;
  const int span = r.L - base;
  if (r.lo > 0) {  // (a sliding window that cuts the row)
    r.n_valid = min(a.max_splits, (span + a.split_tokens - 1) / a.split_tokens);
    // Sliding window: split 0 takes the range's remainder (span - (n_valid -
    // 1) full splits, rounded up to whole 32-key chunks; beyond max_splits
    // splits it absorbs the excess), splits 1 .. full split_tokens after it.
    // A window range is about one window long, so the remainder is a sliver
    // of keys; as split 0 it is the last workgroup of its row to start
    // instead of the first (measured 7 % faster on the Gemma sliding layers;
    // on full-causal rows the plain layout below measured 1-3 % faster).
    const int first = (span - (r.n_valid - 1) * a.split_tokens + 31) & ~31;
    r.start = s == 0 ? base : base + first + (s - 1) * a.split_tokens;
    r.end = min(r.L, s == 0 ? base + first : r.start + a.split_tokens);
  } else {
    // Full causal (or a window that cuts nothing: the same splits, so the
    // result is bit for bit the unwindowed one): split 0 takes the first
    // head_tokens keys, splits 1 .. split_tokens each after it; the last split
    // of the grid also takes any keys beyond max_splits splits (a length above
    // the plan's hint).
    const int hs = a.head_tokens;
    r.n_valid = min(a.max_splits, span <= hs ? 1 : (span - hs + 2 * a.split_tokens - 1) / a.split_tokens);
    r.start = s == 0 ? base : base + hs + (s - 1) * a.split_tokens;
    r.end = (s == a.max_splits - 1) ? r.L : min(r.L, r.start + (s == 0 ? hs : a.split_tokens));
  }
  return r;
}

// Fused append (k_new / v_new given).  The workgroup whose key range ends at
// the row's last key L-1 owns the new token of (b, hk), at position
// seq_lens[b] - 1 as pkv_append would place it; a position past the slot's
// table (a length beyond its capacity, a caller error) is skipped, never
// folded onto the last row of the table.  The token never makes a round trip
// through the pool inside the call:
//   - its K and V rows are loaded into registers when the workgroup starts
//     (NewTok::load), overlapping the row's slot and length loads, and moved
//     to LDS with the first page staging (NewTok::stage);
//   - the chunk holding key L-1 takes them from there: the K row into the
//     wave's stage once its copies have landed, the V values into the MFMA
//     operand registers (NewTok::patch), so the operands are bit for bit what
//     a read of the appended pool would give;
//   - V (page size >= 32): that chunk loads its whole 32-key group of V
//     unmasked (the lanes past the last key address the same page), takes
//     the new key in, and writes the group's 64-byte rows back whole
//     (NewTok::store_v_rows) before masking the operands.  In the d-major V
//     layout the new token touches one row segment per dim: 128 write
//     bursts per (row, kv head) at head_dim 128, where its K row is two
//     lines.  Entering HBM while the grid saturates it with reads, these
//     cost about 4 us of the Llama call, in any form (whole rows, 2-byte
//     stores, write-through; no extra reads by the counters).  On large
//     grids (v_late) the owner skips the write and split 0 -- the last
//     layer of the grid, which runs in its drain -- stores the 2-byte values
//     at its end instead (NewTok::store_late; Llama shape 100.8 -> 99.5 us).
//     It fetches the page id and its values when it starts.  On small grids
//     that store sat on the call's last round trips (Qwen3 +0.6 us).
//   - K (and V for smaller pages): written after the split's result
//     (NewTok::store), where no later wait of the workgroup depends on them.
//     (Written first, the stores sat in front of every chunk load in the
//     in-order memory counter; written last with their own loads, the
//     dependent round trips lengthened the appending workgroups instead.)
// v is kept per wave slice of DW dims as [lane % 16][dt]: the eight V values
// a patching lane needs (dims d0 + 16*dt + lane%16) are one 16-byte read.
template <int D>
struct NewTokLds {
  bf16_t k[D];
  bf16_t v[D];
};
template <int DW>
__device__ __forceinline__ int newtok_v_index(int d) {
  const int rem = d % DW;
  return d - rem + (rem % 16) * (DW / 16) + rem / 16;
}

// VL: split 0 writes the new V at its end (the plan's v_late; key-split
// kernel, page size >= 32); the owner then leaves it out of the pool.
template <int D, bool VL = false>
struct NewTok {
  static constexpr int kNV = (D + 255) / 256;  // v values per thread (>= 256 threads)
  bool on = false;    // this workgroup appends (uniform)
  bool late = false;  // this workgroup (split 0, v_late) writes the new V at its end
  int page = -1;      // physical page of key L-1, -1 if unmapped (then nothing is written)
  int late_page = -1;
  u32x4 k{0, 0, 0, 0};
  bf16_t v[kNV] = {};

  __device__ __forceinline__ void load(const DecodeArgs& a, const RowRange& r, int b, int hk, int s,
                                       const int32_t* table) {
    const bool fits = a.k_new && ((r.L_in - 1) >> a.g.log2ps) < a.pt.pps;
    on = fits && r.end == r.L;
    late = VL && fits && s == 0 && a.g.page_size >= 32;
    if (!on && !late) return;
    const size_t src = ((size_t)b * a.g.n_kv + hk) * D;
    if (on && (int)threadIdx.x < D / 8) k = load16(a.k_new + src + 8 * threadIdx.x);
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const int d = threadIdx.x + 256 * i;
      if (d < D) v[i] = a.v_new[src + d];
    }
    if (late) {
      const int pg = table[(size_t)r.slot * a.pt.pps + ((r.L - 1) >> a.g.log2ps)];
      late_page = (pg >= 1 && pg < a.g.n_pages) ? pg : -1;
    }
  }
  // During the first page staging (a barrier follows); DW = the dims of a
  // wave's slice (D for the key-split kernel).
  template <int DW>
  __device__ __forceinline__ void stage(NewTokLds<D>& L) const {
    if (!on) return;
    if ((int)threadIdx.x < D / 8) store16(L.k + 8 * threadIdx.x, k);
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const int d = threadIdx.x + 256 * i;
      if (d < D) L.v[newtok_v_index<DW>(d)] = v[i];
    }
  }
  // After the staging of the segment that ends the range (s_pg of it).
  __device__ __forceinline__ void find_page(const RowRange& r, int log2ps, int p0, const int* s_pg) {
    if (on) page = __builtin_amdgcn_readfirstlane(s_pg[((r.L - 1) >> log2ps) - p0]);
  }
  // Whether the chunk at t0 holds the new key (and the key is on a page).
  __device__ __forceinline__ bool in_chunk(const RowRange& r, int t0) const {
    return on && page >= 0 && t0 == ((r.L - 1) & ~31);
  }
  // The wave's K stage row and V operands of the chunk at t0: dims [d0, d0 +
  // DW) of the key, stage rows of 2*DW bytes swizzled by kst_swz<DW>, V^T rows
  // d0 + 16*dt + (lane%16) holding keys t0 + 8*(lane/16) ...
  template <int DW, class SWZ>
  __device__ __forceinline__ void patch(const RowRange& r, int t0, int d0, uint8_t* kst, SWZ swz,
                                        const NewTokLds<D>& L, u32x4 (&vop)[DW / 16]) const {
    const int lane = threadIdx.x & 63, qc = lane & 15, quad = lane >> 4;
    const int rr = r.L - 1 - t0;
    for (int c = lane; c < DW / 8; c += 64)
      store16(kst + rr * (2 * DW) + 16 * (c ^ swz(rr)), load16(L.k + d0 + 8 * c));
    if (quad == (rr >> 3)) {
      const int e = rr & 7;
      bf16_t xs[DW / 16];
      static_assert(DW / 16 == 8 || DW / 16 == 4, "one 16- or 8-byte read");
      if constexpr (DW / 16 == 8)
        *reinterpret_cast<u32x4*>(xs) = load16(L.v + d0 + qc * (DW / 16));
      else
        *reinterpret_cast<uint64_t*>(xs) = *reinterpret_cast<const uint64_t*>(L.v + d0 + qc * (DW / 16));
#pragma unroll
      for (int dt = 0; dt < DW / 16; ++dt) {
        const uint32_t x = xs[dt];
        u32x4 o = vop[dt];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (e == 2 * h) o[h] = (o[h] & 0xffff0000u) | x;
          if (e == 2 * h + 1) o[h] = (o[h] & 0x0000ffffu) | (x << 16);
        }
        vop[dt] = o;
      }
    }
  }
  // After the split's result: the pool rows.
  template <int DW>
  __device__ __forceinline__ void store(const DecodeArgs& a, const RowRange& r, int hk,
                                        const NewTokLds<D>& L) const {
    if (!on || page < 0) return;
    const int ps = a.g.page_size;
    const size_t blk = (size_t)ps * D;
    const size_t dst = (size_t)page * a.g.n_kv * blk + hk * blk;
    const int row = (r.L - 1) & (ps - 1);
    for (int i = threadIdx.x; i < D / 8; i += blockDim.x)
      store16(a.kpool_w + dst + (size_t)row * D + 8 * i, load16(L.k + 8 * i));
    if (ps >= 32) return;  // V went out whole with its chunk (store_v_rows)
    for (int d = threadIdx.x; d < D; d += blockDim.x)
      a.vpool_w[dst + v_elem_offset(d, row, D, a.g.log2ps)] = L.v[newtok_v_index<DW>(d)];
  }
  // v_late, split 0 at its end: the new V, one 2-byte store per dim.
  __device__ __forceinline__ void store_late(const DecodeArgs& a, const RowRange& r, int hk) const {
    if (!VL || !late) return;
    const int pg = __builtin_amdgcn_readfirstlane(late_page);
    if (pg < 0) return;
    const int ps = a.g.page_size;
    const size_t dst = (size_t)pg * a.g.n_kv * ps * D + (size_t)hk * ps * D;
    const int row = (r.L - 1) & (ps - 1);
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const int d = threadIdx.x + 256 * i;
      if (d < D) a.vpool_w[dst + v_elem_offset(d, row, D, a.g.log2ps)] = v[i];
    }
  }
  // Page size >= 32, in the chunk holding the new key, after patch(): each
  // lane's 16 bytes of V (rows d0 + 16*dt + lane%16, the 8 keys of its
  // quarter of the group) back to the address it loaded them from; the four
  // quarters make each row's 64 bytes.
  template <int DW>
  __device__ __forceinline__ void store_v_rows(bf16_t* vrow0, int lgv, const u32x4 (&vop)[DW / 16]) const {
#pragma unroll
    for (int dt = 0; dt < DW / 16; ++dt) store16(vrow0 + ((size_t)16 * dt << lgv), vop[dt]);
  }
};

// Stages the page ids of logical pages [p0, p0 + n) of the row into LDS.
__device__ __forceinline__ void stage_pages(const DecodeArgs& a, const int32_t* trow, int p0, int n,
                                            int* s_pg) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int pg = trow[p0 + i];
    s_pg[i] = (pg >= 1 && pg < a.g.n_pages) ? pg : -1;
  }
}

// Device-scope (sc1) accesses of the split partials: coherent across the
// XCDs' L2s without any cache write-back or invalidation.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_dev2(const float* p) {  // p 8-byte aligned
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_dev_u32(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of the n_valid split partials of one (row, kv head), in
// fixed split order (bitwise deterministic whichever workgroup merges).  One
// pass: each thread owns P consecutive output dim pairs of one query head
// (P = G*D/2 over the threads, see merge_splits) and issues the (max, sum) pair
// and the partial o of all of them for up to kU splits together, merging
// them online against a running maximum, so the whole merge costs one memory
// round trip per kU splits.  (One pair per thread at a time made the
// head_dim-512 merge four dependent round trips per kU splits.)  A partial o
// is the split's normalised output o / l in bf16 (accumulated in fp32 and
// rounded once, like the kernel's bf16 output); its weight is f * l with f
// = 2^(m - M).  Partials in fp32, twice the bytes written while the grid
// saturates HBM with reads, measured 99.2 against 96.4 us on the Llama shape
// and 63.0 against 61.1 us on the Gemma full layer.
// OWN: split 0 merges with its own values (o_val, Mof, Lof) in place of its
// published partial, rounded exactly as that partial would be, so the result
// is bit for bit the same.
template <int D, int P, bool OWN, class OFn, class MFn, class LFn>
__device__ void merge_splits_p(const DecodeArgs& a, int b, int hk, int n_valid, OFn o_val, MFn Mof,
                               LFn Lof) {
  const int G = a.G, S = a.max_splits;
  const size_t pbase = ((size_t)b * a.g.n_kv + hk) * S;
  constexpr int kU = 8;  // splits whose loads are in flight together
  constexpr int kMaxP = P;
  const int npairs = G * D / 2;
  const int p0 = (int)threadIdx.x * P;
  if (p0 >= npairs) return;  // (no barrier follows)
  const int g = (2 * p0) / D, d0 = 2 * p0 - g * D;
  const float* ml = a.part_ml + (pbase * G + g) * 2;
  uint32_t* po = a.part_o + ((pbase * G + g) * D + d0) / 2;
  float M = -INFINITY, lsum = 0.f;
  float o[kMaxP][2];
#pragma unroll
  for (int i = 0; i < kMaxP; ++i) o[i][0] = o[i][1] = 0.f;
  for (int t0 = 0; t0 < n_valid; t0 += kU) {
    uint32_t v[kMaxP][kU];
    uint64_t w[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const bool ok = t0 + j < n_valid;
      if (OWN && t0 + j == 0) {
        const float l0 = Lof(g), inv0 = l0 > 0.f ? 1.0f / l0 : 0.f;
        w[j] = (uint64_t)__float_as_uint(Mof(g)) | ((uint64_t)__float_as_uint(l0) << 32);
#pragma unroll
        for (int i = 0; i < kMaxP; ++i)
          v[i][j] = pack_bf16x2(o_val(g, d0 + 2 * i) * inv0, o_val(g, d0 + 2 * i + 1) * inv0);
        continue;
      }
      w[j] = ok ? load_dev2(ml + (size_t)(t0 + j) * G * 2) : 0;
#pragma unroll
      for (int i = 0; i < kMaxP; ++i) v[i][j] = ok ? load_dev_u32(po + (size_t)(t0 + j) * G * D / 2 + i) : 0;
    }
    // A split's (max, sum) is (m, l); l == 0 marks an empty partial, whose
    // o was never written: it is selected away, never multiplied.
    float mg = M;
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (__uint_as_float((uint32_t)(w[j] >> 32)) > 0.f) mg = fmaxf(mg, __uint_as_float((uint32_t)w[j]));
    if (mg > M) {
      const float alpha = fast_exp2(M - mg);  // 0 while M is -inf
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < kMaxP; ++i) {
        o[i][0] *= alpha;
        o[i][1] *= alpha;
      }
      M = mg;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const float l = __uint_as_float((uint32_t)(w[j] >> 32));
      if (l > 0.f) {
        const float fl = fast_exp2(__uint_as_float((uint32_t)w[j]) - M) * l;
        lsum += fl;
#pragma unroll
        for (int i = 0; i < kMaxP; ++i) {
          o[i][0] += fl * bf16lo(v[i][j]);
          o[i][1] += fl * bf16hi(v[i][j]);
        }
      }
    }
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  bf16_t* orow = a.out + ((size_t)b * a.n_q + hk * G + g) * D + d0;
#pragma unroll
  for (int i = 0; i < kMaxP; ++i)
    *reinterpret_cast<uint32_t*>(orow + 2 * i) = pack_bf16x2(o[i][0] * inv, o[i][1] * inv);
  if (a.lse && d0 == 0)
    a.lse[(size_t)b * a.n_q + hk * G + g] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
}

// P: the smallest power of two with P * threads >= G*D/2 (1, 2 or 4, as
// G * D <= 2048 and the workgroups have 256 or 512 threads; a divisor of D/2,
// so a thread's pairs lie in one head).
template <int D, bool OWN, class OFn, class MFn, class LFn>
__device__ void merge_splits(const DecodeArgs& a, int b, int hk, int n_valid, OFn o_val, MFn Mof,
                             LFn Lof) {
  const int npairs = a.G * D / 2;
  if (npairs <= (int)blockDim.x)
    merge_splits_p<D, 1, OWN>(a, b, hk, n_valid, o_val, Mof, Lof);
  else if (npairs <= 2 * (int)blockDim.x)
    merge_splits_p<D, 2, OWN>(a, b, hk, n_valid, o_val, Mof, Lof);
  else
    merge_splits_p<D, 4, OWN>(a, b, hk, n_valid, o_val, Mof, Lof);
}

// Writes this workgroup's result: the final output when it is the row's only
// split, else its partial (o / l as bf16 pairs; the running max in log2 units
// and the sum l in fp32), and the last split to arrive merges all partials.
// o_val(g, d), Mof(g), Lof(g) give the workgroup's values.  EARLY (grids of
// several rounds): split 0, the grid's last layer and so most often the
// row's last split to finish, first reads the row's arrival counter; when
// every other split has counted itself in, it merges at once with its own
// values in place of a published partial (no partial store, no wait for it,
// no increment) and leaves the counter at zero.  Llama shape 96.8 -> 96.4
// us, Gemma full layer 61.2 -> 60.4 us; on one-round grids, where split 0 is
// seldom last, the extra read lengthened its chain (Qwen3 call +0.6 us).
template <int D, bool EARLY, class OFn, class MFn, class LFn>
__device__ void finish(const DecodeArgs& a, const RowRange& r, int b, int hk, int s, OFn o_val,
                       MFn Mof, LFn Lof) {
  const int G = a.G;
  const int tid = threadIdx.x;
  if (r.n_valid <= 1) {
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
      const int g = idx / D, d = idx - g * D;
      const float l = Lof(g);
      a.out[((size_t)b * a.n_q + hk * G + g) * D + d] = f32_to_bf16(l > 0.f ? o_val(g, d) / l : 0.f);
      if (a.lse && d == 0)
        a.lse[(size_t)b * a.n_q + hk * G + g] = l > 0.f ? (Mof(g) + __log2f(l)) * kLn2 : -INFINITY;
    }
    return;
  }
  uint32_t* ctr = a.arrivals_end - 1 - ((size_t)b * a.g.n_kv + hk);
  if (EARLY && s == 0) {
    __shared__ int s_early;
    // (the counter reaches n_valid - 1 only after every other split's
    // partial is complete at the coherent level, as for the arrival below)
    if (tid == 0)
      s_early = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(r.n_valid - 1);
    __syncthreads();
    if (s_early) {
      merge_splits<D, true>(a, b, hk, r.n_valid, o_val, Mof, Lof);
      if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  const size_t pbase = ((size_t)b * a.g.n_kv + hk) * a.max_splits + s;
  for (int idx = tid; idx < G * D / 2; idx += blockDim.x) {
    const int g = (2 * idx) / D, d = 2 * idx - g * D;
    const float l = Lof(g), inv = l > 0.f ? 1.0f / l : 0.f;
    store_dev_u32(a.part_o + ((pbase * G + g) * D + d) / 2, pack_bf16x2(o_val(g, d) * inv, o_val(g, d + 1) * inv));
  }
  for (int g = tid; g < G; g += blockDim.x) {
    store_dev(a.part_ml + (pbase * G + g) * 2, Mof(g));
    store_dev(a.part_ml + (pbase * G + g) * 2 + 1, Lof(g));
  }
  // Ordering of the partials before the arrival, as the gfx950 ISA gives it
  // (not the HIP memory model's release/acquire): the partial stores above
  // are device-scope (sc1) stores, which write through to the memory side
  // that is coherent across all XCDs; s_waitcnt vmcnt(0) returns only once
  // each has been acknowledged there, and the barrier extends that to the
  // whole workgroup before thread 0's atomic increment is issued.  The merging
  // workgroup reads every partial with device-scope (sc1) atomic loads, which
  // are served from that same coherent level and never from a stale L1 / L2
  // line, so no cache invalidation is needed either.  (A release fence instead
  // writes back the XCD's whole L2 per workgroup: measured 3x slower.)
  __builtin_amdgcn_s_waitcnt(0);          // this thread's partial stores are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // (and stay before the arrival below)
  __shared__ int s_last;
  __syncthreads();                        // ... and so are the whole workgroup's
  if (tid == 0) {
    // wraps to 0 on the n_valid-th arrival, ready for the next call that
    // uses this workspace
    const uint32_t old =
        __builtin_amdgcn_atomic_inc32(ctr, (uint32_t)(r.n_valid - 1), __ATOMIC_RELAXED, "agent");
    s_last = old == (uint32_t)(r.n_valid - 1);
  }
  __syncthreads();
  if (s_last) merge_splits<D, false>(a, b, hk, r.n_valid, o_val, Mof, Lof);
}

// An idle row (padding slot or empty context): split 0 writes out = 0 and
// lse = -inf; the other splits have nothing to do.
__device__ __forceinline__ void idle_output(const DecodeArgs& a, int b, int hk, int s, int D) {
  if (s != 0) return;
  for (int idx = threadIdx.x; idx < a.G * D; idx += blockDim.x) {
    const int g = idx / D, d = idx - g * D;
    a.out[((size_t)b * a.n_q + hk * a.G + g) * D + d] = 0;
    if (a.lse && d == 0) a.lse[(size_t)b * a.n_q + hk * a.G + g] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// head_dim <= 128: key split across the NW = 4 waves of the workgroup; K
// rows through the waves' LDS stages.
template <int D, int NW, bool VL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3)))
void decode_keysplit_kernel(const int32_t* slots, const int32_t* seq_lens, const int32_t* table,
                            int max_splits, DecodeArgs a) {
  // slots .. max_splits repeat fields of `a`: passed first, they arrive
  // preloaded in scalar registers (the library builds this file with four
  // preloaded kernel arguments), so the slot and length loads issue at once.
  // dynamic: the waves' K stages ([wave][32 keys][D] bf16) during the key
  // loop, then the waves' outputs s_o ([wave][G][D] fp32) for the merge
  extern __shared__ __attribute__((aligned(16))) float s_o[];
  __shared__ int s_pg[kSegPages];
  __shared__ float s_ml[2 * NW * 16];             // [wave][16] max, then sum
  __shared__ float s_red[NW * 16 + 32];
  __shared__ __attribute__((aligned(16))) NewTokLds<D> s_new;
  constexpr int kStage = 32 * D * 2;              // bytes of a wave's K stage
  const int hk = blockIdx.x, b = blockIdx.y, s = max_splits - 1 - (int)blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qc = lane & 15, quad = lane >> 4;
  const int G = a.G;
  const RowRange r = row_range(a, b, s, slots, seq_lens);
  if (r.idle) {
    idle_output(a, b, hk, s, D);
    return;
  }
  if (s >= r.n_valid) return;  // past the row's last key: not counted by the merge
  NewTok<D, VL> nt;
  nt.load(a, r, b, hk, s, table);

  const int ps = a.g.page_size, log2ps = a.g.log2ps;
  const int32_t* trow = table + (size_t)r.slot * a.pt.pps;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)a.g.n_kv * blk;
  const int lgv = min(log2ps, kLog2VGroup);  // log2 of the V key-group size
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
    __syncthreads();  // previous segment's page ids consumed
    stage_pages(a, trow, p0, ((seg1 - 1) >> log2ps) - p0 + 1, s_pg);
    if (seg0 == r.start) nt.template stage<D>(s_new);
    __syncthreads();
    if (seg1 == r.end) nt.find_page(r, log2ps, p0, s_pg);
    if (seg0 == r.start) {
      // Columns qc >= G repeat head G-1: MFMA columns never mix, and those
      // are never stored.  (Zeroing them here would wait for q before the
      // first chunk's K/V loads are issued.)
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qreg[c] = load16(qrow + 32 * c);
    }
    // A wave's chunk = 32 keys at t0.  K: 1 KB global-to-LDS copies into the
    // wave's stage (copy i, lane l: stage bytes 1024*i + 16*l = row r, slot
    // u, filled from unit u ^ kst_swz(r) of key t0 + r).  Keys >= seg1 read a
    // row of page 0 or of the chunk's own page, always inside the pool; their
    // scores are masked.  V^T: 16-byte loads into operand registers,
    // zero for keys >= seg1 or on an unmapped page (0 * NaN would poison P.V).
    // No prefetch of the next chunk: the registers it would take buy a third
    // wave per SIMD instead, which keeps more bytes in flight per CU.
    uint8_t* kst = reinterpret_cast<uint8_t*>(s_o) + w * kStage;
    for (int t0 = seg0 + 32 * w; t0 < seg1; t0 += 32 * NW) {
      if (ps >= 32) {
        // the chunk lies in one page (t0 < seg1): one scalar page id
        const int pg = __builtin_amdgcn_readfirstlane(max(s_pg[(t0 >> log2ps) - p0], 0));
        const bf16_t* ks = kbase + (size_t)pg * page_stride + (size_t)(t0 & (ps - 1)) * D;
#pragma unroll
        for (int i = 0; i < kStage / 1024; ++i) {
          const int o = 1024 * i + 16 * lane;
          const int rr = o / (2 * D), u = ((o % (2 * D)) >> 4) ^ kst_swz<D>(o / (2 * D));
          __builtin_amdgcn_global_load_lds(ks + rr * D + 8 * u, (lds_void_ptr)(kst + 1024 * i), 16, 0, kNtAux);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kStage / 1024; ++i) {
          const int o = 1024 * i + 16 * lane;
          const int rr = o / (2 * D), u = ((o % (2 * D)) >> 4) ^ kst_swz<D>(o / (2 * D));
          const int tk = t0 + rr;
          const int pg = s_pg[min((tk >> log2ps) - p0, kSegPages - 1)];
          const int page = tk < seg1 ? max(pg, 0) : 0;
          __builtin_amdgcn_global_load_lds(kbase + (size_t)page * page_stride + (size_t)(tk & (ps - 1)) * D + 8 * u,
                                           (lds_void_ptr)(kst + 1024 * i), 16, 0, kNtAux);
        }
      }
      const int tv = t0 + 8 * quad;
      const int vpage = tv < seg1 ? s_pg[(tv >> log2ps) - p0] : -1;
      const int nvalid = seg1 - tv;
      const bool app = nt.in_chunk(r, t0), vrows = app && ps >= 32;
      u32x4 vop[D / 16];
      // V^T row d = 16*dt + qc, keys tv .. tv+7 (inside one key group); the
      // new key's chunk reads its whole group from the new key's page
      const bf16_t* vp = vbase + (size_t)(vrows ? nt.page : max(vpage, 0)) * page_stride +
                         v_elem_offset(qc, tv & (ps - 1), D, log2ps);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) vop[dt] = load16_nt(vp + ((size_t)16 * dt << lgv));
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the K copies have landed in the stage
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // (and the stage reads stay after it)
      if (app) {
        nt.template patch<D>(r, t0, 0, kst, kst_swz<D>, s_new, vop);
        if (vrows && !VL) nt.template store_v_rows<D>(a.vpool_w + (vp - a.vpool), lgv, vop);
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        vop[dt] = vpage >= 0 ? (nvalid < 8 ? keep_first(vop[dt], nvalid) : vop[dt]) : u32x4{0, 0, 0, 0};
      // ---- S^T = K Q^T; MFMA rg row m holds key 8*(m/4) + 4*rg + m%4
      f32x4 S[2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int rr = 8 * (qc >> 2) + 4 * rg + (qc & 3);
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(kst + rr * (2 * D) + 16 * ((4 * c + quad) ^ kst_swz<D>(rr)));
          sacc = mfma16x16x32(kv, qreg[c], sacc);
        }
        S[rg] = sacc;
      }
      // ---- online softmax; lane holds keys t0 + 8*quad + j
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = tv + j;
        const float v = (j < 4 ? S[0][j] : S[1][j - 4]) * a.scale_log2;
        sc[j] = (tk >= r.lo && tk < seg1 && vpage >= 0) ? v : -INFINITY;
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
  __syncthreads();  // every wave is done with its K stage, which s_o reuses

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
  finish<D, VL>(a, r, b, hk, s, o_val, Mof, Lof);
  nt.template store<D>(a, r, hk, s_new);
  nt.store_late(a, r, hk);
}

// ---------------------------------------------------------------------------
// head_dim >= 256: the 4 waves split head_dim; all walk the same chunks.
// Each wave copies the K slice of its dims (32 rows of DW bf16: whole cache
// lines) into its own LDS stage by global-to-LDS copies, like the key-split
// kernel on long splits; the stages become the output buffer at the end.
// At least three waves per SIMD (head_dim 512 would otherwise take 187
// registers and two): more workgroups per CU hide the per-chunk barrier and
// keep more bytes in flight (measured 5 % faster on the Gemma shapes; a
// register double buffer, and four or five waves per SIMD, were slower).
template <int D, bool EM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void decode_dimsplit_kernel(const int32_t* slots, const int32_t* seq_lens, const int32_t* table,
                            int max_splits, DecodeArgs a) {
  // preloaded repeats of fields of `a`, as in the key-split kernel
  constexpr int DW = D / kDecodeWaves;  // dims per wave
  constexpr int kStage = 32 * DW * 2;   // bytes of a wave's K stage
  static_assert(kDecodeWaves * kStage >= kMaxGD * (int)sizeof(float), "s_o must fit the stages");
  __shared__ int s_pg[kSegPages];
  __shared__ f32x4 s_part[2][kDecodeWaves][2][64];  // [buffer][wave][rg][lane]
  // the waves' K stages during the key loop, then s_o = [G][D] final
  // unnormalised output (the loop's last barrier orders the reuse)
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[kDecodeWaves * kStage];
  float* const s_o = reinterpret_cast<float*>(s_stage);
  __shared__ float s_ml[32];
  __shared__ __attribute__((aligned(16))) NewTokLds<D> s_new;
  const int hk = blockIdx.x, b = blockIdx.y, s = max_splits - 1 - (int)blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qc = lane & 15, quad = lane >> 4;
  const int G = a.G;
  const RowRange r = row_range(a, b, s, slots, seq_lens);
  if (r.idle) {
    idle_output(a, b, hk, s, D);
    return;
  }
  if (s >= r.n_valid) return;  // past the row's last key: not counted by the merge
  NewTok<D> nt;
  nt.load(a, r, b, hk, s, table);

  const int dw0 = w * DW;
  u32x4 qreg[DW / 32];  // loaded after the first page staging (see the key-split kernel)
  const bf16_t* qrow = a.q + ((size_t)b * a.n_q + hk * G + min(qc, G - 1)) * D + dw0 + 8 * quad;
  const int ps = a.g.page_size, log2ps = a.g.log2ps;
  const int32_t* trow = table + (size_t)r.slot * a.pt.pps;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)a.g.n_kv * blk;
  const int lgv = min(log2ps, kLog2VGroup);  // log2 of the V key-group size
  const bf16_t* kbase = a.kpool + hk * blk + dw0;
  const bf16_t* vbase = a.vpool + hk * blk;

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
    if (seg0 == r.start) nt.template stage<DW>(s_new);
    __syncthreads();
    if (seg1 == r.end) nt.find_page(r, log2ps, p0, s_pg);
    if (seg0 == r.start) {
#pragma unroll
      for (int c = 0; c < DW / 32; ++c) qreg[c] = load16(qrow + 32 * c);  // (qc >= G: head G-1, unused)
    }
    uint8_t* kst = s_stage + w * kStage;
    for (int t0 = seg0; t0 < seg1; t0 += 32, ++it) {
      // K slice: copy i, lane l fills stage bytes 1024*i + 16*l = row r, slot
      // u from the wave's dims unit u ^ kst_swz(r) of key t0 + r.  Keys >=
      // seg1 read a row of page 0 or of the chunk's own page (in the pool);
      // their scores are masked.
      if (ps >= 32) {
        const int pg = __builtin_amdgcn_readfirstlane(max(s_pg[(t0 >> log2ps) - p0], 0));
        const bf16_t* ks = kbase + (size_t)pg * page_stride + (size_t)(t0 & (ps - 1)) * D;
#pragma unroll
        for (int i = 0; i < kStage / 1024; ++i) {
          const int o = 1024 * i + 16 * lane;
          const int rr = o / (2 * DW), u = ((o % (2 * DW)) >> 4) ^ kst_swz<DW>(o / (2 * DW));
          __builtin_amdgcn_global_load_lds(ks + rr * D + 8 * u, (lds_void_ptr)(kst + 1024 * i), 16, 0, kNtAux);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kStage / 1024; ++i) {
          const int o = 1024 * i + 16 * lane;
          const int rr = o / (2 * DW), u = ((o % (2 * DW)) >> 4) ^ kst_swz<DW>(o / (2 * DW));
          const int tk = t0 + rr;
          const int pg = s_pg[min((tk >> log2ps) - p0, kSegPages - 1)];
          const int page = tk < seg1 ? max(pg, 0) : 0;
          __builtin_amdgcn_global_load_lds(kbase + (size_t)page * page_stride + (size_t)(tk & (ps - 1)) * D + 8 * u,
                                           (lds_void_ptr)(kst + 1024 * i), 16, 0, kNtAux);
        }
      }
      const int tv = t0 + 8 * quad;
      const int vpage = tv < seg1 ? s_pg[(tv >> log2ps) - p0] : -1;
      const int nvalid = seg1 - tv;
      const bool app = nt.in_chunk(r, t0), vrows = app && ps >= 32;
      // V^T row d = dw0 + 16*dt + qc, keys tv .. tv+7 (inside one key group);
      // the new key's chunk reads its whole group from the new key's page
      const bf16_t* vp = vbase + (size_t)(vrows ? nt.page : max(vpage, 0)) * page_stride +
                         v_elem_offset(dw0 + qc, tv & (ps - 1), D, log2ps);
      u32x4 vop[DW / 16];
#pragma unroll
      for (int dt = 0; dt < DW / 16; ++dt) vop[dt] = load16_nt(vp + ((size_t)16 * dt << lgv));
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the K copies have landed in the stage
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // (and the stage reads stay after it)
      if (app) {
        nt.template patch<DW>(r, t0, dw0, kst, kst_swz<DW>, s_new, vop);
        if (vrows) nt.template store_v_rows<DW>(a.vpool_w + (vp - a.vpool), lgv, vop);
      }
#pragma unroll
      for (int dt = 0; dt < DW / 16; ++dt)
        vop[dt] = vpage >= 0 ? (nvalid < 8 ? keep_first(vop[dt], nvalid) : vop[dt]) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int rr = 8 * (qc >> 2) + 4 * rg + (qc & 3);
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DW / 32; ++c) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(kst + rr * (2 * DW) + 16 * ((4 * c + quad) ^ kst_swz<DW>(rr)));
          sacc = mfma16x16x32(kv, qreg[c], sacc);
        }
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
        sc[j] = (tk >= r.lo && tk < seg1 && vpage >= 0) ? v : -INFINITY;
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
  finish<D, EM>(a, r, b, hk, s, o_val, Mof, Lof);
  nt.template store<DW>(a, r, hk, s_new);
}

// Dynamic LDS of the key-split kernel: the larger of the waves' K stages and
// their fp32 outputs (at most 32 KB: 4 waves * 32 keys * 128 * 2 bytes, or
// 4 waves * G * D * 4 bytes with G * D <= 2048).
template <int D>
size_t keysplit_lds_bytes(int waves, int G) {
  const size_t stage = (size_t)waves * 32 * D * 2, outs = (size_t)waves * G * D * sizeof(float);
  return stage > outs ? stage : outs;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  // Splits are the slowest grid dimension and run from the last down: the
  // full-length splits that only long rows have are dispatched first and the
  // first splits, partial for short rows, fill the tail (longest first;
  // measured 11 % faster on the ragged Llama batch, 8 % on Gemma, 4 % on
  // Qwen3).  Heads vary fastest, one per XCD when n_kv is 8.
  dim3 grid(a.g.n_kv, a.B, a.max_splits);
  if constexpr (D <= 128) {
    if (a.v_late)
      hipLaunchKernelGGL((decode_keysplit_kernel<D, kDecodeWaves, true>), grid, dim3(kThreads),
                         keysplit_lds_bytes<D>(kDecodeWaves, a.G), st, a.slots, a.seq_lens,
                         a.pt.table, a.max_splits, a);
    else
      hipLaunchKernelGGL((decode_keysplit_kernel<D, kDecodeWaves, false>), grid, dim3(kThreads),
                         keysplit_lds_bytes<D>(kDecodeWaves, a.G), st, a.slots, a.seq_lens,
                         a.pt.table, a.max_splits, a);
  } else if (a.early_merge) {
    hipLaunchKernelGGL((decode_dimsplit_kernel<D, true>), grid, dim3(kThreads), 0, st, a.slots,
                       a.seq_lens, a.pt.table, a.max_splits, a);
  } else {
    hipLaunchKernelGGL((decode_dimsplit_kernel<D, false>), grid, dim3(kThreads), 0, st, a.slots,
                       a.seq_lens, a.pt.table, a.max_splits, a);
  }
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
  // About 4096 workgroups over the key ranges (16 per CU): enough to cover the
  // 256 CUs several times with a short ragged tail, few enough that the
  // partials written and merged stay small next to the K/V bytes (measured
  // against 1024 / 2048 / 8192 on the ragged Llama batch: 117 / 112 / 113 vs
  // 109 us, other shapes unchanged).  The split count is also capped so that
  // one merge reads at most 1024 (split, head) partials.
  while ((pairs * ((range + split - 1) / split) > 4096 ||
          ((range + split - 1) / split) * G > kMaxMergeUnits) &&
         split < (1 << 24))
    split *= 2;
  // Key split (head_dim <= 128): four 32-key chunks per wave, i.e. 512-key
  // splits over 4 waves, whenever that still gives at least one workgroup per
  // CU -- fewer workgroups than the budget above allows, so fewer set-ups and
  // partials to merge.  Measured on one GPU's share of the Llama shape under
  // 8-way tensor parallelism (64 rows, 3 query / 1 kv head): 21.5 us, against
  // 24.1 / 26.7 / 40.6 with 256- / 1024- / 2048-key splits and 34.4 with
  // 8-wave workgroups over 256-key splits; the full Llama shape already
  // plans 512.  (Short splits, one 32-key chunk per wave, once ran faster as
  // 8-wave workgroups over 256 keys -- half the workgroups and partials; with
  // the partials in bf16 the 4-wave 128-key splits win: Qwen3 call 11.05 ->
  // 10.65 us.)
  if (head_dim <= 128 && split < 512 && pairs * ((range + 511) / 512) >= 256) split = 512;
  p.split_tokens = (int)split;
  p.head_tokens = (int)split;
  p.v_late = 0;
  p.early_merge = 0;
  p.max_splits = (int)((range + split - 1) / split);
  // A short split 0 on large full-causal grids: split 0 of every row is the
  // last layer of the grid to be dispatched, and the call ends as those
  // workgroups drain.  A quarter-length split 0 shortens that drain for one
  // more workgroup per row: Llama shape (4096 workgroups of 512 keys)
  // 103.0 -> 101.2 us; a 64- or 256-key split 0 measured 104.3 and 102.1.
  // Below about 2048 workgroups (under three rounds of the resident slots)
  // the extra workgroups cost more than the drain saves (one GPU's share of
  // the Llama shape under 8-way tensor parallelism, 512 workgroups: +0.6 us).
  if (window <= 0 && split >= 512 && pairs * p.max_splits >= 2048) {
    const int hs = (int)(split / 4);
    const int n = range <= hs ? 1 : (int)((range - hs + 2 * split - 1) / split);
    if (n * G <= kMaxMergeUnits) {
      p.head_tokens = hs;
      p.max_splits = n;
      p.v_late = head_dim <= 128;  // (the key-split kernel's fused append)
    }
  }
  // Split 0 merging early (finish): the key-split instance with the late V
  // store does, on the same large grids; the dim-split kernel from 1024
  // workgroups (several rounds of its resident slots).
  p.early_merge = head_dim <= 128 ? p.v_late : pairs * p.max_splits >= 1024;
  // (One 8-wave workgroup per pair without a split was measured slower than
  // split + merge even for 8 rows: 64 CUs stream ~16 GB/s each with
  // sequential chunks.)
  if (p.max_splits <= 1) {
    p.max_splits = 1;
    p.ws_bytes = 0;
    p.part_o_words = 0;
    return p;
  }
  const size_t units = (size_t)B * n_kv * p.max_splits * G;
  p.part_o_words = (units * head_dim / 2 + 63) & ~(size_t)63;
  // partials from the start, then (at the end, in the workspace's counter
  // region) the (row, kv head) arrival counters, which the kernel addresses
  // back from the workspace's end.  The size makes the region hold this
  // call's counters and keeps the partials below it, with room to spare, for
  // this size and every larger one.
  const size_t part = (p.part_o_words + units * 2) * sizeof(float);
  const size_t ctr = (size_t)B * n_kv * 4;
  size_t ws = std::max(16 * ctr, part + part / 15 + 16);
  ws = (ws + 255) & ~(size_t)255;
  while (part + 16 > ws - ws / 16 || ctr > decode_counter_region(ws)) ws += 256;
  p.ws_bytes = ws;
  return p;
}

// The static scratch of pkv_attn_decode_noalloc: split partials from the
// start, arrival counters in its last bytes (zero when the code object is
// loaded; every call leaves them at zero).  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is taken
// with hipGetSymbolAddress once per device, with that device current, and
// only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
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
