// Packed varlen prefill attention over the paged cache, bf16 MFMA for gfx950.
//
// Work item = (kv head, sequence, block of query tokens).  The G query heads
// of the kv head are packed with the block's tokens into the MFMA column
// dimension (column = token * G + head), so each K/V tile serves all of them.
// A workgroup is 4 wave64s, each owning NT 16-column tiles (32 query columns
// per wave at head_dim <= 128).  Registers are capped so that two waves run
// per SIMD (two independent workgroups per CU), each filling the other's
// latency gaps.  (64 columns per wave halve the LDS operand traffic but need
// ~350 registers and one wave per SIMD; 8-wave workgroups put two waves of
// one item on each SIMD, in lockstep or in an explicit MFMA / softmax
// ping-pong -- all measured slower.)
// With the fused prologue, q is normalised and rotated in registers as an
// item loads it (norm_rope_q); with two or more query heads per kv head the
// item's rotary rows are staged in LDS (one kernel instance per source of
// those rows).
//
// Keys advance in 64-key chunks.  Each chunk's K rows and V^T rows are copied
// from their physical pages straight into LDS with gfx950's global-to-LDS
// loads (16 bytes per lane, no staging registers); the next chunk's copies are
// in flight while the current chunk is computed from the other LDS buffer,
// with one wait + barrier per chunk.  Tiles are XOR-swizzled in 16-byte units
// so that the MFMA operand reads of 16 rows hit 16 distinct bank groups.
// Page ids of the item's key range are staged in LDS once per item.
//
// Per chunk and column tile every wave computes, for its two 32-key halves h,
//
//   S^T[32 keys][16 cols] = K[32][D] . Q^T[D][16]
//   O^T[D][16 cols]      += V^T[D][32] . P^T[32][16]
//
// with the same operand layout as the decode kernel (a lane's 8 key scores
// are directly its P^T k-slots).  The softmax keeps a reference max that only
// moves when some score outgrows it by 2^8, so the O accumulators are rarely
// rescaled and the common path has no cross-lane work.  Chunks entirely above
// a wave's causal diagonal, or entirely left of its sliding window, are
// skipped without MFMA work; chunks entirely visible skip the element mask.
//
// Query blocks run longest-first on a (kv head, sequence, layer) grid; see
// prefill_kernel and its launcher for the dispatch-order details.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kChunk = 64;                // keys per pipeline step

// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are outstanding (n < 64; vmcnt bits [3:0] and [15:14], expcnt and
// lgkmcnt left at their maxima, i.e. not waited on).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) & 3) << 14; }

constexpr int kStagePages = 2048;         // page ids staged in LDS (>= pages_per_slot, host-checked)

// Waves per workgroup and 16-column MFMA tiles per wave: 4 waves of up to
// 256 registers, two waves per SIMD (two workgroups per CU).  (8 waves of
// one tile at 128 registers, four per SIMD, measured no faster and spills.)
// head_dim 256: its double-buffered 64 KB tiles leave room for one
// workgroup per CU, so 8 waves of one tile (198-204 registers, two waves per
// SIMD) -- twice the occupancy of 4, and items of twice the tokens, so half
// the key re-reads: the Gemma-4 sliding layer 80.9 -> 57.5 us.
template <int D>
constexpr int prefill_waves() { return D == 256 ? 8 : 4; }
template <int D>
constexpr int prefill_threads() { return 64 * prefill_waves<D>(); }
template <int D>
constexpr int prefill_nt() { return D <= 128 ? 2 : 1; }
// LDS tile buffers: two (the next chunk's copies in flight during the current
// chunk's math), except at head_dim 512, whose 128 KB tile fits once.
template <int D>
constexpr int prefill_bufs() { return D == 512 ? 1 : 2; }
// Waves per SIMD: two (256 registers each); head_dim 512 runs one workgroup
// per CU (LDS) and so one wave per SIMD, with the 512-register budget.
template <int D>
constexpr int prefill_wpe() { return D == 512 ? 1 : 2; }

template <int D>
constexpr int k_tile_bytes() { return kChunk * D * 2; }   // [64 keys][D] bf16
template <int D>
constexpr int tile_bytes() { return 2 * k_tile_bytes<D>(); }  // + V^T [D][64 keys]
template <int D>
constexpr int dma_per_wave() { return D / (8 * prefill_waves<D>()); }  // 1 KB copies per wave, for K and V each

// Swizzles (16-byte slot of a row).  K row r holds chunk c (dims 8c..8c+7) at
// slot c ^ k_swz(r); V^T row d holds key group g (keys 8g..8g+7) at slot
// g ^ v_swz(d).  Both are bijections within a row; for the 16 rows one MFMA
// operand read touches (K: 16 consecutive rows; V^T: the rows vrow(dt, 0..15)
// below) they give 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 64 ? (((r >> 1) + 2 * (r >> 4)) & 7) : ((r + 4 * (r >> 4)) & 15);
}
__device__ __forceinline__ int v_swz(int d) { return ((d >> 1) & 1) | (((d >> 3) & 3) << 1); }

// The P.V MFMA dt takes as its A row m the V^T row (head_dim index)
//   vrow(dt, m) = 8*(m/4) + m%4 + 32*(dt/2) + 4*(dt%2),
// so the accumulator lane (column, quad) of MFMAs 2k and 2k+1 holds dims
// 32k + 8*quad .. +7 of its column: one 16-byte store each (a bijection of
// the head_dim rows; the swizzle above is the same for all dt).
__device__ __forceinline__ int vrow_step(int dt) { return 32 * (dt >> 1) + 4 * (dt & 1); }

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

// ---------------------------------------------------------------------------
// Per-lane constants.
template <int D>
struct LaneConst {
  // LDS byte offsets (within a tile buffer) of this lane's MFMA operand rows.
  // K row r, dims chunk c sits at kofs ^ (64 * c): the row's swizzle is folded
  // into kofs and 64*c only flips bits inside the row.  V^T rows vrow(dt, qc)
  // share one swizzle across dt, so dt is a plain vrow_step(dt) * 128 byte
  // step from vofs.
  int kofs[2][2], vofs[2];
};

// Source byte offsets of copy k of wave w for lane `lane`, relative to the
// chunk's first key in its page (K) or to the chunk's first 32-key group of
// V (page_size >= 64).  The copy fills tile bytes m*1024 .. m*1024+1023
// (m = w*dpw + k), lane i the 16 bytes at +16*i.  K: tile row r slot s holds
// dims 8*(s ^ k_swz(r)) ..  V^T: row d slot s holds keys 8*g .. 8*g+7 of the
// chunk, g = s ^ v_swz(d): key group g/4, dim d, keys 8*(g%4) .. within it.
// Recomputed at each use: a few ALU ops are cheaper than registers held
// across the chunk math.
template <int D>
__device__ __forceinline__ uint32_t dma_k_off(int k, int lane, int w) {
  const int o = (w * dma_per_wave<D>() + k) * 1024 + 16 * lane;
  const int r = o / (2 * D), sk = (o % (2 * D)) >> 4;
  return 2 * (r * D + 8 * (sk ^ k_swz<D>(r)));
}
template <int D>
__device__ __forceinline__ uint32_t dma_v_off(int k, int lane, int w) {
  const int o = (w * dma_per_wave<D>() + k) * 1024 + 16 * lane;
  const int d = o >> 7, g = ((o >> 4) & 7) ^ v_swz(d);
  return 2 * ((((g >> 2) * D + d) << kLog2VGroup) + 8 * (g & 3));
}

template <int D>
__device__ __forceinline__ void lane_const(LaneConst<D>& lc, int lane, int w, int ps) {
  const int qc = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int r = 32 * h + 8 * (qc >> 2) + 4 * rg + (qc & 3);
      lc.kofs[h][rg] = r * (2 * D) + 16 * (quad ^ k_swz<D>(r));
    }
    const int d0 = 8 * (qc >> 2) + (qc & 3);  // vrow(0, qc)
    lc.vofs[h] = k_tile_bytes<D>() + d0 * 128 + 16 * ((4 * h + quad) ^ v_swz(d0));
  }
  (void)w;
  (void)ps;
}

// ---------------------------------------------------------------------------
// A work item: query block qb (tokens qb*QT ..) of sequence n against kv head
// hk, and its key range [j_start, kv_hi) in 64-key chunks.
struct Item {
  int hk, n;
  int a0, sp, i0, nq;
  bool idle;  // padding sequence (slot 0 / out of range): output 0, lse -inf
  int kv_hi, j_start, n_chunks, pg0, n_pg;
  const int32_t* trow;
};

// A sequence's metadata, the same for all of a workgroup's items; n_pg =
// the logical pages any of its items reads (their ids are staged in LDS
// once per workgroup).
struct SeqMeta {
  int a0, len, sp, slot, n_pg;
};

// Loaded once per workgroup, all four loads in flight together (start_pos,
// when absent, re-reads cu_seqlens[n] and is replaced by 0).
__device__ __forceinline__ SeqMeta seq_meta(const PrefillArgs& a, int n, const int32_t* cu_seqlens,
                                            const int32_t* slots, const int32_t* start_pos) {
  SeqMeta m;
  const int c0 = cu_seqlens[n], c1 = cu_seqlens[n + 1];
  const int spv = (start_pos ? start_pos : cu_seqlens)[n];
  const int slot = slots[n];
  m.a0 = __builtin_amdgcn_readfirstlane(c0);
  m.len = __builtin_amdgcn_readfirstlane(c1 - c0);
  m.sp = start_pos ? __builtin_amdgcn_readfirstlane(spv) : 0;
  m.slot = __builtin_amdgcn_readfirstlane(slot);
  const bool idle = m.slot <= 0 || m.slot >= a.pt.max_slots || m.sp < 0;
  const int kv_end = idle ? 0 : min(m.sp + m.len, a.pt.pps * a.g.page_size);
  m.n_pg = (kv_end + a.g.page_size - 1) >> a.g.log2ps;
  return m;
}

__device__ __forceinline__ void item_init(const PrefillArgs& a, const SeqMeta& sm, int hk, int n,
                                          int qb, Item& it) {
  it.hk = hk;
  it.n = n;
  it.a0 = sm.a0;
  const int len = sm.len;
  it.sp = sm.sp;
  const int slot = sm.slot;
  it.idle = slot <= 0 || slot >= a.pt.max_slots || it.sp < 0;
  it.i0 = qb * a.q_tokens;
  it.nq = min(a.q_tokens, len - it.i0);
  it.trow = a.pt.table + (size_t)(it.idle ? 0 : slot) * a.pt.pps;
  const int cap = a.pt.pps * a.g.page_size;
  it.kv_hi = it.idle ? 0 : min(it.sp + it.i0 + it.nq, cap);
  const int kv_lo = a.window > 0 ? max(0, it.sp + it.i0 - a.window + 1) : 0;
  it.j_start = kv_lo & ~(kChunk - 1);
  it.n_chunks = it.kv_hi > it.j_start ? (it.kv_hi - it.j_start + kChunk - 1) / kChunk : 0;
  it.pg0 = 0;          // s_pg holds the sequence's pages from logical page 0
  it.n_pg = sm.n_pg;
}

// An item parked in LDS (written by one thread) read back as uniform values.
__device__ __forceinline__ Item load_item(const Item* p) {
  const volatile int* v = reinterpret_cast<const volatile int*>(p);
  constexpr int nw = sizeof(Item) / sizeof(int);
  int x[nw];
#pragma unroll
  for (int i = 0; i < nw; ++i) x[i] = __builtin_amdgcn_readfirstlane(v[i]);
  Item it;
  __builtin_memcpy(&it, x, sizeof(Item));
  return it;
}

// Page id as the copies use it: unmapped / out-of-range table entries become
// -1 (read as page 0, whose keys are masked or zeroed).
__device__ __forceinline__ int checked_page(int pg, int n_pages) {
  return (pg >= 1 && pg < n_pages) ? pg : -1;
}

// ---------------------------------------------------------------------------
// This wave's query columns for an item: col = (w*NT + nt)*16 + qc maps to
// token col/G, head col%G.
template <int D, int NT>
struct WaveQ {
  u32x4 q[NT][D / 32];  // B operand of S^T = K Q^T (k-slot j of lane group g = dim 8g+j+32c)
  int pcol[NT];         // query position of the lane's column (-1: no query)
  int lo, hi;           // positions of the wave's first / last query (hi < 0: none)
  bf16_t* qout_row[NT];  // this lane's 16-byte slot of the column's q' row (q_out only)
};

// Sum over the four lanes l, l^16, l^32, l^48 (the 4 dim groups of a column);
// each swap hands every lane its partner's value in one of the two outputs.
__device__ __forceinline__ float quad_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  const uint32_t x = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
}

// Fused Qwen3 q prologue on the loaded Q^T operand: per column (token, head)
// x <- x / sqrt(mean(x^2) + eps) * w over head_dim, then the half-split
// rotation x_i <- x_i cos - x_{i+D/2} sin, x_{i+D/2} <- x_{i+D/2} cos + x_i sin
// at the token's position ([moe-qwen3 compare] flex_gemma4_moe.py, attention
// forward: q_norm, then _apply_rotary_full / _rotate_half).  A lane holds
// dims 8*quad + 32c + j of its column: the mean of squares is a sum over the
// column's 4 lanes, and the partner of chunk c (< D/64) is the same lane's
// chunk c + D/64.  fp32 math, one bf16 rounding (as the operand is used).
// Where the transform takes its rotary rows and norm weights from (one
// kernel instance each, chosen by the host per call):
//  Regs: loaded into registers right after q, so that both latencies overlap
//        (head_dim <= 128, one query head per kv head);
//  Lds:  the item's rows staged in LDS by stage_rope, the weights in
//        registers (head_dim <= 128, two or more query heads per kv head);
//  Load: loaded inside the transform, 16 bytes at a time as they are used
//        (head_dim >= 256, whose per-lane rows would not fit the registers).
// (The weights, the same for every item, are still loaded per item: read
// from LDS inside the transform they cost more than their load beside q.)
enum class RopeSrc { Regs, Lds, Load };
// q modes of the kernel: q given rotated, or raw with the fused transform
constexpr int kQReady = 0, kQRope = 1, kQRopeLds = 2;

template <int D, int NT>
struct QRope {
  float cs[NT][D / 64][8], sn[NT][D / 64][8];  // cos / sin of the lane's first-half dims (Regs)
  u32x4 w[D / 32];                            // q_norm weights of the lane's dims (Regs, Lds)
};

template <int D, int NT>
__device__ __forceinline__ void load_rope_w(const PrefillArgs& a, int quad, QRope<D, NT>& qr) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qr.w[c] = load16(a.q_w + 8 * quad + 32 * c);
}

template <int D, int NT>
__device__ __forceinline__ void load_rope(const PrefillArgs& a, int quad, const WaveQ<D, NT>& wq,
                                          QRope<D, NT>& qr) {
  load_rope_w<D, NT>(a, quad, qr);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // positions past the table (caller error) read its last row: in bounds
    const int pos = min(max(wq.pcol[nt], 0), a.max_pos - 1);
    const float* crow = a.cos_t + (size_t)pos * (D / 2) + 8 * quad;
    const float* srow = a.sin_t + (size_t)pos * (D / 2) + 8 * quad;
#pragma unroll
    for (int c = 0; c < D / 64; ++c)
#pragma unroll
      for (int j = 0; j < 8; j += 4) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(crow + 32 * c + j);
        const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + 32 * c + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qr.cs[nt][c][j + e] = cv[e];
          qr.sn[nt][c][j + e] = sv[e];
        }
      }
  }
}

// Lds: with G query heads per kv head the item's columns share each token's
// cos / sin rows G ways; staged once per item instead of loaded by every lane
// (G-fold redundant), they measured 0.45 us less per Qwen3 prefill call
// (48.27 -> 47.80 us).  The item's Q token rows (cos rows of tokens
// 0 .. Q-1, then the sin rows, D/8 16-byte units each: Q*D*4 bytes, at most
// one tile buffer) go to the second tile buffer, free until the key loop's
// first copy, with global-to-LDS copies issued beside q.  Unit u of token i
// sits at slot u ^ (i % (D/8)), so the reads of one dim group across tokens
// spread over the banks.
template <int D>
constexpr bool rope_stageable(int q_tokens) {
  return D <= 128 && q_tokens * D * 4 <= tile_bytes<D>();
}

template <int D>
__device__ __forceinline__ int rope_pos(const PrefillArgs& a, const Item& it, int i) {
  const int p = (i < it.nq && !it.idle) ? it.sp + it.i0 + i : 0;
  return min(p, a.max_pos - 1);  // positions past the table read its last row: in bounds
}

template <int D>
__device__ __forceinline__ void stage_rope(const PrefillArgs& a, const Item& it, uint8_t* buf, int lane, int w) {
  constexpr int U = D / 8;                   // 16-byte units per row
  const int Q = a.q_tokens, units = 2 * U * Q;
  const int n_copies = (units + 63) / 64;    // 1 KB each
  for (int k = w; k < n_copies; k += prefill_waves<D>()) {
    const int g = 64 * k + lane;
    const float* src = a.cos_t;  // (units past the rows: any in-bounds address)
    if (g < units) {
      const int tab = g / (U * Q), rem = g - tab * (U * Q), i = rem / U, slot = rem - i * U;
      const int unit = slot ^ (i % U);
      src = (tab ? a.sin_t : a.cos_t) + (size_t)rope_pos<D>(a, it, i) * (D / 2) + 4 * unit;
    }
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(buf + 1024 * k), 16, 0, 0);
  }
}

template <int D, int NT, RopeSrc SRC>
__device__ __forceinline__ void norm_rope_q(const PrefillArgs& a, int quad,
                                            const QRope<SRC == RopeSrc::Load ? 64 : D, NT>* qr,
                                            WaveQ<D, NT>& wq, const uint8_t* rope_lds, int w,
                                            int lane) {
  constexpr int C = D / 32;   // 16-byte chunks per lane
  constexpr int H = D / 64;   // chunks in the first half of the dims
  constexpr int U = D / 8;    // 16-byte units of a staged rotary row
  constexpr bool LDS = SRC == RopeSrc::Lds;
  auto wgt = [&](int c) {
    if constexpr (SRC == RopeSrc::Load) return load16(a.q_w + 8 * quad + 32 * c);
    else return qr->w[c];
  };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int pos = min(max(wq.pcol[nt], 0), a.max_pos - 1);
    const float* crow = a.cos_t + (size_t)pos * (D / 2) + 8 * quad;
    const float* srow = a.sin_t + (size_t)pos * (D / 2) + 8 * quad;
    // Lds: the column's token row i (columns without a query read token 0's
    // or the last staged row: their operand stays zero)
    float lcs[LDS ? H : 1][8], lsn[LDS ? H : 1][8];
    if constexpr (LDS) {
      // (an opaque lane index: these per-lane offsets are computed here, not
      // hoisted out of the item loop into registers held across the key loop)
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
      const int col = w * NT * 16 + nt * 16 + (lane_o & 15);
      const int i = min(wq.pcol[nt] < 0 ? 0 : col / a.G, a.q_tokens - 1);
      const float* ct = reinterpret_cast<const float*>(rope_lds) + (size_t)i * (D / 2);
      const float* st = ct + (size_t)a.q_tokens * (D / 2);
#pragma unroll
      for (int c = 0; c < H; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int unit = (2 * (lane_o >> 4) + 8 * c + h) ^ (i % U);
          const f32x4 cv = *reinterpret_cast<const f32x4*>(ct + 4 * unit);
          const f32x4 sv = *reinterpret_cast<const f32x4*>(st + 4 * unit);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lcs[c][4 * h + e] = cv[e];
            lsn[c][4 * h + e] = sv[e];
          }
        }
    }
    auto csv = [&](int c, int j) {
      if constexpr (LDS) return lcs[c][j];
      else if constexpr (SRC == RopeSrc::Regs) return qr->cs[nt][c][j];
      else return crow[32 * c + j];
    };
    auto snv = [&](int c, int j) {
      if constexpr (LDS) return lsn[c][j];
      else if constexpr (SRC == RopeSrc::Regs) return qr->sn[nt][c][j];
      else return srow[32 * c + j];
    };
    float x[C][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = bf16lo(wq.q[nt][c][e]);
        x[c][2 * e + 1] = bf16hi(wq.q[nt][c][e]);
        ss += x[c][2 * e] * x[c][2 * e] + x[c][2 * e + 1] * x[c][2 * e + 1];
      }
    ss = quad_sum(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const u32x4 wv = wgt(c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = x[c][2 * e] * inv * bf16lo(wv[e]);
        x[c][2 * e + 1] = x[c][2 * e + 1] * inv * bf16hi(wv[e]);
      }
    }
#pragma unroll
    for (int c = 0; c < H; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lo = x[c][j], hi = x[c + H][j], cs = csv(c, j), sn = snv(c, j);
        x[c][j] = lo * cs - hi * sn;
        x[c + H][j] = hi * cs + lo * sn;
      }
    if (wq.pcol[nt] < 0) continue;  // no query: the operand stays zero
#pragma unroll
    for (int c = 0; c < C; ++c)
      wq.q[nt][c] = u32x4{pack_bf16x2(x[c][0], x[c][1]), pack_bf16x2(x[c][2], x[c][3]),
                          pack_bf16x2(x[c][4], x[c][5]), pack_bf16x2(x[c][6], x[c][7])};
    if (a.q_out && wq.pcol[nt] < a.max_pos) {  // optional copy of q' (row of this column)
#pragma unroll
      for (int c = 0; c < C; ++c) store16(wq.qout_row[nt] + 32 * c, wq.q[nt][c]);
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void load_q(const PrefillArgs& a, const Item& it, int w, int lane,
                                       WaveQ<D, NT>& wq) {
  const int qc = lane & 15, quad = lane >> 4, G = a.G;
  const int first_col = w * NT * 16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = first_col + nt * 16 + qc;
    const int i = col / G, g = col - i * G;
    const bool valid = i < it.nq && !it.idle;
    wq.pcol[nt] = valid ? it.sp + it.i0 + i : -1;
    const size_t qoff = ((size_t)(it.a0 + it.i0 + (valid ? i : 0)) * a.n_q + it.hk * G + g) * D + 8 * quad;
    const bf16_t* qrow = a.q + qoff;
    wq.qout_row[nt] = a.q_out + qoff;  // (only dereferenced when q_out is given)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) wq.q[nt][c] = load16(qrow + 32 * c);  // (zeroed by mask_q)
  }
  wq.lo = 0x7fffffff;
  wq.hi = -1;
  const int i_lo = first_col / G;
  const int i_hi = min(it.nq - 1, (first_col + NT * 16 - 1) / G);
  if (!it.idle && i_lo < it.nq) {
    wq.lo = it.sp + it.i0 + i_lo;
    wq.hi = it.sp + it.i0 + i_hi;
  }
}

// Zeroes the operand of columns without a query (their loads re-read the
// block's first token).  Applied after the item's first wait, so that no
// use of q forces its loads to complete earlier.
template <int D, int NT>
__device__ __forceinline__ void mask_q(WaveQ<D, NT>& wq) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      if (wq.pcol[nt] < 0) wq.q[nt][c] = u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// Copies the chunk at j0 into LDS buffer buf: this wave's share of the K and
// V^T 1 KB blocks.  Keys past kv_hi (and unmapped pages) read page 0 or stay
// inside the chunk's page, so every address is inside the pool; the scores of
// such keys are masked and their V^T entries zeroed after the copy lands.
template <int D>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, const Item& it, const int* s_pg,
                                           uint8_t* lds, int buf, int j0, const LaneConst<D>& lc,
                                           int lane, int w) {
  const int ps = a.g.page_size, log2ps = a.g.log2ps;
  const size_t blk = (size_t)ps * D;
  const size_t page_stride = (size_t)a.g.n_kv * blk;
  const bf16_t* kbase = a.kpool + it.hk * blk;
  const bf16_t* vbase = a.vpool + it.hk * blk;
  uint8_t* tK = lds + buf * tile_bytes<D>();
  uint8_t* tV = tK + k_tile_bytes<D>();
  if (ps >= kChunk) {
    // The chunk lies inside one page: one (scalar) page id and source base;
    // the lane offsets within the page are fixed.
    int lane_o = lane;
    if constexpr (D >= 256) asm volatile("" : "+v"(lane_o));
    const int page = __builtin_amdgcn_readfirstlane(max(s_pg[(j0 >> log2ps) - it.pg0], 0));
    const size_t base = (size_t)page * page_stride;
    const int in_pg = j0 & (ps - 1);
    const uint8_t* ks = reinterpret_cast<const uint8_t*>(kbase + base + (size_t)in_pg * D);
    const uint8_t* vs = reinterpret_cast<const uint8_t*>(vbase + base + (size_t)in_pg * D);  // group in_pg/32
#pragma unroll
    for (int k = 0; k < dma_per_wave<D>(); ++k)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const bf16_t*>(ks + dma_k_off<D>(k, lane_o, w)),
                                       (lds_void_ptr)(tK + (w * dma_per_wave<D>() + k) * 1024),
                                       16, 0, 0);
#pragma unroll
    for (int k = 0; k < dma_per_wave<D>(); ++k)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const bf16_t*>(vs + dma_v_off<D>(k, lane_o, w)),
                                       (lds_void_ptr)(tV + (w * dma_per_wave<D>() + k) * 1024),
                                       16, 0, 0);
    return;
  }
  // Small pages: a page id per lane and copy (branch-free, so the page id
  // reads are issued together).
#pragma unroll
  for (int k = 0; k < dma_per_wave<D>(); ++k) {
    const int off = (int)dma_k_off<D>(k, lane, w);
    const int r = off / (2 * D), c8 = (off % (2 * D)) >> 1;  // row, first dim
    const int j = j0 + r;
    const int pgv = s_pg[min((j >> log2ps) - it.pg0, it.n_pg - 1)];
    const int page = j < it.kv_hi ? max(pgv, 0) : 0;
    const bf16_t* src = kbase + (size_t)page * page_stride + (size_t)(j & (ps - 1)) * D + c8;
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(tK + (w * dma_per_wave<D>() + k) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < dma_per_wave<D>(); ++k) {
    const int o = (w * dma_per_wave<D>() + k) * 1024 + 16 * lane;
    const int d = o >> 7, g = ((o >> 4) & 7) ^ v_swz(d);
    const int j = j0 + 8 * g;
    const int pgv = s_pg[min((j >> log2ps) - it.pg0, it.n_pg - 1)];
    const int page = j < it.kv_hi ? max(pgv, 0) : 0;
    const bf16_t* src = vbase + (size_t)page * page_stride + v_elem_offset(d, j & (ps - 1), D, log2ps);
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(tV + (w * dma_per_wave<D>() + k) * 1024), 16, 0, 0);
  }
}

// After a tail chunk lands: zero the V^T entries of keys >= kv_hi (stale page
// rows may hold anything, and 0 * NaN would poison P.V).  Returns whether it
// wrote (callers then place a barrier).
template <int D>
__device__ __forceinline__ bool zero_tail(uint8_t* lds, int buf, int j0, int kv_hi, int tid) {
  const int nvk = kv_hi - j0;
  if (nvk >= kChunk) return false;
  uint8_t* tV = lds + buf * tile_bytes<D>() + k_tile_bytes<D>();
  for (int idx = tid; idx < D * 8; idx += prefill_threads<D>()) {
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
  return true;
}

// ---------------------------------------------------------------------------
// Online-softmax state of a wave's NT column tiles.
template <int D, int NT>
struct SoftmaxAcc {
  f32x4 o[NT][D / 16];  // O^T accumulators: lane rows d = vrow(dt, 4*(lane/16) + r), column lane%16
  float m_run[NT];      // reference max (log2 units)
  float neg_m[NT];      // -m_run (0 while m_run = -inf)
  float thr[NT];        // raw-score threshold (m_run + 8) / c above which m_run must move
  float l_run[NT];      // this lane's share of the row sum
};

template <int D, int NT>
__device__ __forceinline__ void acc_init(SoftmaxAcc<D, NT>& s) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    s.m_run[nt] = -INFINITY;
    s.neg_m[nt] = 0.f;
    s.thr[nt] = -INFINITY;
    s.l_run[nt] = 0.f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) s.o[nt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// One 64-key chunk (keys j0 ..) from LDS buffer offset buf_off for this wave.
// NH = the 32-key halves that hold a key some query of this wave sees (1:
// the second half lies past the wave's last query position, as in the last
// chunk of every query block that starts at a multiple of 64; its MFMAs and
// exponentials are skipped).
template <int D, int NT, int NH>
__device__ __forceinline__ void chunk_halves(const PrefillArgs& a, const uint8_t* lds, int buf_off,
                                             int j0, const LaneConst<D>& lc, const WaveQ<D, NT>& wq,
                                             int quad, float inv_c, bool full, SoftmaxAcc<D, NT>& sa) {
  // Scheduling hint for the QK^T block: the compiler's MFMA / LDS-read
  // interleaving strategy 1 (measured 44.8 -> 43.8 us on the Qwen3 prompts;
  // strategy 0, or the hint on the P.V blocks too, were slower).
  __builtin_amdgcn_iglp_opt(1);
  // ---- S^T = K Q^T for the chunk's two 32-key halves h: MFMA rg row m holds
  // key j0 + 32h + 8*(m/4) + 4*rg + m%4
  f32x4 S[NH][NT][2];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(lds + ((buf_off + lc.kofs[h][rg]) ^ (64 * c)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          S[h][nt][rg] = mfma16x16x32(kv, wq.q[nt][c], c ? S[h][nt][rg] : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
  // ---- element mask, only on chunks crossing the diagonal or the window edge
  if (!full) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int pc = wq.pcol[nt];
      const int jmin = a.window > 0 ? pc - a.window + 1 : -0x7fffffff;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = j0 + 32 * h + 8 * quad + 4 * rg + e;
            if (j > pc || j < jmin) S[h][nt][rg][e] = -INFINITY;
          }
    }
  }
  // ---- softmax against a lazily moved per-column reference max m_run:
  // p = 2^(s*c - m_run).  m_run (with O and l rescaled) only moves when a
  // score exceeds it by more than 2^8, which the common path detects with a
  // per-lane compare against the column threshold (m_run + 8) / c -- no
  // cross-lane work unless some lane of the wave crosses it.
  float lmax[NT];
  bool need = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lmax[nt] = NH == 2 ? vmax(max8(S[0][nt]), max8(S[NH - 1][nt])) : max8(S[0][nt]);
    need |= lmax[nt] > sa.thr[nt];
  }
  if (__any(need)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mx = quad_max(lmax[nt]);  // max over the column's 64 keys
      const float m_new = fmaxf(sa.m_run[nt], mx * a.scale_log2);
      float alpha = 1.0f;
      if (m_new > sa.m_run[nt] + 8.0f) {
        alpha = fast_exp2(sa.m_run[nt] - m_new);  // 0 when m_run was -inf
        sa.m_run[nt] = m_new;
        sa.neg_m[nt] = -m_new;
        sa.thr[nt] = (m_new + 8.0f) * inv_c;
      }
      sa.l_run[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) sa.o[nt][dt] *= alpha;
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    u32x4 pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(S[h][nt][e >> 2][e & 3], a.scale_log2, sa.neg_m[nt]));
      pb[nt] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      // fp32 row sum (summing the bf16 weights instead would cost the
      // log-sum-exp up to 2^-9 of relative accuracy)
      sa.l_run[nt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    // ---- O^T += V^T P^T for this half; lane A row = V^T row vrow(dt, qc), keys group 4h + quad
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x4 vv = *reinterpret_cast<const u32x4*>(lds + buf_off + lc.vofs[h] + vrow_step(dt) * 128);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sa.o[nt][dt] = mfma16x16x32(vv, pb[nt], sa.o[nt][dt]);
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void chunk_math(const PrefillArgs& a, const uint8_t* lds, int buf_off,
                                           int j0, const LaneConst<D>& lc, const WaveQ<D, NT>& wq,
                                           int quad, float inv_c, SoftmaxAcc<D, NT>& sa) {
  const bool skip = wq.hi < 0 || j0 > wq.hi || (a.window > 0 && j0 + kChunk - 1 <= wq.lo - a.window);
  if (skip) return;
  const bool full = (j0 + kChunk - 1 <= wq.lo) && (a.window <= 0 || wq.hi - j0 < a.window);
  if (j0 + 32 <= wq.hi)
    chunk_halves<D, NT, 2>(a, lds, buf_off, j0, lc, wq, quad, inv_c, full, sa);
  else
    chunk_halves<D, NT, 1>(a, lds, buf_off, j0, lc, wq, quad, inv_c, full, sa);
}

// Normalise and store the wave's columns of an item (padding rows: 0 / -inf).
template <int D, int NT>
__device__ __forceinline__ void store_out(const PrefillArgs& a, const Item& it, int w, int lane,
                                          const SoftmaxAcc<D, NT>& sa) {
  // (an opaque copy of the lane index: the per-lane row offsets are computed
  // here, once per item, instead of being hoisted out of the item loop into
  // registers held across the key loop -- a spill in the fused-q instance)
  int lane_o = lane;
  asm volatile("" : "+v"(lane_o));
  const int qc = lane_o & 15, quad = lane_o >> 4, G = a.G;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = sa.l_run[nt];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const int col = w * NT * 16 + nt * 16 + qc;
    const int i = col / G, g = col - i * G;
    if (i >= it.nq) continue;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    bf16_t* orow = a.out + ((size_t)(it.a0 + it.i0 + i) * a.n_q + it.hk * G + g) * D;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {  // dims 32k + 8*quad .. +7 (see vrow)
      const f32x4 o0 = sa.o[nt][2 * k], o1 = sa.o[nt][2 * k + 1];
      store16(orow + 32 * k + 8 * quad,
              u32x4{pack_bf16x2(o0[0] * inv, o0[1] * inv), pack_bf16x2(o0[2] * inv, o0[3] * inv),
                    pack_bf16x2(o1[0] * inv, o1[1] * inv), pack_bf16x2(o1[2] * inv, o1[3] * inv)});
    }
    if (a.lse && quad == 0)
      a.lse[(size_t)(it.a0 + it.i0 + i) * a.n_q + it.hk * G + g] =
          l > 0.f ? (sa.m_run[nt] + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// One work item end to end: stage its page ids, stream its key chunks through
// the two LDS tile buffers (the next chunk's copy in flight while the current
// one is computed), normalise and store.
// QM: q arrives rotated (kQReady) or raw, getting the fused Qwen3 norm +
// rotation (norm_rope_q) with its rotary rows in registers (kQRope) or
// staged in LDS (kQRopeLds).
template <int D, int NT, int QM>
__device__ __forceinline__ void run_item(const PrefillArgs& a, const SeqMeta& sm, int hk, int n, int qb,
                                         uint8_t* lds, int* s_pg, const LaneConst<D>& lc,
                                         int tid, int lane, int w, float inv_c) {
  const int quad = lane >> 4;
  Item it;
  item_init(a, sm, hk, n, qb, it);
  // The first key chunk's copies go out first and q (and the transform's
  // inputs) right behind them: one memory round trip before the key loop.
  // (The page ids were staged for the whole sequence; the previous item's
  // loop ended with a barrier, so both tile buffers are free.)  The transform
  // cannot run under the chunk's copies instead: the compiler counts no
  // global-to-LDS copy among the loads in flight, so q's first use waits for
  // every one of them whatever the order.
  if (it.n_chunks > 0) issue_tile<D>(a, it, s_pg, lds, 0, it.j_start, lc, lane, w);
  WaveQ<D, NT> wq;
  load_q<D, NT>(a, it, w, lane, wq);
  constexpr RopeSrc SRC = QM == kQRopeLds ? RopeSrc::Lds : D <= 128 ? RopeSrc::Regs : RopeSrc::Load;
  QRope<(QM != kQReady && SRC != RopeSrc::Load) ? D : 64, NT> qr;
  uint8_t* const rope_buf = lds + tile_bytes<D>();  // the second tile buffer
  if constexpr (QM == kQRope && SRC == RopeSrc::Regs) load_rope<D, NT>(a, quad, wq, qr);
  if constexpr (QM == kQRopeLds) {
    stage_rope<D>(a, it, rope_buf, lane, w);
    load_rope_w<D, NT>(a, quad, qr);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the first chunk, q and the transform's inputs have landed
  __syncthreads();
  mask_q<D, NT>(wq);
  if constexpr (QM != kQReady) {
    norm_rope_q<D, NT, SRC>(a, quad, &qr, wq, rope_buf, w, lane);
    // every wave has read the staged rows before the key loop's copies
    if constexpr (QM == kQRopeLds) __syncthreads();
  }
  // (the accumulators start after the q transform, which would otherwise
  // hold them alongside its own working set)
  SoftmaxAcc<D, NT> sa;
  acc_init(sa);
  if (it.n_chunks > 0 && zero_tail<D>(lds, 0, it.j_start, it.kv_hi, tid)) __syncthreads();
  constexpr int NB = prefill_bufs<D>();
  for (int ck = 0; ck < it.n_chunks; ++ck) {
    const int j0 = it.j_start + ck * kChunk;
    const int nbuf = (ck + 1) & (NB - 1);  // buffer of the next chunk
    if (NB == 2 && ck + 1 < it.n_chunks) issue_tile<D>(a, it, s_pg, lds, nbuf, j0 + kChunk, lc, lane, w);
    chunk_math<D, NT>(a, lds, (ck & (NB - 1)) * tile_bytes<D>(), j0, lc, wq, quad, inv_c, sa);
    if (NB == 1 && ck + 1 < it.n_chunks) {
      __syncthreads();  // every wave is done with the single buffer
      issue_tile<D>(a, it, s_pg, lds, 0, j0 + kChunk, lc, lane, w);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the next chunk's copies have landed
    __syncthreads();
    if (ck + 1 < it.n_chunks && zero_tail<D>(lds, nbuf, j0 + kChunk, it.kv_hi, tid))
      __syncthreads();
  }
  store_out<D, NT>(a, it, w, lane, sa);
}

// ---------------------------------------------------------------------------
// One workgroup per (kv head, sequence, layer of query blocks); layers run
// from the last query block down, so the longest items start first (a
// workgroup whose layer exceeds its sequence's block count exits at once).
// Grid x = kv head: with n_kv a multiple of 8 the XCDs (every 8th workgroup)
// each keep their heads' K/V in their own L2.
template <int D, int NT, int QM>
__global__ __launch_bounds__(prefill_threads<D>())
__attribute__((amdgpu_waves_per_eu(prefill_wpe<D>(), prefill_wpe<D>())))
void prefill_kernel(const int32_t* cu_seqlens, const int32_t* slots, const int32_t* start_pos,
                    const int32_t* table, int n_seqs, PrefillArgs a) {
  // cu_seqlens .. n_seqs repeat fields of `a`: passed first, they arrive
  // preloaded in scalar registers (the library builds this file with five
  // preloaded kernel arguments), so the sequence metadata loads issue at once.
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_pg[kStagePages];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float inv_c = 1.0f / a.scale_log2;  // scale > 0 (host-checked)
  LaneConst<D> lc;
  lane_const<D>(lc, lane, w, a.g.page_size);
  const int hk = blockIdx.x, n = blockIdx.y;
  if (n >= n_seqs) return;  // padding row of the grid (odd y extent)
  const SeqMeta sm = seq_meta(a, n, cu_seqlens, slots, start_pos);
  const int nblk = (sm.len + a.q_tokens - 1) / a.q_tokens;
  if (nblk <= a.n_qblocks - 1 - (int)blockIdx.z) return;  // no item in this layer
  {
    const int32_t* trow = table + (size_t)max(sm.slot, 0) * a.pt.pps;
    for (int i = tid; i < sm.n_pg; i += prefill_threads<D>()) s_pg[i] = checked_page(trow[i], a.g.n_pages);
    __syncthreads();
  }
  for (int qb = a.n_qblocks - 1 - (int)blockIdx.z; qb < nblk; qb += a.n_qblocks)
    run_item<D, NT, QM>(a, sm, hk, n, qb, lds, s_pg, lc, tid, lane, w, inv_c);
}

// ---------------------------------------------------------------------------
template <typename K>
hipError_t set_lds_limit(K* kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, int QM>
hipError_t launch_prefill_qm(const PrefillArgs& a, hipStream_t st) {
  constexpr int NT = prefill_nt<D>();
  const int lds = prefill_bufs<D>() * tile_bytes<D>();
  static const hipError_t attr = set_lds_limit(&prefill_kernel<D, NT, QM>, lds);
  if (attr != hipSuccess) return attr;
  // An XCD hands its workgroups to its 4 shader engines round-robin and
  // dispatches in order, stalling when the next workgroup's engine is full.
  // With an even y extent every layer would send the same sequences to the
  // same engine (engine = sequence mod 4 when the kv heads fill the XCDs), so
  // long prompts pile onto one engine; an odd extent rotates each sequence
  // across the engines layer by layer (measured 10% faster on ragged
  // batches).  (A 1-D grid in exact cost order, mapped in-kernel, balanced
  // the engines too but its per-workgroup set-up cost more than it saved.)
  dim3 grid(a.g.n_kv, a.n_seqs | 1, a.n_qblocks);
  hipLaunchKernelGGL((prefill_kernel<D, NT, QM>), grid, dim3(prefill_threads<D>()), lds, st,
                     a.cu_seqlens, a.slots, a.start_pos, a.pt.table, a.n_seqs, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t st) {
  if (!a.q_w) return launch_prefill_qm<D, kQReady>(a, st);
  if constexpr (D <= 128)
    if (rope_stageable<D>(a.q_tokens)) return launch_prefill_qm<D, kQRopeLds>(a, st);
  return launch_prefill_qm<D, kQRope>(a, st);
}

}  // namespace

int prefill_q_tokens(int G, int head_dim) {
  switch (head_dim) {
    case 64: return prefill_waves<64>() * prefill_nt<64>() * 16 / G;
    case 128: return prefill_waves<128>() * prefill_nt<128>() * 16 / G;
    case 256: return prefill_waves<256>() * prefill_nt<256>() * 16 / G;
    default: return prefill_waves<512>() * prefill_nt<512>() * 16 / G;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.head_dim) {
    case 64: return launch_prefill_d<64>(a, st);
    case 128: return launch_prefill_d<128>(a, st);
    case 256: return launch_prefill_d<256>(a, st);
    case 512: return launch_prefill_d<512>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
