// Internal host <-> kernel interface: argument blocks passed by value to the
// kernels and the launchers each kernel file exports to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

typedef uint16_t bf16_t;

constexpr float kLog2eHost = 1.4426950408889634f;

struct PoolGeom {
  int n_pages;
  int page_size;
  int log2ps;
  int n_kv;
  int head_dim;
};

// V pool block of one (page, kv head): its rows are split into groups of
// kVGroup consecutive keys (the whole page when page_size is smaller), and
// each group is stored d-major: element (d, row) at
// ((row / gs) * head_dim + d) * gs + row % gs, gs = min(page_size, kVGroup).
// A 32-key group of one dim is 64 contiguous bytes and a whole group is one
// contiguous head_dim * 64-byte block.
constexpr int kVGroup = 32;
constexpr int kLog2VGroup = 5;

__host__ __device__ inline size_t v_elem_offset(int d, int row, int head_dim, int log2ps) {
  const int lg = log2ps < kLog2VGroup ? log2ps : kLog2VGroup;
  return (((size_t)(row >> lg) * head_dim + d) << lg) + (row & ((1 << lg) - 1));
}

struct TableRef {
  const int32_t* table;
  int max_slots;
  int pps;  // pages per slot (row stride)
};

struct AppendArgs {
  const bf16_t* k_new;
  const bf16_t* v_new;
  const int32_t* slot;
  const int32_t* pos;
  int T;
  TableRef pt;
  PoolGeom g;
  bf16_t* kpool;
  bf16_t* vpool;
};

struct DecodeArgs {
  const bf16_t* q;
  int n_q;
  int G;  // query heads per kv head
  const int32_t* slots;
  const int32_t* seq_lens;
  int B;
  TableRef pt;
  PoolGeom g;
  const bf16_t* kpool;
  const bf16_t* vpool;
  bf16_t* kpool_w;       // same pools, written by the fused append
  bf16_t* vpool_w;
  const bf16_t* k_new;   // [B][n_kv][D] new token K, or null (no fused append)
  const bf16_t* v_new;
  float scale_log2;      // softmax scale * log2(e)
  int window;
  int split_tokens;      // keys per split (multiple of 128)
  int head_tokens;       // keys of split 0 on full-causal rows (<= split_tokens)
  int max_splits;        // grid extent; 1 = no workspace, write out directly
  uint32_t* part_o;      // [B][n_kv][max_splits][G][D/2] bf16 pairs of the split's o / l
  float* part_ml;        // [B][n_kv][max_splits][G][2]  (running max in log2 units, sum)
  uint32_t* arrivals_end;  // one past the split arrival counters: pair b*n_kv+hk at
                           // arrivals_end[-1 - (b*n_kv+hk)] (the workspace's last bytes)
  bf16_t* out;           // [B][n_q][D]
  float* lse;            // [B][n_q] or null
  // (host side, last so that the fields above keep their offsets) kernel
  // instance selection: v_late, the key-split instance whose split 0 writes
  // the fused append's new V at its end (and merges early); early_merge, the
  // dim-split instance whose split 0 merges early
  int v_late;
  int early_merge;
};

// The prologue kernel handles k (normalise, rotate, append) and v (append);
// q's normalisation and rotation run inside the prefill attention kernel.
struct PrologueArgs {
  const bf16_t* k_raw;
  const bf16_t* v_raw;
  const bf16_t* k_w;
  int v_norm;  // 1: v <- RMSNorm(v) without a gain before the append
  float eps;
  const float* cos_t;
  const float* sin_t;
  int max_pos;
  int T;
  const int32_t* cu_seqlens;
  const int32_t* slots;
  const int32_t* start_pos;  // may be null
  int n_seqs;
  TableRef pt;
  PoolGeom g;
  bf16_t* kpool;
  bf16_t* vpool;
};

struct PrefillArgs {
  const bf16_t* q;  // [T][n_q][D]
  int n_q;
  int G;
  const int32_t* cu_seqlens;
  const int32_t* slots;
  const int32_t* start_pos;  // may be null
  int n_seqs;
  TableRef pt;
  PoolGeom g;
  const bf16_t* kpool;
  const bf16_t* vpool;
  float scale_log2;
  int window;
  int q_tokens;   // query tokens per work item
  int n_qblocks;  // grid extent over query blocks (grid-stride beyond it)
  bf16_t* out;
  float* lse;
  // Fused q RMSNorm * q_w + RoPE (q_w != null): q is read raw and transformed
  // in registers; cos / sin rows [max_pos][D/2] fp32.
  const bf16_t* q_w;
  const float* cos_t;
  const float* sin_t;
  float eps;
  int max_pos;
  bf16_t* q_out;  // optional copy of the transformed q' ([T][n_q][D])
};

// Validation mode flags (see pkv_validation_flags in the public header).
constexpr uint32_t kValidateSlot = 1u;
constexpr uint32_t kValidatePage = 2u;
constexpr uint32_t kValidatePos = 4u;

hipError_t launch_validate_rows(const TableRef& pt, const PoolGeom& g, const int32_t* slots,
                                const int32_t* seq_lens, const int32_t* cu_seqlens,
                                const int32_t* start_pos, int n, hipStream_t st);
hipError_t launch_validate_tokens(const TableRef& pt, const PoolGeom& g, const int32_t* slot,
                                  const int32_t* pos, int T, hipStream_t st);
hipError_t read_validate_flags(uint32_t* host_out, int clear, hipStream_t st);

// Device-side batch reserve and erase (see pkv_pt_device_reserve and
// pkv_pt_device_erase in the public header).
struct ReserveArgs {
  int32_t* table;
  int32_t* free_pages;
  int32_t* free_count;
  int32_t* capacity;
  uint32_t* status;
  const int32_t* slots;
  const int32_t* seq_lens;
  int B, max_slots, pps, page_size, n_pages;
};
constexpr uint32_t kReserveNoPages = 1u;
constexpr uint32_t kReserveTooLong = 2u;
constexpr uint32_t kReserveBadState = 4u;
hipError_t launch_reserve(const ReserveArgs& a, hipStream_t st);
hipError_t launch_erase(const ReserveArgs& a, hipStream_t st);  // seq_lens unused

hipError_t launch_append(const AppendArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);
hipError_t launch_rope_table(float* c, float* s, int max_pos, int head_dim, double theta,
                             int n_rot, hipStream_t st);

// Split-K plan for decode (host): keys per split and grid extent.
struct DecodePlan {
  int split_tokens;
  int head_tokens;
  int v_late;
  int early_merge;
  int max_splits;
  size_t ws_bytes;
  size_t part_o_words;   // partial outputs first (bf16 pairs), then the fp32 (max, sum) pairs
};
DecodePlan plan_decode(int B, int n_q, int n_kv, int head_dim, int max_seq_len_hint,
                       int window);

// A decode workspace of ws bytes keeps its last decode_counter_region(ws)
// bytes for the arrival counters of every call that uses it, whatever that
// call's shape; the split partials stay below that region.  (With counters
// simply after each call's own partials, a call of another shape could write
// partials over counters that a later call relies on being zero.)
inline size_t decode_counter_region(size_t ws) { return (ws / 16) & ~(size_t)15; }

// Static split-K scratch of pkv_attn_decode_noalloc: one buffer of this many
// bytes per device, inside the library's code object.  decode_scratch gives
// the current device's copy (its address is looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);

// Query tokens per prefill workgroup for a GQA ratio.
int prefill_q_tokens(int G, int head_dim);


}  // namespace pkv
