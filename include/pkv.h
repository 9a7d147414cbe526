/*
 * pkv.h -- C ABI of the paged KV-cache attention library for AMD MI355X (gfx950).
 *
 * The library appends new K/V rows into a paged cache addressed through a page
 * table, and runs grouped-query attention over that cache for decode (one new
 * query token per batch row) and for packed variable-length prefill (causal,
 * optionally sliding-window, each sequence seeing only its own slot).  Every
 * step runs in hand-written HIP kernels for gfx950.
 *
 * Pages cited below (a section is a file shown on that page):
 *   [moe-qwen3 compare]
 *     https://git.jhoeven.net/ceos/unsloth/compare/main...danielhanchen/flex-moe-qwen3
 *   [continuous-batching compare]
 *     https://git.jhoeven.net/ceos/unsloth/compare/main...transformers-continuous-batching-qwen3
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 tensors are passed as `void*` to 16-bit storage (IEEE bfloat16).
 *   The kernels move rows in 16-byte units: every bf16 buffer argument (and
 *   the fp32 rotary tables) must be 16-byte aligned, else the call returns
 *   PKV_ERR_INVALID_ARG.
 * - "device" pointers must be device memory of the current HIP device (or
 *   memory the device can read/write); "host" pointers are plain host memory.
 * - Ownership: the caller owns every buffer.  Compute entry points never
 *   allocate, free or synchronise, and keep no device state between calls.
 *   They only enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *   stream) and return; results are ready when the stream reaches them.
 * - Errors: arguments are checked on the host before anything is enqueued;
 *   on a bad argument the call returns a non-zero pkv_status, enqueues nothing
 *   and leaves a message for pkv_last_error().  Device-side contents (page ids,
 *   lengths, slots) cannot be checked on the host; the kernels bounds-check
 *   them instead and never read or write outside the buffers described here:
 *   a page id outside [1, n_pages), a slot outside [1, max_slots) or a
 *   position beyond pages_per_slot*page_size is skipped (append) or treated
 *   as an idle row / absent key (attention).  Such inputs are caller errors
 *   and their results are unspecified, but never out of bounds.
 *
 * Cache layout (one K pool and one V pool per layer, same page geometry):
 *   K pool: bf16 [n_pages][n_kv_heads][page_size][head_dim]   (token rows)
 *   V pool: bf16 [n_pages][n_kv_heads][page_size/gs][head_dim][gs],
 *           gs = min(page_size, 32): the page's rows in groups of 32 keys,
 *           each group d-major (element (d, row) at group row/gs, [d][row%gs])
 *   The pages' cache is a single (1, H, n_pages*page_size, D) buffer per K/V
 *   ([continuous-batching compare] flex_paged_attention.py, PagedKVCache);
 *   here pages are the outer dimension so one (page, head) block is contiguous,
 *   and V is stored d-major inside 32-key groups so the P.V contraction can
 *   feed the matrix cores straight from memory, with one wave's 32 keys of V
 *   one contiguous block.  For page_size <= 32 this is plain d-major pages.
 *
 * Page table ([continuous-batching compare] flex_paged_attention.py, PageTable):
 *   int32 [max_slots][pages_per_slot], entry = physical page of
 *   (slot, logical page), -1 = unmapped.  Token at logical position `pos` of
 *   `slot` lives in page table[slot][pos / page_size], row pos % page_size.
 *   Slot 0 is the reserved no-op slot: it is never read or written.  Page 0
 *   is reserved and never handed out by the allocator below.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent shapes       */
  PKV_ERR_UNSUPPORTED = 2,  /* head_dim / page_size / GQA ratio not implemented    */
  PKV_ERR_LAUNCH = 3,       /* a kernel launch failed (HIP error text attached)   */
  PKV_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required         */
  PKV_ERR_CAPACITY = 5      /* allocator: no free slot / not enough free pages     */
} pkv_status;

/* One layer's pools.  Supported: head_dim in {64, 128, 256, 512};
 * page_size a power of two in [16, 256]; n_pages >= 2. */
typedef struct {
  int32_t n_pages;     /* physical pages, including reserved page 0 */
  int32_t page_size;   /* tokens per page                            */
  int32_t n_kv_heads;
  int32_t head_dim;
} pkv_cache_desc;

/* Device page table (see layout above). */
typedef struct {
  const int32_t* table;   /* device, int32 [max_slots][pages_per_slot]        */
  int32_t max_slots;      /* usable slots + 1 (slot 0 reserved)               */
  int32_t pages_per_slot; /* row stride, in entries                           */
} pkv_page_table;

/* Fused attention prologue for prefill (Qwen3; Gemma-4 with v_norm): per
 * token and head,
 *   x <- RMSNorm(x) * w  over head_dim  (fp32: x / sqrt(mean(x^2) + eps) * w)
 *   x <- x * cos + rotate_half(x) * sin, rotate_half(x) = (-x[D/2:], x[:D/2])
 * applied to k, which is then appended to the pages with v (raw, or with
 * v_norm its RMSNorm without a gain), and to q inside the attention kernel as
 * it loads q (q in memory is not modified).  Order and formulas:
 * [moe-qwen3 compare] unsloth/inference/flex_gemma4_moe.py, attention
 * forward (q_norm / k_norm / v_norm, then rotary, then the paged-KV write)
 * and _rotate_half / _apply_rotary_full.
 * The cos/sin tables are fp32 [max_pos][head_dim/2] (see pkv_rope_table); a
 * token at position p uses row p.  Positions >= max_pos are a caller error:
 * such a token's k is not appended and its q reads row max_pos-1 (in bounds;
 * its results are unspecified). */
typedef struct {
  const void* q_norm_w;   /* device bf16 [head_dim]                     */
  const void* k_norm_w;   /* device bf16 [head_dim]                     */
  float eps;              /* RMSNorm epsilon (Qwen3: 1e-6)              */
  const float* rope_cos;  /* device fp32 [max_pos][head_dim/2]          */
  const float* rope_sin;  /* device fp32 [max_pos][head_dim/2]          */
  int32_t max_pos;
  const void* k_raw;      /* device bf16 [total_tokens][n_kv][head_dim] */
  const void* v_raw;      /* device bf16 [total_tokens][n_kv][head_dim].
                             k_raw and v_raw both NULL: nothing is appended
                             (the keys are already in the pages, e.g. from an
                             earlier call) and only q is normalised and
                             rotated; k_norm_w and v_norm are then unused */
  void* q_out;            /* device bf16 [total_tokens][n_q][head_dim] or NULL:
                             where given, the normalised and rotated q' is
                             also written there (rows of padding sequences and
                             of positions >= max_pos are left untouched) */
  int32_t v_norm;         /* 0: v appended raw (Qwen3); 1: v <- RMSNorm(v)
                             without a gain before the append (Gemma-4
                             v_norm).  For Gemma-4's K=V layers pass the raw
                             k as v_raw. */
} pkv_prologue;

/* ---------------------------------------------------------------------------
 * pkv_append -- scatter T new K/V rows into the pools (bit copy).
 * [continuous-batching compare] flex_paged_attention.py, PageTable.assign
 * (decode form, one token per batch row) and assign_prefill_no_paging (packed
 * prefill form): token t goes to page table[slot[t]][pos[t] / page_size], row
 * pos[t] % page_size, of kv head h, for every h.
 *   k_new, v_new : device bf16 [T][n_kv_heads][head_dim]
 *   slot, pos    : device int32 [T]; slot 0 = no-op token (skipped)
 *   k_pool/v_pool: device bf16 pools (layout above), written in place
 * Two tokens with the same (slot, pos) in one call: unspecified which wins.
 * T == 0 is a no-op.
 */
pkv_status pkv_append(const void* k_new, const void* v_new, const int32_t* slot,
                      const int32_t* pos, int32_t T, pkv_page_table pt,
                      const pkv_cache_desc* cd, void* k_pool, void* v_pool, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_attn_decode -- one query token per batch row against its slot's pages,
 * optionally appending that token's K/V first (fused append).
 * Masks: the query sits at position L-1 (L = seq_lens[b], the key count after
 * the append) and sees key j iff j <= L-1 and, with window W > 0, L-1-j < W
 * ([continuous-batching compare] flex_paged_attention.py,
 * create_causal_blockmask; [moe-qwen3 compare] flex_gemma4_moe.py,
 * _decode_block_mask and _create_sliding_causal_blockmask).  GQA: query head
 * h reads kv head h / (n_q_heads / n_kv_heads).
 * Numerics: scores, softmax sums and P.V accumulate in fp32 (the softmax
 * weights enter the P.V product as bf16).  A row split across workgroups
 * hands each split's normalised output to the merging one as bf16, with its
 * maximum and sum in fp32; the merge runs in fp32.
 *   q        : device bf16 [B][n_q_heads][head_dim]
 *   slots    : device int32 [B]; seq_lens: device int32 [B]
 *              rows with slot 0 or seq_len 0 are idle: out = 0, lse = -inf,
 *              nothing read or written ([continuous-batching compare] results
 *              write-up: padded rows must come out as zeros, not NaN)
 *   max_seq_len_hint : host int >= 1, an upper bound of seq_lens used to size
 *              the split-K grid (results stay correct if exceeded; only speed
 *              changes)
 *   k_pool, v_pool : device pools; written only when k_new / v_new are given
 *   k_new, v_new : device bf16 [B][n_kv_heads][head_dim] or both NULL.  When
 *              given, each active row's new token is first written at position
 *              L-1 of its slot, exactly as pkv_append would (the decode form of
 *              PageTable.assign), and then attended.
 *   scale    : softmax scale applied to q.k (e.g. 1/sqrt(head_dim))
 *   window   : 0 = full causal, W > 0 = sliding window of W keys incl. self
 *   out      : device bf16 [B][n_q_heads][head_dim]
 *   lse      : device fp32 [B][n_q_heads] natural-log sum-exp, or NULL
 *   workspace: device scratch of >= pkv_decode_workspace_size(...) bytes,
 *              16-byte aligned (NULL allowed when that size is 0).  It holds
 *              the split partials (from its start; no initialisation needed)
 *              and one arrival counter per (row, kv head) in its last
 *              4 * B * n_kv_heads bytes: the splits of a (row, kv head) count
 *              themselves in there and the last one merges.  Zero the whole
 *              workspace once when it is created (before its first call,
 *              outside any graph capture); every call leaves its counters at
 *              zero again.  The counters are addressed back from
 *              workspace + workspace_bytes, and whatever the call's shape
 *              they lie in the workspace's last (workspace_bytes / 16,
 *              rounded down to 16) bytes, which no call's partials reach:
 *              calls of different shapes may share a workspace, passed with
 *              the same workspace_bytes each time and at least the size each
 *              of them needs.  Calls that overlap in time (other streams,
 *              other graphs) need separate workspaces; calls with separate
 *              workspaces share nothing.
 * n_q_heads / n_kv_heads must be an integer G in [1, 16] with G * head_dim <= 2048
 * (PKV_ERR_UNSUPPORTED otherwise).  B == 0 is a no-op.
 */
pkv_status pkv_attn_decode(const void* q, int32_t n_q_heads, const int32_t* slots,
                           const int32_t* seq_lens, int32_t B, int32_t max_seq_len_hint,
                           pkv_page_table pt, const pkv_cache_desc* cd, void* k_pool,
                           void* v_pool, const void* k_new, const void* v_new, float scale,
                           int32_t window, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_attn_decode_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture with no allocator at hand, tight serving
 * loops, harnesses that forbid hipMalloc): pkv_attn_decode with the split
 * partials and arrival counters in a static scratch buffer inside the
 * library instead of a workspace argument.  Same arguments, semantics and
 * kernels as pkv_attn_decode (its results are bitwise those of
 * pkv_attn_decode for the same inputs); the caller still passes every input
 * and output.  The call allocates nothing and calls no allocating routine.
 * - The buffer is PKV_DECODE_SCRATCH_BYTES (16 MiB) per device, held by each
 *   device the library runs on until the process ends.  A call whose split
 *   plan needs more (pkv_decode_workspace_size(...) above the limit) returns
 *   PKV_ERR_WORKSPACE and enqueues nothing.
 * - Every call on a device shares that device's buffer and leaves its
 *   arrival counters at zero (they are zero when the library is loaded);
 *   calls that overlap in time on one device (other streams, graphs
 *   replayed concurrently) race and give undefined results.  Use
 *   pkv_attn_decode with separate workspaces for concurrent calls.
 * - The first call on a device looks the buffer's address up
 *   (hipGetSymbolAddress; PKV_ERR_LAUNCH if that fails).
 */
#define PKV_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
pkv_status pkv_attn_decode_noalloc(const void* q, int32_t n_q_heads, const int32_t* slots,
                                   const int32_t* seq_lens, int32_t B,
                                   int32_t max_seq_len_hint, pkv_page_table pt,
                                   const pkv_cache_desc* cd, void* k_pool, void* v_pool,
                                   const void* k_new, const void* v_new, float scale,
                                   int32_t window, void* out, float* lse, void* stream);

/* Bytes of workspace pkv_attn_decode needs for these sizes (0 = none): the
 * split partials, and a last sixteenth (at least 4 * B * n_kv_heads bytes) for
 * the arrival counters that the partials of no call reach. */
size_t pkv_decode_workspace_size(int32_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len_hint,
                                 int32_t window);

/* The split-K plan pkv_attn_decode makes for these sizes (host only, for
 * inspection and tests): out[0] keys per split, out[1] keys of split 0 on
 * full-causal rows, out[2] grid splits per (row, kv head), out[3] 1 when
 * split 0 writes the fused append's new V (large grids), out[4] 1 when split
 * 0 merges at once if the other splits are in, out[5] workspace bytes.
 * out: host int64[6].  PKV_ERR_INVALID_ARG for a NULL out or sizes the
 * decode call would reject as invalid (B, heads <= 0, n_q_heads not a
 * multiple of n_kv_heads). */
pkv_status pkv_decode_plan(int32_t B, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t max_seq_len_hint, int32_t window, int64_t* out);

/* ---------------------------------------------------------------------------
 * pkv_attn_prefill -- packed varlen prefill, K/V read from the pages.
 * Sequence n owns packed tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of slot
 * slots[n]; its query i sits at position start_pos[n] + i and sees keys
 * 0 .. start_pos[n]+i of its own slot (document-causal mask,
 * [continuous-batching compare] flex_paged_attention.py,
 * create_prefill_blockmask_no_paging; sliding form [moe-qwen3 compare]
 * flex_gemma4_moe.py, _create_prefill_sliding_blockmask).  Packing follows the
 * engine's _prefill (prompts concatenated, positions restart at 0 per prompt).
 * With `pro` == NULL every key must already be in the pages (e.g. through
 * pkv_append); with `pro` != NULL a prologue kernel first normalises and
 * rotates k and appends k and the raw v at the queries' positions, and the
 * attention kernel normalises and rotates q in registers as it loads it.
 *   q          : device bf16 [total_tokens][n_q_heads][head_dim], raw (before
 *                the prologue's norm and rotation when pro != NULL); not
 *                modified
 *   cu_seqlens : device int32 [n_seqs+1], non-decreasing, cu[0] = 0,
 *                cu[n_seqs] = total_tokens
 *   slots      : device int32 [n_seqs]; slot 0 = padding sequence: its rows
 *                get out = 0 / lse = -inf, nothing appended or read
 *   start_pos  : device int32 [n_seqs] (cached prefix length) or NULL = all 0
 *   max_seqlen_q_hint : host int >= 1, bound of the per-sequence token counts
 *                used for grid sizing (correct if exceeded; only speed changes)
 *   out        : device bf16 [total_tokens][n_q_heads][head_dim]
 *   scale      : softmax scale applied to q.k, finite and > 0
 *   lse        : device fp32 [total_tokens][n_q_heads] or NULL
 *   workspace  : unused by the current kernels (pass NULL / 0)
 * head_dim 64, 128, 256 and 512 are supported (512: the Gemma-4
 * full-attention layers).  pages_per_slot > 2048, n_seqs > 65535 and, with the
 * prologue, total_tokens > 2097120 are not supported here (PKV_ERR_UNSUPPORTED).
 */
pkv_status pkv_attn_prefill(const void* q, int32_t n_q_heads, const int32_t* cu_seqlens,
                            const int32_t* slots, const int32_t* start_pos,
                            int32_t n_seqs, int32_t total_tokens,
                            int32_t max_seqlen_q_hint, pkv_page_table pt,
                            const pkv_cache_desc* cd, void* k_pool, void* v_pool,
                            float scale, int32_t window, const pkv_prologue* pro,
                            void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_rope_table -- fill fp32 cos/sin tables [max_pos][head_dim/2] with
 * cos(p * theta^(-2i/head_dim)), sin(...), computed in fp64 on the device and
 * rounded to fp32.  This is the "default" rope frequency set (the rope type
 * the pages name for Qwen3-style layers, [moe-qwen3 compare]
 * flex_gemma4_moe.py module docstring); the cos/sin are computed once and
 * reused by every layer, as the engine computes them once per step.
 *   cos_out, sin_out : device fp32 [max_pos][head_dim/2]
 */
pkv_status pkv_rope_table(float* cos_out, float* sin_out, int32_t max_pos,
                          int32_t head_dim, double theta, void* stream);

/* pkv_rope_table_partial -- the same with only the leading rotary_fraction of
 * the head_dim/2 frequencies rotating: i < floor(rotary_fraction * head_dim / 2)
 * use theta^(-2i/head_dim), the rest have a zero frequency (cos 1, sin 0), so
 * the prologue's full-head rotate_half passes those dims through.  This is
 * the "proportional" partial RoPE of the Gemma-4 full-attention layers
 * ([moe-qwen3 compare] flex_gemma4_moe.py, model notes "Two-tier RoPE" and
 * _apply_rotary_full).  rotary_fraction in (0, 1]; 1 = pkv_rope_table.
 */
pkv_status pkv_rope_table_partial(float* cos_out, float* sin_out, int32_t max_pos,
                                  int32_t head_dim, double theta, double rotary_fraction,
                                  void* stream);

/* Bytes of workspace pkv_attn_prefill needs for these sizes: 0 (the prefill
 * kernels use none; the workspace arguments are accepted for a stable ABI). */
size_t pkv_prefill_workspace_size(int32_t total_tokens, int32_t n_seqs, int32_t n_q_heads);

/* ---------------------------------------------------------------------------
 * Validation mode (debugging aid).  The page table's entries, the slots and
 * the lengths / positions live on the device, so the host checks above cannot
 * see them; the pages leave an unmapped -1 entry unchecked
 * ([continuous-batching compare] flex_paged_attention.py, PageTable.assign
 * and the cache write).  With validation on, every pkv_append /
 * pkv_attn_decode / pkv_attn_prefill first enqueues, on its stream, a check of
 * the metadata it is about to use:
 *   a slot outside [0, max_slots)                              PKV_VALIDATE_SLOT
 *   a table entry outside [1, n_pages) for a logical page the
 *   call uses (pages [0, ceil(len / page_size)) of each active
 *   row / sequence; the page of each appended token)           PKV_VALIDATE_PAGE
 *   a length or position < 0 or beyond pages_per_slot*page_size PKV_VALIDATE_POS
 * Slot 0 rows and tokens are the reserved no-op and are never flagged.
 * Findings are OR-ed into a flag word per device; the calls then run as
 * usual (such inputs are handled as described at the top).  Validation is
 * off by default; PKV_VALIDATE=1 in the environment switches it on at the
 * first call, pkv_set_validation at any time (process-wide).
 * pkv_validation_flags synchronises `stream`, writes the device's flag word
 * to *flags (host memory) and, if `clear`, enqueues its reset to 0.  It
 * returns PKV_ERR_INVALID_ARG for a NULL `flags`, PKV_ERR_LAUNCH if the copy
 * fails.  The word is shared by every call on the device.
 */
#define PKV_VALIDATE_SLOT 1u
#define PKV_VALIDATE_PAGE 2u
#define PKV_VALIDATE_POS 4u
pkv_status pkv_set_validation(int32_t on);
pkv_status pkv_validation_flags(uint32_t* flags, int32_t clear, void* stream);

/* Thread-local text of the last non-OK status returned on this thread. */
const char* pkv_last_error(void);

/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

/* ---------------------------------------------------------------------------
 * Host-side slot / page allocator ([continuous-batching compare]
 * flex_paged_attention.py, PageTable: can_reserve, allocate, reserve, erase).
 * Pure host code; it owns only its own host memory and never touches a device.
 * - free pages start as n_pages-1, ..., 2, 1 used as a stack (page 0 never
 *   granted); free slots likewise max_slots-1 ... 1 (slot 0 never granted),
 *   so slots come out 1, 2, 3, ...
 * - reserve(slot, seq_len) grows the slot's capacity (tokens, a multiple of
 *   page_size) to >= seq_len by granting the last k free pages, in stack
 *   order, as its next logical pages; dry_run only reports whether it fits;
 *   otherwise running out is PKV_ERR_CAPACITY with nothing changed.
 * - erase(slot) frees the slot and pushes its pages back in reverse order;
 *   its exported row stays as it was until the slot is allocated again
 *   (allocate resets it to -1), as the pages' device table does.
 * - export renders the device-format table [max_slots][pages_per_slot]
 *   (row 0 all 0, unmapped -1) into a host buffer; the caller copies it to
 *   the device.
 */
typedef struct pkv_pt pkv_pt;

pkv_status pkv_pt_create(int32_t n_pages, int32_t page_size, int32_t max_slots,
                         pkv_pt** out);
void pkv_pt_destroy(pkv_pt* pt);
int32_t pkv_pt_pages_available(const pkv_pt* pt);
int32_t pkv_pt_free_slot_count(const pkv_pt* pt);
/* slot < 0: may a NEW request of `size` tokens be admitted (enough free pages
 * and a free slot)?  slot >= 1: dry-run reserve of that slot to `size`. */
pkv_status pkv_pt_can_reserve(const pkv_pt* pt, int32_t size, int32_t slot, int32_t* ok);
pkv_status pkv_pt_allocate(pkv_pt* pt, int32_t* slot_out);
pkv_status pkv_pt_reserve(pkv_pt* pt, int32_t slot, int32_t seq_len, int32_t dry_run,
                          int32_t* ok_out);
pkv_status pkv_pt_erase(pkv_pt* pt, int32_t slot);
int32_t pkv_pt_capacity(const pkv_pt* pt, int32_t slot);
/* Copies up to max_out page ids owned by `slot` (logical order); returns the
 * count owned (may exceed max_out), or -1 for a bad slot. */
int32_t pkv_pt_row(const pkv_pt* pt, int32_t slot, int32_t* pages_out, int32_t max_out);
/* Copies up to max_out entries of the free-page stack (bottom first); returns
 * its full length. */
int32_t pkv_pt_free_pages(const pkv_pt* pt, int32_t* pages_out, int32_t max_out);
pkv_status pkv_pt_export(const pkv_pt* pt, int32_t* table_out, int32_t pages_per_slot);

/* ---------------------------------------------------------------------------
 * Device-side reserve for a batch ([continuous-batching compare]
 * flex_paged_attention.py, PageTable.reserve), so that a decode step can grow
 * its slots' pages without a host round trip, e.g. inside a captured HIP
 * graph.  The state is the host allocator's, rendered into caller-owned
 * device buffers (pkv_pt_export, pkv_pt_free_pages, pkv_pt_capacity):
 *   table      int32 [max_slots][pages_per_slot]: the page table the
 *              attention calls read; granted pages are written into it
 *   free_pages int32 [n_pages]: the free-page stack, bottom first
 *   free_count int32 [1]: its length (clamped to [0, n_pages] when read)
 *   capacity   int32 [max_slots]: tokens reserved per slot (a multiple of
 *              page_size)
 *   status     uint32 [1]: PKV_RESERVE_* bits of rows that could not be
 *              served are OR-ed in; the call never clears it
 * pkv_pt_device_reserve(dev, slots, seq_lens, B, stream) applies, on
 * `stream`, what B host calls reserve(slots[b], seq_lens[b]) in row order
 * would: a row whose slot is outside [1, max_slots) is skipped; otherwise the
 * slot's capacity grows to >= seq_lens[b] by granting the top k entries of
 * the free stack, in stack order, as its next logical pages.  A row that needs
 * more pages than are free (PKV_RESERVE_NO_PAGES), more than its table row
 * holds (PKV_RESERVE_TOO_LONG), or whose stored capacity is not a multiple of
 * page_size within the row (PKV_RESERVE_BAD_STATE) changes nothing, and the
 * rows after it proceed.  The slots of one call must be distinct (as for
 * decode).  Slot bookkeeping (allocate) stays on the host.
 *   slots, seq_lens : device int32 [B]; B == 0 is a no-op
 * Returns PKV_ERR_INVALID_ARG for NULL pointers or bad sizes (nothing
 * enqueued), PKV_ERR_LAUNCH if the launch fails.
 *
 * pkv_pt_device_erase(dev, slots, B, stream) applies, on `stream`, what B host
 * calls erase(slots[b]) in row order would do to the pages
 * ([continuous-batching compare] flex_paged_attention.py, PageTable.erase):
 * the capacity / page_size pages a slot owns (its first table entries) are
 * pushed back on the free stack in reverse logical order, after those of the
 * rows before it.  Then, unlike the host erase, the slot's capacity is set to
 * 0 and its table row to -1 (what the host allocate does on reuse), so the
 * host may hand the slot out again, and reserve it on the device, with no
 * further call.  Rows whose slot is outside [1, max_slots) are skipped; a row
 * whose stored capacity is not a multiple of page_size within the row, or
 * whose pages would overflow the n_pages entries of free_pages (a state that
 * no sequence of allocator calls produces), changes nothing and sets
 * PKV_RESERVE_BAD_STATE.  The slots of one call must be distinct.
 *   slots : device int32 [B]; B == 0 is a no-op
 * Returns as pkv_pt_device_reserve.
 */
#define PKV_RESERVE_NO_PAGES 1u
#define PKV_RESERVE_TOO_LONG 2u
#define PKV_RESERVE_BAD_STATE 4u
typedef struct {
  int32_t* table;
  int32_t* free_pages;
  int32_t* free_count;
  int32_t* capacity;
  uint32_t* status;
  int32_t max_slots;
  int32_t pages_per_slot;
  int32_t page_size;
  int32_t n_pages;
} pkv_pt_device;

pkv_status pkv_pt_device_reserve(const pkv_pt_device* dev, const int32_t* slots,
                                 const int32_t* seq_lens, int32_t B, void* stream);
pkv_status pkv_pt_device_erase(const pkv_pt_device* dev, const int32_t* slots, int32_t B,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
