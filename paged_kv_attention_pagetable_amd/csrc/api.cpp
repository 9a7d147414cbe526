// C-ABI entry points: host-side argument checks, then kernel launches.
// Nothing here allocates, frees or synchronises device memory.
#include <initializer_list>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

// The kernels move bf16 rows and fp32 table rows in 16-byte units.
bool misaligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15u)) return true;
  return false;
}

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

// Checks the cache descriptor and page table; fills the kernel-side geometry.
pkv_status check_cache(const char* fn, const pkv_cache_desc* cd, const pkv_page_table& pt,
                       bool allow_d512, pkv::PoolGeom* g, pkv::TableRef* tr) {
  if (!cd) return fail(PKV_ERR_INVALID_ARG, "%s: cache descriptor is NULL", fn);
  if (cd->n_pages < 2) return fail(PKV_ERR_INVALID_ARG, "%s: n_pages must be >= 2 (got %d)", fn, cd->n_pages);
  if (!is_pow2(cd->page_size) || cd->page_size < 16 || cd->page_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "%s: page_size must be a power of two in [16, 256] (got %d)", fn,
                cd->page_size);
  const int D = cd->head_dim;
  if (!(D == 64 || D == 128 || D == 256 || (allow_d512 && D == 512)))
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d not supported", fn, D);
  if (cd->n_kv_heads < 1) return fail(PKV_ERR_INVALID_ARG, "%s: n_kv_heads must be >= 1", fn);
  if (!pt.table) return fail(PKV_ERR_INVALID_ARG, "%s: page table pointer is NULL", fn);
  if (pt.max_slots < 2)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_slots must be >= 2 (slot 0 is reserved), got %d", fn,
                pt.max_slots);
  if (pt.pages_per_slot < 1)
    return fail(PKV_ERR_INVALID_ARG, "%s: pages_per_slot must be >= 1", fn);
  if ((long long)pt.pages_per_slot * cd->page_size > (1LL << 30))
    return fail(PKV_ERR_INVALID_ARG, "%s: pages_per_slot * page_size exceeds 2^30 tokens", fn);
  g->n_pages = cd->n_pages;
  g->page_size = cd->page_size;
  g->log2ps = ilog2(cd->page_size);
  g->n_kv = cd->n_kv_heads;
  g->head_dim = D;
  tr->table = pt.table;
  tr->max_slots = pt.max_slots;
  tr->pps = pt.pages_per_slot;
  return PKV_OK;
}

pkv_status check_heads(const char* fn, int n_q, int n_kv, int* G) {
  if (n_q < 1 || n_q % n_kv != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                fn, n_q, n_kv);
  *G = n_q / n_kv;
  if (*G > 16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: query heads per kv head must be <= 16 (got %d)", fn, *G);
  return PKV_OK;
}

// Validation mode: off unless switched on by pkv_set_validation or by
// PKV_VALIDATE=1 in the environment (read on first use).
std::atomic<int> g_validate{-1};

bool validation_on() {
  int v = g_validate.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("PKV_VALIDATE");
    v = (e && e[0] == '1') ? 1 : 0;
    int expected = -1;
    g_validate.compare_exchange_strong(expected, v);
    v = g_validate.load(std::memory_order_relaxed);
  }
  return v == 1;
}

}  // namespace

extern "C" {

pkv_status pkv_set_validation(int32_t on) {
  g_validate.store(on ? 1 : 0, std::memory_order_relaxed);
  return PKV_OK;
}

pkv_status pkv_validation_flags(uint32_t* flags, int32_t clear, void* stream) {
  const char* fn = "pkv_validation_flags";
  if (!flags) return fail(PKV_ERR_INVALID_ARG, "%s: NULL output", fn);
  const hipError_t e = pkv::read_validate_flags(flags, clear, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"

namespace {

// Shared argument checks and marshalling of the device allocator calls.
pkv_status device_state_args(const char* fn, const pkv_pt_device* dev, const int32_t* slots,
                             int32_t B, pkv::ReserveArgs* a) {
  if (!dev) return fail(PKV_ERR_INVALID_ARG, "%s: NULL state", fn);
  if (B < 0) return fail(PKV_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
  if (dev->max_slots < 2 || dev->pages_per_slot < 1 || dev->page_size < 1 || dev->n_pages < 2)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: need max_slots >= 2, pages_per_slot >= 1, page_size >= 1, n_pages >= 2", fn);
  if ((long)dev->pages_per_slot * dev->page_size > (1L << 30))
    return fail(PKV_ERR_INVALID_ARG, "%s: pages_per_slot * page_size exceeds 2^30 tokens", fn);
  if (!dev->table || !dev->free_pages || !dev->free_count || !dev->capacity || !dev->status)
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL state buffer", fn);
  if (B > 0 && !slots) return fail(PKV_ERR_INVALID_ARG, "%s: NULL slots", fn);
  a->table = dev->table;
  a->free_pages = dev->free_pages;
  a->free_count = dev->free_count;
  a->capacity = dev->capacity;
  a->status = dev->status;
  a->slots = slots;
  a->seq_lens = nullptr;
  a->B = B;
  a->max_slots = dev->max_slots;
  a->pps = dev->pages_per_slot;
  a->page_size = dev->page_size;
  a->n_pages = dev->n_pages;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_pt_device_reserve(const pkv_pt_device* dev, const int32_t* slots,
                                 const int32_t* seq_lens, int32_t B, void* stream) {
  const char* fn = "pkv_pt_device_reserve";
  pkv::ReserveArgs a;
  const pkv_status st = device_state_args(fn, dev, slots, B, &a);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  if (!seq_lens) return fail(PKV_ERR_INVALID_ARG, "%s: NULL slots or seq_lens", fn);
  a.seq_lens = seq_lens;
  return launched(pkv::launch_reserve(a, static_cast<hipStream_t>(stream)), fn);
}

pkv_status pkv_pt_device_erase(const pkv_pt_device* dev, const int32_t* slots, int32_t B,
                               void* stream) {
  const char* fn = "pkv_pt_device_erase";
  pkv::ReserveArgs a;
  const pkv_status st = device_state_args(fn, dev, slots, B, &a);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  return launched(pkv::launch_erase(a, static_cast<hipStream_t>(stream)), fn);
}

size_t pkv_prefill_workspace_size(int32_t total_tokens, int32_t n_seqs, int32_t n_q_heads) {
  (void)total_tokens;
  (void)n_seqs;
  (void)n_q_heads;
  return 0;  // the prefill kernels use no workspace
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

pkv_status pkv_append(const void* k_new, const void* v_new, const int32_t* slot,
                      const int32_t* pos, int32_t T, pkv_page_table pt,
                      const pkv_cache_desc* cd, void* k_pool, void* v_pool, void* stream) {
  const char* fn = "pkv_append";
  if (T < 0) return fail(PKV_ERR_INVALID_ARG, "%s: T must be >= 0 (got %d)", fn, T);
  pkv::PoolGeom g;
  pkv::TableRef tr;
  pkv_status st = check_cache(fn, cd, pt, true, &g, &tr);
  if (st != PKV_OK) return st;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !slot || !pos || !k_pool || !v_pool)
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned16({k_new, v_new, k_pool, v_pool}))
    return fail(PKV_ERR_INVALID_ARG, "%s: bf16 buffers must be 16-byte aligned", fn);
  pkv::AppendArgs a;
  a.k_new = static_cast<const pkv::bf16_t*>(k_new);
  a.v_new = static_cast<const pkv::bf16_t*>(v_new);
  a.slot = slot;
  a.pos = pos;
  a.T = T;
  a.pt = tr;
  a.g = g;
  a.kpool = static_cast<pkv::bf16_t*>(k_pool);
  a.vpool = static_cast<pkv::bf16_t*>(v_pool);
  if (validation_on()) {
    st = launched(pkv::launch_validate_tokens(tr, g, slot, pos, T, static_cast<hipStream_t>(stream)), fn);
    if (st != PKV_OK) return st;
  }
  return launched(pkv::launch_append(a, static_cast<hipStream_t>(stream)), fn);
}

size_t pkv_decode_workspace_size(int32_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len_hint, int32_t window) {
  if (B <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return 0;
  if (max_seq_len_hint < 1) max_seq_len_hint = 1;
  return pkv::plan_decode(B, n_q_heads, n_kv_heads, head_dim, max_seq_len_hint,
                          window > 0 ? window : 0)
      .ws_bytes;
}

pkv_status pkv_decode_plan(int32_t B, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t max_seq_len_hint, int32_t window, int64_t* out) {
  static const char* fn = "pkv_decode_plan";
  if (!out) return fail(PKV_ERR_INVALID_ARG, "%s: out is NULL", fn);
  if (B <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: need B, heads > 0 and n_q_heads %% n_kv_heads == 0", fn);
  if (max_seq_len_hint < 1) max_seq_len_hint = 1;
  const pkv::DecodePlan p = pkv::plan_decode(B, n_q_heads, n_kv_heads, head_dim,
                                             max_seq_len_hint, window > 0 ? window : 0);
  out[0] = p.split_tokens;
  out[1] = p.head_tokens;
  out[2] = p.max_splits;
  out[3] = p.v_late;
  out[4] = p.early_merge;
  out[5] = (int64_t)p.ws_bytes;
  return PKV_OK;
}

}  // extern "C"

namespace {

// Shared body of pkv_attn_decode and pkv_attn_decode_noalloc.  no_alloc: the
// split partials and arrival counters go to the library's static scratch
// buffer of this device instead of `workspace`.
pkv_status attn_decode_impl(const char* fn, const void* q, int32_t n_q_heads,
                            const int32_t* slots, const int32_t* seq_lens, int32_t B,
                            int32_t max_seq_len_hint, pkv_page_table pt,
                            const pkv_cache_desc* cd, void* k_pool, void* v_pool,
                            const void* k_new, const void* v_new, float scale, int32_t window,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream, bool no_alloc) {
  if (B < 0) return fail(PKV_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
  if (B > 65535) return fail(PKV_ERR_UNSUPPORTED, "%s: B must be <= 65535 (got %d)", fn, B);
  pkv::PoolGeom g;
  pkv::TableRef tr;
  pkv_status st = check_cache(fn, cd, pt, true, &g, &tr);
  if (st != PKV_OK) return st;
  int G = 0;
  st = check_heads(fn, n_q_heads, g.n_kv, &G);
  if (st != PKV_OK) return st;
  if (G * g.head_dim > 2048)
    return fail(PKV_ERR_UNSUPPORTED,
                "%s: (n_q_heads / n_kv_heads) * head_dim must be <= 2048 (got %d * %d)", fn, G,
                g.head_dim);
  if (window < 0) return fail(PKV_ERR_INVALID_ARG, "%s: window must be >= 0", fn);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (max_seq_len_hint < 1)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_seq_len_hint must be >= 1", fn);
  if (B == 0) return PKV_OK;
  if (!q || !slots || !seq_lens || !k_pool || !v_pool || !out)
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL tensor pointer", fn);
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "%s: k_new and v_new must both be given or both be NULL", fn);
  if (misaligned16({q, k_pool, v_pool, out, k_new, v_new}))
    return fail(PKV_ERR_INVALID_ARG, "%s: bf16 buffers must be 16-byte aligned", fn);
  const pkv::DecodePlan plan =
      pkv::plan_decode(B, n_q_heads, g.n_kv, g.head_dim, max_seq_len_hint, window);
  if (no_alloc && plan.ws_bytes > 0) {
    if (plan.ws_bytes > pkv::kDecodeScratchBytes)
      return fail(PKV_ERR_WORKSPACE,
                  "%s: this call's split partials need %zu bytes, more than the %zu-byte "
                  "static scratch; use pkv_attn_decode with a workspace",
                  fn, plan.ws_bytes, pkv::kDecodeScratchBytes);
    const hipError_t e = pkv::decode_scratch(&workspace);
    if (e != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "%s: no static scratch on this device: %s", fn,
                  hipGetErrorString(e));
    workspace_bytes = pkv::kDecodeScratchBytes;
  }
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(PKV_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn,
                plan.ws_bytes, workspace ? workspace_bytes : (size_t)0);
  // the merge moves partials with 8- and 16-byte device-scope accesses
  if (plan.ws_bytes > 0 && misaligned16({workspace}))
    return fail(PKV_ERR_INVALID_ARG, "%s: the workspace must be 16-byte aligned", fn);
  pkv::DecodeArgs a;
  a.q = static_cast<const pkv::bf16_t*>(q);
  a.n_q = n_q_heads;
  a.G = G;
  a.slots = slots;
  a.seq_lens = seq_lens;
  a.B = B;
  a.pt = tr;
  a.g = g;
  a.kpool = static_cast<const pkv::bf16_t*>(k_pool);
  a.vpool = static_cast<const pkv::bf16_t*>(v_pool);
  a.kpool_w = static_cast<pkv::bf16_t*>(k_pool);
  a.vpool_w = static_cast<pkv::bf16_t*>(v_pool);
  a.k_new = static_cast<const pkv::bf16_t*>(k_new);
  a.v_new = static_cast<const pkv::bf16_t*>(v_new);
  a.scale_log2 = scale * pkv::kLog2eHost;
  a.window = window;
  a.split_tokens = plan.split_tokens;
  a.head_tokens = plan.head_tokens;
  a.v_late = plan.v_late;
  a.early_merge = plan.early_merge;
  a.max_splits = plan.max_splits;
  a.part_o = plan.ws_bytes ? static_cast<uint32_t*>(workspace) : nullptr;
  a.part_ml = plan.ws_bytes ? reinterpret_cast<float*>(a.part_o + plan.part_o_words) : nullptr;
  // the counters sit at the end of the workspace as given, so every call that
  // passes the same (workspace, workspace_bytes) finds them at the same place
  a.arrivals_end =
      plan.ws_bytes ? reinterpret_cast<uint32_t*>(
                          (reinterpret_cast<uintptr_t>(workspace) + workspace_bytes) & ~(uintptr_t)3)
                    : nullptr;
  a.out = static_cast<pkv::bf16_t*>(out);
  a.lse = lse;
  if (validation_on()) {
    st = launched(pkv::launch_validate_rows(tr, g, slots, seq_lens, nullptr, nullptr, B,
                                            static_cast<hipStream_t>(stream)),
                  fn);
    if (st != PKV_OK) return st;
  }
  return launched(pkv::launch_decode(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

pkv_status pkv_attn_decode(const void* q, int32_t n_q_heads, const int32_t* slots,
                           const int32_t* seq_lens, int32_t B, int32_t max_seq_len_hint,
                           pkv_page_table pt, const pkv_cache_desc* cd, void* k_pool,
                           void* v_pool, const void* k_new, const void* v_new, float scale,
                           int32_t window, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return attn_decode_impl("pkv_attn_decode", q, n_q_heads, slots, seq_lens, B, max_seq_len_hint,
                          pt, cd, k_pool, v_pool, k_new, v_new, scale, window, out, lse,
                          workspace, workspace_bytes, stream, false);
}

pkv_status pkv_attn_decode_noalloc(const void* q, int32_t n_q_heads, const int32_t* slots,
                                   const int32_t* seq_lens, int32_t B,
                                   int32_t max_seq_len_hint, pkv_page_table pt,
                                   const pkv_cache_desc* cd, void* k_pool, void* v_pool,
                                   const void* k_new, const void* v_new, float scale,
                                   int32_t window, void* out, float* lse, void* stream) {
  return attn_decode_impl("pkv_attn_decode_noalloc", q, n_q_heads, slots, seq_lens, B,
                          max_seq_len_hint, pt, cd, k_pool, v_pool, k_new, v_new, scale, window,
                          out, lse, nullptr, 0, stream, true);
}

pkv_status pkv_attn_prefill(const void* q, int32_t n_q_heads, const int32_t* cu_seqlens,
                            const int32_t* slots, const int32_t* start_pos,
                            int32_t n_seqs, int32_t total_tokens,
                            int32_t max_seqlen_q_hint, pkv_page_table pt,
                            const pkv_cache_desc* cd, void* k_pool, void* v_pool,
                            float scale, int32_t window, const pkv_prologue* pro,
                            void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  const char* fn = "pkv_attn_prefill";
  if (n_seqs < 0 || total_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: n_seqs and total_tokens must be >= 0", fn);
  if (n_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "%s: n_seqs must be <= 65535", fn);
  pkv::PoolGeom g;
  pkv::TableRef tr;
  pkv_status st = check_cache(fn, cd, pt, true, &g, &tr);
  if (st != PKV_OK) return st;
  int G = 0;
  st = check_heads(fn, n_q_heads, g.n_kv, &G);
  if (st != PKV_OK) return st;
  if (window < 0) return fail(PKV_ERR_INVALID_ARG, "%s: window must be >= 0", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PKV_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (max_seqlen_q_hint < 1)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_seqlen_q_hint must be >= 1", fn);
  if (pt.pages_per_slot > 2048)
    return fail(PKV_ERR_UNSUPPORTED, "%s: pages_per_slot must be <= 2048 (got %d)", fn,
                pt.pages_per_slot);
  if (n_seqs == 0 || total_tokens == 0) return PKV_OK;
  if (!q || !cu_seqlens || !slots || !k_pool || !v_pool || !out)
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned16({q, k_pool, v_pool, out}) ||
      (pro && misaligned16({pro->q_norm_w, pro->k_norm_w, pro->rope_cos, pro->rope_sin, pro->k_raw,
                            pro->v_raw, pro->q_out})))
    return fail(PKV_ERR_INVALID_ARG, "%s: bf16 buffers and rotary tables must be 16-byte aligned", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validation_on()) {
    st = launched(pkv::launch_validate_rows(tr, g, slots, nullptr, cu_seqlens, start_pos, n_seqs, s), fn);
    if (st != PKV_OK) return st;
  }
  // k_raw == v_raw == NULL: the keys are already in the pages; only q gets
  // its norm and rotation (inside the attention kernel)
  const bool append_kv = pro && (pro->k_raw || pro->v_raw);
  if (pro) {
    if (!pro->q_norm_w || !pro->rope_cos || !pro->rope_sin ||
        (append_kv && (!pro->k_norm_w || !pro->k_raw || !pro->v_raw)))
      return fail(PKV_ERR_INVALID_ARG, "%s: NULL pointer in the prologue", fn);
    if (pro->max_pos < 1) return fail(PKV_ERR_INVALID_ARG, "%s: prologue max_pos must be >= 1", fn);
    if ((total_tokens + 31) / 32 > 65535)
      return fail(PKV_ERR_UNSUPPORTED, "%s: with the prologue, total_tokens must be <= 2097120", fn);
    if (!(pro->eps >= 0.f) || !std::isfinite(pro->eps))
      return fail(PKV_ERR_INVALID_ARG, "%s: prologue eps must be finite and >= 0", fn);
    if (append_kv) {
      pkv::PrologueArgs p;
      p.k_raw = static_cast<const pkv::bf16_t*>(pro->k_raw);
      p.v_raw = static_cast<const pkv::bf16_t*>(pro->v_raw);
      p.k_w = static_cast<const pkv::bf16_t*>(pro->k_norm_w);
      p.v_norm = pro->v_norm ? 1 : 0;
      p.eps = pro->eps;
      p.cos_t = pro->rope_cos;
      p.sin_t = pro->rope_sin;
      p.max_pos = pro->max_pos;
      p.T = total_tokens;
      p.cu_seqlens = cu_seqlens;
      p.slots = slots;
      p.start_pos = start_pos;
      p.n_seqs = n_seqs;
      p.pt = tr;
      p.g = g;
      p.kpool = static_cast<pkv::bf16_t*>(k_pool);
      p.vpool = static_cast<pkv::bf16_t*>(v_pool);
      st = launched(pkv::launch_prologue(p, s), fn);
      if (st != PKV_OK) return st;
    }
  }
  pkv::PrefillArgs a;
  a.q = static_cast<const pkv::bf16_t*>(q);
  a.n_q = n_q_heads;
  a.G = G;
  a.cu_seqlens = cu_seqlens;
  a.slots = slots;
  a.start_pos = start_pos;
  a.n_seqs = n_seqs;
  a.pt = tr;
  a.g = g;
  a.kpool = static_cast<const pkv::bf16_t*>(k_pool);
  a.vpool = static_cast<const pkv::bf16_t*>(v_pool);
  a.scale_log2 = scale * pkv::kLog2eHost;
  a.window = window;
  a.q_tokens = pkv::prefill_q_tokens(G, g.head_dim);
  a.n_qblocks = (max_seqlen_q_hint + a.q_tokens - 1) / a.q_tokens;
  if (a.n_qblocks > 65535) a.n_qblocks = 65535;
  a.out = static_cast<pkv::bf16_t*>(out);
  a.lse = lse;
  // q's RMSNorm + RoPE run inside the attention kernel as it loads q
  a.q_w = pro ? static_cast<const pkv::bf16_t*>(pro->q_norm_w) : nullptr;
  a.cos_t = pro ? pro->rope_cos : nullptr;
  a.sin_t = pro ? pro->rope_sin : nullptr;
  a.eps = pro ? pro->eps : 0.f;
  a.max_pos = pro ? pro->max_pos : 0;
  a.q_out = pro ? static_cast<pkv::bf16_t*>(pro->q_out) : nullptr;
  return launched(pkv::launch_prefill(a, s), fn);
}

pkv_status pkv_rope_table_partial(float* cos_out, float* sin_out, int32_t max_pos,
                                  int32_t head_dim, double theta, double rotary_fraction,
                                  void* stream) {
  const char* fn = "pkv_rope_table";
  if (!cos_out || !sin_out) return fail(PKV_ERR_INVALID_ARG, "%s: NULL output", fn);
  if (max_pos < 1 || head_dim < 2 || head_dim % 2)
    return fail(PKV_ERR_INVALID_ARG, "%s: need max_pos >= 1 and an even head_dim >= 2", fn);
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(PKV_ERR_INVALID_ARG, "%s: theta must be finite and > 0", fn);
  if (!(rotary_fraction > 0.0 && rotary_fraction <= 1.0))
    return fail(PKV_ERR_INVALID_ARG, "%s: rotary_fraction must be in (0, 1]", fn);
  // rotating frequencies: floor(f * D / 2), as the proportional rope initialiser counts them
  const int n_rot = (int)std::floor(rotary_fraction * head_dim / 2.0);
  return launched(pkv::launch_rope_table(cos_out, sin_out, max_pos, head_dim, theta, n_rot,
                                         static_cast<hipStream_t>(stream)),
                  fn);
}

pkv_status pkv_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                          double theta, void* stream) {
  return pkv_rope_table_partial(cos_out, sin_out, max_pos, head_dim, theta, 1.0, stream);
}

}  // extern "C"
