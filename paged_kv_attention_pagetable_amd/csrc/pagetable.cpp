// Host-side slot / page allocator.  State machine of the PageTable class on
// the continuous-batching compare page (flex_paged_attention.py): a LIFO stack
// of free pages starting as n_pages-1 .. 1, a LIFO stack of free slots starting
// as max_slots-1 .. 1, capacities in tokens, and a mirror of the device table
// whose rows are reset by allocate and left stale by erase.
#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "../../include/pkv.h"

struct pkv_pt {
  int32_t n_pages;
  int32_t page_size;
  int32_t max_slots;
  std::vector<int32_t> free_pages;          // stack: back() is the top
  std::vector<int32_t> free_slots;          // stack
  std::vector<std::vector<int32_t>> owned;  // pages owned per slot, logical order
  std::vector<std::vector<int32_t>> dev;    // device-table mirror per slot (prefix)
  std::vector<int32_t> capacity;            // tokens
};

namespace {

bool slot_ok(const pkv_pt* pt, int32_t s) { return pt && s >= 1 && s < pt->max_slots; }
}  // namespace

extern "C" {

pkv_status pkv_pt_create(int32_t n_pages, int32_t page_size, int32_t max_slots, pkv_pt** out) {
  if (!out || n_pages < 2 || page_size < 1 || max_slots < 2) return PKV_ERR_INVALID_ARG;
  pkv_pt* pt = new (std::nothrow) pkv_pt();
  if (!pt) return PKV_ERR_CAPACITY;
  pt->n_pages = n_pages;
  pt->page_size = page_size;
  pt->max_slots = max_slots;
  for (int32_t p = n_pages - 1; p >= 1; --p) pt->free_pages.push_back(p);
  for (int32_t s = max_slots - 1; s >= 1; --s) pt->free_slots.push_back(s);
  pt->owned.assign(max_slots, {});
  pt->dev.assign(max_slots, {});
  pt->capacity.assign(max_slots, 0);
  *out = pt;
  return PKV_OK;
}

void pkv_pt_destroy(pkv_pt* pt) { delete pt; }

int32_t pkv_pt_pages_available(const pkv_pt* pt) {
  return pt ? (int32_t)pt->free_pages.size() : 0;
}

int32_t pkv_pt_free_slot_count(const pkv_pt* pt) {
  return pt ? (int32_t)pt->free_slots.size() : 0;
}

pkv_status pkv_pt_reserve(pkv_pt* pt, int32_t slot, int32_t seq_len, int32_t dry_run,
                          int32_t* ok_out) {
  if (!slot_ok(pt, slot) || seq_len < 0 || !ok_out) return PKV_ERR_INVALID_ARG;
  const int64_t cap = pt->capacity[slot];
  if (seq_len <= cap) {
    *ok_out = 1;
    return PKV_OK;
  }
  const int64_t k = (seq_len - cap + pt->page_size - 1) / pt->page_size;
  const bool fits = k <= (int64_t)pt->free_pages.size();
  if (dry_run) {
    *ok_out = fits ? 1 : 0;
    return PKV_OK;
  }
  if (!fits) {
    *ok_out = 0;
    return PKV_ERR_CAPACITY;
  }
  // grant the top k pages of the stack, bottom-most first (free_pages[-k:])
  const size_t first = pt->free_pages.size() - (size_t)k;
  const int64_t start = cap / pt->page_size;
  std::vector<int32_t>& dev = pt->dev[slot];
  for (int64_t i = 0; i < k; ++i) {
    const int32_t page = pt->free_pages[first + (size_t)i];
    pt->owned[slot].push_back(page);
    const size_t li = (size_t)(start + i);
    if (dev.size() <= li) dev.resize(li + 1, -1);
    dev[li] = page;
  }
  pt->free_pages.resize(first);
  pt->capacity[slot] = (int32_t)(cap + k * pt->page_size);
  *ok_out = 1;
  return PKV_OK;
}

pkv_status pkv_pt_can_reserve(const pkv_pt* pt, int32_t size, int32_t slot, int32_t* ok) {
  if (!pt || !ok || size < 0) return PKV_ERR_INVALID_ARG;
  if (slot < 0) {
    *ok = ((int64_t)pt->free_pages.size() * pt->page_size >= size && !pt->free_slots.empty()) ? 1 : 0;
    return PKV_OK;
  }
  return pkv_pt_reserve(const_cast<pkv_pt*>(pt), slot, size, 1, ok);
}

pkv_status pkv_pt_allocate(pkv_pt* pt, int32_t* slot_out) {
  if (!pt || !slot_out) return PKV_ERR_INVALID_ARG;
  if (pt->free_slots.empty()) return PKV_ERR_CAPACITY;
  const int32_t s = pt->free_slots.back();
  pt->free_slots.pop_back();
  pt->capacity[s] = 0;
  pt->dev[s].clear();  // device row reset to -1
  *slot_out = s;
  return PKV_OK;
}

pkv_status pkv_pt_erase(pkv_pt* pt, int32_t slot) {
  if (!slot_ok(pt, slot)) return PKV_ERR_INVALID_ARG;
  if (std::find(pt->free_slots.begin(), pt->free_slots.end(), slot) != pt->free_slots.end())
    return PKV_ERR_INVALID_ARG;  // not allocated
  pt->free_slots.push_back(slot);
  std::vector<int32_t>& o = pt->owned[slot];
  for (auto it = o.rbegin(); it != o.rend(); ++it) pt->free_pages.push_back(*it);
  o.clear();
  return PKV_OK;
}

int32_t pkv_pt_capacity(const pkv_pt* pt, int32_t slot) {
  return slot_ok(pt, slot) ? pt->capacity[slot] : -1;
}

int32_t pkv_pt_row(const pkv_pt* pt, int32_t slot, int32_t* pages_out, int32_t max_out) {
  if (!slot_ok(pt, slot)) return -1;
  const std::vector<int32_t>& o = pt->owned[slot];
  const int32_t n = (int32_t)o.size();
  for (int32_t i = 0; i < n && i < max_out && pages_out; ++i) pages_out[i] = o[i];
  return n;
}

int32_t pkv_pt_free_pages(const pkv_pt* pt, int32_t* pages_out, int32_t max_out) {
  if (!pt) return -1;
  const int32_t n = (int32_t)pt->free_pages.size();
  for (int32_t i = 0; i < n && i < max_out && pages_out; ++i) pages_out[i] = pt->free_pages[i];
  return n;
}

pkv_status pkv_pt_export(const pkv_pt* pt, int32_t* table_out, int32_t pages_per_slot) {
  if (!pt || !table_out || pages_per_slot < 1) return PKV_ERR_INVALID_ARG;
  for (int32_t s = 1; s < pt->max_slots; ++s)
    if ((int32_t)pt->dev[s].size() > pages_per_slot) return PKV_ERR_CAPACITY;
  for (int32_t i = 0; i < pages_per_slot; ++i) table_out[i] = 0;  // row 0
  for (int32_t s = 1; s < pt->max_slots; ++s) {
    int32_t* row = table_out + (size_t)s * pages_per_slot;
    const std::vector<int32_t>& d = pt->dev[s];
    for (int32_t i = 0; i < pages_per_slot; ++i) row[i] = i < (int32_t)d.size() ? d[i] : -1;
  }
  return PKV_OK;
}

}  // extern "C"
