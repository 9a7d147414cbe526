"""Paged KV-cache attention for AMD MI355X (gfx950): Python binding.

Thin argument marshalling over the C ABI in ``include/pkv.h``; every step of
the computation runs in the HIP kernels of ``libpkv.so``.  torch provides
device memory and streams only.  There is no CPU fallback: if the library is
not built, every call raises.

Tensors (all on the same HIP device, contiguous):

* ``k_pool``: bf16 ``[n_pages, n_kv, page_size, head_dim]``
* ``v_pool``: bf16 ``[n_pages, n_kv, page_size // gs, head_dim, gs]`` with
  ``gs = min(page_size, 32)``: each page's rows in groups of 32 keys, each
  group d-major (see ``v_pool_shape``)
* ``table``:  int32 ``[max_slots, pages_per_slot]``, -1 = unmapped, slot 0
  reserved
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import CacheDesc, PageTableRef, Prologue, PkvError, check, lib

__all__ = ["append", "attn_decode", "attn_decode_noalloc", "attn_prefill", "decode_workspace_size", "rope_table",
           "set_validation", "validation_flags", "VALIDATE_SLOT", "VALIDATE_PAGE", "VALIDATE_POS",
           "new_pools", "v_pool_shape", "new_decode_workspace", "PageAllocator", "DevicePageState",
           "RESERVE_NO_PAGES", "RESERVE_TOO_LONG", "RESERVE_BAD_STATE", "PkvError", "lib"]

RESERVE_NO_PAGES, RESERVE_TOO_LONG, RESERVE_BAD_STATE = 1, 2, 4


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _bits16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 (bfloat16 / 16-bit view), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _i32(t, name):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


def _cache(k_pool, v_pool, table):
    _bits16(k_pool, "k_pool")
    _bits16(v_pool, "v_pool")
    _i32(table, "table")
    if k_pool.dim() != 4:
        raise ValueError("k_pool must be 4-D [n_pages, n_kv, page_size, head_dim]")
    n_pages, n_kv, ps, D = k_pool.shape
    if tuple(v_pool.shape) != v_pool_shape(n_pages, n_kv, ps, D):
        raise ValueError(f"v_pool must be [n_pages, n_kv, page_size // gs, head_dim, gs] = "
                         f"{v_pool_shape(n_pages, n_kv, ps, D)}, got {tuple(v_pool.shape)}")
    if table.dim() != 2:
        raise ValueError("table must be [max_slots, pages_per_slot]")
    cd = CacheDesc(n_pages, ps, n_kv, D)
    pt = PageTableRef(table.data_ptr(), table.shape[0], table.shape[1])
    return cd, pt


def v_pool_shape(n_pages, n_kv, page_size, head_dim):
    """Shape of the V pool: 32-key groups of each page, d-major inside a group."""
    gs = min(page_size, 32)
    return (n_pages, n_kv, page_size // gs, head_dim, gs)


def new_pools(n_pages, n_kv, page_size, head_dim, device="cuda", fill=None):
    """Allocate a K and a V pool (bf16) in the library's layout."""
    k = torch.empty((n_pages, n_kv, page_size, head_dim), dtype=torch.bfloat16, device=device)
    v = torch.empty(v_pool_shape(n_pages, n_kv, page_size, head_dim), dtype=torch.bfloat16,
                    device=device)
    if fill is not None:
        k.view(torch.int16).fill_(fill)
        v.view(torch.int16).fill_(fill)
    return k, v


def append(k_new, v_new, slot, pos, table, k_pool, v_pool, stream=None):
    """Scatter ``k_new/v_new [T, n_kv, D]`` to (slot, pos) of the pools."""
    cd, pt = _cache(k_pool, v_pool, table)
    _bits16(k_new, "k_new")
    _bits16(v_new, "v_new")
    _i32(slot, "slot")
    _i32(pos, "pos")
    T = k_new.shape[0]
    if tuple(k_new.shape) != (T, cd.n_kv_heads, cd.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [T, n_kv, head_dim]")
    if slot.numel() != T or pos.numel() != T:
        raise ValueError("slot / pos must have T entries")
    check(lib().pkv_append(_ptr(k_new), _ptr(v_new), _ptr(slot), _ptr(pos), T, pt,
                           ctypes.byref(cd), _ptr(k_pool), _ptr(v_pool),
                           _stream(stream, k_pool.device)))


def decode_workspace_size(B, n_q, n_kv, head_dim, max_seq_len_hint, window=0):
    return int(lib().pkv_decode_workspace_size(B, n_q, n_kv, head_dim, max_seq_len_hint,
                                               window))


def decode_plan(B, n_q, n_kv, head_dim, max_seq_len_hint, window=0):
    """The split-K plan of pkv_attn_decode for these sizes (host only)."""
    out = (ctypes.c_int64 * 6)()
    check(lib().pkv_decode_plan(B, n_q, n_kv, head_dim, max_seq_len_hint, window, out))
    return dict(split_tokens=out[0], head_tokens=out[1], max_splits=out[2],
                v_late=bool(out[3]), early_merge=bool(out[4]), ws_bytes=out[5])


def attn_decode(q, slots, seq_lens, table, k_pool, v_pool, scale=None, window=0,
                max_seq_len_hint=None, out=None, lse=None, workspace=None, k_new=None,
                v_new=None, stream=None):
    """Decode attention; returns ``out [B, n_q, D]`` (bf16).

    With ``k_new``/``v_new`` ``[B, n_kv, D]`` each active row's new token is
    appended at position ``seq_len - 1`` first (fused append).
    """
    cd, pt = _cache(k_pool, v_pool, table)
    _bits16(q, "q")
    _i32(slots, "slots")
    _i32(seq_lens, "seq_lens")
    B, n_q, D = q.shape
    if D != cd.head_dim:
        raise ValueError("q head_dim does not match the pools")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _bits16(k_new, "k_new")
        _bits16(v_new, "v_new")
        if tuple(k_new.shape) != (B, cd.n_kv_heads, D) or v_new.shape != k_new.shape:
            raise ValueError("k_new / v_new must be [B, n_kv, head_dim]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seq_len_hint is None:
        max_seq_len_hint = pt.pages_per_slot * cd.page_size
    if out is None:
        out = torch.empty((B, n_q, D), dtype=torch.bfloat16, device=q.device)
    ws_bytes = decode_workspace_size(B, n_q, cd.n_kv_heads, D, max_seq_len_hint, window)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = new_decode_workspace(ws_bytes, q.device)
    wsize = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().pkv_attn_decode(_ptr(q), n_q, _ptr(slots), _ptr(seq_lens), B,
                                int(max_seq_len_hint), pt, ctypes.byref(cd), _ptr(k_pool),
                                _ptr(v_pool), _ptr(k_new), _ptr(v_new), float(scale),
                                int(window), _ptr(out), _ptr(lse), _ptr(workspace), wsize,
                                _stream(stream, q.device)))
    return out


DECODE_SCRATCH_BYTES = 16 << 20   # the library's static scratch per device


def attn_decode_noalloc(q, slots, seq_lens, table, k_pool, v_pool, out, scale=None, window=0,
                        max_seq_len_hint=None, lse=None, k_new=None, v_new=None, stream=None):
    """``attn_decode`` through ``pkv_attn_decode_noalloc``: no workspace, the split
    partials go to the library's static per-device scratch, and nothing is
    allocated here either, so ``out [B, n_q, D]`` (bf16) must be given.  Calls
    that overlap in time on one device race (they share the scratch)."""
    cd, pt = _cache(k_pool, v_pool, table)
    _bits16(q, "q")
    _bits16(out, "out")
    _i32(slots, "slots")
    _i32(seq_lens, "seq_lens")
    B, n_q, D = q.shape
    if D != cd.head_dim or tuple(out.shape) != (B, n_q, D):
        raise ValueError("q / out shapes do not match the pools")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _bits16(k_new, "k_new")
        _bits16(v_new, "v_new")
        if tuple(k_new.shape) != (B, cd.n_kv_heads, D) or v_new.shape != k_new.shape:
            raise ValueError("k_new / v_new must be [B, n_kv, head_dim]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seq_len_hint is None:
        max_seq_len_hint = pt.pages_per_slot * cd.page_size
    check(lib().pkv_attn_decode_noalloc(_ptr(q), n_q, _ptr(slots), _ptr(seq_lens), B,
                                        int(max_seq_len_hint), pt, ctypes.byref(cd),
                                        _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                                        float(scale), int(window), _ptr(out), _ptr(lse),
                                        _stream(stream, q.device)))
    return out


def new_decode_workspace(nbytes, device="cuda"):
    """A zero-filled decode workspace of ``nbytes``, rounded up to 16 (its last
    bytes hold the split arrival counters, which must start at zero; every
    call leaves them at zero).  Pass the whole tensor to every call that uses
    it."""
    return torch.zeros(max((int(nbytes) + 15) // 16 * 16, 16), dtype=torch.uint8, device=device)


def rope_table(max_pos, head_dim, theta, device="cuda", stream=None, rotary_fraction=1.0):
    """fp32 ``cos, sin [max_pos, head_dim/2]`` of the default rope frequencies
    (``rotary_fraction < 1``: only that leading fraction rotates, the rest
    pass through -- Gemma-4's partial RoPE)."""
    c = torch.empty((max_pos, head_dim // 2), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    check(lib().pkv_rope_table_partial(_ptr(c), _ptr(s), max_pos, head_dim, float(theta),
                                       float(rotary_fraction), _stream(stream, c.device)))
    return c, s


def attn_prefill(q, cu_seqlens, slots, table, k_pool, v_pool, scale=None, window=0,
                 start_pos=None, max_seqlen_q_hint=None, prologue=None, out=None, lse=None,
                 stream=None):
    """Packed varlen prefill attention; returns ``out [T, n_q, D]`` (bf16).

    ``prologue`` (optional) is a dict with ``q_norm_w, k_norm_w, eps, cos, sin,
    k, v`` and optionally ``q_out`` and ``v_norm`` (Gemma-4: v gets RMSNorm
    without a gain; for K=V layers pass the raw k as ``v``): k (normalised and
    rotated) and v are appended before the attention, and q is normalised and rotated inside the
    attention kernel (``q`` itself is not modified; the normalised q' is also
    written to ``q_out`` when given).  With ``k`` and ``v`` None (or absent)
    nothing is appended: the keys are already in the pages and only q is
    normalised and rotated.
    """
    cd, pt = _cache(k_pool, v_pool, table)
    _bits16(q, "q")
    _i32(cu_seqlens, "cu_seqlens")
    _i32(slots, "slots")
    if start_pos is not None:
        _i32(start_pos, "start_pos")
    T, n_q, D = q.shape
    n_seqs = slots.numel()
    if cu_seqlens.numel() != n_seqs + 1:
        raise ValueError("cu_seqlens must have n_seqs + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen_q_hint is None:
        max_seqlen_q_hint = max(T, 1)
    if out is None:
        out = torch.empty((T, n_q, D), dtype=torch.bfloat16, device=q.device)
    pro = None
    if prologue is not None:
        p = prologue
        kr, vr = p.get("k"), p.get("v")
        if (kr is None) != (vr is None):
            raise ValueError("prologue: give both k and v, or neither")
        kw = p.get("k_norm_w")
        for name, t in (("k", kr), ("v", vr), ("q_norm_w", p["q_norm_w"]), ("k_norm_w", kw)):
            if t is not None:
                _bits16(t, name)
        if kr is not None and (tuple(kr.shape) != (T, cd.n_kv_heads, D) or vr.shape != kr.shape):
            raise ValueError("prologue k / v must be [T, n_kv, head_dim]")
        cos, sin = p["cos"], p["sin"]
        if cos.dtype != torch.float32 or tuple(cos.shape[1:]) != (D // 2,) or \
                sin.shape != cos.shape:
            raise ValueError("rope tables must be fp32 [max_pos, head_dim/2]")
        q_out = p.get("q_out")
        if q_out is not None:
            _bits16(q_out, "q_out")
            if tuple(q_out.shape) != (T, n_q, D):
                raise ValueError("prologue q_out must be [T, n_q, head_dim]")
        pro = Prologue(p["q_norm_w"].data_ptr(), kw.data_ptr() if kw is not None else None,
                       float(p["eps"]), cos.data_ptr(), sin.data_ptr(), cos.shape[0],
                       kr.data_ptr() if kr is not None else None,
                       vr.data_ptr() if vr is not None else None,
                       q_out.data_ptr() if q_out is not None else None,
                       1 if p.get("v_norm") else 0)
    check(lib().pkv_attn_prefill(_ptr(q), n_q, _ptr(cu_seqlens), _ptr(slots), _ptr(start_pos),
                                 n_seqs, T, int(max_seqlen_q_hint), pt, ctypes.byref(cd),
                                 _ptr(k_pool), _ptr(v_pool), float(scale), int(window),
                                 ctypes.byref(pro) if pro is not None else None, _ptr(out),
                                 _ptr(lse), None, 0, _stream(stream, q.device)))
    return out


VALIDATE_SLOT, VALIDATE_PAGE, VALIDATE_POS = 1, 2, 4


def set_validation(on=True):
    """Switch validation mode on or off (process-wide; see the header)."""
    check(lib().pkv_set_validation(1 if on else 0))


def validation_flags(clear=True, stream=None, device=None):
    """Synchronise the stream and return the device's validation flag word
    (VALIDATE_SLOT | VALIDATE_PAGE | VALIDATE_POS bits), clearing it if asked."""
    flags = ctypes.c_uint32(0)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    check(lib().pkv_validation_flags(ctypes.byref(flags), 1 if clear else 0, _stream(stream, dev)))
    return int(flags.value)


class PageAllocator:
    """Host-side slot / page allocator (C++), see ``pkv_pt_*`` in the header."""

    def __init__(self, n_pages, page_size, max_slots):
        h = ctypes.c_void_p()
        check(lib().pkv_pt_create(n_pages, page_size, max_slots, ctypes.byref(h)))
        self._h = h
        self.n_pages, self.page_size, self.max_slots = n_pages, page_size, max_slots

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib().pkv_pt_destroy(h)
            self._h = None

    @property
    def pages_available(self):
        return lib().pkv_pt_pages_available(self._h)

    @property
    def free_slot_count(self):
        return lib().pkv_pt_free_slot_count(self._h)

    def can_reserve(self, size, slot=None):
        ok = ctypes.c_int32()
        check(lib().pkv_pt_can_reserve(self._h, size, -1 if slot is None else slot,
                                       ctypes.byref(ok)))
        return bool(ok.value)

    def allocate(self):
        s = ctypes.c_int32()
        st = lib().pkv_pt_allocate(self._h, ctypes.byref(s))
        if st != 0:
            raise PkvError(st, "no free slot")
        return s.value

    def reserve(self, slot, seq_len, dry_run=False):
        ok = ctypes.c_int32()
        st = lib().pkv_pt_reserve(self._h, slot, seq_len, int(dry_run), ctypes.byref(ok))
        if st != 0:
            raise PkvError(st, f"cannot reserve {seq_len} tokens in slot {slot} "
                               f"({self.pages_available} pages free)")
        return bool(ok.value)

    def erase(self, slot):
        check(lib().pkv_pt_erase(self._h, slot))

    def capacity(self, slot):
        return lib().pkv_pt_capacity(self._h, slot)

    def row(self, slot):
        n = lib().pkv_pt_row(self._h, slot, None, 0)
        buf = (ctypes.c_int32 * max(n, 1))()
        lib().pkv_pt_row(self._h, slot, buf, n)
        return list(buf[:n])

    def free_pages(self):
        n = lib().pkv_pt_free_pages(self._h, None, 0)
        buf = (ctypes.c_int32 * max(n, 1))()
        lib().pkv_pt_free_pages(self._h, buf, n)
        return list(buf[:n])

    def to_device(self, pages_per_slot, device="cuda"):
        """This allocator's state as a ``DevicePageState`` for device-side reserves
        and erases."""
        free = self.free_pages()
        fp = torch.zeros(self.n_pages, dtype=torch.int32)
        fp[:len(free)] = torch.tensor(free, dtype=torch.int32)
        cap = torch.tensor([self.capacity(s) if s > 0 else 0 for s in range(self.max_slots)],
                           dtype=torch.int32)
        return DevicePageState(self.export(pages_per_slot).to(device), fp.to(device),
                               torch.tensor([len(free)], dtype=torch.int32, device=device),
                               cap.to(device), self.page_size)

    def export(self, pages_per_slot):
        """Device-format table as an int32 CPU tensor ``[max_slots, pages_per_slot]``."""
        t = torch.empty((self.max_slots, pages_per_slot), dtype=torch.int32)
        check(lib().pkv_pt_export(self._h, ctypes.cast(t.data_ptr(),
                                                       ctypes.POINTER(ctypes.c_int32)),
                                  pages_per_slot))
        return t


class DevicePageState:
    """Device buffers of the allocator state used by ``pkv_pt_device_reserve`` and
    ``pkv_pt_device_erase``:
    ``table`` int32 [max_slots, pages_per_slot], ``free_pages`` int32 [n_pages]
    (the free stack, bottom first), ``free_count`` int32 [1], ``capacity``
    int32 [max_slots] and the ``status`` flag word (uint32 [1], as int32)."""

    def __init__(self, table, free_pages, free_count, capacity, page_size):
        for t, name in ((table, "table"), (free_pages, "free_pages"), (free_count, "free_count"),
                        (capacity, "capacity")):
            _i32(t, name)
        self.table, self.free_pages, self.free_count, self.capacity = (table, free_pages,
                                                                        free_count, capacity)
        self.status = torch.zeros(1, dtype=torch.int32, device=table.device)
        self.page_size = page_size
        self._c = _lib.PtDevice(table.data_ptr(), free_pages.data_ptr(), free_count.data_ptr(),
                                capacity.data_ptr(), self.status.data_ptr(), table.shape[0],
                                table.shape[1], page_size, free_pages.numel())

    def reserve(self, slots, seq_lens, stream=None):
        """Grow the slots of rows b (in order) to seq_lens[b] tokens on the device
        (``pkv_pt_device_reserve``); rows that cannot be served set ``status`` bits."""
        _i32(slots, "slots")
        _i32(seq_lens, "seq_lens")
        check(lib().pkv_pt_device_reserve(ctypes.byref(self._c), _ptr(slots), _ptr(seq_lens),
                                          slots.numel(), _stream(stream, self.table.device)))

    def erase(self, slots, stream=None):
        """Return the pages of the listed slots (in order) to the free stack on the
        device and reset their capacity to 0 and rows to -1
        (``pkv_pt_device_erase``)."""
        _i32(slots, "slots")
        check(lib().pkv_pt_device_erase(ctypes.byref(self._c), _ptr(slots), slots.numel(),
                                        _stream(stream, self.table.device)))
