"""ctypes loader of ``libpkv.so`` and the C structs of ``include/pkv.h``.

The library must be built (``python -m paged_kv_attention_pagetable_amd.build``);
loading fails loudly otherwise.  torch is imported first on purpose: the library
then binds to the HIP runtime torch already loaded, so both share one runtime,
one device context and the same streams.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (see module docstring: load order matters)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pkv.h")

c_int32 = ctypes.c_int32
c_void_p = ctypes.c_void_p
c_size_t = ctypes.c_size_t
c_float = ctypes.c_float

PKV_OK = 0
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_UNSUPPORTED",
                3: "PKV_ERR_LAUNCH", 4: "PKV_ERR_WORKSPACE", 5: "PKV_ERR_CAPACITY"}


class CacheDesc(ctypes.Structure):
    _fields_ = [("n_pages", c_int32), ("page_size", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32)]


class PageTableRef(ctypes.Structure):
    _fields_ = [("table", c_void_p), ("max_slots", c_int32), ("pages_per_slot", c_int32)]


class Prologue(ctypes.Structure):
    _fields_ = [("q_norm_w", c_void_p), ("k_norm_w", c_void_p), ("eps", c_float),
                ("rope_cos", c_void_p), ("rope_sin", c_void_p), ("max_pos", c_int32),
                ("k_raw", c_void_p), ("v_raw", c_void_p), ("q_out", c_void_p),
                ("v_norm", c_int32)]


class PtDevice(ctypes.Structure):
    _fields_ = [("table", c_void_p), ("free_pages", c_void_p), ("free_count", c_void_p),
                ("capacity", c_void_p), ("status", c_void_p), ("max_slots", c_int32),
                ("pages_per_slot", c_int32), ("page_size", c_int32), ("n_pages", c_int32)]


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_SIGS = {
    "pkv_append": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, PageTableRef,
                             ctypes.POINTER(CacheDesc), c_void_p, c_void_p, c_void_p]),
    "pkv_attn_decode": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                  PageTableRef, ctypes.POINTER(CacheDesc), c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_float, c_int32, c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p]),
    "pkv_attn_decode_noalloc": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                          c_int32, PageTableRef, ctypes.POINTER(CacheDesc),
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                          c_int32, c_void_p, c_void_p, c_void_p]),
    "pkv_decode_workspace_size": (c_size_t, [c_int32] * 6),
    "pkv_decode_plan": (c_int32, [c_int32] * 6 + [ctypes.POINTER(ctypes.c_int64)]),
    "pkv_attn_prefill": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_int32, c_int32, PageTableRef, ctypes.POINTER(CacheDesc),
                                   c_void_p, c_void_p, c_float, c_int32,
                                   ctypes.POINTER(Prologue), c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
    "pkv_rope_table": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, ctypes.c_double,
                                 c_void_p]),
    "pkv_rope_table_partial": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, ctypes.c_double,
                                         ctypes.c_double, c_void_p]),
    "pkv_prefill_workspace_size": (c_size_t, [c_int32] * 3),
    "pkv_set_validation": (c_int32, [c_int32]),
    "pkv_validation_flags": (c_int32, [ctypes.POINTER(ctypes.c_uint32), c_int32, c_void_p]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_pt_create": (c_int32, [c_int32, c_int32, c_int32, ctypes.POINTER(c_void_p)]),
    "pkv_pt_destroy": (None, [c_void_p]),
    "pkv_pt_pages_available": (c_int32, [c_void_p]),
    "pkv_pt_free_slot_count": (c_int32, [c_void_p]),
    "pkv_pt_can_reserve": (c_int32, [c_void_p, c_int32, c_int32, ctypes.POINTER(c_int32)]),
    "pkv_pt_allocate": (c_int32, [c_void_p, ctypes.POINTER(c_int32)]),
    "pkv_pt_reserve": (c_int32, [c_void_p, c_int32, c_int32, c_int32, ctypes.POINTER(c_int32)]),
    "pkv_pt_erase": (c_int32, [c_void_p, c_int32]),
    "pkv_pt_capacity": (c_int32, [c_void_p, c_int32]),
    "pkv_pt_row": (c_int32, [c_void_p, c_int32, ctypes.POINTER(c_int32), c_int32]),
    "pkv_pt_free_pages": (c_int32, [c_void_p, ctypes.POINTER(c_int32), c_int32]),
    "pkv_pt_export": (c_int32, [c_void_p, ctypes.POINTER(c_int32), c_int32]),
    "pkv_pt_device_reserve": (c_int32, [ctypes.POINTER(PtDevice), c_void_p, c_void_p, c_int32,
                                        c_void_p]),
    "pkv_pt_device_erase": (c_int32, [ctypes.POINTER(PtDevice), c_void_p, c_int32, c_void_p]),
}

_lib = None


def header_functions():
    """Names of the functions ``include/pkv.h`` declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first with "
                "`python -m paged_kv_attention_pagetable_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int):
    if status != PKV_OK:
        raise PkvError(status, lib().pkv_last_error().decode())
