"""The C-ABI library loads, exports every declared symbol, and its host-only
parts (argument checks, the slot/page allocator) behave as documented.

No compute call runs here: argument checks return before anything touches a
device, and the allocator is pure host code.
"""

import ctypes
import json
import os

import numpy as np
import pytest

import paged_kv_attention_pagetable_amd as pkv
from paged_kv_attention_pagetable_amd import _lib
from oracle import PageTableModel
from tests.conftest import GOLDEN
from tests.test_oracle_pagetable import run_sequence


def test_library_exports_every_header_function():
    names = _lib.header_functions()
    assert len(names) >= 19
    L = pkv.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(_lib._SIGS), "binding signatures and header disagree"
    assert L.pkv_version().decode().startswith("pkv ")


def _desc(n_pages=4, ps=16, n_kv=2, D=64):
    return _lib.CacheDesc(n_pages, ps, n_kv, D)


def _pt(table=1, max_slots=3, pps=4):
    return _lib.PageTableRef(table, max_slots, pps)


P = 256   # a fake, 16-byte aligned device address: every call below returns before a launch


def _decode(**kw):
    args = dict(q=P, n_q=4, slots=P, seq_lens=P, B=2, hint=64, pt=_pt(), cd=_desc(), k=P, v=P,
                scale=0.125, window=0, out=P, lse=None, ws=None, ws_bytes=0)
    args.update(kw)
    a = args
    return pkv.lib().pkv_attn_decode(a["q"], a["n_q"], a["slots"], a["seq_lens"], a["B"],
                                     a["hint"], a["pt"], ctypes.byref(a["cd"]), a["k"], a["v"],
                                     a.get("k_new"), a.get("v_new"), a["scale"], a["window"],
                                     a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_decode_argument_checks_return_before_launch():
    assert _decode(q=None) == 1
    assert _decode(n_q=3) == 1                       # not a multiple of n_kv
    assert _decode(n_q=2 * 17) == 2                  # GQA ratio above 16
    assert _decode(cd=_desc(D=96)) == 2              # unsupported head_dim
    assert _decode(cd=_desc(ps=24)) == 2             # page size not a power of two
    assert _decode(cd=_desc(ps=8)) == 2
    assert _decode(pt=_pt(table=None)) == 1
    assert _decode(pt=_pt(max_slots=1)) == 1         # slot 0 reserved: need >= 2
    assert _decode(window=-1) == 1
    assert _decode(scale=float("nan")) == 1
    assert _decode(hint=0) == 1
    assert _decode(B=-1) == 1
    assert _decode(k_new=P) == 1                     # k_new without v_new
    assert _decode(q=P + 8) == 1                     # bf16 buffers must be 16-byte aligned
    assert b"aligned" in pkv.lib().pkv_last_error()
    assert _decode(out=P + 2) == 1
    assert _decode(k_new=P + 4, v_new=P) == 1
    assert _decode(n_q=2 * 16, cd=_desc(D=256)) == 2  # G * head_dim above 2048
    # a split-K plan needs a workspace
    need = pkv.decode_workspace_size(64, 32, 8, 128, 4096, 0)
    assert need > 0
    assert _decode(B=64, n_q=32, cd=_desc(n_pages=100, ps=128, n_kv=8, D=128),
                   pt=_pt(max_slots=65, pps=32), hint=4096) == 4
    assert b"workspace" in pkv.lib().pkv_last_error()
    # ... 16-byte aligned (the merge moves partials with 8- and 16-byte accesses)
    assert _decode(B=64, n_q=32, cd=_desc(n_pages=100, ps=128, n_kv=8, D=128),
                   pt=_pt(max_slots=65, pps=32), hint=4096, ws=P + 8, ws_bytes=need) == 1
    assert b"workspace must be 16-byte aligned" in pkv.lib().pkv_last_error()
    # B == 0 is a valid no-op (nothing launched)
    assert _decode(B=0) == 0


def test_workspace_size_plan_is_monotone_and_zero_when_unsplit():
    assert pkv.decode_workspace_size(2, 4, 2, 64, 50, 0) == 0     # one split per row
    a = pkv.decode_workspace_size(64, 24, 8, 128, 4096, 0)
    b = pkv.decode_workspace_size(64, 24, 8, 128, 4096, 512)   # window bounds the range
    assert a > 0 and b <= a
    # the size covers the arrival counters (4 bytes per row and kv head) and
    # is a multiple of 16
    assert a % 16 == 0 and a >= 4 * 64 * 8


def test_append_and_prefill_argument_checks():
    L = pkv.lib()
    cd = _desc()
    assert L.pkv_append(P, P, P, P, -1, _pt(), ctypes.byref(cd), P, P, None) == 1
    assert L.pkv_append(P, P, P, P, 0, _pt(), ctypes.byref(cd), P, P, None) == 0  # T = 0 no-op
    assert L.pkv_append(None, P, P, P, 5, _pt(), ctypes.byref(cd), P, P, None) == 1
    assert L.pkv_append(P, P, P, P, 5, _pt(), ctypes.byref(cd), P + 2, P, None) == 1  # misaligned pool
    cd96 = _desc(D=96)        # head_dim not supported (64, 128, 256, 512 are)
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd96), P, P,
                              0.1, 0, None, P, None, None, 0, None) == 2
    assert L.pkv_attn_prefill(None, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P,
                              0.1, 0, None, P, None, None, 0, None) == 1
    bad = _lib.Prologue(None, P, 1e-6, P, P, 16, P, P)
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P, 0.1, 0,
                              ctypes.byref(bad), P, None, None, 0, None) == 1
    # k without v (or v without k) is an error; both NULL = q-only prologue,
    # which still needs q's norm weights and the rotary tables
    half = _lib.Prologue(P, P, 1e-6, P, P, 16, P, None)
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P, 0.1, 0,
                              ctypes.byref(half), P, None, None, 0, None) == 1
    q_only_no_table = _lib.Prologue(P, None, 1e-6, None, P, 16, None, None)
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P, 0.1, 0,
                              ctypes.byref(q_only_no_table), P, None, None, 0, None) == 1
    # the prologue's grid covers at most 65535 blocks of 32 tokens
    good = _lib.Prologue(P, P, 1e-6, P, P, 16, P, P)
    skew = _lib.Prologue(P, P, 1e-6, P + 4, P, 16, P, P)   # misaligned cos table
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P,
                              0.1, 0, ctypes.byref(skew), P, None, None, 0, None) == 1
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 2097121, 8, _pt(), ctypes.byref(cd), P, P,
                              0.1, 0, ctypes.byref(good), P, None, None, 0, None) == 2
    # prefill scale must be > 0
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P,
                              -0.1, 0, None, P, None, None, 0, None) == 1
    assert L.pkv_attn_prefill(P, 4, P, P, None, 1, 8, 8, _pt(), ctypes.byref(cd), P, P,
                              0.0, 0, None, P, None, None, 0, None) == 1
    assert L.pkv_rope_table(None, 1, 8, 64, 1e6, None) == 1
    # the prefill kernels need no workspace; validation-flag reads need an output
    assert L.pkv_prefill_workspace_size(4096, 16, 32) == 0
    assert L.pkv_validation_flags(None, 1, None) == 1
    assert L.pkv_set_validation(0) == 0
    assert L.pkv_rope_table(1, 1, 8, 63, 1e6, None) == 1
    assert L.pkv_rope_table_partial(1, 1, 8, 64, 1e6, 0.0, None) == 1   # fraction in (0, 1]
    assert L.pkv_rope_table_partial(1, 1, 8, 64, 1e6, 1.5, None) == 1


def test_cpp_allocator_follows_golden_sequence():
    with open(os.path.join(GOLDEN, "pagetable_sequence.json")) as f:
        g = json.load(f)
    pt = pkv.PageAllocator(g["n_pages"], g["page_size"], g["max_slots"])

    class Adapter:
        """Gives the C++ allocator the model's interface for the shared driver."""

        def allocate(self):
            return pt.allocate()

        def can_reserve(self, size, slot=None):
            return pt.can_reserve(size, slot)

        def reserve(self, slot, seq_len, dry_run=False):
            try:
                return pt.reserve(slot, seq_len, dry_run)
            except pkv.PkvError as e:
                raise RuntimeError(str(e))

        def erase(self, slot):
            pt.erase(slot)

    def check(_, st):
        if "row" in st:
            assert pt.row(st["slot"]) == st["row"]
        if "capacity" in st:
            assert pt.capacity(st["slot"]) == st["capacity"]
        if "free_pages" in st:
            assert pt.free_pages() == st["free_pages"]

    run_sequence(Adapter(), g["steps"], check)
    assert np.array_equal(pt.export(g["n_pages"]).numpy(), np.array(g["final_device_table"]))


def test_cpp_allocator_matches_model_on_random_ops():
    rng = np.random.default_rng(7)
    n_pages, ps, ms = 60, 16, 9
    model = PageTableModel(n_pages, ps, ms)
    pt = pkv.PageAllocator(n_pages, ps, ms)
    for _ in range(800):
        r = rng.random()
        size = int(rng.integers(0, 500))
        assert pt.can_reserve(size) == model.can_reserve(size)
        if r < 0.25:
            if model.free_slots:
                assert pt.allocate() == model.allocate()
            continue
        s = int(rng.integers(1, ms))
        if s in model.free_slots:
            continue
        if r < 0.75:
            n = int(rng.integers(0, 400))
            dry = bool(rng.random() < 0.3)
            assert pt.can_reserve(n, s) == model.can_reserve(n, s)
            try:
                want = model.reserve(s, n, dry_run=dry)
            except RuntimeError:
                with pytest.raises(pkv.PkvError):
                    pt.reserve(s, n, dry)
                continue
            assert pt.reserve(s, n, dry) == want
        else:
            model.erase(s)
            pt.erase(s)
        assert pt.free_pages() == model.free_pages
        assert pt.pages_available == model.pages_available
        for s2 in range(1, ms):
            assert pt.row(s2) == model.rows[s2]
            if s2 not in model.free_slots:
                assert pt.capacity(s2) == model.capacity[s2]
    pps = int(max((model.device_table[s] >= 0).sum() for s in range(1, ms))) + 2
    assert np.array_equal(pt.export(pps).numpy(), model.table(pps))


def test_allocator_reports_exhaustion_and_bad_slots():
    pt = pkv.PageAllocator(4, 8, 3)
    s = pt.allocate()
    assert s == 1
    assert pt.reserve(s, 24)          # 3 pages
    with pytest.raises(pkv.PkvError):
        pt.reserve(s, 25)
    assert pt.capacity(s) == 24
    assert not pt.reserve(s, 25, dry_run=True)
    assert pt.allocate() == 2
    with pytest.raises(pkv.PkvError):
        pt.allocate()
    with pytest.raises(pkv.PkvError):
        pt.erase(0)                   # slot 0 is never granted
    with pytest.raises(pkv.PkvError):
        pt.reserve(3, 1)              # out of range


def test_device_reserve_argument_checks():
    L = pkv.lib()
    ok = _lib.PtDevice(P, P, P, P, P, 9, 8, 128, 100)
    assert L.pkv_pt_device_reserve(None, P, P, 4, None) == 1
    assert L.pkv_pt_device_reserve(ctypes.byref(ok), P, P, -1, None) == 1
    assert L.pkv_pt_device_reserve(ctypes.byref(ok), P, P, 0, None) == 0      # no-op
    assert L.pkv_pt_device_reserve(ctypes.byref(ok), None, P, 4, None) == 1
    for bad in (_lib.PtDevice(P, P, P, P, P, 1, 8, 128, 100),    # slot 0 reserved: max_slots >= 2
                _lib.PtDevice(P, P, P, P, P, 9, 0, 128, 100),
                _lib.PtDevice(P, P, P, P, P, 9, 8, 0, 100),
                _lib.PtDevice(P, P, P, P, P, 9, 8, 128, 1),
                _lib.PtDevice(None, P, P, P, P, 9, 8, 128, 100),
                _lib.PtDevice(P, P, P, P, None, 9, 8, 128, 100)):
        assert L.pkv_pt_device_reserve(ctypes.byref(bad), P, P, 4, None) == 1


def test_device_erase_argument_checks():
    L = pkv.lib()
    ok = _lib.PtDevice(P, P, P, P, P, 9, 8, 128, 100)
    assert L.pkv_pt_device_erase(None, P, 4, None) == 1
    assert L.pkv_pt_device_erase(ctypes.byref(ok), P, -1, None) == 1
    assert L.pkv_pt_device_erase(ctypes.byref(ok), P, 0, None) == 0      # no-op
    assert L.pkv_pt_device_erase(ctypes.byref(ok), None, 4, None) == 1
    for bad in (_lib.PtDevice(P, P, P, P, P, 1, 8, 128, 100),
                _lib.PtDevice(P, P, P, P, P, 9, 8, 128, 1),
                _lib.PtDevice(P, P, P, None, P, 9, 8, 128, 100),
                _lib.PtDevice(P, P, P, P, P, 9, 1 << 25, 64, 100)):      # 2^31 tokens per row
        assert L.pkv_pt_device_erase(ctypes.byref(bad), P, 4, None) == 1
        assert "pkv_pt_device_erase" in pkv.lib().pkv_last_error().decode()
