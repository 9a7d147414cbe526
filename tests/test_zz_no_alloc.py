"""The allocation-free decode entry point (pkv_attn_decode_noalloc) against
pkv_attn_decode: same kernels and plan, so bitwise equal outputs, lse and pools,
on two calls in a row (the second smaller), plus the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pagetable_amd as pkv
from synth import make_decode_case
from tests.gpu_util import (DEV, assert_attn_close, dev_bits, dev_i32, gpu_decode_setup,
                            host_bits, host_f64, oracle_decode_pools)

pytestmark = pytest.mark.gpu


def _both(case, hint, fused):
    """(out, lse, k_pool, v_pool) of the workspace call and of the no-alloc call,
    each on its own copy of the pools."""
    res = []
    for noalloc in (False, True):
        kp, vp, table = gpu_decode_setup(case, with_new_token=not fused)
        q = dev_bits(case.q)
        out = torch.full((case.B, case.n_q, case.head_dim), -1, dtype=torch.int16,
                         device=DEV).view(torch.bfloat16)
        lse = torch.full((case.B, case.n_q), 7.0, dtype=torch.float32, device=DEV)
        kn = dev_bits(case.k_new) if fused else None
        vn = dev_bits(case.v_new) if fused else None
        args = (q, dev_i32(case.slots), dev_i32(case.seq_lens), table, kp, vp)
        if noalloc:
            pkv.attn_decode_noalloc(*args, out, scale=case.scale, window=case.window,
                                    max_seq_len_hint=hint, lse=lse, k_new=kn, v_new=vn)
        else:
            pkv.attn_decode(*args, scale=case.scale, window=case.window, max_seq_len_hint=hint,
                            out=out, lse=lse, k_new=kn, v_new=vn)
        torch.cuda.synchronize()
        res.append((out, lse, kp, vp))
    return res


def _check(case, hint, fused):
    assert pkv.decode_workspace_size(case.B, case.n_q, case.n_kv, case.head_dim, hint,
                                     case.window) > 0, "the case must use the scratch"
    (o1, l1, k1, v1), (o2, l2, k2, v2) = _both(case, hint, fused)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    okp, ovp = oracle_decode_pools(case)
    assert np.array_equal(host_bits(k2), okp) and np.array_equal(host_bits(v2), ovp)
    ref, ref_lse = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                      case.scale, case.window)
    assert_attn_close(host_f64(o2), ref, "no-alloc decode")
    live = case.seq_lens > 0
    g = l2.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g[live] - ref_lse[live]), initial=0.0) <= 1e-3
    assert np.all(np.isneginf(g[~live]))


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # first call: 12 rows of up to 4000 keys (several splits per row, 4-wave plan)
    big = make_decode_case(24, 8, 128, 128, [4000, 17, 0, 2500, 999, 3100, 1, 4096, 640, 0,
                                             2049, 3333], max_slots=14, seed=4100,
                           spare_pages=2)
    _check(big, 4096, fused=True)
    # second call, smaller: 3 rows, head_dim 256 with a window (dim-split kernel)
    small = make_decode_case(8, 2, 256, 64, [900, 300, 1500], max_slots=5, seed=4101,
                             window=512, spare_pages=2)
    _check(small, 1536, fused=False)


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    """32 rows of G 8, head_dim 256 over 16384 keys: the split partials need
    more than the 16 MiB scratch; the call fails on the host and enqueues
    nothing (out keeps its fill)."""
    need = pkv.decode_workspace_size(32, 8, 1, 256, 16384, 0)
    assert need > pkv.DECODE_SCRATCH_BYTES
    case = make_decode_case(8, 1, 256, 64, [5] * 32, max_slots=33, seed=4102, spare_pages=1)
    kp, vp, table = gpu_decode_setup(case)
    out = torch.full((32, 8, 256), 3, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    with pytest.raises(pkv.PkvError, match="static scratch"):
        pkv.attn_decode_noalloc(dev_bits(case.q), dev_i32(case.slots), dev_i32(case.seq_lens),
                                table, kp, vp, out, max_seq_len_hint=16384)
    torch.cuda.synchronize()
    assert bool((out.view(torch.int16) == 3).all())
