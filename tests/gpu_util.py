"""Helpers for the GPU parity tests: move synth cases to the device, run the
library, and run the oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_attention_pagetable_amd as pkv
from synth import SENTINEL_BITS

DEV = "cuda"
ATOL = 2e-2   # max |gpu - oracle| over an output tensor
RTOL = 1e-2   # max |gpu - oracle| / max |oracle|


def dev_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (numpy) -> bf16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_attn_close(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    mx = float(err.max()) if err.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    assert mx <= ATOL, f"{what}: max abs err {mx:.3e} > {ATOL}"
    if scale > 0:
        assert mx / scale <= RTOL, f"{what}: max rel err {mx / scale:.3e} > {RTOL}"
    return mx


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between two arrays of bf16 bit
    patterns (finite values): the bits mapped to integers in the order of the
    values they encode (negatives mirrored below zero), then subtracted."""
    def key(u):
        u = u.astype(np.int64)
        return np.where(u < 0x8000, u, 0x8000 - u)
    return np.abs(key(a_bits) - key(b_bits))


def gpu_pools(case):
    kp, vp = pkv.new_pools(case.n_pages, case.n_kv, case.page_size, case.head_dim, DEV,
                           fill=int(SENTINEL_BITS.astype(np.int16)))
    return kp, vp


def gpu_decode_setup(case, with_new_token=True):
    """Device pools with the history (and the new token) appended by the library."""
    kp, vp = gpu_pools(case)
    table = dev_i32(case.table)
    hk, hv, hs, hp = case.history_tokens()
    if len(hs):
        pkv.append(dev_bits(hk), dev_bits(hv), dev_i32(hs), dev_i32(hp), table, kp, vp)
    if with_new_token:
        pkv.append(dev_bits(case.k_new), dev_bits(case.v_new), dev_i32(case.append_slots()),
                   dev_i32(case.append_pos()), table, kp, vp)
    return kp, vp, table


def oracle_decode_pools(case):
    kp, vp = case.empty_pools()
    hk, hv, hs, hp = case.history_tokens()
    oracle.append(kp, vp, case.table, hk, hv, hs, hp)
    oracle.append(kp, vp, case.table, case.k_new, case.v_new, case.append_slots(),
                  case.append_pos())
    return kp, vp


def run_gpu_decode(case, kp, vp, table, hint=None, with_lse=True, fused_append=False,
                   workspace=None):
    q = dev_bits(case.q)
    lse = torch.empty((case.B, case.n_q), dtype=torch.float32, device=DEV) if with_lse else None
    kn = dev_bits(case.k_new) if fused_append else None
    vn = dev_bits(case.v_new) if fused_append else None
    out = pkv.attn_decode(q, dev_i32(case.slots), dev_i32(case.seq_lens), table, kp, vp,
                          scale=case.scale, window=case.window,
                          max_seq_len_hint=hint or max(int(case.seq_lens.max()), 1), lse=lse,
                          k_new=kn, v_new=vn, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse
