"""Pins of the oracle's prologue (RMSNorm + half-split RoPE), CPU only.

The pages fix the structure (RMSNorm over head_dim, then
``x*cos + rotate_half(x)*sin``) but print no values; the frequency
convention (``theta ** (-2i/D)``) is a reading, pinned here only by its own
closed forms.
"""

import math

import numpy as np
import pytest

import oracle


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 64))
    assert np.array_equal(oracle.rope_apply(x, 0, oracle.rope_inv_freq(64, 1e6)), x)


def test_rope_basis_vectors_closed_form():
    D, theta, p = 16, 1e4, 7
    inv = oracle.rope_inv_freq(D, theta)
    for i in range(D // 2):
        w = theta ** (-2.0 * i / D)
        e = np.zeros(D)
        e[i] = 1.0
        r = oracle.rope_apply(e, p, inv)
        want = np.zeros(D)
        want[i] = math.cos(p * w)
        want[i + D // 2] = math.sin(p * w)
        assert np.max(np.abs(r - want)) <= 1e-15
        e = np.zeros(D)
        e[i + D // 2] = 1.0
        r = oracle.rope_apply(e, p, inv)
        want = np.zeros(D)
        want[i] = -math.sin(p * w)
        want[i + D // 2] = math.cos(p * w)
        assert np.max(np.abs(r - want)) <= 1e-15


def test_rope_frequencies_closed_form():
    inv = oracle.rope_inv_freq(128, 1e6)
    assert inv[0] == 1.0
    assert abs(inv[-1] - 1e6 ** (-126 / 128)) <= 1e-18
    ratios = inv[1:] / inv[:-1]
    assert np.max(np.abs(ratios - 1e6 ** (-2 / 128))) <= 1e-14


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(1)
    D = 32
    inv = oracle.rope_inv_freq(D, 1e6)
    x = rng.standard_normal(D)
    r = oracle.rope_apply(x, 123, inv)
    h = D // 2
    assert np.max(np.abs(np.hypot(r[:h], r[h:]) - np.hypot(x[:h], x[h:]))) <= 1e-12
    r2 = oracle.rope_apply(oracle.rope_apply(x, 40, inv), 83, inv)
    assert np.max(np.abs(r2 - r)) <= 1e-12


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(2)
    D = 64
    inv = oracle.rope_inv_freq(D, 1e6)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    a = oracle.rope_apply(q, 37, inv) @ oracle.rope_apply(k, 11, inv)
    b = oracle.rope_apply(q, 537, inv) @ oracle.rope_apply(k, 511, inv)
    assert abs(a - b) <= 1e-10


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128)) * 3.0
    y = oracle.rmsnorm(x, np.ones(128), 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1.0)) <= 1e-12
    # scale invariance (eps = 0) and a gain acts elementwise
    assert np.max(np.abs(oracle.rmsnorm(7.5 * x, np.ones(128), 0.0) - y)) <= 1e-12
    w = rng.standard_normal(128)
    assert np.max(np.abs(oracle.rmsnorm(x, w, 0.0) - y * w)) <= 1e-12
    # constant vector c: c / sqrt(c^2 + eps)
    c, eps = 0.01, 1e-6
    out = oracle.rmsnorm(np.full(8, c), np.ones(8), eps)
    assert np.max(np.abs(out - c / math.sqrt(c * c + eps))) <= 1e-15


def test_rmsnorm_matches_torch_rms_norm_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 128))
    w = rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w),
                                       eps=1e-6).numpy()
    assert np.max(np.abs(oracle.rmsnorm(x, w, 1e-6) - ref)) <= 1e-12


def test_prologue_composition_and_v_passthrough():
    from synth import make_prefill_case
    case = make_prefill_case(4, 2, 32, 8, [5, 3], seed=9, start_pos=[0, 4])
    q2, k2, v = oracle.prologue_qwen3(case.q, case.k, case.v, case.q_norm_w, case.k_norm_w,
                                      case.token_pos(), case.eps, case.theta)
    assert np.array_equal(v, oracle.bf16_bits_to_f64(case.v))
    # position 0 rows are plain RMSNorm * w
    t0 = 0
    qn = oracle.rmsnorm(oracle.bf16_bits_to_f64(case.q[t0]),
                        oracle.bf16_bits_to_f64(case.q_norm_w), case.eps)
    assert np.max(np.abs(q2[t0] - qn)) <= 1e-15
    # rotating by -pos undoes the rope; what is left has unit RMS / w
    inv = oracle.rope_inv_freq(32, case.theta)
    pos = case.token_pos()
    t = 6  # second sequence, position 5
    back = oracle.rope_apply(k2[t], -pos[t], inv)
    kn = oracle.rmsnorm(oracle.bf16_bits_to_f64(case.k[t]),
                        oracle.bf16_bits_to_f64(case.k_norm_w), case.eps)
    assert np.max(np.abs(back - kn)) <= 1e-12
