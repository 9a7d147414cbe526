"""Pins of the oracle's prologue (RMSNorm + half-split RoPE), CPU only.

The pages fix the structure (RMSNorm over head_dim, then
``x*cos + rotate_half(x)*sin``) and name the rope types ("default" for the
Qwen3 and Gemma-4 sliding layers, "proportional" with a partial rotary
factor for the Gemma-4 full layers), which they take from the transformers
rotary-embedding classes; they print no values.  Besides closed forms and
invariants, the oracle's frequencies, norms and rotation are pinned here
against that library's own implementation of those rope types (the
default / proportional initialisers, ``Qwen3RMSNorm``, ``Gemma4RMSNorm``,
the rotary-embedding modules and ``apply_rotary_pos_emb``): an independent
implementation, so a wrong exponent, count, sign or half-split fails.
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


# ------------------------------------------------------------ Gemma-4 ----

def test_partial_rotary_frequencies_and_passthrough():
    """Partial rotary: the leading fraction of the frequencies rotates, the
    rest (zero inv_freq) passes through; closed forms at D = 16."""
    D, theta = 16, 100.0
    inv = oracle.rope_inv_freq_partial(D, theta, 0.25)
    # floor(0.25 * 16 / 2) = 2 rotating frequencies: 1 and theta^(-2/16)
    assert inv[0] == 1.0 and abs(inv[1] - theta ** (-0.125)) <= 1e-15
    assert np.all(inv[2:] == 0.0)
    x = np.arange(1, D + 1, dtype=np.float64)
    pos = 3
    y = oracle.rope_apply(x, pos, inv)
    # dims 2..7 and 10..15 are untouched
    keep = np.r_[2:8, 10:16]
    assert np.array_equal(y[keep], x[keep])
    # pairs (0, 8) and (1, 9) are 2x2 rotations by pos * inv_i
    for i in range(2):
        a = pos * inv[i]
        lo, hi = x[i], x[i + 8]
        assert abs(y[i] - (lo * math.cos(a) - hi * math.sin(a))) <= 1e-12
        assert abs(y[i + 8] - (hi * math.cos(a) + lo * math.sin(a))) <= 1e-12
    # fraction 1 is the default table
    assert np.array_equal(oracle.rope_inv_freq_partial(D, theta, 1.0),
                          oracle.rope_inv_freq(D, theta))


def test_gemma4_v_norm_k_eq_v_and_qk_match_qwen3():
    from synth import make_prefill_case
    case = make_prefill_case(4, 2, 32, 8, [5, 3], seed=19, start_pos=[0, 4], theta=1e4)
    args = (case.q, case.k, case.v, case.q_norm_w, case.k_norm_w, case.token_pos(), case.eps,
            case.theta)
    q2, k2, v2 = oracle.prologue_gemma4(*args)
    qq, kq, _ = oracle.prologue_qwen3(*args)
    # with full rotary, q' and k' are the Qwen3 prologue's
    assert np.array_equal(q2, qq) and np.array_equal(k2, kq)
    # v_norm has no gain: v' = v / sqrt(mean(v^2) + eps), i.e. a positive
    # multiple of v per row whose mean square is ms / (ms + eps)
    v = oracle.bf16_bits_to_f64(case.v)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    assert np.max(np.abs(np.mean(v2 * v2, axis=-1, keepdims=True) - ms / (ms + case.eps))) <= 1e-12
    ratio = v2 / v
    assert np.all(ratio > 0)
    assert np.max(np.abs(ratio - ratio[..., :1])) <= 1e-12
    # K=V: the value is v_norm of the raw k (the v argument is ignored)
    _, k3, v3 = oracle.prologue_gemma4(*args, k_eq_v=True)
    junk = np.zeros_like(case.v)
    _, _, v4 = oracle.prologue_gemma4(case.q, case.k, junk, *args[3:], k_eq_v=True)
    kraw = oracle.bf16_bits_to_f64(case.k)
    assert np.array_equal(v3, v4)
    assert np.max(np.abs(v3 - kraw / np.sqrt(np.mean(kraw * kraw, axis=-1, keepdims=True)
                                             + case.eps))) <= 1e-15
    assert np.array_equal(k3, k2)


def test_gemma4_partial_rotary_keeps_tail_and_norm():
    from synth import make_prefill_case
    case = make_prefill_case(4, 2, 64, 8, [6], seed=23, start_pos=[9], theta=1e6)
    q2, k2, _ = oracle.prologue_gemma4(case.q, case.k, case.v, case.q_norm_w, case.k_norm_w,
                                       case.token_pos(), case.eps, case.theta,
                                       rotary_fraction=0.25)
    qn = oracle.rmsnorm(oracle.bf16_bits_to_f64(case.q), oracle.bf16_bits_to_f64(case.q_norm_w),
                        case.eps)
    # 8 of 32 frequencies rotate: dims 8..31 and 40..63 are the normed values
    tail = np.r_[8:32, 40:64]
    assert np.max(np.abs(q2[..., tail] - qn[..., tail])) <= 1e-15
    # a rotation keeps each row's norm
    assert np.max(np.abs(np.linalg.norm(q2, axis=-1) - np.linalg.norm(qn, axis=-1))) <= 1e-12


# ------------------------------------------- pins against transformers ----
# The library computes its tables in float32, so agreement is to float32
# rounding: frequencies to a few ulp, rotated values to ~1e-4 at positions
# up to ~1000 (the fp32 angle pos * inv_freq).  A wrong convention
# (exponent, rotating count, half order, sign) is off by O(1).

def _qwen3_config(head_dim, theta, rope_type="default", fraction=None):
    transformers = pytest.importorskip("transformers")
    rp = {"rope_type": rope_type, "rope_theta": theta}
    if fraction is not None:
        rp["partial_rotary_factor"] = fraction
    return transformers.Qwen3Config(head_dim=head_dim, hidden_size=8 * head_dim,
                                    num_attention_heads=8, num_key_value_heads=2,
                                    rope_parameters=rp)


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_default_rope_frequencies_match_transformers(D, theta):
    pytest.importorskip("transformers")
    from transformers.models.qwen3.modeling_qwen3 import Qwen3RotaryEmbedding
    inv, scaling = Qwen3RotaryEmbedding.compute_default_rope_parameters(_qwen3_config(D, theta))
    assert scaling == 1.0
    ref = inv.double().numpy()
    got = oracle.rope_inv_freq(D, theta)
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref) / ref) <= 4e-7


@pytest.mark.parametrize("D,fraction", [(512, 0.25), (64, 0.27), (64, 0.5), (128, 0.3),
                                        (256, 0.1), (96, 0.75), (512, 1.0)])
def test_proportional_rope_frequencies_match_transformers(D, fraction):
    """Rotating count floor(f * D / 2), default exponents over the full head_dim,
    zero tail: the library's proportional initialiser.  (0.27 at D 64 is a case
    where rounding would give 9 rotating frequencies and the library gives 8.)"""
    pytest.importorskip("transformers")
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    cfg = _qwen3_config(D, 1e6, "proportional", fraction)
    inv, _ = ROPE_INIT_FUNCTIONS["proportional"](cfg, None)
    ref = inv.double().numpy()
    got = oracle.rope_inv_freq_partial(D, 1e6, fraction)
    assert got.shape == ref.shape
    assert np.array_equal(got == 0.0, ref == 0.0), "rotating count differs"
    nz = ref > 0
    assert np.max(np.abs(got[nz] - ref[nz]) / ref[nz]) <= 4e-7


def test_gemma4_layer_rope_tables_match_transformers():
    """The Gemma-4 text config's own two rope types (sliding: default, theta 10K,
    head_dim 256; full: proportional 0.25, theta 1M, head_dim 512)."""
    pytest.importorskip("transformers")
    from transformers.models.gemma4 import configuration_gemma4, modeling_gemma4
    cfg = configuration_gemma4.Gemma4TextConfig()
    rot = modeling_gemma4.Gemma4TextRotaryEmbedding(cfg)
    for lt, D, theta, frac in (("sliding_attention", 256, 1e4, 1.0),
                               ("full_attention", 512, 1e6, 0.25)):
        assert cfg.per_layer_config[lt].head_dim == D
        ref = getattr(rot, f"{lt}_inv_freq").double().numpy()
        got = oracle.rope_inv_freq_partial(D, theta, frac)
        assert np.array_equal(got == 0.0, ref == 0.0)
        nz = ref > 0
        assert np.max(np.abs(got[nz] - ref[nz]) / ref[nz]) <= 4e-7


def _rows(D, seed, n=6, pos_hi=1024):
    rng = np.random.default_rng(seed)
    from synth import randn_bf16
    x = randn_bf16(rng, (n, 3, D))          # [tokens][heads][D] bf16 bits
    w = randn_bf16(rng, (D,), 1.0, 0.1)
    pos = rng.integers(0, pos_hi, size=n).astype(np.int64)
    pos[0] = 0
    return x, w, pos


def test_qwen3_prologue_matches_transformers():
    """q' = rope(RMSNorm(q) * w) via Qwen3RMSNorm, Qwen3RotaryEmbedding and
    apply_rotary_pos_emb (fp32 inputs, so the module's cast back to the input
    dtype rounds nothing) against oracle.prologue_qwen3."""
    torch = pytest.importorskip("torch")
    pytest.importorskip("transformers")
    from transformers.models.qwen3 import modeling_qwen3 as mq
    D, theta, eps = 128, 1e6, 1e-6
    x, w, pos = _rows(D, 31)
    q2, k2, _ = oracle.prologue_qwen3(x, x[:, :2], x[:, :2], w, w, pos, eps, theta)
    xf = torch.from_numpy(oracle.bf16_bits_to_f64(x)).float()      # [T][H][D]
    norm = mq.Qwen3RMSNorm(D, eps=eps)
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(oracle.bf16_bits_to_f64(w)).float())
        rot = mq.Qwen3RotaryEmbedding(_qwen3_config(D, theta))
        cos, sin = rot(xf, torch.from_numpy(pos)[None])             # [1][T][D]
        xn = norm(xf).double()
        ref, _ = mq.apply_rotary_pos_emb(xn[None].transpose(1, 2), xn[None].transpose(1, 2),
                                         cos.double(), sin.double(), unsqueeze_dim=1)
    ref = ref[0].transpose(0, 1).numpy()                           # [T][H][D]
    assert np.max(np.abs(q2 - ref)) <= 5e-4
    assert np.max(np.abs(k2 - ref[:, :2])) <= 5e-4
    # position 0 involves no angle: there the agreement is to fp32 norm rounding
    assert np.max(np.abs(q2[0] - ref[0])) <= 2e-6


@pytest.mark.parametrize("layer", ["sliding_attention", "full_attention"])
def test_gemma4_prologue_matches_transformers(layer):
    """Gemma-4 layers through the library's Gemma4RMSNorm (q_norm / k_norm with
    a gain, v_norm without), its per-layer-type rotary embedding and
    apply_rotary_pos_emb; full layers with K = V (value = v_norm of the raw
    k projection) and the partial rotary."""
    torch = pytest.importorskip("torch")
    pytest.importorskip("transformers")
    from transformers.models.gemma4 import configuration_gemma4, modeling_gemma4 as mg
    cfg = configuration_gemma4.Gemma4TextConfig()
    full = layer == "full_attention"
    D = cfg.per_layer_config[layer].head_dim
    theta, frac = (1e6, 0.25) if full else (1e4, 1.0)
    eps = 1e-6
    x, w, pos = _rows(D, 37 if full else 41)
    kraw = x[:, :2]
    vraw = x[:, 1:3]
    q2, k2, v2 = oracle.prologue_gemma4(x, kraw, vraw, w, w, pos, eps, theta,
                                        rotary_fraction=frac, k_eq_v=full)
    rot = mg.Gemma4TextRotaryEmbedding(cfg)
    xf = torch.from_numpy(oracle.bf16_bits_to_f64(x)).float()
    with torch.no_grad():
        norm = mg.Gemma4RMSNorm(D, eps=eps)
        norm.weight.copy_(torch.from_numpy(oracle.bf16_bits_to_f64(w)).float())
        vnorm = mg.Gemma4RMSNorm(D, eps=eps, with_scale=False)
        cos, sin = rot(xf, torch.from_numpy(pos)[None], layer)
        xn = norm(xf).double()[None]                                 # [1][T][H][D]
        # the attention forward's call: (batch, seq, heads, head_dim), unsqueeze at 2
        ref = mg.apply_rotary_pos_emb(xn, cos.double(), sin.double(), unsqueeze_dim=2)
        vsrc = xf[:, :2] if full else xf[:, 1:3]
        vref = vnorm(vsrc).double().numpy()
    ref = ref[0].numpy()
    assert np.max(np.abs(q2 - ref)) <= 5e-4
    assert np.max(np.abs(k2 - ref[:, :2])) <= 5e-4
    assert np.max(np.abs(v2 - vref)) <= 2e-6
