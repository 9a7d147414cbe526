"""GPU prefill parity (with and without the fused prologue) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pagetable_amd as pkv
from synth import CONFIGS, config_lengths, make_prefill_case
from tests.gpu_util import (DEV, assert_attn_close, bf16_ulp_distance, dev_bits, dev_i32,
                            gpu_pools, host_bits, host_f64)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (n_q, n_kv, D, ps, lengths, start_pos, window)
    "tiny": (4, 2, 64, 16, [37, 50], None, 0),
    "tiny_w20": (4, 2, 64, 16, [37, 50], None, 20),
    "d128_g4_ragged": (32, 8, 128, 128, [1, 33, 130, 7, 257], None, 0),
    "d128_g4_prefix": (32, 8, 128, 128, [40, 100, 3], [5, 128, 300], 0),
    "d128_g3": (24, 8, 128, 64, [70, 1, 200], None, 0),
    "d256_w64": (8, 2, 256, 64, [300, 45], [0, 20], 64),
    # head_dim 512 (one LDS tile buffer, one wave per SIMD)
    "d512_ragged": (8, 2, 512, 64, [70, 1, 130], None, 0),
    "d512_prefix_w40_ps16": (16, 4, 512, 16, [50, 33], [20, 0], 40),
    "g1_ps16": (4, 4, 128, 16, [90, 31], None, 0),
    "g1_d64": (4, 4, 64, 32, [70, 33, 129], [0, 5, 0], 0),
    "g16": (16, 1, 64, 32, [40, 9], None, 0),
    "kv16_g2": (32, 16, 64, 32, [40, 90, 7], None, 0),
    "kv3_g4": (12, 3, 128, 64, [70, 130], [0, 9], 0),
    "slot0_pad": (8, 2, 64, 16, [20, 12, 30], None, 0),
    "ps256_prefix": (16, 4, 128, 256, [300, 520, 17], [0, 250, 0], 0),
    "d64_w100_prefix": (8, 2, 64, 64, [150, 64], [30, 0], 100),
    # empty prompts first, between and last (repeated cu_seqlens entries);
    # the empty ones with a cached prefix still own pages and read nothing
    "empty_prompts": (32, 8, 128, 64, [0, 70, 0, 0, 33, 0], [0, 0, 40, 0, 10, 64], 0),
}


def _pools_with_prefix(case):
    """Device + oracle pools holding each sequence's cached prefix."""
    kp, vp = gpu_pools(case)
    okp, ovp = case.empty_pools()
    table = dev_i32(case.table)
    pk, pv, ps_, pp = case.prefix_tokens()
    if len(ps_):
        pkv.append(dev_bits(pk), dev_bits(pv), dev_i32(ps_), dev_i32(pp), table, kp, vp)
        oracle.append(okp, ovp, case.table, pk, pv, ps_, pp)
    return kp, vp, table, okp, ovp


def _case(name, seed=0):
    n_q, n_kv, D, ps, lengths, sp, window = CASES[name]
    slots = None
    if name == "slot0_pad":
        slots = [1, 0, 2]   # a padding sequence in slot 0
    return make_prefill_case(n_q, n_kv, D, ps, lengths, seed=2000 + seed + D, start_pos=sp,
                             slots=slots, max_slots=4 if slots else None, window=window)


def _run_no_prologue(case, kp, vp, table, hint=None):
    q = dev_bits(case.q)
    lse = torch.empty((case.T, case.n_q), dtype=torch.float32, device=q.device)
    out = pkv.attn_prefill(q, dev_i32(case.cu_seqlens), dev_i32(case.slots), table, kp, vp,
                           scale=case.scale, window=case.window,
                           start_pos=dev_i32(case.start_pos),
                           max_seqlen_q_hint=hint or int(np.diff(case.cu_seqlens).max()),
                           lse=lse)
    torch.cuda.synchronize()
    return q, out, lse


def _check_no_prologue(case, q, out, lse, okp, ovp, name):
    ref, ref_lse = oracle.attn_prefill(case.q, okp, ovp, case.table, case.cu_seqlens,
                                       case.slots, case.start_pos, case.scale, case.window)
    assert_attn_close(host_f64(out), ref, name)
    g_lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(g_lse[~fin]))
    assert np.max(np.abs(g_lse[fin] - ref_lse[fin]), initial=0.0) <= 1e-3
    # q untouched without a prologue; padding rows exactly zero
    assert np.array_equal(host_bits(q), case.q)
    pad = case.token_slots() == 0
    assert np.all(host_bits(out)[pad] == 0)


def _append_tokens(case, kp, vp, table, okp, ovp):
    tsl, tpos = case.token_slots(), case.token_pos()
    pkv.append(dev_bits(case.k), dev_bits(case.v), dev_i32(tsl), dev_i32(tpos), table, kp, vp)
    oracle.append(okp, ovp, case.table, case.k, case.v, tsl, tpos)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_no_prologue_matches_oracle(name):
    case = _case(name)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _append_tokens(case, kp, vp, table, okp, ovp)
    q, out, lse = _run_no_prologue(case, kp, vp, table)
    _check_no_prologue(case, q, out, lse, okp, ovp, name)


def test_prefill_many_sequences_hint_below_longest():
    """531 prompts, a max_seqlen_q_hint below the longest (grid-stride path)."""
    rng = np.random.default_rng(21)
    lengths = [int(x) for x in rng.integers(1, 12, size=530)] + [70]
    case = make_prefill_case(8, 2, 64, 16, lengths, seed=2100, max_slots=len(lengths) + 1)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _append_tokens(case, kp, vp, table, okp, ovp)
    q, out, lse = _run_no_prologue(case, kp, vp, table, hint=8)
    _check_no_prologue(case, q, out, lse, okp, ovp, "530 prompts")


def test_prefill_long_prompt_sampled():
    """A 4200-token prompt beside a short one (525 query blocks), sampled rows."""
    # n_q 16 over 1 kv head: 8 query tokens per item, so 4200 tokens = 525 blocks
    lengths = [4200, 33]
    case = make_prefill_case(16, 1, 64, 64, lengths, seed=2200)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _append_tokens(case, kp, vp, table, okp, ovp)
    q, out, lse = _run_no_prologue(case, kp, vp, table)
    g = host_f64(out)
    gl = lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, 4199, 4200, 4232], rng.choice(case.T, size=8, replace=False)])
    for t in rows:
        n = int(np.searchsorted(case.cu_seqlens, t, side="right") - 1)
        p = t - int(case.cu_seqlens[n])
        K, V = oracle.gather_kv(okp, ovp, case.table, int(case.slots[n]), p + 1)
        ref, ref_lse = oracle.attend_rows(oracle.bf16_bits_to_f64(case.q[t]), K, V, p, case.scale, 0)
        assert_attn_close(g[t], ref, f"token {t}")
        assert np.max(np.abs(gl[t] - ref_lse)) <= 1e-3


def _run_with_prologue(case, kp, vp, table, hint=None, q_out=None):
    D = case.head_dim
    max_pos = int((case.start_pos + np.diff(case.cu_seqlens)).max()) + 1
    cos, sin = pkv.rope_table(max_pos, D, case.theta)
    q = dev_bits(case.q)
    pro = dict(q_norm_w=dev_bits(case.q_norm_w), k_norm_w=dev_bits(case.k_norm_w),
               eps=case.eps, cos=cos, sin=sin, k=dev_bits(case.k), v=dev_bits(case.v),
               q_out=q_out)
    out = pkv.attn_prefill(q, dev_i32(case.cu_seqlens), dev_i32(case.slots), table, kp, vp,
                           scale=case.scale, window=case.window,
                           start_pos=dev_i32(case.start_pos),
                           max_seqlen_q_hint=hint or int(np.diff(case.cu_seqlens).max()),
                           prologue=pro)
    torch.cuda.synchronize()
    return q, out


def _oracle_with_prologue(case, okp, ovp):
    tsl, tpos = case.token_slots(), case.token_pos()
    q2, k2, v = oracle.prologue_qwen3(case.q, case.k, case.v, case.q_norm_w, case.k_norm_w,
                                      tpos, case.eps, case.theta)
    q2b, k2b = oracle.f64_to_bf16_bits(q2), oracle.f64_to_bf16_bits(k2)
    oracle.append(okp, ovp, case.table, k2b, case.v, tsl, tpos)
    return q2, q2b, k2


def _check_with_prologue(case, kp, vp, table, okp, ovp, name, hint=None):
    # q' also copied out (q_out), over a sentinel fill
    q_out = torch.full(case.q.shape, -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    q, out = _run_with_prologue(case, kp, vp, table, hint=hint, q_out=q_out)
    q2, q2b, k2 = _oracle_with_prologue(case, okp, ovp)
    # q is normalised and rotated inside the attention kernel, never written
    assert np.array_equal(host_bits(q), case.q), "q was modified"
    # q': within tolerance of the fp64 value and (almost always) its nearest
    # bf16; rows of padding sequences untouched
    live = case.token_slots() != 0
    gq = host_bits(q_out)
    assert_attn_close(oracle.bf16_bits_to_f64(gq[live]), q2[live], "q'")
    ulp_ok = np.mean(gq[live] == q2b[live])
    assert ulp_ok >= 0.99, f"only {ulp_ok:.4f} of q' match the RNE-rounded fp64 value"
    near = np.mean(bf16_ulp_distance(gq[live], q2b[live]) <= 1)
    assert near >= 0.999, f"only {near:.5f} of q' within 1 bf16 ulp of the RNE-rounded fp64 value"
    assert np.all(gq[~live] == 0xFFFF), "q' written for a padding sequence"
    # the K pool holds k' (within tolerance of the fp64 value, and almost
    # always its nearest bf16), the V pool the raw v bit for bit
    gk = host_bits(kp)
    okb = okp
    written = okb != 0xFFFF
    assert np.array_equal(gk == 0xFFFF, ~written), "K rows written at the wrong places"
    kd = oracle.bf16_bits_to_f64(gk[written]) - oracle.bf16_bits_to_f64(okb[written])
    assert np.max(np.abs(kd)) <= 2e-2
    ulp_ok = np.mean(gk[written] == okb[written])
    assert ulp_ok >= 0.99, f"only {ulp_ok:.4f} of k' match the RNE-rounded fp64 value"
    near = np.mean(bf16_ulp_distance(gk[written], okb[written]) <= 1)
    assert near >= 0.999, f"only {near:.5f} of k' within 1 bf16 ulp of the RNE-rounded fp64 value"
    assert np.array_equal(host_bits(vp), ovp)
    ref, _ = oracle.attn_prefill(q2b, okp, ovp, case.table, case.cu_seqlens, case.slots,
                                 case.start_pos, case.scale, case.window)
    assert_attn_close(host_f64(out), ref, name)


# The prologue's rotary rows come from registers (one query head per kv head:
# g1_ps16, g1_d64), from LDS staging (two or more at head_dim <= 128: 2, 3, 4 and 16
# query heads per kv head, 64 down to 8 tokens per item) or from loads inside
# the transform (head_dim 256 / 512).
@pytest.mark.parametrize("name", ["tiny", "d128_g4_ragged", "d128_g4_prefix", "d256_w64",
                                  "d512_ragged", "g1_ps16", "g1_d64", "d128_g3", "g16", "kv16_g2",
                                  "d64_w100_prefix", "slot0_pad", "empty_prompts"])
def test_prefill_with_prologue_matches_oracle(name):
    case = _case(name, seed=7)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _check_with_prologue(case, kp, vp, table, okp, ovp, name)


@pytest.mark.parametrize("name", ["d128_g4_prefix", "d256_w64", "empty_prompts"])
def test_prefill_q_only_prologue_equals_full_prologue(name):
    """A prologue without k / v (keys already in the pages) normalises and
    rotates q only: on the pages a full-prologue call left behind, its output
    equals that call's bit for bit, and the pools are not written again."""
    case = _case(name, seed=9)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    q, out_full = _run_with_prologue(case, kp, vp, table)
    kp_after, vp_after = kp.clone(), vp.clone()
    max_pos = int((case.start_pos + np.diff(case.cu_seqlens)).max()) + 1
    cos, sin = pkv.rope_table(max_pos, case.head_dim, case.theta)
    pro = dict(q_norm_w=dev_bits(case.q_norm_w), eps=case.eps, cos=cos, sin=sin)
    out_q = pkv.attn_prefill(q, dev_i32(case.cu_seqlens), dev_i32(case.slots), table, kp, vp,
                             scale=case.scale, window=case.window,
                             start_pos=dev_i32(case.start_pos),
                             max_seqlen_q_hint=int(np.diff(case.cu_seqlens).max()), prologue=pro)
    torch.cuda.synchronize()
    assert torch.equal(out_q.view(torch.int16), out_full.view(torch.int16))
    assert torch.equal(kp.view(torch.int16), kp_after.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), vp_after.view(torch.int16))


def test_prefill_with_prologue_many_sequences():
    """601 prompts with cached prefixes: the prologue's sequence metadata is
    too long to stage and is searched in global memory."""
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 12, size=600)] + [70]
    sp = [int(x) for x in rng.integers(0, 20, size=601)]
    case = make_prefill_case(8, 2, 64, 16, lengths, seed=2300, start_pos=sp,
                             max_slots=len(lengths) + 1)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _check_with_prologue(case, kp, vp, table, okp, ovp, "601 prompts", hint=8)


def test_prefill_with_prologue_staged_metadata_boundary():
    """511 prompts (the largest count whose metadata the prologue stages)."""
    rng = np.random.default_rng(32)
    lengths = [int(x) for x in rng.integers(1, 9, size=511)]
    sp = [int(x) for x in rng.integers(0, 9, size=511)]
    case = make_prefill_case(8, 2, 64, 16, lengths, seed=2400, start_pos=sp,
                             max_slots=len(lengths) + 1)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _check_with_prologue(case, kp, vp, table, okp, ovp, "511 prompts")


# Mixed prefill + decode in one launch: decode rows are 1-token sequences
# whose start_pos is their cached length (the new token's position), beside
# prompts with and without a cached prefix.
MIXED_LENGTHS = [40, 1, 100, 1, 1, 7, 1, 1]
MIXED_START = [0, 63, 30, 200, 511, 0, 0, 1000]


def test_mixed_prefill_and_decode_rows_in_one_launch():
    case = make_prefill_case(8, 2, 128, 64, MIXED_LENGTHS, seed=2500, start_pos=MIXED_START)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _append_tokens(case, kp, vp, table, okp, ovp)
    q, out, lse = _run_no_prologue(case, kp, vp, table)
    _check_no_prologue(case, q, out, lse, okp, ovp, "mixed")
    # the 1-token rows are exactly decode steps: same result as the decode oracle
    dec = [n for n, L in enumerate(MIXED_LENGTHS) if L == 1]
    tok = case.cu_seqlens[dec]
    ref_d, _ = oracle.attn_decode(case.q[tok], okp, ovp, case.table, case.slots[dec],
                                  case.start_pos[dec] + 1, case.scale)
    assert_attn_close(host_f64(out)[tok], ref_d, "decode rows")


def test_mixed_prefill_and_decode_rows_with_prologue():
    case = make_prefill_case(8, 2, 128, 64, MIXED_LENGTHS, seed=2501, start_pos=MIXED_START)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _check_with_prologue(case, kp, vp, table, okp, ovp, "mixed with prologue")


@pytest.mark.parametrize("D,fraction,n_rot", [(512, 0.25, 64), (64, 0.27, 8), (128, 0.3, 19),
                                              (256, 0.1, 12)])
def test_rope_table_partial_matches_fp64(D, fraction, n_rot):
    """floor(f * D / 2) rotating frequencies (0.27 at D 64: 8, where rounding
    would give 9), the rest cos 1 / sin 0."""
    theta, max_pos = 1e6, 1024
    c, s = pkv.rope_table(max_pos, D, theta, rotary_fraction=fraction)
    torch.cuda.synchronize()
    inv = oracle.rope_inv_freq_partial(D, theta, fraction)
    assert int((inv > 0).sum()) == n_rot
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    assert np.max(np.abs(c.cpu().numpy() - np.cos(ang))) <= 1e-7
    assert np.max(np.abs(s.cpu().numpy() - np.sin(ang))) <= 1e-7
    assert np.all(c.cpu().numpy()[:, n_rot:] == 1.0) and np.all(s.cpu().numpy()[:, n_rot:] == 0.0)


# Gemma-4 prologue variants: sliding layers (head_dim 256, theta 1e4, window
# 64 here), full-attention layers (head_dim 512, theta 1e6, 25 % rotary, K=V),
# v_norm (RMSNorm without a gain) on v, K=V, and partial rotary.
@pytest.mark.parametrize("D,k_eq_v,fraction", [(256, False, 1.0), (256, True, 1.0),
                                               (256, True, 0.25), (512, True, 0.25),
                                               (512, False, 1.0)])
def test_prefill_with_gemma4_prologue(D, k_eq_v, fraction):
    full = D == 512
    case = make_prefill_case(8, 2, D, 64, [70, 33, 5], seed=2600 + int(k_eq_v) + D,
                             start_pos=[0, 40, 0], theta=1e6 if full else 1e4,
                             window=0 if full else 64)
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    D = case.head_dim
    max_pos = int((case.start_pos + np.diff(case.cu_seqlens)).max()) + 1
    cos, sin = pkv.rope_table(max_pos, D, case.theta, rotary_fraction=fraction)
    q_out = torch.full(case.q.shape, -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    v_in = case.k if k_eq_v else case.v
    pro = dict(q_norm_w=dev_bits(case.q_norm_w), k_norm_w=dev_bits(case.k_norm_w),
               eps=case.eps, cos=cos, sin=sin, k=dev_bits(case.k), v=dev_bits(v_in),
               q_out=q_out, v_norm=True)
    q = dev_bits(case.q)
    out = pkv.attn_prefill(q, dev_i32(case.cu_seqlens), dev_i32(case.slots), table, kp, vp,
                           scale=case.scale, window=case.window,
                           start_pos=dev_i32(case.start_pos), max_seqlen_q_hint=70, prologue=pro)
    torch.cuda.synchronize()
    tsl, tpos = case.token_slots(), case.token_pos()
    q2, k2, v2 = oracle.prologue_gemma4(case.q, case.k, case.v, case.q_norm_w, case.k_norm_w,
                                        tpos, case.eps, case.theta, rotary_fraction=fraction,
                                        k_eq_v=k_eq_v)
    q2b, k2b, v2b = (oracle.f64_to_bf16_bits(x) for x in (q2, k2, v2))
    oracle.append(okp, ovp, case.table, k2b, v2b, tsl, tpos)
    # q', k', v' within tolerance of the fp64 values and almost always their nearest bf16
    gq = host_bits(q_out)
    assert_attn_close(oracle.bf16_bits_to_f64(gq), q2, "q'")
    assert np.mean(gq == q2b) >= 0.99
    for name, g, o in (("k'", host_bits(kp), okp), ("v'", host_bits(vp), ovp)):
        written = o != 0xFFFF
        assert np.array_equal(g == 0xFFFF, ~written), f"{name} rows written at the wrong places"
        d = oracle.bf16_bits_to_f64(g[written]) - oracle.bf16_bits_to_f64(o[written])
        assert np.max(np.abs(d)) <= 2e-2, name
        assert np.mean(g[written] == o[written]) >= 0.99, name
    ref, _ = oracle.attn_prefill(q2b, okp, ovp, case.table, case.cu_seqlens, case.slots,
                                 case.start_pos, case.scale, case.window)
    assert_attn_close(host_f64(out), ref, f"gemma4 k_eq_v={k_eq_v} fraction={fraction}")


def test_rope_table_matches_fp64():
    D, theta, max_pos = 128, 1e6, 4096
    c, s = pkv.rope_table(max_pos, D, theta)
    torch.cuda.synchronize()
    inv = oracle.rope_inv_freq(D, theta)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    assert np.max(np.abs(c.cpu().numpy() - np.cos(ang))) <= 1e-7
    assert np.max(np.abs(s.cpu().numpy() - np.sin(ang))) <= 1e-7


def _full_prefill_case():
    c = CONFIGS["qwen3_prefill"]
    L, slots = config_lengths("qwen3_prefill")
    case = make_prefill_case(c["n_q"], c["n_kv"], c["head_dim"], c["page_size"], L,
                             seed=3407 + c["index"], slots=slots, max_slots=c["max_slots"],
                             eps=c["eps"], theta=c["theta"], spare_pages=4,
                             pages_per_slot=-(-c["len_hi"] // c["page_size"]))
    return case, c["len_hi"]


def test_full_qwen3_prefill_all_tokens():
    """The 16-prompt workload in the bench's launch configuration (fused
    prologue, the bench's grid hint): every token's output, q' and the K/V
    pools against the oracle."""
    case, hint = _full_prefill_case()
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _check_with_prologue(case, kp, vp, table, okp, ovp, "qwen3_prefill", hint=hint)


def test_full_qwen3_prefill_no_prologue_all_tokens():
    """The same workload's attention alone (the instance the roofline times):
    K/V appended first, every token's output and lse against the oracle."""
    case, hint = _full_prefill_case()
    kp, vp, table, okp, ovp = _pools_with_prefix(case)
    _append_tokens(case, kp, vp, table, okp, ovp)
    q, out, lse = _run_no_prologue(case, kp, vp, table, hint=hint)
    _check_no_prologue(case, q, out, lse, okp, ovp, "qwen3_prefill attention")
