"""Pins of the oracle's paged-KV functions (CPU only, no GPU).

Each test checks the oracle against something other than itself: hand-derived
golden fixtures, closed forms, invariants, explicit-loop brute force, and
torch's float64 scaled_dot_product_attention as an independent library routine.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged
from synth import SENTINEL_BITS, make_decode_case, make_prefill_case, randn_bf16
from tests.conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- bf16 ----

def test_bf16_golden_patterns():
    vals = {"1.0": 1.0, "-2.0": -2.0, "0.5": 0.5, "0.0": 0.0, "1/3": 1.0 / 3.0,
            "1+2^-8": 1 + 2.0 ** -8, "1+3*2^-8": 1 + 3 * 2.0 ** -8,
            "1+2^-8+2^-20": 1 + 2.0 ** -8 + 2.0 ** -20, "65504.0": 65504.0}
    for c in _load("bf16.json")["cases"]:
        got = int(oracle.f64_to_bf16_bits(np.array([vals[c["value"]]]))[0])
        assert got == int(c["bits"], 16), c


def test_bf16_roundtrip_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f64(bits)
    fin = np.isfinite(x)
    back = oracle.f64_to_bf16_bits(x[fin])
    # -0.0 and +0.0 both survive with their sign
    assert np.array_equal(back, bits[fin])


def test_bf16_upcast_exact_against_fp32_view():
    # 0x3F80 -> 1.0, 0x4049 -> 3.140625, 0xC2F7 -> -123.5
    b = np.array([0x3F80, 0x4049, 0xC2F7], dtype=np.uint16)
    assert list(oracle.bf16_bits_to_f64(b)) == [1.0, 3.140625, -123.5]


# --------------------------------------------------------- addressing ----

def test_addressing_golden():
    g = _load("addressing.json")
    table = np.array(g["table"], dtype=np.int32)
    for c in g["cases"]:
        assert paged.physical_page(table, c["slot"], c["pos"], g["page_size"]) == c["page"]
        assert c["pos"] % g["page_size"] == c["row"]


def test_append_places_rows_at_golden_addresses_and_nowhere_else():
    g = _load("addressing.json")
    table = np.array(g["table"], dtype=np.int32)
    ps, n_kv, D = g["page_size"], 2, 8
    kp = np.full((8, n_kv, ps, D), SENTINEL_BITS, np.uint16)
    vp = np.full((8, n_kv, 1, D, ps), SENTINEL_BITS, np.uint16)   # page_size 4: one key group
    T = len(g["cases"])
    rng = np.random.default_rng(0)
    kn = rng.integers(0, 0x7F00, size=(T, n_kv, D)).astype(np.uint16)
    vn = rng.integers(0, 0x7F00, size=(T, n_kv, D)).astype(np.uint16)
    slot = np.array([c["slot"] for c in g["cases"]], np.int32)
    pos = np.array([c["pos"] for c in g["cases"]], np.int32)
    oracle.append(kp, vp, table, kn, vn, slot, pos)
    touched_k = np.zeros(kp.shape, bool)
    touched_v = np.zeros(vp.shape, bool)
    for t, c in enumerate(g["cases"]):
        P, r = c["page"], c["row"]
        for h in range(n_kv):
            for d in range(D):
                assert kp[P, h, r, d] == kn[t, h, d]
                assert vp[P, h, 0, d, r] == vn[t, h, d]     # d-major inside the group
                touched_k[P, h, r, d] = True
                touched_v[P, h, 0, d, r] = True
    assert np.all(kp[~touched_k] == SENTINEL_BITS)
    assert np.all(vp[~touched_v] == SENTINEL_BITS)


def test_append_v_key_groups_of_32():
    """V rows of a 64-key page land in two 32-key groups, each d-major.

    Flat offsets inside the (page, head) block, worked by hand from the
    layout: element (d, row) sits at ((row // 32) * D + d) * 32 + row % 32
    (D = 4): row 0 dim 0 -> 0, row 31 dim 3 -> 127, row 32 dim 0 -> 128,
    row 33 dim 2 -> 193, row 63 dim 1 -> 191.
    """
    ps, D = 64, 4
    table = np.array([[0], [2]], np.int32)
    kp = np.full((3, 1, ps, D), SENTINEL_BITS, np.uint16)
    vp = np.full((3, 1, 2, D, 32), SENTINEL_BITS, np.uint16)
    rows = np.array([0, 31, 32, 33, 63], np.int32)
    vn = (np.arange(5 * D, dtype=np.uint16) + 1).reshape(5, 1, D)
    oracle.append(kp, vp, table, vn, vn, np.ones(5, np.int32), rows)
    flat = vp[2, 0].reshape(-1)
    expect = {(0, 0): 0, (1, 3): 127, (2, 0): 128, (3, 2): 193, (4, 1): 191}
    for (t, d), off in expect.items():
        assert flat[off] == vn[t, 0, d]
    assert np.count_nonzero(flat != SENTINEL_BITS) == 5 * D
    assert np.all(vp[:2] == SENTINEL_BITS)
    # and the gather reads them back at their logical positions
    K, V = oracle.gather_kv(kp, vp, table, 1, 64)
    for t, r in enumerate(rows):
        assert np.array_equal(V[r, 0], oracle.bf16_bits_to_f64(vn[t, 0]))


def test_append_skips_slot_zero():
    table = np.zeros((2, 2), np.int32)
    table[1] = [1, 2]
    kp = np.full((3, 1, 4, 2), SENTINEL_BITS, np.uint16)
    vp = np.full((3, 1, 1, 2, 4), SENTINEL_BITS, np.uint16)
    kn = np.ones((2, 1, 2), np.uint16)
    oracle.append(kp, vp, table, kn, kn, np.array([0, 0], np.int32), np.array([0, 5], np.int32))
    assert np.all(kp == SENTINEL_BITS) and np.all(vp == SENTINEL_BITS)


def _history_pools(case):
    kp, vp = case.empty_pools()
    hk, hv, hs, hp = case.history_tokens()
    oracle.append(kp, vp, case.table, hk, hv, hs, hp)
    oracle.append(kp, vp, case.table, case.k_new, case.v_new, case.append_slots(),
                  case.append_pos())
    return kp, vp


def test_gather_returns_contiguous_history():
    case = make_decode_case(4, 2, 16, 4, [9, 1, 0, 14], max_slots=6, seed=5,
                            slot_of_row=[3, 1, 2, 5])
    kp, vp = _history_pools(case)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        if L == 0:
            continue
        K, V = oracle.gather_kv(kp, vp, case.table, int(case.slots[b]), L)
        dense_k = np.concatenate([case.hist_k[b], case.k_new[b:b + 1]])
        dense_v = np.concatenate([case.hist_v[b], case.v_new[b:b + 1]])
        assert np.array_equal(K, oracle.bf16_bits_to_f64(dense_k))
        assert np.array_equal(V, oracle.bf16_bits_to_f64(dense_v))


# ------------------------------------------------------------- masks ----

def test_mask_predicates_golden():
    g = _load("masks.json")
    q = np.arange(4)[:, None]
    k = np.arange(4)[None, :]
    assert np.array_equal(oracle.visible(q, k, 0).astype(int), g["causal_4"])
    q = np.arange(5)[:, None]
    k = np.arange(5)[None, :]
    assert np.array_equal(oracle.visible(q, k, 2).astype(int), g["sliding_5_w2"])
    assert np.array_equal(oracle.visible(5, np.arange(6), 3).astype(int),
                          g["decode_len6_w3_row"])


def _prefill_visibility(lengths, slots, window):
    """Visibility matrix recovered from the prefill oracle's outputs.

    K = 0 makes every visible key weigh the same; V[j] = e_j one-hot turns
    the output row into that weight vector, so ``out > 0`` is the mask.
    """
    D = 8
    case = make_prefill_case(1, 1, D, 4, lengths, seed=1, slots=slots, window=window)
    kp, vp = case.empty_pools()
    T = case.T
    k = np.zeros((T, 1, D), np.uint16)
    v = np.zeros((T, 1, D), np.uint16)
    tpos = case.token_pos()
    for t in range(T):
        v[t, 0, tpos[t]] = 0x3F80  # 1.0 at the key's own position
    oracle.append(kp, vp, case.table, k, v, case.token_slots(), tpos)
    out, _ = oracle.attn_prefill(case.q, kp, vp, case.table, case.cu_seqlens, case.slots,
                                 case.start_pos, 1.0, window)
    vis = np.zeros((T, T), int)
    for t in range(T):
        for u in range(T):
            if case.token_slots()[t] == case.token_slots()[u]:
                vis[t, u] = int(out[t, 0, tpos[u]] > 0)
    return vis


def test_prefill_document_causal_mask_golden():
    g = _load("masks.json")
    assert np.array_equal(_prefill_visibility([2, 3], [1, 2], 0), g["docs_1_1_2_2_2"])
    assert np.array_equal(_prefill_visibility([2, 3], [1, 2], 2), g["docs_1_1_2_2_2_w2"])


# -------------------------------------------------------- attention ----

def _brute_decode_row(q, K, V, pos, scale, window):
    """Explicit scalar loops with the math module; independent of numpy matmul."""
    n_q, D = q.shape
    n_kv = K.shape[1]
    G = n_q // n_kv
    out = [[0.0] * D for _ in range(n_q)]
    for h in range(n_q):
        hk = h // G
        scores = []
        for j in range(K.shape[0]):
            ok = j <= pos and (window == 0 or pos - j < window)
            if ok:
                s = 0.0
                for d in range(D):
                    s += float(q[h, d]) * float(K[j, hk, d])
                scores.append((j, s * scale))
        if not scores:
            continue
        m = max(s for _, s in scores)
        z = sum(math.exp(s - m) for _, s in scores)
        for d in range(D):
            acc = 0.0
            for j, s in scores:
                acc += math.exp(s - m) * float(V[j, hk, d])
            out[h][d] = acc / z
    return np.array(out)


@pytest.mark.parametrize("window", [0, 5])
def test_decode_brute_force_tiny(window):
    case = make_decode_case(4, 2, 8, 4, [7, 3, 0, 11], max_slots=5, seed=11,
                            window=window, scale=0.3)
    kp, vp = _history_pools(case)
    out, _ = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                case.scale, window)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        if L == 0:
            assert np.all(out[b] == 0)
            continue
        K = oracle.bf16_bits_to_f64(np.concatenate([case.hist_k[b], case.k_new[b:b + 1]]))
        V = oracle.bf16_bits_to_f64(np.concatenate([case.hist_v[b], case.v_new[b:b + 1]]))
        ref = _brute_decode_row(oracle.bf16_bits_to_f64(case.q[b]), K, V, L - 1, case.scale,
                                window)
        assert np.max(np.abs(out[b] - ref)) <= 1e-12


def test_decode_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    case = make_decode_case(8, 2, 32, 8, [40, 17, 64], max_slots=4, seed=3)
    kp, vp = _history_pools(case)
    out, lse = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                  case.scale, 0)
    G = case.n_q // case.n_kv
    for b in range(case.B):
        L = int(case.seq_lens[b])
        K = oracle.bf16_bits_to_f64(np.concatenate([case.hist_k[b], case.k_new[b:b + 1]]))
        V = oracle.bf16_bits_to_f64(np.concatenate([case.hist_v[b], case.v_new[b:b + 1]]))
        qt = torch.from_numpy(oracle.bf16_bits_to_f64(case.q[b]))[:, None, :]  # [H,1,D]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        mask = torch.ones(1, L, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=case.scale)
        assert np.max(np.abs(out[b] - ref[:, 0, :].numpy())) <= 1e-12
        # log-sum-exp of the scores, via scipy
        from scipy.special import logsumexp
        s = (qt @ kt.transpose(1, 2)).numpy()[:, 0, :] * case.scale
        assert np.max(np.abs(lse[b] - logsumexp(s, axis=-1))) <= 1e-12


def test_prefill_sliding_matches_torch_sdpa_with_explicit_mask():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    W = 6
    case = make_prefill_case(4, 2, 16, 4, [13, 5], seed=21, start_pos=[3, 0], window=W)
    kp, vp = case.empty_pools()
    pk, pv, psl, ppos = case.prefix_tokens()
    oracle.append(kp, vp, case.table, pk, pv, psl, ppos)
    oracle.append(kp, vp, case.table, case.k, case.v, case.token_slots(), case.token_pos())
    out, _ = oracle.attn_prefill(case.q, kp, vp, case.table, case.cu_seqlens, case.slots,
                                 case.start_pos, case.scale, W)
    for n in range(2):
        a, b = int(case.cu_seqlens[n]), int(case.cu_seqlens[n + 1])
        P = int(case.start_pos[n])
        K = oracle.bf16_bits_to_f64(np.concatenate([case.prefix_k[n], case.k[a:b]]))
        V = oracle.bf16_bits_to_f64(np.concatenate([case.prefix_v[n], case.v[a:b]]))
        qf = torch.from_numpy(oracle.bf16_bits_to_f64(case.q[a:b])).permute(1, 0, 2)
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(2, 0).contiguous()
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(2, 0).contiguous()
        qi = torch.arange(b - a)[:, None] + P
        kj = torch.arange(P + b - a)[None, :]
        mask = (kj <= qi) & (qi - kj < W)
        ref = F.scaled_dot_product_attention(qf, kt, vt, attn_mask=mask, scale=case.scale)
        assert np.max(np.abs(out[a:b] - ref.permute(1, 0, 2).numpy())) <= 1e-12


def test_page_permutation_invariance_bitwise():
    case = make_decode_case(4, 2, 16, 4, [23, 9, 30], max_slots=4, seed=8, spare_pages=3)
    kp, vp = _history_pools(case)
    out1, lse1 = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                    case.scale)
    rng = np.random.default_rng(99)
    relabel = np.concatenate([[0], 1 + rng.permutation(case.n_pages - 1)])
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[relabel] = kp
    vp2[relabel] = vp
    t2 = np.where(case.table > 0, relabel[np.maximum(case.table, 0)], case.table)
    out2, lse2 = oracle.attn_decode(case.q, kp2, vp2, t2, case.slots, case.seq_lens,
                                    case.scale)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_softmax_weights_sum_to_one():
    # V one-hot per key: the output row is the weight vector itself.
    L, D = 12, 16
    case = make_decode_case(2, 1, D, 4, [L], max_slots=2, seed=4)
    case.hist_v[0][:] = 0
    case.v_new[:] = 0
    for j in range(L - 1):
        case.hist_v[0][j, 0, j] = 0x3F80
    case.v_new[0, 0, L - 1] = 0x3F80
    kp, vp = _history_pools(case)
    for W in (0, 5):
        out, lse = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                      case.scale, W)
        w = out[0][:, :L]
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12)
        if W:
            assert np.all(w[:, : L - W] == 0)


def test_sliding_equals_full_over_window_slice():
    L, W = 29, 7
    case = make_decode_case(4, 2, 16, 8, [L], max_slots=2, seed=13, window=W)
    kp, vp = _history_pools(case)
    out_w, _ = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                  case.scale, W)
    K, V = oracle.gather_kv(kp, vp, case.table, 1, L)
    ref, _ = oracle.attend_rows(oracle.bf16_bits_to_f64(case.q[0]), K[L - W:], V[L - W:],
                                W - 1, case.scale, 0)
    assert np.max(np.abs(out_w[0] - ref)) <= 1e-12
    # window >= L equals full attention exactly
    out_big, _ = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                    case.scale, L)
    out_full, _ = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                     case.scale, 0)
    assert np.array_equal(out_big, out_full)


def test_closed_forms():
    # L = 1: the only key is the new one -> out = v_new exactly.
    case = make_decode_case(4, 2, 16, 4, [1, 1], max_slots=3, seed=2)
    kp, vp = _history_pools(case)
    out, lse = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                  case.scale)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], oracle.bf16_bits_to_f64(case.v_new[b, h // 2]))
    # q = 0: uniform weights -> mean of the visible V rows (window edges exact).
    L, W = 19, 6
    case = make_decode_case(2, 1, 8, 4, [L], max_slots=2, seed=6)
    case.q[:] = 0
    kp, vp = _history_pools(case)
    K, V = oracle.gather_kv(kp, vp, case.table, 1, L)
    for win, lo in ((0, 0), (W, L - W)):
        out, lse = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                      1.0, win)
        assert np.max(np.abs(out[0, 0] - V[lo:, 0].mean(axis=0))) <= 1e-12
        assert abs(lse[0, 0] - math.log(L - lo)) <= 1e-12
    # constant V -> that constant, whatever the scores.
    case = make_decode_case(2, 1, 8, 4, [15], max_slots=2, seed=7)
    case.hist_v[0][:] = 0x4040  # 3.0
    case.v_new[:] = 0x4040
    kp, vp = _history_pools(case)
    out, _ = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens, 0.7)
    assert np.max(np.abs(out - 3.0)) <= 1e-12


def test_idle_rows_zero_and_never_read():
    case = make_decode_case(4, 2, 16, 4, [0, 9, 0], max_slots=4, seed=12,
                            slot_of_row=[2, 1, 0])
    kp, vp = _history_pools(case)
    # page 0 and unowned pages hold NaN sentinels; nothing may read them.
    out, lse = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                  case.scale)
    assert np.all(np.isfinite(out))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(kp[0] == SENTINEL_BITS) and np.all(vp[0] == SENTINEL_BITS)


def test_gqa_equals_repeated_kv():
    case = make_decode_case(6, 2, 16, 4, [21], max_slots=2, seed=14)
    kp, vp = _history_pools(case)
    out, _ = oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                                case.scale)
    K, V = oracle.gather_kv(kp, vp, case.table, 1, 21)
    Kr, Vr = np.repeat(K, 3, axis=1), np.repeat(V, 3, axis=1)
    ref, _ = oracle.attend_rows(oracle.bf16_bits_to_f64(case.q[0]), Kr, Vr, 20, case.scale, 0)
    assert np.max(np.abs(out[0] - ref)) <= 1e-12


def test_prefill_equals_decode_at_each_position():
    # Query i of a prompt sees exactly what a decode step at length i+1 sees.
    case = make_prefill_case(4, 2, 16, 4, [11], seed=31)
    kp, vp = case.empty_pools()
    oracle.append(kp, vp, case.table, case.k, case.v, case.token_slots(), case.token_pos())
    out, lse = oracle.attn_prefill(case.q, kp, vp, case.table, case.cu_seqlens, case.slots,
                                   case.start_pos, case.scale, 0)
    for i in range(11):
        o, l = oracle.attn_decode(case.q[i:i + 1], kp, vp, case.table, case.slots,
                                  np.array([i + 1], np.int32), case.scale, 0)
        assert np.array_equal(o[0], out[i]) and np.array_equal(l[0], lse[i])


def test_prefill_sequences_are_isolated():
    case = make_prefill_case(2, 1, 8, 4, [6, 7], seed=41)
    kp, vp = case.empty_pools()
    oracle.append(kp, vp, case.table, case.k, case.v, case.token_slots(), case.token_pos())
    out1, _ = oracle.attn_prefill(case.q, kp, vp, case.table, case.cu_seqlens, case.slots,
                                  case.start_pos, case.scale)
    k2 = case.k.copy()
    k2[6:] = randn_bf16(np.random.default_rng(5), k2[6:].shape)  # perturb sequence 2 only
    kp2, vp2 = case.empty_pools()
    oracle.append(kp2, vp2, case.table, k2, case.v, case.token_slots(), case.token_pos())
    out2, _ = oracle.attn_prefill(case.q, kp2, vp2, case.table, case.cu_seqlens, case.slots,
                                  case.start_pos, case.scale)
    assert np.array_equal(out1[:6], out2[:6])
    assert not np.array_equal(out1[6:], out2[6:])
