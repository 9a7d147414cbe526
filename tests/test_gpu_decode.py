"""GPU decode parity against the fp64 oracle, plus exact GPU-side invariants."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pagetable_amd as pkv
from synth import CONFIGS, config_lengths, make_decode_case
from tests.gpu_util import (DEV, assert_attn_close, dev_bits, dev_i32, gpu_decode_setup,
                            host_bits, host_f64, oracle_decode_pools, run_gpu_decode)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (n_q, n_kv, D, ps, lengths, window, scale)
    "tiny": (4, 2, 64, 16, [37, 50], 0, 1 / 8),
    "tiny_w20": (4, 2, 64, 16, [37, 50], 20, 1 / 8),
    "d128_g4_edges": (32, 8, 128, 128, [1, 127, 128, 129, 0, 700, 1024, 31], 0, None),
    "d128_g3_ps64": (24, 8, 128, 64, [3000, 5, 0, 1, 2049, 640], 0, None),
    "d128_ps16": (8, 2, 128, 16, [300, 17, 16, 1000], 0, None),
    "d256_w512": (8, 2, 256, 64, [256, 511, 512, 513, 1536, 900], 512, None),
    # head_dim 256 at the largest group (G * head_dim = 2048) on 16-token
    # pages: per-key page lookups in the K copies, the new V row stored apart
    "d256_g8_ps16": (16, 2, 256, 16, [300, 17, 16, 1000, 0, 65], 0, None),
    "d512_full": (8, 2, 512, 64, [256, 1536, 777], 0, None),
    # G * head_dim = 1536: the merge's 768 dim pairs take 4 per thread (a
    # power of two, so a thread's pairs stay inside one query head)
    "d512_g3": (6, 2, 512, 64, [700, 1536, 33, 1100], 0, None),
    "g1": (8, 8, 128, 128, [500, 1], 0, None),
    "g16": (16, 1, 64, 32, [200, 33], 0, None),
    "w1": (4, 2, 64, 16, [37, 50], 1, None),
    "d128_ps256": (16, 4, 128, 256, [700, 255, 256, 257, 1, 0, 2000], 0, None),
    "all_idle": (32, 8, 128, 128, [0, 0, 0], 0, None),
    # one long row of many splits beside short one-split rows, with idle rows
    # among them
    "long_among_short": (32, 8, 128, 64, [4000] + [3, 40, 0, 65, 1, 33, 0] * 4, 0, None),
    # many short rows (80 rows, one split each)
    "many_short": (8, 2, 64, 16, [int(x) for x in np.arange(1, 81) * 7 % 97], 0, None),
    # 64 rows x 8 kv heads up to 2100 keys: a grid of 2560 512-key splits,
    # which gets the 128-key split 0; lengths on and around the split edges
    # (128, 640, 1152, 1664) among seeded ones, idle rows included
    "head_split": (16, 8, 64, 64, [0, 1, 127, 128, 129, 639, 640, 641, 1151, 1152, 1153, 1663,
                                   1664, 1665, 2100, 0]
                   + [int(x) for x in np.arange(1, 49) * 1237 % 2099 + 1], 0, None),
    # the same grid on 16-token pages: the large-grid kernel instance, whose
    # split 0 writes the new V only for pages of 32 keys or more, so here the
    # owner still writes it
    "head_split_ps16": (16, 8, 64, 16, [0, 1, 15, 16, 17, 127, 128, 129, 639, 640, 641, 2100]
                        + [int(x) for x in np.arange(1, 53) * 1237 % 2099 + 1], 0, None),
}


def _run(name, seed=0):
    n_q, n_kv, D, ps, lengths, window, scale = CASES[name]
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=len(lengths) + 2,
                            seed=1000 + seed + D, window=window, scale=scale, spare_pages=2)
    kp, vp, table = gpu_decode_setup(case)
    out, lse = run_gpu_decode(case, kp, vp, table)
    return case, kp, vp, table, out, lse


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    case, kp, vp, table, out, lse = _run(name)
    okp, ovp = oracle_decode_pools(case)
    ref, ref_lse = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                      case.scale, case.window)
    assert_attn_close(host_f64(out), ref, name)
    g_lse = lse.cpu().numpy().astype(np.float64)
    idle = case.seq_lens == 0
    assert np.all(np.isneginf(g_lse[idle]))
    assert np.max(np.abs(g_lse[~idle] - ref_lse[~idle]), initial=0.0) <= 1e-3
    # idle rows are exactly zero
    assert np.all(host_bits(out)[idle] == 0)


# A length hint far above the real lengths makes the splits long (several
# 32-key chunks per wave of 4-wave workgroups); the default hint of these
# small cases gives 128-key splits (one chunk per wave).  With 100000 the
# splits are 256 to 2048 keys, so the longer rows still have several splits
# to merge.
LONG_SPLIT_HINT = 1_000_000


@pytest.mark.parametrize("hint", [100_000, LONG_SPLIT_HINT])
@pytest.mark.parametrize("name", [n for n in CASES if CASES[n][2] <= 256])
def test_decode_long_splits_match_oracle(name, hint):
    n_q, n_kv, D, ps, lengths, window, scale = CASES[name]
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=len(lengths) + 2,
                            seed=1200 + D, window=window, scale=scale, spare_pages=2)
    kp, vp, table = gpu_decode_setup(case)
    out, lse = run_gpu_decode(case, kp, vp, table, hint=hint)
    okp, ovp = oracle_decode_pools(case)
    ref, ref_lse = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                      case.scale, case.window)
    assert_attn_close(host_f64(out), ref, f"{name} long splits")
    idle = case.seq_lens == 0
    g_lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isneginf(g_lse[idle]))
    assert np.max(np.abs(g_lse[~idle] - ref_lse[~idle]), initial=0.0) <= 1e-3
    assert np.all(host_bits(out)[idle] == 0)
    # the fused append on the same path: pools bit-exact, output unchanged
    kp2, vp2, table2 = gpu_decode_setup(case, with_new_token=False)
    out2, lse2 = run_gpu_decode(case, kp2, vp2, table2, hint=hint, fused_append=True)
    assert np.array_equal(host_bits(kp2), okp) and np.array_equal(host_bits(vp2), ovp)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)) and torch.equal(lse2, lse)


@pytest.mark.parametrize("name", ["tiny", "d128_g4_edges", "d128_ps16", "d256_w512",
                                  "d256_g8_ps16", "d512_full", "head_split", "head_split_ps16"])
def test_decode_fused_append_equals_append_then_decode(name):
    n_q, n_kv, D, ps, lengths, window, scale = CASES[name]
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=len(lengths) + 2,
                            seed=1500 + D, window=window, scale=scale, spare_pages=2)
    kp, vp, table = gpu_decode_setup(case)
    ref_out, ref_lse = run_gpu_decode(case, kp, vp, table)
    kp2, vp2, table2 = gpu_decode_setup(case, with_new_token=False)
    out, lse = run_gpu_decode(case, kp2, vp2, table2, fused_append=True)
    okp, ovp = oracle_decode_pools(case)
    assert np.array_equal(host_bits(kp2), okp), "fused append: K pool differs from the oracle"
    assert np.array_equal(host_bits(vp2), ovp), "fused append: V pool differs from the oracle"
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)


def test_decode_workspace_reused_across_calls_and_shapes():
    """One workspace serves successive calls of different sizes: the partials
    region may hold anything (it is never read before written), only the
    arrival counters at its end start at zero, and each call leaves them so."""
    ws = pkv.new_decode_workspace(pkv.decode_workspace_size(64, 32, 8, 128, 4096), "cuda")
    ws.fill_(0x7F)  # garbage in the partials
    ws[-4 * 64 * 8:].zero_()  # the counters of up to 64 rows x 8 kv heads
    for seed, lengths in ((1, [4000, 17, 0, 2500, 999]), (2, [129, 3000]), (3, [4096] * 6)):
        case = make_decode_case(32, 8, 128, 128, lengths, max_slots=len(lengths) + 1,
                                seed=seed, spare_pages=1)
        kp, vp, table = gpu_decode_setup(case)
        out, _ = run_gpu_decode(case, kp, vp, table, hint=4096, workspace=ws)
        okp, ovp = oracle_decode_pools(case)
        ref, _ = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                    case.scale, 0)
        assert_attn_close(host_f64(out), ref, f"reuse {seed}")


def test_decode_two_shapes_share_one_workspace():
    """Calls of two shapes alternate on one workspace sized for both: one with
    few (row, kv head) pairs whose long rows fill the partials up to the top
    of its plan (4 rows, G 16, rows of 64k keys in 64 splits), one with many
    pairs and their counters (64 rows x 8 kv heads, two splits per row).  The
    first call's partials must not reach the counters the second relies on
    being zero: every call matches the oracle and leaves the counters at 0."""
    big = make_decode_case(16, 1, 128, 128, [65536, 100, 65535, 65536], max_slots=6, seed=2101,
                           spare_pages=2)
    rng = np.random.default_rng(2102)
    many = make_decode_case(32, 8, 64, 16, [int(x) for x in rng.integers(600, 1025, size=64)],
                            max_slots=66, seed=2103, spare_pages=2)
    hints = {id(big): 65536, id(many): 1024}
    need = [pkv.decode_workspace_size(c.B, c.n_q, c.n_kv, c.head_dim, hints[id(c)])
            for c in (big, many)]
    assert min(need) > 0 and need[0] > need[1]
    ws = pkv.new_decode_workspace(max(need), DEV)
    runs = []
    for c in (big, many):
        kp, vp, table = gpu_decode_setup(c)
        okp, ovp = oracle_decode_pools(c)
        ref, _ = oracle.attn_decode(c.q, okp, ovp, c.table, c.slots, c.seq_lens, c.scale, 0)
        runs.append((c, kp, vp, table, ref))
    region = (ws.numel() // 16) // 16 * 16          # the counters' bytes at the end
    for it in range(2):
        for c, kp, vp, table, ref in runs:
            out, _ = run_gpu_decode(c, kp, vp, table, hint=hints[id(c)], workspace=ws)
            assert_attn_close(host_f64(out), ref, f"shape B={c.B} call {it}")
            assert int(ws[-region:].count_nonzero()) == 0


def test_decode_fused_append_past_capacity_is_skipped():
    """A row whose length exceeds its slot's table (a caller error): the fused
    append must skip its new token, as pkv_append does, and leave the cached
    rows intact; the other rows are unaffected."""
    case = make_decode_case(8, 2, 128, 64, [128, 70, 100], max_slots=5, seed=41, spare_pages=2,
                            pages_per_slot=2)
    assert int(case.seq_lens[0]) == 128  # row 0 fills its 2 pages of 64 exactly
    kp, vp, table = gpu_decode_setup(case, with_new_token=False)
    lens = case.seq_lens.copy()
    lens[0] = 129                          # one past the table: its token has no page
    out = pkv.attn_decode(dev_bits(case.q), dev_i32(case.slots), dev_i32(lens), table, kp, vp,
                          scale=case.scale, max_seq_len_hint=4096, k_new=dev_bits(case.k_new),
                          v_new=dev_bits(case.v_new))
    torch.cuda.synchronize()
    okp, ovp = case.empty_pools()
    hk, hv, hs, hp = case.history_tokens()
    oracle.append(okp, ovp, case.table, hk, hv, hs, hp)
    # rows 1 and 2 append at L-1; row 0's token (position 128) has no page
    cap = 2 * 64
    keep = [b for b in range(case.B) if 0 < lens[b] <= cap]
    assert keep == [1, 2]
    oracle.append(okp, ovp, case.table, case.k_new[keep], case.v_new[keep], case.slots[keep],
                  lens[keep] - 1)
    assert np.array_equal(host_bits(kp), okp), "K pool: a token past the table was written"
    assert np.array_equal(host_bits(vp), ovp), "V pool: a token past the table was written"
    ref, _ = oracle.attn_decode(case.q[1:], okp, ovp, case.table, case.slots[1:], lens[1:],
                                case.scale, 0)
    assert_attn_close(host_f64(out)[1:], ref, "in-table rows")


def test_decode_two_streams_with_separate_workspaces():
    """Two decode calls on two streams at once, each with its own workspace
    (and so its own arrival counters), repeatedly: both match the oracle."""
    cases = []
    for seed, lengths in ((61, [3000, 17, 2049, 0, 900, 4000]), (62, [129, 2500, 1, 3333])):
        case = make_decode_case(32, 8, 128, 128, lengths, max_slots=len(lengths) + 1, seed=seed,
                                spare_pages=1)
        kp, vp, table = gpu_decode_setup(case)
        okp, ovp = oracle_decode_pools(case)
        ref, _ = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                    case.scale, 0)
        ws = pkv.new_decode_workspace(pkv.decode_workspace_size(case.B, 32, 8, 128, 4096), DEV)
        cases.append(dict(case=case, kp=kp, vp=vp, table=table, ref=ref, ws=ws,
                          q=dev_bits(case.q), slots=dev_i32(case.slots),
                          lens=dev_i32(case.seq_lens), stream=torch.cuda.Stream(),
                          outs=[torch.empty((case.B, 32, 128), dtype=torch.bfloat16, device=DEV)
                                for _ in range(8)]))
    torch.cuda.synchronize()
    for it in range(8):
        for c in cases:
            with torch.cuda.stream(c["stream"]):
                pkv.attn_decode(c["q"], c["slots"], c["lens"], c["table"], c["kp"], c["vp"],
                                scale=c["case"].scale, max_seq_len_hint=4096, out=c["outs"][it],
                                workspace=c["ws"], stream=c["stream"])
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        for it in range(8):
            assert_attn_close(host_f64(c["outs"][it]), c["ref"], f"stream {i} call {it}")
        # the counters are back at zero after every call
        assert int(c["ws"][-4 * c["case"].B * 8:].count_nonzero()) == 0


def test_decode_length_one_returns_v_exactly():
    case = make_decode_case(8, 2, 128, 16, [1, 1, 1], max_slots=5, seed=3)
    kp, vp, table = gpu_decode_setup(case)
    out, _ = run_gpu_decode(case, kp, vp, table, hint=1)
    want = np.repeat(case.v_new, 4, axis=1)   # head h reads kv head h // 4
    assert np.array_equal(host_bits(out), want)


def test_decode_bitwise_deterministic_and_page_permutation_invariant():
    n_q, n_kv, D, ps, lengths, window, scale = CASES["d128_g3_ps64"]
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=8, seed=77, spare_pages=5)
    kp, vp, table = gpu_decode_setup(case)
    o1, l1 = run_gpu_decode(case, kp, vp, table, hint=3000)
    o2, l2 = run_gpu_decode(case, kp, vp, table, hint=3000)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    # relabel physical pages: same logical content, different page ids
    rng = np.random.default_rng(4)
    relabel = np.concatenate([[0], 1 + rng.permutation(case.n_pages - 1)]).astype(np.int64)
    kp2 = torch.empty_like(kp)
    vp2 = torch.empty_like(vp)
    idx = torch.from_numpy(relabel).to(kp.device)
    kp2[idx] = kp
    vp2[idx] = vp
    t2 = np.where(case.table > 0, relabel[np.maximum(case.table, 0)], case.table).astype(np.int32)
    o3, l3 = run_gpu_decode(case, kp2, vp2, dev_i32(t2), hint=3000)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)
    # the same with long splits (K through LDS)
    o4, l4 = run_gpu_decode(case, kp, vp, table, hint=LONG_SPLIT_HINT)
    o5, l5 = run_gpu_decode(case, kp2, vp2, dev_i32(t2), hint=LONG_SPLIT_HINT)
    assert torch.equal(o4.view(torch.int16), o5.view(torch.int16)) and torch.equal(l4, l5)


@pytest.mark.parametrize("shape", ["head_split", "d512_rounds"])
def test_decode_split0_early_merge_bitwise(shape):
    """On grids of several rounds split 0 merges at once, with its own values,
    when the row's other splits are already in, else publishes its partial
    like any split: which path runs depends on timing.  Repeated calls (with
    and without the fused append) must agree bit for bit, and with the
    oracle.  head_split: 2560 key-split workgroups; d512_rounds: 48 rows x 2
    kv heads at head_dim 512, 1152 dim-split workgroups."""
    if shape == "head_split":
        n_q, n_kv, D, ps, lengths, window, scale = CASES["head_split"]
    else:
        rng = np.random.default_rng(31)
        n_q, n_kv, D, ps, window, scale = 8, 2, 512, 64, 0, None
        lengths = [int(x) for x in rng.integers(256, 1537, size=48)]
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=len(lengths) + 2, seed=1700 + D,
                            window=window, scale=scale, spare_pages=2)
    kp, vp, table = gpu_decode_setup(case)
    outs = [run_gpu_decode(case, kp, vp, table) for _ in range(4)]
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])
    okp, ovp = oracle_decode_pools(case)
    ref, _ = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                case.scale, case.window)
    assert_attn_close(host_f64(outs[0][0]), ref, shape)
    for _ in range(2):
        kp2, vp2, table2 = gpu_decode_setup(case, with_new_token=False)
        o2, l2 = run_gpu_decode(case, kp2, vp2, table2, fused_append=True)
        assert torch.equal(o2.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l2, outs[0][1])
        assert np.array_equal(host_bits(kp2), okp) and np.array_equal(host_bits(vp2), ovp)


def test_decode_window_at_least_length_equals_full_bitwise():
    case = make_decode_case(8, 2, 128, 64, [300, 77, 512], max_slots=5, seed=9)
    kp, vp, table = gpu_decode_setup(case)
    full, _ = run_gpu_decode(case, kp, vp, table, hint=512)
    case.window = 512
    win, _ = run_gpu_decode(case, kp, vp, table, hint=512)
    assert torch.equal(full.view(torch.int16), win.view(torch.int16))


def test_decode_hint_below_lengths_still_correct():
    case = make_decode_case(8, 2, 128, 128, [2000, 700], max_slots=4, seed=12)
    kp, vp, table = gpu_decode_setup(case)
    out, _ = run_gpu_decode(case, kp, vp, table, hint=256)   # plan sized for 256 keys
    okp, ovp = oracle_decode_pools(case)
    ref, _ = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                case.scale, 0)
    assert_attn_close(host_f64(out), ref, "hint<L")


# ---- full-size workloads, every row, in the bench's launch configuration ----
# (fused append of the new token, the bench's length hint; pools bit-exact,
# every output row and lse against the oracle)

def _full_case(name, layer_dim=None, window=0, salt=0):
    c = CONFIGS[name]
    L, slots = config_lengths(name, salt)
    D = layer_dim or c["head_dim"]
    case = make_decode_case(c["n_q"], c["n_kv"], D, c["page_size"], L,
                            max_slots=c["max_slots"], seed=3407 + c["index"] + salt,
                            slot_of_row=slots, window=window, spare_pages=4,
                            pages_per_slot=-(-c["len_hi"] // c["page_size"]))
    return case, c["len_hi"]


def _full_check(case, hint):
    kp, vp, table = gpu_decode_setup(case, with_new_token=False)
    out, lse = run_gpu_decode(case, kp, vp, table, hint=hint, fused_append=True)
    okp, ovp = oracle_decode_pools(case)
    assert np.array_equal(host_bits(kp), okp), "K pool differs from the oracle"
    assert np.array_equal(host_bits(vp), ovp), "V pool differs from the oracle"
    ref, ref_lse = oracle.attn_decode(case.q, okp, ovp, case.table, case.slots, case.seq_lens,
                                      case.scale, case.window)
    assert_attn_close(host_f64(out), ref, "all rows")
    idle = case.seq_lens == 0
    g_lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isneginf(g_lse[idle]))
    assert np.max(np.abs(g_lse[~idle] - ref_lse[~idle]), initial=0.0) <= 1e-3
    assert np.all(host_bits(out)[idle] == 0)


def test_full_qwen3_decode_all_rows():
    case, hint = _full_case("qwen3_decode")
    _full_check(case, hint)


def test_full_llama_decode_all_rows():
    case, hint = _full_case("llama_decode")
    assert (case.seq_lens == 0).sum() == 6
    _full_check(case, hint)


def test_full_llama_tp8_share_all_rows():
    """One GPU's share of the Llama call under 8-way tensor parallelism."""
    case, hint = _full_case("llama_decode_tp8_share")
    assert (case.seq_lens == 0).sum() == 6 and case.n_q == 3 and case.n_kv == 1
    _full_check(case, hint)


def test_full_gemma_sliding_layer_all_rows():
    c = CONFIGS["gemma_mixed"]
    case, hint = _full_case("gemma_mixed", layer_dim=c["sliding_dim"], window=c["window"])
    _full_check(case, hint)


def test_full_gemma_full_layer_all_rows():
    c = CONFIGS["gemma_mixed"]
    case, hint = _full_case("gemma_mixed", layer_dim=c["full_dim"])
    _full_check(case, hint)


@pytest.mark.parametrize("shape", ["small", "large_grid"])
def test_decode_graph_replays_track_new_inputs(shape):
    """One decode call (fused append) captured in a HIP graph and replayed with
    new q, new-token K/V and shorter lengths written into its static inputs
    between replays: every replay equals the eager call on the same inputs
    bit for bit and matches the oracle.  (Replays reuse the workspace's split
    arrival counters; the path records no memset nodes.)  large_grid: the
    64-row head_split shape, whose plan takes the short split 0, the late V
    store and the early merge of split 0."""
    if shape == "small":
        case = make_decode_case(32, 8, 128, 128, [900, 300, 0, 2049, 77], max_slots=7,
                                seed=1700, spare_pages=2)
    else:
        n_q, n_kv, D, ps, lengths, window, scale = CASES["head_split"]
        case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=len(lengths) + 2,
                                seed=1710, spare_pages=2)
    kp, vp, table = gpu_decode_setup(case, with_new_token=False)
    hint = int(case.seq_lens.max())
    ws = pkv.new_decode_workspace(
        pkv.decode_workspace_size(case.B, case.n_q, case.n_kv, case.head_dim, hint), "cuda")
    q_s = dev_bits(case.q)
    kn_s, vn_s = dev_bits(case.k_new), dev_bits(case.v_new)
    slots_s, lens_s = dev_i32(case.slots), dev_i32(case.seq_lens)
    out_s = torch.empty_like(q_s)
    lse_s = torch.empty((case.B, case.n_q), dtype=torch.float32, device=DEV)

    def call(out, lse):
        pkv.attn_decode(q_s, slots_s, lens_s, table, kp, vp, scale=case.scale,
                        max_seq_len_hint=hint, k_new=kn_s, v_new=vn_s, out=out, lse=lse,
                        workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_s, lse_s)                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_s, lse_s)

    okp, ovp = case.empty_pools()
    hk, hv, hs, hp = case.history_tokens()
    oracle.append(okp, ovp, case.table, hk, hv, hs, hp)
    rng = np.random.default_rng(5)
    lens = case.seq_lens.copy()
    for r in range(3):
        if r:  # new inputs: fresh q and new token, one key fewer for the active rows
            lens = np.where(lens > 1, lens - 1, lens)
        q_r = case.q if r == 0 else \
            oracle.f64_to_bf16_bits(rng.standard_normal(case.q.shape))
        kn_r = case.k_new if r == 0 else \
            oracle.f64_to_bf16_bits(rng.standard_normal(case.k_new.shape))
        vn_r = case.v_new if r == 0 else \
            oracle.f64_to_bf16_bits(rng.standard_normal(case.v_new.shape))
        q_s.copy_(dev_bits(q_r))
        kn_s.copy_(dev_bits(kn_r))
        vn_s.copy_(dev_bits(vn_r))
        lens_s.copy_(dev_i32(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out_s.clone(), lse_s.clone()
        # the oracle: this replay's new token lands at position len-1 of each active row
        act = (case.slots != 0) & (lens > 0)
        oracle.append(okp, ovp, case.table, kn_r[act], vn_r[act], case.slots[act], lens[act] - 1)
        ref, _ = oracle.attn_decode(q_r, okp, ovp, case.table, case.slots, lens, case.scale, 0)
        assert_attn_close(host_f64(got), ref, f"replay {r}")
        # eager call on the same (now already appended) inputs: identical bits
        e_out, e_lse = torch.empty_like(out_s), torch.empty_like(lse_s)
        call(e_out, e_lse)
        torch.cuda.synchronize()
        assert torch.equal(e_out.view(torch.int16), got.view(torch.int16)), f"replay {r} vs eager"
        assert torch.equal(e_lse, got_lse)
    assert np.array_equal(host_bits(kp), okp) and np.array_equal(host_bits(vp), ovp)


def test_decode_graph_batch_buckets_with_slot0_padding():
    """Decode steps captured once per batch bucket -- the ladder 1, 2, 4, 8,
    then every 16 up to 64 ([moe-qwen3 compare] flex_gemma4_moe.py,
    capture_decode_cudagraph); a batch of n rows runs in the smallest bucket
    >= n, the rest padded with slot-0 rows.  Each replay appends every real
    row's new token and attends; real rows match the oracle, the whole bucket
    equals an eager call on the same padded inputs bit for bit, padding rows
    are exactly 0 and write nothing."""
    n_q, n_kv, D, ps = 32, 8, 128, 128
    lengths = list(np.random.default_rng(1901).integers(3, 2000, size=64))
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=66, seed=1900, spare_pages=4,
                            pages_per_slot=17)
    kp, vp, table = gpu_decode_setup(case, with_new_token=False)
    hint = 17 * ps
    okp, ovp = case.empty_pools()
    hk, hv, hs, hp = case.history_tokens()
    oracle.append(okp, ovp, case.table, hk, hv, hs, hp)
    lens = case.seq_lens.copy() - 1                 # keys before this test's first token
    buckets = {}
    for nb in (1, 2, 4, 8, 16, 32, 48, 64):
        st = dict(q=torch.zeros((nb, n_q, D), dtype=torch.bfloat16, device=DEV),
                  kn=torch.zeros((nb, n_kv, D), dtype=torch.bfloat16, device=DEV),
                  vn=torch.zeros((nb, n_kv, D), dtype=torch.bfloat16, device=DEV),
                  slots=dev_i32(np.zeros(nb)), lens=dev_i32(np.zeros(nb)),
                  out=torch.empty((nb, n_q, D), dtype=torch.bfloat16, device=DEV),
                  ws=pkv.new_decode_workspace(
                      pkv.decode_workspace_size(nb, n_q, n_kv, D, hint), "cuda"))

        def call(st=st):
            pkv.attn_decode(st["q"], st["slots"], st["lens"], table, kp, vp, scale=case.scale,
                            max_seq_len_hint=hint, k_new=st["kn"], v_new=st["vn"],
                            out=st["out"], workspace=st["ws"])

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):      # all-padding inputs: the capture itself writes nothing
            call()
        buckets[nb] = (g, st)
    torch.cuda.synchronize()
    rng = np.random.default_rng(19)
    for step, n in enumerate([5, 1, 8, 3, 17, 64, 2, 33, 50, 7, 47, 16, 4]):
        rows = np.sort(rng.choice(case.B, size=n, replace=False))
        nb = min(b for b in buckets if b >= n)
        g, st = buckets[nb]
        lens[rows] += 1
        q_r = oracle.f64_to_bf16_bits(rng.standard_normal((n, n_q, D)))
        kn_r = oracle.f64_to_bf16_bits(rng.standard_normal((n, n_kv, D)))
        vn_r = oracle.f64_to_bf16_bits(rng.standard_normal((n, n_kv, D)))
        pad = nb - n
        st["q"].copy_(dev_bits(np.concatenate([q_r, np.full((pad, n_q, D), 0x3F80, np.uint16)])))
        st["kn"].copy_(dev_bits(np.concatenate([kn_r, np.full((pad, n_kv, D), 0x3F80, np.uint16)])))
        st["vn"].copy_(dev_bits(np.concatenate([vn_r, np.full((pad, n_kv, D), 0x3F80, np.uint16)])))
        st["slots"].copy_(dev_i32(np.concatenate([case.slots[rows], np.zeros(pad)])))
        st["lens"].copy_(dev_i32(np.concatenate([lens[rows], np.zeros(pad)])))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = st["out"].clone()
        assert np.all(host_bits(got[n:]) == 0), f"step {step}: padding rows not zero"
        oracle.append(okp, ovp, case.table, kn_r, vn_r, case.slots[rows], lens[rows] - 1)
        ref, _ = oracle.attn_decode(q_r, okp, ovp, case.table, case.slots[rows], lens[rows],
                                    case.scale, 0)
        assert_attn_close(host_f64(got[:n]), ref, f"step {step} (n={n}, bucket {nb})")
        # the same padded batch, eager, tokens already appended: identical bits
        # (the split plan depends on the batch size, so only a call of the
        # bucket's size is bitwise comparable)
        e_out = pkv.attn_decode(st["q"], st["slots"], st["lens"], table, kp, vp,
                                scale=case.scale, max_seq_len_hint=hint)
        torch.cuda.synchronize()
        assert torch.equal(e_out.view(torch.int16), got.view(torch.int16)), f"step {step}"
    assert np.array_equal(host_bits(kp), okp) and np.array_equal(host_bits(vp), ovp)
