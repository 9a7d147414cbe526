"""The decode split-K plan (host logic, no GPU): the rules the kernels' launch
depends on, pinned on the bench's decode shapes."""

import pytest

import paged_kv_attention_pagetable_amd as pkv


def plan(*a):
    return pkv.decode_plan(*a)


def test_llama_shape_gets_the_large_grid_path():
    # 64 rows x 8 kv heads up to 4096 keys: 512-key splits, a 128-key split 0
    # (4096 + 512 workgroups), the late V store and the early merge
    p = plan(64, 24, 8, 128, 4096, 0)
    assert (p["split_tokens"], p["head_tokens"], p["max_splits"]) == (512, 128, 9)
    assert p["v_late"] and p["early_merge"]


def test_tensor_parallel_share_keeps_the_plain_splits():
    # 64 (row, kv head) pairs: 512 workgroups, under three rounds of slots
    p = plan(64, 3, 1, 128, 4096, 0)
    assert (p["split_tokens"], p["head_tokens"], p["max_splits"]) == (512, 512, 8)
    assert not p["v_late"] and not p["early_merge"]


def test_qwen3_call_takes_one_chunk_per_wave():
    p = plan(8, 32, 8, 128, 1024, 0)
    assert (p["split_tokens"], p["head_tokens"], p["max_splits"]) == (128, 128, 8)
    assert not p["v_late"] and not p["early_merge"]


def test_gemma_layers():
    # sliding: the window bounds the range (512 + 31 keys), no short split 0
    s = plan(64, 8, 2, 256, 1536, 512)
    assert (s["split_tokens"], s["head_tokens"], s["max_splits"]) == (128, 128, 5)
    assert not s["v_late"] and not s["early_merge"]   # 640 workgroups: one round
    # full: 1536 dim-split workgroups, several rounds: early merge only
    f = plan(64, 8, 2, 512, 1536, 0)
    assert (f["split_tokens"], f["head_tokens"], f["max_splits"]) == (128, 128, 12)
    assert not f["v_late"] and f["early_merge"]


@pytest.mark.parametrize("args", [(64, 24, 8, 128, 4096, 0), (8, 32, 8, 128, 1024, 0),
                                  (64, 8, 2, 512, 1536, 0), (1, 16, 1, 128, 10**6, 0),
                                  (3, 4, 2, 64, 50, 0), (512, 32, 8, 128, 100000, 0)])
def test_plan_invariants(args):
    p = plan(*args)
    B, n_q, n_kv, D, hint, window = args
    G = n_q // n_kv
    assert p["ws_bytes"] == pkv.decode_workspace_size(*args)
    assert p["split_tokens"] % 128 == 0 and 0 < p["head_tokens"] <= p["split_tokens"]
    assert p["max_splits"] * G <= 1024                      # one merge reads at most 1024 partials
    assert (p["max_splits"] == 1) == (p["ws_bytes"] == 0)   # one split: no workspace
    # the splits cover the hinted range: split 0, then full splits after it
    if p["max_splits"] > 1:
        assert p["head_tokens"] + (p["max_splits"] - 1) * p["split_tokens"] >= hint
    assert p["v_late"] <= p["early_merge"] or D > 128       # the late V store comes with it
    if p["v_late"]:
        assert D <= 128 and p["head_tokens"] < p["split_tokens"]


def test_plan_rejects_invalid_sizes():
    for bad in ((0, 8, 2, 128, 100, 0), (4, 6, 4, 128, 100, 0), (4, 8, 0, 128, 100, 0)):
        with pytest.raises(pkv.PkvError):
            plan(*bad)
