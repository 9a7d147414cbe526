"""GPU append parity: pools bit-exact against the oracle, sentinels untouched."""

import numpy as np
import pytest
import torch

import oracle
from synth import make_decode_case
from tests.gpu_util import gpu_decode_setup, host_bits, oracle_decode_pools

pytestmark = pytest.mark.gpu

CASES = [
    # (n_q, n_kv, D, page_size, lengths, slots)
    (4, 2, 64, 16, [37, 50], [1, 2]),                    # tiny workload
    (8, 8, 128, 128, [1, 127, 128, 129, 0, 700], None),  # page edges, an idle row
    (6, 2, 256, 64, [300, 65, 0, 1], [4, 2, 1, 3]),
    (8, 2, 512, 64, [130, 64, 3], None),
    (4, 1, 128, 16, [33, 17, 16, 15], None),
]


@pytest.mark.parametrize("cfg", CASES, ids=[f"D{c[2]}_ps{c[3]}" for c in CASES])
def test_append_bit_exact(cfg):
    n_q, n_kv, D, ps, lengths, slots = cfg
    B = len(lengths)
    case = make_decode_case(n_q, n_kv, D, ps, lengths, max_slots=B + 2, seed=100 + D + ps,
                            slot_of_row=slots, spare_pages=3)
    kp, vp, _ = gpu_decode_setup(case)
    torch.cuda.synchronize()
    ok, ov = oracle_decode_pools(case)
    assert np.array_equal(host_bits(kp), ok), "K pool differs from the oracle scatter"
    assert np.array_equal(host_bits(vp), ov), "V pool differs from the oracle scatter"


def test_append_slot_zero_and_out_of_table_tokens_are_skipped():
    from tests.gpu_util import dev_bits, dev_i32, gpu_pools
    import paged_kv_attention_pagetable_amd as pkv
    case = make_decode_case(4, 2, 64, 16, [20], max_slots=3, seed=5, spare_pages=2)
    kp, vp = gpu_pools(case)
    table = dev_i32(case.table)
    T = 5
    rng = np.random.default_rng(1)
    k = rng.integers(0, 0x7F00, size=(T, 2, 64)).astype(np.uint16)
    slot = np.array([0, 0, 2, 1, 1], np.int32)      # slot 2 has no pages (row is -1)
    pos = np.array([0, 3, 0, 10 ** 6, 19], np.int32)  # 10**6 is past the table row
    pkv.append(dev_bits(k), dev_bits(k), dev_i32(slot), dev_i32(pos), table, kp, vp)
    torch.cuda.synchronize()
    ok, ov = case.empty_pools()
    oracle.append(ok, ov, case.table, k[4:], k[4:], slot[4:], pos[4:])
    assert np.array_equal(host_bits(kp), ok)
    assert np.array_equal(host_bits(vp), ov)
