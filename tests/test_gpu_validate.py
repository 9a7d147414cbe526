"""Validation mode: device checks of slots, positions and page-table entries.

Bad metadata here is handled by the kernels' own bounds checks (skipped
tokens, idle rows, absent keys), so these calls stay in bounds; only the
flag word is checked, not the (unspecified) outputs of the bad calls.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_pagetable_amd as pkv
from synth import make_decode_case, make_prefill_case
from tests.gpu_util import dev_bits, dev_i32, gpu_decode_setup, gpu_pools, run_gpu_decode

pytestmark = pytest.mark.gpu


@pytest.fixture
def validation():
    pkv.validation_flags(clear=True)
    pkv.set_validation(True)
    yield
    pkv.set_validation(False)
    pkv.validation_flags(clear=True)


def _decode_case():
    # rows 0..2 active (slots 1..3), row 3 idle (slot 0)
    return make_decode_case(8, 2, 64, 16, [37, 50, 5, 0], max_slots=6, seed=901)


def test_valid_calls_raise_no_flags(validation):
    case = _decode_case()
    kp, vp, table = gpu_decode_setup(case)
    run_gpu_decode(case, kp, vp, table)
    pcase = make_prefill_case(8, 2, 64, 16, [20, 33], seed=902)
    kp2, vp2 = gpu_pools(pcase)
    t2 = dev_i32(pcase.table)
    pkv.attn_prefill(dev_bits(pcase.q), dev_i32(pcase.cu_seqlens), dev_i32(pcase.slots), t2,
                     kp2, vp2, start_pos=dev_i32(pcase.start_pos), max_seqlen_q_hint=33)
    assert pkv.validation_flags() == 0


def test_decode_unmapped_page_and_bad_slot(validation):
    case = _decode_case()
    kp, vp, table = gpu_decode_setup(case)
    assert pkv.validation_flags() == 0
    # an unmapped entry inside row 1's used pages
    slot1 = int(case.slots[1])
    bad = case.table.copy()
    bad[slot1, 1] = -1
    run_gpu_decode(case, kp, vp, dev_i32(bad))
    assert pkv.validation_flags() == pkv.VALIDATE_PAGE
    # entries past a row's length are not used: no flag
    unused = case.table.copy()
    slot2 = int(case.slots[2])      # length 5: only page 0 is used
    unused[slot2, 1:] = -1
    run_gpu_decode(case, kp, vp, dev_i32(unused))
    assert pkv.validation_flags() == 0
    # a slot beyond max_slots
    slots = case.slots.copy()
    slots[0] = case.max_slots + 3
    lens = dev_i32(case.seq_lens)
    pkv.attn_decode(dev_bits(case.q), dev_i32(slots), lens, dev_i32(case.table), kp, vp,
                    scale=case.scale, max_seq_len_hint=64)
    assert pkv.validation_flags() == pkv.VALIDATE_SLOT


def test_append_position_beyond_capacity(validation):
    case = _decode_case()
    kp, vp = gpu_pools(case)
    table = dev_i32(case.table)
    cap = case.pages_per_slot * case.page_size
    slot = dev_i32([1, 2])
    pos = dev_i32([3, cap])          # the second is one past the slot's capacity
    kn = dev_bits(np.zeros((2, case.n_kv, case.head_dim), np.uint16))
    pkv.append(kn, kn, slot, pos, table, kp, vp)
    assert pkv.validation_flags() == pkv.VALIDATE_POS
    pkv.append(kn, kn, dev_i32([0, 0]), dev_i32([-5, cap + 7]), table, kp, vp)  # slot 0: no-op
    assert pkv.validation_flags() == 0


def test_prefill_unmapped_page_flagged_and_flags_accumulate(validation):
    pcase = make_prefill_case(8, 2, 64, 16, [20, 33], seed=903)
    kp, vp = gpu_pools(pcase)
    bad = pcase.table.copy()
    bad[int(pcase.slots[1]), 2] = 0      # page 0 is reserved: never a valid entry
    args = (dev_bits(pcase.q), dev_i32(pcase.cu_seqlens), dev_i32(pcase.slots), dev_i32(bad),
            kp, vp)
    pkv.attn_prefill(*args, start_pos=dev_i32(pcase.start_pos), max_seqlen_q_hint=33)
    slots = pcase.slots.copy()
    slots[0] = -2
    pkv.attn_prefill(args[0], args[1], dev_i32(slots), dev_i32(pcase.table), kp, vp,
                     start_pos=dev_i32(pcase.start_pos), max_seqlen_q_hint=33)
    assert pkv.validation_flags(clear=False) == pkv.VALIDATE_PAGE | pkv.VALIDATE_SLOT
    assert pkv.validation_flags() == pkv.VALIDATE_PAGE | pkv.VALIDATE_SLOT
    assert pkv.validation_flags() == 0


def test_validation_off_checks_nothing():
    pkv.set_validation(False)
    pkv.validation_flags(clear=True)
    case = _decode_case()
    kp, vp, table = gpu_decode_setup(case)
    bad = case.table.copy()
    bad[int(case.slots[0]), 0] = -1
    run_gpu_decode(case, kp, vp, dev_i32(bad))
    assert pkv.validation_flags() == 0
