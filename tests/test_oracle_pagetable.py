"""Pins of the allocator model against the hand-derived golden op sequence."""

import json
import os

import numpy as np
import pytest

from oracle import PageTableModel
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "pagetable_sequence.json")) as f:
        return json.load(f)


def run_sequence(pt, steps, check):
    """Drive an allocator through the golden ops; ``check`` compares state."""
    for st in steps:
        op = st["op"]
        if op == "allocate":
            assert pt.allocate() == st["expect"]
        elif op == "can_reserve":
            assert pt.can_reserve(st["size"], st.get("slot")) == st["expect"]
        elif op == "reserve":
            dry = st.get("dry_run", False)
            if st["expect"] == "error":
                with pytest.raises(RuntimeError):
                    pt.reserve(st["slot"], st["seq_len"], dry_run=dry)
            else:
                assert pt.reserve(st["slot"], st["seq_len"], dry_run=dry) == st["expect"]
        elif op == "erase":
            pt.erase(st["slot"])
        check(pt, st)


def _check_model(pt, st):
    if "row" in st:
        assert pt.rows[st["slot"]] == st["row"]
    if "capacity" in st:
        assert pt.capacity[st["slot"]] == st["capacity"]
    if "free_pages" in st:
        assert pt.free_pages == st["free_pages"]


def test_model_follows_golden_sequence():
    g = _golden()
    pt = PageTableModel(g["n_pages"], g["page_size"], g["max_slots"])
    run_sequence(pt, g["steps"], _check_model)
    assert np.array_equal(pt.table(g["n_pages"]), np.array(g["final_device_table"]))


def test_model_page_conservation_random_ops():
    rng = np.random.default_rng(0)
    pt = PageTableModel(40, 8, 6)
    live = set()
    for _ in range(500):
        r = rng.random()
        if r < 0.3 and pt.free_slots:
            live.add(pt.allocate())
        elif r < 0.8 and live:
            s = int(rng.choice(sorted(live)))
            n = int(rng.integers(1, 120))
            if pt.can_reserve(n, s):
                pt.reserve(s, n)
        elif live:
            s = int(rng.choice(sorted(live)))
            pt.erase(s)
            live.discard(s)
        owned = [p for s in range(6) for p in pt.rows[s]]
        # every page is in exactly one of {free, some slot}; page 0 in neither
        assert sorted(owned + pt.free_pages) == list(range(1, 40))
        assert 0 not in owned and 0 not in pt.free_slots
