"""Device-side batch reserve (pkv_pt_device_reserve) against the oracle
allocator model: tables, free stacks, capacities and flags bit for bit; and a
captured decode step that grows its slots on the device."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pagetable_amd as pkv
from oracle.pagetable import PageTableModel
from tests.gpu_util import DEV, assert_attn_close, dev_bits, dev_i32, host_f64

pytestmark = pytest.mark.gpu


def _history(rng, n_pages, ps, max_slots, pps, steps=40):
    """A model with a random history of allocate / reserve / erase."""
    m = PageTableModel(n_pages, ps, max_slots)
    live = []
    for _ in range(steps):
        op = rng.integers(0, 3)
        if op == 0 and m.free_slots:
            live.append(m.allocate())
        elif op == 1 and live:
            s = int(rng.choice(live))
            want = m.capacity[s] + int(rng.integers(1, 3 * ps))
            if want <= pps * ps and m.can_reserve(want, s):
                m.reserve(s, want)
        elif op == 2 and live:
            s = live.pop(int(rng.integers(0, len(live))))
            m.erase(s)
    while m.free_slots and len(live) < max_slots - 1:
        live.append(m.allocate())
    return m, live


def _to_device(m, pps):
    fp = np.zeros(m.n_pages, np.int32)
    fp[:len(m.free_pages)] = m.free_pages
    st = pkv.DevicePageState(dev_i32(m.table(pps)), dev_i32(fp),
                             dev_i32([len(m.free_pages)]),
                             dev_i32(np.asarray(m.capacity, np.int32)), m.page_size)
    return st


def _model_batch(m, pps, slots, lens):
    """What successive host reserve calls do, with the device call's flags."""
    flags = 0
    for s, L in zip(slots, lens):
        s, L = int(s), int(L)
        if not (1 <= s < m.max_slots) or L <= m.capacity[s]:
            continue
        k = -(-(L - m.capacity[s]) // m.page_size)
        if m.capacity[s] // m.page_size + k > pps:
            flags |= pkv.RESERVE_TOO_LONG
            continue
        if k > m.pages_available:
            flags |= pkv.RESERVE_NO_PAGES
            continue
        m.reserve(s, L)
    return flags


def _compare(st, m, pps, flags):
    torch.cuda.synchronize()
    assert np.array_equal(st.table.cpu().numpy(), m.table(pps))
    n = int(st.free_count.item())
    assert n == len(m.free_pages)
    assert np.array_equal(st.free_pages.cpu().numpy()[:n], np.asarray(m.free_pages, np.int32))
    assert np.array_equal(st.capacity.cpu().numpy(), np.asarray(m.capacity, np.int32))
    assert int(st.status.item()) == flags


@pytest.mark.parametrize("seed", range(6))
def test_device_reserve_matches_model(seed):
    rng = np.random.default_rng(50 + seed)
    ps = int(rng.choice([16, 64, 128]))
    n_pages, max_slots, pps = int(rng.integers(40, 200)), int(rng.integers(4, 40)), 16
    m, live = _history(rng, n_pages, ps, max_slots, pps)
    st = _to_device(m, pps)
    # one decode-like batch: every live slot grows by 0 .. 2 pages' worth,
    # plus padding rows (slot 0) and a too-long request
    slots = list(live) + [0, 0]
    lens = [m.capacity[s] - int(rng.integers(0, 3)) + int(rng.integers(0, 2 * ps + 2))
            for s in live] + [5, 0]
    if live:
        lens[0] = pps * ps + 1          # beyond its table row
    order = rng.permutation(len(slots))
    slots = [slots[i] for i in order]
    lens = [max(int(lens[i]), 0) for i in order]
    st.reserve(dev_i32(slots), dev_i32(lens))
    flags = _model_batch(m, pps, slots, lens)
    _compare(st, m, pps, flags)
    # a second batch on the state the first left behind
    lens2 = [L + int(rng.integers(0, ps)) for L in lens]
    st.reserve(dev_i32(slots), dev_i32(lens2))
    flags |= _model_batch(m, pps, slots, lens2)
    _compare(st, m, pps, flags)


def test_device_reserve_exhaustion_serves_rows_in_order():
    """More demand than free pages: rows that do not fit are skipped and
    flagged, later smaller rows still get pages (the sequential fallback)."""
    ps, pps = 16, 64
    m = PageTableModel(30, ps, 12)
    slots = [m.allocate() for _ in range(11)]
    st = _to_device(m, pps)
    lens = [ps * 10, ps * 12, 5, ps * 9, 1, ps * 30, 17, 3, ps * 2, 40, 16]
    st.reserve(dev_i32(slots), dev_i32(lens))
    flags = _model_batch(m, pps, slots, lens)
    assert flags == pkv.RESERVE_NO_PAGES
    _compare(st, m, pps, flags)


def test_device_reserve_many_rows_across_tiles():
    """600 rows (three 256-row tiles): each tile sees the previous ones' grants."""
    rng = np.random.default_rng(9)
    ps, pps = 16, 8
    m = PageTableModel(1600, ps, 601)
    slots = [m.allocate() for _ in range(600)]
    st = _to_device(m, pps)
    lens = [int(x) for x in rng.integers(0, 3 * ps, size=600)]
    st.reserve(dev_i32(slots), dev_i32(lens))
    flags = _model_batch(m, pps, slots, lens)
    _compare(st, m, pps, flags)
    lens2 = [L + int(x) for L, x in zip(lens, rng.integers(0, 6 * ps, size=600))]
    st.reserve(dev_i32(slots), dev_i32(lens2))
    flags |= _model_batch(m, pps, slots, lens2)
    _compare(st, m, pps, flags)


def test_graph_decode_step_reserves_pages_on_device():
    """A captured decode step = device reserve of each row's new length, then
    decode with the fused append of the new token.  Replayed token after token
    (crossing page boundaries), it matches the oracle on every replay, and the
    final table equals the host model's."""
    n_q, n_kv, D, ps = 8, 2, 128, 16
    rng = np.random.default_rng(77)
    B, max_slots, n_pages, pps = 4, 6, 64, 16
    m = PageTableModel(n_pages, ps, max_slots)
    slots = [m.allocate() for _ in range(B)]
    start = [int(x) for x in rng.integers(1, 40, size=B)]
    for s, L in zip(slots, start):
        m.reserve(s, L)
    st = _to_device(m, pps)
    kp, vp = pkv.new_pools(n_pages, n_kv, ps, D, fill=-1)   # NaN sentinel
    # history of each row, written with the standalone append
    hist_k = [rng.standard_normal((L, n_kv, D)).astype(np.float32) for L in start]
    hist_v = [rng.standard_normal((L, n_kv, D)).astype(np.float32) for L in start]
    bf = lambda x: oracle.f64_to_bf16_bits(np.asarray(x, np.float64))
    tok_slot = np.concatenate([[s] * L for s, L in zip(slots, start)]).astype(np.int32)
    tok_pos = np.concatenate([np.arange(L) for L in start]).astype(np.int32)
    pkv.append(dev_bits(bf(np.concatenate(hist_k))), dev_bits(bf(np.concatenate(hist_v))),
               dev_i32(tok_slot), dev_i32(tok_pos), st.table, kp, vp)
    hist_k = [oracle.bf16_bits_to_f64(bf(h)) for h in hist_k]
    hist_v = [oracle.bf16_bits_to_f64(bf(h)) for h in hist_v]
    # static inputs of the captured step
    d_slots = dev_i32(slots)
    d_lens = dev_i32([L + 1 for L in start])
    q = torch.empty((B, n_q, D), dtype=torch.bfloat16, device=DEV)
    kn = torch.empty((B, n_kv, D), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty((B, n_kv, D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, n_q, D), dtype=torch.bfloat16, device=DEV)
    hint = pps * ps
    ws = pkv.new_decode_workspace(pkv.decode_workspace_size(B, n_q, n_kv, D, hint), DEV)

    def step():
        st.reserve(d_slots, d_lens)
        pkv.attn_decode(q, d_slots, d_lens, st.table, kp, vp, window=0, max_seq_len_hint=hint,
                        k_new=kn, v_new=vn, out=out, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    lens = list(start)
    for it in range(20):
        qb = bf(rng.standard_normal((B, n_q, D)))
        kb = bf(rng.standard_normal((B, n_kv, D)))
        vb = bf(rng.standard_normal((B, n_kv, D)))
        q.copy_(dev_bits(qb).view(torch.bfloat16))
        kn.copy_(dev_bits(kb).view(torch.bfloat16))
        vn.copy_(dev_bits(vb).view(torch.bfloat16))
        lens = [L + 1 for L in lens]
        d_lens.copy_(dev_i32(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b in range(B):
            hist_k[b] = np.concatenate([hist_k[b], oracle.bf16_bits_to_f64(kb[b:b + 1])])
            hist_v[b] = np.concatenate([hist_v[b], oracle.bf16_bits_to_f64(vb[b:b + 1])])
        got = host_f64(out)
        for b in range(B):
            ref, _ = oracle.attend_rows(oracle.bf16_bits_to_f64(qb[b]), hist_k[b], hist_v[b],
                                        lens[b] - 1, 1.0 / np.sqrt(D), 0)
            assert_attn_close(got[b], ref, f"replay {it} row {b}")
        _model_batch(m, pps, slots, lens)
    _compare(st, m, pps, 0)


def _model_erase(m, slots):
    """The device erase on the model: the pages' erase of each listed slot in
    order, then the reset the allocate of each does (capacity 0, row -1)."""
    done = [int(s) for s in slots if 1 <= int(s) < m.max_slots]
    for s in done:
        m.erase(s)
    for _ in done:
        m.allocate()


@pytest.mark.parametrize("seed", range(6))
def test_device_erase_matches_model(seed):
    rng = np.random.default_rng(150 + seed)
    ps = int(rng.choice([16, 64, 128]))
    n_pages, max_slots, pps = int(rng.integers(40, 200)), int(rng.integers(4, 40)), 16
    m, live = _history(rng, n_pages, ps, max_slots, pps, steps=60)
    st = _to_device(m, pps)
    k = int(rng.integers(1, len(live) + 1))
    gone = [int(s) for s in rng.choice(live, size=k, replace=False)]
    rows = gone + [0, max_slots]          # padding and out-of-range rows are skipped
    rows = [rows[i] for i in rng.permutation(len(rows))]
    st.erase(dev_i32(rows))
    _model_erase(m, rows)
    _compare(st, m, pps, 0)
    # the freed pages are granted again, in stack order, by a device reserve
    lens = [int(rng.integers(1, pps * ps + 1)) for _ in gone]
    st.reserve(dev_i32(gone), dev_i32(lens))
    flags = _model_batch(m, pps, gone, lens)
    _compare(st, m, pps, flags)


def test_device_erase_many_rows_across_tiles():
    """Erase 450 of 600 slots (two 256-row tiles), then reserve them again."""
    rng = np.random.default_rng(19)
    ps, pps = 16, 8
    m = PageTableModel(5000, ps, 601)
    slots = [m.allocate() for _ in range(600)]
    for s, L in zip(slots, rng.integers(0, pps * ps + 1, size=600)):
        m.reserve(s, int(L))
    st = _to_device(m, pps)
    gone = [int(s) for s in rng.permutation(slots)[:450]]
    st.erase(dev_i32(gone))
    _model_erase(m, gone)
    _compare(st, m, pps, 0)
    lens = [int(x) for x in rng.integers(0, pps * ps + 1, size=450)]
    st.reserve(dev_i32(gone), dev_i32(lens))
    flags = _model_batch(m, pps, gone, lens)
    _compare(st, m, pps, flags)


def test_device_erase_flags_inconsistent_state():
    """States no allocator sequence produces: a capacity that is not a whole
    number of pages, and owned pages that would overflow the free stack.  The
    row is left unchanged, flagged, and the rows after it proceed."""
    ps, pps, n_pages, max_slots = 16, 4, 10, 5
    table = np.full((max_slots, pps), -1, np.int32)
    table[0] = 0
    table[1, :3] = [7, 8, 9]
    table[2, :1] = [5]
    table[3, :2] = [3, 4]
    cap = np.array([0, 3 * ps, ps, 2 * ps - 1, 0], np.int32)
    free = np.zeros(n_pages, np.int32)
    free[:8] = [1, 2, 6, 1, 2, 6, 1, 2]       # 8 entries: slot 1's 3 pages cannot fit
    st = pkv.DevicePageState(dev_i32(table), dev_i32(free), dev_i32([8]), dev_i32(cap), ps)
    st.erase(dev_i32([1, 3, 2]))
    torch.cuda.synchronize()
    assert int(st.status.item()) == pkv.RESERVE_BAD_STATE
    assert int(st.free_count.item()) == 9
    got_free = st.free_pages.cpu().numpy()
    assert got_free[8] == 5 and np.array_equal(got_free[:8], free[:8])
    t = st.table.cpu().numpy()
    want = table.copy()
    want[2] = -1
    assert np.array_equal(t, want)
    assert np.array_equal(st.capacity.cpu().numpy(), [0, 3 * ps, 0, 2 * ps - 1, 0])


def test_graph_step_erases_and_reserves_on_device():
    """A captured step that erases the finished slots and then grows the live
    ones, replayed with new inputs each time, matches the model after every
    replay (no host round trip inside the step)."""
    rng = np.random.default_rng(23)
    ps, pps, max_slots, n_pages = 16, 8, 9, 96
    m = PageTableModel(n_pages, ps, max_slots)
    slots = [m.allocate() for _ in range(8)]
    lens = [int(x) for x in rng.integers(1, 3 * ps, size=8)]
    for s, L in zip(slots, lens):
        m.reserve(s, L)
    st = _to_device(m, pps)
    d_gone = dev_i32([0] * 8)
    d_slots = dev_i32(slots)
    d_lens = dev_i32(lens)

    def step():
        st.erase(d_gone)
        st.reserve(d_slots, d_lens)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    flags = 0
    for it in range(12):
        # a few slots finish (row slot, else 0 = padding) and restart short
        gone = [s_ if rng.random() < 0.25 else 0 for s_ in slots]
        lens = [int(rng.integers(1, ps)) if g_ else L + int(rng.integers(0, ps))
                for g_, L in zip(gone, lens)]
        lens = [min(L, pps * ps) for L in lens]
        d_gone.copy_(dev_i32(gone))
        d_lens.copy_(dev_i32(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _model_erase(m, gone)
        flags |= _model_batch(m, pps, slots, lens)
        _compare(st, m, pps, flags)


def test_slot_reuse_after_device_erase_decodes_correctly():
    """Requests finish and new ones take over their slots with the device
    allocator only: erase returns the pages, reserve hands the same (recycled)
    pages to the new request, whose history is appended over the old one's.
    Decode with the fused append must see only the new request's keys, even
    though the recycled pages still hold the old request's rows past them."""
    n_q, n_kv, D, ps = 8, 2, 128, 16
    B, max_slots, n_pages, pps = 3, 4, 16, 8
    rng = np.random.default_rng(91)
    bf = lambda x: oracle.f64_to_bf16_bits(np.asarray(x, np.float64))
    m = PageTableModel(n_pages, ps, max_slots)
    slots = [m.allocate() for _ in range(B)]
    st = _to_device(m, pps)
    kp, vp = pkv.new_pools(n_pages, n_kv, ps, D, fill=-1)   # NaN sentinel
    hist_k, hist_v = [None] * B, [None] * B
    ws = pkv.new_decode_workspace(pkv.decode_workspace_size(B, n_q, n_kv, D, pps * ps), DEV)
    d_slots = dev_i32(slots)

    def start(rows, lengths):
        """New requests on these rows: device reserve, then their history appended."""
        lens = [0] * B
        for b, L in zip(rows, lengths):
            lens[b] = L
        st.reserve(dev_i32([slots[b] for b in rows]), dev_i32(lengths))
        flags = _model_batch(m, pps, [slots[b] for b in rows], lengths)
        assert flags == 0
        ks, vs, ts, tp = [], [], [], []
        for b, L in zip(rows, lengths):
            k = bf(rng.standard_normal((L, n_kv, D)))
            v = bf(rng.standard_normal((L, n_kv, D)))
            hist_k[b], hist_v[b] = oracle.bf16_bits_to_f64(k), oracle.bf16_bits_to_f64(v)
            ks.append(k)
            vs.append(v)
            ts.append(np.full(L, slots[b], np.int32))
            tp.append(np.arange(L, dtype=np.int32))
        pkv.append(dev_bits(np.concatenate(ks)), dev_bits(np.concatenate(vs)),
                   dev_i32(np.concatenate(ts)), dev_i32(np.concatenate(tp)), st.table, kp, vp)

    def decode_steps(n):
        for _ in range(n):
            lens = [h.shape[0] + 1 for h in hist_k]
            st.reserve(d_slots, dev_i32(lens))
            assert _model_batch(m, pps, slots, lens) == 0
            qb = bf(rng.standard_normal((B, n_q, D)))
            kb = bf(rng.standard_normal((B, n_kv, D)))
            vb = bf(rng.standard_normal((B, n_kv, D)))
            out = pkv.attn_decode(dev_bits(qb).view(torch.bfloat16), d_slots, dev_i32(lens),
                                  st.table, kp, vp, window=0, max_seq_len_hint=pps * ps,
                                  k_new=dev_bits(kb).view(torch.bfloat16),
                                  v_new=dev_bits(vb).view(torch.bfloat16), workspace=ws)
            got = host_f64(out)
            for b in range(B):
                hist_k[b] = np.concatenate([hist_k[b], oracle.bf16_bits_to_f64(kb[b:b + 1])])
                hist_v[b] = np.concatenate([hist_v[b], oracle.bf16_bits_to_f64(vb[b:b + 1])])
                ref, _ = oracle.attend_rows(oracle.bf16_bits_to_f64(qb[b]), hist_k[b],
                                            hist_v[b], lens[b] - 1, 1.0 / np.sqrt(D), 0)
                assert_attn_close(got[b], ref, f"row {b} length {lens[b]}")

    start([0, 1, 2], [40, 70, 20])         # 3 + 5 + 2 of the 15 pages
    decode_steps(3)
    # row 1 finishes; a shorter request takes its slot and recycled pages
    st.erase(dev_i32([slots[1]]))
    _model_erase(m, [slots[1]])
    start([1], [23])
    decode_steps(3)
    # rows 0 and 2 finish; longer requests reuse pages row 1's first request held
    st.erase(dev_i32([slots[0], slots[2]]))
    _model_erase(m, [slots[0], slots[2]])
    start([0, 2], [51, 33])
    decode_steps(4)
    _compare(st, m, pps, 0)
