"""Oracle: paged KV cache addressing, append, gather and masked GQA attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  numpy float64.

Storage format (the library's documented pool layout; the pages' own cache is
one ``(1, H, n_pages*page_size, D)`` buffer per K and V, see
[continuous-batching compare] scripts/benchmarks/flex_paged_attention.py,
``PagedKVCache.__init__``):

* K pool: bf16 ``[n_pages][n_kv][page_size][D]``  (token rows, D contiguous)
* V pool: bf16 ``[n_pages][n_kv][page_size/gs][D][gs]``, ``gs = min(page_size,
  32)``: a page's rows in groups of ``gs`` consecutive keys, each group stored
  d-major; element (d, row) is ``v_pool[page, head, row // gs, d, row % gs]``
* page table: int ``[max_slots][pages_per_slot]``; entry ``-1`` = unmapped;
  slot 0 is the reserved no-op slot and page 0 the reserved page.

bf16 values are carried as their uint16 bit patterns so the append can be
compared byte for byte.

Parity: every function here is pinned by ``tests/test_oracle_paged.py``.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bf16 <-> float64 (exact upcast; round-to-nearest-even downcast)
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64 (bf16 = top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 to bf16 (8 significant bits) with ties-to-even, return bits.

    Rounds once, directly from float64 (no intermediate fp32 rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    xf = x[fin]
    ax = np.abs(xf)
    # exponent E with 2**E <= |x| < 2**(E+1); bf16 keeps 7 fraction bits.
    _, e = np.frexp(ax)  # ax = m * 2**e, 0.5 <= m < 1  ->  E = e - 1
    E = np.where(ax > 0, e - 1, -126)
    E = np.maximum(E, -126)  # subnormal range shares the 2**-133 quantum
    quantum = np.ldexp(1.0, E - 7)
    r = np.rint(xf / quantum) * quantum  # numpy rint: round half to even
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, xf), r)
    out[fin] = r
    out[~fin] = x[~fin]
    bits32 = out.astype(np.float32).view(np.uint32)
    res = (bits32 >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    res[nan] = np.uint16(0x7FC0)
    return res


# --------------------------------------------------------------------------
# Addressing, append, gather
# --------------------------------------------------------------------------


def physical_page(table, slot: int, pos: int, page_size: int) -> int:
    """Physical page of logical token ``pos`` of ``slot``.

    The logical page is ``pos // page_size`` and the row inside it
    ``pos % page_size`` ([continuous-batching compare]
    scripts/benchmarks/flex_paged_attention.py, ``PageTable.assign`` -- "find
    address" -- and ``assign_prefill_no_paging``).
    """
    return int(table[slot][pos // page_size])


def append(k_pool, v_pool, table, k_new, v_new, slot, pos) -> None:
    """Scatter new K/V rows into the pools, in token order (bit copy).

    ``k_new``/``v_new``: uint16 ``[T][n_kv][D]``; ``slot``/``pos``: ``[T]``.
    Tokens whose slot is 0 are skipped: slot 0 is the reserved no-op slot
    ([continuous-batching compare] flex_paged_attention.py, ``PageTable.__init__``,
    "batch_idx 0 is reserved for no-op").  Covers both the decode form
    (``PageTable.assign``) and the packed prefill form
    (``PageTable.assign_prefill_no_paging``): each token lands at
    ``page_table[slot, pos // page_size]``, row ``pos % page_size``.
    """
    ps = k_pool.shape[2]
    gs = v_pool.shape[4]
    for t in range(len(slot)):
        s = int(slot[t])
        if s == 0:
            continue
        p = int(pos[t])
        phys = physical_page(table, s, p, ps)
        row = p % ps
        k_pool[phys, :, row, :] = k_new[t]
        v_pool[phys, :, row // gs, :, row % gs] = v_new[t]


def gather_kv(k_pool, v_pool, table, slot: int, length: int):
    """Dense float64 ``K, V [length][n_kv][D]`` of ``slot``'s logical tokens."""
    n_kv, ps, D = k_pool.shape[1], k_pool.shape[2], k_pool.shape[3]
    gs = v_pool.shape[4]
    K = np.empty((length, n_kv, D), dtype=np.float64)
    V = np.empty((length, n_kv, D), dtype=np.float64)
    for j in range(length):
        phys = physical_page(table, slot, j, ps)
        K[j] = bf16_bits_to_f64(k_pool[phys, :, j % ps, :])
        row = j % ps
        V[j] = bf16_bits_to_f64(v_pool[phys, :, row // gs, :, row % gs])
    return K, V


# --------------------------------------------------------------------------
# Masks and attention
# --------------------------------------------------------------------------


def visible(q_pos, kv_pos, window: int):
    """Causal (+ sliding window) visibility of key ``kv_pos`` from query ``q_pos``.

    Causal: ``q >= kv`` ([continuous-batching compare] flex_paged_attention.py,
    ``create_causal_blockmask``).  Sliding: additionally ``q - kv < W``
    ([moe-qwen3 compare] unsloth/inference/flex_gemma4_moe.py,
    ``_create_sliding_causal_blockmask``), i.e. W keys including the query's own.
    ``window == 0`` means no window.  Decode uses the same predicate with the
    query at its absolute position (``_decode_block_mask``: ``q_idx + off[b]``).
    """
    q_pos = np.asarray(q_pos)
    kv_pos = np.asarray(kv_pos)
    vis = kv_pos <= q_pos
    if window > 0:
        vis = vis & ((q_pos - kv_pos) < window)
    return vis


def attend_rows(q, K, V, q_pos: int, scale: float, window: int):
    """Textbook masked softmax attention of all query heads of one token.

    ``q``: float64 ``[n_q][D]``; ``K, V``: float64 ``[Lk][n_kv][D]`` holding the
    keys at logical positions ``0..Lk-1``.  GQA: query head ``h`` reads kv head
    ``h // (n_q // n_kv)`` (``flex_attention(..., enable_gqa=True)`` in
    [moe-qwen3 compare] flex_gemma4_moe.py, attention forward).
    Returns ``out [n_q][D]`` and natural-log ``lse [n_q]``.  A query that sees
    no key gets ``out = 0`` and ``lse = -inf`` (the pages require padded rows to
    come out as zeros, not NaN: [continuous-batching compare] results write-up,
    correctness breaks, ``ROWS_GUARANTEED_SAFE``).
    """
    n_q, D = q.shape
    n_kv = K.shape[1]
    G = n_q // n_kv
    Lk = K.shape[0]
    vis = visible(q_pos, np.arange(Lk), window)
    out = np.zeros((n_q, D), dtype=np.float64)
    lse = np.full((n_q,), -np.inf, dtype=np.float64)
    if not vis.any():
        return out, lse
    for h in range(n_q):
        hk = h // G
        s = scale * (K[:, hk, :] @ q[h])
        s_vis = s[vis]
        m = s_vis.max()
        p = np.where(vis, np.exp(s - m), 0.0)
        l = p.sum()
        out[h] = (p @ V[:, hk, :]) / l
        lse[h] = m + np.log(l)
    return out, lse


def attn_decode(q, k_pool, v_pool, table, slots, seq_lens, scale: float, window: int = 0):
    """Decode attention: one query token per batch row, at position ``L - 1``.

    ``q``: uint16 ``[B][n_q][D]``; ``slots[b]``, ``seq_lens[b]`` = keys visible
    after the append (the new token sits at ``L - 1``, matching the decode loop's
    ``cur_pos = total_length - 1``).  Rows with slot 0 or ``L == 0`` are idle:
    zero output, ``lse = -inf``, and nothing is read.
    """
    B, n_q, D = q.shape
    out = np.zeros((B, n_q, D), dtype=np.float64)
    lse = np.full((B, n_q), -np.inf, dtype=np.float64)
    for b in range(B):
        s, L = int(slots[b]), int(seq_lens[b])
        if s == 0 or L == 0:
            continue
        K, V = gather_kv(k_pool, v_pool, table, s, L)
        out[b], lse[b] = attend_rows(bf16_bits_to_f64(q[b]), K, V, L - 1, scale, window)
    return out, lse


def attn_prefill(q, k_pool, v_pool, table, cu_seqlens, slots, start_pos, scale: float,
                 window: int = 0, q_is_f64: bool = False):
    """Packed varlen prefill attention reading K/V from the pages.

    Sequence ``n`` owns packed tokens ``cu_seqlens[n] .. cu_seqlens[n+1]-1``;
    its query ``i`` sits at position ``start_pos[n] + i`` and sees keys
    ``0 .. start_pos[n] + i`` of its own slot only (document-causal mask:
    [continuous-batching compare] flex_paged_attention.py,
    ``create_prefill_blockmask_no_paging``; sliding form in [moe-qwen3 compare]
    flex_gemma4_moe.py, ``_create_prefill_sliding_blockmask``).  The keys must
    already be in the pages.  Sequences in slot 0 produce zeros.
    """
    T, n_q, D = q.shape
    qf = q if q_is_f64 else bf16_bits_to_f64(q)
    out = np.zeros((T, n_q, D), dtype=np.float64)
    lse = np.full((T, n_q), -np.inf, dtype=np.float64)
    n_seqs = len(slots)
    for n in range(n_seqs):
        s = int(slots[n])
        t0, t1 = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        sp = 0 if start_pos is None else int(start_pos[n])
        if s == 0 or t1 == t0:
            continue
        K, V = gather_kv(k_pool, v_pool, table, s, sp + (t1 - t0))
        for t in range(t0, t1):
            qp = sp + (t - t0)
            out[t], lse[t] = attend_rows(qf[t], K[: qp + 1], V[: qp + 1], qp, scale, window)
    return out, lse
