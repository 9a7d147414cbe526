"""Seeded generators for decode and prefill cases (input generation only)."""

from __future__ import annotations

import dataclasses
import math

import numpy as np

# 0xFFFF is a bf16 NaN: any stray read of an unwritten row, of page 0 or of a
# page no slot owns shows up as NaN in an output.
SENTINEL_BITS = np.uint16(0xFFFF)
# V pools store each page's rows in groups of this many keys (storage shape only)
V_KEY_GROUP = 32

CONFIGS = {
    "tiny": dict(index=0, n_q=4, n_kv=2, head_dim=64, page_size=16, lengths=(37, 50),
                 max_slots=3, n_pages=16, scale=1.0 / 8.0, window=0),
    "qwen3_decode": dict(index=1, n_q=32, n_kv=8, head_dim=128, page_size=128, B=8,
                         max_slots=9, len_lo=64, len_hi=1024, layers=36, window=0),
    "llama_decode": dict(index=2, n_q=24, n_kv=8, head_dim=128, page_size=128, B=64,
                         max_slots=65, len_lo=128, len_hi=4096, idle_frac=0.10, window=0,
                         layers=2),
    # one GPU's share of llama_decode under 8-way tensor parallelism (kv heads
    # split across GPUs): 3 query heads over 1 kv head, the same rows and lengths
    "llama_decode_tp8_share": dict(index=2, n_q=3, n_kv=1, head_dim=128, page_size=128, B=64,
                                   max_slots=65, len_lo=128, len_hi=4096, idle_frac=0.10,
                                   window=0, layers=2),
    "qwen3_prefill": dict(index=3, n_q=32, n_kv=8, head_dim=128, page_size=128,
                          n_seqs=16, max_slots=17, len_lo=32, len_hi=512, eps=1e-6,
                          theta=1e6, layers=36),
    "gemma_mixed": dict(index=4, n_q=8, n_kv=2, page_size=64, B=64, max_slots=65,
                        len_lo=256, len_hi=1536, sliding_dim=256, window=512,
                        full_dim=512, layers=4),
    # Gemma-4-shaped prefill with its prologue: a sliding layer (head_dim 256,
    # window 512, theta 1e4, full rotary) and a full-attention layer (head_dim
    # 512, theta 1e6, 25 % rotary, K = V); v_norm on both.  Prompts up to 1024
    # tokens, so the window cuts the longer ones.
    "gemma_prefill": dict(index=5, n_q=8, n_kv=2, page_size=64, n_seqs=16, max_slots=17,
                          len_lo=128, len_hi=1024, eps=1e-6, sliding_dim=256, window=512,
                          sliding_theta=1e4, full_dim=512, full_theta=1e6, full_rotary=0.25),
    # Qwen3-shaped chunked prefill mixed with decode in one launch: 8 prompt
    # chunks of U[64,512] new tokens on cached prefixes of U[256,1024], and 56
    # decode rows (one new token on a cached U[64,1024]); the Qwen3 prologue.
    "qwen3_chunked_mixed": dict(index=6, n_q=32, n_kv=8, head_dim=128, page_size=128,
                                n_chunks=8, chunk_lo=64, chunk_hi=512, prefix_lo=256,
                                prefix_hi=1024, n_decode=56, ctx_lo=64, ctx_hi=1024,
                                max_slots=65, eps=1e-6, theta=1e6),
}


def rng_for(config_index: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(3407 + config_index + 1000 * salt))


def randn_bf16(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0):
    """N(mean, std) samples quantised to bf16 (round to nearest even), as bits."""
    x = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
         + np.float32(mean))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def split_tokens(lengths):
    """Prefix offsets ``[0, l0, l0+l1, ...]`` of packed sequences (int32)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _page_assignment(rng, slot_lengths: dict, page_size: int, pages_per_slot: int,
                     max_slots: int, spare_pages: int):
    """Random physical pages for each slot; unused pages stay unmapped.

    Returns ``(n_pages, table)``: page 0 is reserved and never mapped, the rest
    are a seeded random permutation handed out slot by slot.  ``spare_pages``
    extra pages exist that no slot owns.
    """
    need = {s: math.ceil(l / page_size) for s, l in slot_lengths.items()}
    total = sum(need.values())
    n_pages = 1 + total + spare_pages
    perm = rng.permutation(np.arange(1, n_pages, dtype=np.int32))
    table = np.full((max_slots, pages_per_slot), -1, dtype=np.int32)
    table[0, :] = 0
    k = 0
    for s in sorted(slot_lengths):
        table[s, : need[s]] = perm[k: k + need[s]]
        k += need[s]
    return n_pages, table


@dataclasses.dataclass
class DecodeCase:
    """One decode layer call.

    ``hist_k/hist_v``: per batch row, bf16 bits ``[L-1][n_kv][D]`` (history
    already in the cache before this step); ``k_new/v_new [B][n_kv][D]`` the
    new token's K/V (appended at position ``L-1``); ``q [B][n_q][D]``.
    Rows with ``seq_lens == 0`` are idle and use slot 0 in the append.
    """
    n_q: int
    n_kv: int
    head_dim: int
    page_size: int
    max_slots: int
    pages_per_slot: int
    n_pages: int
    table: np.ndarray
    slots: np.ndarray
    seq_lens: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    hist_k: list
    hist_v: list
    scale: float
    window: int

    @property
    def B(self):
        return len(self.slots)

    def append_slots(self):
        """Per row: the slot the new token is appended to (0 for idle rows)."""
        return np.where(self.seq_lens > 0, self.slots, 0).astype(np.int32)

    def append_pos(self):
        return np.maximum(self.seq_lens - 1, 0).astype(np.int32)

    def history_tokens(self):
        """Packed history for one append call: ``(k, v, slot, pos)``."""
        ks, vs, sl, ps = [], [], [], []
        for b in range(self.B):
            L = int(self.seq_lens[b])
            if L <= 1:
                continue
            ks.append(self.hist_k[b])
            vs.append(self.hist_v[b])
            sl.append(np.full(L - 1, self.slots[b], dtype=np.int32))
            ps.append(np.arange(L - 1, dtype=np.int32))
        if not ks:
            z = np.zeros((0, self.n_kv, self.head_dim), dtype=np.uint16)
            return z, z.copy(), np.zeros(0, np.int32), np.zeros(0, np.int32)
        return (np.concatenate(ks), np.concatenate(vs), np.concatenate(sl),
                np.concatenate(ps))

    def empty_pools(self):
        shape_k = (self.n_pages, self.n_kv, self.page_size, self.head_dim)
        gs = min(self.page_size, V_KEY_GROUP)
        shape_v = (self.n_pages, self.n_kv, self.page_size // gs, self.head_dim, gs)
        return (np.full(shape_k, SENTINEL_BITS, dtype=np.uint16),
                np.full(shape_v, SENTINEL_BITS, dtype=np.uint16))


def make_decode_case(n_q, n_kv, head_dim, page_size, lengths, max_slots, seed,
                     scale=None, window=0, slot_of_row=None, spare_pages=2,
                     pages_per_slot=None, with_history=True):
    """Build a decode case with the given per-row lengths (0 = idle row)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int32)
    B = len(lengths)
    if slot_of_row is None:
        slot_of_row = np.arange(1, B + 1, dtype=np.int32)
    slot_of_row = np.asarray(slot_of_row, dtype=np.int32)
    if pages_per_slot is None:
        pages_per_slot = max(1, math.ceil(max(int(lengths.max(initial=1)), 1) / page_size))
    slot_lengths = {int(slot_of_row[b]): int(lengths[b]) for b in range(B)
                    if lengths[b] > 0}
    n_pages, table = _page_assignment(rng, slot_lengths, page_size, pages_per_slot,
                                      max_slots, spare_pages)
    q = randn_bf16(rng, (B, n_q, head_dim))
    k_new = randn_bf16(rng, (B, n_kv, head_dim))
    v_new = randn_bf16(rng, (B, n_kv, head_dim))
    hist_k, hist_v = [], []
    for b in range(B):
        L = int(lengths[b])
        n = max(L - 1, 0) if with_history else 0
        hist_k.append(randn_bf16(rng, (n, n_kv, head_dim)))
        hist_v.append(randn_bf16(rng, (n, n_kv, head_dim)))
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeCase(n_q, n_kv, head_dim, page_size, max_slots, pages_per_slot, n_pages,
                      table, slot_of_row, lengths, q, k_new, v_new, hist_k, hist_v,
                      float(scale), int(window))


@dataclasses.dataclass
class PrefillCase:
    """One packed prefill layer call.

    ``q [T][n_q][D]``, ``k/v [T][n_kv][D]`` raw projections; sequence ``n``
    occupies packed tokens ``cu_seqlens[n]..cu_seqlens[n+1]-1`` at positions
    ``start_pos[n] + i`` of slot ``slots[n]``.  ``prefix_k/prefix_v[n]`` hold
    the cached prefix (positions ``0..start_pos[n]-1``) already in the pages.
    """
    n_q: int
    n_kv: int
    head_dim: int
    page_size: int
    max_slots: int
    pages_per_slot: int
    n_pages: int
    table: np.ndarray
    slots: np.ndarray
    cu_seqlens: np.ndarray
    start_pos: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_norm_w: np.ndarray
    k_norm_w: np.ndarray
    prefix_k: list
    prefix_v: list
    scale: float
    window: int
    eps: float
    theta: float

    @property
    def T(self):
        return int(self.cu_seqlens[-1])

    def token_slots(self):
        out = np.zeros(self.T, dtype=np.int32)
        for n in range(len(self.slots)):
            out[self.cu_seqlens[n]: self.cu_seqlens[n + 1]] = self.slots[n]
        return out

    def token_pos(self):
        out = np.zeros(self.T, dtype=np.int32)
        for n in range(len(self.slots)):
            a, b = int(self.cu_seqlens[n]), int(self.cu_seqlens[n + 1])
            out[a:b] = self.start_pos[n] + np.arange(b - a, dtype=np.int32)
        return out

    def prefix_tokens(self):
        ks, vs, sl, ps = [], [], [], []
        for n in range(len(self.slots)):
            P = int(self.start_pos[n])
            if P == 0:
                continue
            ks.append(self.prefix_k[n])
            vs.append(self.prefix_v[n])
            sl.append(np.full(P, self.slots[n], dtype=np.int32))
            ps.append(np.arange(P, dtype=np.int32))
        if not ks:
            z = np.zeros((0, self.n_kv, self.head_dim), dtype=np.uint16)
            return z, z.copy(), np.zeros(0, np.int32), np.zeros(0, np.int32)
        return (np.concatenate(ks), np.concatenate(vs), np.concatenate(sl),
                np.concatenate(ps))

    def empty_pools(self):
        shape_k = (self.n_pages, self.n_kv, self.page_size, self.head_dim)
        gs = min(self.page_size, V_KEY_GROUP)
        shape_v = (self.n_pages, self.n_kv, self.page_size // gs, self.head_dim, gs)
        return (np.full(shape_k, SENTINEL_BITS, dtype=np.uint16),
                np.full(shape_v, SENTINEL_BITS, dtype=np.uint16))


def make_prefill_case(n_q, n_kv, head_dim, page_size, lengths, seed, start_pos=None,
                      slots=None, max_slots=None, scale=None, window=0, eps=1e-6,
                      theta=1e6, spare_pages=2, pages_per_slot=None, norm_std=0.1):
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int32)
    n = len(lengths)
    if start_pos is None:
        start_pos = np.zeros(n, dtype=np.int32)
    start_pos = np.asarray(start_pos, dtype=np.int32)
    if slots is None:
        slots = np.arange(1, n + 1, dtype=np.int32)
    slots = np.asarray(slots, dtype=np.int32)
    if max_slots is None:
        max_slots = int(slots.max(initial=0)) + 1
    total = lengths + start_pos
    if pages_per_slot is None:
        pages_per_slot = max(1, math.ceil(int(total.max(initial=1)) / page_size))
    slot_lengths = {int(slots[i]): int(total[i]) for i in range(n)
                    if slots[i] != 0 and total[i] > 0}
    n_pages, table = _page_assignment(rng, slot_lengths, page_size, pages_per_slot,
                                      max_slots, spare_pages)
    cu = split_tokens(lengths)
    T = int(cu[-1])
    q = randn_bf16(rng, (T, n_q, head_dim))
    k = randn_bf16(rng, (T, n_kv, head_dim))
    v = randn_bf16(rng, (T, n_kv, head_dim))
    qw = randn_bf16(rng, (head_dim,), mean=1.0, std=norm_std)
    kw = randn_bf16(rng, (head_dim,), mean=1.0, std=norm_std)
    pk, pv = [], []
    for i in range(n):
        P = int(start_pos[i])
        pk.append(randn_bf16(rng, (P, n_kv, head_dim)))
        pv.append(randn_bf16(rng, (P, n_kv, head_dim)))
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PrefillCase(n_q, n_kv, head_dim, page_size, max_slots, pages_per_slot, n_pages,
                       table, slots, cu, start_pos, q, k, v, qw, kw, pk, pv, float(scale),
                       int(window), float(eps), float(theta))


def config_lengths(name: str, salt: int = 0):
    """Per-row lengths (and slot mapping) of a named workload, seeded."""
    c = CONFIGS[name]
    rng = rng_for(c["index"], salt)
    if name == "tiny":
        return np.asarray(c["lengths"], dtype=np.int32), np.array([1, 2], dtype=np.int32)
    if name in ("qwen3_decode",):
        L = rng.integers(c["len_lo"], c["len_hi"] + 1, size=c["B"]).astype(np.int32)
        return L, np.arange(1, c["B"] + 1, dtype=np.int32)
    if name in ("llama_decode", "llama_decode_tp8_share"):
        B = c["B"]
        L = rng.integers(c["len_lo"], c["len_hi"] + 1, size=B).astype(np.int32)
        idle = rng.choice(B, size=int(round(c["idle_frac"] * B)), replace=False)
        L[idle] = 0
        slots = rng.permutation(np.arange(1, B + 1, dtype=np.int32))
        return L, slots
    if name == "gemma_mixed":
        L = rng.integers(c["len_lo"], c["len_hi"] + 1, size=c["B"]).astype(np.int32)
        return L, np.arange(1, c["B"] + 1, dtype=np.int32)
    if name in ("qwen3_prefill", "gemma_prefill"):
        L = rng.integers(c["len_lo"], c["len_hi"] + 1, size=c["n_seqs"]).astype(np.int32)
        return L, np.arange(1, c["n_seqs"] + 1, dtype=np.int32)
    raise KeyError(name)


def chunked_mixed_rows(name: str = "qwen3_chunked_mixed"):
    """(new tokens, cached prefix, slots) per sequence of the mixed launch:
    the prompt chunks first, then the decode rows (one new token each)."""
    c = CONFIGS[name]
    rng = rng_for(c["index"])
    n1, n2 = c["n_chunks"], c["n_decode"]
    new = np.concatenate([rng.integers(c["chunk_lo"], c["chunk_hi"] + 1, size=n1),
                          np.ones(n2, dtype=np.int64)]).astype(np.int32)
    prefix = np.concatenate([rng.integers(c["prefix_lo"], c["prefix_hi"] + 1, size=n1),
                             rng.integers(c["ctx_lo"], c["ctx_hi"], size=n2)]).astype(np.int32)
    return new, prefix, np.arange(1, n1 + n2 + 1, dtype=np.int32)


def prefill_page_table(page_size, lengths, start_pos, slots, max_slots, seed, pages_per_slot,
                       spare_pages=2):
    """(n_pages, table) for sequences of ``start_pos + lengths`` keys on a
    seeded random page permutation (no token data drawn)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    total = np.asarray(lengths, dtype=np.int64) + np.asarray(start_pos, dtype=np.int64)
    slot_lengths = {int(slots[i]): int(total[i]) for i in range(len(total))
                    if slots[i] != 0 and total[i] > 0}
    return _page_assignment(rng, slot_lengths, page_size, pages_per_slot, max_slots,
                            spare_pages)
