#!/usr/bin/env python3
"""Throughput bench of the paged KV-cache attention path on one MI355X.

Default workload (``llama_decode``): a Llama-3.2-3B-shaped decode step -- 64
slots (10 % idle, length 0), 24 query / 8 kv heads, head_dim 128, page 128,
context lengths U[128, 4096], two layers with their own K/V pools (together
above the 256 MB Infinity Cache).  One step = for every layer: the split-K
decode kernel, which appends each row's new token's K/V into its page and
then attends (+ the in-kernel log-sum-exp merge).  This is the largest
single-GPU decode configuration; it gives the JSON line's ``value`` and
``roofline``.  The other decode workloads -- ``qwen3_decode`` (8 rows of a
Qwen3-4B step, 36 layers) and ``gemma_mixed`` (64 rows, one Gemma-4 sliding
head_dim-256 and one full head_dim-512 layer per step) and
``llama_decode_tp8_share`` (one GPU's share of the Llama step under 8-way
tensor parallelism: 3 query heads over 1 kv head, the same rows; its kernel
instance is also the Llama step's, so its counter traffic comes from a run of
it alone) -- are
reported under ``extra_decode`` with their own rooflines, and the Qwen3-4B chunked prefill
(16 prompts U[32, 512], fused q/k RMSNorm + RoPE + append prologue, then MFMA
prefill attention, 36 layers) under ``prefill``.  ``extra_prefill`` adds the
Gemma-4-shaped prefill layers with their prologue (sliding head_dim 256 and
full head_dim 512) and a Qwen3-shaped launch of prompt chunks on cached
prefixes mixed with decode rows: per call, a whole layer and the attention
with the fused q transform, against both rooflines.

Every phase is captured once in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: inputs are resident in HBM before the timed region, and the timed
region is bracketed by torch.cuda.synchronize().  Kernel durations for the
rooflines come from HIP events around graphs of back-to-back calls of one
kernel, recorded on the stream the kernels run on.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this path runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn HBM GB/s (% peak) + prefill attn TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_attention_pagetable_amd", "csrc")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def contiguous_table(table):
    """The same page table with each slot's mapped logical pages renumbered to
    consecutive physical pages (slot by slot, from page 1): the layout of a
    cache whose pages were granted in order, to time the page indirection."""
    t = table.copy()
    rows, cols = np.nonzero(t[1:] > 0)
    t[1:][rows, cols] = np.arange(1, len(rows) + 1, dtype=t.dtype)
    return t


class DecodeWorkload:
    """Per-layer pools with history already appended; one shared page table."""

    def __init__(self, name, device="cuda", contiguous=False):
        import torch

        import paged_kv_attention_pagetable_amd as pkv
        from synth import CONFIGS, config_lengths, make_decode_case
        from synth.device import DeviceRandom

        self.pkv, self.torch = pkv, torch
        c = CONFIGS[name]
        self.name, self.c = name, c
        lengths, slots = config_lengths(name)
        ps = c["page_size"]
        pps = -(-c["len_hi"] // ps)
        if name == "gemma_mixed":
            kinds = [(c["sliding_dim"], c["window"]), (c["full_dim"], 0)] * c["layers"]
        else:
            kinds = [(c["head_dim"], c.get("window", 0))] * c["layers"]
        base = make_decode_case(c["n_q"], c["n_kv"], kinds[0][0], ps, lengths,
                                max_slots=c["max_slots"], seed=3407 + c["index"],
                                slot_of_row=slots, pages_per_slot=pps, with_history=False)
        if contiguous:
            base.table = contiguous_table(base.table)
        self.case = base
        self.hint = c["len_hi"]
        dev = device
        self.table = torch.from_numpy(base.table).to(dev)
        self.slots = torch.from_numpy(base.slots).to(dev)
        self.seq_lens = torch.from_numpy(base.seq_lens).to(dev)
        self.aslots = torch.from_numpy(base.append_slots()).to(dev)
        self.apos = torch.from_numpy(base.append_pos()).to(dev)
        hist_slot, hist_pos = [], []
        for b in range(base.B):
            n = max(int(base.seq_lens[b]) - 1, 0)
            hist_slot.append(np.full(n, base.slots[b], np.int32))
            hist_pos.append(np.arange(n, dtype=np.int32))
        hs = torch.from_numpy(np.concatenate(hist_slot)).to(dev)
        hp = torch.from_numpy(np.concatenate(hist_pos)).to(dev)
        rnd = DeviceRandom(3407 + 100 * c["index"], dev)
        B, n_q, n_kv = base.B, c["n_q"], c["n_kv"]
        self.layers = []
        for D, window in kinds:
            kp, vp = pkv.new_pools(base.n_pages, n_kv, ps, D, dev, fill=-1)
            pkv.append(rnd.bf16((hs.numel(), n_kv, D)), rnd.bf16((hs.numel(), n_kv, D)), hs, hp,
                       self.table, kp, vp)
            ws_bytes = pkv.decode_workspace_size(B, n_q, n_kv, D, self.hint, window)
            self.layers.append(dict(
                D=D, window=window, kp=kp, vp=vp, q=rnd.bf16((B, n_q, D)),
                k_new=rnd.bf16((B, n_kv, D)), v_new=rnd.bf16((B, n_kv, D)),
                out=torch.empty((B, n_q, D), dtype=torch.bfloat16, device=dev),
                ws=pkv.new_decode_workspace(ws_bytes, dev),
                scale=1.0 / math.sqrt(D)))
        torch.cuda.synchronize()
        self.n_calls = len(self.layers)

    def attn(self, ly, fused_append=False):
        self.pkv.attn_decode(ly["q"], self.slots, self.seq_lens, self.table, ly["kp"], ly["vp"],
                             scale=ly["scale"], window=ly["window"], max_seq_len_hint=self.hint,
                             out=ly["out"], workspace=ly["ws"],
                             k_new=ly["k_new"] if fused_append else None,
                             v_new=ly["v_new"] if fused_append else None)

    def step(self):
        """Every layer: append the new token's K/V, then attend (one fused kernel)."""
        for ly in self.layers:
            self.attn(ly, fused_append=True)

    def attn_only(self):
        for ly in self.layers:
            self.attn(ly)

    def step_kind(self, D):
        """The step's calls of one head_dim only (per-layer-kind timing)."""
        for ly in self.layers:
            if ly["D"] == D:
                self.attn(ly, fused_append=True)

    def attn_bytes(self, ly):
        """Algorithmic HBM bytes of one attention call: visible K/V rows, Q, O, page ids."""
        c, case = self.c, self.case
        L = case.seq_lens.astype(np.int64)
        if ly["window"] > 0:
            L = np.minimum(L, ly["window"])
        kv = int(L.sum()) * c["n_kv"] * ly["D"] * 2 * 2
        active = int((case.seq_lens > 0).sum())
        qo = active * c["n_q"] * ly["D"] * 2 * 2
        pages = int(np.ceil(L / case.page_size).sum()) * 4
        return kv + qo + pages

    def append_bytes(self, ly):
        active = int((self.case.seq_lens > 0).sum())
        return active * self.c["n_kv"] * ly["D"] * 2 * 2 * 2   # read + write, K and V

    def describe(self):
        c, case = self.c, self.case
        d = dict(workload=self.name, batch=int(case.B), active=int((case.seq_lens > 0).sum()),
                 n_q=c["n_q"], n_kv=c["n_kv"], page_size=c["page_size"],
                 layers=len(self.layers), head_dims=sorted({ly["D"] for ly in self.layers}),
                 context=f"U[{c['len_lo']},{c['len_hi']}]",
                 mean_context=float(case.seq_lens[case.seq_lens > 0].mean()))
        if any(ly["window"] for ly in self.layers):
            d["window"] = max(ly["window"] for ly in self.layers)
        return d


class PrefillWorkload:
    def __init__(self, device="cuda", contiguous=False):
        import torch

        import paged_kv_attention_pagetable_amd as pkv
        from synth import CONFIGS, config_lengths, make_prefill_case
        from synth.device import DeviceRandom

        self.pkv, self.torch = pkv, torch
        c = CONFIGS["qwen3_prefill"]
        self.c = c
        lengths, slots = config_lengths("qwen3_prefill")
        ps, D = c["page_size"], c["head_dim"]
        case = make_prefill_case(c["n_q"], c["n_kv"], D, ps, lengths, seed=3407 + c["index"],
                                 slots=slots, max_slots=c["max_slots"],
                                 pages_per_slot=-(-c["len_hi"] // ps))
        if contiguous:
            case.table = contiguous_table(case.table)
        self.case = case
        dev = device
        self.table = torch.from_numpy(case.table).to(dev)
        self.slots = torch.from_numpy(case.slots).to(dev)
        self.cu = torch.from_numpy(case.cu_seqlens).to(dev)
        self.start = torch.from_numpy(case.start_pos).to(dev)
        self.cos, self.sin = pkv.rope_table(c["len_hi"] + 1, D, c["theta"], dev)
        rnd = DeviceRandom(3407 + 100 * c["index"], dev)
        T = case.T
        self.layers = []
        for _ in range(c["layers"]):
            kp, vp = pkv.new_pools(case.n_pages, c["n_kv"], ps, D, dev, fill=-1)
            self.layers.append(dict(
                kp=kp, vp=vp, q=rnd.bf16((T, c["n_q"], D)), k=rnd.bf16((T, c["n_kv"], D)),
                v=rnd.bf16((T, c["n_kv"], D)), qw=rnd.bf16((D,), 1.0, 0.1),
                kw=rnd.bf16((D,), 1.0, 0.1),
                out=torch.empty((T, c["n_q"], D), dtype=torch.bfloat16, device=dev)))
        torch.cuda.synchronize()
        self.n_calls = len(self.layers)
        self.scale = 1.0 / math.sqrt(D)

    def _call(self, ly, with_prologue):
        pro = None
        if with_prologue:
            pro = dict(q_norm_w=ly["qw"], k_norm_w=ly["kw"], eps=self.c["eps"], cos=self.cos,
                       sin=self.sin, k=ly["k"], v=ly["v"])
        self.pkv.attn_prefill(ly["q"], self.cu, self.slots, self.table, ly["kp"], ly["vp"],
                              scale=self.scale, start_pos=self.start,
                              max_seqlen_q_hint=self.c["len_hi"], prologue=pro, out=ly["out"])

    def _call_q_only(self, ly):
        """Attention with the fused q norm + RoPE, keys already in the pages."""
        pro = dict(q_norm_w=ly["qw"], eps=self.c["eps"], cos=self.cos, sin=self.sin)
        self.pkv.attn_prefill(ly["q"], self.cu, self.slots, self.table, ly["kp"], ly["vp"],
                              scale=self.scale, start_pos=self.start,
                              max_seqlen_q_hint=self.c["len_hi"], prologue=pro, out=ly["out"])

    def step(self):
        for ly in self.layers:
            self._call(ly, True)

    def attn_only(self):
        for ly in self.layers:
            self._call(ly, False)

    def attn_fused_q(self):
        for ly in self.layers:
            self._call_q_only(ly)

    def flops_per_call(self):
        """Causal attention FLOPs: 2 (QK^T) + 2 (PV) per visible (query, key) pair."""
        L = np.diff(self.case.cu_seqlens).astype(np.int64)
        c = self.c
        return int((2 * 2 * c["head_dim"] * c["n_q"] * L * (L + 1) // 2).sum())

    def attn_bytes(self):
        """Compulsory HBM bytes of one attention call: q read and out written once
        ([T][n_q][D] bf16 each), every sequence's K and V rows (its cached
        prefix and its prompt) read once, and its page ids."""
        c, case = self.c, self.case
        L = np.diff(case.cu_seqlens).astype(np.int64)
        keys = L + np.asarray(case.start_pos, dtype=np.int64)
        qo = case.T * c["n_q"] * c["head_dim"] * 2 * 2
        kv = int(keys.sum()) * c["n_kv"] * c["head_dim"] * 2 * 2
        pages = int(np.ceil(keys / c["page_size"]).sum()) * 4
        return qo + kv + pages

    def prologue_bytes(self):
        """Bytes of the prologue kernel: k and v rows read and written (q's norm
        and rotation run inside the attention kernel, which reads q anyway)."""
        c, T = self.c, self.case.T
        rows = T * 2 * c["n_kv"]
        return rows * c["head_dim"] * 2 * 2   # read + write

    def describe(self):
        c, case = self.c, self.case
        return dict(workload="qwen3_prefill", prompts=len(case.slots), tokens=case.T,
                    n_q=c["n_q"], n_kv=c["n_kv"], head_dim=c["head_dim"],
                    page_size=c["page_size"], layers=c["layers"],
                    lengths=f"U[{c['len_lo']},{c['len_hi']}]", prologue="rmsnorm+rope theta 1e6")


class _PrefillLayers:
    """Copies of one prefill layer shape (own pools, q, k, v, out each), for
    the extra prefill workloads: a whole layer is the prologue + attention
    call, and the attention alone is the call with only the q transform
    (keys already appended by an earlier layer call)."""

    N_COPIES = 4   # layer calls per captured graph

    def __init__(self, pkv, rnd, dev, n_q, n_kv, D, ps, n_pages, T, theta, max_pos, eps,
                 fraction=1.0, k_eq_v=False, prefill_pools=False):
        import torch
        self.pkv, self.D, self.eps = pkv, D, eps
        self.cos, self.sin = pkv.rope_table(max_pos, D, theta, dev, rotary_fraction=fraction)
        self.copies = []
        for _ in range(self.N_COPIES):
            kp, vp = pkv.new_pools(n_pages, n_kv, ps, D, dev, fill=-1)
            if prefill_pools:   # cached prefixes: random rows on every page
                kp.copy_(rnd.bf16(tuple(kp.shape)))
                vp.copy_(rnd.bf16(tuple(vp.shape)))
            k = rnd.bf16((T, n_kv, D))
            self.copies.append(dict(
                kp=kp, vp=vp, q=rnd.bf16((T, n_q, D)), k=k,
                v=k if k_eq_v else rnd.bf16((T, n_kv, D)), qw=rnd.bf16((D,), 1.0, 0.1),
                kw=rnd.bf16((D,), 1.0, 0.1),
                out=torch.empty((T, n_q, D), dtype=torch.bfloat16, device=dev)))

    def run(self, w, with_kv, v_norm, window):
        for ly in self.copies:
            pro = dict(q_norm_w=ly["qw"], eps=self.eps, cos=self.cos, sin=self.sin)
            if with_kv:
                pro.update(k_norm_w=ly["kw"], k=ly["k"], v=ly["v"], v_norm=v_norm)
            self.pkv.attn_prefill(ly["q"], w.cu, w.slots, w.table, ly["kp"], ly["vp"],
                                  scale=1.0 / math.sqrt(self.D), window=window,
                                  start_pos=w.start, max_seqlen_q_hint=w.hint, prologue=pro,
                                  out=ly["out"])


def _prefill_flops(new, prefix, n_q, D, window):
    """Attention FLOPs (2 for QK^T and 2 for PV per visible query-key pair) of
    sequences of ``new`` queries after ``prefix`` cached keys."""
    tot = 0
    for L, P in zip(np.asarray(new, dtype=np.int64), np.asarray(prefix, dtype=np.int64)):
        keys = P + np.arange(1, L + 1)
        if window > 0:
            keys = np.minimum(keys, window)
        tot += int(keys.sum())
    return 4 * D * n_q * tot


def _prefill_bytes(new, prefix, n_q, n_kv, D, ps):
    """Compulsory bytes of one attention call: q read and out written once,
    each sequence's K and V rows (prefix and new) read once, its page ids."""
    new = np.asarray(new, dtype=np.int64)
    keys = new + np.asarray(prefix, dtype=np.int64)
    return (int(new.sum()) * n_q * D * 2 * 2 + int(keys.sum()) * n_kv * D * 2 * 2
            + int(np.ceil(keys / ps).sum()) * 4)


class GemmaPrefillWorkload:
    """Gemma-4-shaped prefill with its prologue: a sliding layer and a
    full-attention layer (head_dim 256 and 512), see synth's gemma_prefill."""

    def __init__(self, device="cuda"):
        import torch

        import paged_kv_attention_pagetable_amd as pkv
        from synth import CONFIGS, config_lengths, prefill_page_table, split_tokens
        from synth.device import DeviceRandom
        c = self.c = CONFIGS["gemma_prefill"]
        self.new, slots = config_lengths("gemma_prefill")
        self.prefix = np.zeros_like(self.new)
        ps = c["page_size"]
        n_pages, table = prefill_page_table(ps, self.new, self.prefix, slots, c["max_slots"],
                                            3407 + c["index"], -(-c["len_hi"] // ps))
        self.table = torch.from_numpy(table).to(device)
        self.slots = torch.from_numpy(slots).to(device)
        self.cu = torch.from_numpy(split_tokens(self.new)).to(device)
        self.start = torch.from_numpy(self.prefix).to(device)
        self.hint = c["len_hi"]
        T = int(self.new.sum())
        rnd = DeviceRandom(3407 + 100 * c["index"], device)
        self.kinds = {
            c["sliding_dim"]: (_PrefillLayers(pkv, rnd, device, c["n_q"], c["n_kv"],
                                              c["sliding_dim"], ps, n_pages, T,
                                              c["sliding_theta"], c["len_hi"] + 1, c["eps"]),
                               c["window"]),
            c["full_dim"]: (_PrefillLayers(pkv, rnd, device, c["n_q"], c["n_kv"], c["full_dim"],
                                           ps, n_pages, T, c["full_theta"], c["len_hi"] + 1,
                                           c["eps"], fraction=c["full_rotary"], k_eq_v=True),
                            0),
        }
        torch.cuda.synchronize()

    def layer(self, D):
        lay, window = self.kinds[D]
        lay.run(self, True, True, window)

    def attn_fused_q(self, D):
        lay, window = self.kinds[D]
        lay.run(self, False, True, window)

    def flops(self, D):
        return _prefill_flops(self.new, self.prefix, self.c["n_q"], D, self.kinds[D][1])

    def attn_bytes(self, D):
        c = self.c
        return _prefill_bytes(self.new, self.prefix, c["n_q"], c["n_kv"], D, c["page_size"])

    def describe(self):
        c = self.c
        return dict(workload="gemma_prefill", prompts=len(self.new), tokens=int(self.new.sum()),
                    n_q=c["n_q"], n_kv=c["n_kv"], page_size=c["page_size"],
                    lengths=f"U[{c['len_lo']},{c['len_hi']}]",
                    layers="sliding D 256 (window 512, theta 1e4) + full D 512 (theta 1e6, "
                           "25 % rotary, K = V); v_norm")


class ChunkedMixedWorkload:
    """Qwen3-shaped prompt chunks on cached prefixes and decode rows in one
    prefill launch with the Qwen3 prologue, see synth's qwen3_chunked_mixed."""

    def __init__(self, device="cuda"):
        import torch

        import paged_kv_attention_pagetable_amd as pkv
        from synth import CONFIGS, chunked_mixed_rows, prefill_page_table, split_tokens
        from synth.device import DeviceRandom
        c = self.c = CONFIGS["qwen3_chunked_mixed"]
        self.new, self.prefix, slots = chunked_mixed_rows()
        ps, D = c["page_size"], c["head_dim"]
        total = self.new + self.prefix
        n_pages, table = prefill_page_table(ps, self.new, self.prefix, slots, c["max_slots"],
                                            3407 + c["index"], -(-int(total.max()) // ps))
        self.table = torch.from_numpy(table).to(device)
        self.slots = torch.from_numpy(slots).to(device)
        self.cu = torch.from_numpy(split_tokens(self.new)).to(device)
        self.start = torch.from_numpy(self.prefix).to(device)
        self.hint = c["chunk_hi"]
        T = int(self.new.sum())
        rnd = DeviceRandom(3407 + 100 * c["index"], device)
        self.lay = _PrefillLayers(pkv, rnd, device, c["n_q"], c["n_kv"], D, ps, n_pages, T,
                                  c["theta"], int(total.max()) + 1, c["eps"], prefill_pools=True)
        torch.cuda.synchronize()

    def layer(self):
        self.lay.run(self, True, False, 0)

    def attn_fused_q(self):
        self.lay.run(self, False, False, 0)

    def flops(self):
        return _prefill_flops(self.new, self.prefix, self.c["n_q"], self.c["head_dim"], 0)

    def attn_bytes(self):
        c = self.c
        return _prefill_bytes(self.new, self.prefix, c["n_q"], c["n_kv"], c["head_dim"],
                              c["page_size"])

    def describe(self):
        c = self.c
        return dict(workload="qwen3_chunked_mixed", chunks=c["n_chunks"],
                    chunk=f"U[{c['chunk_lo']},{c['chunk_hi']}]",
                    prefix=f"U[{c['prefix_lo']},{c['prefix_hi']}]", decode_rows=c["n_decode"],
                    decode_context=f"U[{c['ctx_lo']},{c['ctx_hi']})", tokens=int(self.new.sum()),
                    n_q=c["n_q"], n_kv=c["n_kv"], head_dim=c["head_dim"],
                    page_size=c["page_size"], prologue="rmsnorm+rope theta 1e6")


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------

def reserve_timing(wl, calls=16, reps=8):
    """Device-side page reservation (pkv_pt_device_reserve) for the decode batch:
    us per call when every row with a slot takes one new page.  The state comes
    from the library's host allocator; it is restored before each timed replay of
    a graph of `calls` reserves (call i grows each row to i more pages).  Also
    the device erase (pkv_pt_device_erase) of the same rows' slots."""
    import torch
    pkv, case = wl.pkv, wl.case
    ps = case.page_size
    slots = [int(s) for s in case.slots]
    lens = [int(L) for L in case.seq_lens]
    pps = -(-max(lens + [1]) // ps) + calls + 1
    alloc = pkv.PageAllocator(case.B * pps + 2, ps, case.max_slots)
    got = [alloc.allocate() for _ in range(case.max_slots - 1)]
    for s, L in zip(slots, lens):
        if s > 0 and L > 0:
            alloc.reserve(s, L)
    st = alloc.to_device(pps)
    saved = [t.clone() for t in (st.table, st.free_pages, st.free_count, st.capacity)]
    cap = st.capacity.cpu()
    d_slots = torch.tensor(slots, dtype=torch.int32, device="cuda")
    d_lens = [torch.tensor([int(cap[s]) + i * ps + 1 if s > 0 else 0 for s in slots],
                           dtype=torch.int32, device="cuda") for i in range(calls)]

    def restore():
        for t, t0 in zip((st.table, st.free_pages, st.free_count, st.capacity), saved):
            t.copy_(t0)

    def run():
        for ln in d_lens:
            st.reserve(d_slots, ln)

    run()
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    times = []
    for _ in range(reps):
        restore()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / calls * 1e3)
    assert int(st.status.item()) == 0, "device reserve reported a failure"
    # the erase of every row's slot (pages back on the free stack): a graph of
    # `calls` erases, each on its own copy of the allocator state
    copies = [alloc.to_device(pps) for _ in range(calls)]
    saved_c = [[t.clone() for t in (c.table, c.free_pages, c.free_count, c.capacity)]
               for c in copies]

    def restore_copies():
        for c, sv in zip(copies, saved_c):
            for t, t0 in zip((c.table, c.free_pages, c.free_count, c.capacity), sv):
                t.copy_(t0)

    torch.cuda.synchronize()
    ge = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ge):
        for c in copies:
            c.erase(d_slots)
    erase_times = []
    for _ in range(reps):
        restore_copies()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ge.replay()
        b.record()
        torch.cuda.synchronize()
        erase_times.append(a.elapsed_time(b) / calls * 1e3)
    st = copies[-1]
    assert int(st.status.item()) == 0, "device erase reported a failure"
    assert int(st.capacity.sum().item()) == 0
    del got
    return dict(us_per_call=round(float(np.median(times)), 3), rows=len(slots),
                pages_per_call=sum(1 for s in slots if s > 0),
                kernel="device page reserve (pkv_pt_device_reserve, one workgroup)",
                erase_us_per_call=round(float(np.median(erase_times)), 3),
                erase_pages=int(sum(-(-int(cap[s]) // ps) for s in slots if s > 0)))


def capture(fn):
    import torch
    fn()                       # eager warm-up: no allocation happens inside fn
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps, warmup):
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps   # ms per replay


def time_graph_each(g, reps):
    """Per-replay times (ms) of `reps` back-to-back replays, one event pair each."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for s, e in ev:
        s.record()
        g.replay()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _pmc_record(part):
    path = os.path.join(PROFILES, f"{part}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha({**PMC_PARTS, **PMC_SOLO_PARTS}[part][1]):
        return None   # kernel changed since the counters were taken
    return rec


def pmc_traffic(part, instance=None):
    """HBM bytes per call from a committed rocprofv3 PMC summary, if current:
    of the part's counted kernels, or of the kernel whose name starts with
    ``instance`` (a template name and its first arguments, e.g.
    ``decode_dimsplit_kernel<512``; one instance ran per such prefix)."""
    rec = _pmc_record(part)
    if rec is None:
        return None
    if instance is None:
        return rec.get("hbm_bytes_per_call")
    ks = [k for name, k in rec.get("kernels", {}).items()
          if name.startswith(instance) and name[len(instance):len(instance) + 1] in (">", ",")]
    return ks[0]["fetch_bytes"] + ks[0]["write_bytes"] if len(ks) == 1 else None


# ----------------------------------------------------------------------------
# rocprofv3 summaries (kernel durations, HBM counters)
# ----------------------------------------------------------------------------

def _kernel_rows(db_path):
    import sqlite3
    db = sqlite3.connect(db_path)
    return db.execute("select name, duration from kernels").fetchall()


def summarize_trace(db_path, out_path, command=""):
    rows = _kernel_rows(db_path)
    stats = {}
    for name, dur in rows:
        stats.setdefault(name, []).append(dur / 1e3)
    lines = ["# rocprofv3 kernel trace summary", "",
             f"Command: `{command}`" if command else "", "",
             "| kernel | dispatches | avg us | min us | max us | total us |",
             "|---|---|---|---|---|---|"]
    for name, d in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        if "pkv::" not in name and "copy" not in name:
            continue
        short = name.replace("void ", "").replace("pkv::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {short} | {len(d)} | {np.mean(d):.3f} | {np.min(d):.3f} | "
                     f"{np.max(d):.3f} | {np.sum(d):.1f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _pmc_per_kernel(db_path, counter):
    """Counter values per dispatch, grouped by kernel name."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, dispatch_id, sum(counter_value) from pmc_events "
                      "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
    acc = {}
    for name, _, v in rows:
        acc.setdefault(name, []).append(v)
    return acc


DECODE_SRC = ["decode.hip", "pkv_device.h", "pkv_internal.h"]
PREFILL_SRC = ["prefill.hip", "pkv_device.h", "pkv_internal.h"]
PMC_PARTS = {
    # part: (substrings a counted kernel instance's name contains, sources whose
    # hash the record keeps).  The three decode workloads run distinct
    # instances (Llama: 4-wave key split whose split 0 writes the new V;
    # Qwen3: the plain 4-wave key split (the main counter runs leave the
    # tensor-parallel share, which runs it too, out); Gemma: the head_dim-256 and -512 dim-split
    # kernels, one call of each per step).
    "decode_llama_decode": (("decode_keysplit_kernel<128, 4, true>",), DECODE_SRC),
    "decode_qwen3_decode": (("decode_keysplit_kernel<128, 4, false>",), DECODE_SRC),
    "decode_gemma_mixed": (("decode_dimsplit_kernel<",), DECODE_SRC),
    # prefill attention without the q transform (keys appended beforehand):
    # the instance of q mode 0
    "prefill_qwen3_prefill": (("prefill_kernel<", ", 0>"), PREFILL_SRC),
    # prefill attention with the fused q norm + RoPE: with 4 query heads per
    # kv head, the instance whose rotary rows are staged in LDS (q mode 2)
    "prefill_fused_q_qwen3_prefill": (("prefill_kernel<", ", 2>"), PREFILL_SRC),
}
# Parts summarized only from counter runs named for them (``--pmc-parts``):
# the tensor-parallel share, whose kernel instance the Llama step runs too
# (from bench.py --workload <name> --no-extra-decode --no-prefill), and the
# Gemma-4 prefill layers (from a run with the extra prefill records, which the
# main counter runs leave out: its mixed launch runs the Qwen3 fused-q
# instance).
PMC_SOLO_PARTS = {
    # one GPU's share of the Llama step at 8-way tensor parallelism: a
    # head_dim-128 key split like the Llama and Qwen3 calls
    "decode_llama_decode_tp8_share": (("decode_keysplit_kernel<128, ",), DECODE_SRC),
    # the Gemma-4 prefill layers of extra_prefill (head_dim 256 and 512, the q
    # transform loading its rotary rows: q mode 1), from a run with the extra
    # prefill records, whose mixed launch shares the Qwen3 fused-q instance
    # (the main counter and trace runs leave extra_prefill out)
    "prefill_gemma_prefill_d256": (("prefill_kernel<256, ", ", 1>"), PREFILL_SRC),
    "prefill_gemma_prefill_d512": (("prefill_kernel<512, ", ", 1>"), PREFILL_SRC),
}


def summarize_pmc(fetch_db, write_db, out_dir, command="", only=None):
    """HBM bytes per call of every part's kernel(s) = FETCH_SIZE + WRITE_SIZE (KiB
    per dispatch), each scaled by what the counter reads for a 256 MiB device
    copy (``--calibrate-copy``): one ``<part>_pmc.json`` per part whose kernels
    ran.  Per call = the counted dispatches' bytes over their number.  Other
    library kernels of the run are listed for reference.  ``only``: the names
    of the parts to summarize (the solo parts are summarized only when named)."""
    fetch = _pmc_per_kernel(fetch_db, "FETCH_SIZE")
    write = _pmc_per_kernel(write_db, "WRITE_SIZE")
    copy_bytes = 128 * 2**20 * 2

    def copy_scale(tab):
        vals = [v for k, vs in tab.items() if "copyBuffer" in k for v in vs]
        return copy_bytes / (max(vals) * 1024.0) if vals else None

    f_scale, w_scale = copy_scale(fetch), copy_scale(write)
    table = {**PMC_PARTS, **PMC_SOLO_PARTS} if only else PMC_PARTS
    for part, (key, sources) in table.items():
        if only and part not in only:
            continue
        total, n = 0.0, 0
        parts = {}
        for k in sorted(set(fetch) | set(write)):
            if "pkv::" not in k:
                continue
            fv, wv = fetch.get(k, []), write.get(k, [])
            fb = float(np.mean(fv or [0.0])) * 1024.0 * (f_scale or 1.0)
            wb = float(np.mean(wv or [0.0])) * 1024.0 * (w_scale or 1.0)
            counted = all(part_key in k for part_key in key)
            if counted:
                total += (fb + wb) * len(fv)
                n += len(fv)
            short = k.replace("void ", "").replace("pkv::(anonymous namespace)::", "").split("(")[0]
            parts[short] = dict(fetch_bytes=round(fb), write_bytes=round(wb),
                                dispatches=len(fv), counted=counted)
        if n == 0:
            continue
        rec = dict(part=part, source_sha=source_sha(sources), hbm_bytes_per_call=round(total / n),
                   kernels=parts, copy_scale=dict(fetch=f_scale, write=w_scale,
                                                  copy_bytes=copy_bytes),
                   command=command)
        with open(os.path.join(out_dir, f"{part}_pmc.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(dict(part=part, hbm_bytes_per_call=rec["hbm_bytes_per_call"])))


MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_WAVES",
                 "GRBM_GUI_ACTIVE"]
N_CU, N_XCD = 256, 8
FLOP_PER_MFMA = 16 * 16 * 32 * 2   # v_mfma_f32_16x16x32_bf16, one wave instruction


def summarize_mfma(db_path, out_path, command=""):
    """Matrix-core counters of the prefill attention kernel (the instance the
    roofline times) from one `rocprofv3 --pmc` run: MFMA busy fraction of all
    SIMD cycles (busy cycles over GRBM_GUI_ACTIVE per XCD x CUs x 4 SIMDs) and
    MFMA FLOPs executed vs algorithmic."""
    import sqlite3
    db = sqlite3.connect(db_path)
    key = "%prefill_kernel<%, 0>%"
    vals = {}
    for c in MFMA_COUNTERS:
        rows = db.execute("select dispatch_id, sum(counter_value) from pmc_events where name like ? "
                          "and counter_name = ? group by dispatch_id", (key, c)).fetchall()
        vals[c] = float(np.mean([r[1] for r in rows])) if rows else None
    durs = [r[0] for r in db.execute("select duration from kernels where name like ?", (key,))]
    dur_ns = float(np.mean(durs)) if durs else None
    pw_flops = None
    try:
        from synth import CONFIGS, config_lengths
        c = CONFIGS["qwen3_prefill"]
        lengths, _ = config_lengths("qwen3_prefill")
        pw_flops = int(sum(2 * c["head_dim"] * c["n_q"] * int(L) * (int(L) + 1) for L in lengths))
    except Exception:  # pragma: no cover
        pass
    gui = vals.get("GRBM_GUI_ACTIVE")
    busy = vals.get("SQ_VALU_MFMA_BUSY_CYCLES")
    rec = dict(kernel="prefill_kernel<128, 2, 0> (qwen3_prefill attention)",
               source_sha=source_sha(PREFILL_SRC), counters=vals,
               kernel_ns_under_counters=dur_ns, command=command)
    if gui and busy:
        rec["mfma_busy_fraction"] = round(busy / (gui / N_XCD * N_CU * 4), 4)
    if vals.get("SQ_INSTS_MFMA") and pw_flops:
        executed = vals["SQ_INSTS_MFMA"] * FLOP_PER_MFMA
        rec["mfma_flops_executed"] = executed
        rec["algorithmic_flops"] = pw_flops
        rec["executed_over_algorithmic"] = round(executed / pw_flops, 3)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


SQ_INSTANCES = {
    # summary key: SQL name pattern of the kernel instance
    "prefill_attention": "%prefill_kernel<%, 0>%",
    "prefill_attention_fused_q": "%prefill_kernel<%, 2>%",
    "decode_llama": "%decode_keysplit_kernel<128, 4, true>%",
}


def summarize_sq(db_paths, out_path, command=""):
    """Shader-sequencer counters of the prefill instances (and, for contrast,
    the Llama decode kernel) from one or more `rocprofv3 --pmc` runs, each
    counter's mean per dispatch.  Derived: the share of wave-cycles spent
    waiting (SQ_WAIT_ANY), waiting to issue an LDS instruction
    (SQ_WAIT_INST_LDS) and issuing VALU / LDS / vector-memory instructions
    (SQ_ACTIVE_INST_*), all over SQ_WAVE_CYCLES; LDS bank-conflict cycles over
    LDS-active cycles; MFMA busy over all SIMD cycles."""
    import sqlite3
    recs = {}
    for name, key in SQ_INSTANCES.items():
        vals, durs = {}, []
        for path in db_paths.split(","):
            db = sqlite3.connect(path)
            names = [r[0] for r in db.execute(
                "select distinct counter_name from pmc_events where name like ?", (key,))]
            for c in names:
                rows = db.execute("select dispatch_id, sum(counter_value) from pmc_events where name "
                                  "like ? and counter_name = ? group by dispatch_id", (key, c)).fetchall()
                vals[c] = float(np.mean([r[1] for r in rows]))
            durs += [r[0] for r in db.execute("select duration from kernels where name like ?", (key,))]
        if not vals:
            continue
        rec = dict(counters=vals, kernel_ns_under_counters=float(np.mean(durs)) if durs else None)
        wc = vals.get("SQ_WAVE_CYCLES")
        if wc:
            for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
                      "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
                      "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC"):
                if c in vals:
                    rec[c.lower()[3:] + "_over_wave_cycles"] = round(vals[c] / wc, 4)
        if vals.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in vals:
            rec["lds_bank_conflict_over_lds_active"] = round(
                vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_LDS_IDX_ACTIVE"], 4)
        gui, busy = vals.get("GRBM_GUI_ACTIVE"), vals.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if gui and busy:
            rec["mfma_busy_fraction"] = round(busy / (gui / N_XCD * N_CU * 4), 4)
        recs[name] = rec
    out = dict(source_sha=dict(prefill=source_sha(PREFILL_SRC), decode=source_sha(DECODE_SRC)),
               instances=recs, command=command)
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: {kk: vv for kk, vv in v.items() if kk != "counters"} for k, v in recs.items()}))


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ----------------------------------------------------------------------------

CPU_SAMPLE_ROWS = 8   # rows of the decode workload one oracle sample call covers


def _cpu_decode_sample(name):
    """The first CPU_SAMPLE_ROWS rows of a decode workload (same lengths,
    slots, heads and pages as the GPU run), pools holding the history, and the
    algorithmic bytes of one fused call on them (append of the new token +
    attention, counted as on the GPU)."""
    import oracle
    from synth import CONFIGS, config_lengths, make_decode_case
    c = CONFIGS[name]
    lengths, slots = config_lengths(name)
    lengths, slots = lengths[:CPU_SAMPLE_ROWS], slots[:CPU_SAMPLE_ROWS]
    D = c.get("head_dim", c.get("full_dim"))
    case = make_decode_case(c["n_q"], c["n_kv"], D, c["page_size"], lengths,
                            max_slots=c["max_slots"], seed=3407 + c["index"], slot_of_row=slots,
                            pages_per_slot=-(-c["len_hi"] // c["page_size"]))
    kp, vp = case.empty_pools()
    hk, hv, hs, hp = case.history_tokens()
    oracle.append(kp, vp, case.table, hk, hv, hs, hp)
    L = case.seq_lens.astype(np.int64)
    active = int((L > 0).sum())
    per_call = (int(L.sum()) * c["n_kv"] * D * 4 + active * c["n_q"] * D * 4
                + int(np.ceil(L / case.page_size).sum()) * 4
                + active * c["n_kv"] * D * 2 * 4)
    return case, kp, vp, per_call


def _cpu_decode_run(name, seconds):
    """One process, one BLAS thread: fused oracle calls for ~`seconds`."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    case, kp, vp, per_call = _cpu_decode_sample(name)
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.append(kp, vp, case.table, case.k_new, case.v_new, case.append_slots(),
                          case.append_pos())
            oracle.attn_decode(case.q, kp, vp, case.table, case.slots, case.seq_lens,
                               case.scale, 0)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return n, n * per_call, el


def cpu_decode_baseline(name, seconds, processes=1):
    """The fp64 oracle on a bounded sample of the decode workload, scaled to
    GB/s of the same algorithmic bytes as the GPU line.  processes > 1: that
    many concurrent oracle processes (one BLAS thread each, started fresh,
    never forked from this GPU process), aggregate bytes over the longest
    one's time."""
    if processes <= 1:
        n, nbytes, el = _cpu_decode_run(name, seconds)
        calls, cores = n, 1
    else:
        import multiprocessing as mp
        with mp.get_context("spawn").Pool(processes) as pool:
            res = pool.starmap(_cpu_decode_run, [(name, seconds)] * processes)
        calls = sum(r[0] for r in res)
        nbytes = sum(r[1] for r in res)
        el = max(r[2] for r in res)
        cores = processes
    return dict(value=round(nbytes / el / 1e9, 6), unit="GB/s", cores=cores, kind="oracle",
                sample=f"{calls} {name} fused calls (append + attention) on the workload's "
                       f"first {CPU_SAMPLE_ROWS} rows, fp64 numpy, "
                       + ("1 BLAS thread" if cores == 1 else
                          f"{cores} concurrent processes of 1 BLAS thread each")
                       + f", in {el:.1f} s",
                seconds=round(el, 2))


def _cpu_prefill_run(seconds):
    """One process, one BLAS thread: the prefill oracle (prologue and append of
    every token, then attention token by token) until `seconds` pass."""
    import oracle
    from synth import CONFIGS, config_lengths, make_prefill_case
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    c = CONFIGS["qwen3_prefill"]
    lengths, slots = config_lengths("qwen3_prefill")
    case = make_prefill_case(c["n_q"], c["n_kv"], c["head_dim"], c["page_size"], lengths,
                             seed=3407 + c["index"], slots=slots, max_slots=c["max_slots"],
                             pages_per_slot=-(-c["len_hi"] // c["page_size"]))
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    flops, t0 = 0, time.perf_counter()
    try:
        kp, vp = case.empty_pools()
        tsl, tpos = case.token_slots(), case.token_pos()
        q2, k2, v = oracle.prologue_qwen3(case.q, case.k, case.v, case.q_norm_w, case.k_norm_w,
                                          tpos, case.eps, case.theta)
        oracle.append(kp, vp, case.table, oracle.f64_to_bf16_bits(k2), case.v, tsl, tpos)
        qb = oracle.f64_to_bf16_bits(q2)
        done = 0
        for n in range(len(case.slots)):
            a, b = int(case.cu_seqlens[n]), int(case.cu_seqlens[n + 1])
            K, V = oracle.gather_kv(kp, vp, case.table, int(case.slots[n]), b - a)
            for t in range(a, b):
                p = t - a
                oracle.attend_rows(oracle.bf16_bits_to_f64(qb[t]), K[: p + 1], V[: p + 1], p,
                                   case.scale, 0)
                flops += 4 * c["head_dim"] * c["n_q"] * (p + 1)
                done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return flops, el, done, case.T


def cpu_prefill_baseline(seconds, processes=1):
    if processes <= 1:
        flops, el, done, T = _cpu_prefill_run(seconds)
        cores = 1
    else:
        import multiprocessing as mp
        with mp.get_context("spawn").Pool(processes) as pool:
            res = pool.map(_cpu_prefill_run, [seconds] * processes)
        flops = sum(r[0] for r in res)
        el = max(r[1] for r in res)
        done = sum(r[2] for r in res)
        T = res[0][3]
        cores = processes
    return dict(value=round(flops / el / 1e12, 9), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"prologue + append of all {T} tokens, then attention of "
                       + (f"the first {done} query tokens (fp64 numpy, 1 BLAS thread)"
                          if cores == 1 else
                          f"{done} query tokens in all ({cores} concurrent processes of 1 BLAS "
                          "thread, each running the whole sample)")
                       + f" in {el:.1f} s",
                seconds=round(el, 2))


# ----------------------------------------------------------------------------

def decode_record(name, args, headline=False):
    """Time one decode workload's step (every layer: the fused append +
    attention kernel) and its kernel; returns the record for the JSON line."""
    import torch
    log(f"setting up {name}")
    wl = DecodeWorkload(name, contiguous=args.contiguous_pages)
    g_step = capture(wl.step)
    log(f"timing {name}")
    torch.cuda.synchronize()
    ms_step = time_graph(g_step, args.steps, args.warmup)
    each = time_graph_each(g_step, args.steps)
    # kernel time per call: the same graph replayed back to back (HIP events on
    # the graph's stream); every dispatch of the step is one decode kernel
    ms_call = time_graph(g_step, args.kernel_reps, 2) / wl.n_calls
    call_bytes = [wl.attn_bytes(ly) + wl.append_bytes(ly) for ly in wl.layers]
    step_bytes = sum(call_bytes)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = (step_bytes / wl.n_calls) / (ms_call * 1e-3) / 1e9
    traffic = None if args.contiguous_pages else pmc_traffic(f"decode_{name}")
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel="decode (split-K kernel: fused append of the new token, attention, "
                           "last split merges)",
                    algorithmic_bytes_per_call=int(step_bytes / wl.n_calls),
                    us_per_call=round(ms_call * 1e3, 3))
    rec = dict(config=wl.describe(), ms_per_step=round(ms_step, 4), value=round(value, 1),
               unit="GB/s", roofline=roofline,
               step_ms_median=round(float(np.median(each)), 4), step_ms_best=round(min(each), 4))
    dims = sorted({ly["D"] for ly in wl.layers})
    if len(dims) > 1:
        # per layer kind (Gemma: the sliding head_dim-256 and full head_dim-512 calls)
        rec["per_kind"] = {}
        for D in dims:
            g = capture(lambda D=D: wl.step_kind(D))
            lys = [ly for ly in wl.layers if ly["D"] == D]
            ms = time_graph(g, args.kernel_reps, 2) / len(lys)
            b = sum(wl.attn_bytes(ly) + wl.append_bytes(ly) for ly in lys) / len(lys)
            rec["per_kind"][f"head_dim_{D}"] = dict(
                us_per_call=round(ms * 1e3, 3), algorithmic_bytes_per_call=int(b),
                achieved=round(b / (ms * 1e-3) / 1e9, 1),
                frac=round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                traffic=None if args.contiguous_pages else pmc_traffic(
                    f"decode_{name}", f"decode_dimsplit_kernel<{D}"),
                window=max(ly["window"] for ly in lys))
            del g
    if args.attn_only:
        g_attn = capture(wl.attn_only)
        ms_a = time_graph(g_attn, args.kernel_reps, 2) / wl.n_calls
        ab = sum(wl.attn_bytes(ly) for ly in wl.layers) / wl.n_calls
        rec["attn_only"] = dict(us_per_call=round(ms_a * 1e3, 3),
                                achieved=round(ab / (ms_a * 1e-3) / 1e9, 1))
        del g_attn
    if headline:
        rec["device_reserve"] = reserve_timing(wl)
    del g_step, wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def prefill_record(args):
    import torch
    log("setting up qwen3_prefill")
    pw = PrefillWorkload(contiguous=args.contiguous_pages)
    gp_step = capture(pw.step)
    gp_attn = capture(pw.attn_only)
    gp_fq = capture(pw.attn_fused_q)
    log("timing prefill")
    ms_p = time_graph(gp_step, args.steps, args.warmup)
    each_p = time_graph_each(gp_step, args.steps)
    ms_pa = time_graph(gp_attn, args.kernel_reps, 2) / pw.n_calls
    ms_fq = time_graph(gp_fq, args.kernel_reps, 2) / pw.n_calls
    fl = pw.flops_per_call()
    ab = pw.attn_bytes()
    # Reference stream: a plain device copy of each layer's q into its out
    # buffer (the q read and out write every attention call makes, 81.7 MB),
    # timed the same way -- what the compulsory q / out traffic alone takes.
    def copy_q_out():
        for ly in pw.layers:
            ly["out"].copy_(ly["q"])
    gp_copy = capture(copy_q_out)
    ms_copy = time_graph(gp_copy, args.kernel_reps, 2) / pw.n_calls
    copy_bytes = 2 * pw.layers[0]["q"].numel() * pw.layers[0]["q"].element_size()
    del gp_copy

    def roof(ms, part, kernel):
        tf = fl / (ms * 1e-3) / 1e12
        return dict(bound="mfma", achieved=round(tf, 2), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                    traffic=None if args.contiguous_pages else pmc_traffic(part),
                    kernel=kernel, algorithmic_flops_per_call=fl,
                    us_per_call=round(ms * 1e3, 3))

    rec = {
        "config": pw.describe(), "ms_per_step": round(ms_p, 4),
        "step_ms_median": round(float(np.median(each_p)), 4),
        "step_ms_best": round(min(each_p), 4),
        # a whole layer: k/v prologue kernel + attention with the fused q transform
        "tflops_step": round(fl * pw.n_calls / (ms_p * 1e-3) / 1e12, 2),
        "roofline": roof(ms_pa, "prefill_qwen3_prefill",
                         "prefill attention (keys already in the pages, q as given)"),
        "roofline_fused_q": roof(ms_fq, "prefill_fused_q_qwen3_prefill",
                                 "prefill attention with the fused q RMSNorm + RoPE (the "
                                 "instance a prefill layer with the prologue runs)"),
        # The same kernel against the HBM roofline: its arithmetic intensity
        # (FLOPs per compulsory byte: q and out once, each sequence's K/V once)
        # lies below the bf16 ridge, so its bytes bound it before its FLOPs.
        "roofline_hbm": dict(
            bound="hbm", achieved=round(ab / (ms_pa * 1e-3) / 1e9, 1), peak=HBM_PEAK_GBS,
            unit="GB/s", frac=round(ab / (ms_pa * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            traffic=None if args.contiguous_pages else pmc_traffic("prefill_qwen3_prefill"),
            algorithmic_bytes_per_call=ab, us_per_call=round(ms_pa * 1e3, 3),
            arithmetic_intensity=round(fl / ab, 1),
            ridge=round(MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9), 1)),
        "q_out_copy_reference": dict(
            us_per_call=round(ms_copy * 1e3, 3), bytes_per_call=copy_bytes,
            achieved=round(copy_bytes / (ms_copy * 1e-3) / 1e9, 1), unit="GB/s",
            kernel="torch copy_ of q into out (the attention's compulsory q / out traffic)"),
        "prologue_us_per_call": round((ms_p / pw.n_calls - ms_fq) * 1e3, 3),
        "prologue_bytes_per_call": pw.prologue_bytes(),
    }
    del gp_step, gp_attn, gp_fq, pw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def _extra_prefill_roofs(fl, ab, ms_layer, ms_attn, kernel, part=None):
    tf = fl / (ms_attn * 1e-3) / 1e12
    gbs = ab / (ms_attn * 1e-3) / 1e9
    traffic = pmc_traffic(part) if part else None
    return dict(
        us_per_layer=round(ms_layer * 1e3, 3), prologue_us=round((ms_layer - ms_attn) * 1e3, 3),
        roofline=dict(bound="mfma", achieved=round(tf, 2), peak=MFMA_BF16_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), traffic=traffic,
                      kernel=kernel, algorithmic_flops_per_call=fl,
                      us_per_call=round(ms_attn * 1e3, 3)),
        roofline_hbm=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                          algorithmic_bytes_per_call=ab, us_per_call=round(ms_attn * 1e3, 3),
                          arithmetic_intensity=round(fl / ab, 1)))


def extra_prefill_records(args):
    """The Gemma-4 prefill layers and the chunked prefill + decode launch:
    per call, a whole layer (prologue + attention) and the attention with the
    fused q transform alone, each against the MFMA and HBM rooflines."""
    import torch
    out = {}
    log("setting up gemma_prefill")
    gw = GemmaPrefillWorkload()
    rec = dict(config=gw.describe(), per_kind={})
    for D in sorted(gw.kinds):
        g_l = capture(lambda D=D: gw.layer(D))
        g_a = capture(lambda D=D: gw.attn_fused_q(D))
        n = _PrefillLayers.N_COPIES
        ms_l = time_graph(g_l, args.kernel_reps, 2) / n
        ms_a = time_graph(g_a, args.kernel_reps, 2) / n
        rec["per_kind"][f"head_dim_{D}"] = dict(
            window=gw.kinds[D][1], **_extra_prefill_roofs(
                gw.flops(D), gw.attn_bytes(D), ms_l, ms_a,
                f"prefill attention with the fused q transform, head_dim {D}",
                part=f"prefill_gemma_prefill_d{D}"))
        del g_l, g_a
    out["gemma_prefill"] = rec
    del gw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("setting up qwen3_chunked_mixed")
    mw = ChunkedMixedWorkload()
    g_l = capture(mw.layer)
    g_a = capture(mw.attn_fused_q)
    n = _PrefillLayers.N_COPIES
    ms_l = time_graph(g_l, args.kernel_reps, 2) / n
    ms_a = time_graph(g_a, args.kernel_reps, 2) / n
    out["qwen3_chunked_mixed"] = dict(config=mw.describe(), **_extra_prefill_roofs(
        mw.flops(), mw.attn_bytes(), ms_l, ms_a,
        "prefill attention with the fused q transform (prompt chunks and decode rows)"))
    del g_l, g_a, mw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-tp8-share", action="store_true",
                    help="leave out the llama_decode_tp8_share line (profiler runs: its kernel "
                         "instance is also the Llama step's, whose per-dispatch figures it would "
                         "mix)")
    ap.add_argument("--workload", default="llama_decode",
                    choices=["llama_decode", "qwen3_decode", "gemma_mixed",
                             "llama_decode_tp8_share"],
                    help="the decode workload of the headline line (default: the largest)")
    ap.add_argument("--no-extra-decode", action="store_true",
                    help="skip the other decode workloads")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="skip the Gemma-4 prefill layers and the chunked prefill + decode launch")
    ap.add_argument("--attn-only", action="store_true",
                    help="also time decode attention without the fused append")
    ap.add_argument("--contiguous-pages", action="store_true",
                    help="map each slot's pages to consecutive physical pages instead of a "
                         "random permutation (times the page indirection)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--cpu-processes", type=int, default=0,
                    help="processes of the all-cores CPU leg (0: the host's cores, at most 16)")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="replays of the graphs timed for kernel durations")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DB", "OUT"),
                    help="write a kernel-duration summary of a rocprofv3 database and exit")
    ap.add_argument("--pmc-parts", default="",
                    help="with --summarize-pmc: comma-separated parts to summarize (default: "
                         "every part of a full bench run; the solo parts only when named)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "OUT_DIR"),
                    help="write HBM traffic per call of every part's kernels from two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("DB", "OUT"),
                    help="write the prefill kernel's matrix-core counters from one rocprofv3 "
                         "--pmc run and exit")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("DBS", "OUT"),
                    help="write the SQ counter summary of comma-separated --pmc databases and exit")
    ap.add_argument("--command", default="", help="command line recorded in summaries")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command=args.command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, command=args.command)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq, command=args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, command=args.command,
                      only=args.pmc_parts.split(",") if args.pmc_parts else None)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this bench runs the single-GPU path only; "
                                   f"--gpus {args.gpus} is not supported (use --gpus 1)"}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    import paged_kv_attention_pagetable_amd as pkv
    pkv.lib()

    head = decode_record(args.workload, args, headline=True)
    result = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, "
                + ("contiguous pages)" if args.contiguous_pages else "random page permutation)"),
        "config": head["config"], "roofline": head["roofline"],
        "step_ms_median": head["step_ms_median"], "step_ms_best": head["step_ms_best"],
        "device_reserve": head["device_reserve"],
    }
    for k in ("attn_only", "per_kind"):
        if k in head:
            result[k] = head[k]
    if not args.no_extra_decode:
        result["extra_decode"] = {}
        names = ["qwen3_decode", "llama_decode", "gemma_mixed"]
        if not args.no_tp8_share:
            names.append("llama_decode_tp8_share")
        for name in names:
            if name != args.workload:
                result["extra_decode"][name] = decode_record(name, args)
    if args.calibrate_copy:
        src = torch.empty(128 * 2**20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_prefill:
        result["prefill"] = prefill_record(args)
        if not args.no_extra_prefill:
            result["extra_prefill"] = extra_prefill_records(args)

    if not args.no_cpu_baseline:
        procs = args.cpu_processes or min(len(os.sched_getaffinity(0)), 16)
        log(f"CPU oracle baselines (~{args.cpu_seconds:.0f} s each; all-cores leg: "
            f"{procs} processes)")
        result["cpu_baseline"] = cpu_decode_baseline(args.workload, args.cpu_seconds)
        result["cpu_baseline_all_cores"] = cpu_decode_baseline(args.workload, args.cpu_seconds,
                                                               procs)
        if "prefill" in result:
            result["prefill"]["cpu_baseline"] = cpu_prefill_baseline(args.cpu_seconds)
            result["prefill"]["cpu_baseline_all_cores"] = cpu_prefill_baseline(
                args.cpu_seconds, procs)
    else:
        result["cpu_baseline"] = None
    result["host"] = dict(cpu_count=os.cpu_count(),
                          affinity=len(os.sched_getaffinity(0)),
                          device=torch.cuda.get_device_name(0))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
