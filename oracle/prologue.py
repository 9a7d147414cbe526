"""Oracle: the Qwen3 and Gemma-4 attention prologues (per-head RMSNorm, then RoPE).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  numpy float64.

Order of operations, per token and head (the Gemma sibling of the Qwen3 engine
shows it: [moe-qwen3 compare] unsloth/inference/flex_gemma4_moe.py, attention
forward -- ``q_norm``/``k_norm`` on the head_dim axis, then rotary, then the
paged-KV write; the engine write-up on [continuous-batching compare]
scripts/benchmarks README says Qwen3's only arch-specific branch is this
per-head q/k RMSNorm):

1. ``x_hat = x / sqrt(mean(x**2) + eps) * w``  over the head_dim axis;
2. ``rope(x_hat, pos) = x_hat * cos + rotate_half(x_hat) * sin`` with
   ``rotate_half(x) = cat(-x[D/2:], x[:D/2])`` and cos/sin of ``pos * w_i``
   repeated over both halves ([moe-qwen3 compare] flex_gemma4_moe.py,
   ``_rotate_half`` / ``_apply_rotary_full``);
3. k' (normed + rotated) and the raw v are appended; q' is returned.

Reading taken where the pages are silent: the frequencies are the "default"
rope type's ``w_i = theta ** (-2 i / D)``, ``i = 0 .. D/2-1`` (the pages name
the rope type and theta only, and hand both rope types to the transformers
rotary-embedding classes).  ``tests/test_oracle_prologue.py`` pins this,
and the partial ("proportional") variant below, against those library
classes -- the default and proportional rope initialisers, the Qwen3 and
Gemma-4 RMSNorm modules and ``apply_rotary_pos_emb`` -- besides closed forms
and invariants.
"""

from __future__ import annotations

import math

import numpy as np

from .paged import bf16_bits_to_f64


def rmsnorm(x, w, eps: float):
    """``x / sqrt(mean(x^2, axis=-1) + eps) * w`` in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_inv_freq(head_dim: int, theta: float):
    """Default rotary frequencies ``theta ** (-2i / D)`` for ``i < D/2``."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / head_dim)


def rope_inv_freq_partial(head_dim: int, theta: float, rotary_fraction: float):
    """Partial ("proportional") rotary frequencies of the Gemma-4 full layers.

    [moe-qwen3 compare] flex_gemma4_moe.py (model notes, "Two-tier RoPE", and
    the ``_apply_rotary_full`` docstring): only the leading
    ``rotary_fraction`` of the frequencies rotate; the tail entries of
    ``inv_freq`` are zero, so their cos = 1, sin = 0 and ``rotate_half`` over
    the full head_dim passes those dims through.  (The
    ``_compute_rotary_per_layer_type`` docstring puts the same thing as the
    initialiser slicing the head dim to ``rotary_fraction * head_dim``
    rotating dims.)  Reading taken where the pages are silent: the rotating
    frequencies keep the default exponents over the full head_dim,
    ``theta ** (-2i / D)`` for ``i < floor(rotary_fraction * D / 2)`` -- the
    count the library's proportional initialiser takes.
    """
    inv = rope_inv_freq(head_dim, theta)
    n_rot = int(math.floor(rotary_fraction * head_dim / 2))
    inv[n_rot:] = 0.0
    return inv


def rope_apply(x, pos, inv_freq):
    """Half-split rotary embedding of ``x [..., D]`` at integer positions ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq  # [..., D/2]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=-1)
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=-1)
    rot = np.concatenate([-x[..., half:], x[..., :half]], axis=-1)
    return x * cos + rot * sin


def prologue_qwen3(q, k, v, q_norm_w, k_norm_w, positions, eps: float, theta: float):
    """Apply the prologue to packed tokens.

    ``q``: uint16 bf16 bits ``[T][n_q][D]``; ``k``, ``v``: ``[T][n_kv][D]``;
    ``q_norm_w``, ``k_norm_w``: ``[D]`` bits; ``positions``: ``[T]`` logical
    positions.  Returns float64 ``(q', k', v)`` with ``v`` unchanged.
    """
    qf, kf, vf = bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v)
    wq, wk = bf16_bits_to_f64(q_norm_w), bf16_bits_to_f64(k_norm_w)
    D = qf.shape[-1]
    inv = rope_inv_freq(D, theta)
    pos = np.asarray(positions, dtype=np.float64)[:, None]  # broadcast over heads
    q2 = rope_apply(rmsnorm(qf, wq, eps), pos, inv)
    k2 = rope_apply(rmsnorm(kf, wk, eps), pos, inv)
    return q2, k2, vf


def prologue_gemma4(q, k, v, q_norm_w, k_norm_w, positions, eps: float, theta: float,
                    rotary_fraction: float = 1.0, k_eq_v: bool = False):
    """The Gemma-4 attention prologue ([moe-qwen3 compare] flex_gemma4_moe.py,
    attention forward and model notes 3-4): q and k get RMSNorm with their
    gains, v gets RMSNorm without a gain (``v_norm``, ``with_scale=False``);
    with K=V the value is the raw k projection (before ``k_norm`` and
    rotary), then ``v_norm``.  q and k are then rotated (``rotary_fraction``
    < 1: the full layers' partial RoPE).  Same bit-pattern inputs as
    ``prologue_qwen3``; ``v`` is ignored when ``k_eq_v``.  Returns float64
    ``(q', k', v')``.
    """
    qf, kf = bf16_bits_to_f64(q), bf16_bits_to_f64(k)
    vf = kf if k_eq_v else bf16_bits_to_f64(v)
    wq, wk = bf16_bits_to_f64(q_norm_w), bf16_bits_to_f64(k_norm_w)
    D = qf.shape[-1]
    inv = rope_inv_freq_partial(D, theta, rotary_fraction)
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    q2 = rope_apply(rmsnorm(qf, wq, eps), pos, inv)
    k2 = rope_apply(rmsnorm(kf, wk, eps), pos, inv)
    v2 = rmsnorm(vf, 1.0, eps)
    return q2, k2, v2
