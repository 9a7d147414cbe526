"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds only input generation (random numbers, shapes, page-table
layouts and length mixes).  It contains none of the method's arithmetic: no
addressing, no append, no attention, no normalisation.  Both the oracle side and
the GPU side start from the arrays made here.

Workloads (shaped like the pages' Qwen3-4B / Llama-3.2-3B / Gemma-4-E2B
generation runs; the pages' own prompts and checkpoints are not used -- random
N(0,1) bf16 tensors of the same shapes stand in for them):

* ``tiny``          2 decode rows in slots 1-2, n_q 4 / n_kv 2, D 64, page 16,
                    lengths 37 and 50, 16-page pool, scale 1/8.
* ``qwen3_decode``  8 rows in slots 1-8 of 9, 32/8 heads, D 128, page 128,
                    lengths U[64, 1024]; 36 distinct layer pools.
* ``llama_decode``  64 rows, 24/8, D 128, page 128, lengths U[128, 4096],
                    10% of rows idle (length 0).
* ``qwen3_prefill`` 16 prompts, lengths U[32, 512], 32/8, D 128, page 128,
                    fused q/k RMSNorm (eps 1e-6, weights N(1, 0.1)) + RoPE
                    theta 1e6.
* ``gemma_mixed``   64 rows, lengths U[256, 1536], n_q 8 / n_kv 2, page 64;
                    one sliding layer (D 256, window 512) and one full layer
                    (D 512) per step.
* ``gemma_prefill`` 16 prompts U[128, 1024], n_q 8 / n_kv 2, page 64, the
                    Gemma-4 prologue; a sliding layer (D 256, window 512,
                    theta 1e4) and a full layer (D 512, theta 1e6, 25 %
                    rotary, K = V).
* ``qwen3_chunked_mixed`` one launch of 8 prompt chunks U[64, 512] on cached
                    prefixes U[256, 1024] and 56 decode rows (one token on a
                    cached U[64, 1024]); Qwen3 heads and prologue.

Seeds are ``3407 + config index`` (3407 is the seed the pages' scripts use).
"""

from .gen import (  # noqa: F401
    SENTINEL_BITS,
    CONFIGS,
    DecodeCase,
    PrefillCase,
    rng_for,
    randn_bf16,
    make_decode_case,
    make_prefill_case,
    split_tokens,
    config_lengths,
    chunked_mixed_rows,
    prefill_page_table,
)
