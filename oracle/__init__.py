"""Plain, slow CPU oracle of the paged KV-cache attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports it, and this
package imports nothing from the product path.

Everything is numpy float64 (bf16 inputs are upcast exactly from their bits),
written as the plain definition of what the pages describe:

* ``paged``     -- page-table addressing, the append scatter, page gather and
                   textbook masked-softmax GQA attention for decode and packed
                   varlen prefill (causal / sliding-window / document masks).
* ``prologue``  -- per-head RMSNorm followed by half-split rotary embedding
                   (Qwen3; Gemma-4 with v_norm, K=V and partial rotary).
* ``pagetable`` -- the host-side slot / page allocator state machine.

Pages cited (by title / address; a section is a file shown on that page):

* [moe-qwen3 compare]
  https://git.jhoeven.net/ceos/unsloth/compare/main...danielhanchen/flex-moe-qwen3
* [engine PR tests]
  https://git.jhoeven.net/ceos/unsloth/src/commit/35231d4ff40cbecc3ea4f4eae17d2d53cbea8ffa/tests
* [continuous-batching compare]
  https://git.jhoeven.net/ceos/unsloth/compare/main...transformers-continuous-batching-qwen3

Parity status of each function is stated in its docstring; every function here
is pinned by ``tests/test_oracle_*.py`` (closed forms, invariants, brute force,
a library routine and hand-derived golden fixtures) -- none is "parity unpinned"
except where a docstring says so.
"""

from . import paged, prologue, pagetable  # noqa: F401
from .paged import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    append,
    gather_kv,
    visible,
    attend_rows,
    attn_decode,
    attn_prefill,
)
from .prologue import (rmsnorm, rope_inv_freq, rope_inv_freq_partial, rope_apply,  # noqa: F401
                       prologue_qwen3, prologue_gemma4)
from .pagetable import PageTableModel  # noqa: F401
