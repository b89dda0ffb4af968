"""CPU oracle for batched-decode PagedAttention — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  It is written from the pages' statement of the
method, in float64 numpy (plus a pure-Python Decimal/mpmath brute force for
tiny inputs), and it shares no code with the HIP path: it imports nothing from
``paged_kv_cache_208_amd`` and the HIP path imports nothing from here.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
never falls back to it.

Sources followed (page title, section):
  * "Distributed LLM Inference Serving Platform", section 2 (Mental Model):
    a sequence's tokens live in fixed 16-token logical blocks that a block
    table maps to non-contiguous physical blocks; paging is address
    translation only, so the result equals attention over the contiguous
    sequence.
  * Same page, section 5.1 (request lifecycle): each decode step writes the
    new token's K/V into its physical block, then attends over every block in
    the sequence's table.
  * Same page, section 11 (Lab 1 worked solution) and section 7 (block
    manager): copy-on-write clones a shared tail block into a fresh one.
  * "Roadmap: vLLM-style serving features for TornadoVM batched decode",
    Core batched decode (per-head QK-norm + split-half RoPE for Qwen3),
    Serving / scheduling (PagedAttention: block-pool KV + per-slot block
    table), Sampling / logits (quantized Q8/FP8 KV cache as a listed item).

Parity pins (what fixes the oracle other than itself) live in tests/ and are
listed per function in the module docstrings.  No function here is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    gather_sequence_kv,
    attn_ref,
    attn_weights_ref,
    partials_ref,
    combine_ref,
    mq_attn_ref,
)
from .e4m3 import e4m3_table, e4m3_decode  # noqa: F401
from .append import append_ref, rmsnorm_rope_ref, fused_append_ref  # noqa: F401
from .blocks import copy_blocks_ref  # noqa: F401
from .e4m3 import e4m3_encode  # noqa: F401
from .fp8_append import append_e4m3_ref  # noqa: F401
