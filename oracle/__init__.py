"""fp64 CPU oracle for the SegPagedAttention prefill path — TEST INFRASTRUCTURE.

This package is the checker, not the product. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with ``head_aware_paged_amd`` (the HIP path) and
imports nothing from it; the two meet only in the seeded inputs drawn by
``workloads``.

Every function evaluates the plain definition of what the method computes, in
fp64, with no blocking, fusion or reordering beyond that definition. The pages
(RedKnot: head-aware KV reuse and SegPagedAttention) describe the method in
prose only; where they leave a step open the reading taken is stated in the
function's docstring.

Parity status per function:
  bf16 rounding, rope/relocate, visibility (two independent routines),
  page tables, spans, move lists, attention (brute force + vectorised),
  decode attention (brute force + vectorised, and against the prefill
  attention of a one-token-longer query segment), importance, top-k, sparse
  FFN, the layer glue (projection + RoPE + append, output projection),
  masked-dense attention, the elastic layer stack: pinned by ``tests/test_oracle_*.py``.
  Agreement with RedKnot's own implementation (its RoPE pairing, window
  inclusivity, dense-vs-global semantics) cannot be pinned: the pages print
  no worked example. That end-to-end numerical match is "parity unpinned".
"""
from .bf16 import bf16_bits_to_f64, round_bf16, f64_to_bf16_bits, ulp_bf16  # noqa: F401
from .rope import inv_freq, rope, relocate  # noqa: F401
from .store import gather_kv  # noqa: F401
from .visibility import (visible_brute, visible_intervals, page_table, page_tables,  # noqa: F401
                         visible_spans, move_list, visible_count)
from .attention import attention, attention_brute  # noqa: F401
from .decode import decode, decode_brute  # noqa: F401
from .importance import importance, topk_select  # noqa: F401
from .ffn import sparse_ffn, swiglu_activation  # noqa: F401
from .dense import dense_layout, masked_dense  # noqa: F401
from .stack import shallow_layout, stack  # noqa: F401
from .layer import row_positions, qkv_rope, append_query_kv, out_proj_residual, layer  # noqa: F401
