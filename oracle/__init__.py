"""CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, fp64 statement of
what the GPU library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product library
(``paged_kv_attention_write_amd``) never imports, links or calls it, and it
imports nothing from the product library.  The two share no code: not a
kernel, header, helper, table or constant generator.  The only code both
sides are fed from is the seeded input generator in ``workloads/``, which holds
no arithmetic of the method.

Sources (the four pages this library follows):

* "How Easy Is It to Start Serving LLMs?" (Geodesic blog), section
  "Phase 4: inside FlashInfer": §1 block-sparse KV memory (the page table in
  CSR form, shared prompt pages), §3 load balancing (the split-KV planner and
  the merge of split chunks).
* "nanoserve" (README): the paged KV cache and its block table, the one-engine-
  step description (each layer writes this step's K/V through per-token slots
  and then attends over the whole context), the gather + SDPA attention path.
* "How to design an LLM serving system (a vLLM deep dive)": block table,
  ``slot_mapping``, the kv-bytes-per-token formula.
* "PageServe": the correctness invariants (block size, batch size, prefix
  sharing, neighbour independence, incremental decode = recompute).

Modules:

* :mod:`oracle.numerics`  - bf16 and OCP FP8 E4M3FN codecs, written from the
  format definitions.
* :mod:`oracle.paged_attention` - the KV write, the gather, exact softmax
  attention (fp64), partial attention over a key range and the LSE merge.
* :mod:`oracle.plan` - the split-KV planner as the blog's §3 describes it
  (the reading the library follows, and the illustration's steps as printed).

Parity status of each function is stated in its docstring; every function is
pinned by ``tests/test_oracle_*.py`` against closed forms, brute force,
invariants, library routines or the printed numbers under ``tests/golden/``.
"""

from .numerics import (
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    e4m3_decode,
    e4m3_encode,
    e4m3_value_table,
    decode_storage,
)
from .paged_attention import (
    kv_write,
    gather_kv,
    paged_attention,
    attention_over_range,
    lse_merge,
)
from .plan import illustration_plan, split_kv_plan, split_lengths

__all__ = [
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "e4m3_decode",
    "e4m3_encode",
    "e4m3_value_table",
    "decode_storage",
    "kv_write",
    "gather_kv",
    "paged_attention",
    "attention_over_range",
    "lse_merge",
    "split_kv_plan",
    "illustration_plan",
    "split_lengths",
]
