"""Plain, slow, fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code, header, table or helper with the HIP library under
``paged_kv_cache_234_amd/`` and never imports it.

What it computes (sources are the four pages on paged KV caches: InferX,
infer-lab, llm-infer and RustInfer):

* ``fp8_e4m3``   -- OCP 8-bit float E4M3 ("e4m3fn") decode table and a
  round-to-nearest-even, saturating encoder (InferX, "The kernels underneath",
  FP8 KV cache paragraph, names the format; the OCP FP8 specification defines
  it).
* ``bf16``       -- exact bfloat16 bit-pattern decode.
* ``paged_attention`` -- the KV-append byte semantics, the block-table
  gather and textbook softmax(scale * q K^T) V attention for decode rows and
  causal prefill chunks, split-K partition partials and their combine.

Every function is pinned by ``tests/test_oracle_*.py`` to facts that do not
come from the oracle itself (closed forms, invariants, library routines,
specification values).  No function here is "parity unpinned".
"""

from . import bf16, fp8_e4m3, paged_attention  # noqa: F401
