"""Attention over a paged KV cache on AMD MI355X (gfx950).

The compute path is libpagedattn.so (HIP, include/pa.h); this package is its
thin binding: ``_lib`` (ctypes marshalling of the C entry points) and ``pool``
(torch allocation of the K/V pools).
"""

from ._lib import (  # noqa: F401
    PAError, load, pa_kv_append, pa_decode, pa_decode_append, pa_decode_cascade, pa_decode_multi,
    pa_decode_plan, pa_decode_plan_bytes, decode_plan_buffer,
    pa_decode_splitk_reduce, pa_prefill_chunk,
    pa_decode_workspace_bytes, pa_selftest, status_string, pa_decode_noalloc,
    pa_decode_noalloc_max_bytes, pa_read_probe,
)
from .pool import KVPool  # noqa: F401
