"""Device memory for one layer's paged K/V pool (torch allocation only).

K pool [num_blocks][num_kv_heads][head_dim / X][16][X] (X = 16 bytes of
elements), V pool [num_blocks][num_kv_heads][head_dim][16]; fp8 pools are
uint8 OCP e4m3 codes
with per-KV-head fp32 scales.  The caller owns block assignment; this class
only allocates and, optionally, fills every element with a NaN pattern so
that a kernel reading a slot no sequence owns shows up as NaN.
"""

import torch

from . import _lib

TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
NAN_BITS = {"f32": None, "bf16": 0x7FC0, "fp8": 0x7F}


class KVPool:
    def __init__(self, num_blocks, num_kv_heads, head_dim, cache_dtype, device="cuda",
                 block_size=_lib.BLOCK_SIZE, poison=True, k_scale=None, v_scale=None):
        dt = TORCH_STORAGE[cache_dtype]
        self.cache_dtype = cache_dtype
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        self.block_size = block_size
        x = 16 // torch.empty((), dtype=dt).element_size()
        # K and V share one allocation, K first.  Separate allocations land
        # wherever the driver puts them, and the decode reading block b of
        # both at once ran slower: long-context batch (8 sequences, 537k
        # tokens, bf16) in a same-box A/B over eight processes, layer-step
        # 360-364 us with one allocation against 365-370 us with two.
        n = num_blocks * num_kv_heads * head_dim * block_size
        self._kv = torch.empty(2 * n, dtype=dt, device=device)
        self.k = self._kv[:n].view(num_blocks, num_kv_heads, head_dim // x, block_size, x)
        self.v = self._kv[n:].view(num_blocks, num_kv_heads, head_dim, block_size)
        if poison:
            self.poison()
        self.k_scale = None if k_scale is None else torch.as_tensor(k_scale, dtype=torch.float32,
                                                                     device=device).contiguous()
        self.v_scale = None if v_scale is None else torch.as_tensor(v_scale, dtype=torch.float32,
                                                                     device=device).contiguous()

    def poison(self):
        for t in (self.k, self.v):
            if self.cache_dtype == "f32":
                t.fill_(float("nan"))
            elif self.cache_dtype == "bf16":
                t.view(torch.int16).fill_(NAN_BITS["bf16"])
            else:
                t.fill_(NAN_BITS["fp8"])

    def nbytes(self):
        return self.k.numel() * self.k.element_size() * 2

    def append(self, k_new, v_new, slot_mapping, stream=None):
        _lib.pa_kv_append(k_new, v_new, self.k, self.v, slot_mapping, self.k_scale, self.v_scale,
                          stream=stream)
