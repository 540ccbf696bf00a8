"""Seeded synthetic paged-KV workloads.

Structure (lengths, block ids, slots) is drawn with NumPy's PCG64 generator;
values (Q, K, V) with a torch generator on the target device, so multi-GB
pools can be drawn where they will live.  Draw order: context lengths ->
block assignment -> Q (decode, then prefill) -> K -> V.

The five named workloads mirror the shapes the pages serve:

1. tiny fp32 decode: B=4, L={17,64,100,250}, 4/2 heads, D=64, 64-block pool,
   Q/K/V uniform[-1, 1]; one appended token per sequence.
2. Qwen2.5-3B-shaped bf16 decode (InferX serves Qwen2.5-3B-Instruct): 16/2
   heads, D=128, B=64, L uniform in [256, 4096], pool 1.25x the blocks needed.
3. Llama-3-8B-shaped bf16 decode with prefix sharing (llm-infer's "256 cached
   prompt tokens, 128 new tokens" at 256 concurrent): 32/8 heads, B=256, each
   context 256 prompt tokens + 0..128 generated; groups of 8 sequences share
   their 16 prompt blocks (same physical ids).
4. long-context bf16 decode, split into 512-token partitions: 32/8 heads, B=8,
   L lognormal (median 65536, sigma ln2/2) clipped to [32768, 131072].
5. mixed chunked-prefill step with an fp8-e4m3 KV cache: 32/8 heads; 60 decode
   sequences with L uniform in [512, 8192] plus 4 prefill chunks of 512 query
   tokens after 0..2048 cached tokens; per-KV-head fp32 scales absmax/448.

Conventions shared with both sides: K pool [NB][Hkv][D/X][bs][X] (X = 16
bytes of elements: 4 fp32, 8 bf16, 16 fp8), V pool [NB][Hkv][D][bs]
(token-minor); slot = block * bs + offset; context lengths include this step's
token; unused block-table entries are -1.  This module draws values and
structure only and does no attention arithmetic.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

CONFIG_NAMES = {
    1: "tiny-fp32-decode",
    2: "qwen2.5-3b-bf16-decode-b64",
    3: "llama3-8b-bf16-decode-prefix-shared-b256",
    4: "long-context-bf16-splitk-b8",
    5: "mixed-chunked-prefill-fp8kv",
}

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    seed: int
    q_dtype: str                 # "f32" | "bf16"
    cache_dtype: str             # "f32" | "bf16" | "fp8"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float                 # exactly a float32 value (1/sqrt(D) rounded to fp32)
    # decode sequences
    context_lens: np.ndarray     # int32 [B]
    block_tables: np.ndarray     # int32 [B, W], -1 padded
    q: torch.Tensor              # [B, Hq, D]
    # prefill chunks (may be empty)
    query_start_loc: np.ndarray  # int32 [C + 1]
    chunk_context_lens: np.ndarray   # int32 [C]
    chunk_block_tables: np.ndarray   # int32 [C, W2]
    q_prefill: torch.Tensor      # [total_q, Hq, D]
    # every occupied slot exactly once, with its K/V (input dtype)
    fill_slots: np.ndarray       # int32 [F]
    fill_k: torch.Tensor         # [F, Hkv, D]
    fill_v: torch.Tensor
    # the tokens appended by this step (rows of the fill set, or slot -1)
    new_slots: np.ndarray        # int32 [T]
    new_rows: np.ndarray         # int64 [T] row of fill_k/fill_v holding its values
    k_scale: np.ndarray = None   # float32 [Hkv] (fp8 caches)
    v_scale: np.ndarray = None
    partition_size: int = 0      # split-K partition the workload is defined with (0: none)
    prefix_groups: list = field(default_factory=list)  # [(member seq ids, shared blocks)]

    # ---- derived sizes -------------------------------------------------
    @property
    def batch(self):
        return int(len(self.context_lens))

    @property
    def num_chunks(self):
        return int(len(self.chunk_context_lens))

    @property
    def in_dtype(self):
        return "f32" if self.q_dtype == "f32" else "bf16"

    @property
    def new_k(self):
        return self.fill_k[torch.as_tensor(self.new_rows, device=self.fill_k.device)]

    @property
    def new_v(self):
        return self.fill_v[torch.as_tensor(self.new_rows, device=self.fill_v.device)]

    def kv_bytes_per_token(self):
        return 2 * self.num_kv_heads * self.head_dim * ELEM_BYTES[self.cache_dtype]

    def pool_bytes(self):
        """Bytes of one layer's K + V pool."""
        return self.num_blocks * self.block_size * self.kv_bytes_per_token()

    def decode_kv_bytes_logical(self):
        """KV bytes a decode step reads, counting shared blocks once per reader."""
        return int(self.context_lens.astype(np.int64).sum()) * self.kv_bytes_per_token()

    def decode_kv_bytes_unique(self):
        """KV bytes of the distinct (block, offset) slots decode reads."""
        seen = set()
        bs = self.block_size
        for b in range(self.batch):
            L = int(self.context_lens[b])
            n = -(-L // bs)
            for i in range(n):
                phys = int(self.block_tables[b, i])
                used = min(bs, L - i * bs)
                for t in range(used):
                    seen.add(phys * bs + t)
        return len(seen) * self.kv_bytes_per_token()

    def prefill_kv_bytes(self):
        return int(self.chunk_context_lens.astype(np.int64).sum()) * self.kv_bytes_per_token()

    def prefill_flops(self):
        """2*D flops for each visible (query, key) pair, twice (QK^T and PV), per q head."""
        total = 0
        qsl = self.query_start_loc
        for c in range(self.num_chunks):
            C = int(qsl[c + 1] - qsl[c])
            L = int(self.chunk_context_lens[c])
            P = L - C
            pairs = C * P + C * (C + 1) // 2
            total += pairs
        return 4 * self.head_dim * self.num_heads * total

    def max_partitions(self, partition_size):
        if partition_size <= 0:
            return 1
        m = int(self.context_lens.max()) if self.batch else 0
        return max(1, -(-m // partition_size))

    # ---- host copies (raw storage) for the oracle ----------------------
    @staticmethod
    def host_raw(t):
        t = t.detach().to("cpu")
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()


def _scale_for(d):
    return float(np.float32(1.0) / np.float32(math.sqrt(d)))


def _draw(gen, shape, dist, device, dtype):
    if dist == "uniform":
        x = torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * 2.0 - 1.0
    else:
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(TORCH_DT[dtype])


def build_workload(name, *, seed, device="cpu", q_dtype="bf16", cache_dtype="bf16",
                   num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                   decode_lens=(), prefill_chunks=(), prefix_groups=(),
                   num_blocks=None, pool_factor=1.25, dist="normal",
                   partition_size=0, rng=None):
    """Generic builder.

    decode_lens     context length of each decode sequence (includes the new token)
    prefill_chunks  (cached_prefix, chunk_len) per chunk; the chunk's tokens are new
    prefix_groups   (list of decode sequence ids, number of shared leading blocks);
                    the members' first blocks get the same physical ids
    num_blocks      pool size; default ceil(pool_factor * unique blocks needed)
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    bs = block_size
    dl = [int(x) for x in decode_lens]
    chunks = [(int(p), int(c)) for p, c in prefill_chunks]
    B, C = len(dl), len(chunks)

    # ---- which logical blocks are shared ------------------------------
    share_of = {}            # (seq, logical block) -> key of the shared block
    for gi, (members, nshared) in enumerate(prefix_groups):
        for b in members:
            need = -(-dl[b] // bs)
            if need < nshared:
                raise ValueError("a sharing sequence must cover the shared blocks")
            for i in range(nshared):
                share_of[(b, i)] = ("g", gi, i)

    # ---- block assignment ----------------------------------------------
    owners = []              # list of (kind, index, n_blocks)
    for b, L in enumerate(dl):
        owners.append(("d", b, -(-L // bs)))
    for c, (P, Cn) in enumerate(chunks):
        owners.append(("p", c, -(-(P + Cn) // bs)))
    keys = []
    for kind, idx, n in owners:
        for i in range(n):
            k = share_of.get((idx, i)) if kind == "d" else None
            keys.append(k if k is not None else (kind, idx, i))
    unique_keys = list(dict.fromkeys(keys))
    need = len(unique_keys)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need))
    if num_blocks < need:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int64)
    phys_of = {k: int(perm[j]) for j, k in enumerate(unique_keys)}

    W = max([n for kind, _, n in owners if kind == "d"] or [1])
    W2 = max([n for kind, _, n in owners if kind == "p"] or [1])
    bt = np.full((B, W), -1, dtype=np.int32)
    cbt = np.full((max(C, 0), W2), -1, dtype=np.int32)
    for kind, idx, n in owners:
        for i in range(n):
            k = share_of.get((idx, i)) if kind == "d" else None
            ph = phys_of[k if k is not None else (kind, idx, i)]
            if kind == "d":
                bt[idx, i] = ph
            else:
                cbt[idx, i] = ph

    # ---- occupied slots (each once) -------------------------------------
    slot_row = {}
    fill = []
    def occupy(phys, pos_in_block):
        s = phys * bs + pos_in_block
        if s not in slot_row:
            slot_row[s] = len(fill)
            fill.append(s)
        return s
    for b, L in enumerate(dl):
        for p in range(L):
            occupy(int(bt[b, p // bs]), p % bs)
    for c, (P, Cn) in enumerate(chunks):
        for p in range(P + Cn):
            occupy(int(cbt[c, p // bs]), p % bs)
    fill_slots = np.asarray(fill, dtype=np.int32)

    # ---- this step's appended tokens ------------------------------------
    new_slots, new_rows = [], []
    for b, L in enumerate(dl):
        if L == 0:
            continue
        p = L - 1
        s = int(bt[b, p // bs]) * bs + p % bs
        shared = (b, p // bs) in share_of
        new_slots.append(-1 if shared else s)
        new_rows.append(slot_row[s])
    for c, (P, Cn) in enumerate(chunks):
        for p in range(P, P + Cn):
            s = int(cbt[c, p // bs]) * bs + p % bs
            new_slots.append(s)
            new_rows.append(slot_row[s])

    # ---- values ------------------------------------------------------------
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    in_dt = "f32" if q_dtype == "f32" else "bf16"
    q = _draw(gen, (B, num_heads, head_dim), dist, device, q_dtype)
    total_q = sum(cn for _, cn in chunks)
    qp = _draw(gen, (total_q, num_heads, head_dim), dist, device, q_dtype)
    F = len(fill_slots)
    fk = _draw(gen, (F, num_kv_heads, head_dim), dist, device, in_dt)
    fv = _draw(gen, (F, num_kv_heads, head_dim), dist, device, in_dt)

    k_scale = v_scale = None
    if cache_dtype == "fp8":
        # caller's scale policy: absmax over every token of the head / 448
        ka = fk.abs().float().amax(dim=(0, 2)).cpu().numpy().astype(np.float32)
        va = fv.abs().float().amax(dim=(0, 2)).cpu().numpy().astype(np.float32)
        k_scale = np.where(ka == 0, np.float32(1), ka / np.float32(448)).astype(np.float32)
        v_scale = np.where(va == 0, np.float32(1), va / np.float32(448)).astype(np.float32)

    qsl = np.zeros(C + 1, dtype=np.int32)
    for c, (_, cn) in enumerate(chunks):
        qsl[c + 1] = qsl[c] + cn

    return Workload(
        name=name, seed=int(seed), q_dtype=q_dtype, cache_dtype=cache_dtype,
        num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=bs, num_blocks=int(num_blocks), scale=_scale_for(head_dim),
        context_lens=np.asarray(dl, dtype=np.int32), block_tables=bt, q=q,
        query_start_loc=qsl,
        chunk_context_lens=np.asarray([p + cn for p, cn in chunks], dtype=np.int32),
        chunk_block_tables=cbt, q_prefill=qp,
        fill_slots=fill_slots, fill_k=fk, fill_v=fv,
        new_slots=np.asarray(new_slots, dtype=np.int32),
        new_rows=np.asarray(new_rows, dtype=np.int64),
        k_scale=k_scale, v_scale=v_scale, partition_size=int(partition_size),
        prefix_groups=[(list(m), int(n)) for m, n in prefix_groups],
    )


def make_config(index, seed=None, device="cpu"):
    """The five named workloads (seed defaults to the config number)."""
    seed = index if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    name = CONFIG_NAMES[index]
    if index == 1:
        return build_workload(name, seed=seed, device=device, q_dtype="f32", cache_dtype="f32",
                              num_heads=4, num_kv_heads=2, head_dim=64,
                              decode_lens=[17, 64, 100, 250], num_blocks=64, dist="uniform",
                              rng=rng)
    if index == 2:
        lens = rng.integers(256, 4096, size=64, endpoint=True)
        return build_workload(name, seed=seed, device=device, num_heads=16, num_kv_heads=2,
                              head_dim=128, decode_lens=lens, rng=rng)
    if index == 3:
        gen = rng.integers(0, 128, size=256, endpoint=True)
        lens = 256 + gen
        groups = [(list(range(8 * g, 8 * g + 8)), 16) for g in range(32)]
        return build_workload(name, seed=seed, device=device, num_heads=32, num_kv_heads=8,
                              head_dim=128, decode_lens=lens, prefix_groups=groups, rng=rng)
    if index == 4:
        z = rng.normal(size=8)
        lens = np.clip(np.round(np.exp(math.log(65536) + (math.log(2) / 2) * z)), 32768, 131072)
        return build_workload(name, seed=seed, device=device, num_heads=32, num_kv_heads=8,
                              head_dim=128, decode_lens=lens.astype(np.int64),
                              partition_size=512, rng=rng)
    if index == 5:
        lens = rng.integers(512, 8192, size=60, endpoint=True)
        prefix = rng.integers(0, 2048, size=4, endpoint=True)
        return build_workload(name, seed=seed, device=device, q_dtype="bf16", cache_dtype="fp8",
                              num_heads=32, num_kv_heads=8, head_dim=128, decode_lens=lens,
                              prefill_chunks=[(int(p), 512) for p in prefix], rng=rng)
    raise KeyError(index)


SPEC_VERIFY_NAME = "qwen2.5-3b-bf16-spec-verify-b64"


def make_spec_verify(seed=6, device="cpu"):
    """Draft verification step on the Qwen2.5-3B decode shape (16 query / 2 KV
    heads, head_dim 128, bf16): 64 sequences with U[256, 4096] cached
    positions, each checking U[2, 8] draft tokens whose K/V are appended in
    this step (causal among themselves)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cached = rng.integers(256, 4096, size=64, endpoint=True)
    drafts = rng.integers(2, 8, size=64, endpoint=True)
    return build_workload(SPEC_VERIFY_NAME, seed=seed, device=device, num_heads=16,
                          num_kv_heads=2, head_dim=128,
                          prefill_chunks=[(int(p), int(k)) for p, k in zip(cached, drafts)],
                          rng=rng)

