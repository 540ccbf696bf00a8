"""fp64 reference for attention over a paged KV cache.  Oracle / test
infrastructure: only tests, the smoke check and the CPU-baseline leg of the
benchmark may use it; it shares no code with the HIP library.

Sources (the four pages on paged KV caches):

* Paged pool + block tables: infer-lab, technique table ("PagedAttention --
  block allocator, block tables, refcounting, copy-on-write"); llm-infer,
  "What It Does" ("Paged KV cache with block tables ..."); InferX, "Status"
  and roadmap milestone M3.
* KV write into the cache before attention in the same layer step:
  llm-infer, "What It Does" (graphs capture "KV writes and FlashInfer
  attention"); fp8 KV write with frozen per-layer scales: InferX, "The kernels
  underneath", FP8 KV cache paragraph.
* Attention itself: softmax(scale * q K^T) V with grouped-query heads
  (infer-lab, layout section, "GQA"), online-softmax tiling as an equivalent
  (infer-lab, "tiled attention == naive attention"; llm-infer, References:
  FlashAttention-2), chunked prefill that is causal within the chunk
  (infer-lab, "chunked prefill == one-shot prefill"; llm-infer, "ragged
  batched prefill"), prefix blocks shared between sequences (infer-lab,
  RadixAttention row; llm-infer, "Prefix caching for prompts that share
  leading blocks").

Storage conventions (the pages leave them open; these are the readings the
library also uses, so appended bytes can be compared one for one):

* K pool: [num_blocks][num_kv_heads][head_dim / X][block_size][X] with
  X = 16 bytes of elements (4 fp32, 8 bf16, 16 fp8): for each run of X
  consecutive head-dim elements, the block's 16 tokens one after another.
* V pool: [num_blocks][num_kv_heads][head_dim][block_size]  (token-minor)
* element storage: "f32" -> float32, "bf16" -> uint16 bit patterns,
  "fp8" -> uint8 OCP E4M3 codes with one fp32 scale per KV head (K and V
  separately); real value = decode(code) * scale[h].
* slot s of the pool is block s // block_size, offset s % block_size.
* context_lens include the token appended in this step; a decode query sits
  at position L - 1 and sees positions 0..L-1.
* query head hq reads KV head hq // G, G = num_heads / num_kv_heads.
* a prefill chunk of C queries with context length L has cached prefix
  P = L - C; its query i (position P + i) sees keys 0..P+i inclusive.
* L == 0 gives an all-zero output row.
"""

import math

import numpy as np

from . import bf16 as _bf16
from . import fp8_e4m3 as _fp8

STORAGE_DTYPES = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def k_chunk(dtype):
    """X: head-dim elements per 16-byte run of the K pool layout."""
    return 16 // np.dtype(STORAGE_DTYPES[dtype]).itemsize


def pool_shapes(num_blocks, num_kv_heads, head_dim, dtype, block_size=16):
    """(K pool shape, V pool shape) of the storage layout."""
    x = k_chunk(dtype)
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x),
            (num_blocks, num_kv_heads, head_dim, block_size))


# ---------------------------------------------------------------------------
# element conversions
# ---------------------------------------------------------------------------

def storage_to_f64(raw, dtype):
    """Exact value of stored elements (no scale applied)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return _bf16.to_f64(raw)
    if dtype == "fp8":
        return _fp8.decode(raw)
    raise ValueError("unknown storage dtype %r" % (dtype,))


def encode_for_cache(x_raw, in_dtype, cache_dtype, scale_per_head):
    """New-token K or V rows [T, Hkv, D] (storage of in_dtype) -> cache storage.

    f32->f32 and bf16->bf16 are byte copies.  bf16->fp8 divides by the head's
    scale in binary32 and rounds to E4M3 (oracle.fp8_e4m3.encode).
    """
    if (in_dtype, cache_dtype) in (("f32", "f32"), ("bf16", "bf16")):
        return np.array(x_raw, dtype=STORAGE_DTYPES[cache_dtype], copy=True)
    if (in_dtype, cache_dtype) == ("bf16", "fp8"):
        x32 = _bf16.to_f64(x_raw).astype(np.float32)          # exact
        s = np.asarray(scale_per_head, dtype=np.float32)[None, :, None]
        return _fp8.encode(x32, s)
    raise ValueError("unsupported (input, cache) dtype pair %r" % ((in_dtype, cache_dtype),))


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

def oracle_append(k_pool, v_pool, k_new, v_new, slot_mapping, in_dtype, cache_dtype,
                  k_scale=None, v_scale=None, block_size=16):
    """Return copies of the pools after writing the new tokens' K/V.

    For every token t with slot_mapping[t] >= 0: block = slot // block_size,
    offset = slot % block_size, and for every KV head h and head-dim index d
        K[block, h, d // X, offset, d % X] = enc(k_new[t, h, d]),
        V[block, h, d, offset]             = enc(v_new[t, h, d]).
    Tokens with a negative slot are skipped.  No other element changes.
    Duplicate slots are a caller error (result unspecified) and are rejected.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if not keep.any():
        return k_out, v_out
    s = slots[keep]
    if len(np.unique(s)) != len(s):
        raise ValueError("duplicate slots in one append")
    num_blocks = k_pool.shape[0]
    if s.max() >= num_blocks * block_size:
        raise ValueError("slot beyond the pool")
    blk = s // block_size
    off = s % block_size
    k_enc = encode_for_cache(np.asarray(k_new)[keep], in_dtype, cache_dtype, k_scale)
    v_enc = encode_for_cache(np.asarray(v_new)[keep], in_dtype, cache_dtype, v_scale)
    t_n, hkv, d = k_enc.shape
    x = k_pool.shape[4]
    k_out[blk, :, :, off, :] = k_enc.reshape(t_n, hkv, d // x, x)   # lands on (blk, :, :, off, :)
    v_out[blk, :, :, off] = v_enc                                   # lands on (blk, :, :, off)
    return k_out, v_out


# ---------------------------------------------------------------------------
# gather through the block table
# ---------------------------------------------------------------------------

def gather_sequence(k_pool, v_pool, block_table_row, context_len, cache_dtype,
                    k_scale=None, v_scale=None, block_size=16):
    """Contiguous fp64 K, V of one sequence: arrays [L, Hkv, D].

    Logical position p lives in physical block block_table_row[p // bs] at
    offset p % bs.  Only the first ceil(L / bs) table entries are read; the
    function asserts they are valid block ids.
    """
    L = int(context_len)
    num_blocks, hkv = k_pool.shape[0], k_pool.shape[1]
    d = k_pool.shape[2] * k_pool.shape[4]
    n = -(-L // block_size)
    ids = np.asarray(block_table_row[:n], dtype=np.int64)
    if len(ids) != n or (n and (ids.min() < 0 or ids.max() >= num_blocks)):
        raise ValueError("block table does not cover the context with valid ids")
    kb = storage_to_f64(k_pool[ids], cache_dtype)                 # [n, Hkv, D/X, bs, X]
    vb = storage_to_f64(v_pool[ids], cache_dtype)                 # [n, Hkv, D, bs]
    if cache_dtype == "fp8":
        kb = kb * np.asarray(k_scale, dtype=np.float32).astype(np.float64)[None, :, None, None, None]
        vb = vb * np.asarray(v_scale, dtype=np.float32).astype(np.float64)[None, :, None, None]
    K = kb.transpose(0, 3, 1, 2, 4).reshape(n * block_size, hkv, d)[:L]
    V = vb.transpose(0, 3, 1, 2).reshape(n * block_size, hkv, d)[:L]
    return K, V


# ---------------------------------------------------------------------------
# textbook attention
# ---------------------------------------------------------------------------

def attend_rows(q_rows, positions, K, V, scale):
    """Textbook grouped-query attention for query rows of one sequence.

    q_rows [R, Hq, D] float64, positions [R] (absolute position of each row),
    K, V [L, Hkv, D] float64.  Row r, head hq sees keys 0..positions[r]:
        s_j = scale * q . K[j, hq // G],  p_j = exp(s_j - max s),
        out = sum_j p_j V[j, hq // G] / sum_j p_j.
    """
    R, hq_n, d = q_rows.shape
    hkv = K.shape[1]
    G = hq_n // hkv
    out = np.zeros((R, hq_n, d), dtype=np.float64)
    sc = np.float64(np.float32(scale))
    for r in range(R):
        n_vis = int(positions[r]) + 1
        for hq in range(hq_n):
            h = hq // G
            s = sc * (K[:n_vis, h, :] @ q_rows[r, hq])              # [n_vis]
            p = np.exp(s - s.max())
            out[r, hq, :] = (p @ V[:n_vis, h, :]) / p.sum()
    return out


def _q_f64(q, q_dtype):
    return storage_to_f64(q, q_dtype)


def oracle_decode(q, q_dtype, k_pool, v_pool, cache_dtype, block_tables, context_lens, scale,
                  k_scale=None, v_scale=None, block_size=16, seqs=None):
    """Decode attention: one query row per sequence at position L - 1.

    q [B, Hq, D] (storage of q_dtype).  Returns float64 [B, Hq, D]; with
    ``seqs`` only those rows are computed (the rest stay zero).
    """
    qf = _q_f64(q, q_dtype)
    B = qf.shape[0]
    out = np.zeros(qf.shape, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_sequence(k_pool, v_pool, block_tables[b], L, cache_dtype,
                               k_scale, v_scale, block_size)
        out[b:b + 1] = attend_rows(qf[b:b + 1], [L - 1], K, V, scale)
    return out


def oracle_prefill(q, q_dtype, query_start_loc, k_pool, v_pool, cache_dtype, block_tables,
                   context_lens, scale, k_scale=None, v_scale=None, block_size=16, chunks=None):
    """Causal prefill chunks over cached prefixes.

    q [total_q, Hq, D]; chunk c owns rows query_start_loc[c]..[c+1]-1, its
    context length L_c includes the chunk, so the cached prefix is
    P = L_c - C_c and row i sits at position P + i.
    """
    qf = _q_f64(q, q_dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for c in (range(len(qsl) - 1) if chunks is None else chunks):
        a, e = int(qsl[c]), int(qsl[c + 1])
        C, L = e - a, int(context_lens[c])
        if C == 0:
            continue
        P = L - C
        if P < 0:
            raise ValueError("chunk longer than its context")
        K, V = gather_sequence(k_pool, v_pool, block_tables[c], L, cache_dtype,
                               k_scale, v_scale, block_size)
        out[a:e] = attend_rows(qf[a:e], np.arange(P, P + C), K, V, scale)
    return out


# ---------------------------------------------------------------------------
# split-K partitions and their combine
# ---------------------------------------------------------------------------

def oracle_partitions(q, q_dtype, k_pool, v_pool, cache_dtype, block_tables, context_lens, scale,
                      partition_size, max_partitions, k_scale=None, v_scale=None, block_size=16,
                      seqs=None):
    """Per-partition softmax statistics of a decode row.

    Partition p of sequence b covers positions p*PS .. min(L, (p+1)*PS) - 1.
    For each query head: m_p = max s_j, l_p = sum exp(s_j - m_p),
    o_p = sum exp(s_j - m_p) V_j / l_p.  Arrays are [B, Hq, Pmax] and
    [B, Hq, Pmax, D]; partitions past ceil(L / PS) are NaN.
    """
    qf = _q_f64(q, q_dtype)
    B, hq_n, d = qf.shape
    m = np.full((B, hq_n, max_partitions), np.nan)
    l = np.full((B, hq_n, max_partitions), np.nan)
    o = np.full((B, hq_n, max_partitions, d), np.nan)
    sc = np.float64(np.float32(scale))
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_sequence(k_pool, v_pool, block_tables[b], L, cache_dtype,
                               k_scale, v_scale, block_size)
        hkv = K.shape[1]
        G = hq_n // hkv
        nparts = -(-L // partition_size)
        if nparts > max_partitions:
            raise ValueError("context needs more partitions than max_partitions")
        for p in range(nparts):
            a, e = p * partition_size, min(L, (p + 1) * partition_size)
            for hq in range(hq_n):
                h = hq // G
                s = sc * (K[a:e, h, :] @ qf[b, hq])
                mp = s.max()
                w = np.exp(s - mp)
                m[b, hq, p] = mp
                l[b, hq, p] = w.sum()
                o[b, hq, p] = (w @ V[a:e, h, :]) / w.sum()
    return m, l, o


def oracle_combine(part_max, part_sum, part_out, context_lens, partition_size):
    """Merge partition statistics into the attention output.

    For each (b, hq) with P = ceil(L_b / PS) partitions:
        M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
    L_b == 0 gives zeros.
    """
    B, hq_n, _ = part_max.shape
    d = part_out.shape[3]
    out = np.zeros((B, hq_n, d), dtype=np.float64)
    for b in range(B):
        P = -(-int(context_lens[b]) // partition_size)
        if P == 0:
            continue
        for hq in range(hq_n):
            mp = np.asarray(part_max[b, hq, :P], dtype=np.float64)
            lp = np.asarray(part_sum[b, hq, :P], dtype=np.float64)
            op = np.asarray(part_out[b, hq, :P], dtype=np.float64)
            M = mp.max()
            w = lp * np.exp(mp - M)
            out[b, hq] = (w @ op) / w.sum()
    return out


def num_partitions(context_len, partition_size):
    return int(math.ceil(int(context_len) / partition_size))
