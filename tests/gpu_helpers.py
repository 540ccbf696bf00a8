"""Shared set-up for the GPU parity tests: the same seeded workload feeds the
HIP path (through the C ABI) and the fp64 oracle (on host copies)."""

import numpy as np
import torch

from oracle import paged_attention as opa
from paged_kv_cache_234_amd import (KVPool, decode_plan_buffer, pa_decode, pa_decode_cascade,
                                    pa_decode_multi, pa_decode_plan, pa_decode_splitk_reduce,
                                    pa_prefill_chunk)

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 3e-2}
POISON = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}


def i32(a, device="cuda"):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=device)


def host(t):
    """Raw host copy (bf16 as uint16 bit patterns)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def gpu_pool(w, device="cuda", without_new=False):
    """Poisoned pool filled through pa_kv_append with every occupied slot (or
    every slot but those of this step's new decode tokens)."""
    pool = KVPool(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype, device=device,
                  k_scale=w.k_scale, v_scale=w.v_scale)
    rows = np.arange(len(w.fill_slots))
    if without_new:
        new = set(int(r) for r, s in zip(w.new_rows, w.new_slots) if s >= 0)
        rows = np.array([r for r in rows if r not in new], dtype=np.int64)
    idx = torch.as_tensor(rows, device=w.fill_k.device)
    pool.append(w.fill_k[idx].to(device).contiguous(), w.fill_v[idx].to(device).contiguous(),
                i32(w.fill_slots[rows], device))
    return pool


def decode_new_tokens(w, device="cuda"):
    """Per decode sequence: its newest token's K/V [B, Hkv, D] and slot [B]
    (-1 for L = 0 or when the token sits in a prefix-shared block)."""
    B = w.batch
    rows = np.zeros(B, np.int64)
    slots = np.full(B, -1, np.int32)
    j = 0
    for b in range(B):
        if int(w.context_lens[b]) == 0:
            continue
        rows[b] = w.new_rows[j]
        slots[b] = w.new_slots[j]
        j += 1
    idx = torch.as_tensor(rows, device=w.fill_k.device)
    k = w.fill_k[idx].to(device).contiguous()
    v = w.fill_v[idx].to(device).contiguous()
    return k, v, i32(slots, device)


def oracle_pool(w, seqs=None, chunks=None):
    """The oracle's own pool: poisoned, then oracle_append of the fill set
    (restricted to the slots of the given decode sequences / chunks)."""
    st = opa.STORAGE_DTYPES[w.cache_dtype]
    shape_k, shape_v = opa.pool_shapes(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype,
                                       w.block_size)
    kp = np.full(shape_k, POISON[w.cache_dtype], dtype=st)
    vp = np.full(shape_v, POISON[w.cache_dtype], dtype=st)
    rows = np.arange(len(w.fill_slots))
    if seqs is not None or chunks is not None:
        blocks = set()
        for b in (seqs or []):
            n = -(-int(w.context_lens[b]) // w.block_size)
            blocks.update(int(x) for x in w.block_tables[b, :n])
        for c in (chunks or []):
            n = -(-int(w.chunk_context_lens[c]) // w.block_size)
            blocks.update(int(x) for x in w.chunk_block_tables[c, :n])
        sel = np.isin(w.fill_slots // w.block_size, np.fromiter(blocks, dtype=np.int64))
        rows = rows[sel]
    idx = torch.as_tensor(rows, device=w.fill_k.device)
    fk = host(w.fill_k[idx])
    fv = host(w.fill_v[idx])
    return opa.oracle_append(kp, vp, fk, fv, w.fill_slots[rows], w.in_dtype, w.cache_dtype,
                             w.k_scale, w.v_scale, w.block_size)


def run_decode(w, pool, partition_size=0, q=None, block_tables=None, context_lens=None,
               device="cuda"):
    """Decode through the C ABI; split-K runs pa_decode + pa_decode_splitk_reduce.
    Returns (out, (part_max, part_sum, part_out) or None)."""
    q = (w.q if q is None else q).to(device).contiguous()
    bt = i32(w.block_tables if block_tables is None else block_tables, device)
    lens_np = w.context_lens if context_lens is None else context_lens
    lens = i32(lens_np, device)
    out = torch.empty_like(q)
    if partition_size == 0:
        pa_decode(out, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale, pool.v_scale)
        return out, None
    pmax = max(1, -(-int(np.max(lens_np)) // partition_size)) if len(lens_np) else 1
    B, hq, d = q.shape
    pm = torch.full((B, hq, pmax), float("nan"), device=device)
    ps = torch.full((B, hq, pmax), float("nan"), device=device)
    po = torch.full((B, hq, pmax, d), float("nan"), device=device)
    pa_decode(None, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale, pool.v_scale,
              partition_size=partition_size, max_partitions=pmax, part_max=pm, part_sum=ps,
              part_out=po)
    pa_decode_splitk_reduce(out, pm, ps, po, lens, partition_size)
    return out, (pm, ps, po)


def run_prefill(w, pool, device="cuda"):
    qp = w.q_prefill.to(device).contiguous()
    out = torch.full_like(qp, float("nan"))       # a row the launch skips stays NaN
    qsl = w.query_start_loc
    maxq = int(np.max(np.diff(qsl))) if len(qsl) > 1 else 0
    pa_prefill_chunk(out, qp, i32(qsl, device), maxq, pool.k, pool.v,
                     i32(w.chunk_block_tables, device), i32(w.chunk_context_lens, device), w.scale,
                     pool.k_scale, pool.v_scale)
    return out


def as_f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_abs_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - want))) if got.size else 0.0


def group_arrays(w, extra_empty_groups=0, device="cuda"):
    """group_start / group_seqs / group_prefix_lens for the workload's prefix
    groups (prefix = the shared blocks' positions); optionally followed by
    groups without members."""
    start, seqs, plens = [0], [], []
    for members, nshared in w.prefix_groups:
        seqs.extend(int(b) for b in members)
        start.append(len(seqs))
        plens.append(int(nshared) * w.block_size)
    for _ in range(extra_empty_groups):
        start.append(len(seqs))
        plens.append(64)
    mg = max([len(m) for m, _ in w.prefix_groups] + [0])
    seqs = seqs or [0]            # never read when no group has members
    return i32(start, device), i32(seqs, device), i32(plens, device), mg


def run_cascade(w, pool, partition_size, extra_empty_groups=0, device="cuda", planned=False,
                appended=None):
    """pa_decode_cascade + pa_decode_splitk_reduce (optionally through a
    launch plan, optionally appending (k_new, v_new, new_slots) in the same
    launch); returns (out, (pm, ps, po))."""
    q = w.q.to(device).contiguous()
    bt, lens = i32(w.block_tables, device), i32(w.context_lens, device)
    pmax = max(1, -(-int(np.max(w.context_lens)) // partition_size))
    B, hq, d = q.shape
    pm = torch.full((B, hq, pmax), float("nan"), device=device)
    ps = torch.full((B, hq, pmax), float("nan"), device=device)
    po = torch.full((B, hq, pmax, d), float("nan"), device=device)
    gs, gq, gp, mg = group_arrays(w, extra_empty_groups, device)
    plan = None
    if planned:
        plan = decode_plan_buffer(B + gs.numel() - 1, pool.k, d, device)
        pa_decode_plan(plan, bt, lens, w.num_heads, pool.k, pool.v, partition_size, pmax,
                       groups=(gs, gq, gp, mg),
                       new_slots=appended[2] if appended else None)
    kw = dict(zip(("k_new", "v_new", "new_slots"), appended)) if appended else {}
    pa_decode_cascade(q, pool.k, pool.v, bt, lens, w.scale, gs, gq, gp, mg, partition_size, pmax,
                      pm, ps, po, pool.k_scale, pool.v_scale, plan=plan, **kw)
    out = torch.empty_like(q)
    pa_decode_splitk_reduce(out, pm, ps, po, lens, partition_size)
    return out, (pm, ps, po)


def token_lens(w):
    """Visible context of every chunk row: P_c + i + 1 for row i of chunk c."""
    out = []
    for c in range(w.num_chunks):
        q0, q1 = int(w.query_start_loc[c]), int(w.query_start_loc[c + 1])
        P = int(w.chunk_context_lens[c]) - (q1 - q0)
        out.extend(P + i + 1 for i in range(q1 - q0))
    return np.asarray(out, np.int64)


def chunk_new_tokens(w, device="cuda"):
    """The chunks' query tokens, in q_prefill's row order: K/V [T, Hkv, D]
    and their slots [T] (the last T entries of the step's new tokens)."""
    T = int(w.query_start_loc[-1])
    rows, slots = w.new_rows[len(w.new_rows) - T:], w.new_slots[len(w.new_slots) - T:]
    idx = torch.as_tensor(rows, device=w.fill_k.device)
    return (w.fill_k[idx].to(device).contiguous(), w.fill_v[idx].to(device).contiguous(),
            i32(slots, device))


def run_multi(w, pool, partition_size, device="cuda", planned=False, appended=None,
              plan_lists=True):
    """pa_decode_multi over the workload's chunks (optionally through a
    launch plan, optionally appending (k_new, v_new, new_slots) in the same
    launch; plan_lists: the plan is made with those new_slots) +
    pa_decode_splitk_reduce over their rows; returns (out, (pm, ps, po),
    token_lens)."""
    qp = w.q_prefill.to(device).contiguous()
    T, hq, d = qp.shape
    qsl = w.query_start_loc
    maxq = int(np.max(np.diff(qsl))) if len(qsl) > 1 else 0
    tl = token_lens(w)
    pmax = max(1, -(-int(np.max(w.chunk_context_lens)) // partition_size))
    pm = torch.full((T, hq, pmax), float("nan"), device=device)
    ps = torch.full((T, hq, pmax), float("nan"), device=device)
    po = torch.full((T, hq, pmax, d), float("nan"), device=device)
    qslt, cbt, clens = (i32(qsl, device), i32(w.chunk_block_tables, device),
                        i32(w.chunk_context_lens, device))
    plan = None
    if planned:
        plan = decode_plan_buffer(w.num_chunks, pool.k, d, device)
        pa_decode_plan(plan, cbt, clens, w.num_heads, pool.k, pool.v, partition_size, pmax,
                       queries=(qslt, maxq),
                       new_slots=appended[2] if appended and plan_lists else None)
    kw = dict(zip(("k_new", "v_new", "new_slots"), appended)) if appended else {}
    pa_decode_multi(qp, qslt, maxq, pool.k, pool.v, cbt, clens, w.scale, partition_size, pmax, pm,
                    ps, po, pool.k_scale, pool.v_scale, plan=plan, **kw)
    out = torch.empty_like(qp)
    pa_decode_splitk_reduce(out, pm, ps, po, i32(tl, device), partition_size)
    return out, (pm, ps, po), tl
