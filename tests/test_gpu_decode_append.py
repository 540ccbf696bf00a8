"""pa_decode_append (each sequence's newest token appended by the decode
launch itself) against pa_kv_append + pa_decode: the same pool bytes and
bit-identical outputs and partials, on every cache type, both head sizes,
single-pass and split-K, with zero-length sequences and tokens that sit in
prefix-shared blocks (slot -1); plus the oracle."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as opa
from paged_kv_cache_234_amd import (pa_decode, pa_decode_append, pa_decode_splitk_reduce,
                                    pa_kv_append)
from tests.gpu_helpers import (TOL, as_f64, decode_new_tokens, gpu_pool, host, i32, max_abs_err,
                               oracle_pool, run_decode)
from workloads import build_workload, make_config

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 0, 250, 513, 1000, 4000]


def _run(w, pool, ps, fused):
    q = w.q.contiguous()
    B, hq, d = q.shape
    bt, lens = i32(w.block_tables), i32(w.context_lens)
    k_new, v_new, slots = decode_new_tokens(w)
    pmax = max(1, -(-int(np.max(w.context_lens)) // ps)) if ps else 1
    pm = torch.full((B, hq, pmax), float("nan"), device="cuda")
    psum = torch.full_like(pm, float("nan"))
    po = torch.full((B, hq, pmax, d), float("nan"), device="cuda")
    out = torch.empty_like(q)
    kw = dict(partition_size=ps, max_partitions=pmax, part_max=pm, part_sum=psum, part_out=po) \
        if ps else {}
    if fused:
        pa_decode_append(None if ps else out, q, k_new, v_new, slots, pool.k, pool.v, bt, lens,
                         w.scale, pool.k_scale, pool.v_scale, **kw)
    else:
        pa_kv_append(k_new, v_new, pool.k, pool.v, slots, pool.k_scale, pool.v_scale)
        pa_decode(None if ps else out, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale,
                  pool.v_scale, **kw)
    if ps:
        pa_decode_splitk_reduce(out, pm, psum, po, lens, ps)
    torch.cuda.synchronize()
    return out, (pm, psum, po)


def _check(w, ps):
    pool_a, pool_b = gpu_pool(w, without_new=True), gpu_pool(w, without_new=True)
    out_a, parts_a = _run(w, pool_a, ps, fused=False)
    out_b, parts_b = _run(w, pool_b, ps, fused=True)
    assert torch.equal(pool_a.k.view(torch.uint8), pool_b.k.view(torch.uint8))
    assert torch.equal(pool_a.v.view(torch.uint8), pool_b.v.view(torch.uint8))
    assert torch.equal(out_a, out_b)
    if ps:
        for a, b in zip(parts_a, parts_b):
            assert torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))
    return out_b


@pytest.mark.parametrize("ps", [0, 64, 256])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_fused_append_equals_append_then_decode(cache, d, ps):
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = build_workload("fa", seed=d + ps, device="cuda", q_dtype=q_dtype, cache_dtype=cache,
                       num_heads=16, num_kv_heads=2, head_dim=d, decode_lens=LENS)
    out = _check(w, ps)
    kp, vp = oracle_pool(w)
    ref = opa.oracle_decode(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                            w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size)
    assert max_abs_err(as_f64(out), ref) <= TOL[cache]


def test_fused_append_skips_tokens_in_shared_blocks():
    """Sequences whose newest token falls in a prefix-shared block carry slot
    -1: nothing is written and attention reads the shared block."""
    lens = [128, 129, 64, 300, 48, 96]
    groups = [([0, 1, 2, 3], 4), ([4, 5], 3)]
    w = build_workload("fs", seed=3, device="cuda", num_heads=8, num_kv_heads=2, head_dim=128,
                       decode_lens=lens, prefix_groups=groups)
    _, _, slots = decode_new_tokens(w)
    assert int((slots < 0).sum()) >= 2
    _check(w, 64)


@pytest.mark.parametrize("cfg,ps", [(2, 256), (4, 512)])
def test_fused_append_full_size(cfg, ps):
    _check(make_config(cfg, device="cuda"), ps)


@pytest.mark.parametrize("ps", [0, 64])
def test_decode_append_without_append_is_pa_decode(ps):
    """k_new, v_new and new_slots all None: the launch only decodes, with
    pa_decode's exact results."""
    w = build_workload("fn", seed=11 + ps, device="cuda", num_heads=16, num_kv_heads=2,
                       head_dim=128, decode_lens=LENS)
    pool = gpu_pool(w)
    want, parts_w = run_decode(w, pool, ps)
    q = w.q.contiguous()
    B, hq, d = q.shape
    out = torch.empty_like(q)
    kw = {}
    if ps:
        pmax = -(-int(np.max(w.context_lens)) // ps)
        kw = dict(partition_size=ps, max_partitions=pmax,
                  part_max=torch.full((B, hq, pmax), float("nan"), device="cuda"),
                  part_sum=torch.full((B, hq, pmax), float("nan"), device="cuda"),
                  part_out=torch.full((B, hq, pmax, d), float("nan"), device="cuda"))
    pa_decode_append(None if ps else out, q, None, None, None, pool.k, pool.v, i32(w.block_tables),
                     i32(w.context_lens), w.scale, **kw)
    if ps:
        pa_decode_splitk_reduce(out, kw["part_max"], kw["part_sum"], kw["part_out"],
                                i32(w.context_lens), ps)
    torch.cuda.synchronize()
    assert torch.equal(out, want)


def test_fused_append_ignores_a_slot_off_the_table():
    """A new_slots entry that is not the table's slot of position L - 1
    writes nothing."""
    w = build_workload("fo", seed=12, device="cuda", num_heads=8, num_kv_heads=2, head_dim=128,
                       decode_lens=[40, 70, 5])
    pool = gpu_pool(w, without_new=True)
    before_k, before_v = pool.k.clone(), pool.v.clone()
    k_new, v_new, slots = decode_new_tokens(w)
    bad = slots.clone()
    bad[:] = torch.where(bad >= 0, bad + 1, bad)       # the next slot: off the table's position
    q = w.q.contiguous()
    out = torch.empty_like(q)
    pa_decode_append(out, q, k_new, v_new, bad, pool.k, pool.v, i32(w.block_tables),
                     i32(w.context_lens), w.scale)
    torch.cuda.synchronize()
    assert torch.equal(pool.k.view(torch.uint8), before_k.view(torch.uint8))
    assert torch.equal(pool.v.view(torch.uint8), before_v.view(torch.uint8))


def _plan_for(w, pool, ps, listed=True):
    """A plan for pa_decode_append over w; listed: it also lists each
    wavefront's appended tokens (made with the launch's new_slots)."""
    from paged_kv_cache_234_amd import decode_plan_buffer, pa_decode_plan
    pmax = max(1, -(-int(np.max(w.context_lens)) // ps)) if ps else 1
    plan = decode_plan_buffer(w.batch, pool.k, w.head_dim)
    pa_decode_plan(plan, i32(w.block_tables), i32(w.context_lens), w.num_heads, pool.k, pool.v,
                   partition_size=ps, max_partitions=pmax,
                   new_slots=decode_new_tokens(w)[2] if listed else None)
    return plan


def _run_planned(w, pool, ps, plan, out_fill=float("nan")):
    q = w.q.contiguous()
    B, hq, d = q.shape
    pmax = max(1, -(-int(np.max(w.context_lens)) // ps)) if ps else 1
    pm = torch.full((B, hq, pmax), float("nan"), device="cuda")
    psum = torch.full_like(pm, float("nan"))
    po = torch.full((B, hq, pmax, d), float("nan"), device="cuda")
    out = torch.full_like(q, out_fill)
    kw = dict(partition_size=ps, max_partitions=pmax, part_max=pm, part_sum=psum, part_out=po) \
        if ps else {}
    k_new, v_new, slots = decode_new_tokens(w)
    pa_decode_append(None if ps else out, q, k_new, v_new, slots, pool.k, pool.v,
                     i32(w.block_tables), i32(w.context_lens), w.scale, pool.k_scale, pool.v_scale,
                     plan=plan, **kw)
    if ps:
        pa_decode_splitk_reduce(out, pm, psum, po, i32(w.context_lens), ps)
    torch.cuda.synchronize()
    return out, (pm, psum, po)


@pytest.mark.parametrize("listed", [True, False])
@pytest.mark.parametrize("ps", [0, 64, 256])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_planned_launch_equals_unplanned(cache, d, ps, listed):
    """A launch that reads its prologue from a plan gives the pools, outputs
    and partials of the launch that computes it, bit for bit."""
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = build_workload("fp", seed=3 * d + ps + 1, device="cuda", q_dtype=q_dtype,
                       cache_dtype=cache, num_heads=16, num_kv_heads=2, head_dim=d,
                       decode_lens=LENS)
    pool_a, pool_b = gpu_pool(w, without_new=True), gpu_pool(w, without_new=True)
    want, parts_a = _run(w, pool_a, ps, fused=True)
    plan = _plan_for(w, pool_b, ps, listed)
    got, parts_b = _run_planned(w, pool_b, ps, plan)
    assert torch.equal(pool_a.k.view(torch.uint8), pool_b.k.view(torch.uint8))
    assert torch.equal(pool_a.v.view(torch.uint8), pool_b.v.view(torch.uint8))
    assert torch.equal(got, want)
    if ps:
        for a, b in zip(parts_a, parts_b):
            assert torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))


def test_one_plan_serves_every_layer():
    """One plan, several layers' pools (different K/V, same batch): each
    launch equals its unplanned twin."""
    w = build_workload("fl", seed=21, device="cuda", num_heads=16, num_kv_heads=2, head_dim=128,
                       decode_lens=LENS * 2)
    plan = None
    for layer in range(3):
        w.fill_k = (w.fill_k.float() * (1 + 0.25 * layer)).to(w.fill_k.dtype)
        pool_a, pool_b = gpu_pool(w, without_new=True), gpu_pool(w, without_new=True)
        if plan is None:
            plan = _plan_for(w, pool_b, 64)
        want, _ = _run(w, pool_a, 64, fused=True)
        got, _ = _run_planned(w, pool_b, 64, plan)
        assert torch.equal(got, want)


@pytest.mark.parametrize("plan_ps,ps", [(64, 0), (64, 256), (0, 64)])
def test_a_plan_for_other_arguments_gives_nan(plan_ps, ps):
    """A plan made for another partition size: the launch computes and
    appends nothing, and every element of its output (or partial buffers,
    hence of the reduced output) is NaN, so the mistake cannot pass for a
    result."""
    w = build_workload("fw", seed=22, device="cuda", num_heads=16, num_kv_heads=2, head_dim=128,
                       decode_lens=[100, 700, 33])
    pool = gpu_pool(w, without_new=True)
    before_k, before_v = pool.k.clone(), pool.v.clone()
    plan = _plan_for(w, pool, plan_ps)
    got, parts = _run_planned(w, pool, ps, plan, out_fill=3.0)
    assert torch.all(torch.isnan(got))
    if ps:
        for t in parts:
            assert torch.all(torch.isnan(t))
    assert torch.equal(pool.k.view(torch.uint8), before_k.view(torch.uint8))
    assert torch.equal(pool.v.view(torch.uint8), before_v.view(torch.uint8))


@pytest.mark.parametrize("cfg,ps", [(2, 256), (4, 512), (1, 0)])
def test_planned_launch_full_size(cfg, ps):
    w = make_config(cfg, device="cuda")
    pool_a, pool_b = gpu_pool(w, without_new=True), gpu_pool(w, without_new=True)
    want, _ = _run(w, pool_a, ps, fused=True)
    got, _ = _run_planned(w, pool_b, ps, _plan_for(w, pool_b, ps))
    assert torch.equal(pool_a.k.view(torch.uint8), pool_b.k.view(torch.uint8))
    assert torch.equal(got, want)


def test_planned_append_list_overflow_falls_back_to_the_scan():
    """Waves holding more new tokens than a plan lists (4096 one-tile
    sequences over 4 KV heads: 16 per wave) scan for them as unplanned
    launches do: the same pools and outputs."""
    w = build_workload("fov", seed=41, device="cuda", num_heads=8, num_kv_heads=4, head_dim=64,
                       decode_lens=[16] * 4096)
    pool_a, pool_b = gpu_pool(w, without_new=True), gpu_pool(w, without_new=True)
    want, _ = _run(w, pool_a, 64, fused=True)
    got, _ = _run_planned(w, pool_b, 64, _plan_for(w, pool_b, 64))
    assert torch.equal(pool_a.k.view(torch.uint8), pool_b.k.view(torch.uint8))
    assert torch.equal(pool_a.v.view(torch.uint8), pool_b.v.view(torch.uint8))
    assert torch.equal(got, want)


@pytest.mark.parametrize("ps", [0, 64, 256])
@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_planned_launch_without_append_equals_pa_decode(cache, ps):
    """A plan made without new tokens, read by a launch that appends none:
    the outputs and partials of pa_decode, bit for bit."""
    from paged_kv_cache_234_amd import decode_plan_buffer, pa_decode_plan
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = build_workload("fn", seed=ps + 5, device="cuda", q_dtype=q_dtype, cache_dtype=cache,
                       num_heads=16, num_kv_heads=2, head_dim=128, decode_lens=LENS * 3)
    pool = gpu_pool(w)
    want, parts_a = run_decode(w, pool, ps)
    q = w.q.contiguous()
    B, hq, d = q.shape
    pmax = max(1, -(-int(np.max(w.context_lens)) // ps)) if ps else 1
    bt, lens = i32(w.block_tables), i32(w.context_lens)
    plan = decode_plan_buffer(B, pool.k, d)
    pa_decode_plan(plan, bt, lens, w.num_heads, pool.k, pool.v, partition_size=ps,
                   max_partitions=pmax)
    pm = torch.full((B, hq, pmax), float("nan"), device="cuda")
    psum = torch.full_like(pm, float("nan"))
    po = torch.full((B, hq, pmax, d), float("nan"), device="cuda")
    out = torch.empty_like(q)
    kw = dict(partition_size=ps, max_partitions=pmax, part_max=pm, part_sum=psum, part_out=po) \
        if ps else {}
    pa_decode_append(None if ps else out, q, None, None, None, pool.k, pool.v, bt, lens, w.scale,
                     pool.k_scale, pool.v_scale, plan=plan, **kw)
    if ps:
        pa_decode_splitk_reduce(out, pm, psum, po, lens, ps)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    if ps:
        for a, b in zip(parts_a, (pm, psum, po)):
            assert torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))


@pytest.mark.parametrize("seed", range(12))
def test_fused_append_seeded_random_configurations(seed):
    """Seeded random shapes: cache type, head size, GQA shape, partition size
    (single pass, or a multiple of 16 up to 1024), 1-48 sequences of 0-3000
    positions.  The fused launch equals pa_kv_append + pa_decode bit for bit,
    and the planned fused launch equals the unplanned one."""
    rng = np.random.default_rng(2000 + seed)
    cache = ["f32", "bf16", "fp8"][int(rng.integers(3))]
    hq, hkv = [(4, 4), (8, 2), (16, 2), (16, 1), (12, 4), (32, 8)][int(rng.integers(6))]
    d = [64, 128][int(rng.integers(2))]
    lens = [int(x) for x in rng.integers(0, 3001, size=int(rng.integers(1, 49)))]
    ps = 0 if int(rng.integers(6)) == 0 else 16 * int(rng.integers(1, 65))
    print("fused append:", seed, cache, hq, hkv, d, ps, lens, flush=True)
    w = build_workload("fr", seed=seed, device="cuda", q_dtype="f32" if cache == "f32" else "bf16",
                       cache_dtype=cache, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       decode_lens=lens)
    want = _check(w, ps)
    pool = gpu_pool(w, without_new=True)
    got, _ = _run_planned(w, pool, ps, _plan_for(w, pool, ps))
    full = gpu_pool(w)
    assert torch.equal(pool.k.view(torch.uint8), full.k.view(torch.uint8))
    assert torch.equal(pool.v.view(torch.uint8), full.v.view(torch.uint8))
    assert torch.equal(got, want)
