"""A captured layer-step (append + split-K decode + reduce + prefill chunk)
replays to exactly the eager result, replay after replay, with eager work and
synchronisations in between, and every replay matches the fp64 oracle (the
engines on the pages capture each decode step in a graph: InferX milestone
M6, llm-infer "What It Does", RustInfer).  The full-size step bench.py
captures is covered in test_gpu_full_size.py."""

import numpy as np
import pytest
import torch

from paged_kv_cache_234_amd import (pa_decode, pa_decode_splitk_reduce, pa_kv_append,
                                    pa_prefill_chunk)
from oracle import paged_attention as opa
from tests.gpu_helpers import TOL, as_f64, gpu_pool, host, i32, max_abs_err, oracle_pool
from workloads import build_workload

pytestmark = pytest.mark.gpu


def _oracle(w):
    """Decode rows and prefill rows of the workload, fp64 oracle."""
    kp, vp = oracle_pool(w)
    dec = opa.oracle_decode(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                            w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size)
    pre = opa.oracle_prefill(host(w.q_prefill), w.q_dtype, w.query_start_loc, kp, vp,
                             w.cache_dtype, w.chunk_block_tables, w.chunk_context_lens, w.scale,
                             w.k_scale, w.v_scale, w.block_size)
    return dec, pre


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_graph_replays_equal_eager(cache):
    w = build_workload("g", seed=31, device="cuda", cache_dtype=cache, num_heads=16,
                       num_kv_heads=4, head_dim=128, decode_lens=[1, 33, 700, 2000, 65],
                       prefill_chunks=[(40, 70)])
    pool = gpu_pool(w)
    ps = 64
    q = w.q.contiguous()
    B, hq, d = q.shape
    pmax = w.max_partitions(ps)
    pm = torch.empty((B, hq, pmax), device="cuda")
    psum = torch.empty_like(pm)
    po = torch.empty((B, hq, pmax, d), device="cuda")
    out = torch.empty_like(q)
    qp = w.q_prefill.contiguous()
    outp = torch.empty_like(qp)
    lens, bt = i32(w.context_lens), i32(w.block_tables)
    qsl, cbt, clens = i32(w.query_start_loc), i32(w.chunk_block_tables), i32(w.chunk_context_lens)
    nk, nv, ns = w.new_k.contiguous(), w.new_v.contiguous(), i32(w.new_slots)

    def step():
        pa_kv_append(nk, nv, pool.k, pool.v, ns, pool.k_scale, pool.v_scale)
        pa_decode(None, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale, pool.v_scale,
                  partition_size=ps, max_partitions=pmax, part_max=pm, part_sum=psum,
                  part_out=po)
        pa_decode_splitk_reduce(out, pm, psum, po, lens, ps)
        pa_prefill_chunk(outp, qp, qsl, 70, pool.k, pool.v, cbt, clens, w.scale, pool.k_scale,
                         pool.v_scale)

    step()
    torch.cuda.synchronize()
    ref, refp = out.clone(), outp.clone()
    kref, vref = pool.k.clone(), pool.v.clone()
    dec, pre = _oracle(w)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        outp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "decode output differs on replay %d" % rep
        assert torch.equal(outp, refp), "prefill output differs on replay %d" % rep
        assert max_abs_err(as_f64(out), dec) <= TOL[cache]
        assert max_abs_err(as_f64(outp), pre) <= TOL[cache]
        # bytes, not values: unowned slots hold NaN patterns
        assert torch.equal(pool.k.view(torch.uint8), kref.view(torch.uint8))
        assert torch.equal(pool.v.view(torch.uint8), vref.view(torch.uint8))
        # unrelated eager work between replays
        x = torch.randn(1024, 1024, device="cuda")
        (x @ x).sum().item()


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_two_stream_graph_replays_equal_serial_eager(cache):
    """The mixed step with the prefill forked onto a second stream after the
    append and joined before the step ends (decode + reduce on the first):
    every replay, and an eager two-stream run, equal the serial eager step
    bit for bit, with a later step's append ordered after the join."""
    w = build_workload("g2", seed=37, device="cuda", cache_dtype=cache, num_heads=32,
                       num_kv_heads=8, head_dim=128, decode_lens=[5, 900, 3000, 64, 1],
                       prefill_chunks=[(200, 300), (0, 96)])
    pool = gpu_pool(w)
    ps = 256
    q = w.q.contiguous()
    B, hq, d = q.shape
    pmax = w.max_partitions(ps)
    pm = torch.empty((B, hq, pmax), device="cuda")
    psum = torch.empty_like(pm)
    po = torch.empty((B, hq, pmax, d), device="cuda")
    out = torch.empty_like(q)
    qp = w.q_prefill.contiguous()
    outp = torch.empty_like(qp)
    lens, bt = i32(w.context_lens), i32(w.block_tables)
    qsl, cbt, clens = i32(w.query_start_loc), i32(w.chunk_block_tables), i32(w.chunk_context_lens)
    nk, nv, ns = w.new_k.contiguous(), w.new_v.contiguous(), i32(w.new_slots)
    side = torch.cuda.Stream()

    def decode_reduce():
        pa_decode(None, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale, pool.v_scale,
                  partition_size=ps, max_partitions=pmax, part_max=pm, part_sum=psum,
                  part_out=po)
        pa_decode_splitk_reduce(out, pm, psum, po, lens, ps)

    def prefill():
        pa_prefill_chunk(outp, qp, qsl, 300, pool.k, pool.v, cbt, clens, w.scale, pool.k_scale,
                         pool.v_scale)

    def serial_step():
        pa_kv_append(nk, nv, pool.k, pool.v, ns, pool.k_scale, pool.v_scale)
        decode_reduce()
        prefill()

    def forked_step():
        pa_kv_append(nk, nv, pool.k, pool.v, ns, pool.k_scale, pool.v_scale)
        # the current stream: under capture, the capturing one
        main = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            prefill()
        join = torch.cuda.Event()
        join.record(side)
        decode_reduce()
        main.wait_event(join)

    serial_step()
    torch.cuda.synchronize()
    ref, refp = out.clone(), outp.clone()
    kref, vref = pool.k.clone(), pool.v.clone()

    dec, pre = _oracle(w)
    assert max_abs_err(as_f64(ref), dec) <= TOL[cache]
    assert max_abs_err(as_f64(refp), pre) <= TOL[cache]

    def check(what):
        assert torch.equal(out, ref), "decode output differs: %s" % what
        assert torch.equal(outp, refp), "prefill output differs: %s" % what
        assert torch.equal(pool.k.view(torch.uint8), kref.view(torch.uint8))
        assert torch.equal(pool.v.view(torch.uint8), vref.view(torch.uint8))

    out.fill_(float("nan"))
    outp.fill_(float("nan"))
    forked_step()
    torch.cuda.synchronize()
    check("eager two-stream step")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forked_step()
        forked_step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        outp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check("replay %d" % rep)
        x = torch.randn(1024, 1024, device="cuda")
        (x @ x).sum().item()
