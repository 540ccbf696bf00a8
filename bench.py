"""Benchmark one paged-attention layer-step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole hot path over one batch: pa_kv_append of the
step's new tokens, split-K pa_decode, pa_decode_splitk_reduce, and for the
mixed workload (config 5) pa_prefill_chunk.  Inputs are resident in HBM
before timing starts.  The pool of every step is a different layer copy
(rotating over R copies, R * pool >= 1 GiB), so each step reads its KV from
HBM rather than from the 256 MB Infinity Cache, as a real layer-step does.

Prints one JSON line: the headline metric is KV GB/s of the whole step
(logical KV bytes read / step time), with us per layer-step, the fraction of
the 8 TB/s HBM peak, per-kernel HIP-event durations, the roofline of the
decode kernel and the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-decode KV GB/s (% of HBM peak) + µs per layer-step, 1×MI355X"
HBM_PEAK_GBPS = 8000.0
# Plain decode steps read their launch prologue from a plan made once per
# model step for all its layers: one pa_decode_plan per PLAN_LAYERS
# layer-steps (32 is Llama-3-8B's layer count; Qwen2.5-3B has 36).
PLAN_LAYERS = 32
# split-K partition per workload: 256 for bf16 sequence batches (8 tiles of
# 32 tokens per item; the prefix-shared batch also needs its 256-token prefix
# to be whole partitions), 512 for the long-context batch (its definition),
# 1024 for the fp8 mixed batch (16 tiles of 64 tokens per item: at 256 the
# per-item cost of 4-tile items dominates), 512 for draft verification
DEFAULT_PS = {1: 64, 2: 256, 3: 256, 4: 512, 5: 1024}
SPEC_VERIFY_PS = 512


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--workload", default=None, choices=["spec-verify"],
                    help="instead of a numbered config: the draft-verification step "
                         "(pa_decode_multi over U[2, 8] causal query tokens per sequence)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-fuse-append", action="store_true",
                    help="append the decode tokens with pa_kv_append before pa_decode instead of "
                         "pa_decode_append's single launch")
    ap.add_argument("--no-plan", action="store_true",
                    help="plain decode launches compute their prologue instead of reading a "
                         "per-step plan")
    ap.add_argument("--no-cascade", action="store_true",
                    help="decode prefix-sharing batches with pa_decode instead of pa_decode_cascade")
    ap.add_argument("--eager", action="store_true",
                    help="launch the kernels one by one instead of replaying captured graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU budget of the oracle baseline")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the paged-attention path here is built and timed on "
              "a single MI355X (no sharding, no collectives); --gpus %d is not supported"
              % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_234_amd import (KVPool, decode_plan_buffer, pa_decode, pa_decode_append,
                                        pa_decode_plan, pa_decode_cascade,
                                        pa_decode_multi, pa_decode_splitk_reduce, pa_prefill_chunk,
                                        pa_selftest)
    from workloads import make_config, make_spec_verify

    dev = "cuda:0"
    torch.cuda.set_device(0)
    pa_selftest()
    spec = args.workload == "spec-verify"
    if spec:
        w = make_spec_verify(device=dev) if args.seed is None else make_spec_verify(args.seed, dev)
        ps = SPEC_VERIFY_PS if args.partition_size is None else args.partition_size
        if ps <= 0:
            raise SystemExit("the draft-verification step is split-K only (--partition-size > 0)")
    else:
        w = make_config(args.config, seed=args.seed, device=dev)
        ps = DEFAULT_PS[args.config] if args.partition_size is None else args.partition_size

    def i32(a):
        return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=dev)

    # ---- resident inputs ---------------------------------------------------
    R = max(2, math.ceil((1 << 30) / w.pool_bytes()))
    pools = []
    fill_slots = i32(w.fill_slots)
    for _ in range(R):
        p = KVPool(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype, device=dev,
                   poison=False, k_scale=w.k_scale, v_scale=w.v_scale)
        p.append(w.fill_k, w.fill_v, fill_slots)
        pools.append(p)
    new_k, new_v = w.new_k.contiguous(), w.new_v.contiguous()
    new_slots = i32(w.new_slots)
    if spec:
        # the query tokens are the rows of the workload's chunks
        q = w.q_prefill.contiguous()
        lens, bt = i32(w.chunk_context_lens), i32(w.chunk_block_tables)
        qsl = i32(w.query_start_loc)
        max_q = int(np.max(np.diff(w.query_start_loc)))
        tok_lens = []
        for c in range(w.num_chunks):
            n = int(w.query_start_loc[c + 1] - w.query_start_loc[c])
            tok_lens.extend(int(w.chunk_context_lens[c]) - n + i + 1 for i in range(n))
        tok_lens = i32(tok_lens)
        pmax = max(1, -(-int(np.max(w.chunk_context_lens)) // ps))
    else:
        q = w.q.contiguous()
        lens, bt = i32(w.context_lens), i32(w.block_tables)
        pmax = w.max_partitions(ps)
    B, hq, d = q.shape
    part_max = torch.empty((B, hq, pmax), device=dev)
    part_sum = torch.empty((B, hq, pmax), device=dev)
    part_out = torch.empty((B, hq, pmax, d), device=dev)
    out = torch.empty_like(q)
    # prefix groups: the shared blocks are read once per group (cascade)
    cascade = bool(w.prefix_groups) and ps > 0 and not args.no_cascade
    if cascade:
        g_start, g_seqs, g_plens = [0], [], []
        for members, nshared in w.prefix_groups:
            g_seqs.extend(int(b) for b in members)
            g_start.append(len(g_seqs))
            g_plens.append(int(nshared) * w.block_size)
        g_start, g_seqs, g_plens = i32(g_start), i32(g_seqs), i32(g_plens)
        g_max = max(len(m) for m, _ in w.prefix_groups)
    has_prefill = w.num_chunks > 0 and not spec
    # plain and cascade decode steps append each sequence's new token inside
    # the decode launch (fused: the plain step's pa_decode_append)
    fuse_append = not (spec or has_prefill or args.no_fuse_append)
    fused = fuse_append and not cascade
    if fuse_append:
        rows = np.zeros(B, np.int64)
        fslots = np.full(B, -1, np.int32)
        j = 0
        for b in range(B):
            if int(w.context_lens[b]) > 0:
                rows[b], fslots[b] = w.new_rows[j], w.new_slots[j]
                j += 1
        ridx = torch.as_tensor(rows, device=dev)
        fk, fv, fslots = w.fill_k[ridx].contiguous(), w.fill_v[ridx].contiguous(), i32(fslots)
    # every decode launch reads its prologue from a plan made once per model
    # step (the plain decode of the mixed step through pa_decode_append with
    # no append arrays)
    planned = not args.no_plan
    plan = None
    if planned:
        plan = decode_plan_buffer(B + (len(w.prefix_groups) if cascade else 0), pools[0].k, d)

    def make_plan():
        extra = {}
        if spec:
            extra = dict(queries=(qsl, max_q))
        elif cascade:
            extra = dict(groups=(g_start, g_seqs, g_plens, g_max))
        pa_decode_plan(plan, bt, lens, w.num_heads, pools[0].k, pools[0].v, partition_size=ps,
                       max_partitions=pmax, new_slots=fslots if fuse_append else None, **extra)
    if has_prefill:
        qp = w.q_prefill.contiguous()
        outp = torch.empty_like(qp)
        qsl = i32(w.query_start_loc)
        maxq = int(np.max(np.diff(w.query_start_loc)))
        cbt, clens = i32(w.chunk_block_tables), i32(w.chunk_context_lens)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(layer, ev=None):
        pool = pools[layer % R]
        if ev is not None:
            ev[0].record(stream)
        if planned and layer % PLAN_LAYERS == 0:
            make_plan()
        if not fuse_append:
            pool.append(new_k, new_v, new_slots)
        if ev is not None:
            ev[1].record(stream)
        decode_only(layer)
        if ev is not None:
            ev[2].record(stream)
        if spec:
            pa_decode_splitk_reduce(out, part_max, part_sum, part_out, tok_lens, ps)
        elif ps > 0:
            pa_decode_splitk_reduce(out, part_max, part_sum, part_out, lens, ps)
        if ev is not None:
            ev[3].record(stream)
        if has_prefill:
            pa_prefill_chunk(outp, qp, qsl, maxq, pool.k, pool.v, cbt, clens, w.scale,
                             pool.k_scale, pool.v_scale)
            if ev is not None:
                ev[4].record(stream)

    def decode_only(layer):
        pool = pools[layer % R]
        if fused:
            pa_decode_append(out if ps == 0 else None, q, fk, fv, fslots, pool.k, pool.v, bt, lens,
                             w.scale, pool.k_scale, pool.v_scale, partition_size=ps,
                             max_partitions=pmax, part_max=part_max, part_sum=part_sum,
                             part_out=part_out, plan=plan)
        elif spec:
            pa_decode_multi(q, qsl, max_q, pool.k, pool.v, bt, lens, w.scale, ps, pmax, part_max,
                            part_sum, part_out, pool.k_scale, pool.v_scale, plan=plan)
        elif cascade:
            appended = dict(k_new=fk, v_new=fv, new_slots=fslots) if fuse_append else {}
            pa_decode_cascade(q, pool.k, pool.v, bt, lens, w.scale, g_start, g_seqs, g_plens, g_max,
                              ps, pmax, part_max, part_sum, part_out, pool.k_scale, pool.v_scale,
                              plan=plan, **appended)
        elif planned:
            pa_decode_append(out if ps == 0 else None, q, None, None, None, pool.k, pool.v, bt,
                             lens, w.scale, pool.k_scale, pool.v_scale, partition_size=ps,
                             max_partitions=pmax, part_max=part_max, part_sum=part_sum,
                             part_out=part_out, plan=plan)
        elif ps > 0:
            pa_decode(None, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale, pool.v_scale,
                      partition_size=ps, max_partitions=pmax, part_max=part_max,
                      part_sum=part_sum, part_out=part_out)
        else:
            pa_decode(out, q, pool.k, pool.v, bt, lens, w.scale, pool.k_scale, pool.v_scale)

    if planned:
        make_plan()
    for i in range(max(args.warmup, 1)):
        step(i)
        decode_only(i)
    torch.cuda.synchronize()

    # The engines on the pages replay their decode step as a captured graph
    # covering every layer; here one graph holds the K timed layer-steps (each
    # on the next layer copy), another the warm-up steps, a third the K
    # decode kernels alone.
    def steps_of(fn, first, count):
        for i in range(count):
            fn(first + i)

    def captured(fn, first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            steps_of(fn, first, count)
        return g

    if not args.eager:
        g_warm = captured(step, 0, max(args.warmup, 1))
        g_steps = captured(step, args.warmup, args.steps)
        g_decode = captured(decode_only, args.warmup, args.steps)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        g_warm.replay()
    else:
        steps_of(step, 0, args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ------------------------------------
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    if args.eager:
        steps_of(step, args.warmup, args.steps)
    else:
        g_steps.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # ---- the decode kernel alone: K back-to-back launches between two events
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    if args.eager:
        steps_of(decode_only, args.warmup, args.steps)
    else:
        g_decode.replay()
    d1.record(stream)
    torch.cuda.synchronize()
    decode_ms = d0.elapsed_time(d1) / args.steps

    # ---- per-kernel durations, eager, HIP events around each launch ---------
    nev = 5 if has_prefill else 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    names = (["(append fused)" + (", plan / %d layers" % PLAN_LAYERS if planned else ""),
              "decode_append" if fused else "decode"] if fuse_append else
             ["kv_append", "decode"]) + \
        ["splitk_reduce", "prefill_chunk"]
    names = names[:nev - 1]
    kern_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
               for j, n in enumerate(names)}

    # ---- accounting -----------------------------------------------------------
    kv_logical = w.prefill_kv_bytes() if spec else w.decode_kv_bytes_logical()
    kv_unique = w.prefill_kv_bytes() if spec else w.decode_kv_bytes_unique()
    step_bytes = kv_logical + (w.prefill_kv_bytes() if has_prefill else 0)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_unique / (decode_ms * 1e-3) / 1e9

    # achievable copy bandwidth, same process (context for the peak)
    nbytes = 1 << 30
    src = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    result_entry = ("pa_decode_append" if fused or (planned and not (spec or cascade)) else
                    "pa_decode_multi" if spec else "pa_decode_cascade" if cascade else "pa_decode")
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cache_dtype if w.cache_dtype != "fp8" else "fp8-e4m3 KV, bf16 Q",
        "data": "synthetic (seeded; no dataset, no weights)",
        "config": {
            "workload": w.name, "seed": w.seed, "batch": w.num_chunks if spec else w.batch,
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size,
            "context_tokens": int((w.chunk_context_lens if spec else w.context_lens).sum()),
            "new_tokens": int(len(w.new_slots)),
            "prefill_chunks": w.num_chunks, "partition_size": ps, "max_partitions": pmax,
            "pool_blocks": w.num_blocks, "layer_copies": R,
            "decode_entry": result_entry,
            "plan": ("pa_decode_plan once per %d layer-steps" % PLAN_LAYERS) if planned else None,
            "step_entries": ("pa_decode_cascade (append fused) + pa_decode_splitk_reduce"
                             if fuse_append and cascade else
                             "pa_decode_append + pa_decode_splitk_reduce" if fused and ps > 0
                             else "pa_decode_append" if fused
                             else "pa_kv_append + %s%s%s" % (
                                 result_entry,
                                 " + pa_decode_splitk_reduce" if ps > 0 else "",
                                 " + pa_prefill_chunk" if has_prefill else "")),
        },
        "us_per_layer_step": round(ms_per_step * 1e3, 3),
        "pct_hbm_peak": round(100.0 * (kv_unique / (ms_per_step * 1e-3) / 1e9) / HBM_PEAK_GBPS, 2),
        "kv_bytes_logical": kv_logical,
        "kv_bytes_unique": kv_unique,
        "launch": "eager" if args.eager else "one HIP graph holding the K layer-steps",
        "decode_kernel_us": round(decode_ms * 1e3, 3),
        "eager_event_us": {k: round(v * 1e3, 3) for k, v in kern_ms.items()},
        "copy_GBps": round(copy_gbps, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": result_entry,
            "duration_us": round(decode_ms * 1e3, 3),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(w.name, ps, result_entry),
        },
    }
    if has_prefill:
        pf_ms = kern_ms["prefill_chunk"]
        result["prefill_tflops"] = round(w.prefill_flops() / (pf_ms * 1e-3) / 1e12, 2)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, ms_per_step, kv_logical)
    print(json.dumps(result), flush=True)


def decode_source_hash():
    """sha256 of the decode kernel's sources with comments and blank lines
    removed (the key under which profiles/ stores measured HBM traffic)."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_234_amd", "csrc")
    for f in ("pa_decode.hip", "pa_tiles.hpp", "pa_device.hpp", "pa_internal.hpp", "pa_write.hpp"):
        with open(os.path.join(csrc, f)) as fh:
            lines = [re.sub(r"//.*", "", ln).rstrip() for ln in fh.read().splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()


def measured_traffic(workload, ps, entry):
    """HBM bytes per decode launch from the FETCH_SIZE / WRITE_SIZE counter
    runs summarised under profiles/ (copy-calibrated), or None when no
    summary matches this workload, partition size, entry point and decode
    source."""
    import glob
    want = {"workload": workload, "partition_size": str(ps), "decode_entry": entry,
            "decode_source_sha256": decode_source_hash()}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_bytes.md"))):
        kv = {}
        with open(path) as fh:
            for ln in fh:
                if ":" in ln and not ln.startswith(("|", "#", " ")):
                    k, v = ln.split(":", 1)
                    kv[k.strip()] = v.strip()
        if all(kv.get(k) == v for k, v in want.items()) and "traffic_bytes_per_launch" in kv:
            return int(kv["traffic_bytes_per_launch"])
    return None


def cpu_baseline(w, budget_s, gpu_ms, gpu_bytes):
    """The fp64 oracle, as it stands, on a bounded sample of the workload's
    decode sequences (or, for a workload of chunks only, its chunks); scaled
    to the metric's unit (KV GB/s)."""
    from oracle import paged_attention as opa
    import torch
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))

    def raw(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    chunks_only = w.batch == 0
    n_units = w.num_chunks if chunks_only else w.batch
    lens_of = w.chunk_context_lens if chunks_only else w.context_lens
    tables_of = w.chunk_block_tables if chunks_only else w.block_tables
    rng = np.random.default_rng(0)
    order = rng.permutation(n_units)
    st = opa.STORAGE_DTYPES[w.cache_dtype]
    shape_k, shape_v = opa.pool_shapes(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype,
                                       w.block_size)
    kp = np.zeros(shape_k, st)
    vp = np.zeros(shape_v, st)
    qh = raw(w.q_prefill if chunks_only else w.q)
    # The first pass fills the oracle's pool sequence by sequence (untimed)
    # and times each sequence; when the whole workload takes less than the
    # budget, further passes over the same pool repeat the timed part.
    done, tokens, elapsed, passes = [], 0, 0.0, 0
    while elapsed < budget_s or not done:          # at least one sequence
        for b in order:
            if passes == 0:
                n = -(-int(lens_of[b]) // w.block_size)
                blocks = tables_of[b, :n].astype(np.int64)
                sel = np.flatnonzero(np.isin(w.fill_slots // w.block_size, blocks))
                idx = torch.as_tensor(sel, device=w.fill_k.device)
                kp, vp = opa.oracle_append(kp, vp, raw(w.fill_k[idx]), raw(w.fill_v[idx]),
                                           w.fill_slots[sel], w.in_dtype, w.cache_dtype,
                                           w.k_scale, w.v_scale, w.block_size)
            elif int(b) not in done_set:
                continue
            t = time.perf_counter()
            if chunks_only:
                opa.oracle_prefill(qh, w.q_dtype, w.query_start_loc, kp, vp, w.cache_dtype,
                                   w.chunk_block_tables, w.chunk_context_lens, w.scale, w.k_scale,
                                   w.v_scale, w.block_size, chunks=[int(b)])
            else:
                opa.oracle_decode(qh, w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                                  w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size,
                                  seqs=[int(b)])
            elapsed += time.perf_counter() - t
            if passes == 0:
                done.append(int(b))
            tokens += int(lens_of[b])
            if elapsed >= budget_s:
                break
        passes += 1
        done_set = set(done)
    kv = tokens * w.kv_bytes_per_token()
    return {
        "value": round(kv / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "fp64 oracle %s of %d of %d %s, %d pass(es) (%d context tokens, %.1f s), "
                  "host affinity %d cores" % ("causal chunks" if chunks_only else "decode",
                                              len(done), n_units,
                                              "sequences' query tokens" if chunks_only else
                                              "sequences", passes, tokens, elapsed,
                                              len(os.sched_getaffinity(0))),
        "seconds": round(elapsed, 3),
        "gpu_over_cpu": round((gpu_bytes / (gpu_ms * 1e-3)) / (kv / elapsed), 1)
        if elapsed > 0 else None,
    }


if __name__ == "__main__":
    main()
