"""Benchmark paged-attention layer-steps on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all]

A step is one pass of the whole hot path over one batch: the append of the
step's new tokens, split-K decode, pa_decode_splitk_reduce, and for the mixed
workload pa_prefill_chunk.  The default run times every workload, one after
another in this process:

  tiny-fp32-decode                          B=4 fp32, D=64 (launch-bound)
  qwen2.5-3b-bf16-decode-b64                bf16, 16/2 heads (gate config)
  llama3-8b-bf16-decode-prefix-shared-b256  bf16, 32/8 heads, groups of 8
                                            sharing 16 blocks (gate config)
  long-context-bf16-splitk-b8               bf16, 32/8 heads, L in [32k, 128k]
  mixed-chunked-prefill-fp8kv               fp8 KV, 60 decode + 4 x 512 prefill
  qwen2.5-3b-bf16-spec-verify-b64           draft verification, 2-8 tokens each

and prints ONE JSON line.  Its headline (value, ms_per_step, config,
roofline, cpu_baseline) is the long-context batch, the largest workload that
one GPU holds; "configs" carries the same figures for every workload.

Inputs are resident in HBM before timing starts.  The pool of every step is
a different layer copy (rotating over R copies, R * pool >= 1 GiB), so each
step reads its KV from HBM rather than from the 256 MB Infinity Cache, as a
real layer-step does.  K timed steps are one captured graph, as the pages'
engines replay their decode step; the decode launches read a plan made once
per PLAN_LAYERS layer-steps, and each captured region holds its share of
plan launches (ceil(K / PLAN_LAYERS)).

Per workload: µs per layer-step, KV GB/s (logical KV bytes read / step
time), the fraction of the 8 TB/s HBM peak on unique KV bytes, per-kernel
HIP-event durations, the roofline of the decode kernel (algorithmic bytes /
its duration, HIP events on its launch stream, plus the copy-calibrated HBM
traffic that profiles/ records for the current decode sources), and the
fp64 CPU oracle timed on a bounded sample of the same workload, with all the
host's cores and with one thread.
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
# Decode launches read their prologue from a plan made once per model step
# for all its layers: one pa_decode_plan per PLAN_LAYERS layer-steps (32 is
# Llama-3-8B's layer count; Qwen2.5-3B has 36).
PLAN_LAYERS = 32
# split-K partition per workload: 256 for bf16 sequence batches (8 tiles of
# 32 tokens per item; the prefix-shared batch also needs its 256-token prefix
# to be whole partitions), 512 for the long-context batch (its definition),
# 1024 for the fp8 mixed batch (16 tiles of 64 tokens per item: at 256 the
# per-item cost of 4-tile items dominates), 512 for draft verification; the
# tiny fp32 batch uses one-tile items, which no wavefront shares
DEFAULT_PS = {1: 16, 2: 512, 3: 256, 4: 512, 5: 1024}
SPEC_VERIFY_PS = 512
HEADLINE = "long-context-bf16-splitk-b8"
# the bf16 configs the >= 70 % of HBM peak target applies to
GATE = ("qwen2.5-3b-bf16-decode-b64", "llama3-8b-bf16-decode-prefix-shared-b256")


def plan_due(layer, base):
    """Whether layer-step `layer` of a region starting at `base` remakes the
    plan: the region's first step and every PLAN_LAYERS-th after it, so a
    region of K steps holds ceil(K / PLAN_LAYERS) plan launches."""
    return (layer - base) % PLAN_LAYERS == 0


def workload_names():
    from workloads import CONFIG_NAMES, SPEC_VERIFY_NAME
    return [CONFIG_NAMES[i] for i in sorted(CONFIG_NAMES)] + [SPEC_VERIFY_NAME]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    help="all (default), or one workload name: " + ", ".join(workload_names()))
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="one numbered workload (same as --workload <its name>)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-fuse-append", action="store_true",
                    help="append the decode tokens with pa_kv_append before pa_decode instead of "
                         "pa_decode_append's single launch")
    ap.add_argument("--no-plan", action="store_true",
                    help="decode launches compute their prologue instead of reading a "
                         "per-step plan")
    ap.add_argument("--no-cascade", action="store_true",
                    help="decode prefix-sharing batches with pa_decode instead of pa_decode_cascade")
    ap.add_argument("--eager", action="store_true",
                    help="launch the kernels one by one instead of replaying captured graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=None,
                    help="CPU budget of the oracle baseline per workload, all cores (default "
                         "3 s per workload when timing all of them, 12 s for one)")
    ap.add_argument("--cpu-seconds-1t", type=float, default=None,
                    help="the same with one thread (default half of --cpu-seconds)")
    args = ap.parse_args(argv)
    names = workload_names()
    if args.config is not None:
        args.workload = names[args.config - 1]
    if args.workload != "all" and args.workload not in names:
        ap.error("unknown workload %r" % args.workload)
    if args.cpu_seconds is None:
        args.cpu_seconds = 3.0 if args.workload == "all" else 12.0
    if args.cpu_seconds_1t is None:
        args.cpu_seconds_1t = args.cpu_seconds / 2
    return args


def make_workload(name, seed, dev):
    """(workload, default partition size, draft-verification step?)"""
    from workloads import CONFIG_NAMES, SPEC_VERIFY_NAME, make_config, make_spec_verify
    if name == SPEC_VERIFY_NAME:
        w = make_spec_verify(device=dev) if seed is None else make_spec_verify(seed, dev)
        return w, SPEC_VERIFY_PS, True
    index = {v: k for k, v in CONFIG_NAMES.items()}[name]
    return make_config(index, seed=seed, device=dev), DEFAULT_PS[index], False


class LayerStep:
    """The layer-step the bench times, on device-resident inputs.

    step(layer, base) enqueues one layer-step on layer copy `layer % R` of
    the pool: the append of the step's new tokens (inside the decode launch,
    but for the mixed step's chunk tokens), pa_decode_plan when
    plan_due(layer, base), the decode launch, pa_decode_splitk_reduce and,
    for the mixed workload, pa_prefill_chunk.  decode_only(layer) enqueues
    the decode launch alone.  Results land in .out (decode rows, or the
    draft tokens' rows) and .outp (prefill rows).

    layer_copies: R (default: enough copies for 1 GiB, at least 2).
    fill_new: the pools already hold the step's new tokens (the timed steps
    rewrite them with the same bytes); False leaves those slots to the
    step's own append, as a test does to check it.
    poison: unowned pool bytes hold NaN patterns (tests) instead of
    whatever the allocation held.
    """

    def __init__(self, w, ps, spec, dev, fuse_append=True, planned=True, cascade=True,
                 layer_copies=None, fill_new=True, poison=False):
        import torch
        from paged_kv_cache_234_amd import KVPool, decode_plan_buffer
        self.w, self.ps, self.spec, self.dev = w, ps, spec, dev
        i32 = self._i32
        self.R = layer_copies or max(2, math.ceil((1 << 30) / w.pool_bytes()))
        rows = np.arange(len(w.fill_slots))
        if not fill_new:
            new = set(int(r) for r, s in zip(w.new_rows, w.new_slots) if s >= 0)
            rows = np.array([r for r in rows if r not in new], dtype=np.int64)
        ridx = torch.as_tensor(rows, device=w.fill_k.device)
        fk_all, fv_all = w.fill_k[ridx].contiguous(), w.fill_v[ridx].contiguous()
        fill_slots = i32(w.fill_slots[rows])
        self.pools = []
        for _ in range(self.R):
            p = KVPool(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype, device=dev,
                       poison=poison, k_scale=w.k_scale, v_scale=w.v_scale)
            p.append(fk_all, fv_all, fill_slots)
            self.pools.append(p)
        del fk_all, fv_all
        self.new_k, self.new_v = w.new_k.contiguous(), w.new_v.contiguous()
        self.new_slots = i32(w.new_slots)
        if spec:
            # the query tokens are the rows of the workload's chunks
            self.q = w.q_prefill.contiguous()
            self.lens, self.bt = i32(w.chunk_context_lens), i32(w.chunk_block_tables)
            self.qsl = i32(w.query_start_loc)
            self.max_q = int(np.max(np.diff(w.query_start_loc)))
            tok_lens = []
            for c in range(w.num_chunks):
                n = int(w.query_start_loc[c + 1] - w.query_start_loc[c])
                tok_lens.extend(int(w.chunk_context_lens[c]) - n + i + 1 for i in range(n))
            self.tok_lens = i32(tok_lens)
            self.pmax = max(1, -(-int(np.max(w.chunk_context_lens)) // ps))
        else:
            self.q = w.q.contiguous()
            self.lens, self.bt = i32(w.context_lens), i32(w.block_tables)
            self.pmax = w.max_partitions(ps) if ps > 0 else 1
        B, hq, d = self.q.shape
        self.part_max = torch.empty((B, hq, self.pmax), device=dev)
        self.part_sum = torch.empty((B, hq, self.pmax), device=dev)
        self.part_out = torch.empty((B, hq, self.pmax, d), device=dev)
        self.out = torch.empty_like(self.q)
        # prefix groups: the shared blocks are read once per group (cascade)
        self.cascade = bool(w.prefix_groups) and ps > 0 and cascade
        if self.cascade:
            g_start, g_seqs, g_plens = [0], [], []
            for members, nshared in w.prefix_groups:
                g_seqs.extend(int(b) for b in members)
                g_start.append(len(g_seqs))
                g_plens.append(int(nshared) * w.block_size)
            self.groups = (i32(g_start), i32(g_seqs), i32(g_plens),
                           max(len(m) for m, _ in w.prefix_groups))
        self.has_prefill = w.num_chunks > 0 and not spec
        # decode steps append each sequence's new token, and the draft step
        # its draft tokens, inside the decode launch (fused: the plain
        # step's pa_decode_append)
        self.fuse_append = not self.has_prefill and fuse_append
        self.fused = self.fuse_append and not (self.cascade or spec)
        if self.fuse_append and spec:
            # the draft tokens, in the query rows' order, are the new tokens
            if len(w.new_slots) != int(w.query_start_loc[-1]):
                raise ValueError("a draft step appends its draft tokens only")
            self.fk, self.fv, self.fslots = self.new_k, self.new_v, self.new_slots
        elif self.fuse_append:
            rows = np.zeros(B, np.int64)
            fslots = np.full(B, -1, np.int32)
            j = 0
            for b in range(B):
                if int(w.context_lens[b]) > 0:
                    rows[b], fslots[b] = w.new_rows[j], w.new_slots[j]
                    j += 1
            ridx = torch.as_tensor(rows, device=dev)
            self.fk, self.fv = w.fill_k[ridx].contiguous(), w.fill_v[ridx].contiguous()
            self.fslots = i32(fslots)
        # every decode launch reads its prologue from a plan made once per
        # model step (the plain decode of the mixed step through
        # pa_decode_append with no append arrays)
        self.planned = planned
        self.plan = None
        if planned:
            self.plan = decode_plan_buffer(B + (len(w.prefix_groups) if self.cascade else 0),
                                           self.pools[0].k, d)
        if self.has_prefill:
            self.qp = w.q_prefill.contiguous()
            self.outp = torch.empty_like(self.qp)
            self.pqsl = i32(w.query_start_loc)
            self.maxq = int(np.max(np.diff(w.query_start_loc)))
            self.cbt, self.clens = i32(w.chunk_block_tables), i32(w.chunk_context_lens)
        self.entry = ("pa_decode_append" if self.fused or (planned and not (spec or self.cascade))
                      else "pa_decode_multi" if spec else
                      "pa_decode_cascade" if self.cascade else "pa_decode")

    def _i32(self, a):
        import torch
        return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=self.dev)

    def make_plan(self):
        from paged_kv_cache_234_amd import pa_decode_plan
        w = self.w
        extra = {}
        if self.spec:
            extra = dict(queries=(self.qsl, self.max_q))
        elif self.cascade:
            extra = dict(groups=self.groups)
        pa_decode_plan(self.plan, self.bt, self.lens, w.num_heads, self.pools[0].k,
                       self.pools[0].v, partition_size=self.ps, max_partitions=self.pmax,
                       new_slots=self.fslots if self.fuse_append else None, **extra)

    def step(self, layer, base, ev=None, stream=None):
        from paged_kv_cache_234_amd import pa_decode_splitk_reduce, pa_prefill_chunk
        w, ps = self.w, self.ps
        pool = self.pools[layer % self.R]
        if ev is not None:
            ev[0].record(stream)
        if not self.fuse_append:
            pool.append(self.new_k, self.new_v, self.new_slots)
        if ev is not None:
            ev[1].record(stream)
        if self.planned and plan_due(layer, base):
            self.make_plan()
        self.decode_only(layer)
        if ev is not None:
            ev[2].record(stream)
        if self.spec:
            pa_decode_splitk_reduce(self.out, self.part_max, self.part_sum, self.part_out,
                                    self.tok_lens, ps)
        elif ps > 0:
            pa_decode_splitk_reduce(self.out, self.part_max, self.part_sum, self.part_out,
                                    self.lens, ps)
        if ev is not None:
            ev[3].record(stream)
        if self.has_prefill:
            self.prefill_only(layer)
            if ev is not None:
                ev[4].record(stream)

    def prefill_only(self, layer, base=None):
        from paged_kv_cache_234_amd import pa_prefill_chunk
        w, pool = self.w, self.pools[layer % self.R]
        pa_prefill_chunk(self.outp, self.qp, self.pqsl, self.maxq, pool.k, pool.v, self.cbt,
                         self.clens, w.scale, pool.k_scale, pool.v_scale)

    def decode_only(self, layer, base=None):
        from paged_kv_cache_234_amd import (pa_decode, pa_decode_append, pa_decode_cascade,
                                            pa_decode_multi)
        w, ps, pmax = self.w, self.ps, self.pmax
        pool = self.pools[layer % self.R]
        parts = dict(part_max=self.part_max, part_sum=self.part_sum, part_out=self.part_out)
        if self.fused:
            pa_decode_append(self.out if ps == 0 else None, self.q, self.fk, self.fv, self.fslots,
                             pool.k, pool.v, self.bt, self.lens, w.scale, pool.k_scale,
                             pool.v_scale, partition_size=ps, max_partitions=pmax, plan=self.plan,
                             **parts)
        elif self.spec:
            appended = (dict(k_new=self.fk, v_new=self.fv, new_slots=self.fslots)
                        if self.fuse_append else {})
            pa_decode_multi(self.q, self.qsl, self.max_q, pool.k, pool.v, self.bt, self.lens,
                            w.scale, ps, pmax, self.part_max, self.part_sum, self.part_out,
                            pool.k_scale, pool.v_scale, plan=self.plan, **appended)
        elif self.cascade:
            g_start, g_seqs, g_plens, g_max = self.groups
            appended = (dict(k_new=self.fk, v_new=self.fv, new_slots=self.fslots)
                        if self.fuse_append else {})
            pa_decode_cascade(self.q, pool.k, pool.v, self.bt, self.lens, w.scale, g_start,
                              g_seqs, g_plens, g_max, ps, pmax, self.part_max, self.part_sum,
                              self.part_out, pool.k_scale, pool.v_scale, plan=self.plan,
                              **appended)
        elif self.planned:
            pa_decode_append(self.out if ps == 0 else None, self.q, None, None, None, pool.k,
                             pool.v, self.bt, self.lens, w.scale, pool.k_scale, pool.v_scale,
                             partition_size=ps, max_partitions=pmax, plan=self.plan, **parts)
        elif ps > 0:
            pa_decode(None, self.q, pool.k, pool.v, self.bt, self.lens, w.scale, pool.k_scale,
                      pool.v_scale, partition_size=ps, max_partitions=pmax, **parts)
        else:
            pa_decode(self.out, self.q, pool.k, pool.v, self.bt, self.lens, w.scale,
                      pool.k_scale, pool.v_scale)


def capture(body, stream):
    """A HIP graph of the launches body() makes, captured on stream (a side
    stream, not the current one) with capture_begin / capture_end.  The
    torch.cuda.graph context manager would first hand every cached block
    back to the driver, which moves where the next workload's pools land
    (see the end of run_workload)."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.capture_begin()
        try:
            body()
        finally:
            g.capture_end()
    return g


def run_workload(name, args, dev):
    """Time one workload; returns its record (all figures but the CPU legs)
    and the workload itself."""
    import torch

    w, ps, spec = make_workload(name, args.seed, dev)
    if args.partition_size is not None:
        ps = args.partition_size
    if spec and ps <= 0:
        raise SystemExit("the draft-verification step is split-K only (--partition-size > 0)")
    ls = LayerStep(w, ps, spec, dev, fuse_append=not args.no_fuse_append,
                   planned=not args.no_plan, cascade=not args.no_cascade)
    planned, fuse_append, fused, has_prefill = ls.planned, ls.fuse_append, ls.fused, ls.has_prefill
    cascade = ls.cascade
    step, decode_only, make_plan = ls.step, ls.decode_only, ls.make_plan
    pmax, R = ls.pmax, ls.R
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    warm = max(args.warmup, 1)
    if planned:
        make_plan()
    for i in range(warm):
        step(i, 0)
        decode_only(i)
    torch.cuda.synchronize()

    # The engines on the pages replay their decode step as a captured graph
    # covering every layer; here one graph holds the K timed layer-steps (each
    # on the next layer copy), another the warm-up steps, a third the K
    # decode kernels alone (reading the plan the steps before made).
    def steps_of(fn, first, count):
        for i in range(count):
            fn(first + i, first)

    capture_stream = torch.cuda.Stream()

    def captured(fn, first, count):
        return capture(lambda: steps_of(fn, first, count), capture_stream)

    if not args.eager:
        g_warm = captured(step, 0, warm)
        g_steps = captured(step, args.warmup, args.steps)
        g_decode = captured(decode_only, args.warmup, args.steps)
        g_prefill = captured(ls.prefill_only, args.warmup, args.steps) if has_prefill else None
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        g_warm.replay()
    else:
        steps_of(step, 0, warm)
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

    # ---- the prefill kernel alone, the same way (mixed workload) -----------
    prefill_ms = None
    if has_prefill:
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        if args.eager:
            steps_of(ls.prefill_only, args.warmup, args.steps)
        else:
            g_prefill.replay()
        f1.record(stream)
        torch.cuda.synchronize()
        prefill_ms = f0.elapsed_time(f1) / args.steps

    # ---- per-kernel durations, eager, HIP events around each launch ---------
    nev = 5 if has_prefill else 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    first = args.warmup + args.steps
    for i in range(args.steps):
        step(first + i, first, evs[i], stream)
    torch.cuda.synchronize()
    names = ["append" if fuse_append else "kv_append",
             ("plan / %d layers + " % PLAN_LAYERS if planned else "") +
             ("decode_append" if fused else "decode"), "splitk_reduce", "prefill_chunk"]
    names = names[:nev - 1]
    kern_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
               for j, n in enumerate(names)}
    if fuse_append:
        del kern_ms["append"]                     # inside the decode launch
    plan_us = None
    if planned:
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for _ in range(args.steps):
            make_plan()
        p1.record(stream)
        torch.cuda.synchronize()
        plan_us = p0.elapsed_time(p1) * 1e3 / args.steps

    # ---- accounting -----------------------------------------------------------
    kv_logical = w.prefill_kv_bytes() if spec else w.decode_kv_bytes_logical()
    kv_unique = w.prefill_kv_bytes() if spec else w.decode_kv_bytes_unique()
    step_bytes = kv_logical + (w.prefill_kv_bytes() if has_prefill else 0)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_unique / (decode_ms * 1e-3) / 1e9

    entry = ls.entry
    rec = {
        "workload": w.name,
        "gate_70pct_hbm": w.name in GATE,
        "us_per_layer_step": round(ms_per_step * 1e3, 3),
        "ms_per_step": round(ms_per_step, 6),
        "kv_GBps": round(gbps, 2),
        "pct_hbm_peak": round(100.0 * (kv_unique / (ms_per_step * 1e-3) / 1e9) / HBM_PEAK_GBPS, 2),
        "kv_bytes_logical": kv_logical,
        "kv_bytes_unique": kv_unique,
        "decode_kernel_us": round(decode_ms * 1e3, 3),
        "eager_event_us": {k: round(v * 1e3, 3) for k, v in kern_ms.items()},
        "plan_us": None if plan_us is None else round(plan_us, 3),
        "dtype": w.cache_dtype if w.cache_dtype != "fp8" else "fp8-e4m3 KV, bf16 Q",
        "config": {
            "workload": w.name, "seed": w.seed, "batch": w.num_chunks if spec else w.batch,
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size,
            "context_tokens": int((w.chunk_context_lens if spec else w.context_lens).sum()),
            "new_tokens": int(len(w.new_slots)),
            "prefill_chunks": 0 if spec else w.num_chunks, "partition_size": ps,
            "max_partitions": pmax, "pool_blocks": w.num_blocks, "layer_copies": R,
            "decode_entry": entry,
            "plan": ("pa_decode_plan once per %d layer-steps, inside the timed graph"
                     % PLAN_LAYERS) if planned else None,
            "step_entries": ("pa_decode_cascade (append fused) + pa_decode_splitk_reduce"
                             if fuse_append and cascade else
                             "pa_decode_multi (append fused) + pa_decode_splitk_reduce"
                             if fuse_append and spec else
                             "pa_decode_append + pa_decode_splitk_reduce" if fused and ps > 0
                             else "pa_decode_append" if fused
                             else "pa_kv_append + %s%s%s" % (
                                 entry, " + pa_decode_splitk_reduce" if ps > 0 else "",
                                 " + pa_prefill_chunk" if has_prefill else "")),
        },
        "launch": "eager" if args.eager else "one HIP graph holding the K layer-steps",
        "roofline": {
            "bound": "hbm",
            "kernel": entry,
            "duration_us": round(decode_ms * 1e3, 3),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(w.name, ps, entry),
        },
    }
    if has_prefill:
        # K back-to-back graph-replayed launches, as for the decode kernel
        rec["prefill_kernel_us"] = round(prefill_ms * 1e3, 3)
        rec["prefill_tflops"] = round(w.prefill_flops() / (prefill_ms * 1e-3) / 1e12, 2)
        rec["prefill_mfma_frac_bf16"] = round(rec["prefill_tflops"] / 2500.0, 4)
    del ls
    if not args.eager:
        del g_warm, g_steps, g_decode, g_prefill
    torch.cuda.synchronize()
    # The freed memory stays in torch's cache for the next workload, as a
    # serving process keeps its pools: handing it back to the driver (here,
    # or on entry to each graph capture) made the pools allocated next land
    # where the decode read them slower (long-context layer-step 359-360 ->
    # 347-348 us, mixed fp8 178-179 -> 174-176 us, draft verification
    # 53.6-53.7 -> 52.6-53.2 us, three same-box runs of every workload each
    # way).
    return rec, w


def read_probe_bandwidth(dev):
    """HBM read bandwidth of the decode's access pattern: pa_read_probe over
    4 GiB read as 4 KB chunks in a seeded random order (best of 3 launches,
    HIP events on its stream).  Context for the roofline fractions, which
    are taken against the published 8 TB/s."""
    import torch
    from paged_kv_cache_234_amd import pa_read_probe
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    ids = torch.as_tensor(np.random.default_rng(0).permutation(nbytes // 4096).astype(np.int32),
                          device=dev)
    props = torch.cuda.get_device_properties(dev)
    sink = torch.empty(props.multi_processor_count * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    pa_read_probe(buf, ids, sink)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa_read_probe(buf, ids, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del buf, ids, sink
    torch.cuda.empty_cache()
    return nbytes / (best * 1e-3) / 1e9


def copy_bandwidth(dev):
    """Achievable copy bandwidth in this process (context for the peak)."""
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    return 2 * nbytes * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the paged-attention path here is built and timed on "
              "a single MI355X (no sharding, no collectives); --gpus %d is not supported"
              % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_234_amd import pa_selftest

    dev = "cuda:0"
    torch.cuda.set_device(0)
    names = workload_names() if args.workload == "all" else [args.workload]
    headline = HEADLINE if HEADLINE in names else names[0]
    recs = {}
    for name in names:
        pa_selftest()             # (also marks where each workload starts in a kernel trace)
        print("bench: %s" % name, file=sys.stderr, flush=True)
        rec, w = run_workload(name, args, dev)
        if not args.no_cpu_baseline:
            rec["cpu_baseline"], rec["cpu_baseline_1thread"] = cpu_baselines(
                w, args.cpu_seconds, args.cpu_seconds_1t, rec["ms_per_step"],
                rec["kv_bytes_logical"])
        del w
        recs[name] = rec
    copy_gbps = copy_bandwidth(dev)
    probe_gbps = read_probe_bandwidth(dev)

    h = recs[headline]
    result = {
        "metric": METRIC,
        "value": h["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic (seeded; no dataset, no weights)",
        "config": h["config"],
        "us_per_layer_step": h["us_per_layer_step"],
        "pct_hbm_peak": h["pct_hbm_peak"],
        "kv_bytes_logical": h["kv_bytes_logical"],
        "kv_bytes_unique": h["kv_bytes_unique"],
        "launch": h["launch"],
        "decode_kernel_us": h["decode_kernel_us"],
        "eager_event_us": h["eager_event_us"],
        "plan_us": h["plan_us"],
        "copy_GBps": round(copy_gbps, 1),
        "read_probe_GBps": round(probe_gbps, 1),
        "roofline": h["roofline"],
    }
    for k in ("prefill_kernel_us", "prefill_tflops", "prefill_mfma_frac_bf16"):
        if k in h:
            result[k] = h[k]
    if "cpu_baseline" in h:
        result["cpu_baseline"] = h["cpu_baseline"]
        result["cpu_baseline_1thread"] = h["cpu_baseline_1thread"]
    if len(recs) > 1:
        result["headline"] = ("the long-context batch: the largest workload one GPU holds; "
                              "'configs' has every workload")
        result["configs"] = recs
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


def cpu_baseline(w, budget_s, gpu_ms, gpu_bytes, one_thread=False):
    """The fp64 oracle, as it stands, on a bounded sample of the workload's
    decode sequences (or, for a workload of chunks only, its chunks); scaled
    to the metric's unit (KV GB/s).  one_thread: BLAS limited to one thread
    (the rest of the oracle is single-threaded NumPy either way)."""
    if one_thread:
        return cpu_baselines(w, 0.0, budget_s, gpu_ms, gpu_bytes, all_cores=False)[1]
    return cpu_baselines(w, budget_s, None, gpu_ms, gpu_bytes)[0]


def cpu_baselines(w, budget_s, budget_1t, gpu_ms, gpu_bytes, all_cores=True):
    """(all-core record, one-thread record or None).  The all-core leg fills
    the oracle's pool sequence by sequence as it goes (untimed) and times
    each sequence; the one-thread leg times the sequences the pool already
    holds (at least one) with BLAS limited to one thread."""
    from oracle import paged_attention as opa
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])

    def raw(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    chunks_only = w.batch == 0
    n_units = w.num_chunks if chunks_only else w.batch
    lens_of = w.chunk_context_lens if chunks_only else w.context_lens
    tables_of = w.chunk_block_tables if chunks_only else w.block_tables
    order = np.random.default_rng(0).permutation(n_units)
    st = opa.STORAGE_DTYPES[w.cache_dtype]
    shape_k, shape_v = opa.pool_shapes(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype,
                                       w.block_size)
    pool = [np.zeros(shape_k, st), np.zeros(shape_v, st)]
    qh = raw(w.q_prefill if chunks_only else w.q)
    filled = []

    def fill(b):
        n = -(-int(lens_of[b]) // w.block_size)
        blocks = tables_of[b, :n].astype(np.int64)
        sel = np.flatnonzero(np.isin(w.fill_slots // w.block_size, blocks))
        idx = torch.as_tensor(sel, device=w.fill_k.device)
        pool[0], pool[1] = opa.oracle_append(pool[0], pool[1], raw(w.fill_k[idx]),
                                             raw(w.fill_v[idx]), w.fill_slots[sel], w.in_dtype,
                                             w.cache_dtype, w.k_scale, w.v_scale, w.block_size)
        filled.append(int(b))

    def timed(b):
        t = time.perf_counter()
        if chunks_only:
            opa.oracle_prefill(qh, w.q_dtype, w.query_start_loc, pool[0], pool[1],
                               w.cache_dtype, w.chunk_block_tables, w.chunk_context_lens,
                               w.scale, w.k_scale, w.v_scale, w.block_size, chunks=[int(b)])
        else:
            opa.oracle_decode(qh, w.q_dtype, pool[0], pool[1], w.cache_dtype, w.block_tables,
                              w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size,
                              seqs=[int(b)])
        return time.perf_counter() - t

    def leg(budget, grow, nthreads):
        """Passes over the workload until the budget is spent (at least one
        sequence); grow: the first pass adds sequences to the pool."""
        used, tokens, elapsed, passes = set(), 0, 0.0, 0
        while elapsed < budget or not used:
            seq = order if (grow and passes == 0) else [b for b in order if int(b) in filled]
            for b in seq:
                if int(b) not in filled:
                    fill(b)
                elapsed += timed(b)
                used.add(int(b))
                tokens += int(lens_of[b])
                if elapsed >= budget:
                    break
            passes += 1
        kv = tokens * w.kv_bytes_per_token()
        return _baseline_record(w, kv, elapsed, nthreads, used, n_units, passes, tokens,
                                chunks_only, gpu_ms, gpu_bytes)

    rec_all = leg(budget_s, True, threads) if all_cores else None
    rec_1t = None
    if budget_1t is not None:
        if not filled:
            fill(order[0])
        with threadpool_limits(limits=1):
            rec_1t = leg(budget_1t, False, 1)
    return rec_all, rec_1t


def _baseline_record(w, kv, elapsed, threads, done, n_units, passes, tokens, chunks_only,
                     gpu_ms, gpu_bytes):
    return {
        "value": round(kv / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "fp64 oracle %s of %d of %d %s, %d pass(es) (%d context tokens, %.1f s), "
                  "host affinity %d cores, BLAS threads %d" % (
                      "causal chunks" if chunks_only else "decode", len(done), n_units,
                      "sequences' query tokens" if chunks_only else "sequences", passes, tokens,
                      elapsed, len(os.sched_getaffinity(0)), threads),
        "seconds": round(elapsed, 3),
        "gpu_over_cpu": round((gpu_bytes / (gpu_ms * 1e-3)) / (kv / elapsed), 1)
        if elapsed > 0 else None,
    }


if __name__ == "__main__":
    main()
