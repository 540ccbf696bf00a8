"""Host-side logic of bench.py, on the CPU: the oracle baseline's sampling
and the lookup of measured HBM traffic under profiles/."""

import os
import re

import numpy as np
import pytest

import bench
from workloads import make_config


def test_cpu_baseline_repeats_passes_until_the_budget():
    """A workload shorter than the budget is timed over repeated passes, and
    every pass counts all of its context tokens."""
    w = make_config(1, device="cpu")
    r = bench.cpu_baseline(w, 0.5, 0.01, 441344)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] >= 1
    assert r["seconds"] >= 0.5
    passes = int(r["sample"].split(" pass(es)")[0].rsplit(" ", 1)[1])
    assert passes >= 2
    ctx = int(np.sum(w.context_lens))
    tokens = int(re.search(r"\((\d+) context tokens", r["sample"]).group(1))
    # whole passes plus a prefix of the last one
    assert (passes - 1) * ctx < tokens <= passes * ctx
    assert r["value"] == pytest.approx(tokens * w.kv_bytes_per_token() / r["seconds"] / 1e9,
                                       rel=1e-2)


def test_cpu_baseline_stops_inside_a_pass_when_the_budget_is_spent():
    w = make_config(1, device="cpu")
    r = bench.cpu_baseline(w, 0.0, 0.01, 441344)
    assert " 1 pass(es)" in r["sample"]
    assert r["sample"].startswith("fp64 oracle decode of 1 of 4 sequences")


BENCH_ENTRY = {
    "tiny-fp32-decode": "pa_decode_append",
    "qwen2.5-3b-bf16-decode-b64": "pa_decode_append",
    "llama3-8b-bf16-decode-prefix-shared-b256": "pa_decode_cascade",
    "long-context-bf16-splitk-b8": "pa_decode_append",
    "mixed-chunked-prefill-fp8kv": "pa_decode_append",
    "qwen2.5-3b-bf16-spec-verify-b64": "pa_decode_multi",
}


def _bench_partition_size(workload):
    from workloads import CONFIG_NAMES, SPEC_VERIFY_NAME
    if workload == SPEC_VERIFY_NAME:
        return bench.SPEC_VERIFY_PS
    return bench.DEFAULT_PS[{v: k for k, v in CONFIG_NAMES.items()}[workload]]


@pytest.mark.parametrize("workload", sorted(BENCH_ENTRY))
def test_every_bench_workload_has_measured_traffic_for_the_current_sources(workload):
    """profiles/ holds a copy-calibrated FETCH_SIZE + WRITE_SIZE summary for
    each workload at the partition size the bench uses, taken from the
    decode sources as they stand (a kernel change, or a new bench partition
    size, makes this fail until the counters are taken again)."""
    assert sorted(BENCH_ENTRY) == sorted(bench.workload_names())
    t = bench.measured_traffic(workload, _bench_partition_size(workload), BENCH_ENTRY[workload])
    assert t is not None and t > 0


def test_traffic_lookup_refuses_other_partitions_and_entries():
    assert bench.measured_traffic("qwen2.5-3b-bf16-decode-b64", 128, "pa_decode_append") is None
    assert bench.measured_traffic("qwen2.5-3b-bf16-decode-b64", 256, "pa_decode") is None


def test_bench_defaults_match_the_summaries():
    assert bench.DEFAULT_PS[5] == 1024 and bench.SPEC_VERIFY_PS == 512 and bench.DEFAULT_PS[1] == 16
    assert bench.DEFAULT_PS[2] == 512 and bench.DEFAULT_PS[3] == 256 and bench.DEFAULT_PS[4] == 512
    assert os.path.isdir(os.path.join(bench.ROOT, "profiles"))


def test_one_thread_leg_reuses_the_pool_and_limits_blas():
    w = make_config(1, device="cpu")
    rec_all, rec_1t = bench.cpu_baselines(w, 0.2, 0.1, 0.01, 441344)
    assert rec_all["cores"] >= 1 and rec_1t["cores"] == 1
    assert "BLAS threads 1" in rec_1t["sample"]
    assert rec_1t["seconds"] >= 0.1 and rec_1t["value"] > 0


@pytest.mark.parametrize("k", [1, 5, 20, 31, 32, 33, 50, 64, 100])
@pytest.mark.parametrize("base", [0, 5, 10, 37])
def test_every_timed_region_holds_its_share_of_plans(k, base):
    """A captured region of K layer-steps starting anywhere makes
    ceil(K / PLAN_LAYERS) plans, the first at its first step."""
    due = [bench.plan_due(base + i, base) for i in range(k)]
    assert due[0] and sum(due) == -(-k // bench.PLAN_LAYERS)


def test_default_run_times_every_workload_with_the_long_context_headline():
    args = bench.parse([])
    assert args.workload == "all" and args.gpus == 1
    names = bench.workload_names()
    assert len(names) == 6 and bench.HEADLINE in names
    assert set(bench.GATE) <= set(names)
    assert args.cpu_seconds * len(names) <= 30          # a bounded CPU sample
    assert bench.parse(["--config", "4"]).workload == bench.HEADLINE


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_pool_k_and_v_share_one_allocation(cache):
    """A pool's K and V are views of one allocation, V directly after K, in
    the layouts the kernels take; the poison fills both, and filling K
    leaves V untouched."""
    import torch
    from paged_kv_cache_234_amd import KVPool
    nb, hkv, d = 5, 2, 64
    p = KVPool(nb, hkv, d, cache, device="cpu")
    x = 16 // p.k.element_size()
    assert tuple(p.k.shape) == (nb, hkv, d // x, 16, x)
    assert tuple(p.v.shape) == (nb, hkv, d, 16)
    assert p.k.is_contiguous() and p.v.is_contiguous()
    assert p.k.untyped_storage().data_ptr() == p.v.untyped_storage().data_ptr()
    kbytes = p.k.numel() * p.k.element_size()
    assert p.v.data_ptr() == p.k.data_ptr() + kbytes
    assert p.k.untyped_storage().nbytes() == 2 * kbytes == p.nbytes()

    def poisoned(t):
        if cache == "f32":
            return bool(torch.isnan(t).all())
        if cache == "bf16":
            return bool((t.view(torch.int16) == 0x7FC0).all())
        return bool((t == 0x7F).all())

    assert poisoned(p.k) and poisoned(p.v)
    p.k.zero_()
    assert poisoned(p.v) and not poisoned(p.k)
