"""pa_decode_noalloc (split-K decode + reduce with the partials in the
library's static per-GPU scratch) against the entry points it stands for,
pa_decode with caller-owned partial buffers followed by
pa_decode_splitk_reduce: the same bits, and the oracle's tolerance.  Two calls
in a row, the second smaller, so the second reads nothing the first left."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as opa
from paged_kv_cache_234_amd import PAError, pa_decode_noalloc, pa_decode_noalloc_max_bytes
from paged_kv_cache_234_amd import _lib
from tests.gpu_helpers import TOL, as_f64, gpu_pool, host, i32, max_abs_err, oracle_pool, run_decode
from workloads import build_workload, make_config

pytestmark = pytest.mark.gpu


def _noalloc(w, pool, ps, rows=None):
    rows = np.arange(w.batch) if rows is None else np.asarray(rows)
    q = w.q[torch.as_tensor(rows, device="cuda")].contiguous()
    lens = w.context_lens[rows]
    pmax = max(1, -(-int(np.max(lens)) // ps))
    out = torch.full_like(q, float("nan"))
    pa_decode_noalloc(out, q, pool.k, pool.v, i32(w.block_tables[rows]), i32(lens), w.scale,
                      ps, pmax, pool.k_scale, pool.v_scale)
    return out


def _check(w, pool, ps, rows):
    got = _noalloc(w, pool, ps, rows)
    want, _ = run_decode(w, pool, ps, q=w.q[torch.as_tensor(rows, device="cuda")],
                         block_tables=w.block_tables[rows], context_lens=w.context_lens[rows])
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    return got


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_noalloc_equals_decode_then_reduce_twice(cache):
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = build_workload("na", seed=71, device="cuda", q_dtype=q_dtype, cache_dtype=cache,
                       num_heads=16, num_kv_heads=2, head_dim=128,
                       decode_lens=[1, 33, 700, 4000, 65, 2500, 16, 129])
    pool = gpu_pool(w)
    kp, vp = oracle_pool(w)
    ref = opa.oracle_decode(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                            w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size)
    full = _check(w, pool, 64, np.arange(w.batch))
    assert max_abs_err(as_f64(full), ref) <= TOL[cache]
    small = [6, 1, 4]                          # fewer rows, fewer partitions
    part = _check(w, pool, 64, small)
    assert max_abs_err(as_f64(part), ref[small]) <= TOL[cache]


def test_noalloc_long_context_full_size():
    """The long-context batch (8 x 32 heads x up to 256 partitions of 512:
    32.5 MiB of partials), then the Qwen2.5-3B-shaped batch, in a row."""
    w = make_config(4, device="cuda")
    pool = gpu_pool(w)
    _check(w, pool, 512, np.arange(w.batch))
    del pool
    w2 = make_config(2, device="cuda")
    pool2 = gpu_pool(w2)
    got = _check(w2, pool2, 256, np.arange(w2.batch))
    seqs = [0, 31, 63]
    kp, vp = oracle_pool(w2, seqs=seqs)
    ref = opa.oracle_decode(host(w2.q), w2.q_dtype, kp, vp, w2.cache_dtype, w2.block_tables,
                            w2.context_lens, w2.scale, w2.k_scale, w2.v_scale, w2.block_size,
                            seqs=seqs)
    assert max_abs_err(as_f64(got)[seqs], ref[seqs]) <= TOL["bf16"]


def test_noalloc_refuses_partials_beyond_its_scratch():
    w = build_workload("nb", seed=72, device="cuda", num_heads=32, num_kv_heads=8,
                       head_dim=128, decode_lens=[40] * 8)
    pool = gpu_pool(w)
    q = w.q.contiguous()
    out = torch.full_like(q, 7.0)
    pmax = 1 + pa_decode_noalloc_max_bytes() // (8 * 32 * 130 * 4)
    with pytest.raises(PAError) as e:
        pa_decode_noalloc(out, q, pool.k, pool.v, i32(w.block_tables), i32(w.context_lens),
                          w.scale, 64, pmax)
    assert e.value.status == _lib.PA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)               # nothing was launched
