"""pa_decode / pa_decode_splitk_reduce parity with the fp64 oracle on the GPU.

Small cases span several tiles and ragged tails (every block/tile boundary
neighbourhood), all GQA group sizes, both head sizes and all three cache
types, on pools whose unowned bytes are NaN.  GPU-side invariants (batch
invariance, shared == private blocks) are checked bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention as opa
from paged_kv_cache_234_amd import pa_decode_splitk_reduce
from tests.gpu_helpers import (TOL, as_f64, gpu_pool, host, i32, max_abs_err, oracle_pool,
                               run_decode)
from workloads import build_workload, make_config

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 250, 513, 1000]


def _case(q_dtype, cache, hq, hkv, d, lens, seed, dist="normal"):
    return build_workload("t", seed=seed, device="cuda", q_dtype=q_dtype, cache_dtype=cache,
                          num_heads=hq, num_kv_heads=hkv, head_dim=d, decode_lens=lens, dist=dist)


def _check(w, partition_size, seqs=None, tol=None):
    pool = gpu_pool(w)
    out, parts = run_decode(w, pool, partition_size)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w, seqs=seqs)
    ref = opa.oracle_decode(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                            w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size, seqs=seqs)
    got = as_f64(out)
    if seqs is not None:
        got, ref = got[seqs], ref[seqs]
    err = max_abs_err(got, ref)
    tol = TOL[w.cache_dtype] if tol is None else tol
    assert err <= tol, "max abs err %g > %g" % (err, tol)
    return pool, out, parts, (kp, vp)


@pytest.mark.parametrize("ps", [0, 16, 32, 64, 512])
def test_tiny_fp32_config(ps):
    w = make_config(1, device="cuda")
    _check(w, ps)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (8, 2), (16, 4), (16, 1), (12, 4)])
@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_edge_lengths_all_groups(cache, hq, hkv, d):
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = _case(q_dtype, cache, hq, hkv, d, EDGE_LENS, seed=hq * 131 + hkv * 7 + d)
    _check(w, 0)


@pytest.mark.parametrize("ps", [16, 48, 64, 128, 512, 1024])
@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_split_k_partials_and_reduce(cache, ps):
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = _case(q_dtype, cache, 8, 2, 128, EDGE_LENS, seed=7 + ps)
    pool, out, (pm, ps_, po), (kp, vp) = _check(w, ps)
    pmax = pm.shape[2]
    m, l, o = opa.oracle_partitions(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                                    w.context_lens, w.scale, ps, pmax, w.k_scale, w.v_scale)
    valid = ~np.isnan(m)
    gm, gl, go = as_f64(pm), as_f64(ps_), as_f64(po)
    # partitions past ceil(L/PS) are left untouched (still NaN)
    assert np.all(np.isnan(gm[~valid]))
    tol = TOL[w.cache_dtype]
    assert np.max(np.abs(gm[valid] - m[valid])) <= tol
    assert np.max(np.abs(gl[valid] / l[valid] - 1)) <= 4 * tol
    assert np.max(np.abs(go[valid] - o[valid])) <= tol


@pytest.mark.parametrize("PS", [64, 32, 16, 8])
def test_reduce_kernel_on_oracle_partials(PS):
    """Up to 64 partitions one wavefront per (sequence, head) reduces; up to
    128 and 256 four wavefronts do (32 / 64 rows each); beyond that the
    general kernel."""
    rng = np.random.default_rng(5 + PS)
    B, hq, d = 6, 8, 128
    lens = np.array([0, 1, 64, 65, 700, 4096], np.int32)
    pmax = -(-int(lens.max()) // PS)
    m = rng.normal(0, 3, (B, hq, pmax))
    l = rng.uniform(0.5, 60, (B, hq, pmax))
    o = rng.normal(0, 1, (B, hq, pmax, d))
    ref = opa.oracle_combine(m, l, o, lens, PS)
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    t = lambda a: torch.as_tensor(a.astype(np.float32), device="cuda").contiguous()
    pa_decode_splitk_reduce(out, t(m), t(l), t(o), i32(lens), PS)
    torch.cuda.synchronize()
    got = as_f64(out)
    ref32 = opa.oracle_combine(m.astype(np.float32), l.astype(np.float32), o.astype(np.float32), lens, PS)
    assert np.max(np.abs(got - ref32)) <= 1e-5
    assert np.max(np.abs(got - ref)) <= 1e-5
    assert np.all(got[0] == 0)


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("ps", [0, 32])
def test_zero_length_sequences_give_zeros(cache, ps):
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = _case(q_dtype, cache, 4, 2, 64, [0, 5, 0, 40], seed=3)
    pool = gpu_pool(w)
    bt = w.block_tables.copy()
    bt[w.context_lens == 0] = -1
    out, _ = run_decode(w, pool, ps, block_tables=bt)
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.all(got[[0, 2]] == 0)
    kp, vp = oracle_pool(w)
    ref = opa.oracle_decode(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, bt, w.context_lens,
                            w.scale, w.k_scale, w.v_scale)
    assert max_abs_err(got, ref) <= TOL[cache]


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("ps", [0, 64])
def test_batched_equals_sequential_and_runs_repeat_bit_exact(cache, ps):
    """infer-lab: batched decode == sequential decode, bit for bit.  Where the
    batch cuts a sequence's work between wavefronts changes, but each item is
    one online softmax over its tiles in order whichever wavefronts hold
    them, so the result does not."""
    w = _case("bf16", cache, 16, 2, 128, [33, 700, 1, 250, 4000], seed=11)
    pool = gpu_pool(w)
    full, _ = run_decode(w, pool, ps)
    again, _ = run_decode(w, pool, ps)
    assert torch.equal(full, again)
    for b in range(w.batch):
        one, _ = run_decode(w, pool, ps, q=w.q[b:b + 1], block_tables=w.block_tables[b:b + 1],
                            context_lens=w.context_lens[b:b + 1])
        assert torch.equal(one[0], full[b]), "sequence %d differs alone" % b


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_full_size_batch_invariance_bit_exact(cache):
    """The Qwen2.5-3B-shaped batch (64 sequences, partition 256): every
    sequence of the batch equals the same sequence in a batch of its own and
    in the batch reversed, bit for bit (different cut points each time)."""
    w = make_config(2, device="cuda")
    if cache == "fp8":
        w = _case("bf16", "fp8", 16, 2, 128, list(w.context_lens[:24]), seed=91)
    pool = gpu_pool(w)
    ps = 256
    full, _ = run_decode(w, pool, ps)
    rev = np.arange(w.batch)[::-1].copy()
    back, _ = run_decode(w, pool, ps, q=w.q[torch.as_tensor(rev, device="cuda")],
                         block_tables=w.block_tables[rev], context_lens=w.context_lens[rev])
    assert torch.equal(back.flip(0), full)
    for b in [0, 5, int(np.argmax(w.context_lens)), w.batch - 1]:
        one, _ = run_decode(w, pool, ps, q=w.q[b:b + 1], block_tables=w.block_tables[b:b + 1],
                            context_lens=w.context_lens[b:b + 1])
        assert torch.equal(one[0], full[b]), "sequence %d differs alone" % b


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_shared_prefix_blocks_equal_private_copies_bit_exact(cache):
    """infer-lab: prefix-cached == uncached.  Sequences 1..3 share sequence
    0's first 4 blocks; a second pool holds private copies of them."""
    lens = [100, 90, 64, 130]
    groups = [([0, 1, 2, 3], 4)]
    ws = build_workload("s", seed=21, device="cuda", cache_dtype=cache, num_heads=8,
                        num_kv_heads=2, head_dim=128, decode_lens=lens, prefix_groups=groups)
    wp = build_workload("p", seed=21, device="cuda", cache_dtype=cache, num_heads=8,
                        num_kv_heads=2, head_dim=128, decode_lens=lens)
    # give every private slot the value the shared workload holds at the same
    # (sequence, position), so both pools describe identical logical K/V
    ws_row = {int(s): r for r, s in enumerate(ws.fill_slots)}
    rows_p = np.empty(len(wp.fill_slots), np.int64)
    wp_row = {int(s): r for r, s in enumerate(wp.fill_slots)}
    for b, L in enumerate(lens):
        for p in range(L):
            s_shared = int(ws.block_tables[b, p // 16]) * 16 + p % 16
            s_private = int(wp.block_tables[b, p // 16]) * 16 + p % 16
            rows_p[wp_row[s_private]] = ws_row[s_shared]
    idx = torch.as_tensor(rows_p, device="cuda")
    wp.fill_k = ws.fill_k[idx].contiguous()
    wp.fill_v = ws.fill_v[idx].contiguous()
    wp.q = ws.q
    wp.k_scale, wp.v_scale = ws.k_scale, ws.v_scale
    out_s, _ = run_decode(ws, gpu_pool(ws))
    out_p, _ = run_decode(wp, gpu_pool(wp))
    assert torch.equal(out_s, out_p)


# ---- the full-size workloads, in the launch configuration the bench times --------

BENCH_PS = {2: 256, 3: 256, 4: 512, 5: 1024}


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_config_sampled_rows(cfg):
    w = make_config(cfg, device="cuda")
    rng = np.random.default_rng(cfg)
    B = w.batch
    seqs = sorted(set([0, B - 1, int(np.argmax(w.context_lens)), int(np.argmin(w.context_lens))] +
                      list(rng.choice(B, size=min(B, 4 if cfg == 4 else 6), replace=False))))
    _check(w, BENCH_PS[cfg], seqs=seqs)


def test_full_size_mixed_fp8_at_256_token_partitions():
    """The mixed fp8 batch's decode rows at the partition size it ran with
    before (4-tile items), on sampled sequences."""
    w = make_config(5, device="cuda")
    rng = np.random.default_rng(55)
    B = w.batch
    seqs = sorted(set([0, B - 1] + list(rng.choice(B, size=4, replace=False))))
    _check(w, 256, seqs=seqs)


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("ps", [0, 64])
def test_large_scores_stay_finite_and_exact(cache, ps):
    """Q scaled by 64: scores spread over hundreds of units, so a wrong running
    max (e.g. a broken cross-lane reduction) overflows exp2 and shows up."""
    q_dtype = "f32" if cache == "f32" else "bf16"
    w = _case(q_dtype, cache, 8, 2, 128, EDGE_LENS, seed=77)
    w.q = (w.q.float() * 64).to(w.q.dtype)
    # fp32 score rounding is relative to the score: scaling Q by 64 scales the
    # absolute score error, hence the output error, by 64 as well
    _check(w, ps, tol=TOL[cache] * (64 if cache == "f32" else 1))


@pytest.mark.parametrize("seed", range(8))
def test_decode_seeded_random_configurations(seed):
    """Seeded random shapes against the oracle: cache type, head size, GQA
    shape (G = 1 .. 16, 3 included), 1-16 sequences of 0-3000 positions,
    single pass or a partition size that is a multiple of 16 up to 1024."""
    rng = np.random.default_rng(4000 + seed)
    cache = ["f32", "bf16", "fp8"][int(rng.integers(3))]
    hq, hkv = [(4, 4), (8, 2), (16, 2), (16, 1), (12, 4), (32, 8), (6, 2)][int(rng.integers(7))]
    d = [64, 128][int(rng.integers(2))]
    lens = [int(x) for x in rng.integers(0, 3001, size=int(rng.integers(1, 17)))]
    ps = 0 if int(rng.integers(5)) == 0 else 16 * int(rng.integers(1, 65))
    print("decode:", seed, cache, hq, hkv, d, ps, lens, flush=True)
    _check(_case("f32" if cache == "f32" else "bf16", cache, hq, hkv, d, lens, seed=seed), ps)


@pytest.mark.parametrize("cache,hq,hkv,batch,pmax_big", [("bf16", 32, 8, 8, 128),
                                                      ("bf16", 16, 1, 64, 128),
                                                      ("fp8", 32, 8, 16, 256)])
def test_split_k_rows_collected_in_lds_equal_direct_stores(cache, hq, hkv, batch, pmax_big):
    """Long ranges: a launch whose bound on tiles per wavefront is large
    collects each wavefront's split-K rows in LDS and writes them at the end
    of its range.  The bound follows max_partitions, so the same batch runs
    both ways (the partitions it needs: direct stores; pmax_big: collected);
    the partials and outputs agree bit for bit.  G = 4 and 16 rows per item,
    bf16 and fp8 caches."""
    from paged_kv_cache_234_amd import pa_decode
    rng = np.random.default_rng(77 + batch)
    lens = [int(x) for x in rng.integers(28000, 40001, size=batch)]
    w = _case("bf16", cache, hq, hkv, 128, lens, seed=77 + batch)
    pool = gpu_pool(w)
    q = w.q.contiguous()
    bt, cl = i32(w.block_tables), i32(w.context_lens)
    B, hq, d = q.shape
    need = -(-max(lens) // 512)
    assert need < 80
    got = {}
    for pmax in (need, pmax_big):
        pm = torch.full((B, hq, pmax), float("nan"), device="cuda")
        psum = torch.full_like(pm, float("nan"))
        po = torch.full((B, hq, pmax, d), float("nan"), device="cuda")
        pa_decode(None, q, pool.k, pool.v, bt, cl, w.scale, pool.k_scale, pool.v_scale,
                  partition_size=512, max_partitions=pmax, part_max=pm, part_sum=psum, part_out=po)
        out = torch.empty_like(q)
        pa_decode_splitk_reduce(out, pm, psum, po, cl, 512)
        torch.cuda.synchronize()
        got[pmax] = (out, pm[:, :, :need], psum[:, :, :need], po[:, :, :need])
    a, b = got[need], got[pmax_big]
    assert torch.equal(a[0], b[0])
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(x.nan_to_num(7.0), y.nan_to_num(7.0))
