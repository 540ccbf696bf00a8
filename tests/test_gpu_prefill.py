"""pa_prefill_chunk parity with the fp64 oracle on the GPU, plus the pages'
"chunked prefill == one-shot prefill" invariant checked bit for bit."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as opa
from tests.gpu_helpers import (TOL, as_f64, gpu_pool, host, i32, max_abs_err, oracle_pool,
                               run_decode, run_prefill)
from paged_kv_cache_234_amd import pa_prefill_chunk
from workloads import build_workload, make_config

pytestmark = pytest.mark.gpu

CHUNKS = [(0, 1), (0, 16), (1, 5), (15, 33), (16, 64), (17, 100), (100, 31), (250, 129)]


def _case(cache, hq, hkv, d, chunks, seed, decode_lens=()):
    q_dtype = "f32" if cache == "f32" else "bf16"
    return build_workload("pf", seed=seed, device="cuda", q_dtype=q_dtype, cache_dtype=cache,
                          num_heads=hq, num_kv_heads=hkv, head_dim=d, decode_lens=decode_lens,
                          prefill_chunks=chunks)


def _oracle(w, kp, vp, chunks=None):
    return opa.oracle_prefill(host(w.q_prefill), w.q_dtype, w.query_start_loc, kp, vp,
                              w.cache_dtype, w.chunk_block_tables, w.chunk_context_lens, w.scale,
                              w.k_scale, w.v_scale, w.block_size, chunks=chunks)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (32, 8), (12, 4), (16, 1)])
@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_prefill_chunks_match_oracle(cache, hq, hkv, d):
    w = _case(cache, hq, hkv, d, CHUNKS, seed=hq * 17 + hkv + d)
    out = run_prefill(w, gpu_pool(w))
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w)
    err = max_abs_err(as_f64(out), _oracle(w, kp, vp))
    assert err <= TOL[cache], err


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_chunked_equals_one_shot_bit_exact(cache):
    """One 96-row chunk after 40 cached tokens vs the same rows as two chunks
    (the second one's context includes the first one's rows)."""
    w = _case(cache, 8, 2, 128, [(40, 96)], seed=5)
    pool = gpu_pool(w)
    one = run_prefill(w, pool)
    qp = w.q_prefill.cuda().contiguous()
    two = torch.empty_like(qp)
    bt = np.concatenate([w.chunk_block_tables, w.chunk_block_tables])
    pa_prefill_chunk(two, qp, i32([0, 37, 96]), 59, pool.k, pool.v, i32(bt), i32([40 + 37, 136]),
                     w.scale, pool.k_scale, pool.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(one, two)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_last_prefill_row_matches_decode(cache):
    w = _case(cache, 8, 2, 128, [(300, 20)], seed=9)
    pool = gpu_pool(w)
    out = run_prefill(w, pool)
    dec, _ = run_decode(w, pool, 0, q=w.q_prefill[-1:], block_tables=w.chunk_block_tables,
                        context_lens=w.chunk_context_lens)
    torch.cuda.synchronize()
    assert np.max(np.abs(as_f64(out[-1]) - as_f64(dec[0]))) <= TOL[cache]


def test_mixed_chunked_prefill_config_sampled_rows():
    w = make_config(5, device="cuda")
    pool = gpu_pool(w)
    out = run_prefill(w, pool)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w, seqs=[], chunks=list(range(w.num_chunks)))
    got = as_f64(out)
    qf = opa.storage_to_f64(host(w.q_prefill), w.q_dtype)
    for c in range(w.num_chunks):
        a, e = int(w.query_start_loc[c]), int(w.query_start_loc[c + 1])
        L = int(w.chunk_context_lens[c])
        P = L - (e - a)
        rows = np.array([0, 1, 2, 3, 4, 255, 256, e - a - 5, e - a - 2, e - a - 1])
        K, V = opa.gather_sequence(kp, vp, w.chunk_block_tables[c], L, w.cache_dtype,
                                   w.k_scale, w.v_scale, w.block_size)
        ref = opa.attend_rows(qf[a + rows], P + rows, K, V, w.scale)
        assert max_abs_err(got[a + rows], ref) <= TOL["fp8"]
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("scale", [-0.3, 0.0])
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_prefill_negative_and_zero_scale(cache, scale):
    """softmax(scale * QK^T) for a negative scale (the kernel moves its sign
    into Q) and for zero (uniform weights over the visible keys)."""
    w = _case(cache, 8, 2, 128, [(40, 96), (0, 33)], seed=13)
    pool = gpu_pool(w)
    qp = w.q_prefill.cuda().contiguous()
    out = torch.empty_like(qp)
    qsl = w.query_start_loc
    pa_prefill_chunk(out, qp, i32(qsl), int(np.max(np.diff(qsl))), pool.k, pool.v,
                     i32(w.chunk_block_tables), i32(w.chunk_context_lens), scale, pool.k_scale,
                     pool.v_scale)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w)
    want = opa.oracle_prefill(host(w.q_prefill), w.q_dtype, w.query_start_loc, kp, vp,
                              w.cache_dtype, w.chunk_block_tables, w.chunk_context_lens, scale,
                              w.k_scale, w.v_scale, w.block_size)
    assert max_abs_err(as_f64(out), want) <= TOL[cache]


@pytest.mark.parametrize("nchunks", [24, 40])
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_prefill_launch_order_many_chunks(cache, nchunks):
    """Many chunks of mixed lengths (32 rows per workgroup): 24 x 7 (chunk,
    row group) classes are ranked by tile count across three registers of
    classes; 40 x 13 classes go past the ranking's limit and take the natural
    order.  Every row must be written once and match the oracle."""
    rng = np.random.default_rng(nchunks)
    rows = 200 if nchunks == 24 else 416
    chunks = [(int(rng.integers(0, 400)), int(rng.integers(1, rows + 1))) for _ in range(nchunks)]
    chunks[0] = (int(chunks[0][0]), rows)
    w = _case(cache, 8, 2, 128, chunks, seed=nchunks + 1)
    out = run_prefill(w, gpu_pool(w))
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w)
    err = max_abs_err(as_f64(out), _oracle(w, kp, vp))
    assert err <= TOL[cache], err


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 2)])
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_prefill_long_prefix(cache, hq, hkv):
    """Chunks after 4,100-9,000 cached tokens: a workgroup stages more than 64
    tiles, so its per-lane register of block ids is refilled, and the launch
    ranking searches tile counts past 128.  With 8 KV heads the ranking runs
    per XCD."""
    chunks = [(9000, 40), (4100, 17), (0, 24), (6000, 1)]
    w = _case(cache, hq, hkv, 128, chunks, seed=77 + hkv)
    out = run_prefill(w, gpu_pool(w))
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w)
    err = max_abs_err(as_f64(out), _oracle(w, kp, vp))
    assert err <= TOL[cache], err


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_prefill_context_beyond_the_table_is_clamped(cache):
    """A context length past max_blocks_per_seq * 16 is taken as that bound,
    as in pa_decode, so nothing past the chunk's block-table row is read: a
    chunk whose real context fills its row gives the same bits when its
    context length is stated larger."""
    w = _case(cache, 8, 2, 128, [(100, 28)], seed=9)
    assert w.chunk_block_tables.shape[1] * 16 == int(w.chunk_context_lens[0]) == 128
    pool = gpu_pool(w)
    ref = run_prefill(w, pool)
    qp = w.q_prefill.cuda().contiguous()
    out = torch.full_like(qp, float("nan"))
    pa_prefill_chunk(out, qp, i32(w.query_start_loc), 28, pool.k, pool.v,
                     i32(w.chunk_block_tables), i32([200]), w.scale, pool.k_scale, pool.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("seed", range(8))
def test_prefill_seeded_random_configurations(seed):
    """Seeded random shapes against the oracle: cache type, head size, GQA
    shape, 1-6 chunks of 1-300 rows over prefixes of 0-1500."""
    rng = np.random.default_rng(6000 + seed)
    cache = ["f32", "bf16", "fp8"][int(rng.integers(3))]
    hq, hkv = [(4, 4), (8, 2), (16, 2), (16, 1), (12, 4), (32, 8), (6, 2)][int(rng.integers(7))]
    d = [64, 128][int(rng.integers(2))]
    chunks = [(int(rng.integers(0, 1501)), int(rng.integers(1, 301)))
              for _ in range(int(rng.integers(1, 7)))]
    print("prefill:", seed, cache, hq, hkv, d, chunks, flush=True)
    w = _case(cache, hq, hkv, d, chunks, seed=seed)
    out = run_prefill(w, gpu_pool(w))
    torch.cuda.synchronize()
    kp, vp = oracle_pool(w)
    err = max_abs_err(as_f64(out), _oracle(w, kp, vp))
    assert err <= TOL[cache], err
