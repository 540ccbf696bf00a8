"""pa_kv_append and the library self test on the GPU: bit-exact against the
oracle's append, including every bf16 bit pattern through the fp8 encoder."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as opa
from paged_kv_cache_234_amd import KVPool, pa_kv_append, pa_selftest
from tests.gpu_helpers import host, i32

pytestmark = pytest.mark.gpu


def test_selftest_runs_gfx950_code():
    pa_selftest()


def _random_pool_bytes(pool, rng):
    for t in (pool.k, pool.v):
        raw = torch.from_numpy(rng.integers(0, 256, t.numel() * t.element_size(), dtype=np.uint8))
        t.view(torch.uint8).view(-1).copy_(raw.to(t.device))


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_is_bit_exact(cache, d):
    rng = np.random.default_rng(100 + d)
    nb, hkv, T = 13, 3, 40
    scales = np.array([0.011, 0.0047, 0.02], np.float32) if cache == "fp8" else None
    pool = KVPool(nb, hkv, d, cache, k_scale=scales, v_scale=scales[::-1].copy() if scales is not None else None)
    _random_pool_bytes(pool, rng)
    k_before, v_before = host(pool.k).copy(), host(pool.v).copy()
    in_dt = torch.float32 if cache == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(d)
    kn = torch.randn(T, hkv, d, generator=g).to(in_dt)
    vn = torch.randn(T, hkv, d, generator=g).to(in_dt)
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int32)
    slots[[3, 17, 31]] = -1
    pa_kv_append(kn.cuda(), vn.cuda(), pool.k, pool.v, i32(slots), pool.k_scale, pool.v_scale)
    torch.cuda.synchronize()
    in_name = "f32" if cache == "f32" else "bf16"
    k_ref, v_ref = opa.oracle_append(k_before, v_before, host(kn), host(vn), slots, in_name, cache,
                                     scales, None if scales is None else scales[::-1].copy())
    assert host(pool.k).tobytes() == k_ref.tobytes()
    assert host(pool.v).tobytes() == v_ref.tobytes()


@pytest.mark.parametrize("scale", [1.0, 0.0125558, 0.125])
def test_fp8_encoder_matches_oracle_on_every_bf16_pattern(scale):
    d, hkv = 128, 1
    T = 65536 // d
    bits = np.arange(65536, dtype=np.uint16).reshape(T, hkv, d)
    kn = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    vn = torch.from_numpy(bits[::-1].copy().view(np.int16)).view(torch.bfloat16).cuda()
    s = np.array([scale], np.float32)
    pool = KVPool(T // 16, hkv, d, "fp8", k_scale=s, v_scale=s)
    slots = np.arange(T, dtype=np.int32)
    pool.append(kn, vn, i32(slots))
    torch.cuda.synchronize()
    k_ref, v_ref = opa.oracle_append(host(pool.k) * 0, host(pool.v) * 0, bits, bits[::-1].copy(),
                                     slots, "bf16", "fp8", s, s)
    got_k, got_v = host(pool.k), host(pool.v)
    bad = np.flatnonzero(got_k.reshape(-1) != k_ref.reshape(-1))
    assert bad.size == 0, "first mismatches at flat %s: got %s want %s" % (
        bad[:5], got_k.reshape(-1)[bad[:5]], k_ref.reshape(-1)[bad[:5]])
    assert got_v.tobytes() == v_ref.tobytes()


def test_append_of_zero_tokens_is_a_no_op():
    pool = KVPool(2, 1, 64, "bf16")
    before = host(pool.k).copy()
    e = torch.empty((0, 1, 64), dtype=torch.bfloat16, device="cuda")
    pa_kv_append(e, e, pool.k, pool.v, i32(np.zeros(0)))
    torch.cuda.synchronize()
    assert host(pool.k).tobytes() == before.tobytes()


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_of_a_contiguous_run_is_bit_exact(cache, d):
    """A prefill chunk's tokens: 101 consecutive slots starting at offset 10
    of a block (groups of 16 tokens straddle two blocks), then 7 scattered
    ones; bit-exact against the oracle."""
    rng = np.random.default_rng(7 + d)
    nb, hkv = 12, 2
    scales = np.array([0.013, 0.006], np.float32) if cache == "fp8" else None
    pool = KVPool(nb, hkv, d, cache, k_scale=scales, v_scale=scales[::-1].copy() if scales is not None else None)
    _random_pool_bytes(pool, rng)
    k_before, v_before = host(pool.k).copy(), host(pool.v).copy()
    run = np.arange(16 * 2 + 10, 16 * 2 + 10 + 101)
    rest = rng.choice(np.setdiff1d(np.arange(nb * 16), run), size=7, replace=False)
    slots = np.concatenate([run, rest]).astype(np.int32)
    T = len(slots)
    in_dt = torch.float32 if cache == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(3 * d)
    kn = torch.randn(T, hkv, d, generator=g).to(in_dt)
    vn = torch.randn(T, hkv, d, generator=g).to(in_dt)
    pa_kv_append(kn.cuda(), vn.cuda(), pool.k, pool.v, i32(slots), pool.k_scale, pool.v_scale)
    torch.cuda.synchronize()
    in_name = "f32" if cache == "f32" else "bf16"
    k_ref, v_ref = opa.oracle_append(k_before, v_before, host(kn), host(vn), slots, in_name, cache,
                                     scales, None if scales is None else scales[::-1].copy())
    assert host(pool.k).tobytes() == k_ref.tobytes()
    assert host(pool.v).tobytes() == v_ref.tobytes()
