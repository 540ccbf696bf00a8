"""Structure of the seeded synthetic workloads (CPU only)."""

import os

import numpy as np
import pytest

from workloads import build_workload, make_config
from workloads.configs import ELEM_BYTES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "inferx_pool_size.txt")


def _check_tables(w):
    bs = w.block_size
    used = {}
    for b, L in enumerate(w.context_lens):
        n = -(-int(L) // bs)
        row = w.block_tables[b]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < w.num_blocks)
        assert np.all(row[n:] == -1)
        for i in range(n):
            used.setdefault(int(row[i]), set()).add(b)
    return used


def test_tiny_config_matches_its_definition():
    w = make_config(1)
    assert list(w.context_lens) == [17, 64, 100, 250]
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks) == (4, 2, 64, 16, 64)
    assert w.q_dtype == w.cache_dtype == "f32"
    assert w.scale == 0.125
    used = _check_tables(w)
    assert len(used) == 29 and all(len(s) == 1 for s in used.values())
    assert len(w.fill_slots) == 431 == len(set(w.fill_slots.tolist()))
    # the appended token of each sequence is its last position
    for b, L in enumerate(w.context_lens):
        p = int(L) - 1
        assert w.new_slots[b] == w.block_tables[b, p // 16] * 16 + p % 16
    assert float(w.fill_k.abs().max()) <= 1.0 and float(w.q.abs().max()) <= 1.0


def test_qwen_shaped_config():
    w = make_config(2)
    assert w.batch == 64 and (w.num_heads, w.num_kv_heads, w.head_dim) == (16, 2, 128)
    assert w.context_lens.min() >= 256 and w.context_lens.max() <= 4096
    need = sum(-(-int(L) // 16) for L in w.context_lens)
    assert w.num_blocks == int(np.ceil(1.25 * need))
    used = _check_tables(w)
    assert len(used) == need
    assert str(w.q.dtype) == "torch.bfloat16"
    assert np.float32(w.scale) == np.float32(1) / np.float32(np.sqrt(128))


def test_prefix_shared_config_shares_exactly_the_prompt_blocks():
    w = make_config(3)
    assert w.batch == 256
    assert np.all((w.context_lens >= 256) & (w.context_lens <= 384))
    used = _check_tables(w)
    for g in range(32):
        rows = w.block_tables[8 * g:8 * g + 8]
        assert np.all(rows[:, :16] == rows[0, :16])
    shared = [blk for blk, users in used.items() if len(users) > 1]
    assert len(shared) == 32 * 16
    assert all(len(used[blk]) == 8 for blk in shared)
    # a sequence whose new token falls in a shared block appends nothing
    for b, L in enumerate(w.context_lens):
        assert (w.new_slots[b] < 0) == (int(L) == 256)
    assert w.decode_kv_bytes_unique() < w.decode_kv_bytes_logical()


def test_mixed_prefill_config():
    w = make_config(5)
    assert w.batch == 60 and w.num_chunks == 4 and w.cache_dtype == "fp8"
    assert list(w.query_start_loc) == [0, 512, 1024, 1536, 2048]
    assert np.all(w.chunk_context_lens >= 512) and np.all(w.chunk_context_lens <= 2560)
    assert len(w.new_slots) == 60 + 2048
    assert w.k_scale.dtype == np.float32 and w.k_scale.shape == (8,)
    ka = w.fill_k.float().abs().amax(dim=(0, 2)).numpy().astype(np.float32)
    assert np.array_equal(w.k_scale, ka / np.float32(448))
    assert len(set(w.fill_slots.tolist())) == len(w.fill_slots)


def test_long_context_lengths_are_clipped_lognormal():
    rng = np.random.Generator(np.random.PCG64(4))
    z = rng.normal(size=8)
    lens = np.clip(np.round(np.exp(np.log(65536) + (np.log(2) / 2) * z)), 32768, 131072)
    assert np.all((lens >= 32768) & (lens <= 131072))


def test_seeded_generation_is_reproducible():
    a = make_config(1, seed=7)
    b = make_config(1, seed=7)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert bool((a.fill_k == b.fill_k).all()) and bool((a.q == b.q).all())
    c = make_config(1, seed=8)
    assert not np.array_equal(a.block_tables, c.block_tables)


def test_pool_size_arithmetic_reproduces_inferx_figures():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = float(v)
    for dt, key in (("bf16", "bf16_GB"), ("fp8", "fp8_GB")):
        w = build_workload("pool", seed=0, cache_dtype=dt, q_dtype="bf16",
                           num_heads=16, num_kv_heads=int(vals["kv_heads"]),
                           head_dim=int(vals["head_dim"]), decode_lens=[16],
                           num_blocks=int(vals["blocks"]))
        per_layer = w.pool_bytes()
        assert per_layer == vals["blocks"] * vals["block_size"] * 2 * vals["kv_heads"] * vals["head_dim"] * ELEM_BYTES[dt]
        total_gb = per_layer * vals["layers"] / 1e9
        assert round(total_gb, 2) == vals[key]


def test_prefix_groups_must_cover_shared_blocks():
    with pytest.raises(ValueError):
        build_workload("bad", seed=0, decode_lens=[10, 40], prefix_groups=[([0, 1], 2)])
