"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant replaces one oracle function with a plausible wrong version (a
wrong index, a dropped term, a transposed operand, a wrong rounding rule);
the test then runs the pins and requires at least one of them to fail.
"""

import numpy as np
import pytest

from oracle import fp8_e4m3 as fp8
from oracle import paged_attention as pa

import tests.test_oracle_attention as A
import tests.test_oracle_fp8 as F

ATTENTION_PINS = [
    lambda: A.test_single_token_context_returns_that_v_row_exactly("f32"),
    lambda: A.test_single_token_context_returns_that_v_row_exactly("fp8"),
    A.test_zero_query_gives_mean_of_visible_values,
    A.test_huge_scores_select_the_unique_best_key_without_overflow,
    A.test_tiled_online_softmax_equals_the_oracle,
    lambda: A.test_decode_matches_torch_sdpa_on_unpaged_arrays(4, 2),
    lambda: A.test_decode_matches_torch_sdpa_on_unpaged_arrays(8, 2),
    A.test_prefill_matches_torch_sdpa_with_causal_offset,
    A.test_chunked_prefill_equals_one_shot_and_decode_equals_last_row,
    lambda: A.test_partition_combine_equals_unsplit(48),
    A.test_partition_stats_are_consistent_with_a_direct_sum,
    lambda: A.test_append_writes_the_layout_and_nothing_else("f32"),
    A.test_append_fp8_encodes_with_per_head_scale,
    A.test_append_then_gather_roundtrips_values,
    lambda: A.test_fp8_decode_matches_sdpa_on_dequantised_arrays(6, 3),
    A.test_fp8_prefill_matches_sdpa_on_dequantised_arrays,
    A.test_fp8_append_then_gather_returns_the_dequantised_codes,
]

FP8_PINS = [
    F.test_encode_roundtrips_every_finite_code,
    F.test_midpoints_round_to_even_and_neighbours_to_nearest,
    F.test_saturation_nan_and_signed_zero,
    lambda: F.test_encode_matches_torch_on_every_bf16_pattern_in_range(0.125),
]


def _some_pin_fails(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


# ---- attention mutants -----------------------------------------------------

def _attend_factory(head_map=None, vis_shift=0, use_scale=True, subtract_max=True):
    def attend(q_rows, positions, K, V, scale):
        R, hq_n, d = q_rows.shape
        hkv = K.shape[1]
        G = hq_n // hkv
        out = np.zeros((R, hq_n, d))
        sc = np.float64(np.float32(scale)) if use_scale else 1.0
        for r in range(R):
            n_vis = int(positions[r]) + 1 + vis_shift
            n_vis = max(1, min(n_vis, K.shape[0]))
            for hq in range(hq_n):
                h = head_map(hq, G, hkv) if head_map else hq // G
                with np.errstate(all="ignore"):
                    s = sc * (K[:n_vis, h] @ q_rows[r, hq])
                    p = np.exp(s - s.max()) if subtract_max else np.exp(s)
                    out[r, hq] = (p @ V[:n_vis, h]) / p.sum()
        return out
    return attend


def _gather_v_like_k(k_pool, v_pool, row, L, dt, ks=None, vs=None, block_size=16):
    K, _ = ORIG_GATHER(k_pool, v_pool, row, L, dt, ks, vs, block_size)
    n = -(-L // block_size)
    ids = np.asarray(row[:n], dtype=np.int64)
    vb = pa.storage_to_f64(v_pool[ids], dt)                 # read as if it had K's layout
    if dt == "fp8":
        vb = vb * np.asarray(vs, np.float64)[None, :, None, None]
    hkv, x = k_pool.shape[1], k_pool.shape[4]
    d = k_pool.shape[2] * x
    V = vb.reshape(n, hkv, d // x, block_size, x).transpose(0, 3, 1, 2, 4) \
        .reshape(n * block_size, hkv, d)[:L]
    return K, V


def _gather_without_v_scale(k_pool, v_pool, row, L, dt, ks=None, vs=None, block_size=16):
    return ORIG_GATHER(k_pool, v_pool, row, L, dt, ks,
                       None if vs is None else np.ones_like(vs), block_size)


def _gather_without_k_scale(k_pool, v_pool, row, L, dt, ks=None, vs=None, block_size=16):
    return ORIG_GATHER(k_pool, v_pool, row, L, dt,
                       None if ks is None else np.ones_like(ks), vs, block_size)


def _gather_k_with_v_scale(k_pool, v_pool, row, L, dt, ks=None, vs=None, block_size=16):
    return ORIG_GATHER(k_pool, v_pool, row, L, dt, vs, vs, block_size)


def _gather_v_with_k_scale(k_pool, v_pool, row, L, dt, ks=None, vs=None, block_size=16):
    return ORIG_GATHER(k_pool, v_pool, row, L, dt, ks, ks, block_size)


def _gather_off_by_one_block(k_pool, v_pool, row, L, dt, ks=None, vs=None, block_size=16):
    row = np.asarray(row).copy()
    n = -(-L // block_size)
    if n >= 2:
        row[[0, 1]] = row[[1, 0]]
    return ORIG_GATHER(k_pool, v_pool, row, L, dt, ks, vs, block_size)


def _combine_without_partition_sums(m, l, o, lens, ps):
    return ORIG_COMBINE(m, np.ones_like(l), o, lens, ps)


def _append_v_untransposed(k_pool, v_pool, k_new, v_new, slots, in_dt, c_dt, ks=None, vs=None,
                           block_size=16):
    k2, _ = ORIG_APPEND(k_pool, v_pool, k_new, v_new, slots, in_dt, c_dt, ks, vs, block_size)
    v2 = np.array(v_pool, copy=True)
    s = np.asarray(slots, dtype=np.int64)
    keep = s >= 0
    enc = pa.encode_for_cache(np.asarray(v_new)[keep], in_dt, c_dt, vs)
    flat = v2.reshape(v2.shape[0], v2.shape[1], -1)
    for i, sl in enumerate(s[keep]):
        blk, off = sl // block_size, sl % block_size
        flat[blk, :, off * enc.shape[2]:(off + 1) * enc.shape[2]] = enc[i]
    return k2, v2


ORIG_GATHER = pa.gather_sequence
ORIG_COMBINE = pa.oracle_combine
ORIG_APPEND = pa.oracle_append

ATTENTION_MUTANTS = {
    "gqa head map hq % Hkv": ("attend_rows", _attend_factory(head_map=lambda hq, G, hkv: hq % hkv)),
    "causal sees one key too few": ("attend_rows", _attend_factory(vis_shift=-1)),
    "causal sees one key too many": ("attend_rows", _attend_factory(vis_shift=+1)),
    "scale dropped": ("attend_rows", _attend_factory(use_scale=False)),
    "max not subtracted": ("attend_rows", _attend_factory(subtract_max=False)),
    "V read with K's layout": ("gather_sequence", _gather_v_like_k),
    "V scale not applied": ("gather_sequence", _gather_without_v_scale),
    "K scale not applied": ("gather_sequence", _gather_without_k_scale),
    "K dequantised with V's scale": ("gather_sequence", _gather_k_with_v_scale),
    "V dequantised with K's scale": ("gather_sequence", _gather_v_with_k_scale),
    "block table entries swapped": ("gather_sequence", _gather_off_by_one_block),
    "combine ignores partition sums": ("oracle_combine", _combine_without_partition_sums),
    "append writes V untransposed": ("oracle_append", _append_v_untransposed),
}


@pytest.mark.parametrize("name", sorted(ATTENTION_MUTANTS))
def test_attention_mutant_is_caught(name, monkeypatch):
    attr, fn = ATTENTION_MUTANTS[name]
    monkeypatch.setattr(pa, attr, fn)
    assert _some_pin_fails(ATTENTION_PINS), "no pin caught: " + name


# ---- fp8 mutants -----------------------------------------------------------

def _encode_ties_away(x, scale=1.0):
    codes = ORIG_ENCODE(x, scale)
    xf = np.asarray(x, np.float32) / np.asarray(scale, np.float32)
    pos = fp8.DECODE_TABLE[:0x7F]
    mag = np.abs(xf.astype(np.float64))
    out = codes.copy()
    for idx in np.ndindex(np.shape(codes)):
        m = mag[idx] if np.ndim(mag) else mag
        hi = np.searchsorted(pos, m)
        if 0 < hi < 0x7F and m == (pos[hi - 1] + pos[hi]) / 2:
            c = hi | (0x80 if np.signbit(xf[idx] if np.ndim(xf) else xf) else 0)
            if np.ndim(out):
                out[idx] = c
            else:
                out = np.uint8(c)
    return out


def _encode_no_saturation(x, scale=1.0):
    codes = ORIG_ENCODE(x, scale)
    y = np.asarray(x, np.float32) / np.asarray(scale, np.float32)
    return np.where(np.abs(y) > 464, np.uint8(0x7F), codes).astype(np.uint8)


def _encode_truncating(x, scale=1.0):
    y = np.asarray(x, np.float32) / np.asarray(scale, np.float32)
    pos = fp8.DECODE_TABLE[:0x7F]
    mag = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    code = np.searchsorted(pos, mag, side="right") - 1
    code = np.where(np.signbit(y), code | 0x80, code)
    return np.where(np.isnan(y), 0x7F, code).astype(np.uint8)


def _encode_sign_dropped_for_zero(x, scale=1.0):
    codes = ORIG_ENCODE(x, scale)
    return np.where(codes == 0x80, np.uint8(0), codes).astype(np.uint8)


ORIG_ENCODE = fp8.encode

FP8_MUTANTS = {
    "ties away from zero": _encode_ties_away,
    "overflow gives NaN": _encode_no_saturation,
    "truncation instead of rounding": _encode_truncating,
    "negative zero lost": _encode_sign_dropped_for_zero,
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(fp8, "encode", FP8_MUTANTS[name])
    assert _some_pin_fails(FP8_PINS), "no pin caught: " + name


def test_unmutated_oracle_passes_every_pin_used_above():
    assert not _some_pin_fails(ATTENTION_PINS)
    assert not _some_pin_fails(FP8_PINS)
