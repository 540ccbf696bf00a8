"""Pins for the fp64 paged-attention oracle (CPU only).

Each test checks the oracle against something other than itself: a closed
form, an invariant the pages assert (infer-lab's equivalence list: batched ==
sequential, chunked == one-shot, prefix-cached == uncached, tiled == naive),
or torch's CPU float64 scaled_dot_product_attention on contiguous K/V.
The pool used by these tests is written with the storage layout formula
directly (not through oracle_append), so the gather is pinned independently.
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention as pa
from oracle import fp8_e4m3 as fp8

BS = 16


# ---------------------------------------------------------------------------
# helpers: build pools from contiguous K/V using the layout definition
# ---------------------------------------------------------------------------

def layout_pool(Kc_list, Vc_list, tables, num_blocks, dtype="f32"):
    """Write contiguous per-sequence K/V (storage dtype) into pools.

    K element (seq, pos, h, d) -> k_pool.flat[(((blk*Hkv + h)*(D/X) + d//X)*BS + off)*X + d%X]
    V element (seq, pos, h, d) -> v_pool.flat[((blk*Hkv + h)*D + d)*BS + off]
    with blk = table[pos // BS], off = pos % BS and X = 16 bytes of elements.
    Unowned elements are NaN (f32), 0x7FC0 (bf16) or 0x7F (fp8).
    """
    hkv, d = Kc_list[0].shape[1], Kc_list[0].shape[2]
    st = pa.STORAGE_DTYPES[dtype]
    X = 16 // np.dtype(st).itemsize
    poison = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[dtype]
    kf = np.full(num_blocks * hkv * BS * d, poison, dtype=st)
    vf = np.full(num_blocks * hkv * BS * d, poison, dtype=st)
    for Kc, Vc, tab in zip(Kc_list, Vc_list, tables):
        for pos in range(Kc.shape[0]):
            blk, off = int(tab[pos // BS]), pos % BS
            for h in range(hkv):
                for dd in range(d):
                    kf[(((blk * hkv + h) * (d // X) + dd // X) * BS + off) * X + dd % X] = Kc[pos, h, dd]
                    vf[((blk * hkv + h) * d + dd) * BS + off] = Vc[pos, h, dd]
    return kf.reshape(num_blocks, hkv, d // X, BS, X), vf.reshape(num_blocks, hkv, d, BS)


def random_case(rng, lens, hq, hkv, d, num_blocks=None, dist="normal"):
    need = sum(-(-L // BS) for L in lens)
    nb = num_blocks or need + 7
    perm = rng.permutation(nb)
    tables, k, v = [], [], []
    j = 0
    W = max(-(-L // BS) for L in lens)
    for L in lens:
        n = -(-L // BS)
        t = np.full(W, -1, dtype=np.int32)
        t[:n] = perm[j:j + n]
        j += n
        tables.append(t)
        draw = (lambda s: rng.uniform(-1, 1, s)) if dist == "uniform" else (lambda s: rng.standard_normal(s))
        k.append(draw((L, hkv, d)).astype(np.float32))
        v.append(draw((L, hkv, d)).astype(np.float32))
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    return q, k, v, np.stack(tables), nb


def sdpa_reference(q_rows, positions, Kc, Vc, scale):
    """torch CPU float64 SDPA with KV heads repeated G times and an explicit mask."""
    R, hq, d = q_rows.shape
    hkv = Kc.shape[1]
    G = hq // hkv
    L = Kc.shape[0]
    qt = torch.from_numpy(q_rows.astype(np.float64)).permute(1, 0, 2)            # [Hq, R, D]
    kt = torch.from_numpy(Kc.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(Vc.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    mask = torch.zeros(R, L, dtype=torch.bool)
    for r, p in enumerate(positions):
        mask[r, :p + 1] = True
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=float(np.float64(np.float32(scale))))
    return out.permute(1, 0, 2).numpy()


SCALE64 = float(np.float32(1.0) / np.float32(8.0))     # 1/sqrt(64)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_single_token_context_returns_that_v_row_exactly(dtype):
    rng = np.random.default_rng(0)
    q, k, v, tables, nb = random_case(rng, [1, 1, 1], 4, 2, 64)
    if dtype == "f32":
        kc, vc = k, v
        ks = vs = None
    elif dtype == "bf16":
        kc = [torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16) for x in k]
        vc = [torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16) for x in v]
        ks = vs = None
    else:
        ks = np.array([0.01, 0.02], dtype=np.float32)
        vs = np.array([0.03, 0.005], dtype=np.float32)
        kc = [fp8.encode(x, ks[None, :, None]) for x in k]
        vc = [fp8.encode(x, vs[None, :, None]) for x in v]
    kp, vp = layout_pool(kc, vc, tables, nb, dtype)
    out = pa.oracle_decode(q, "f32", kp, vp, dtype, tables, [1, 1, 1], SCALE64, ks, vs)
    for b in range(3):
        for hq in range(4):
            h = hq // 2
            raw = vc[b][0, h]
            want = pa.storage_to_f64(raw, dtype) * (1.0 if dtype != "fp8" else float(vs[h]))
            assert np.array_equal(out[b, hq], want)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(1)
    lens = [17, 64, 100]
    q, k, v, tables, nb = random_case(rng, lens, 4, 2, 64)
    kp, vp = layout_pool(k, v, tables, nb)
    out = pa.oracle_decode(np.zeros_like(q), "f32", kp, vp, "f32", tables, lens, SCALE64)
    for b, L in enumerate(lens):
        for hq in range(4):
            mean = v[b][:L, hq // 2].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[b, hq], mean, rtol=0, atol=1e-15)


def test_constant_values_give_that_value():
    rng = np.random.default_rng(2)
    lens = [33, 5]
    q, k, v, tables, nb = random_case(rng, lens, 2, 1, 64)
    u = rng.standard_normal(64).astype(np.float32)
    v = [np.broadcast_to(u, x.shape).copy() for x in v]
    kp, vp = layout_pool(k, v, tables, nb)
    out = pa.oracle_decode(q * 3, "f32", kp, vp, "f32", tables, lens, SCALE64)
    np.testing.assert_allclose(out, np.broadcast_to(u.astype(np.float64), out.shape), rtol=0, atol=1e-14)


def test_huge_scores_select_the_unique_best_key_without_overflow():
    rng = np.random.default_rng(3)
    L = 40
    q, k, v, tables, nb = random_case(rng, [L], 1, 1, 64)
    best = 23
    k[0][best, 0] = 2 * q[0, 0]          # q.k = 2|q|^2 ~ 128, far above any random key
    out = pa.oracle_decode(q * np.float32(1e4), "f32", *layout_pool(k, v, tables, nb), "f32",
                           tables, [L], SCALE64)
    assert np.all(np.isfinite(out))
    np.testing.assert_array_equal(out[0, 0], v[0][best, 0].astype(np.float64))


def test_tiled_online_softmax_equals_the_oracle():
    """infer-lab: tiled attention == naive attention (here to 1e-13)."""
    rng = np.random.default_rng(4)
    lens = [250, 100]
    q, k, v, tables, nb = random_case(rng, lens, 4, 2, 64)
    kp, vp = layout_pool(k, v, tables, nb)
    out = pa.oracle_decode(q, "f32", kp, vp, "f32", tables, lens, SCALE64)
    for b, L in enumerate(lens):
        for hq in range(4):
            kk = k[b][:L, hq // 2].astype(np.float64)
            vv = v[b][:L, hq // 2].astype(np.float64)
            m, l, acc = -np.inf, 0.0, np.zeros(64)
            for a in range(0, L, 16):                     # 16-row tiles, running max/sum
                s = SCALE64 * (kk[a:a + 16] @ q[b, hq].astype(np.float64))
                m_new = max(m, s.max())
                alpha = np.exp(m - m_new)
                p = np.exp(s - m_new)
                l = alpha * l + p.sum()
                acc = alpha * acc + p @ vv[a:a + 16]
                m = m_new
            np.testing.assert_allclose(out[b, hq], acc / l, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# against a library routine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 2), (4, 4), (8, 1)])
def test_decode_matches_torch_sdpa_on_unpaged_arrays(hq, hkv):
    rng = np.random.default_rng(5 + hq + hkv)
    lens = [17, 64, 100, 250, 1]
    q, k, v, tables, nb = random_case(rng, lens, hq, hkv, 64)
    kp, vp = layout_pool(k, v, tables, nb)
    out = pa.oracle_decode(q, "f32", kp, vp, "f32", tables, lens, SCALE64)
    for b, L in enumerate(lens):
        ref = sdpa_reference(q[b:b + 1], [L - 1], k[b], v[b], SCALE64)
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)


def test_prefill_matches_torch_sdpa_with_causal_offset():
    rng = np.random.default_rng(6)
    P, C = 37, 29
    L = P + C
    _, k, v, tables, nb = random_case(rng, [L], 8, 2, 64)
    qp = rng.standard_normal((C, 8, 64)).astype(np.float32)
    kp, vp = layout_pool(k, v, tables, nb)
    out = pa.oracle_prefill(qp, "f32", [0, C], kp, vp, "f32", tables, [L], SCALE64)
    ref = sdpa_reference(qp, list(range(P, P + C)), k[0], v[0], SCALE64)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_prefill_from_empty_prefix_is_full_causal_attention():
    rng = np.random.default_rng(7)
    L = 45
    _, k, v, tables, nb = random_case(rng, [L], 2, 2, 64)
    qp = rng.standard_normal((L, 2, 64)).astype(np.float32)
    kp, vp = layout_pool(k, v, tables, nb)
    out = pa.oracle_prefill(qp, "f32", [0, L], kp, vp, "f32", tables, [L], SCALE64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qp.astype(np.float64)).permute(1, 0, 2),
        torch.from_numpy(k[0].astype(np.float64)).permute(1, 0, 2),
        torch.from_numpy(v[0].astype(np.float64)).permute(1, 0, 2),
        is_causal=True, scale=SCALE64).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# equivalences (infer-lab's invariant list; exact in fp64)
# ---------------------------------------------------------------------------

def test_permuting_physical_blocks_with_the_table_changes_nothing():
    rng = np.random.default_rng(8)
    lens = [17, 64, 100, 250]
    q, k, v, tables, nb = random_case(rng, lens, 4, 2, 64, num_blocks=64)
    out1 = pa.oracle_decode(q, "f32", *layout_pool(k, v, tables, nb), "f32", tables, lens, SCALE64)
    sigma = rng.permutation(nb)
    t2 = np.where(tables >= 0, sigma[np.maximum(tables, 0)], -1).astype(np.int32)
    out2 = pa.oracle_decode(q, "f32", *layout_pool(k, v, t2, nb), "f32", t2, lens, SCALE64)
    assert np.array_equal(out1, out2)


def test_shared_prefix_blocks_equal_private_copies():
    rng = np.random.default_rng(9)
    L0 = 48                     # 3 shared blocks
    lens = [L0 + 5, L0 + 20, L0]
    _, kbase, vbase, _, _ = random_case(rng, [L0], 4, 2, 64)
    q = rng.standard_normal((3, 4, 64)).astype(np.float32)
    k, v = [], []
    for L in lens:
        tail = L - L0
        k.append(np.concatenate([kbase[0], rng.standard_normal((tail, 2, 64)).astype(np.float32)]))
        v.append(np.concatenate([vbase[0], rng.standard_normal((tail, 2, 64)).astype(np.float32)]))
    W = 5
    private = np.full((3, W), -1, np.int32)
    shared = np.full((3, W), -1, np.int32)
    nxt = 0
    for b, L in enumerate(lens):
        n = -(-L // BS)
        private[b, :n] = np.arange(nxt, nxt + n)
        nxt += n
    nxt2 = 3
    for b, L in enumerate(lens):
        n = -(-L // BS)
        shared[b, :3] = [0, 1, 2]
        shared[b, 3:n] = np.arange(nxt2, nxt2 + n - 3)
        nxt2 += n - 3
    nb = nxt + 2
    out_p = pa.oracle_decode(q, "f32", *layout_pool(k, v, private, nb), "f32", private, lens, SCALE64)
    out_s = pa.oracle_decode(q, "f32", *layout_pool(k, v, shared, nb), "f32", shared, lens, SCALE64)
    assert np.array_equal(out_p, out_s)


def test_batched_equals_sequential():
    rng = np.random.default_rng(10)
    lens = [17, 64, 100, 250]
    q, k, v, tables, nb = random_case(rng, lens, 4, 2, 64)
    kp, vp = layout_pool(k, v, tables, nb)
    full = pa.oracle_decode(q, "f32", kp, vp, "f32", tables, lens, SCALE64)
    for b in range(4):
        one = pa.oracle_decode(q[b:b + 1], "f32", kp, vp, "f32", tables[b:b + 1], lens[b:b + 1], SCALE64)
        assert np.array_equal(one[0], full[b])


def test_gqa_equals_mha_on_repeated_kv_heads():
    rng = np.random.default_rng(11)
    lens = [40, 77]
    G = 4
    q, k, v, tables, nb = random_case(rng, lens, 8, 2, 64)
    out_gqa = pa.oracle_decode(q, "f32", *layout_pool(k, v, tables, nb), "f32", tables, lens, SCALE64)
    k_mha = [np.repeat(x, G, axis=1) for x in k]
    v_mha = [np.repeat(x, G, axis=1) for x in v]
    out_mha = pa.oracle_decode(q, "f32", *layout_pool(k_mha, v_mha, tables, nb), "f32", tables, lens, SCALE64)
    assert np.array_equal(out_gqa, out_mha)


def test_chunked_prefill_equals_one_shot_and_decode_equals_last_row():
    rng = np.random.default_rng(12)
    P, C = 40, 50
    L = P + C
    _, k, v, tables, nb = random_case(rng, [L], 4, 2, 64)
    qp = rng.standard_normal((C, 4, 64)).astype(np.float32)
    kp, vp = layout_pool(k, v, tables, nb)
    one = pa.oracle_prefill(qp, "f32", [0, C], kp, vp, "f32", tables, [L], SCALE64)
    # two chunks of 20 and 30 over the same pool: chunk 1 has context P+20
    two_t = np.concatenate([tables, tables])
    two = pa.oracle_prefill(qp, "f32", [0, 20, 50], kp, vp, "f32", two_t, [P + 20, L], SCALE64)
    assert np.array_equal(one, two)
    dec = pa.oracle_decode(qp[-1:], "f32", kp, vp, "f32", tables, [L], SCALE64)
    assert np.array_equal(dec[0], one[-1])


# ---------------------------------------------------------------------------
# split-K partitions
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ps", [16, 48, 512])
def test_partition_combine_equals_unsplit(ps):
    rng = np.random.default_rng(13)
    lens = [17, 64, 100, 250, 600, 0]
    q, k, v, tables, nb = random_case(rng, [max(L, 1) for L in lens], 4, 2, 64)
    kp, vp = layout_pool(k, v, tables, nb)
    pmax = -(-max(lens) // ps)
    m, l, o = pa.oracle_partitions(q, "f32", kp, vp, "f32", tables, lens, SCALE64, ps, pmax)
    comb = pa.oracle_combine(m, l, o, lens, ps)
    ref = pa.oracle_decode(q, "f32", kp, vp, "f32", tables, lens, SCALE64)
    np.testing.assert_allclose(comb, ref, rtol=0, atol=1e-12)
    assert np.array_equal(comb[5], np.zeros_like(comb[5]))


def test_single_partition_combine_is_identity():
    rng = np.random.default_rng(14)
    m = rng.standard_normal((2, 3, 1))
    l = rng.uniform(0.5, 5, (2, 3, 1))
    o = rng.standard_normal((2, 3, 1, 8))
    out = pa.oracle_combine(m, l, o, [10, 16], 16)
    np.testing.assert_allclose(out, o[:, :, 0], rtol=1e-15, atol=0)


def test_partition_stats_are_consistent_with_a_direct_sum():
    rng = np.random.default_rng(15)
    L = 70
    q, k, v, tables, nb = random_case(rng, [L], 2, 1, 64)
    kp, vp = layout_pool(k, v, tables, nb)
    m, l, o = pa.oracle_partitions(q, "f32", kp, vp, "f32", tables, [L], SCALE64, 32, 3)
    kk = k[0][:, 0].astype(np.float64)
    for p in range(3):
        s = SCALE64 * (kk[32 * p:32 * p + 32] @ q[0, 0].astype(np.float64))
        assert m[0, 0, p] == s.max()
        np.testing.assert_allclose(l[0, 0, p], np.exp(s - s.max()).sum(), rtol=1e-15)


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_writes_the_layout_and_nothing_else(dtype):
    rng = np.random.default_rng(16)
    nb, hkv, d = 6, 2, 64
    st = pa.STORAGE_DTYPES[dtype]
    X = 16 // np.dtype(st).itemsize
    if dtype == "f32":
        kp = rng.standard_normal((nb, hkv, d // X, BS, X)).astype(np.float32)
        vp = rng.standard_normal((nb, hkv, d, BS)).astype(np.float32)
        kn = rng.standard_normal((5, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((5, hkv, d)).astype(np.float32)
    else:
        kp = rng.integers(0, 65536, (nb, hkv, d // X, BS, X)).astype(np.uint16)
        vp = rng.integers(0, 65536, (nb, hkv, d, BS)).astype(np.uint16)
        kn = rng.integers(0, 65536, (5, hkv, d)).astype(np.uint16)
        vn = rng.integers(0, 65536, (5, hkv, d)).astype(np.uint16)
    slots = np.array([3, -1, 16 * 5 + 15, 16, 40], dtype=np.int32)
    k2, v2 = pa.oracle_append(kp, vp, kn, vn, slots, dtype, dtype)
    kf, vf = kp.reshape(-1).copy(), vp.reshape(-1).copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = s // BS, s % BS
        for h in range(hkv):
            for dd in range(d):
                kf[(((blk * hkv + h) * (d // X) + dd // X) * BS + off) * X + dd % X] = kn[t, h, dd]
                vf[((blk * hkv + h) * d + dd) * BS + off] = vn[t, h, dd]
    assert k2.dtype == st and v2.dtype == st
    assert k2.reshape(-1).tobytes() == kf.tobytes()
    assert v2.reshape(-1).tobytes() == vf.tobytes()


def test_append_fp8_encodes_with_per_head_scale():
    rng = np.random.default_rng(17)
    nb, hkv, d = 3, 2, 64
    kp = np.zeros((nb, hkv, d // 16, BS, 16), np.uint8)
    vp = np.zeros((nb, hkv, d, BS), np.uint8)
    g = torch.Generator().manual_seed(17)
    kn = torch.randn(4, hkv, d, generator=g).bfloat16()
    vn = torch.randn(4, hkv, d, generator=g).bfloat16()
    kbits = kn.view(torch.int16).numpy().view(np.uint16)
    vbits = vn.view(torch.int16).numpy().view(np.uint16)
    # per-head absmax/448 keeps every quotient inside torch's non-saturating range
    ks = (kn.float().abs().amax(dim=(0, 2)).numpy() / np.float32(448)).astype(np.float32)
    vs = (vn.float().abs().amax(dim=(0, 2)).numpy() / np.float32(448)).astype(np.float32)
    slots = np.array([0, 17, 33, 47], np.int32)
    k2, v2 = pa.oracle_append(kp, vp, kbits, vbits, slots, "bf16", "fp8", ks, vs)
    for t, s in enumerate(slots):
        for h in range(hkv):
            want_k = torch.from_numpy((kn[t, h].float().numpy() / ks[h]).astype(np.float32)) \
                .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            want_v = torch.from_numpy((vn[t, h].float().numpy() / vs[h]).astype(np.float32)) \
                .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(k2[s // BS, h, :, s % BS, :].reshape(-1), want_k)
            assert np.array_equal(v2[s // BS, h, :, s % BS], want_v)


def test_append_then_gather_roundtrips_values():
    rng = np.random.default_rng(18)
    L = 37
    nb = 8
    table = np.array([5, 2, 7], np.int32)
    kn = rng.standard_normal((L, 2, 64)).astype(np.float32)
    vn = rng.standard_normal((L, 2, 64)).astype(np.float32)
    slots = np.array([table[p // BS] * BS + p % BS for p in range(L)], np.int32)
    kp = np.full((nb, 2, 16, BS, 4), np.nan, np.float32)
    vp = np.full((nb, 2, 64, BS), np.nan, np.float32)
    kp, vp = pa.oracle_append(kp, vp, kn, vn, slots, "f32", "f32")
    K, V = pa.gather_sequence(kp, vp, table, L, "f32")
    assert np.array_equal(K, kn.astype(np.float64))
    assert np.array_equal(V, vn.astype(np.float64))


def test_gather_refuses_tables_that_do_not_cover_the_context():
    kp = np.zeros((4, 1, 16, BS, 4), np.float32)
    vp = np.zeros((4, 1, 64, BS), np.float32)
    with pytest.raises(ValueError):
        pa.gather_sequence(kp, vp, np.array([1, -1], np.int32), 20, "f32")


# ---------------------------------------------------------------------------
# fp8 pools: the K and V scales (InferX, "The kernels underneath", FP8 KV cache
# paragraph: per-layer K/V scales; the mixed chunked-prefill workload's
# per-KV-head absmax/448 scales).  Codes are drawn over every finite E4M3 code,
# K and V get different scales on every head, and the expected values are
# dequantised by torch's own float8_e4m3fn conversion, not by oracle.fp8_e4m3.
# ---------------------------------------------------------------------------

FINITE_E4M3 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
FP8_K_SCALE = np.array([0.013, 0.0071, 0.029], np.float32)
FP8_V_SCALE = np.array([0.0047, 0.021, 0.0095], np.float32)


def _torch_dequant(codes, scale):
    """[L, Hkv, D] codes -> float64 values, decode(code) * scale[h], via torch."""
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    return (v * torch.from_numpy(scale.astype(np.float64))[None, :, None]).numpy()


def fp8_case(rng, lens, hq, hkv, d):
    """Random finite E4M3 codes for K and V of each sequence, laid out in a pool."""
    _, _, _, tables, nb = random_case(rng, lens, hq, hkv, d)
    kc = [FINITE_E4M3[rng.integers(0, len(FINITE_E4M3), (L, hkv, d))] for L in lens]
    vc = [FINITE_E4M3[rng.integers(0, len(FINITE_E4M3), (L, hkv, d))] for L in lens]
    return kc, vc, tables, nb


@pytest.mark.parametrize("hq,hkv", [(6, 3), (12, 3)])
def test_fp8_decode_matches_sdpa_on_dequantised_arrays(hq, hkv):
    rng = np.random.default_rng(40 + hq)
    lens = [17, 40, 77, 130]
    ks, vs = FP8_K_SCALE[:hkv], FP8_V_SCALE[:hkv]
    kc, vc, tables, nb = fp8_case(rng, lens, hq, hkv, 64)
    # scores of O(1): |code| <= 448, so a small query keeps softmax non-degenerate
    q = (rng.standard_normal((len(lens), hq, 64)) * 0.05).astype(np.float32)
    kp, vp = layout_pool(kc, vc, tables, nb, "fp8")
    out = pa.oracle_decode(q, "f32", kp, vp, "fp8", tables, lens, SCALE64, ks, vs)
    for b, L in enumerate(lens):
        ref = sdpa_reference(q[b:b + 1], [L - 1], _torch_dequant(kc[b], ks),
                             _torch_dequant(vc[b], vs), SCALE64)
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)


def test_fp8_prefill_matches_sdpa_on_dequantised_arrays():
    rng = np.random.default_rng(44)
    P, C, hq, hkv = 35, 30, 6, 3
    L = P + C
    ks, vs = FP8_K_SCALE[:hkv], FP8_V_SCALE[:hkv]
    kc, vc, tables, nb = fp8_case(rng, [L], hq, hkv, 64)
    qp = (rng.standard_normal((C, hq, 64)) * 0.05).astype(np.float32)
    kp, vp = layout_pool(kc, vc, tables, nb, "fp8")
    out = pa.oracle_prefill(qp, "f32", [0, C], kp, vp, "fp8", tables, [L], SCALE64, ks, vs)
    ref = sdpa_reference(qp, list(range(P, P + C)), _torch_dequant(kc[0], ks),
                         _torch_dequant(vc[0], vs), SCALE64)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_fp8_append_then_gather_returns_the_dequantised_codes():
    """bf16 rows -> oracle_append (fp8) -> gather_sequence equals torch's own
    float8_e4m3fn round trip of x / scale, times the head's scale, for K and V
    with different scales."""
    rng = np.random.default_rng(45)
    L, nb, hkv, d = 37, 8, 3, 64
    table = np.array([5, 2, 7], np.int32)
    g = torch.Generator().manual_seed(45)
    kn = torch.randn(L, hkv, d, generator=g).bfloat16()
    vn = torch.randn(L, hkv, d, generator=g).bfloat16()
    ks = (kn.float().abs().amax(dim=(0, 2)).numpy() / np.float32(448)).astype(np.float32)
    vs = (vn.float().abs().amax(dim=(0, 2)).numpy() / np.float32(448) * np.float32(1.5)).astype(np.float32)
    slots = np.array([table[p // BS] * BS + p % BS for p in range(L)], np.int32)
    kp = np.full((nb, hkv, d // 16, BS, 16), 0x7F, np.uint8)
    vp = np.full((nb, hkv, d, BS), 0x7F, np.uint8)
    kbits = kn.view(torch.int16).numpy().view(np.uint16)
    vbits = vn.view(torch.int16).numpy().view(np.uint16)
    kp, vp = pa.oracle_append(kp, vp, kbits, vbits, slots, "bf16", "fp8", ks, vs)
    K, V = pa.gather_sequence(kp, vp, table, L, "fp8", ks, vs)

    def want(x, s):
        y = torch.from_numpy((x.float().numpy() / s[None, :, None]).astype(np.float32))
        return _torch_dequant(y.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s)
    assert np.array_equal(K, want(kn, ks))
    assert np.array_equal(V, want(vn, vs))
