// Tile policies: how one wavefront loads a tile of paged K/V into MFMA
// operands and runs S^T = K Q^T and O^T += V^T P^T on it.
//
// Shared by the decode and prefill kernels.  A "tile" is TT consecutive
// logical positions (TB whole 16-token blocks).  Rows of S^T are keys, its 16
// columns are query rows (the GQA group in decode, padded to 16), so after
// the QK MFMAs lane l owns query column g = l % 16 and four keys per M-tile;
// the running max / sum of the online softmax therefore stay lane-local, and
// the same lane owns column g of the O^T accumulator.
//
// Within a tile the keys are permuted (the softmax is order-free): the
// permutation is chosen so that the P^T fragment a lane owns after QK is
// exactly the B operand the PV MFMA needs, and so that every lane's V^T
// operand is one 16-byte load from the token-minor V pool.
//
// Pools:  K [NB][Hkv][16][D]  (row = one token),  V [NB][Hkv][D][16].
#pragma once

#include "pa_device.hpp"

namespace pa {

// Query operand: the B operand of S^T = K Q^T for all D/32 (bf16) or D/4
// (fp32) k-steps, loaded once per wave.
template <int KIND, int D> struct TileOps;

// ----------------------------------------------------------------------------
// bf16 cache: 32-token tiles (2 blocks).
//   M-tile i (0,1), row m: block m/8, token 8*((m/4)&1) + 4i + (m&3)
//   => lane (g = l%16, q = l/16) owns positions 8q + 4i + r (r = 0..3) after QK
//   => its P^T B operand (k = 8q..8q+7) is positions 8q..8q+7,
//      its V^T A operand is V[block q/2][d][8(q&1) .. +7]: 16 bytes.
//   K-step s (D/32 of them), lane group q reads d = 8*(4s + q) .. +7.
// ----------------------------------------------------------------------------
template <int D> struct TileOps<kBF16, D> {
    static constexpr int TT = 32, TB = 2, NMT = 2, NS = D / 32, NVT = D / 16;
    static constexpr int ELEM = 2;
    struct Q { bf16x8 op[NS]; };
    struct Regs { u32x4 k[NMT][NS]; u32x4 v[NVT]; };

    // block of the tile this lane's K rows / V columns come from
    __device__ static int k_block(int lane) { return (lane & 15) >> 3; }
    __device__ static int v_block(int lane) { return (lane >> 4) >> 1; }

    __device__ static void load_q(Q& q, const uint16_t* qrow_g, bool valid, int lane) {
        const int grp = lane >> 4;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 v = valid ? load16_cached(qrow_g + 8 * (4 * s + grp)) : u32x4{0, 0, 0, 0};
            q.op[s] = as_bf16x8(v);
        }
    }
    // kblk/vblk: byte address of this lane's (block, head) K / V tile
    __device__ static void load(Regs& r, const char* kblk, const char* vblk, int lane) {
        const int m = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
            const int tok = 8 * ((m >> 2) & 1) + 4 * i + (m & 3);
            const char* row = kblk + tok * D * ELEM;
#pragma unroll
            for (int s = 0; s < NS; ++s) r.k[i][s] = load16(row + 16 * (4 * s + grp));
        }
        const char* vcol = vblk + (lane & 15) * kBlock * ELEM + 16 * (grp & 1);
#pragma unroll
        for (int t = 0; t < NVT; ++t) r.v[t] = load16(vcol + t * 16 * kBlock * ELEM);
    }
    __device__ static void qk(const Regs& r, const Q& q, f32x4 (&s)[NMT]) {
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NS; ++k) acc = mfma_bf16(as_bf16x8(r.k[i][k]), q.op[k], acc);
            s[i] = acc;
        }
    }
    // position (within the tile) of score (M-tile i, element e) of lane group grp
    __device__ static int pos(int i, int e, int grp) { return 8 * grp + 4 * i + e; }
    // zero V^T elements at positions >= nvalid (their bits may be NaN)
    __device__ static void mask_v(Regs& r, int nvalid, int lane) {
        const int base = 8 * (lane >> 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t keep = (base + 2 * w < nvalid ? 0x0000FFFFu : 0u) |
                            (base + 2 * w + 1 < nvalid ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int t = 0; t < NVT; ++t) r.v[t][w] &= keep;
        }
    }
    // p[i][e]: probabilities in the lane's score layout
    __device__ static void pv(const Regs& r, const float (&p)[NMT][4], f32x4 (&o)[NVT]) {
        u32x4 pk;
        pk[0] = pack_bf16x2(p[0][0], p[0][1]);
        pk[1] = pack_bf16x2(p[0][2], p[0][3]);
        pk[2] = pack_bf16x2(p[1][0], p[1][1]);
        pk[3] = pack_bf16x2(p[1][2], p[1][3]);
        const bf16x8 b = as_bf16x8(pk);
#pragma unroll
        for (int t = 0; t < NVT; ++t) o[t] = mfma_bf16(as_bf16x8(r.v[t]), b, o[t]);
    }
};

// ----------------------------------------------------------------------------
// fp8 (OCP e4m3) cache: 64-token tiles (4 blocks), converted to bf16 in
// registers (exact) and multiplied on the bf16 MFMA.
//   M-tile i (0..3), row m: block m/4, token 4i + (m&3)
//   => lane group q owns block q, positions 16q + 4i + r
//   => PV MFMA a (0,1) takes k = 8q+j <-> position 16q + 8a + j, so the V^T
//      operand of lane (d, q) is one 16-byte row V[block q][d][0..15].
//   K loads: lane group q reads bytes 16(q + 4u) .. +15 of a row (u < D/64);
//   k-step s = 2u + h covers d = 16(q + 4u) + 8h .. +7.
// ----------------------------------------------------------------------------
template <int D> struct TileOps<kFP8, D> {
    static constexpr int TT = 64, TB = 4, NMT = 4, NS = D / 32, NU = D / 64, NVT = D / 16;
    static constexpr int ELEM = 1;
    struct Q { bf16x8 op[NS]; };
    struct Regs { u32x4 k[NMT][NU]; u32x4 v[NVT]; };

    __device__ static int k_block(int lane) { return (lane & 15) >> 2; }
    __device__ static int v_block(int lane) { return lane >> 4; }

    __device__ static void load_q(Q& q, const uint16_t* qrow_g, bool valid, int lane) {
        const int grp = lane >> 4;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d0 = 16 * (grp + 4 * (s >> 1)) + 8 * (s & 1);
            u32x4 v = valid ? load16_cached(qrow_g + d0) : u32x4{0, 0, 0, 0};
            q.op[s] = as_bf16x8(v);
        }
    }
    __device__ static void load(Regs& r, const char* kblk, const char* vblk, int lane) {
        const int m = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
            const char* row = kblk + (4 * i + (m & 3)) * D;
#pragma unroll
            for (int u = 0; u < NU; ++u) r.k[i][u] = load16(row + 16 * (grp + 4 * u));
        }
        const char* vcol = vblk + (lane & 15) * kBlock;
#pragma unroll
        for (int t = 0; t < NVT; ++t) r.v[t] = load16(vcol + t * 16 * kBlock);
    }
    __device__ static void qk(const Regs& r, const Q& q, f32x4 (&s)[NMT]) {
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                acc = mfma_bf16(fp8x8_to_bf16x8(r.k[i][u][0], r.k[i][u][1]), q.op[2 * u], acc);
                acc = mfma_bf16(fp8x8_to_bf16x8(r.k[i][u][2], r.k[i][u][3]), q.op[2 * u + 1], acc);
            }
            s[i] = acc;
        }
    }
    __device__ static int pos(int i, int e, int grp) { return 16 * grp + 4 * i + e; }
    __device__ static void mask_v(Regs& r, int nvalid, int lane) {
        const int base = 16 * (lane >> 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t keep = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                keep |= (base + 4 * w + b < nvalid ? 0xFFu : 0u) << (8 * b);
#pragma unroll
            for (int t = 0; t < NVT; ++t) r.v[t][w] &= keep;
        }
    }
    __device__ static void pv(const Regs& r, const float (&p)[NMT][4], f32x4 (&o)[NVT]) {
        u32x4 p0, p1;
        p0[0] = pack_bf16x2(p[0][0], p[0][1]);
        p0[1] = pack_bf16x2(p[0][2], p[0][3]);
        p0[2] = pack_bf16x2(p[1][0], p[1][1]);
        p0[3] = pack_bf16x2(p[1][2], p[1][3]);
        p1[0] = pack_bf16x2(p[2][0], p[2][1]);
        p1[1] = pack_bf16x2(p[2][2], p[2][3]);
        p1[2] = pack_bf16x2(p[3][0], p[3][1]);
        p1[3] = pack_bf16x2(p[3][2], p[3][3]);
        const bf16x8 b0 = as_bf16x8(p0), b1 = as_bf16x8(p1);
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            o[t] = mfma_bf16(fp8x8_to_bf16x8(r.v[t][0], r.v[t][1]), b0, o[t]);
            o[t] = mfma_bf16(fp8x8_to_bf16x8(r.v[t][2], r.v[t][3]), b1, o[t]);
        }
    }
};

// ----------------------------------------------------------------------------
// fp32 cache: 16-token tiles (1 block) on the fp32 MFMA (k = 4 per step).
//   token order is the identity; lane group q owns positions 4q + r.
//   K loads: lane group q reads d = 16u + 4q .. +3 (u < D/16); k-step (u, j)
//   covers d = 16u + 4q + j.  PV step i takes k = q <-> position 4q + i, so
//   the V^T operand of lane (d, q) is V[d][4q .. 4q+3]: 16 bytes.
// ----------------------------------------------------------------------------
template <int D> struct TileOps<kF32, D> {
    static constexpr int TT = 16, TB = 1, NMT = 1, NU = D / 16, NVT = D / 16;
    static constexpr int ELEM = 4;
    struct Q { f32x4 op[NU]; };
    struct Regs { f32x4 k[NU]; f32x4 v[NVT]; };

    __device__ static int k_block(int) { return 0; }
    __device__ static int v_block(int) { return 0; }

    __device__ static void load_q(Q& q, const float* qrow_g, bool valid, int lane) {
        const int grp = lane >> 4;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            u32x4 v = valid ? load16_cached(qrow_g + 16 * u + 4 * grp) : u32x4{0, 0, 0, 0};
            q.op[u] = __builtin_bit_cast(f32x4, v);
        }
    }
    __device__ static void load(Regs& r, const char* kblk, const char* vblk, int lane) {
        const int m = lane & 15, grp = lane >> 4;
        const char* row = kblk + m * D * ELEM;
#pragma unroll
        for (int u = 0; u < NU; ++u)
            r.k[u] = __builtin_bit_cast(f32x4, load16(row + (16 * u + 4 * grp) * ELEM));
        const char* vcol = vblk + (lane & 15) * kBlock * ELEM + 16 * grp;
#pragma unroll
        for (int t = 0; t < NVT; ++t)
            r.v[t] = __builtin_bit_cast(f32x4, load16(vcol + t * 16 * kBlock * ELEM));
    }
    __device__ static void qk(const Regs& r, const Q& q, f32x4 (&s)[NMT]) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = mfma_f32(r.k[u][j], q.op[u][j], acc);
        s[0] = acc;
    }
    __device__ static int pos(int, int e, int grp) { return 4 * grp + e; }
    __device__ static void mask_v(Regs& r, int nvalid, int lane) {
        const int base = 4 * (lane >> 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool keep = base + e < nvalid;
#pragma unroll
            for (int t = 0; t < NVT; ++t) r.v[t][e] = keep ? r.v[t][e] : 0.0f;
        }
    }
    __device__ static void pv(const Regs& r, const float (&p)[NMT][4], f32x4 (&o)[NVT]) {
#pragma unroll
        for (int t = 0; t < NVT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[t] = mfma_f32(r.v[t][e], p[0][e], o[t]);
    }
};

}  // namespace pa

namespace pa {

// Online-softmax state of one wavefront over a 16-column query tile.
// Lane (g = l%16, grp = l/16) owns column g: m and the lane-partial l are per
// column (l is summed over the 4 lane groups at the end), o[t] holds
// O^T[d = 16t + 4grp + i][g].
template <int KIND, int D> struct WaveSoftmax {
    using Ops = TileOps<KIND, D>;
    static constexpr int NMT = Ops::NMT, NVT = Ops::NVT, TT = Ops::TT;
    float m = -INFINITY, l = 0.f;
    f32x4 o[NVT];

    __device__ void init() {
#pragma unroll
        for (int t = 0; t < NVT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One tile.  c: log2-domain score multiplier.  nvalid: positions of the
    // tile that hold real tokens (V of the rest is zeroed, their scores are
    // -inf).  limit: this lane's last visible tile position (causal rows;
    // >= TT-1 means no causal cut).  masked: some position needs masking.
    __device__ void step(typename Ops::Regs& r, const typename Ops::Q& q, float c, int nvalid,
                         int limit, bool masked, int lane) {
        const int grp = lane >> 4;
        f32x4 s4[NMT];
        Ops::qk(r, q, s4);
        float s[NMT][4];
#pragma unroll
        for (int i = 0; i < NMT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[i][e] = s4[i][e] * c;
        if (masked) {
            const int lim = min(limit, nvalid - 1);
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[i][e] = Ops::pos(i, e, grp) <= lim ? s[i][e] : -INFINITY;
            if (nvalid < TT) Ops::mask_v(r, nvalid, lane);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < NMT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, s[i][e]);
        tmax = max_over_groups(tmax);
        const float m_new = fmaxf(m, tmax);
        // a column with nothing visible yet keeps m = -inf: use 0 as reference
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_ref);
        m = m_new;
        float p[NMT][4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < NMT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[i][e] = fast_exp2(s[i][e] - m_ref);
                psum += p[i][e];
            }
        l = l * alpha + psum;
#pragma unroll
        for (int t = 0; t < NVT; ++t) o[t] *= alpha;
        Ops::pv(r, p, o);
    }
};

}  // namespace pa
