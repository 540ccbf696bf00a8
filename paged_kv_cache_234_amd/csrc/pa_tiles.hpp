// Tile policies: how one wavefront loads a tile of paged K/V into MFMA
// operands and runs S^T = K Q^T and O^T += V^T P^T on it.
//
// Shared by the decode and prefill kernels.  A "tile" is TT consecutive
// logical positions, i.e. TB whole 16-token blocks.  Rows of S^T are keys,
// its 16 columns are query rows (the GQA group in decode, padded to 16), so
// after the QK MFMAs lane l owns query column g = l % 16 and four keys per
// M-tile; the running max / sum of the online softmax therefore stay
// lane-local, and the same lane owns column g of the O^T accumulator.
//
// Pools (X = 16 bytes of elements: 4 fp32, 8 bf16, 16 fp8):
//   K [NB][Hkv][D/X][16][X]   -- one M-tile = one block; the A operand of
//                                k-step s for lane l is the 16 bytes at
//                                chunk (lane group + 4s), token (l % 16), so
//                                each load instruction reads 1 KB contiguous
//   V [NB][Hkv][D][16]        -- token-minor: a lane's PV operand (8 or 16
//                                consecutive keys of one head-dim column) is
//                                one 16-byte load
// After QK, lane group q holds keys 4q..4q+3 of every block of the tile.  For
// bf16 and fp8 the probabilities are then exchanged between lane groups with
// v_permlane16/32_swap (on packed bf16 pairs) so that each lane group owns
// whole runs of keys, matching the V operand it loads.
#pragma once

#include "pa_device.hpp"

namespace pa {

template <int KIND, int D> struct TileOps;

// Occupancy the streaming kernels are compiled for: the D = 128 bf16 / fp8
// variants keep two tiles of K/V (32 KB per wave) in registers, which fits
// without spilling only at one wave per SIMD; four such waves per CU already
// keep enough bytes in flight to saturate HBM.
constexpr int waves_per_simd(int kind, int d) { return d == 128 ? 1 : 2; }

// ----------------------------------------------------------------------------
// bf16 cache: 32-token tiles (2 blocks).
//   M-tile i = block i; lane group q holds keys 16i + 4q + r after QK.
//   PV (16x16x32): lane group q owns keys 8q .. 8q+7 = block q/2, tokens
//   8(q&1) .. +7, so its V operand is V[block q/2][d][8(q&1) .. +7].
//   Exchange: with P_i the packed probabilities of block i (row j = lane
//   group j = keys 4j..4j+3), swap32(P0, P1) then swap16(P0', P1') leaves
//   row q of (P0'', P1'') = keys 8q..8q+3, 8q+4..8q+7.
// ----------------------------------------------------------------------------
template <int D> struct TileOps<kBF16, D> {
    static constexpr int TT = 32, TB = 2, NMT = 2, NS = D / 32, NVT = D / 16;
    static constexpr int ELEM = 2;
    struct Q { bf16x8 op[NS]; };
    struct Regs { u32x4 k[NMT][NS]; u32x4 v[NVT]; };

    __device__ static void load_q(Q& q, const uint16_t* qrow_g, bool valid, int lane) {
        const int grp = lane >> 4;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 v = valid ? load16_cached(qrow_g + 8 * (4 * s + grp)) : u32x4{0, 0, 0, 0};
            q.op[s] = as_bf16x8(v);
        }
    }
    // kbase / vbase: this head's tile in block 0; phys[i]: physical id of the
    // tile's i-th block; blk: bytes between consecutive physical blocks
    __device__ static void load(Regs& r, const char* kbase, const char* vbase, long blk,
                                const int (&phys)[TB], int lane) {
#pragma unroll
        for (int i = 0; i < NMT; ++i)
#pragma unroll
            for (int s = 0; s < NS; ++s)
                r.k[i][s] = load16(kbase + phys[i] * blk + 1024 * s + 16 * lane);
        const int grp = lane >> 4;
        const long pv = (grp >> 1) ? phys[1] : phys[0];
        const char* vcol = vbase + pv * blk + (lane & 15) * kBlock * ELEM + 16 * (grp & 1);
#pragma unroll
        for (int t = 0; t < NVT; ++t) r.v[t] = load16(vcol + t * 16 * kBlock * ELEM);
    }
    // S^T for NC query tiles sharing the K operand
    template <int NC>
    __device__ static void qk(const Regs& r, const Q (&q)[NC], f32x4 (&s)[NC][NMT]) {
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
#pragma unroll
            for (int n = 0; n < NC; ++n) s[n][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const bf16x8 a = as_bf16x8(r.k[i][k]);
#pragma unroll
                for (int n = 0; n < NC; ++n) s[n][i] = mfma_bf16(a, q[n].op[k], s[n][i]);
            }
        }
    }
    // position (within the tile) of score (M-tile i, element e) of lane group grp
    __device__ static int pos(int i, int e, int grp) { return 16 * i + 4 * grp + e; }
    // zero V^T elements at positions >= nvalid (their bits may be NaN);
    // lane group q holds positions 8q .. 8q+7
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
    template <int NC>
    __device__ static void pv(const Regs& r, const float (&p)[NC][NMT][4],
                              f32x4 (&o)[NC][NVT]) {
        bf16x8 b[NC];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            uint32_t a0 = pack_bf16x2(p[n][0][0], p[n][0][1]), b0 = pack_bf16x2(p[n][0][2], p[n][0][3]);
            uint32_t a1 = pack_bf16x2(p[n][1][0], p[n][1][1]), b1 = pack_bf16x2(p[n][1][2], p[n][1][3]);
            permlane32_swap(a0, a1);
            permlane32_swap(b0, b1);
            permlane16_swap(a0, a1);
            permlane16_swap(b0, b1);
            b[n] = as_bf16x8(u32x4{a0, b0, a1, b1});
        }
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const bf16x8 a = as_bf16x8(r.v[t]);
#pragma unroll
            for (int n = 0; n < NC; ++n) o[n][t] = mfma_bf16(a, b[n], o[n][t]);
        }
    }
};

// ----------------------------------------------------------------------------
// fp8 (OCP e4m3) cache: 64-token tiles (4 blocks), widened to bf16 in
// registers (exact) and multiplied on the bf16 MFMA.
//   M-tile i = block i; lane group q holds keys 16i + 4q + r after QK.
//   K loads: lane group q reads chunk (q + 4u) (d = 16(q+4u) .. +15), u < D/64;
//   k-step s = 2u + h covers d = 16(q + 4u) + 8h .. +7.
//   A 4x4 transpose of (block, lane group) by swap32 then swap16 gives lane
//   group q all 16 keys of block q (register k: keys 4k..4k+3); PV MFMA a
//   (0, 1) takes keys 8a..8a+7, so its V operand is one 16-byte row
//   V[block q][d][0..15].
// ----------------------------------------------------------------------------
template <int D> struct TileOps<kFP8, D> {
    static constexpr int TT = 64, TB = 4, NMT = 4, NS = D / 32, NU = D / 64, NVT = D / 16;
    static constexpr int ELEM = 1;
    struct Q { bf16x8 op[NS]; };
    struct Regs { u32x4 k[NMT][NU]; u32x4 v[NVT]; };

    __device__ static void load_q(Q& q, const uint16_t* qrow_g, bool valid, int lane) {
        const int grp = lane >> 4;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d0 = 16 * (grp + 4 * (s >> 1)) + 8 * (s & 1);
            u32x4 v = valid ? load16_cached(qrow_g + d0) : u32x4{0, 0, 0, 0};
            q.op[s] = as_bf16x8(v);
        }
    }
    __device__ static void load(Regs& r, const char* kbase, const char* vbase, long blk,
                                const int (&phys)[TB], int lane) {
#pragma unroll
        for (int i = 0; i < NMT; ++i)
#pragma unroll
            for (int u = 0; u < NU; ++u)
                r.k[i][u] = load16(kbase + phys[i] * blk + 1024 * u + 16 * lane);
        const int grp = lane >> 4;
        const long pv = grp == 0 ? phys[0] : grp == 1 ? phys[1] : grp == 2 ? phys[2] : phys[3];
        const char* vcol = vbase + pv * blk + (lane & 15) * kBlock;
#pragma unroll
        for (int t = 0; t < NVT; ++t) r.v[t] = load16(vcol + t * 16 * kBlock);
    }
    template <int NC>
    __device__ static void qk(const Regs& r, const Q (&q)[NC], f32x4 (&s)[NC][NMT]) {
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
#pragma unroll
            for (int n = 0; n < NC; ++n) s[n][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const bf16x8 a0 = fp8x8_to_bf16x8(r.k[i][u][0], r.k[i][u][1]);
                const bf16x8 a1 = fp8x8_to_bf16x8(r.k[i][u][2], r.k[i][u][3]);
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    s[n][i] = mfma_bf16(a0, q[n].op[2 * u], s[n][i]);
                    s[n][i] = mfma_bf16(a1, q[n].op[2 * u + 1], s[n][i]);
                }
            }
        }
    }
    __device__ static int pos(int i, int e, int grp) { return 16 * i + 4 * grp + e; }
    // lane group q holds positions 16q .. 16q+15 (block q)
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
    template <int NC>
    __device__ static void pv(const Regs& r, const float (&p)[NC][NMT][4],
                              f32x4 (&o)[NC][NVT]) {
        bf16x8 b0[NC], b1[NC];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            uint32_t a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = pack_bf16x2(p[n][i][0], p[n][i][1]);
                b[i] = pack_bf16x2(p[n][i][2], p[n][i][3]);
            }
            permlane32_swap(a[0], a[2]);
            permlane32_swap(b[0], b[2]);
            permlane32_swap(a[1], a[3]);
            permlane32_swap(b[1], b[3]);
            permlane16_swap(a[0], a[1]);
            permlane16_swap(b[0], b[1]);
            permlane16_swap(a[2], a[3]);
            permlane16_swap(b[2], b[3]);
            b0[n] = as_bf16x8(u32x4{a[0], b[0], a[1], b[1]});
            b1[n] = as_bf16x8(u32x4{a[2], b[2], a[3], b[3]});
        }
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const bf16x8 v0 = fp8x8_to_bf16x8(r.v[t][0], r.v[t][1]);
            const bf16x8 v1 = fp8x8_to_bf16x8(r.v[t][2], r.v[t][3]);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                o[n][t] = mfma_bf16(v0, b0[n], o[n][t]);
                o[n][t] = mfma_bf16(v1, b1[n], o[n][t]);
            }
        }
    }
};

// ----------------------------------------------------------------------------
// fp32 cache: 16-token tiles (1 block) on the fp32 MFMA (k = 4 per step).
//   K loads: lane group q reads chunk 4u + q (d = 16u + 4q .. +3); k-step
//   (u, j) covers d = 16u + 4q + j.  Lane group q holds keys 4q .. 4q+3; PV
//   step i takes k = q <-> key 4q + i, so the V^T operand of lane (d, q) is
//   V[d][4q .. 4q+3]: 16 bytes, and a load instruction reads 1 KB contiguous.
// ----------------------------------------------------------------------------
template <int D> struct TileOps<kF32, D> {
    static constexpr int TT = 16, TB = 1, NMT = 1, NU = D / 16, NVT = D / 16;
    static constexpr int ELEM = 4;
    struct Q { f32x4 op[NU]; };
    struct Regs { f32x4 k[NU]; f32x4 v[NVT]; };

    __device__ static void load_q(Q& q, const float* qrow_g, bool valid, int lane) {
        const int grp = lane >> 4;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            u32x4 v = valid ? load16_cached(qrow_g + 16 * u + 4 * grp) : u32x4{0, 0, 0, 0};
            q.op[u] = __builtin_bit_cast(f32x4, v);
        }
    }
    __device__ static void load(Regs& r, const char* kbase, const char* vbase, long blk,
                                const int (&phys)[TB], int lane) {
        const char* kb = kbase + phys[0] * blk;
#pragma unroll
        for (int u = 0; u < NU; ++u)
            r.k[u] = __builtin_bit_cast(f32x4, load16(kb + 1024 * u + 16 * lane));
        const char* vcol = vbase + phys[0] * blk + (lane & 15) * kBlock * ELEM + 16 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < NVT; ++t)
            r.v[t] = __builtin_bit_cast(f32x4, load16(vcol + t * 16 * kBlock * ELEM));
    }
    template <int NC>
    __device__ static void qk(const Regs& r, const Q (&q)[NC], f32x4 (&s)[NC][NMT]) {
#pragma unroll
        for (int n = 0; n < NC; ++n) s[n][0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int n = 0; n < NC; ++n) s[n][0] = mfma_f32(r.k[u][j], q[n].op[u][j], s[n][0]);
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
    template <int NC>
    __device__ static void pv(const Regs& r, const float (&p)[NC][NMT][4],
                              f32x4 (&o)[NC][NVT]) {
#pragma unroll
        for (int t = 0; t < NVT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int n = 0; n < NC; ++n) o[n][t] = mfma_f32(r.v[t][e], p[n][0][e], o[n][t]);
    }
};

// Online-softmax state of one wavefront over a 16-column query tile.
// Lane (g = l%16, grp = l/16) owns column g: the running max m, the exponent
// reference mr and the lane-partial l are per column (l is summed over the 4
// lane groups at the end), o[t] holds O^T[d = 16t + 4grp + i][g].
//
// The reference mr only moves when a tile's max exceeds it by more than
// kRescaleSlack (log2 units), so the rescale of O (32 registers at D = 128) is
// skipped on most tiles; probabilities are then at most 2^kRescaleSlack, well
// inside fp32 and bf16 range.  The result o / l does not depend on mr, and
// finish() re-expresses l against the true max.
constexpr float kRescaleSlack = 8.0f;

template <int KIND, int D, int NC = 1>
struct WaveSoftmax {
    using Ops = TileOps<KIND, D>;
    static constexpr int NMT = Ops::NMT, NVT = Ops::NVT, TT = Ops::TT;
    float m[NC], mr[NC], l[NC];
    f32x4 o[NC][NVT];

    __device__ void init() {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            m[n] = -INFINITY;
            mr[n] = -INFINITY;
            l[n] = 0.f;
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[n][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // One tile for NC query tiles.  c: log2-domain score multiplier.  nvalid:
    // positions of the tile that hold real tokens (V of the rest is zeroed,
    // their scores are -inf).  limit[n]: this lane's last visible tile
    // position in query tile n (causal rows; >= TT-1 means no causal cut).
    // masked: some position of some query tile needs masking.
    __device__ void step(typename Ops::Regs& r, const typename Ops::Q (&q)[NC], float c,
                         int nvalid, const int (&limit)[NC], bool masked, int lane) {
        const int grp = lane >> 4;
        f32x4 s4[NC][NMT];
        Ops::template qk<NC>(r, q, s4);
        if (masked && nvalid < TT) Ops::mask_v(r, nvalid, lane);
        float p[NC][NMT][4];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            float s[NMT][4];
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[i][e] = s4[n][i][e] * c;
            if (masked) {
                const int lim = min(limit[n], nvalid - 1);
#pragma unroll
                for (int i = 0; i < NMT; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[i][e] = Ops::pos(i, e, grp) <= lim ? s[i][e] : -INFINITY;
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, s[i][e]);
            rescale(n, max_over_groups(tmax));
            // a column with nothing visible yet keeps mr = -inf: use 0 as reference
            const float ref = (mr[n] == -INFINITY) ? 0.f : mr[n];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[n][i][e] = fast_exp2(s[i][e] - ref);
                    psum += p[n][i][e];
                }
            l[n] += psum;
        }
        Ops::template pv<NC>(r, p, o);
    }

    // bump the reference scale of query tile n to the running max when the
    // tile max tmax exceeds it by more than the slack
    __device__ void rescale(int n, float tmax) {
        m[n] = fmaxf(m[n], tmax);
        const bool bump = tmax > mr[n] + kRescaleSlack;     // true for the first finite max
        if (__builtin_amdgcn_ballot_w64(bump)) {
            // columns that keep their reference scale by exactly 1 (a column
            // that has seen nothing yet keeps mr = -inf, where exp2(mr - mr)
            // would be NaN); a first finite max scales by 0
            const float mr_new = bump ? m[n] : mr[n];
            const float alpha = bump ? fast_exp2(mr[n] - mr_new) : 1.0f;
            mr[n] = mr_new;
            l[n] *= alpha;
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[n][t] *= alpha;
        }
    }
};

// Stream tiles [n0, n1) of one wavefront through `compute(regs, n)`.
//
// Tile n covers logical blocks blk0 + n*TB .. +TB-1 (clamped to last_blk; the
// clamped copies are masked by the caller).  Block ids come from a register
// holding 64 consecutive block-table entries (one coalesced load per 64
// blocks, read back with v_readlane), so no memory latency sits between two
// tiles' loads.  The next tile's loads are always in flight while the current
// tile is multiplied, and the loop is peeled so that every multiply site has
// a fixed number of loads issued after its own: the compiler's vmcnt waits
// then cover exactly the tile being consumed.
template <int KIND, int D, class Compute>
__device__ __forceinline__ void stream_tiles(const int32_t* __restrict__ bt_row, int blk0,
                                             int last_blk, int n0, int n1, const char* kbase,
                                             const char* vbase, long blk_stride, int lane,
                                             Compute&& compute) {
    using Ops = TileOps<KIND, D>;
    constexpr int TB = Ops::TB, TPC = kWave / TB;        // tiles per 64-block chunk
    for (int c0 = n0; c0 < n1; c0 += TPC) {
        const int c1 = min(n1, c0 + TPC);
        const int base = blk0 + c0 * TB;
        const int span = last_blk - base;                // last valid index into `ids`
        const int ids = (lane <= span) ? bt_row[base + lane] : 0;
        auto issue = [&](typename Ops::Regs& r, int n) {
            const int rel = (n - c0) * TB;
            int ph[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j) ph[j] = __builtin_amdgcn_readlane(ids, min(rel + j, span));
            Ops::load(r, kbase, vbase, blk_stride, ph, lane);
        };
        typename Ops::Regs ra, rb;
        int n = c0;
        issue(ra, n);
        while (true) {
            if (n + 1 < c1) {
                issue(rb, n + 1);
                compute(ra, n);
            } else {
                compute(ra, n);
                break;
            }
            ++n;
            if (n + 1 < c1) {
                issue(ra, n + 1);
                compute(rb, n);
            } else {
                compute(rb, n);
                break;
            }
            ++n;
        }
    }
}

}  // namespace pa
