// Causal prefill chunks over a paged cache, gfx950.
//
// A chunk of C query tokens starting after P cached tokens (context length
// L = P + C, its own K/V already appended) attends causally: query i, at
// position P + i, sees keys 0 .. P + i (InferX, "Status": chunked prefill;
// infer-lab, invariants: prefilling in chunks gives the one-shot result;
// llm-infer, "What It Does": prefill of ragged batches, optionally chunked).
//
// Work decomposition: the 16 MFMA columns of a wavefront's query tile are
// npos = 16 / G consecutive query positions times the G query heads of one KV
// head, so each K/V tile a wavefront loads feeds npos * G query rows.  A
// workgroup holds NW consecutive query tiles of the same (chunk, KV head);
// their K/V streams overlap, so the later wavefronts mostly hit L2.  Each
// wavefront walks key tiles 0 .. (its last position) with the next tile's
// loads in flight, masking per column only on the tiles that cross a causal
// boundary or the end of the context.
#include <cfloat>

#include "pa_internal.hpp"
#include "pa_tiles.hpp"

namespace pa {

struct PrefillArgs {
    void* out;
    const void* q;
    const char* k_cache;
    const char* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* query_start_loc;
    int max_blocks_per_seq;
    int num_heads;
    int num_kv_heads;
    int group;          // G
    int npos;           // query positions per 16-column tile
    int wg_per_head;    // workgroups per (chunk, KV head)
    int num_chunks;
    int num_cus;        // compute units: the stride between workgroups sharing one
    float scale_log2;
};

template <int KIND> struct PQType { using T = uint16_t; };
template <> struct PQType<kF32> { using T = float; };

// Query tiles per wavefront: each K/V tile a wavefront loads (and, for fp8,
// widens to bf16) feeds NC * 16 query rows.
constexpr int prefill_tiles_per_wave(int kind, int d) {
    return kind == kF32 ? 1 : 2;
}

template <int KIND, int D, int NW, int NC>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(waves_per_simd(KIND, D))))
void prefill_kernel(PrefillArgs a) {
    using Ops = TileOps<KIND, D>;
    using QT = typename PQType<KIND>::T;
    constexpr int TT = Ops::TT, NVT = Ops::NVT, ELEM = Ops::ELEM;

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int tg = item % a.wg_per_head;
    const int h = (item / a.wg_per_head) % a.num_kv_heads;
    const int c = item / (a.wg_per_head * a.num_kv_heads);

    const int q0 = a.query_start_loc[c];
    const int C = a.query_start_loc[c + 1] - q0;
    // positions past the chunk's block-table row are never read
    const int L = min(a.context_lens[c], a.max_blocks_per_seq * kBlock);
    const int P = L - C;
    const int npos = a.npos;
    const int row0 = (tg * NW + wave) * NC * npos;       // first chunk row of this wavefront
    if (row0 >= C || P < 0) return;
    const int wrows = min(NC * npos, C - row0);

    const int g = lane & 15, grp = lane >> 4;
    const int pi = g / a.group, gh = g % a.group;        // column -> (row in tile, head)
    typename Ops::Q qop[NC];
    int my_last[NC];                                     // last key each column sees
    bool col_valid[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int r = n * npos + pi;
        col_valid[n] = pi < npos && r < wrows;
        const QT* qrow = reinterpret_cast<const QT*>(a.q) +
                         ((long)(q0 + row0 + r) * a.num_heads + h * a.group + gh) * D;
        Ops::load_q(qop[n], qrow, col_valid[n], lane);
        my_last[n] = P + row0 + (col_valid[n] ? r : 0);
    }

    float cs = a.scale_log2;
    if (KIND == kFP8) cs *= a.k_scale[h];

    const int min_last = P + row0;                       // smallest over the wavefront
    const int kend = P + row0 + wrows;                   // keys [0, kend) are touched
    const int ntiles = (kend + TT - 1) / TT;
    const int last_blk = (kend - 1) / kBlock;
    const int32_t* bt = a.block_tables + (long)c * a.max_blocks_per_seq;

    const long head_stride = (long)kBlock * D * ELEM;
    const long blk_stride = head_stride * a.num_kv_heads;
    const char* kbase = a.k_cache + h * head_stride;
    const char* vbase = a.v_cache + h * head_stride;
    WaveSoftmax<KIND, D, NC> st;
    st.init();
    stream_tiles<KIND, D>(bt, 0, last_blk, 0, ntiles, kbase, vbase, blk_stride, lane,
                          [&](typename Ops::Regs& r, int n) {
                              const int t0 = n * TT;
                              const int nvalid = kend - t0;
                              const bool masked = (t0 + TT - 1 > min_last) || (nvalid < TT);
                              int limit[NC];
#pragma unroll
                              for (int k = 0; k < NC; ++k) limit[k] = my_last[k] - t0;
                              st.step(r, qop, cs, nvalid, limit, masked, lane);
                          });

    const float vs = KIND == kFP8 ? a.v_scale[h] : 1.0f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float l = sum_over_groups(st.l[n]);        // against the reference mr
        if (!col_valid[n]) continue;
        const float inv = vs / l;
        const long orow =
            ((long)(q0 + row0 + n * npos + pi) * a.num_heads + h * a.group + gh) * D;
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const int d = 16 * t + 4 * grp;
            const f32x4 v = st.o[n][t] * inv;
            if (KIND == kF32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow + d) = v;
            } else {
                u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow + d) = pk;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// LDS-staged prefill for bf16 and fp8 caches.
//
// The register-streaming kernel above loads every K/V tile once per
// wavefront, so at 32 query rows per wavefront the bytes it pulls from L2
// per MFMA are several times what L2 can feed.  Here the four wavefronts of
// a workgroup work on the same (chunk, KV head) and share each 64-position
// K/V tile through LDS: wavefront w loads block w of the tile (its physical
// id is wave-uniform, a scalar load), widens fp8 to bf16 on the way, and
// writes it in the layouts the bf16 MFMA operands read as one contiguous
// 1 KB per wave-wide 16-byte LDS read:
//   K  [half][M-tile][D/8][16 rows][8 dims]       (rows in key-pair order)
//   V  [half][D/16][key run q][16 dims][8 keys]   (half = 32 positions; run q
//                                                  = keys 8q .. 8q+7)
// Each wavefront then runs NC 16-column query tiles over the tile, two
// 32-position halves through the bf16 tile operations.  Tiles are double
// buffered: the next tile's global loads are in flight during the multiply,
// and one barrier per tile orders the LDS writes against the reads.
// ---------------------------------------------------------------------------
constexpr int kLdsTile = 64;                  // positions per staged tile (4 blocks)
constexpr int kLdsCols = 2;                   // 16-column query tiles per wavefront

// Staged K rows in key-pair order: in each 32-position half, M-tile i row
// 4j + e holds key 8j + 4i + e.  After QK^T lane group j then holds keys
// 8j .. 8j+7 of its query column (M-tile 0: 8j .. 8j+3, M-tile 1: 8j+4 ..
// 8j+7), which is already the PV operand layout: no lane exchange.
template <int D> struct StagedOps : TileOps<kBF16, D> {
    using Base = TileOps<kBF16, D>;
    using Regs = typename Base::Regs;
    static constexpr int NMT = Base::NMT, NVT = Base::NVT;
    __device__ static int pos(int i, int e, int grp) { return 8 * grp + 4 * i + e; }
    // M-tile and row of key k (< 32) of a half
    __host__ __device__ static constexpr int tile_of(int k) { return (k >> 2) & 1; }
    __host__ __device__ static constexpr int row_of(int k) { return 4 * (k >> 3) + (k & 3); }
    // S^T of query tile n is complete before tile n + 1's is started
    template <int NC>
    __device__ static void qk(const Regs& r, const typename Base::Q (&q)[NC],
                              f32x4 (&s)[NC][NMT]) {
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
            for (int i = 0; i < NMT; ++i) {
                s[n][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < Base::NS; ++k)
                    s[n][i] = mfma_bf16(as_bf16x8(r.k[i][k]), q[n].op[k], s[n][i]);
            }
    }
    // O^T of one query tile from its probabilities, and the column sums of
    // the same bf16 probabilities on the matrix core: an all-ones A operand
    // gives every row of the 16x16 result the sum over the 32 keys, so the
    // normaliser needs no VALU adds and no exchange between lane groups
    __device__ static void pv_column(const Regs& r, const float (&p)[NMT][4], f32x4 (&o)[NVT],
                                     f32x4& lsum) {
        const bf16x8 b = as_bf16x8(u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                         pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])});
#pragma unroll
        for (int t = 0; t < NVT; ++t) o[t] = mfma_bf16(as_bf16x8(r.v[t]), b, o[t]);
        constexpr uint32_t kOne2 = 0x3F803F80u;              // two bf16 1.0
        lsum = mfma_bf16(as_bf16x8(u32x4{kOne2, kOne2, kOne2, kOne2}), b, lsum);
    }
};

// Online softmax of the staged prefill: NC 16-column query tiles per
// wavefront, scores folded into the exponent as exp2(s * c - mr) (c > 0).
//
// The reference mr of a column moves only when a score exceeds it by more
// than kRescaleSlack (log2 units); between moves the exponent offset -mr and
// the raw-score threshold thr = (mr + slack) / c are constants, so the common
// tile costs each lane one maximum over its own 8 scores and one compare,
// and a wave-wide ballot decides whether any column must move.  Only then is
// the column maximum formed across the four lane groups.  A move happens
// exactly when the tile holds a score above mr + slack, so that tile's
// maximum is the running maximum and becomes the new reference.  The row
// sums l are accumulated on the matrix core from the same bf16 probabilities
// the PV product uses.
template <int D, int NC> struct StagedSoftmax {
    using Ops = StagedOps<D>;
    static constexpr int NMT = Ops::NMT, NVT = Ops::NVT;
    float mr[NC], thr[NC], nref[NC];
    f32x4 o[NC][NVT];
    f32x4 lsum[NC];

    __device__ void init() {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            mr[n] = -INFINITY;
            thr[n] = -INFINITY;
            nref[n] = 0.f;
            lsum[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[n][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // move column n's reference to the tile maximum where it exceeds thr
    __device__ void bump(int n, float lmax, float c) {
        const float tmax = max_over_groups_nan(lmax);        // the column's tile maximum
        const bool move = tmax > thr[n];
        const float mr_new = move ? tmax * c : mr[n];
        // a column that has seen nothing yet (mr = -inf) scales by 0
        const float alpha = move ? fast_exp2(mr[n] - mr_new) : 1.0f;
        mr[n] = mr_new;
        thr[n] = move ? (mr_new + kRescaleSlack) / c : thr[n];
        nref[n] = mr_new == -INFINITY ? 0.f : -mr_new;
        lsum[n] *= alpha;
#pragma unroll
        for (int t = 0; t < NVT; ++t) o[n][t] *= alpha;
    }

    // One 32-position half for all NC query tiles.  vsrc: the half's staged
    // V; limit[n]: this lane's last visible position in query tile n
    // (relative to the half); nvalid: real tokens in the half; masked: some
    // position of some tile needs masking.  The V operand is read from LDS
    // once QK^T has consumed the K registers, which keeps the wavefront
    // within the register budget of two wavefronts per SIMD.  The reference
    // test of every tile comes first, so that from the exponentials on the
    // half is one branch-free stretch.  The PV products run at raised wave
    // priority, so that the other wavefront on the SIMD issues its VALU work
    // while they occupy the matrix core (about 1.5% faster in a same-box A/B).
    __device__ void step(typename Ops::Regs& r, const char* vsrc, const typename Ops::Q (&q)[NC],
                         float c, int nvalid, const int (&limit)[NC], bool masked, int lane) {
        const int grp = lane >> 4;
        f32x4 s4[NC][NMT];
        Ops::template qk<NC>(r, q, s4);
#pragma unroll
        for (int v = 0; v < NVT; ++v)
            r.v[v] = *reinterpret_cast<const u32x4*>(vsrc + ((v * 4 + grp) * 16 + (lane & 15)) * 16);
        // V of positions past the context may hold any bits (NaN included)
        if (masked && nvalid < 32) Ops::mask_v(r, nvalid, lane);
        float s[NC][NMT][4];
        float lmax[NC];
        bool over = false;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[n][i][e] = s4[n][i][e];
            if (masked) {
                // -inf: excluded from the maximum, and exp2(fma(-inf, c, .)) = 0
                const int lim = min(limit[n], nvalid - 1);
#pragma unroll
                for (int i = 0; i < NMT; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[n][i][e] = Ops::pos(i, e, grp) <= lim ? s[n][i][e] : -INFINITY;
            }
            lmax[n] = -INFINITY;
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) lmax[n] = fmax_nan(lmax[n], s[n][i][e]);
            over |= lmax[n] > thr[n];
        }
        if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
            for (int n = 0; n < NC; ++n) bump(n, lmax[n], c);
        }
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            float p[NMT][4];
#pragma unroll
            for (int i = 0; i < NMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) p[i][e] = fast_exp2(__builtin_fmaf(s[n][i][e], c, nref[n]));
            __builtin_amdgcn_s_setprio(1);
            Ops::pv_column(r, p, o[n], lsum[n]);
            __builtin_amdgcn_s_setprio(0);
        }
    }
};

// Launch order.  Workgroups are placed breadth-first over the CUs, so block b
// shares its CU with blocks b +- num_cus, and a CU's time is set by the sum of
// its workgroups' tiles.  Items (chunk, KV head, row group) are ranked by tile
// count, longest first (ties: KV head, chunk, row group), and pass p of
// num_cus blocks takes ranks p * num_cus .. in alternating direction: the
// longest items share a CU with the shortest (longest-processing-time order).
// Every (chunk, row group) class's count is held in registers, 64 per
// register: up to 64 * kOrderGroups classes, else the natural order.
//
// Blocks are dealt round-robin to the 8 XCDs (block b to XCD b % 8), each
// with its own L2.  When the KV heads divide by 8, XCD x takes every item of
// KV heads x, x + 8, ..., ranked the same way over its own blocks and CUs:
// all row groups of one (chunk, KV head) then read their K/V through one L2,
// and each XCD gets the same mix of item sizes.
constexpr int kOrderGroups = 8;

__device__ __forceinline__ int launch_rank(int b, int nblocks, int stride) {
    const int p = b / stride, pos = b - p * stride;
    const int m = min(stride, nblocks - p * stride);           // blocks in pass p
    return p * stride + ((p & 1) ? m - 1 - pos : pos);
}

// (chunk c, KV head h, row group tg) of the item at rank r among the items of
// KV heads h0 + hstep * j, j < nh; false: no work
__device__ bool item_at_rank(const PrefillArgs& a, int rows, int r, int lane, int h0, int hstep,
                             int nh, int& c, int& h, int& tg) {
    const int wpg = a.wg_per_head, ncls = a.num_chunks * wpg;
    int cost[kOrderGroups];                    // tiles of class 64 g + lane (0: no rows)
#pragma unroll
    for (int g = 0; g < kOrderGroups; ++g) {
        const int cls = 64 * g + lane;
        cost[g] = 0;
        if (cls < ncls) {
            const int cc = cls / wpg, t = cls - cc * wpg;
            const int q0 = a.query_start_loc[cc];
            const int C = a.query_start_loc[cc + 1] - q0;
            const int P = min(a.context_lens[cc], a.max_blocks_per_seq * kBlock) - C;
            if (P >= 0 && t * rows < C) {
                const int kend = P + min(C, rows * (t + 1));
                cost[g] = (kend - 1) / kLdsTile + 1;
            }
        }
    }
    const int ngroups = (ncls + 63) / 64;
    auto count_ge = [&](int x) {             // classes with at least x tiles
        int n = 0;
#pragma unroll
        for (int g = 0; g < kOrderGroups; ++g)
            if (g < ngroups) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(cost[g] >= x));
        return n;
    };
    const int H = nh;
    // the search below only needs the bits of the largest count
    int cmax = 0;
#pragma unroll
    for (int g = 0; g < kOrderGroups; ++g) cmax = max(cmax, cost[g]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cmax = max(cmax, __shfl_xor(cmax, off));
    cmax = __builtin_amdgcn_readfirstlane(cmax);
    if (cmax == 0) return false;
    // the item's tile count: the largest x with H * count_ge(x) > r
    int x = 0;
    for (int bit = 31 - __builtin_clz(cmax); bit >= 0; --bit) {
        const int cand = x | (1 << bit);
        if ((long)H * count_ge(cand) > r) x = cand;
    }
    if (x == 0) return false;
    const int above = count_ge(x + 1), ncl = count_ge(x) - above;
    const int j = r - H * above;               // among the H * ncl items with x tiles
    const int hh = j / ncl;
    h = h0 + hstep * hh;
    int k = j - hh * ncl;                      // the k-th class with x tiles, by index
    int cls = 0;
#pragma unroll
    for (int g = 0; g < kOrderGroups; ++g) {
        if (g >= ngroups) break;
        const uint64_t m = __builtin_amdgcn_ballot_w64(cost[g] == x);
        const int n = __builtin_popcountll(m);
        if (k < n) {
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const uint64_t hit = __builtin_amdgcn_ballot_w64(cost[g] == x && below == k);
            cls = 64 * g + __builtin_ctzll(hit);
            break;
        }
        k -= n;
    }
    c = cls / wpg;
    tg = cls - c * wpg;
    return true;
}

template <int KIND, int D, int NC>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_lds_kernel(PrefillArgs a) {
    using Ops = TileOps<kBF16, D>;            // staged operands are bf16 for both caches
    using SOps = StagedOps<D>;
    using QT = uint16_t;
    constexpr int NW = 4, NS = Ops::NS, NVT = Ops::NVT;
    constexpr int KB = kBlock * D * 2;        // one block's K (or V) in bf16
    constexpr int ELEM = KIND == kFP8 ? 1 : 2;
    constexpr int NLD = KIND == kFP8 ? D / 64 : D / 32;     // 16-byte loads per lane for K (and V)
    __shared__ __align__(16) char s_k[2][4 * KB];
    __shared__ __align__(16) char s_v[2][4 * KB];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wg_rows = NW * NC * a.npos;
    int c, h, tg;
    if (a.num_cus > 0 && a.num_chunks * a.wg_per_head <= 64 * kOrderGroups) {
        // every wavefront finds the same item (wave-uniform ballots)
        constexpr int kXcd = 8;
        const bool per_xcd = a.num_kv_heads % kXcd == 0 && a.num_cus % kXcd == 0;
        const int xcd = blockIdx.x % kXcd;
        const int rank = per_xcd ? launch_rank(blockIdx.x / kXcd, gridDim.x / kXcd, a.num_cus / kXcd)
                                 : launch_rank(blockIdx.x, gridDim.x, a.num_cus);
        if (!item_at_rank(a, wg_rows, rank, lane, per_xcd ? xcd : 0, per_xcd ? kXcd : 1,
                          per_xcd ? a.num_kv_heads / kXcd : a.num_kv_heads, c, h, tg))
            return;                                       // the whole workgroup
        c = __builtin_amdgcn_readfirstlane(c);
        h = __builtin_amdgcn_readfirstlane(h);
        tg = __builtin_amdgcn_readfirstlane(tg);
    } else {
        const int item = xcd_remap(blockIdx.x, gridDim.x);
        tg = item % a.wg_per_head;
        h = (item / a.wg_per_head) % a.num_kv_heads;
        c = item / (a.wg_per_head * a.num_kv_heads);
    }

    const int q0 = a.query_start_loc[c];
    const int C = a.query_start_loc[c + 1] - q0;
    // positions past the chunk's block-table row are never read
    const int L = min(a.context_lens[c], a.max_blocks_per_seq * kBlock);
    const int P = L - C;
    const int npos = a.npos;
    const int wg_row0 = tg * wg_rows;
    if (wg_row0 >= C || P < 0) return;                   // the whole workgroup leaves together
    const int kend = P + min(C, wg_row0 + wg_rows);      // keys [0, kend) are touched
    const int ntiles = (kend + kLdsTile - 1) / kLdsTile;
    const int last_blk = (kend - 1) / kBlock;

    // this wavefront's query columns
    const int row0 = wg_row0 + wave * NC * npos;
    const int wrows = max(0, min(NC * npos, C - row0));
    const int g = lane & 15, grp = lane >> 4;
    const int pi = g / a.group, gh = g % a.group;
    typename Ops::Q qop[NC];
    int my_last[NC];
    bool col_valid[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int r = n * npos + pi;
        col_valid[n] = pi < npos && r < wrows;
        const QT* qrow = reinterpret_cast<const QT*>(a.q) +
                         ((long)(q0 + row0 + (col_valid[n] ? r : 0)) * a.num_heads + h * a.group + gh) * D;
        Ops::load_q(qop[n], qrow, col_valid[n], lane);
        my_last[n] = P + row0 + (col_valid[n] ? r : 0);
    }
    const int w_kend = P + row0 + wrows;                 // keys this wavefront needs
    const int min_last = P + row0;
    float cs = a.scale_log2;
    if (KIND == kFP8) cs *= load_invariant(a.k_scale + h);
    // the folded softmax takes a positive multiplier: a negative one moves
    // its sign into Q; zero becomes the least normal float, with which every
    // exp2 argument rounds as with zero (scores far below 2^100)
    if (cs < 0.f) {
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
            for (int k = 0; k < NS; ++k)
                qop[n].op[k] = as_bf16x8(__builtin_bit_cast(u32x4, qop[n].op[k]) ^ 0x80008000u);
        cs = -cs;
    }
    cs = fmaxf(cs, FLT_MIN);

    const int32_t* bt = a.block_tables + (long)c * a.max_blocks_per_seq;
    const long head_stride = (long)kBlock * D * ELEM;
    const long blk_stride = head_stride * a.num_kv_heads;
    const char* kbase = a.k_cache + h * head_stride;
    const char* vbase = a.v_cache + h * head_stride;

    // ---- staging: wavefront w moves block w of tile t --------------------------
    u32x4 sk[NLD], sv[NLD];
    // physical ids of the blocks this wavefront stages, one tile per lane:
    // lane j holds block 4 (ids_t0 + j) + wave (clamped to the last), so no
    // memory latency sits between two tiles' loads
    int ids = 0, ids_t0 = 0;
    auto fetch_ids = [&](int t0) {
        ids_t0 = t0;
        ids = bt[min(4 * (t0 + lane) + wave, last_blk)];
    };
    fetch_ids(0);
    auto stage_load = [&](int t) {
        if (t - ids_t0 >= kWave) fetch_ids(t);
        const long phys = __builtin_amdgcn_readlane(ids, t - ids_t0);
        const char* kb = kbase + phys * blk_stride;
        const char* vb = vbase + phys * blk_stride;
        // ordinary (temporal) loads: the row groups of one (chunk, KV head)
        // run on one XCD and read the same blocks, so L2 should keep them
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            sk[u] = load16_cached(kb + 16 * (lane + kWave * u));
            sv[u] = load16_cached(vb + 16 * (lane + kWave * u));
        }
    };
    // token tok of the staged block: key 16 (wave & 1) + tok of half wave >> 1
    auto k_dst = [&](int buf, int chunk, int tok) {
        const int k = 16 * (wave & 1) + tok;
        return s_k[buf] + (wave >> 1) * (2 * KB) + SOps::tile_of(k) * KB +
               (chunk * 16 + SOps::row_of(k)) * 16;
    };
    auto stage_store = [&](int buf) {
        char* vd = s_v[buf] + (wave >> 1) * (2 * KB);
        const int run0 = (wave & 1) * 2;
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int piece = lane + kWave * u;
            if (KIND == kFP8) {
                // K piece = (16-dim chunk c16, token): two bf16 chunks (2 c16, 2 c16 + 1)
                const int c16 = piece >> 4, tok = piece & 15;
                const bf16x8 lo = fp8x8_to_bf16x8(sk[u][0], sk[u][1]);
                const bf16x8 hi = fp8x8_to_bf16x8(sk[u][2], sk[u][3]);
                *reinterpret_cast<bf16x8*>(k_dst(buf, 2 * c16, tok)) = lo;
                *reinterpret_cast<bf16x8*>(k_dst(buf, 2 * c16 + 1, tok)) = hi;
                // V piece = dim d, 16 tokens: runs run0 (tokens 0-7) and run0 + 1 (8-15)
                const int d = piece;
                const bf16x8 v0 = fp8x8_to_bf16x8(sv[u][0], sv[u][1]);
                const bf16x8 v1 = fp8x8_to_bf16x8(sv[u][2], sv[u][3]);
                const int t16 = d >> 4, dd = d & 15;
                *reinterpret_cast<bf16x8*>(vd + ((t16 * 4 + run0) * 16 + dd) * 16) = v0;
                *reinterpret_cast<bf16x8*>(vd + ((t16 * 4 + run0 + 1) * 16 + dd) * 16) = v1;
            } else {
                // K piece = (8-dim chunk, token); V piece = half of dim d's 32 bytes
                *reinterpret_cast<u32x4*>(k_dst(buf, piece >> 4, piece & 15)) = sk[u];
                const int d = piece >> 1, half = piece & 1;
                const int t16 = d >> 4, dd = d & 15;
                *reinterpret_cast<u32x4*>(vd + ((t16 * 4 + run0 + half) * 16 + dd) * 16) = sv[u];
            }
        }
    };

    StagedSoftmax<D, NC> st;
    st.init();
    auto compute = [&](int buf, int t) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int t0 = t * kLdsTile + hh * 32;
            if (t0 >= w_kend) continue;
            typename Ops::Regs r;
            const char* ks = s_k[buf] + 2 * hh * KB;
            const char* vs = s_v[buf] + hh * (2 * KB);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int k = 0; k < NS; ++k)
                    r.k[i][k] = *reinterpret_cast<const u32x4*>(ks + i * KB + ((4 * k + grp) * 16 + g) * 16);
            const int nvalid = min(kend - t0, 32);
            const bool masked = (t0 + 31 > min_last) || (nvalid < 32);
            int limit[NC];
#pragma unroll
            for (int n = 0; n < NC; ++n) limit[n] = my_last[n] - t0;
            st.step(r, vs, qop, cs, nvalid, limit, masked, lane);
        }
    };

    stage_load(0);
    stage_store(0);
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) stage_load(t + 1);
        __syncthreads();                       // tile t is in LDS; tile t-1's readers are done
        if (wrows > 0) compute(buf, t);
        if (t + 1 < ntiles) stage_store(buf ^ 1);
    }

    const float vsc = KIND == kFP8 ? load_invariant(a.v_scale + h) : 1.0f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float l = st.lsum[n][0];                   // against the reference mr
        if (!col_valid[n]) continue;
        const float inv = vsc / l;
        const long orow =
            ((long)(q0 + row0 + n * npos + pi) * a.num_heads + h * a.group + gh) * D;
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const int d = 16 * t + 4 * grp;
            const f32x4 v = st.o[n][t] * inv;
            u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow + d) = pk;
        }
    }
}

template <int KIND, int D, int NC>
static hipError_t launch_prefill_lds(PrefillArgs a, int num_chunks, int max_query_len,
                                     hipStream_t stream) {
    const int rows = 4 * NC * a.npos;
    a.wg_per_head = (max_query_len + rows - 1) / rows;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    a.num_cus = cus;                          // 0: the natural order
    const long grid = (long)num_chunks * a.num_kv_heads * a.wg_per_head;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_lds_kernel<KIND, D, NC>), dim3((unsigned)grid), dim3(4 * kWave),
                       0, stream, a);
    return hipGetLastError();
}

template <int KIND, int D>
static hipError_t launch_prefill(PrefillArgs a, int num_chunks, int max_query_len,
                                 hipStream_t stream) {
    constexpr int NW = 4, NC = prefill_tiles_per_wave(KIND, D);
    const int tiles = (max_query_len + a.npos - 1) / a.npos;
    const int waves = (tiles + NC - 1) / NC;
    a.wg_per_head = (waves + NW - 1) / NW;
    const long grid = (long)num_chunks * a.num_kv_heads * a.wg_per_head;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_kernel<KIND, D, NW, NC>), dim3((unsigned)grid), dim3(NW * kWave),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_prefill_chunk(void* out, const void* q, pa_dtype_t q_dtype,
                                        const int32_t* query_start_loc, int32_t num_chunks,
                                        int32_t max_query_len, const void* k_cache,
                                        const void* v_cache, pa_dtype_t cache_dtype,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        float scale, hipStream_t stream) {
    pa_status_t st = check_attention_shape(q_dtype, cache_dtype, k_scale, v_scale, num_heads,
                                           num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (num_chunks < 0 || max_query_len < 0 || max_blocks_per_seq < 1) return PA_ERR_ARG;
    if (num_chunks == 0 || max_query_len == 0) return PA_OK;
    if (!out || !q || !query_start_loc || !k_cache || !v_cache || !block_tables || !context_lens)
        return PA_ERR_ARG;
    if (!std::isfinite(scale)) return PA_ERR_ARG;
    PrefillArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start_loc = query_start_loc;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.npos = 16 / a.group;
    a.wg_per_head = 1;
    a.num_chunks = num_chunks;
    a.num_cus = 0;
    a.scale_log2 = scale * kLog2e;
    hipError_t e;
    const int kind = cache_kind(cache_dtype);
    if (kind == kBF16 && head_dim == 128) e = launch_prefill_lds<kBF16, 128, kLdsCols>(a, num_chunks, max_query_len, stream);
    else if (kind == kBF16 && head_dim == 64) e = launch_prefill_lds<kBF16, 64, kLdsCols>(a, num_chunks, max_query_len, stream);
    else if (kind == kFP8 && head_dim == 128) e = launch_prefill_lds<kFP8, 128, kLdsCols>(a, num_chunks, max_query_len, stream);
    else if (kind == kFP8 && head_dim == 64) e = launch_prefill_lds<kFP8, 64, kLdsCols>(a, num_chunks, max_query_len, stream);
    else if (kind == kF32 && head_dim == 128) e = launch_prefill<kF32, 128>(a, num_chunks, max_query_len, stream);
    else if (kind == kF32 && head_dim == 64) e = launch_prefill<kF32, 64>(a, num_chunks, max_query_len, stream);
    else return PA_ERR_UNSUPPORTED;
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
