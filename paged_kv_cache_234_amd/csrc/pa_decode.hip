// Paged decode attention for gfx950: persistent wave streaming.
//
// Operation: grouped-query softmax(scale * q K^T) V for one query token per
// sequence, over a paged cache (infer-lab: technique table, PagedAttention
// row; layout section, GQA; tiled online-softmax attention; llm-infer, "What
// It Does": a paged KV cache with block tables; the tiling follows the
// FlashAttention-2 reference llm-infer cites).  With partition_size > 0 the
// context is cut into fixed partitions whose softmax partials (m, l, o) are
// merged by pa_decode_splitk_reduce (flash-decoding split-K).
//
// Work decomposition.  A work item is (sequence b, KV head h, partition p):
// partition_size tokens of one sequence for the whole GQA group of one KV head
// (G <= 16 query heads form one 16-column MFMA operand, so every K/V byte is
// read once).  Without split the item is the whole context.  Items are ordered
// b, h, p and numbered densely (sequences with L = 0 have none); each
// workgroup first builds the prefix of per-sequence item counts in LDS.  The
// grid is sized to be resident at once, and wavefront w takes the contiguous
// item range [I*w/W, I*(w+1)/W).  A wavefront streams the tiles of its items
// back to back: the next tile's K/V loads -- across item boundaries too --
// are in flight while the current tile is multiplied, and each finished item
// writes its partial (or its output) straight from registers.
#include <algorithm>

#include "pa_internal.hpp"
#include "pa_tiles.hpp"

namespace pa {

constexpr int kMaxDecodeBatch = 4096;

struct DecodeArgs {
    void* out;
    const void* q;
    const char* k_cache;
    const char* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* part_max;
    float* part_sum;
    float* part_out;
    int max_blocks_per_seq;
    int batch;
    int num_heads;
    int num_kv_heads;
    int group;             // G
    int partition_size;    // tokens per item (split), or the whole table row (single pass)
    int max_partitions;    // slots per (sequence, query head) in the partial buffers
    int split;             // write partials instead of out
    float scale_log2;      // scale * log2(e)
};

template <int KIND> struct QType { using T = uint16_t; };
template <> struct QType<kF32> { using T = float; };

// Partitions (items) per KV head of a sequence of context length L.
__device__ __forceinline__ int items_of(const DecodeArgs& a, int L) {
    if (L <= 0) return 0;
    return a.split ? (L + a.partition_size - 1) / a.partition_size : 1;
}

// Tiles per KV head of a sequence: full items hold tpi tiles, the last one
// the tiles its remaining positions need.
__device__ __forceinline__ int tiles_of(const DecodeArgs& a, int L, int tt, int tpi) {
    const int n = items_of(a, L);
    if (n == 0) return 0;
    return (n - 1) * tpi + (L - (n - 1) * a.partition_size + tt - 1) / tt;
}

// Online-softmax state of one wavefront's piece of an item, parked in LDS
// until the wavefront owning the item's first tile merges it.
template <int NVT> struct SegSlot {
    f32x4 o[NVT][kWave];
    float m[kWave], mr[kWave], l[kWave];
};

template <int KIND, int D, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(waves_per_simd(KIND, D))))
void decode_kernel(DecodeArgs a) {
    using Ops = TileOps<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int TT = Ops::TT, TB = Ops::TB, NVT = Ops::NVT, ELEM = Ops::ELEM;
    constexpr int NT = NW * kWave;

    __shared__ int s_len[kMaxDecodeBatch];       // context lengths
    __shared__ int s_tpre[kMaxDecodeBatch + 1];  // exclusive prefix of tiles per KV head
    __shared__ int s_wsum[NW];
    __shared__ SegSlot<NVT> s_seg[NW][2];        // [wave][0: first piece, 1: last piece]

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int B = a.batch;
    const int tpi = (a.partition_size + TT - 1) / TT;     // tiles of a full item

    // ---- prefix of per-sequence tile counts (each thread: a run of sequences)
    const int per = (B + NT - 1) / NT;
    const int bs0 = tid * per;
    int local = 0;
    for (int k = 0; k < per; ++k)
        if (bs0 + k < B) {
            const int L = a.context_lens[bs0 + k];
            s_len[bs0 + k] = L;
            local += tiles_of(a, L, TT, tpi);
        }
    int incl = local;                                     // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int wbase = 0, total_tiles = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wbase += (w < wave) ? s_wsum[w] : 0;
        total_tiles += s_wsum[w];
    }
    {
        int run = wbase + incl - local;
        for (int k = 0; k < per; ++k)
            if (bs0 + k < B) {
                s_tpre[bs0 + k] = run;
                run += tiles_of(a, s_len[bs0 + k], TT, tpi);
            }
        if (tid == 0) s_tpre[B] = total_tiles;
    }
    // single pass: sequences with L = 0 have no tile; their rows are zeros
    if (!a.split) {
        const long rows = (long)B * a.num_heads * D;
        for (long r = (long)blockIdx.x * NT + tid; r < rows; r += (long)gridDim.x * NT) {
            if (a.context_lens[r / ((long)a.num_heads * D)] <= 0) {
                if (KIND == kF32) reinterpret_cast<float*>(a.out)[r] = 0.f;
                else reinterpret_cast<uint16_t*>(a.out)[r] = 0;
            }
        }
    }
    __syncthreads();

    // ---- tile ranges ----------------------------------------------------------
    // Tiles are numbered b-major, then KV head, then position.  Workgroup k
    // takes the items whose first tile lies in [T k / NWG, T (k+1) / NWG): a
    // range of whole items of about T / NWG tiles.  Its NW wavefronts split
    // that range into NW equal runs of tiles, cutting items where they must.
    const int Hkv = a.num_kv_heads;
    const long T = (long)Hkv * total_tiles;

    // sequence b with Hkv*tpre[b] <= g < Hkv*tpre[b+1] (g < T): the largest
    // such b, searched 64 candidates at a time (two LDS round trips for 4096
    // sequences).  tpre is nondecreasing, so the lanes whose candidate
    // qualifies form a prefix of the wave.
    auto seq_of = [&](long g) {
        int lo = 0, span = B;
        while (span > 1) {
            const int stride = (span + kWave - 1) / kWave;
            const int idx = lo + lane * stride;
            const bool ok = idx < lo + span && (long)Hkv * s_tpre[idx] <= g;
            const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok));
            const int end = lo + span;
            lo += (cnt - 1) * stride;
            span = min(stride, end - lo);
        }
        return lo;
    };
    // first tile of the first item starting at or after tile g
    auto item_start_at_or_after = [&](long g) -> long {
        if (g >= T) return T;
        const int b = seq_of(g);
        const int tb = s_tpre[b + 1] - s_tpre[b];
        const long base = (long)Hkv * s_tpre[b];
        const int h = (int)((g - base) / tb);
        const int j = (int)(g - base - (long)h * tb);
        const int p = (j + tpi - 1) / tpi;
        if (p < items_of(a, s_len[b])) return base + (long)h * tb + (long)p * tpi;
        return base + (long)(h + 1) * tb;
    };
    const long nwg = gridDim.x;
    const long wg_a = item_start_at_or_after(T * (long)blockIdx.x / nwg);
    const long wg_e = item_start_at_or_after(T * ((long)blockIdx.x + 1) / nwg);
    auto wave_start = [&](int w) { return wg_a + (wg_e - wg_a) * w / NW; };
    const long g0 = wave_start(wave), g1 = wave_start(wave + 1);
    const int ntiles = (int)(g1 - g0);

    const int g = lane & 15, grp = lane >> 4;
    const long head_stride = (long)kBlock * D * ELEM;              // one (block, head) tile
    const long blk_stride = head_stride * Hkv;

    // Tile cursor: sequence b, KV head h, item p, tile jj of the item; the
    // item covers positions [tb, te) in nti tiles; t0 is its first tile's
    // global number.
    struct Cursor {
        int b, h, p, jj, n, tb, te, nti;
        long t0;
    };
    auto set_item = [&](Cursor& c, int b, int h, int p, long t0) {
        c.b = b;
        c.h = h;
        c.p = p;
        c.n = items_of(a, s_len[b]);
        c.tb = p * a.partition_size;
        c.te = min(s_len[b], c.tb + a.partition_size);
        c.nti = (c.te - c.tb + TT - 1) / TT;
        c.t0 = t0;
    };
    // only called while another tile of this wavefront's run exists
    auto advance = [&](Cursor& c) {
        if (++c.jj < c.nti) return;
        const long t0 = c.t0 + c.nti;
        int b = c.b, h = c.h, p = c.p + 1;
        if (p == c.n) {
            p = 0;
            if (++h == Hkv) {
                h = 0;
                do { ++b; } while (s_tpre[b + 1] == s_tpre[b]);    // skip L = 0 sequences
            }
        }
        c.jj = 0;
        set_item(c, b, h, p, t0);
    };

    Cursor cc;          // tile being computed
    if (ntiles > 0) {
        const int b = seq_of(g0);
        const int tb = s_tpre[b + 1] - s_tpre[b];
        const long base = (long)Hkv * s_tpre[b];
        const int h = (int)((g0 - base) / tb);
        const int j = (int)(g0 - base - (long)h * tb);
        const int p = j / tpi;
        set_item(cc, b, h, p, base + (long)h * tb + (long)p * tpi);
        cc.jj = j - p * tpi;
    }
    bool tail_open = false;       // this wave's last piece ends inside its item
    Cursor tail_item;

    WaveSoftmax<KIND, D> st;
    typename Ops::Q qop[1];
    float c = a.scale_log2;
    auto load_q = [&]() {
        const int hq = cc.h * a.group + g;
        const QT* qrow = reinterpret_cast<const QT*>(a.q) + ((long)cc.b * a.num_heads + hq) * D;
        Ops::load_q(qop[0], qrow, g < a.group, lane);
        c = a.scale_log2;
        if (KIND == kFP8) c *= a.k_scale[cc.h];
    };

    // write an item's result from st: a split-K partial, or the output rows
    auto finish_item = [&](const Cursor& it) {
        const float lt = sum_over_groups(st.l[0]);          // against the reference mr
        if (g < a.group) {
            const int hq = it.h * a.group + g;
            const float vs = (KIND == kFP8) ? a.v_scale[it.h] : 1.0f;
            const float inv = vs / lt;
            if (a.split) {
                const long pi = ((long)it.b * a.num_heads + hq) * a.max_partitions + it.p;
                float* po = a.part_out + pi * D;
#pragma unroll
                for (int t = 0; t < NVT; ++t)
                    *reinterpret_cast<f32x4*>(po + 16 * t + 4 * grp) = st.o[0][t] * inv;
                if (grp == 0) {
                    a.part_max[pi] = st.m[0] * kLn2;
                    a.part_sum[pi] = lt * fast_exp2(st.mr[0] - st.m[0]);   // against the true max
                }
            } else {
                const long oi = ((long)it.b * a.num_heads + hq) * D;
#pragma unroll
                for (int t = 0; t < NVT; ++t) {
                    const f32x4 v = st.o[0][t] * inv;
                    const int d = 16 * t + 4 * grp;
                    if (KIND == kF32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + oi + d) = v;
                    } else {
                        u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + oi + d) = pk;
                    }
                }
            }
        }
    };
    auto park = [&](SegSlot<NVT>& s) {
#pragma unroll
        for (int t = 0; t < NVT; ++t) s.o[t][lane] = st.o[0][t];
        s.m[lane] = st.m[0];
        s.mr[lane] = st.mr[0];
        s.l[lane] = st.l[0];
    };

    if (ntiles > 0) {
        Cursor lc = cc;     // tile being loaded (one ahead)
        int nloaded = 0;
        int phys[TB];
        auto fetch_ids = [&]() {
            const int32_t* bt = a.block_tables + (long)lc.b * a.max_blocks_per_seq;
            const int lb = (lc.tb + lc.jj * TT) / kBlock;
            const int last = (lc.te - 1) / kBlock;
#pragma unroll
            for (int j = 0; j < TB; ++j) phys[j] = bt[min(lb + j, last)];
        };
        auto issue = [&](typename Ops::Regs& r) {
            const long hoff = (long)lc.h * head_stride;
            Ops::load(r, a.k_cache + hoff, a.v_cache + hoff, blk_stride, phys, lane);
            if (++nloaded < ntiles) {
                advance(lc);
                fetch_ids();
            }
        };
        int ncomputed = 0;
        bool piece_from_start = cc.jj == 0;
        auto compute = [&](typename Ops::Regs& r) {
            const int nvalid = cc.te - (cc.tb + cc.jj * TT);
            const int nolimit[1] = {TT};
            st.step(r, qop, c, nvalid, nolimit, nvalid < TT, lane);
            ++ncomputed;
            const bool item_done = cc.jj + 1 == cc.nti;
            const bool run_done = ncomputed == ntiles;
            if (item_done || run_done) {
                if (piece_from_start && item_done) {
                    finish_item(cc);
                } else if (!piece_from_start) {
                    park(s_seg[wave][0]);           // continues an item of the previous wave
                } else {
                    tail_open = true;               // continued by the next wave(s)
                    tail_item = cc;
                }
                if (!run_done) {
                    const int ob = cc.b, oh = cc.h;
                    advance(cc);
                    piece_from_start = true;
                    if (!tail_open) st.init();
                    if (cc.b != ob || cc.h != oh) load_q();
                }
            } else {
                advance(cc);
            }
        };

        st.init();
        load_q();
        fetch_ids();
        typename Ops::Regs ra, rb;
        issue(ra);
        while (true) {
            if (nloaded < ntiles) {
                issue(rb);
                compute(ra);
            } else {
                compute(ra);
                break;
            }
            if (nloaded < ntiles) {
                issue(ra);
                compute(rb);
            } else {
                compute(rb);
                break;
            }
        }
    }

    // ---- merge items cut between wavefronts --------------------------------
    __syncthreads();
    if (tail_open) {
        const long item_end = tail_item.t0 + tail_item.nti;
        for (int w = wave + 1; w < NW; ++w) {
            const long s0 = wave_start(w), s1 = wave_start(w + 1);
            if (s0 >= item_end) break;
            if (s1 == s0) continue;
            const SegSlot<NVT>& s = s_seg[w][0];
            const float mr2 = s.mr[lane];
            const float mnew = fmaxf(st.mr[0], mr2);
            const float a1 = st.mr[0] == mnew ? 1.f : fast_exp2(st.mr[0] - mnew);
            const float a2 = mr2 == mnew ? 1.f : fast_exp2(mr2 - mnew);
            st.mr[0] = mnew;
            st.m[0] = fmaxf(st.m[0], s.m[lane]);
            st.l[0] = st.l[0] * a1 + s.l[lane] * a2;
#pragma unroll
            for (int t = 0; t < NVT; ++t) st.o[0][t] = st.o[0][t] * a1 + s.o[t][lane] * a2;
        }
        finish_item(tail_item);
    }
}

template <int KIND, int D>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    constexpr int NW = 4;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // every workgroup resident at once: CUs x (waves per SIMD) workgroups of 4 waves
    const long tpi = (a.partition_size + TileOps<KIND, D>::TT - 1) / TileOps<KIND, D>::TT;
    const long max_tiles = (long)a.batch * a.num_kv_heads * a.max_partitions * tpi;
    long grid = (long)cus * waves_per_simd(KIND, D);
    grid = std::min(grid, (max_tiles + NW - 1) / NW);
    grid = std::max(grid, 1L);
    hipLaunchKernelGGL((decode_kernel<KIND, D, NW>), dim3((unsigned)grid), dim3(NW * kWave), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_decode(void* out, const void* q, pa_dtype_t q_dtype, const void* k_cache,
                                 const void* v_cache, pa_dtype_t cache_dtype, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, float scale,
                                 int32_t partition_size, int32_t max_partitions, float* part_max,
                                 float* part_sum, float* part_out, hipStream_t stream) {
    pa_status_t st = check_attention_shape(q_dtype, cache_dtype, k_scale, v_scale, num_heads,
                                           num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (batch < 0 || max_blocks_per_seq < 1 || partition_size < 0) return PA_ERR_ARG;
    if (batch == 0) return PA_OK;
    if (batch > kMaxDecodeBatch) return PA_ERR_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_ARG;
    if (!std::isfinite(scale)) return PA_ERR_ARG;
    DecodeArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.part_max = part_max;
    a.part_sum = part_sum;
    a.part_out = part_out;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.batch = batch;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.scale_log2 = scale * kLog2e;
    if (partition_size > 0) {
        if (partition_size % block_size) return PA_ERR_ARG;
        if (max_partitions < 1) return PA_ERR_ARG;
        if (!part_max || !part_sum || !part_out) return PA_ERR_ARG;
        a.partition_size = partition_size;
        a.max_partitions = max_partitions;
        a.split = 1;
    } else {
        if (!out) return PA_ERR_ARG;
        // one item covers every position a block-table row can address
        a.partition_size = max_blocks_per_seq * block_size;
        a.max_partitions = 1;
        a.split = 0;
    }
    hipError_t e = hipSuccess;
    const int kind = cache_kind(cache_dtype);
    if (kind == kBF16 && head_dim == 128) e = launch_decode<kBF16, 128>(a, stream);
    else if (kind == kBF16 && head_dim == 64) e = launch_decode<kBF16, 64>(a, stream);
    else if (kind == kFP8 && head_dim == 128) e = launch_decode<kFP8, 128>(a, stream);
    else if (kind == kFP8 && head_dim == 64) e = launch_decode<kFP8, 64>(a, stream);
    else if (kind == kF32 && head_dim == 128) e = launch_decode<kF32, 128>(a, stream);
    else if (kind == kF32 && head_dim == 64) e = launch_decode<kF32, 64>(a, stream);
    else return PA_ERR_UNSUPPORTED;
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
