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

// Items per KV head of a sequence of context length L.
__device__ __forceinline__ int items_of(const DecodeArgs& a, int L) {
    if (L <= 0) return 0;
    return a.split ? (L + a.partition_size - 1) / a.partition_size : 1;
}

template <int KIND, int D, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(waves_per_simd(KIND, D))))
void decode_kernel(DecodeArgs a) {
    using Ops = TileOps<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int TT = Ops::TT, TB = Ops::TB, NVT = Ops::NVT, ELEM = Ops::ELEM;
    constexpr int NT = NW * kWave;

    __shared__ int s_pre[kMaxDecodeBatch + 1];   // exclusive prefix of items per head
    __shared__ int s_len[kMaxDecodeBatch];       // context lengths
    __shared__ int s_scan[NT];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int B = a.batch;

    // ---- prefix of per-sequence item counts (each thread: a run of sequences)
    const int per = (B + NT - 1) / NT;
    const int bs0 = tid * per;
    int local = 0;
    for (int k = 0; k < per; ++k)
        if (bs0 + k < B) {
            const int L = a.context_lens[bs0 + k];
            s_len[bs0 + k] = L;
            local += items_of(a, L);
        }
    s_scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const int v = tid >= off ? s_scan[tid - off] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    {
        int run = s_scan[tid] - local;
        for (int k = 0; k < per; ++k)
            if (bs0 + k < B) {
                s_pre[bs0 + k] = run;
                run += items_of(a, s_len[bs0 + k]);
            }
        if (tid == 0) s_pre[B] = s_scan[NT - 1];
    }
    // single pass: sequences with L = 0 have no item; their rows are zeros
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

    // ---- this wavefront's item range -----------------------------------------
    const int Hkv = a.num_kv_heads;
    const long total = (long)Hkv * s_pre[B];
    const long W = (long)gridDim.x * NW;
    const long gw = (long)blockIdx.x * NW + wave;
    const long i0 = total * gw / W, i1 = total * (gw + 1) / W;
    if (i0 >= i1) return;
    const long nitems = i1 - i0;

    // first item: the sequence b with Hkv*pre[b] <= i0 < Hkv*pre[b+1]
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long)Hkv * s_pre[mid] <= i0) lo = mid; else hi = mid - 1;
    }

    const int g = lane & 15, grp = lane >> 4;
    const long head_stride = (long)kBlock * D * ELEM;              // one (block, head) tile
    const long blk_stride = head_stride * Hkv;

    // Item cursor: (b, h, p), items per head n of sequence b, token range [tb, te).
    struct Item {
        int b, h, p, n, tb, te, nt;
    };
    auto set_item = [&](Item& it, int b, int h, int p) {
        it.b = b;
        it.h = h;
        it.p = p;
        it.n = s_pre[b + 1] - s_pre[b];
        it.tb = p * a.partition_size;
        it.te = min(s_len[b], it.tb + a.partition_size);
        it.nt = (it.te - it.tb + TT - 1) / TT;
    };
    // only called while another item of this wavefront's range exists
    auto next_item = [&](Item& it) {
        int b = it.b, h = it.h, p = it.p + 1;
        if (p == it.n) {
            p = 0;
            if (++h == Hkv) {
                h = 0;
                do { ++b; } while (s_pre[b + 1] == s_pre[b]);    // skip L = 0 sequences
            }
        }
        set_item(it, b, h, p);
    };

    Item ci;   // item being computed
    {
        const long r = i0 - (long)Hkv * s_pre[lo];
        const int n = s_pre[lo + 1] - s_pre[lo];
        set_item(ci, lo, (int)(r / n), (int)(r % n));
    }
    Item li = ci;          // item of the tile being loaded (one tile ahead)
    int ln = 0;            // tile index within li
    long lcount = 1;       // items entered by the load cursor
    bool lvalid = true;

    // block ids of the load cursor's tile, fetched one tile ahead
    int phys[TB];
    auto fetch_ids = [&]() {
        const int32_t* bt = a.block_tables + (long)li.b * a.max_blocks_per_seq;
        const int lb = (li.tb + ln * TT) / kBlock;
        const int last = (li.te - 1) / kBlock;
#pragma unroll
        for (int j = 0; j < TB; ++j) phys[j] = bt[min(lb + j, last)];
    };
    auto issue = [&](typename Ops::Regs& r) {
        const long hoff = (long)li.h * head_stride;
        Ops::load(r, a.k_cache + hoff, a.v_cache + hoff, blk_stride, phys, lane);
    };
    auto advance_load = [&]() {
        if (++ln == li.nt) {
            ln = 0;
            if (lcount == nitems) {
                lvalid = false;
                return;
            }
            ++lcount;
            next_item(li);
        }
        fetch_ids();
    };

    // per-item compute state
    typename Ops::Q qop[1];
    float c = a.scale_log2;
    auto load_q = [&]() {
        const int hq = ci.h * a.group + g;
        const QT* qrow = reinterpret_cast<const QT*>(a.q) + ((long)ci.b * a.num_heads + hq) * D;
        Ops::load_q(qop[0], qrow, g < a.group, lane);
        c = a.scale_log2;
        if (KIND == kFP8) c *= a.k_scale[ci.h];
    };
    WaveSoftmax<KIND, D> st;
    st.init();
    int cn = 0;            // tile index within ci
    long ccount = 1;       // items entered by the compute cursor

    auto finish_item = [&]() {
        const float lt = sum_over_groups(st.l[0]);          // against the reference mr
        if (g < a.group) {
            const int hq = ci.h * a.group + g;
            const float vs = (KIND == kFP8) ? a.v_scale[ci.h] : 1.0f;
            const float inv = vs / lt;
            if (a.split) {
                const long pi = ((long)ci.b * a.num_heads + hq) * a.max_partitions + ci.p;
                float* po = a.part_out + pi * D;
#pragma unroll
                for (int t = 0; t < NVT; ++t)
                    *reinterpret_cast<f32x4*>(po + 16 * t + 4 * grp) = st.o[0][t] * inv;
                if (grp == 0) {
                    a.part_max[pi] = st.m[0] * kLn2;
                    a.part_sum[pi] = lt * fast_exp2(st.mr[0] - st.m[0]);   // against the true max
                }
            } else {
                const long oi = ((long)ci.b * a.num_heads + hq) * D;
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
    auto compute = [&](typename Ops::Regs& r) {
        const int nvalid = ci.te - (ci.tb + cn * TT);
        const int nolimit[1] = {TT};
        st.step(r, qop, c, nvalid, nolimit, nvalid < TT, lane);
        if (++cn == ci.nt) {
            finish_item();
            cn = 0;
            if (ccount < nitems) {
                ++ccount;
                const int ob = ci.b, oh = ci.h;
                next_item(ci);
                st.init();
                if (ci.b != ob || ci.h != oh) load_q();
            }
        }
    };

    load_q();
    fetch_ids();
    typename Ops::Regs ra, rb;
    issue(ra);
    advance_load();
    while (true) {
        if (lvalid) {
            issue(rb);
            advance_load();
            compute(ra);
        } else {
            compute(ra);
            break;
        }
        if (lvalid) {
            issue(ra);
            advance_load();
            compute(rb);
        } else {
            compute(rb);
            break;
        }
    }
}

template <int KIND, int D>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    constexpr int NW = 4;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // every workgroup resident at once: CUs x (waves per SIMD) workgroups of 4 waves
    const long max_items = (long)a.batch * a.num_kv_heads * a.max_partitions;
    long grid = (long)cus * waves_per_simd(KIND, D);
    grid = std::min(grid, (max_items + NW - 1) / NW);
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
