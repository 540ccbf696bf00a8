// Paged decode attention for gfx950.
//
// One workgroup of NW wavefronts per (sequence, KV head, partition).  The
// whole GQA group of that KV head (G <= 16 query heads) is one 16-column MFMA
// operand, so every K/V byte is read once per workgroup.  The partition's
// 16-token blocks are split into contiguous runs of whole tiles, one run per
// wavefront; each wavefront streams its tiles with the next tile's loads in
// flight while the current tile is multiplied, keeps its own online-softmax
// state (running max m, sum l, O^T accumulator), and the NW states are merged
// through LDS at the end.  With partition_size > 0 the merged state is the
// partition's (m, l, o) for the split-K reduce; otherwise it is the output.
//
// Operation: grouped-query softmax(scale * q K^T) V over a paged cache
// (infer-lab: technique table "PagedAttention", layout section "GQA", tiled
// online-softmax attention; llm-infer: "What It Does", paged KV cache with
// block tables; FlashAttention-2 tiling per llm-infer's references).
#include "pa_internal.hpp"
#include "pa_tiles.hpp"

namespace pa {

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
    int num_heads;
    int num_kv_heads;
    int group;             // G
    int partition_size;    // tokens; the whole context when not split
    int max_partitions;    // 1 when not split
    int split;             // write partials instead of out
    float scale_log2;      // scale * log2(e)
};

template <int KIND> struct QType { using T = uint16_t; };
template <> struct QType<kF32> { using T = float; };

template <int KIND, int D, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(DecodeArgs a) {
    using Ops = TileOps<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int TT = Ops::TT, TB = Ops::TB, NVT = Ops::NVT;
    constexpr int ELEM = Ops::ELEM;

    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ float s_o[NW][D][17];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int p = item % a.max_partitions;
    const int h = (item / a.max_partitions) % a.num_kv_heads;
    const int b = item / (a.max_partitions * a.num_kv_heads);

    const int L = a.context_lens[b];
    const int t_begin = p * a.partition_size;
    if (L > 0 && t_begin >= L) return;                  // empty partition
    if (L == 0 && (a.split || p > 0)) return;           // reduce writes the zeros
    const int t_end = min(L, t_begin + a.partition_size);

    // ---- this wavefront's run of tiles --------------------------------------
    const int ntiles = (t_end - t_begin + TT - 1) / TT;
    const int n0 = (int)(((long)ntiles * wave) / NW);
    const int n1 = (int)(((long)ntiles * (wave + 1)) / NW);
    const int last_blk = (t_end - 1) / kBlock;          // last logical block in range
    const int32_t* bt = a.block_tables + (long)b * a.max_blocks_per_seq;

    const int g = lane & 15, grp = lane >> 4;
    const int hq = h * a.group + g;
    const QT* qrow = reinterpret_cast<const QT*>(a.q) + ((long)b * a.num_heads + hq) * D;
    typename Ops::Q qop;
    Ops::load_q(qop, qrow, g < a.group, lane);

    float c = a.scale_log2;
    if (KIND == kFP8) c *= a.k_scale[h];

    const long head_stride = (long)kBlock * D * ELEM;              // one (block, head) tile
    const long blk_stride = head_stride * a.num_kv_heads;
    const char* kbase = a.k_cache + h * head_stride;
    const char* vbase = a.v_cache + h * head_stride;
    const int kb = Ops::k_block(lane), vb = Ops::v_block(lane);

    auto issue = [&](typename Ops::Regs& r, int n) {
        const int lb = (t_begin + n * TT) / kBlock;
        int phys[TB];
#pragma unroll
        for (int j = 0; j < TB; ++j) phys[j] = bt[min(lb + j, last_blk)];
        int pk = phys[0], pv = phys[0];
#pragma unroll
        for (int j = 1; j < TB; ++j) {
            pk = (kb == j) ? phys[j] : pk;
            pv = (vb == j) ? phys[j] : pv;
        }
        Ops::load(r, kbase + (long)pk * blk_stride, vbase + (long)pv * blk_stride, lane);
    };

    WaveSoftmax<KIND, D> st;
    st.init();
    auto compute = [&](typename Ops::Regs& r, int n) {
        const int nvalid = t_end - (t_begin + n * TT);
        st.step(r, qop, c, nvalid, TT, nvalid < TT, lane);
    };

    if (n0 < n1) {
        typename Ops::Regs ra, rb;
        issue(ra, n0);
        for (int n = n0; n < n1; n += 2) {
            if (n + 1 < n1) issue(rb, n + 1);
            compute(ra, n);
            if (n + 1 >= n1) break;
            if (n + 2 < n1) issue(ra, n + 2);
            compute(rb, n + 1);
        }
    }
    float m_run = st.m, l_run = st.l;
    f32x4 (&o)[NVT] = st.o;

    // ---- merge the NW wavefront states -------------------------------------
    l_run = sum_over_groups(l_run);
    if (grp == 0) {
        s_m[wave][g] = m_run;
        s_l[wave][g] = l_run;
    }
#pragma unroll
    for (int t = 0; t < NVT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][16 * t + 4 * grp + i][g] = o[t][i];
    __syncthreads();

    const float vs = (KIND == kFP8) ? a.v_scale[h] : 1.0f;
    for (int idx = threadIdx.x; idx < a.group * D; idx += NW * kWave) {
        const int gg = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][gg]);
        float lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(s_m[w][gg] - M);     // 0 for an idle wave (m = -inf)
            lsum += f * s_l[w][gg];
            acc += f * s_o[w][d][gg];
        }
        const int qh = h * a.group + gg;
        const float val = (L > 0) ? acc / lsum * vs : 0.f;
        if (a.split) {
            const long pi = ((long)b * a.num_heads + qh) * a.max_partitions + p;
            a.part_out[pi * D + d] = val;
            if (d == 0) {
                a.part_max[pi] = M * kLn2;
                a.part_sum[pi] = lsum;
            }
        } else {
            const long oi = ((long)b * a.num_heads + qh) * D + d;
            if (KIND == kF32)
                reinterpret_cast<float*>(a.out)[oi] = val;
            else
                reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(val);
        }
    }
}

template <int KIND, int D>
static hipError_t launch_decode(const DecodeArgs& a, int batch, hipStream_t stream) {
    constexpr int NW = 4;
    const long grid = (long)batch * a.num_kv_heads * a.max_partitions;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
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
        // one pass covers every position a block-table row can address
        a.partition_size = max_blocks_per_seq * block_size;
        a.max_partitions = 1;
        a.split = 0;
    }
    hipError_t e = hipSuccess;
    const int kind = cache_kind(cache_dtype);
    if (kind == kBF16 && head_dim == 128) e = launch_decode<kBF16, 128>(a, batch, stream);
    else if (kind == kBF16 && head_dim == 64) e = launch_decode<kBF16, 64>(a, batch, stream);
    else if (kind == kFP8 && head_dim == 128) e = launch_decode<kFP8, 128>(a, batch, stream);
    else if (kind == kFP8 && head_dim == 64) e = launch_decode<kFP8, 64>(a, batch, stream);
    else if (kind == kF32 && head_dim == 128) e = launch_decode<kF32, 128>(a, batch, stream);
    else if (kind == kF32 && head_dim == 64) e = launch_decode<kF32, 64>(a, batch, stream);
    else return PA_ERR_UNSUPPORTED;
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
