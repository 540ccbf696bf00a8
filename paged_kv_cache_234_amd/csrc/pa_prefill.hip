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
    const int L = a.context_lens[c];
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
    a.scale_log2 = scale * kLog2e;
    hipError_t e;
    const int kind = cache_kind(cache_dtype);
    if (kind == kBF16 && head_dim == 128) e = launch_prefill<kBF16, 128>(a, num_chunks, max_query_len, stream);
    else if (kind == kBF16 && head_dim == 64) e = launch_prefill<kBF16, 64>(a, num_chunks, max_query_len, stream);
    else if (kind == kFP8 && head_dim == 128) e = launch_prefill<kFP8, 128>(a, num_chunks, max_query_len, stream);
    else if (kind == kFP8 && head_dim == 64) e = launch_prefill<kFP8, 64>(a, num_chunks, max_query_len, stream);
    else if (kind == kF32 && head_dim == 128) e = launch_prefill<kF32, 128>(a, num_chunks, max_query_len, stream);
    else if (kind == kF32 && head_dim == 64) e = launch_prefill<kF32, 64>(a, num_chunks, max_query_len, stream);
    else return PA_ERR_UNSUPPORTED;
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
