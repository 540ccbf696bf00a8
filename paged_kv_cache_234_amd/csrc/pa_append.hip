// KV append: scatter this step's new K/V rows into their pool slots.
//
// llm-infer ("What It Does") captures the KV write next to attention in the
// per-layer decode graph; InferX ("The kernels underneath", FP8 KV cache
// paragraph) writes the cache as fp8 e4m3 with per-layer K/V scales frozen
// at warm-up.  Here the scale is one fp32 value per KV head (K and V apart).
//
// One thread moves 8 consecutive head_dim elements of one (token, head)
// (write_token_chunk in pa_write.hpp: layouts and fp8 encoding).  Lanes run
// over 16 consecutive tokens first: V is stored token-minor (a block's 16
// tokens of one dimension are adjacent), so the V stores of one instruction
// for tokens that fill consecutive slots fall into one 16-byte row -- one
// memory request instead of sixteen.  Then over 4 chunks of the same tokens.
#include "pa_internal.hpp"
#include "pa_write.hpp"

namespace pa {

template <int IN, int CACHE, int D>
__global__ __launch_bounds__(256) void append_kernel(const void* __restrict__ k_new,
                                                     const void* __restrict__ v_new,
                                                     char* __restrict__ k_cache,
                                                     char* __restrict__ v_cache,
                                                     const float* __restrict__ k_scale,
                                                     const float* __restrict__ v_scale,
                                                     const int32_t* __restrict__ slots,
                                                     int num_tokens, int num_kv_heads) {
    constexpr int CH = D / 8;                         // 8-element chunks per row
    constexpr int IB = (IN == kF32) ? 4 : 2;          // input element bytes
    // idx = ((token group * heads + h) * CH / 4 + chunk group) * 64 + 16 c_lo + t_lo
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = (int)(idx & 63);
    const long rest = idx >> 6;
    const int cg = (int)(rest % (CH / 4));
    const int h = (int)((rest / (CH / 4)) % num_kv_heads);
    const long tg = rest / ((long)(CH / 4) * num_kv_heads);
    const long t = tg * 16 + (lane & 15);
    const int c = cg * 4 + (lane >> 4);
    if (t >= num_tokens) return;
    // the row, the slot and the scales go out together: one memory round
    // trip before the stores instead of two (slot, then row)
    const long row = (t * num_kv_heads + h) * D * IB;
    const TokenChunk<CACHE> tok = load_token_chunk<CACHE, D>(static_cast<const char*>(k_new) + row,
                                                             static_cast<const char*>(v_new) + row, c);
    int slot = slots[t];
    const float ksc = CACHE == kFP8 ? k_scale[h] : 1.0f;
    const float vsc = CACHE == kFP8 ? v_scale[h] : 1.0f;
    // The slot is tested only after every load has been issued: the empty
    // asm takes the row and the scales and hands the slot on, so the test
    // cannot be scheduled between the loads (left to itself the compiler
    // tests the slot first and sinks the row loads below the test, after
    // the slot's round trip).
    asm volatile("" : "+v"(slot) : "v"(tok.k[0]), "v"(tok.v[0]), "v"(tok.k[tok.N - 1]),
                 "v"(tok.v[tok.N - 1]), "v"(ksc), "v"(vsc));
    if (slot < 0) return;
    store_token_chunk<CACHE, D>(tok, k_cache, v_cache, slot / kBlock, slot % kBlock, h,
                                num_kv_heads, c, ksc, vsc);
}

template <int IN, int CACHE, int D>
static hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                const float* k_scale, const float* v_scale, const int32_t* slots,
                                int num_tokens, int num_kv_heads, hipStream_t stream) {
    const long total = (long)((num_tokens + 15) / 16) * 16 * num_kv_heads * (D / 8);
    const long blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((append_kernel<IN, CACHE, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       k_new, v_new, static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                       k_scale, v_scale, slots, num_tokens, num_kv_heads);
    return hipGetLastError();
}

}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_kv_append(const void* k_new, const void* v_new, pa_dtype_t in_dtype,
                                    void* k_cache, void* v_cache, pa_dtype_t cache_dtype,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, hipStream_t stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(cache_dtype)) return PA_ERR_ARG;
    if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_ARG;
    if (!supported_pair(in_dtype, cache_dtype)) return PA_ERR_UNSUPPORTED;
    if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_ARG;
    if (cache_dtype == PA_DT_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_ARG;
    hipError_t e;
    const int kind = cache_kind(cache_dtype);
#define PA_APPEND(IN, CK, DD)                                                                    \
    e = launch_append<IN, CK, DD>(k_new, v_new, k_cache, v_cache, k_scale, v_scale, slot_mapping, \
                                  num_tokens, num_kv_heads, stream)
    if (kind == kF32) {
        if (head_dim == 128) PA_APPEND(kF32, kF32, 128); else PA_APPEND(kF32, kF32, 64);
    } else if (kind == kBF16) {
        if (head_dim == 128) PA_APPEND(kBF16, kBF16, 128); else PA_APPEND(kBF16, kBF16, 64);
    } else {
        if (head_dim == 128) PA_APPEND(kBF16, kFP8, 128); else PA_APPEND(kBF16, kFP8, 64);
    }
#undef PA_APPEND
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
