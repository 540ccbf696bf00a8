// KV append: scatter this step's new K/V rows into their pool slots.
//
// llm-infer ("What It Does") captures the KV write next to attention in the
// per-layer decode graph; InferX ("The kernels underneath", FP8 KV cache
// paragraph) writes the cache as fp8 e4m3 with per-layer K/V scales frozen
// at warm-up.  Here the scale is one fp32 value per KV head (K and V apart).
//
// One thread moves 8 consecutive head_dim elements of one (token, head):
// a 16-byte (bf16) or 32-byte (fp32) read, contiguous stores into the K pool
// (K[block][head][d / X][offset][d % X], X = 16 bytes of elements) and 8
// element stores into the token-minor V tile (V[block][head][d][offset]).  fp8 encoding is an IEEE binary32 divide by
// the scale, saturation to +-448 and the hardware's round-to-nearest-even
// OCP e4m3 conversion; NaN is written as 0x7F.
#include "pa_internal.hpp"

namespace pa {

__device__ __forceinline__ uint32_t encode_e4m3_pair(float x0, float x1, float s) {
    float y0 = x0 / s;                     // correctly rounded (built with
    float y1 = x1 / s;                     // -fhip-fp32-correctly-rounded-divide-sqrt)
    const bool n0 = y0 != y0, n1 = y1 != y1;
    y0 = fminf(fmaxf(y0, -448.0f), 448.0f);
    y1 = fminf(fmaxf(y1, -448.0f), 448.0f);
    uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
    if (n0) pk = (pk & 0xFF00u) | 0x7Fu;
    if (n1) pk = (pk & 0x00FFu) | 0x7F00u;
    return pk;
}

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
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)num_tokens * num_kv_heads * CH;
    if (idx >= total) return;
    const int c = (int)(idx % CH);
    const int h = (int)((idx / CH) % num_kv_heads);
    const long t = idx / ((long)CH * num_kv_heads);
    const int slot = slots[t];
    if (slot < 0) return;
    const long blk = slot / kBlock;
    const int off = slot % kBlock;
    const long src = (t * num_kv_heads + h) * D + 8 * c;
    // element index of K[blk][h][d / X][off][d % X] for d = 8c (X elements per 16 bytes)
    constexpr int X = (CACHE == kF32) ? 4 : (CACHE == kBF16 ? 8 : 16);
    auto kidx = [&](int d) -> long {
        return (((blk * num_kv_heads + h) * (D / X) + d / X) * kBlock + off) * X + d % X;
    };
    const long vdst = ((blk * num_kv_heads + h) * D + 8 * c) * kBlock + off;

    if (CACHE == kF32) {
        const float* ks = static_cast<const float*>(k_new) + src;
        const float* vsrc = static_cast<const float*>(v_new) + src;
        u32x4 k0 = load16_cached(ks), k1 = load16_cached(ks + 4);
        u32x4 v0 = load16_cached(vsrc), v1 = load16_cached(vsrc + 4);
        float* kc = reinterpret_cast<float*>(k_cache);
        *reinterpret_cast<u32x4*>(kc + kidx(8 * c)) = k0;
        *reinterpret_cast<u32x4*>(kc + kidx(8 * c + 4)) = k1;
        uint32_t* vd = reinterpret_cast<uint32_t*>(v_cache) + vdst;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vd[e * kBlock] = v0[e];
            vd[(e + 4) * kBlock] = v1[e];
        }
    } else if (CACHE == kBF16) {
        u32x4 kv = load16_cached(static_cast<const uint16_t*>(k_new) + src);
        u32x4 vv = load16_cached(static_cast<const uint16_t*>(v_new) + src);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(k_cache) + kidx(8 * c)) = kv;
        uint16_t* vd = reinterpret_cast<uint16_t*>(v_cache) + vdst;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vd[(2 * e) * kBlock] = (uint16_t)(vv[e] & 0xFFFFu);
            vd[(2 * e + 1) * kBlock] = (uint16_t)(vv[e] >> 16);
        }
    } else {  // bf16 -> fp8 e4m3
        const float ksc = k_scale[h], vsc = v_scale[h];
        u32x4 kv = load16_cached(static_cast<const uint16_t*>(k_new) + src);
        u32x4 vv = load16_cached(static_cast<const uint16_t*>(v_new) + src);
        uint32_t kq[2], vq[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t ka = kv[2 * w], kb = kv[2 * w + 1];
            const uint32_t lo = encode_e4m3_pair(bf16_bits_to_f32(ka & 0xFFFF), bf16_bits_to_f32(ka >> 16), ksc);
            const uint32_t hi = encode_e4m3_pair(bf16_bits_to_f32(kb & 0xFFFF), bf16_bits_to_f32(kb >> 16), ksc);
            kq[w] = lo | (hi << 16);
            const uint32_t va = vv[2 * w], vb2 = vv[2 * w + 1];
            const uint32_t vlo = encode_e4m3_pair(bf16_bits_to_f32(va & 0xFFFF), bf16_bits_to_f32(va >> 16), vsc);
            const uint32_t vhi = encode_e4m3_pair(bf16_bits_to_f32(vb2 & 0xFFFF), bf16_bits_to_f32(vb2 >> 16), vsc);
            vq[w] = vlo | (vhi << 16);
        }
        u32x2 kk = {kq[0], kq[1]};
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(k_cache) + kidx(8 * c)) = kk;
        uint8_t* vd = reinterpret_cast<uint8_t*>(v_cache) + vdst;
#pragma unroll
        for (int e = 0; e < 8; ++e) vd[e * kBlock] = (uint8_t)(vq[e >> 2] >> (8 * (e & 3)));
    }
}

template <int IN, int CACHE, int D>
static hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                const float* k_scale, const float* v_scale, const int32_t* slots,
                                int num_tokens, int num_kv_heads, hipStream_t stream) {
    const long total = (long)num_tokens * num_kv_heads * (D / 8);
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
