// Writing one new token's K/V row into the pools, shared by pa_kv_append and
// the decode kernel's fused append.
//
// A chunk is 8 consecutive head_dim elements (chunk c) of one (token, head):
// contiguous stores into the K pool (K[block][head][d / X][offset][d % X],
// X = 16 bytes of elements) and 8 element stores into the token-minor V tile
// (V[block][head][d][offset]).  fp8 encoding is an IEEE binary32 divide by
// the scale (built with -fhip-fp32-correctly-rounded-divide-sqrt),
// saturation to +-448 and the hardware's round-to-nearest-even OCP e4m3
// conversion; NaN is written as 0x7F.
#pragma once

#include "pa_device.hpp"

namespace pa {

__device__ __forceinline__ uint32_t encode_e4m3_pair(float x0, float x1, float s) {
    float y0 = x0 / s;
    float y1 = x1 / s;
    const bool n0 = y0 != y0, n1 = y1 != y1;
    y0 = fminf(fmaxf(y0, -448.0f), 448.0f);
    y1 = fminf(fmaxf(y1, -448.0f), 448.0f);
    uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
    if (n0) pk = (pk & 0xFF00u) | 0x7Fu;
    if (n1) pk = (pk & 0x00FFu) | 0x7F00u;
    return pk;
}

// One lane's chunk of a token row as loaded from the input: 8 elements of K
// and of V (fp32: two 16-byte pieces each).
template <int CACHE> struct TokenChunk {
    static constexpr int N = CACHE == kF32 ? 2 : 1;
    u32x4 k[N], v[N];
};

// k_src / v_src: the token's row for this head (D elements of the input type)
template <int CACHE, int D>
__device__ __forceinline__ TokenChunk<CACHE> load_token_chunk(const void* k_src, const void* v_src,
                                                              int c) {
    TokenChunk<CACHE> t;
    if (CACHE == kF32) {
        const float* ks = static_cast<const float*>(k_src) + 8 * c;
        const float* vs = static_cast<const float*>(v_src) + 8 * c;
        t.k[0] = load16_cached(ks);
        t.k[t.N - 1] = load16_cached(ks + 4);
        t.v[0] = load16_cached(vs);
        t.v[t.N - 1] = load16_cached(vs + 4);
    } else {
        t.k[0] = load16_cached(static_cast<const uint16_t*>(k_src) + 8 * c);
        t.v[0] = load16_cached(static_cast<const uint16_t*>(v_src) + 8 * c);
    }
    return t;
}

// blk / off: the token's slot; ksc / vsc: the head's fp8 scales (fp8 caches only)
template <int CACHE, int D>
__device__ __forceinline__ void store_token_chunk(const TokenChunk<CACHE>& t, char* k_cache,
                                                  char* v_cache, long blk, int off, int h,
                                                  int num_kv_heads, int c, float ksc, float vsc) {
    // element index of K[blk][h][d / X][off][d % X] for d = 8c (X elements per 16 bytes)
    constexpr int X = (CACHE == kF32) ? 4 : (CACHE == kBF16 ? 8 : 16);
    auto kidx = [&](int d) -> long {
        return (((blk * num_kv_heads + h) * (D / X) + d / X) * kBlock + off) * X + d % X;
    };
    const long vdst = ((blk * num_kv_heads + h) * D + 8 * c) * kBlock + off;

    if (CACHE == kF32) {
        float* kc = reinterpret_cast<float*>(k_cache);
        *reinterpret_cast<u32x4*>(kc + kidx(8 * c)) = t.k[0];
        *reinterpret_cast<u32x4*>(kc + kidx(8 * c + 4)) = t.k[t.N - 1];
        uint32_t* vd = reinterpret_cast<uint32_t*>(v_cache) + vdst;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vd[e * kBlock] = t.v[0][e];
            vd[(e + 4) * kBlock] = t.v[t.N - 1][e];
        }
    } else if (CACHE == kBF16) {
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(k_cache) + kidx(8 * c)) = t.k[0];
        uint16_t* vd = reinterpret_cast<uint16_t*>(v_cache) + vdst;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vd[(2 * e) * kBlock] = (uint16_t)(t.v[0][e] & 0xFFFFu);
            vd[(2 * e + 1) * kBlock] = (uint16_t)(t.v[0][e] >> 16);
        }
    } else {  // bf16 -> fp8 e4m3
        const u32x4 kv = t.k[0], vv = t.v[0];
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

template <int CACHE, int D>
__device__ __forceinline__ void write_token_chunk(const void* k_src, const void* v_src,
                                                  char* k_cache, char* v_cache, long blk, int off,
                                                  int h, int num_kv_heads, int c, float ksc,
                                                  float vsc) {
    store_token_chunk<CACHE, D>(load_token_chunk<CACHE, D>(k_src, v_src, c), k_cache, v_cache,
                                blk, off, h, num_kv_heads, c, ksc, vsc);
}

}  // namespace pa
