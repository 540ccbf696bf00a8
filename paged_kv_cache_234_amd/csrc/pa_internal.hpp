// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <cmath>

#include "pa.h"
#include "pa_device.hpp"

namespace pa {

inline int cache_kind(pa_dtype_t t) {
    switch (t) {
        case PA_DT_F32: return kF32;
        case PA_DT_BF16: return kBF16;
        case PA_DT_FP8_E4M3: return kFP8;
    }
    return -1;
}

inline bool valid_dtype(pa_dtype_t t) {
    return t == PA_DT_F32 || t == PA_DT_BF16 || t == PA_DT_FP8_E4M3;
}

// (q / new-token dtype, cache dtype) pairs the kernels are built for.
inline bool supported_pair(pa_dtype_t in, pa_dtype_t cache) {
    return (in == PA_DT_F32 && cache == PA_DT_F32) || (in == PA_DT_BF16 && cache == PA_DT_BF16) ||
           (in == PA_DT_BF16 && cache == PA_DT_FP8_E4M3);
}

// Validation common to the attention entry points (no device access).
inline pa_status_t check_attention_shape(pa_dtype_t q_dtype, pa_dtype_t cache_dtype,
                                         const float* k_scale, const float* v_scale,
                                         int num_heads, int num_kv_heads, int head_dim,
                                         int block_size) {
    if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PA_ERR_ARG;
    if (num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0) return PA_ERR_ARG;
    if (num_heads % num_kv_heads) return PA_ERR_ARG;
    if (!supported_pair(q_dtype, cache_dtype)) return PA_ERR_UNSUPPORTED;
    if (block_size != kBlock) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (num_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
    if (cache_dtype == PA_DT_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_ARG;
    return PA_OK;
}

}  // namespace pa
