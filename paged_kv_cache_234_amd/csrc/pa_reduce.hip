// Split-K (flash-decoding) reduce: merge per-partition softmax statistics.
//
// For each (sequence b, query head hq) with P = ceil(L_b / PS) partitions:
//   M = max_p m_p,  w_p = l_p * exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// This is the standard merge of online-softmax partial states (the same
// identity that makes tiled attention equal to naive attention, infer-lab's
// invariant list); the pages themselves do not describe split-K.
//
// One 256-thread workgroup per (b, hq): the weights go to LDS, then each
// thread accumulates float4 columns of o_p over a strided subset of the
// partitions and the subsets are summed through LDS.
#include "pa_internal.hpp"

namespace pa {

constexpr int kMaxReducePartitions = 4096;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void reduce_kernel(void* __restrict__ out,
                                                     const float* __restrict__ part_max,
                                                     const float* __restrict__ part_sum,
                                                     const float* __restrict__ part_out,
                                                     const int32_t* __restrict__ context_lens,
                                                     int num_heads, int partition_size,
                                                     int max_partitions) {
    constexpr int NT = 256, D4 = D / 4, NPH = NT / D4;
    __shared__ float s_w[kMaxReducePartitions];
    __shared__ float s_red[NT / kWave];
    __shared__ f32x4 s_acc[NPH][D4];

    const int bh = blockIdx.x;
    const int b = bh / num_heads;
    const int tid = threadIdx.x, wave = tid / kWave;
    const int L = context_lens[b];
    // never trust L beyond the caller-declared bound: it sizes LDS and rows
    const int P = min((L + partition_size - 1) / partition_size, max_partitions);
    const long base = (long)bh * max_partitions;

    float M = -INFINITY;
    for (int i = tid; i < P; i += NT) M = fmaxf(M, part_max[base + i]);
    M = wave_max(M);
    if ((tid & (kWave - 1)) == 0) s_red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();

    float wsum = 0.f;
    for (int i = tid; i < P; i += NT) {
        const float w = part_sum[base + i] * fast_exp2((part_max[base + i] - M) * kLog2e);
        s_w[i] = w;
        wsum += w;
    }
    wsum = wave_sum(wsum);
    if ((tid & (kWave - 1)) == 0) s_red[wave] = wsum;
    __syncthreads();
    const float W = s_red[0] + s_red[1] + s_red[2] + s_red[3];

    const int d4 = tid % D4, ph = tid / D4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4* po = reinterpret_cast<const f32x4*>(part_out + base * D) + d4;
    for (int i = ph; i < P; i += NPH) acc += s_w[i] * po[(long)i * D4];
    s_acc[ph][d4] = acc;
    __syncthreads();
    if (tid < D4) {
        f32x4 s = s_acc[0][tid];
#pragma unroll
        for (int k = 1; k < NPH; ++k) s += s_acc[k][tid];
        const float inv = (P > 0) ? 1.0f / W : 0.0f;
        s = (P > 0) ? s * inv : f32x4{0.f, 0.f, 0.f, 0.f};
        if (OUT_BF16) {
            uint16_t* o = static_cast<uint16_t*>(out) + (long)bh * D + 4 * tid;
            u32x2 pk = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
            *reinterpret_cast<u32x2*>(o) = pk;
        } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (long)bh * D + 4 * tid) = s;
        }
    }
}

// Few partitions (max_partitions <= 64): one wavefront per (sequence, query
// head), four per workgroup.  Lane p holds partition p's (m, l); the weights
// are broadcast with v_readlane while each lane accumulates D/64 columns.
// The first U partition rows (U: max_partitions rounded up to a power of two,
// at most 16) are loaded together with (m, l), so up to U partitions cost one
// memory round trip.
template <int D, bool OUT_BF16, int U>
__global__ __launch_bounds__(256) void reduce_wave_kernel(void* __restrict__ out,
                                                          const float* __restrict__ part_max,
                                                          const float* __restrict__ part_sum,
                                                          const float* __restrict__ part_out,
                                                          const int32_t* __restrict__ context_lens,
                                                          int num_heads, int partition_size,
                                                          int max_partitions, int npairs) {
    constexpr int C = D / kWave;                       // columns per lane
    const int lane = lane_id();
    const int bh = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
    if (bh >= npairs) return;
    const int b = bh / num_heads;
    const int L = context_lens[b];
    const int P = min((L + partition_size - 1) / partition_size, max_partitions);
    const long base = (long)bh * max_partitions;
    // Every load is unconditional, at an index clamped into the caller's
    // buffer rather than into [0, P), so none waits for the context length
    // (or for another load); values at or past P are masked by selects.
    const float* po = part_out + base * D + C * lane;
    auto load_rows = [&](float (&row)[U][C], int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < C; ++k)
                row[u][k] = po[(long)min(p0 + u, max_partitions - 1) * D + k];
    };
    const int pl = min(lane, max_partitions - 1);
    const float m_raw = part_max[base + pl], l_raw = part_sum[base + pl];
    float row[U][C];
    load_rows(row, 0);
    __builtin_amdgcn_sched_barrier(0);          // all of them out before the first wait
    const float mp = lane < P ? m_raw : -INFINITY;
    const float M = wave_max(mp);
    const float w = lane < P ? l_raw * fast_exp2((mp - M) * kLog2e) : 0.f;
    const float W = wave_sum(w);
    float acc[C];
#pragma unroll
    for (int k = 0; k < C; ++k) acc[k] = 0.f;
    auto accumulate = [&](const float (&row)[U][C], int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int pp = min(p0 + u, kWave - 1);
            const float wp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                           __builtin_bit_cast(int, w), pp));
#pragma unroll
            for (int k = 0; k < C; ++k) acc[k] += (p0 + u < P) ? wp * row[u][k] : 0.f;
        }
    };
    accumulate(row, 0);                         // unconditional: the loads stay up front
    for (int p0 = U; p0 < P; p0 += U) {
        load_rows(row, p0);
        accumulate(row, p0);
    }
    const float inv = P > 0 ? 1.0f / W : 0.f;
    if (OUT_BF16) {
        uint16_t* o = static_cast<uint16_t*>(out) + (long)bh * D + C * lane;
#pragma unroll
        for (int k = 0; k < C; ++k) o[k] = f32_to_bf16_bits(acc[k] * inv);
    } else {
        float* o = static_cast<float*>(out) + (long)bh * D + C * lane;
#pragma unroll
        for (int k = 0; k < C; ++k) o[k] = acc[k] * inv;
    }
}

// Up to 256 partitions: one workgroup of four wavefronts per (sequence,
// query head).  Wavefront w takes partitions w, w + 4, w + 8, .. (lane j holds
// partition w + 4j's (m, l)) and reduces them as reduce_wave_kernel does,
// with all of its rows loaded in one round trip (U >= its partition count);
// the four (max, weight sum, sums) are then combined through LDS.  Row
// indices are clamped to the sequence's own last partition, so the loads
// past it (U is sized for the longest sequence) re-read a cached row.
template <int D, bool OUT_BF16, int U>
__global__ __launch_bounds__(256) void reduce_wave4_kernel(void* __restrict__ out,
                                                           const float* __restrict__ part_max,
                                                           const float* __restrict__ part_sum,
                                                           const float* __restrict__ part_out,
                                                           const int32_t* __restrict__ context_lens,
                                                           int num_heads, int partition_size,
                                                           int max_partitions) {
    constexpr int C = D / kWave;                       // columns per lane
    __shared__ float s_m[4], s_w[4];
    __shared__ float s_acc[4][D];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int bh = blockIdx.x;
    const int b = bh / num_heads;
    const int L = context_lens[b];
    const int P = min((L + partition_size - 1) / partition_size, max_partitions);
    const long base = (long)bh * max_partitions;
    const int n = P > wave ? (P - wave + 3) / 4 : 0;   // this wave's partitions
    // unconditional loads at indices clamped to this wave's last partition
    const int last = max(min(wave + 4 * (n - 1), max_partitions - 1), 0);
    const int pl = min(wave + 4 * lane, last);
    const float m_raw = part_max[base + pl], l_raw = part_sum[base + pl];
    const float* po = part_out + base * D + C * lane;
    float row[U][C];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < C; ++k)
            row[u][k] = po[(long)min(wave + 4 * u, last) * D + k];
    __builtin_amdgcn_sched_barrier(0);          // all of them out before the first wait
    const float mp = lane < n ? m_raw : -INFINITY;
    const float M = wave_max(mp);
    const float w = lane < n ? l_raw * fast_exp2((mp - M) * kLog2e) : 0.f;
    const float W = wave_sum(w);
    float acc[C];
#pragma unroll
    for (int k = 0; k < C; ++k) acc[k] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float wp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                       __builtin_bit_cast(int, w), u));
#pragma unroll
        for (int k = 0; k < C; ++k) acc[k] += (u < n) ? wp * row[u][k] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < C; ++k) s_acc[wave][C * lane + k] = acc[k];
    if (lane == 0) {
        s_m[wave] = M;
        s_w[wave] = W;
    }
    __syncthreads();
    if (wave != 0) return;
    const float Mg = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float a[4], Wg = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        a[v] = s_m[v] == -INFINITY ? 0.f : fast_exp2((s_m[v] - Mg) * kLog2e);
        Wg += a[v] * s_w[v];
    }
    const float inv = P > 0 ? 1.0f / Wg : 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
        float x = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) x += a[v] * s_acc[v][C * lane + k];
        x *= inv;
        if (OUT_BF16)
            static_cast<uint16_t*>(out)[(long)bh * D + C * lane + k] = f32_to_bf16_bits(x);
        else
            static_cast<float*>(out)[(long)bh * D + C * lane + k] = x;
    }
}

template <int D, bool OUT_BF16>
static hipError_t launch_reduce(void* out, const float* pm, const float* ps, const float* po,
                                const int32_t* lens, int batch, int num_heads, int partition_size,
                                int max_partitions, hipStream_t stream) {
    const long pairs = (long)batch * num_heads;
    if (pairs > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (max_partitions <= kWave) {
        const dim3 grid((unsigned)((pairs + 3) / 4));
#define PA_REDUCE_WAVE(UU)                                                                    \
    hipLaunchKernelGGL((reduce_wave_kernel<D, OUT_BF16, UU>), grid, dim3(256), 0, stream, out, \
                       pm, ps, po, lens, num_heads, partition_size, max_partitions, (int)pairs)
        if (max_partitions <= 2) PA_REDUCE_WAVE(2);
        else if (max_partitions <= 4) PA_REDUCE_WAVE(4);
        else if (max_partitions <= 8) PA_REDUCE_WAVE(8);
        else PA_REDUCE_WAVE(16);
#undef PA_REDUCE_WAVE
    } else if (max_partitions <= 4 * kWave) {
#define PA_REDUCE_WAVE4(UU)                                                                   \
    hipLaunchKernelGGL((reduce_wave4_kernel<D, OUT_BF16, UU>), dim3((unsigned)pairs), dim3(256), \
                       0, stream, out, pm, ps, po, lens, num_heads, partition_size, max_partitions)
        if (max_partitions <= 128) PA_REDUCE_WAVE4(32);
        else PA_REDUCE_WAVE4(64);
#undef PA_REDUCE_WAVE4
    } else {
        hipLaunchKernelGGL((reduce_kernel<D, OUT_BF16>), dim3((unsigned)pairs), dim3(256), 0,
                           stream, out, pm, ps, po, lens, num_heads, partition_size,
                           max_partitions);
    }
    return hipGetLastError();
}

}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_decode_splitk_reduce(void* out, pa_dtype_t out_dtype,
                                               const float* part_max, const float* part_sum,
                                               const float* part_out, const int32_t* context_lens,
                                               int32_t batch, int32_t num_heads, int32_t head_dim,
                                               int32_t partition_size, int32_t max_partitions,
                                               hipStream_t stream) {
    if (!valid_dtype(out_dtype)) return PA_ERR_ARG;
    if (batch < 0 || num_heads <= 0 || head_dim <= 0 || partition_size <= 0 || max_partitions < 1)
        return PA_ERR_ARG;
    if (out_dtype == PA_DT_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (max_partitions > kMaxReducePartitions) return PA_ERR_UNSUPPORTED;
    if (batch == 0) return PA_OK;
    if (!out || !part_max || !part_sum || !part_out || !context_lens) return PA_ERR_ARG;
    hipError_t e;
    const bool bf = out_dtype == PA_DT_BF16;
    if (head_dim == 128)
        e = bf ? launch_reduce<128, true>(out, part_max, part_sum, part_out, context_lens, batch,
                                          num_heads, partition_size, max_partitions, stream)
               : launch_reduce<128, false>(out, part_max, part_sum, part_out, context_lens, batch,
                                           num_heads, partition_size, max_partitions, stream);
    else
        e = bf ? launch_reduce<64, true>(out, part_max, part_sum, part_out, context_lens, batch,
                                         num_heads, partition_size, max_partitions, stream)
               : launch_reduce<64, false>(out, part_max, part_sum, part_out, context_lens, batch,
                                          num_heads, partition_size, max_partitions, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
