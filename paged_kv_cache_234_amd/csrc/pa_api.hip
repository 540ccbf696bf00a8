// Library-level entry points: status strings, workspace sizing, self test.
//
// The self test exists because a build that "succeeds" but cannot run is
// worse than an honest failure (infer-lab, ADR-0009: artifacts are verified
// before use): it launches a one-wave kernel compiled for gfx950 and checks
// what it wrote, so a missing or wrong-target code object is reported as
// PA_ERR_LAUNCH instead of surfacing later as wrong numbers.
#include "pa_internal.hpp"

namespace pa {

__device__ uint32_t g_selftest[kWave];

__global__ void selftest_kernel(uint32_t magic) {
    const int l = lane_id();
    // one MFMA so the check also proves the matrix cores run: a 16x16x4 fp32
    // product of all-ones operands gives 4 in every output element
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    c = mfma_f32(1.0f, 1.0f, c);
    g_selftest[l] = magic ^ (uint32_t)l ^ (c[0] == 4.0f && c[3] == 4.0f ? 0u : 0x80000000u);
}

// Read-bandwidth probe: every wavefront reads 4 KB chunks of `buf` in the
// order `chunk_ids` gives, with kProbeFlight chunks in flight, as the decode
// streams its K/V block tiles; each lane folds what it read into one word so
// the loads stay live.  One workgroup of four wavefronts per compute unit.
constexpr int kProbeFlight = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const char* __restrict__ buf,
                                                         const int32_t* __restrict__ ids,
                                                         int nchunks, uint32_t* sink) {
    const int lane = lane_id();
    const int gw = blockIdx.x * 4 + threadIdx.x / kWave;
    const int nw = gridDim.x * 4;
    uint32_t acc = 0;
    for (int c0 = gw * kProbeFlight; c0 < nchunks; c0 += nw * kProbeFlight) {
        u32x4 v[kProbeFlight][4];
#pragma unroll
        for (int f = 0; f < kProbeFlight; ++f) {
            const char* base = buf + (long)ids[min(c0 + f, nchunks - 1)] * 4096;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[f][k] = load16(base + 1024 * k + 16 * lane);
        }
#pragma unroll
        for (int f = 0; f < kProbeFlight; ++f)
#pragma unroll
            for (int k = 0; k < 4; ++k) acc ^= v[f][k][0] ^ v[f][k][1] ^ v[f][k][2] ^ v[f][k][3];
    }
    sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_read_probe(const void* buf, size_t bytes, const int32_t* chunk_ids,
                                     int32_t num_chunks, uint32_t* sink, size_t sink_bytes,
                                     hipStream_t stream) {
    if (!buf || !chunk_ids || !sink || num_chunks <= 0) return PA_ERR_ARG;
    if (bytes < 4096 || (size_t)num_chunks > bytes / 4096) return PA_ERR_ARG;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (sink_bytes < (size_t)cus * 256 * sizeof(uint32_t)) return PA_ERR_ARG;
    hipLaunchKernelGGL(read_probe_kernel, dim3(cus), dim3(256), 0, stream,
                       static_cast<const char*>(buf), chunk_ids, num_chunks, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" const char* pa_status_string(pa_status_t s) {
    switch (s) {
        case PA_OK: return "PA_OK";
        case PA_ERR_ARG: return "PA_ERR_ARG: null pointer or invalid size";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: dtype/head_dim/block_size/GQA combination not built";
        case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case PA_ERR_TOO_LARGE: return "PA_ERR_TOO_LARGE: the partials exceed pa_decode_noalloc's static scratch";
    }
    return "PA_ERR_UNKNOWN";
}

extern "C" size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim,
                                            int32_t max_partitions) {
    if (batch < 0 || num_heads < 0 || head_dim < 0 || max_partitions < 0) return 0;
    const size_t n = (size_t)batch * num_heads * max_partitions;
    return n * sizeof(float) * (2 + (size_t)head_dim);
}

extern "C" pa_status_t pa_selftest(void) {
    const uint32_t magic = 0x5A17C0DEu;
    hipLaunchKernelGGL(selftest_kernel, dim3(1), dim3(kWave), 0, 0, magic);
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
    if (hipDeviceSynchronize() != hipSuccess) return PA_ERR_LAUNCH;
    uint32_t host[kWave];
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(g_selftest), sizeof(host), 0, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return PA_ERR_LAUNCH;
    for (int l = 0; l < kWave; ++l)
        if (host[l] != (magic ^ (uint32_t)l)) return PA_ERR_LAUNCH;
    return PA_OK;
}
