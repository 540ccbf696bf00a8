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

}  // namespace pa

using namespace pa;

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
