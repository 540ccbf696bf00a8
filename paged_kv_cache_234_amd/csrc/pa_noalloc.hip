// Split-K decode that allocates nothing: for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc) and so cannot provide pa_decode's partial buffers.
//
// The partials (m_p, l_p, o_p) go to `scratch`, a fixed array in the
// library's own device memory: each GPU the library runs on holds one copy,
// kScratchBytes large, until the process ends.  The call is pa_decode with
// partition_size > 0 writing into that array, then pa_decode_splitk_reduce
// reading it into `out`; the kernels are the same, so the results are the
// same bits.  Every call on a GPU shares that GPU's array, so two calls that
// overlap on one GPU (different streams, or different threads without
// ordering) race.  Nothing in it needs to start at zero: the reduce reads only
// the partitions the decode of the same call writes.
#include <mutex>

#include "pa_internal.hpp"

namespace pa {

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Host code must not use `scratch` itself (a host-side stand-in): the device
// address of each GPU's copy is looked up once, with that GPU current.
constexpr int kMaxDevices = 64;
static void* g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

static pa_status_t scratch_address(void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return PA_ERR_LAUNCH;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return PA_OK;
}

constexpr size_t align256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace pa

using namespace pa;

extern "C" size_t pa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" pa_status_t pa_decode_noalloc(void* out, const void* q, pa_dtype_t q_dtype,
                                         const void* k_cache, const void* v_cache,
                                         pa_dtype_t cache_dtype, const float* k_scale,
                                         const float* v_scale, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, float scale,
                                         int32_t partition_size, int32_t max_partitions,
                                         hipStream_t stream) {
    // every host argument is checked before the device is touched
    pa_status_t st = check_attention_shape(q_dtype, cache_dtype, k_scale, v_scale, num_heads,
                                           num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (batch < 0 || max_blocks_per_seq < 1 || partition_size <= 0 || max_partitions < 1)
        return PA_ERR_ARG;
    if (partition_size % kBlock) return PA_ERR_ARG;
    if (!std::isfinite(scale)) return PA_ERR_ARG;
    if (batch == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_ARG;
    const size_t n = (size_t)batch * num_heads * max_partitions;
    const size_t off_sum = align256(n * sizeof(float));
    const size_t off_out = off_sum + align256(n * sizeof(float));
    if (off_out + n * head_dim * sizeof(float) > kScratchBytes) return PA_ERR_TOO_LARGE;
    void* base = nullptr;
    st = scratch_address(&base);
    if (st != PA_OK) return st;
    unsigned char* s = static_cast<unsigned char*>(base);
    float* part_max = reinterpret_cast<float*>(s);
    float* part_sum = reinterpret_cast<float*>(s + off_sum);
    float* part_out = reinterpret_cast<float*>(s + off_out);
    st = pa_decode(nullptr, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale,
                   block_tables, max_blocks_per_seq, context_lens, batch, num_heads, num_kv_heads,
                   head_dim, block_size, scale, partition_size, max_partitions, part_max, part_sum,
                   part_out, stream);
    if (st != PA_OK) return st;
    return pa_decode_splitk_reduce(out, q_dtype, part_max, part_sum, part_out, context_lens, batch,
                                   num_heads, head_dim, partition_size, max_partitions, stream);
}
