// store_kv.hip -- KV-cache write: token t's K and V rows go to pool row
// slot_mapping[t] ("nano-vLLM interactive guide" ch.08, attention and cache
// writes; "Visual atlas" figure index, slot example: each K component is
// filled into its cell of the physical pool).
//
// One workgroup row per token: blockIdx.y strides over tokens, and the
// 2 * row_elems / 8 sixteen-byte chunks of the token's K and V rows are spread
// over the x dimension.  The copy is a plain 16-byte load/store, so the pool
// receives the token's bits unchanged.  Tokens with a negative slot (padding)
// are skipped.  HBM-bound: every byte is read once and written once.
#include "pa_common.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void store_kv_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, uint4 *__restrict__ k_cache,
    uint4 *__restrict__ v_cache, const int32_t *__restrict__ slot_mapping, int32_t num_tokens,
    int32_t row_chunks)
{
    const int32_t chunk = blockIdx.x * kThreads + threadIdx.x;   // over K chunks then V chunks
    if (chunk >= 2 * row_chunks)
        return;
    const bool is_v = chunk >= row_chunks;
    const int32_t c = is_v ? chunk - row_chunks : chunk;
    const uint4 *src = is_v ? v : k;
    uint4 *dst = is_v ? v_cache : k_cache;
    for (int32_t t = blockIdx.y; t < num_tokens; t += gridDim.y) {
        const int32_t slot = slot_mapping[t];
        if (slot < 0)
            continue;
        dst[(int64_t)slot * row_chunks + c] = src[(int64_t)t * row_chunks + c];
    }
}

}  // namespace

hipError_t launch_store_kv(const void *k, const void *v, void *k_cache, void *v_cache,
                           const int32_t *slot_mapping, int32_t num_tokens, int32_t row_elems,
                           hipStream_t stream)
{
    const int32_t row_chunks = row_elems / 8;
    dim3 grid((2 * row_chunks + kThreads - 1) / kThreads, num_tokens < 65535 ? num_tokens : 65535);
    hipLaunchKernelGGL(store_kv_kernel, grid, dim3(kThreads), 0, stream,
                       static_cast<const uint4 *>(k), static_cast<const uint4 *>(v),
                       static_cast<uint4 *>(k_cache), static_cast<uint4 *>(v_cache),
                       slot_mapping, num_tokens, row_chunks);
    return hipGetLastError();
}

}  // namespace pa
