// noalloc.hip -- pa_decode_noalloc: pa_decode for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The decode partials, which pa_decode keeps in a
// caller-supplied workspace, live here in one file-scope device array of a
// fixed size instead.
//
// Each device the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name only stands in for it; its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept, and only that address is ever passed on.
#include <hip/hip_runtime.h>

#include <atomic>

#include "pa.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // PA_NOALLOC_SCRATCH_BYTES in pa.h
static_assert(kScratchBytes == PA_NOALLOC_SCRATCH_BYTES, "header and library disagree");

// the decode partials of every pa_decode_noalloc call on this device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// device address of the current device's copy of the scratch array (looked up on
// the first call on that device; concurrent first calls store the same value)
int scratch_ptr(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return PA_ERR_LAUNCH;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return PA_ERR_LAUNCH;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, int32_t num_seqs,
                                 int32_t max_context_len, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 float scale, int32_t partition_size, void *out,
                                 hipStream_t stream)
{
    // the same size checks as pa_decode, then the partials must fit the array
    const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_context_len, partition_size);
    if (need > kScratchBytes)
        return PA_ERR_SCRATCH;
    void *ws = nullptr;
    if (num_seqs > 0) {
        const int st = scratch_ptr(&ws);
        if (st != PA_OK)
            return st;
    }
    return pa_decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                     scale, partition_size, ws, ws ? kScratchBytes : 0, out, stream);
}
