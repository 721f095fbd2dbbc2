// pa_api.cpp -- the extern "C" entry points of libpa.so (declared in
// include/pa.h): host-side argument checks, kernel selection and launch.
// Nothing here reads device memory, allocates, or synchronises, so every
// device entry point can be captured into a HIP graph.
#include <initializer_list>
#include <math.h>
#include <stdint.h>

#include "pa.h"
#include "pa_common.h"

namespace {

constexpr int kHeadDim = 128;
// library decode partitioning (partition_size == 0); see resolve_partition
constexpr int64_t kDecodeWholeSequencePairs = 1024;   // (sequence, KV head) pairs that fill the chip
constexpr int64_t kDecodeWholeSequencePairsMha = 4096;   // the same with one Q head per KV head
constexpr int32_t kDecodePartMax = 4096;              // keys: the largest partition
constexpr int32_t kDecodePartMin = 256;               // keys: the last partition of a sequence
constexpr int32_t kDecodePartMinMfma = 512;           // the same for groups of 8 (MFMA kernel)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_if_pow2(int32_t x) {
    if (x <= 0 || (x & (x - 1)) != 0)
        return -1;
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

bool group_supported(int32_t hq, int32_t hkv) {
    if (hkv <= 0 || hq <= 0 || hq % hkv != 0)
        return false;
    const int32_t g = hq / hkv;
    return g == 1 || g == 2 || g == 4 || g == 8;
}

struct Plan {
    int32_t P, u;   // pa::plan_count / plan_range parameters
};

// Decode partitioning (host integers only, tuned on MI355X).  An explicit
// partition_size gives fixed partitions of that many keys.  Otherwise, with at
// least 1024 (sequence, KV head) pairs every sequence is one partition: the grid
// already fills the chip several times over, and whole-sequence workgroups need no
// partials or merge pass.  One Q head per KV head is the exception up to 4096
// pairs: its kernel runs three workgroups per CU (two for larger groups), and the
// shorter tail outweighs the partials and the merge pass (256 ragged contexts at
// Hq 8 / Hkv 8: 359 -> 343 us per step, while at Hq 16 / Hkv 8 whole sequences
// stay ahead, 357 against 363-369 us).  With fewer pairs the keys are split into partitions of
// at most 4096 keys that shrink to 256 toward the end of each sequence, so the
// workgroups launched last are short and the chip drains evenly (measured on
// MI355X against fixed 1024-key partitions: 16 x 32768 keys at Hkv 8 354 -> 343 us,
// 256 ragged contexts at Hq 8 / Hkv 1 78 -> 65 us; then 2048 -> 4096 for the largest
// partition: the 16 x 32768 step 342 -> 337 us, 8192 or 16384 340 us, 1024 353 us; the
// plans differ only for contexts past 5632 keys).  Groups of 8 run the MFMA kernel,
// whose workgroups cost more to start and less per key, and take 512-key tail
// partitions (256 ragged contexts at Hq 8 / Hkv 1: 61.1 -> 59.6 us per step launched
// directly; 1024-key tails 64.7 us; at Hq 8 / Hkv 2, on the dot-product kernel, 512-key
// tails cost 98.3 -> 100.8 us, so groups up to 4 keep 256).
Plan resolve_partition(int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t max_context_len) {
    if (partition_size != 0)
        return {partition_size, 0};
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    const int64_t whole_at = num_q_heads == num_kv_heads ? kDecodeWholeSequencePairsMha
                                                         : kDecodeWholeSequencePairs;
    if (pairs >= whole_at) {
        const int64_t whole = ((int64_t)max_context_len + 255) / 256 * 256;
        return {(int32_t)(whole < 256 ? 256 : whole > (1 << 30) ? (1 << 30) : whole), 0};
    }
    return {kDecodePartMax, num_q_heads / num_kv_heads >= 8 ? kDecodePartMinMfma : kDecodePartMin};
}

int32_t num_partitions(int32_t max_context_len, Plan pl) {
    return pa::plan_count(max_context_len, pl.P, pl.u);
}

}  // namespace

extern "C" {

const char *pa_status_string(int status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes are invalid or inconsistent";
    case PA_ERR_UNSUPPORTED: return "sizes are valid but not supported by this build";
    case PA_ERR_WORKSPACE: return "workspace is too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_SCRATCH: return "the call needs more than the library's fixed device scratch";
    case PA_ERR_GRAPH: return "the HIP runtime refused a graph capture, instantiation or launch";
    default: return "unknown status";
    }
}

int pa_slot_mapping(const int32_t *cu_seqlens_q, const int32_t *seqlens_k, int32_t num_seqs,
                    const int32_t *block_tables, int32_t max_blocks_per_seq, int32_t block_size,
                    int32_t *slot_mapping, int32_t num_tokens)
{
    if (!cu_seqlens_q || (num_seqs > 0 && (!seqlens_k || !block_tables)) ||
        (num_tokens > 0 && !slot_mapping))
        return PA_ERR_NULL;
    if (num_seqs < 0 || num_tokens < 0 || block_size < 1 || max_blocks_per_seq < 0)
        return PA_ERR_SHAPE;
    if (cu_seqlens_q[0] != 0 || cu_seqlens_q[num_seqs] != num_tokens)
        return PA_ERR_SHAPE;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t first_row = cu_seqlens_q[s];
        const int32_t n_new = cu_seqlens_q[s + 1] - first_row;
        if (n_new < 0 || seqlens_k[s] < n_new)
            return PA_ERR_SHAPE;
        const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int32_t i = 0; i < n_new; ++i) {
            const int32_t pos = seqlens_k[s] - n_new + i;
            const int32_t logical = pos / block_size;
            if (logical >= max_blocks_per_seq || table[logical] < 0)
                return PA_ERR_SHAPE;
            const int64_t slot = (int64_t)table[logical] * block_size + pos % block_size;
            if (slot > INT32_MAX)
                return PA_ERR_SHAPE;
            slot_mapping[first_row + i] = (int32_t)slot;
        }
    }
    return PA_OK;
}

int pa_store_kv(const void *k, const void *v, void *k_cache, void *v_cache,
                const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, hipStream_t stream)
{
    if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1)
        return PA_ERR_SHAPE;
    if ((int64_t)num_blocks * block_size > INT32_MAX)
        return PA_ERR_SHAPE;
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (row % 8 != 0 || row / 8 > (int64_t)65535 * 256)
        return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0)
        return PA_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_UNSUPPORTED;
    hipError_t e = pa::launch_store_kv(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                       (int32_t)row, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

size_t pa_kv_pool_layout(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, size_t *v_offset)
{
    // v_cache starts 384 bytes past a 1 KiB boundary after k_cache (the pools then
    // differ modulo 1 KiB, which keeps a row's K and V reads apart in the HBM interleave)
    constexpr uint64_t kAlign = 1024, kShift = 384;
    if (!v_offset || num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1)
        return 0;
    uint64_t pool = 2u;   // bytes of one pool, with every product checked for overflow
    for (int32_t f : {num_blocks, block_size, num_kv_heads, head_dim})
        if (__builtin_mul_overflow(pool, (uint64_t)f, &pool))
            return 0;
    if (pool > (uint64_t)SIZE_MAX / 2 - 2 * kAlign)
        return 0;
    const uint64_t voff = (pool + kAlign - 1) / kAlign * kAlign + kShift;
    const uint64_t total = voff + pool;
    *v_offset = (size_t)voff;
    return (size_t)total;
}

size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim)
{
    if (head_dim != kHeadDim || max_seqlen_k < max_seqlen_q)
        return 0;
    const int64_t items = pa::prefill_split_items(num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads,
                                                  num_kv_heads);
    if (items <= 0)
        return 0;
    // [items][2] partials, then [items] int32 arrival counters
    return (size_t)items * 2 * pa::kPrefillPartBytes + (size_t)items * sizeof(int32_t);
}

namespace {

int prefill_impl(const void *q, const void *k, const void *v, const void *k_cache,
                 const void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                 int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                 bool with_workspace, void *workspace, size_t workspace_bytes, void *out,
                 hipStream_t stream)
{
    const bool paged = block_tables != nullptr;
    if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_q_heads < 1 ||
        num_kv_heads < 1 || head_dim < 1 || num_q_heads % num_kv_heads != 0)
        return PA_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale))
        return PA_ERR_SHAPE;
    if (paged && (block_size < 1 || max_blocks_per_seq < 1))
        return PA_ERR_SHAPE;
    if (head_dim != kHeadDim || !group_supported(num_q_heads, num_kv_heads))
        return PA_ERR_UNSUPPORTED;
    if (num_kv_heads >= 65536)   // a K/V row (Hkv * 256 B) must stay below 2^24 bytes
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || max_seqlen_q == 0)
        return PA_OK;
    if (!q || !out || !cu_seqlens_q || !cu_seqlens_k)
        return PA_ERR_NULL;
    if (paged ? (!k_cache || !v_cache) : (!k || !v))
        return PA_ERR_NULL;
    const void *kk = paged ? k_cache : k;
    const void *vv = paged ? v_cache : v;
    if (!aligned16(q) || !aligned16(out) || !aligned16(kk) || !aligned16(vv))
        return PA_ERR_UNSUPPORTED;
    const int32_t g = num_q_heads / num_kv_heads;
    const int64_t n_qblk = ((int64_t)max_seqlen_q + 128 / g - 1) / (128 / g);
    if (n_qblk * num_seqs * num_kv_heads > INT32_MAX)
        return PA_ERR_UNSUPPORTED;

    pa::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.cu_seqlens_q = cu_seqlens_q;
    a.cu_seqlens_k = cu_seqlens_k;
    a.out = out;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = paged ? block_size : 1;
    a.bs_shift = log2_if_pow2(a.block_size);
    a.paged = paged;
    a.scale_log2 = scale * pa::kLog2e;
    a.split = 0;
    a.ws_part = nullptr;
    a.ws_cnt = nullptr;
    if (with_workspace) {
        const size_t need = pa_prefill_workspace_size(num_seqs, max_seqlen_q, max_seqlen_k,
                                                      num_q_heads, num_kv_heads, head_dim);
        if (need > 0) {
            if (workspace_bytes < need)
                return PA_ERR_WORKSPACE;
            if (!workspace)
                return PA_ERR_NULL;
            if (!aligned16(workspace))
                return PA_ERR_UNSUPPORTED;
            const size_t items = (need / (2 * pa::kPrefillPartBytes + sizeof(int32_t)));
            a.split = 1;
            a.ws_part = workspace;
            a.ws_cnt = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                   items * 2 * pa::kPrefillPartBytes);
        }
    }
    hipError_t e = pa::launch_prefill(a, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

int pa_prefill_varlen(const void *q, const void *k, const void *v, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                      void *out, hipStream_t stream)
{
    return prefill_impl(q, k, v, k_cache, v_cache, block_tables, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads,
                        num_kv_heads, head_dim, block_size, scale, false, nullptr, 0, out, stream);
}

int pa_prefill_varlen_ws(const void *q, const void *k, const void *v, const void *k_cache,
                         const void *v_cache, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q,
                         const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, float scale, void *workspace,
                         size_t workspace_bytes, void *out, hipStream_t stream)
{
    return prefill_impl(q, k, v, k_cache, v_cache, block_tables, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads,
                        num_kv_heads, head_dim, block_size, scale, true, workspace,
                        workspace_bytes, out, stream);
}

int32_t pa_decode_num_partitions(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t partition_size)
{
    if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_context_len < 0 ||
        partition_size < 0 || partition_size % 32 != 0)
        return 0;
    return num_partitions(max_context_len, resolve_partition(partition_size, num_seqs, num_q_heads,
                                                             num_kv_heads, max_context_len));
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t partition_size)
{
    if (num_q_heads < 1 || head_dim < 1)
        return 0;
    const int32_t np = pa_decode_num_partitions(num_seqs, num_q_heads, num_kv_heads,
                                                max_context_len, partition_size);
    return (size_t)num_seqs * num_q_heads * np * (head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

int decode_passes(const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                  const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  float scale, int32_t partition_size, void *workspace, size_t workspace_bytes,
                  void *out, hipStream_t stream, int passes, const void *k_new = nullptr,
                  const void *v_new = nullptr, const int32_t *slot_mapping = nullptr)
{
    if (num_seqs < 0 || max_context_len < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
        head_dim < 1 || block_size < 1 || max_blocks_per_seq < 1 ||
        num_q_heads % num_kv_heads != 0 || partition_size < 0 || partition_size % 32 != 0)
        return PA_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale))
        return PA_ERR_SHAPE;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return PA_ERR_SHAPE;
    if (head_dim != kHeadDim || !group_supported(num_q_heads, num_kv_heads))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535)
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0)
        return PA_OK;
    const Plan part = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads,
                                        max_context_len);
    if (num_partitions(max_context_len, part) > 65535)
        return PA_ERR_UNSUPPORTED;   // partitions are a grid dimension
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
        return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_UNSUPPORTED;
    const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_context_len, partition_size);
    if (workspace_bytes < need)
        return PA_ERR_WORKSPACE;
    if (need > 0 && !workspace)
        return PA_ERR_NULL;
    if (!aligned16(workspace))
        return PA_ERR_UNSUPPORTED;

    pa::DecodeArgs a;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.n_part = num_partitions(max_context_len, part);
    a.ws_o = static_cast<float *>(workspace);
    a.ws_ml = a.ws_o + (size_t)num_seqs * num_q_heads * a.n_part * head_dim;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.bs_shift = log2_if_pow2(block_size);
    a.part_tokens = part.P;
    a.part_min = part.u;
    // row z of the grid holds sequence (y + seq_rot z) mod S at position y; with
    // S - seq_rot odd, a sequence moves by an odd multiple of Hkv positions modulo 8
    // (its XCD) from one partition row to the next
    a.seq_rot = (num_seqs % 2 == 0) ? 1 : 2;
    a.scale_log2 = scale * pa::kLog2e;
    hipError_t e = pa::launch_decode(a, passes, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

#define PA_DECODE_ARGS                                                                         \
    const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,     \
        int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,            \
        int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, \
        int32_t block_size, float scale, int32_t partition_size, void *workspace,             \
        size_t workspace_bytes, void *out, hipStream_t stream
#define PA_DECODE_FWD                                                                          \
    q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,            \
        max_context_len, num_q_heads, num_kv_heads, head_dim, block_size, scale,              \
        partition_size, workspace, workspace_bytes, out, stream

int pa_decode(PA_DECODE_ARGS) { return decode_passes(PA_DECODE_FWD, 3); }

int pa_decode_store(const void *q, const void *k_new, const void *v_new,
                    const int32_t *slot_mapping, void *k_cache, void *v_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, int32_t partition_size, void *workspace,
                    size_t workspace_bytes, void *out, hipStream_t stream)
{
    if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
        return PA_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new))
        return PA_ERR_UNSUPPORTED;
    return decode_passes(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                         num_seqs, max_context_len, num_q_heads, num_kv_heads, head_dim,
                         block_size, scale, partition_size, workspace, workspace_bytes, out,
                         stream, 3, k_new, v_new, slot_mapping);
}
int pa_decode_split(PA_DECODE_ARGS) { return decode_passes(PA_DECODE_FWD, 1); }
int pa_decode_reduce(PA_DECODE_ARGS) { return decode_passes(PA_DECODE_FWD, 2); }

}  // extern "C"
