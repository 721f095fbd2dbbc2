// pa_common.h -- device helpers and launcher declarations shared by the HIP
// kernels of libpa.so (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
// Running-max floor: finite, so an all-masked row gives exp2(floor - floor) = 1
// for the rescale factor and exp2(-inf - floor) = 0 for every weight.
constexpr float kMaxFloor = -3.0e38f;

// bf16 pair packed in a 32-bit word -> two fp32 values (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the same
// bit-exact total (each step adds a value to its mirror, which commutes).
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0xB1, 0xF, 0xF, false)); // quad_perm [1,0,3,2]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x4E, 0xF, 0xF, false)); // quad_perm [2,3,0,1]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x141, 0xF, 0xF, false)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x140, 0xF, 0xF, false)); // row_mirror
    return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are pre-validated.

hipError_t launch_store_kv(const void *k, const void *v, void *k_cache, void *v_cache,
                           const int32_t *slot_mapping, int32_t num_tokens,
                           int32_t row_elems, hipStream_t stream);

struct DecodeArgs {
    const void *q;
    const void *k_new;            // fused store: new token rows [S, Hkv, D] (or null)
    const void *v_new;
    const int32_t *slot_mapping;  // fused store: pool row of each sequence's new token
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    void *out;
    float *ws_o;      // [S, Hq, n_part, head_dim] unnormalised partial outputs
    float *ws_ml;     // [S, Hq, n_part, 2] running max (log2 domain) and sum
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t bs_shift;   // log2(block_size) if a power of two, else -1
    int32_t part_tokens;   // P: the largest partition (see plan_count)
    int32_t part_min;      // 0: fixed partitions; else the smallest tail partition
    int32_t n_part;        // plan_count(max_context_len): grid depth and partial slots
    int32_t seq_rot;       // grid-to-sequence rotation per partition row (XCD balance)
    float scale_log2;   // scale * log2(e)
};

// ------------------------------------------------ decode partition plan
// How the n keys of one sequence are split into partitions, each reduced to one
// partial by one workgroup.
//  * part_min == 0: fixed partitions [p P, (p + 1) P), ceil(n / P) of them.
//  * part_min = u > 0 (u a multiple of 64, P = u 2^k, k >= 1): partitions shrink
//    toward the end of the key range.  Counted from the end of n64 = n rounded
//    up to 64, their sizes are u, u, 2u, 2u, ..., P/2, P/2 (the tail, 2 (P - u)
//    keys), then P up to the start, where the first partition takes what is
//    left.  A grid of fixed-size partitions ends with a wave of full-size
//    workgroups that run nearly alone; here the last workgroups launched are small.
// Every boundary of the second kind is a multiple of 64 keys; a sequence with
// n <= 0 has one (empty) partition.
__host__ __device__ inline int32_t plan_tail_size(int32_t j, int32_t u) { return u << (j >> 1); }

__host__ __device__ inline int32_t plan_count(int32_t n, int32_t P, int32_t u)
{
    if (n <= 0)
        return 1;
    if (u == 0)
        return (int32_t)(((int64_t)n + P - 1) / P);
    const int64_t n64 = ((int64_t)n + 63) / 64 * 64;
    const int64_t T = 2 * ((int64_t)P - u);
    if (n64 > T) {
        int32_t nt = 0;
        for (int32_t v = u; v < P; v *= 2) nt += 2;
        return (int32_t)((n64 - T + P - 1) / P) + nt;
    }
    int64_t c = 0;
    int32_t m = 0;
    while (c < n64) c += plan_tail_size(m++, u);
    return m;
}

// keys [b, e) of partition p (0 <= p < plan_count) of a sequence of n > 0 keys
__host__ __device__ inline void plan_range(int32_t p, int32_t n, int32_t P, int32_t u, int32_t &b,
                                           int32_t &e)
{
    if (u == 0) {
        b = p * P;
        e = (int32_t)((int64_t)b + P < n ? b + P : n);
        return;
    }
    const int64_t n64 = ((int64_t)n + 63) / 64 * 64;
    const int64_t T = 2 * ((int64_t)P - u);
    const int32_t cnt = plan_count(n, P, u);
    int64_t ee, bb;
    int32_t nt = 0;
    for (int32_t v = u; v < P; v *= 2) nt += 2;
    const int32_t nh = n64 > T ? cnt - nt : 0;   // full-size partitions ahead of the tail
    if (p < nh) {
        ee = n64 - T - (int64_t)(nh - 1 - p) * P;
        bb = ee - P;
    } else {
        const int32_t j = cnt - 1 - p;             // tail index, 0 = the last partition
        int64_t c = 0;
        for (int32_t i = 0; i < j; ++i) c += plan_tail_size(i, u);
        ee = n64 - c;
        bb = ee - plan_tail_size(j, u);
    }
    b = (int32_t)(bb > 0 ? bb : 0);
    e = (int32_t)(ee < n ? ee : n);
}
// passes: bit 0 = partition (split) pass, bit 1 = reduce pass
hipError_t launch_decode(const DecodeArgs &a, int passes, hipStream_t stream);

struct PrefillArgs {
    const void *q;
    const void *k;        // flat source (paged == false)
    const void *v;
    const void *k_cache;  // paged source (paged == true)
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *cu_seqlens_q;
    const int32_t *cu_seqlens_k;
    void *out;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t max_seqlen_q;
    int32_t max_seqlen_k;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t bs_shift;
    bool paged;
    float scale_log2;
    // key-split mode (split != 0): an item with at least kPrefillMinSplitTiles key tiles
    // is computed as two halves of its key range by two workgroups; each half stores
    // its partial in ws_part and the second to arrive (counter ws_cnt) merges them
    int32_t split;
    void *ws_part;      // [items][2] partials of kPrefillPartBytes each
    int32_t *ws_cnt;    // [items] arrival counters; zero between calls
};
// bytes of one half's partial: O / l as fp32 [4 waves][64][64 lanes], then the column max
// and sum as fp32 [4 waves][2][64 lanes]
constexpr size_t kPrefillPartBytes = (4 * 64 * 64 + 4 * 2 * 64) * 4;
constexpr int kPrefillMinSplitTiles = 4;
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
// items of a batch of these sizes that key-split mode would cover on the current
// device (0: the batch is not split)
int64_t prefill_split_items(int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t num_q_heads, int32_t num_kv_heads);

}  // namespace pa
