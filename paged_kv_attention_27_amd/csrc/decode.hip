// decode.hip -- paged decode attention: one new query per sequence attends
// over its whole history through its block table ("Visual atlas" ch.21
// captions: one decode step; "nano-vLLM offline" course, THE IMPORTANT
// DETAILS item 02: logical blocks map to non-contiguous physical blocks).
//
// Memory-bound split-K design for gfx950:
//   * one workgroup per (KV head, sequence, partition); the partition plan (the
//     keys each partition covers, pa_common.h) and the grid order that spreads
//     the work over the eight XCDs are in sequence_of_block and
//     partition_of_block.  The g = Hq/Hkv
//     query heads of the group share every K/V row the workgroup loads (GQA
//     without a physical repeat, "Visual atlas" ch.18).
//   * decode_split_kernel (groups of 1, 2, 4): a token's 256-byte K row is read
//     by 16 lanes x 16 bytes, so each wave64 load instruction moves four whole
//     rows; a wave iteration covers 4*U keys and keeps 2*U loads per lane in
//     flight.  When the block size and the partition boundaries are multiples of
//     4*U the iteration's keys share one block, found by one scalar table lookup.
//     Scores use v_dot2_f32_bf16 and a 4-step DPP row reduction; weighted values
//     use v_dot2_f32_bf16 over pairs of keys, with the weights rounded to bf16
//     (the same rounding the prefill MFMA applies).
//   * decode_mfma_kernel (groups of 8): both products on MFMA, V through LDS.
//   * The softmax runs online in the log2 domain with a lazily updated running
//     max (rescale only when it grows by more than 2^8).  Each wave keeps its
//     own running max/sum/output; the four waves are merged in LDS.
//   * If a sequence fits in one partition, that workgroup writes the final
//     bf16 output (an empty context writes a zero row); otherwise it writes
//     the partition's running max, sum and unnormalised output row (fp32) to
//     the workspace and
//   * with the fused store, the workgroup holding position ctx-1 takes the new
//     token's K/V from the caller's rows, writes them to their pool slot, and
//     attends to them from registers (no separate store launch, no re-read);
//   * decode_reduce_kernel merges a sequence's partitions with the usual
//     log-sum-exp rescaling: M = max m_p, L = sum 2^(m_p - M) l_p,
//     o = sum 2^(m_p - M) o_p / L.
// Keys at or past context_lens[s] are never loaded, so stale pool slots
// (a free block is not cleared, "Visual atlas" ch.25) cannot reach the output.
#include "pa_common.h"

#include <type_traits>

namespace pa {
namespace {

constexpr int D = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kLazyTau = 8.0f;   // log2 growth of a running max tolerated before rescaling

// v[i] += v[i] from the lane the DPP control CTRL selects, for N independent values
template <int CTRL, int N>
__device__ __forceinline__ void dpp_add_all(float *v)
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                    0, __builtin_bit_cast(int, v[i]), CTRL, 0xF, 0xF, false));
}

// row16_sum of N independent values, one DPP step across all of them at a time
// (each lane of a 16-lane row ends with the row's bit-identical total)
template <int N>
__device__ __forceinline__ void row16_sum_all(float *v)
{
    dpp_add_all<0xB1, N>(v);    // quad_perm [1,0,3,2]
    dpp_add_all<0x4E, N>(v);    // quad_perm [2,3,0,1]
    dpp_add_all<0x141, N>(v);   // row_half_mirror
    dpp_add_all<0x140, N>(v);   // row_mirror
}

// The partition this workgroup reduces.  Grid = (KV head, sequence row, partition
// row).  Workgroups go to the eight XCDs round-robin by linear id, so the partition
// row is the slowest dimension (XCD = (kvh + Hkv y + Hkv S z) mod 8 spreads every
// row over all XCDs), and the sequence of a row is rotated by the row index so that
// a sequence's partitions visit different XCDs (a fixed (sequence, head) -> XCD map
// left the XCDs 10-15 % apart on ragged lengths).  The sequence follows from the
// grid position alone, so a workgroup can load its queries before its context
// length arrives.
__device__ __forceinline__ int sequence_of_block(const DecodeArgs &a)
{
    return (int)((blockIdx.y + (uint32_t)a.seq_rot * blockIdx.z) % (uint32_t)a.num_seqs);
}

// With shrinking partitions, row z holds partition p = z - (n_part - n_s) of a
// sequence with n_s of them, so the last rows launched are every sequence's small
// tail.  Returns false if the sequence has no partition in this row.
__device__ __forceinline__ bool partition_of_block(const DecodeArgs &a, int ctx, int &p, int &n_s)
{
    const int z = (int)blockIdx.z;
    n_s = plan_count(ctx, a.part_tokens, a.part_min);
    p = a.part_min ? z - (a.n_part - n_s) : z;
    return p >= 0 && p < n_s;
}

template <int G, int U, bool CHUNK_IN_BLOCK, bool FUSED_STORE>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a)
{
    const int s = sequence_of_block(a);
    const int kvh = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int r = lane >> 4;   // lane group: which of the four rows a load instruction covers
    const int c = lane & 15;   // 8-element slice of the head dimension
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;

    // q in the dot-product layout: lane c of every lane group holds q[8c .. 8c+8)
    // (issued first: the loads overlap the context-length load)
    const bf16 *q = static_cast<const bf16 *>(a.q);
    uint32_t qw[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uint4 v = *reinterpret_cast<const uint4 *>(q + ((int64_t)s * Hq + kvh * G + h) * D + 8 * c);
        qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
    }

    const int ctx = a.context_lens[s];
    int p, n_part_s, t_begin, t_end;
    if (!partition_of_block(a, ctx, p, n_part_s))
        return;
    if (ctx <= 0) {   // empty context: a zero output row, defined by the C-ABI
        uint16_t *out = static_cast<uint16_t *>(a.out) + ((int64_t)s * a.num_q_heads + kvh * G) * D;
        for (int i = threadIdx.x; i < G * D; i += kThreads)
            out[i] = 0;
        return;
    }
    plan_range(p, ctx, a.part_tokens, a.part_min, t_begin, t_end);
    // fused store: the partition holding position ctx-1 takes the new token's K/V
    // from k_new/v_new (and writes it to its slot) instead of reading the pool
    int new_slot = -1;
    if (FUSED_STORE && t_end == ctx)
        new_slot = a.slot_mapping[s];
    const int t_stop = new_slot >= 0 ? ctx - 1 : t_end;   // keys read from the pool

    __shared__ float red_m[kWaves][G];
    __shared__ float red_l[kWaves][G];
    __shared__ float red_o[kWaves][G][D];

    const int bs = a.block_size, shift = a.bs_shift;
    const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
    const int64_t row_elems = (int64_t)Hkv * D;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kMaxFloor;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    const bf16 *kc = static_cast<const bf16 *>(a.k_cache);
    const bf16 *vc = static_cast<const bf16 *>(a.v_cache);
    const float sl2 = a.scale_log2;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    constexpr int kChunk = 4 * U;   // keys per wave iteration (lane group r owns U consecutive keys)
    const int n_chunks = (t_stop - t_begin + kChunk - 1) / kChunk;
    const int64_t lane_off = (int64_t)(r * U) * row_elems + kvh * D + 8 * c;

    // every K/V byte is read once: nontemporal loads (measured on MI355X: a plain
    // 2 GiB streaming read goes from ~6.1 to ~7.0 TB/s with the hint)
    auto ld = [](const bf16 *p) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    };
    for (int ch = wave; ch < n_chunks; ch += kWaves) {
        const int cs = t_begin + ch * kChunk;
        const int base = cs + r * U;
        uint4 kr[U], vr[U];
        if (CHUNK_IN_BLOCK) {
            // the whole chunk lies in one block: one (scalar) table lookup
            const int lb = __builtin_amdgcn_readfirstlane(shift >= 0 ? (cs >> shift) : (cs / bs));
            const int64_t row0 = (int64_t)__builtin_amdgcn_readfirstlane(bt_row[lb]) * bs + (cs - lb * bs);
            const bf16 *kb = kc + row0 * row_elems + lane_off;
            const bf16 *vb = vc + row0 * row_elems + lane_off;
            // all K rows first, then all V rows: the scores need only K, so they can start
            // while the V rows are still in flight, and K and V requests (same offsets in
            // two pools) are not interleaved (measured ~4 % faster in a read-only probe)
#pragma unroll
            for (int u = 0; u < U; ++u)
                kr[u] = base + u < t_stop ? ld(kb + u * row_elems) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < U; ++u)
                vr[u] = base + u < t_stop ? ld(vb + u * row_elems) : make_uint4(0, 0, 0, 0);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u;
                if (j < t_stop) {
                    const int lb = shift >= 0 ? (j >> shift) : (j / bs);
                    const int64_t off = ((int64_t)bt_row[lb] * bs + (j - lb * bs)) * row_elems + kvh * D + 8 * c;
                    kr[u] = ld(kc + off);
                    vr[u] = ld(vc + off);
                } else {
                    kr[u] = make_uint4(0, 0, 0, 0);
                    vr[u] = make_uint4(0, 0, 0, 0);
                }
            }
        }

        // raw scores q.k (all 16 lanes of a group hold the bit-identical total).  The
        // partial dot products of every key and head are formed first and then reduced
        // one DPP step at a time across all of them, so the steps' latencies overlap
        // (summed whatever the key's validity: its lanes hold zeros then).
        float sc[G][U];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d0 = 0.f, d1 = 0.f;
                d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][0]),
                                                     __builtin_bit_cast(bf16x2, kr[u].x), d0, false);
                d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][1]),
                                                     __builtin_bit_cast(bf16x2, kr[u].y), d1, false);
                d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][2]),
                                                     __builtin_bit_cast(bf16x2, kr[u].z), d0, false);
                d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][3]),
                                                     __builtin_bit_cast(bf16x2, kr[u].w), d1, false);
                sc[h][u] = d0 + d1;
            }
        row16_sum_all<G * U>(&sc[0][0]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = base + u < t_stop;
#pragma unroll
            for (int h = 0; h < G; ++h) sc[h][u] = valid ? sc[h][u] : -INFINITY;
        }

        // lazy running max: rescale only when some head's max grew by more than 2^8
        bool grow_any = false;
        float mcand[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = sc[h][0];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[h][u]);
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            mcand[h] = mx * sl2;
            grow_any |= mcand[h] > m[h] + kLazyTau;
        }
        if (grow_any) {   // wave-uniform: the maxima are reduced over the whole wave
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mnew = fmaxf(m[h], mcand[h]);
                const float alpha = fast_exp2(m[h] - mnew);
                m[h] = mnew;
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
            }
        }

        // weighted values, two keys at a time: v_dot2 over (p_u, p_u+1) x (v_u, v_u+1)
#pragma unroll
        for (int u = 0; u < U; u += 2) {
            uint32_t vlo[4], vhi[4];
            const uint32_t w0[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
            const uint32_t w1[4] = {vr[u + 1].x, vr[u + 1].y, vr[u + 1].z, vr[u + 1].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                vlo[w] = __builtin_amdgcn_perm(w1[w], w0[w], 0x05040100u);   // (v_u[2w],   v_u+1[2w])
                vhi[w] = __builtin_amdgcn_perm(w1[w], w0[w], 0x07060302u);   // (v_u[2w+1], v_u+1[2w+1])
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p0 = fast_exp2(fmaf(sc[h][u], sl2, -m[h]));
                const float p1 = fast_exp2(fmaf(sc[h][u + 1], sl2, -m[h]));
                const bf16x2 pp = {(bf16)p0, (bf16)p1};
                l[h] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l[h], false);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc[h][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, vlo[w]),
                                                                    acc[h][2 * w], false);
                    acc[h][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, vhi[w]),
                                                                        acc[h][2 * w + 1], false);
                }
            }
        }
    }

    if (FUSED_STORE && new_slot >= 0 && wave == 0) {
        // the new token: K/V from k_new/v_new, stored to its slot by lane group 0
        const int64_t src = ((int64_t)s * Hkv + kvh) * D + 8 * c;
        const uint4 kn = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(a.k_new) + src);
        const uint4 vn = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(a.v_new) + src);
        if (r == 0) {
            const int64_t dst = ((int64_t)new_slot * Hkv + kvh) * D + 8 * c;
            *reinterpret_cast<uint4 *>(static_cast<bf16 *>(const_cast<void *>(a.k_cache)) + dst) = kn;
            *reinterpret_cast<uint4 *>(static_cast<bf16 *>(const_cast<void *>(a.v_cache)) + dst) = vn;
        }
        const float vf[8] = {bf16_lo(vn.x), bf16_hi(vn.x), bf16_lo(vn.y), bf16_hi(vn.y),
                             bf16_lo(vn.z), bf16_hi(vn.z), bf16_lo(vn.w), bf16_hi(vn.w)};
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float d0 = 0.f;
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][0]), __builtin_bit_cast(bf16x2, kn.x), d0, false);
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][1]), __builtin_bit_cast(bf16x2, kn.y), d0, false);
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][2]), __builtin_bit_cast(bf16x2, kn.z), d0, false);
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][3]), __builtin_bit_cast(bf16x2, kn.w), d0, false);
            const float sc_new = row16_sum(d0) * sl2;     // identical in all four lane groups
            const float mnew = fmaxf(m[h], sc_new);
            const float alpha = fast_exp2(m[h] - mnew);
            m[h] = mnew;
            const float pw = r == 0 ? fast_exp2(sc_new - mnew) : 0.f;   // counted once
            l[h] = fmaf(l[h], alpha, pw);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(acc[h][e], alpha, pw * vf[e]);
        }
    }

    // merge the four lane groups of the wave (they share the running max)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] += shfl_xor_f(l[h], 16);
        l[h] += shfl_xor_f(l[h], 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += shfl_xor_f(acc[h][e], 16);
            acc[h][e] += shfl_xor_f(acc[h][e], 32);
        }
    }
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[wave][h][8 * c + e] = acc[h][e];
            if (c == 0) {
                red_m[wave][h] = m[h];
                red_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();

    // merge the waves and emit the partition's result
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, dd = idx % D;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(red_m[w][h] - M);
            L = fmaf(f, red_l[w][h], L);
            o = fmaf(f, red_o[w][h][dd], o);
        }
        const int head = kvh * G + h;
        if (n_part_s == 1) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
            out[((int64_t)s * Hq + head) * D + dd] = f32_to_bf16_bits(o / L);
        } else {
            const int64_t slot = ((int64_t)s * Hq + head) * a.n_part + p;
            a.ws_o[slot * D + dd] = o;
            if (dd == 0) {
                a.ws_ml[slot * 2 + 0] = M;
                a.ws_ml[slot * 2 + 1] = L;
            }
        }
    }
}

// ----------------------------------------------------------------------------
// Decode for groups of 8 Q heads: both products on MFMA.
//
// The dot-product kernel above costs VALU work per key in proportion to the group
// size (the weighted values alone are 9 v_dot2 per key pair and head): about 19
// wave instructions per key for a group of 8 even with MFMA scores, against ~39
// per key and CU at the HBM rate, so it cannot overlap its loads well (measured on
// MI355X: 256 ragged contexts at Hq 8 / Hkv 1 took 74 us there, 65 us here; for
// groups of 4 the dot-product kernel, at three workgroups per CU, was as fast or
// faster).  Here each wave step takes 32 keys:
//   S = K Q^T   v_mfma_f32_16x16x32_bf16, A = K rows straight from global memory
//               (lane l: key 16 kb + l%16, head-dim 32 q4 + 8 (l/16) .. +8),
//               B = Q^T in registers (column n = head, zero past G); lane l ends
//               with head l%16 and keys 16 kb + 4 (l/16) + i.
//   O^T += V^T P^T   same instruction, M = 16 head-dim rows per tile (8 tiles),
//               K = the 32 keys in the order slot 8 g + j -> key 4 g + j (j < 4),
//               16 + 4 g + j - 4 (j >= 4), which is exactly the order in which lane
//               l = 16 g + n already holds its weights (no shuffle); the A operand
//               V^T comes from the V rows staged in LDS through the transposing
//               ds_read_b64_tr_b16 (a 16-lane group reads a 4-row x 16-column
//               block, lane i receiving column i of the 4 rows).
// V rows reach LDS by DMA (buffer_load ... lds / global_load_lds, no registers),
// each wave owning two 8 KB stages: the K loads and V copies of the wave's next
// step are issued before the current step computes, so one step's loads are
// always in flight.  Rows are 256 B, 16-byte chunk c of row r stored at
// c ^ (4 (r mod 4) + (r div 4) mod 4), which keeps the transposing reads of 4
// rows x 32 B free of bank conflicts.  Keys past the last one re-read it (finite
// values, masked to weight 0).  Each lane keeps the softmax state of one head
// (lane mod 16); weights are rounded to bf16 for the MFMA and the sum, as in the
// dot-product kernel.  Partials and outputs have the dot-product kernel's format,
// so decode_reduce_kernel merges either.  With the steps inside blocks, the
// block-table entries of the partition's first 64 blocks are read once, one per
// lane, and each step takes its entry from that register (v_readlane) instead of
// a scalar load in front of its K/V loads (measured on MI355X: 256 ragged
// contexts at Hq 8 / Hkv 1, 62.4 -> 61.1 us per step launched directly; the
// dot-product kernels gained nothing from the same change).
constexpr int kMStep = 32;                 // keys per wave step
constexpr int kMStageB = kMStep * 2 * D;   // 8 KB of V rows

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ int vswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}

// the table entries of blocks lb0 .. lb0 + 63 of a row, one per lane, clamped to
// blocks lb0 .. lb_last (those that hold the keys read)
__device__ __forceinline__ int32_t table_window(const int32_t *bt_row, int lb0, int lb_last)
{
    const int lane = threadIdx.x & (kWave - 1);
    return bt_row[lb0 + min(lane, max(lb_last - lb0, 0))];
}

// entry of block lb (wave-uniform): from the window when it covers lb, else a load
__device__ __forceinline__ int32_t table_entry(const int32_t *bt_row, int32_t win, int lb0, int lb)
{
    const int rel = lb - lb0;
    return rel < kWave ? __builtin_amdgcn_readlane(win, rel) : __builtin_amdgcn_readfirstlane(bt_row[lb]);
}

// merge the four waves' (m, l, o) of each head and emit the partition's result:
// the final bf16 row when the context is one partition, else the fp32 partial
template <int G>
__device__ __forceinline__ void emit_partition(const DecodeArgs &a, int s, int kvh, int p,
                                               int n_part_s, const float (*red_m)[G],
                                               const float (*red_l)[G], const float *red_o,
                                               int red_o_wave_stride)
{
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int h = idx / D, dd = idx % D;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(red_m[w][h] - M);
            L = fmaf(f, red_l[w][h], L);
            o = fmaf(f, red_o[w * red_o_wave_stride + h * D + dd], o);
        }
        const int head = kvh * G + h;
        if (n_part_s == 1) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
            out[((int64_t)s * a.num_q_heads + head) * D + dd] = f32_to_bf16_bits(o / L);
        } else {
            const int64_t slot = ((int64_t)s * a.num_q_heads + head) * a.n_part + p;
            a.ws_o[slot * D + dd] = o;
            if (dd == 0) {
                a.ws_ml[slot * 2 + 0] = M;
                a.ws_ml[slot * 2 + 1] = L;
            }
        }
    }
}

template <int G, bool CHUNK_IN_BLOCK, bool FUSED_STORE>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeArgs a)
{
    static_assert(G <= 16, "heads of a group fill the 16 MFMA columns");
    const int s = sequence_of_block(a);
    const int kvh = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: descriptors and M0
    const int g = lane >> 4;     // 16-lane group
    const int col = lane & 15;   // head column of the score / output accumulators
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const bf16 *q = static_cast<const bf16 *>(a.q);

    // B operand of the scores: lane l holds Q[head l%16][32 q4 + 8 (l/16) .. +8]
    // (issued first: the loads overlap the context-length load)
    bf16x8 qt[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
        qt[q4] = col < G ? *reinterpret_cast<const bf16x8 *>(q + ((int64_t)s * Hq + kvh * G + col) * D +
                                                               32 * q4 + 8 * g)
                         : bf16x8{};

    const int ctx = a.context_lens[s];
    int p, n_part_s, t_begin, t_end;
    if (!partition_of_block(a, ctx, p, n_part_s))
        return;
    if (ctx <= 0) {   // empty context: a zero output row, defined by the C-ABI
        uint16_t *out = static_cast<uint16_t *>(a.out) + ((int64_t)s * a.num_q_heads + kvh * G) * D;
        for (int i = threadIdx.x; i < G * D; i += kThreads)
            out[i] = 0;
        return;
    }
    plan_range(p, ctx, a.part_tokens, a.part_min, t_begin, t_end);
    int new_slot = -1;
    if (FUSED_STORE && t_end == ctx)
        new_slot = a.slot_mapping[s];
    const int t_stop = new_slot >= 0 ? ctx - 1 : t_end;   // keys read from the pool

    __shared__ __attribute__((aligned(16))) char vst0[kWaves][kMStageB];
    __shared__ __attribute__((aligned(16))) char vst1[kWaves][kMStageB];

    const int bs = a.block_size, shift = a.bs_shift;
    const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
    const int64_t row_elems = (int64_t)Hkv * D;
    const uint32_t row_bytes = (uint32_t)row_elems * 2;
    const bf16 *kc = static_cast<const bf16 *>(a.k_cache);
    const bf16 *vc = static_cast<const bf16 *>(a.v_cache);
    const float sl2 = a.scale_log2;

    // transposing-read offsets within a stage: tile t covers head-dim 16 t .. 16 t + 15;
    // lane i of group g reads row 4 g + i/4 (and 16 rows further), columns 16 t + 4 (i%4) .. +4
    const int tr_row = 4 * g + (col >> 2);
    int toff[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
        toff[t] = tr_row * 2 * D + 16 * ((2 * t + ((col & 3) >> 1)) ^ vswz(tr_row)) + 8 * (col & 1);

    float m = kMaxFloor, l = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4{};

    const int n_steps = (t_stop - t_begin + kMStep - 1) / kMStep;
    const int n_mine = n_steps > wave ? (n_steps - wave + kWaves - 1) / kWaves : 0;
    const int lb0 = shift >= 0 ? (t_begin >> shift) : (t_begin / bs);
    int32_t win = 0;
    if (CHUNK_IN_BLOCK && t_stop > t_begin)
        win = table_window(bt_row, lb0, shift >= 0 ? ((t_stop - 1) >> shift) : ((t_stop - 1) / bs));

    // issue step j's K loads (into kf) and V copies (into the stage)
    auto issue = [&](int j, uint4 (&kf)[2][4], char *stage) __attribute__((always_inline)) {
        const int cs = t_begin + (wave + kWaves * j) * kMStep;
        const int last = t_stop - 1 - cs;   // >= 0: last valid key of the step
        if (CHUNK_IN_BLOCK) {
            // the step's 32 keys are consecutive rows of one block
            const int lb = __builtin_amdgcn_readfirstlane(shift >= 0 ? (cs >> shift) : (cs / bs));
            const int64_t row0 = (int64_t)table_entry(bt_row, win, lb0, lb) * bs + (cs - lb * bs);
            const __amdgpu_buffer_rsrc_t kr = rsrc_of(kc + row0 * row_elems + kvh * D);
            const __amdgpu_buffer_rsrc_t vr = rsrc_of(vc + row0 * row_elems + kvh * D);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint32_t o = (uint32_t)min(16 * kb + col, last) * row_bytes + 16 * g;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, o + 64 * q4, 0, 2));
                    kf[kb][q4] = make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + g;
                const uint32_t o = (uint32_t)min(r, last) * row_bytes + 16 * (col ^ vswz(r));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(stage + 1024 * i), 16, o, 0, 0, 2);
            }
        } else {
            auto row_of = [&](int key) {
                const int lb = shift >= 0 ? (key >> shift) : (key / bs);
                return ((int64_t)bt_row[lb] * bs + (key - lb * bs)) * row_elems + kvh * D;
            };
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16 *src = kc + row_of(cs + min(16 * kb + col, last)) + 8 * g;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + 32 * q4));
                    kf[kb][q4] = make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + g;
                const bf16 *src = vc + row_of(cs + min(r, last)) + 8 * (col ^ vswz(r));
                __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)(stage + 1024 * i), 16, 0, 0);
            }
        }
    };

    // step j from kf and the stage; PENDING = memory operations issued after it
    auto compute = [&](auto pending, int j, const uint4 (&kf)[2][4], const char *stage) __attribute__((always_inline)) {
        constexpr int kPending = decltype(pending)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70 | kPending);   // vmcnt(kPending): this step's copies landed
        const int cs = t_begin + (wave + kWaves * j) * kMStep;
        f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kf[kb][q4]), qt[q4], sacc[kb], 0, 0, 0);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cs + 16 * kb + 4 * g + i >= t_stop) sacc[kb][i] = -INFINITY;
                mx = fmaxf(mx, sacc[kb][i]);
            }
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float mc = mx * sl2;   // this lane's head: maximum over the step, log2 domain
        if (__builtin_amdgcn_ballot_w64(mc > m + kLazyTau)) {
            const float mnew = mc > m + kLazyTau ? mc : m;
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[t] *= alpha;
        }
        // weights in the slot order 8 g + j: keys 4 g + j, then 16 + 4 g + j
        bf16x8 pb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pb[4 * kb + i] = (bf16)fast_exp2(fmaf(sacc[kb][i], sl2, -m));
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2 * i], pb[2 * i + 1]}, ones, l, false);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(stage + toff[t]));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(stage + toff[t] + 16 * 2 * D));
            const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[t], 0, 0, 0);
        }
    };

    if (n_mine > 0) {
        uint4 ka[2][4], kb_[2][4];
        char *sa = vst0[wave];
        char *sb = vst1[wave];
        issue(0, ka, sa);
        for (int j = 0;;) {
            if (j + 1 < n_mine) {
                issue(j + 1, kb_, sb);
                compute(std::integral_constant<int, 16>{}, j, ka, sa);
            } else {
                compute(std::integral_constant<int, 0>{}, j, ka, sa);
                break;
            }
            ++j;
            if (j + 1 < n_mine) {
                issue(j + 1, ka, sa);
                compute(std::integral_constant<int, 16>{}, j, kb_, sb);
            } else {
                compute(std::integral_constant<int, 0>{}, j, kb_, sb);
                break;
            }
            ++j;
        }
    }

    if (FUSED_STORE && new_slot >= 0 && wave == 0) {
        // the new token: K/V from k_new/v_new (stored to its slot by the col == 0 lanes);
        // this lane's head-dim positions are 16 t + 4 g + i
        const int64_t src = ((int64_t)s * Hkv + kvh) * D;
        const bf16 *kn = static_cast<const bf16 *>(a.k_new) + src;
        const bf16 *vn = static_cast<const bf16 *>(a.v_new) + src;
        const bf16 *qh = q + ((int64_t)s * Hq + kvh * G + min(col, G - 1)) * D;
        float part = 0.f;
        uint2 vv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d0 = 16 * t + 4 * g;
            const uint2 kk = *reinterpret_cast<const uint2 *>(kn + d0);
            const uint2 qq = *reinterpret_cast<const uint2 *>(qh + d0);
            vv[t] = *reinterpret_cast<const uint2 *>(vn + d0);
            part = fmaf(bf16_lo(qq.x), bf16_lo(kk.x), part);
            part = fmaf(bf16_hi(qq.x), bf16_hi(kk.x), part);
            part = fmaf(bf16_lo(qq.y), bf16_lo(kk.y), part);
            part = fmaf(bf16_hi(qq.y), bf16_hi(kk.y), part);
            if (col == 0) {
                const int64_t dst = ((int64_t)new_slot * Hkv + kvh) * D + d0;
                *reinterpret_cast<uint2 *>(static_cast<bf16 *>(const_cast<void *>(a.k_cache)) + dst) = kk;
                *reinterpret_cast<uint2 *>(static_cast<bf16 *>(const_cast<void *>(a.v_cache)) + dst) = vv[t];
            }
        }
        part += shfl_xor_f(part, 16);
        part += shfl_xor_f(part, 32);
        const float sc_new = part * sl2;
        const float mnew = fmaxf(m, sc_new);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        const float pw = fast_exp2(sc_new - mnew);
        l = fmaf(l, alpha, g == 0 ? pw : 0.f);   // counted once per head
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float vf[4] = {bf16_lo(vv[t].x), bf16_hi(vv[t].x), bf16_lo(vv[t].y), bf16_hi(vv[t].y)};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(acc[t][i], alpha, pw * vf[i]);
        }
    }

    // per head: sum the weights of the four lane groups
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    // stage (m, l, o) per wave in LDS, then merge the waves
    __shared__ float red_m[kWaves][G];
    __shared__ float red_l[kWaves][G];
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no copy into this wave's stage in flight
    float *red_o = reinterpret_cast<float *>(vst0[wave]);   // [G][D] of this wave
    if (col < G) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) red_o[col * D + 16 * t + 4 * g + i] = acc[t][i];
        if (g == 0) {
            red_m[wave][col] = m;
            red_l[wave][col] = l;
        }
    }
    __syncthreads();
    emit_partition<G>(a, s, kvh, p, n_part_s, red_m, red_l,
                      reinterpret_cast<const float *>(vst0[0]), kMStageB / 4);
}

constexpr int kReduceThreads = 256;   // two Q heads of one sequence per workgroup
constexpr int kReduceStage = 512;     // partitions staged in LDS per pass
constexpr int kReduceRegParts = 32;   // up to this many partitions: merged in registers

__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeArgs a)
{
    const int hh = threadIdx.x / D;          // which of the workgroup's two heads
    const int dd = threadIdx.x % D;
    const bool active = 2 * (int)blockIdx.x + hh < a.num_q_heads;   // odd Hq: last half idles
    const int h = active ? 2 * blockIdx.x + hh : a.num_q_heads - 1;
    const int s = blockIdx.y;
    const int ctx = a.context_lens[s];
    const int np = plan_count(ctx, a.part_tokens, a.part_min);   // uniform over the workgroup
    if (np == 1)
        return;  // a single partition (or an empty context) wrote the output itself
    uint16_t *out = static_cast<uint16_t *>(a.out) + ((int64_t)s * a.num_q_heads + h) * D + dd;
    const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.n_part;
    const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + base;
    const float *wo = a.ws_o + base * D + dd;

    if (np <= kReduceRegParts) {
        // every load issued at once (the (max, sum) pairs are the same for the 128 threads
        // of a head), then the merge in registers: one memory round trip, no barrier;
        // the same operations in the same order as the staged path below
        float2 mlv[kReduceRegParts];
        float ov[kReduceRegParts];
#pragma unroll
        for (int p = 0; p < kReduceRegParts; ++p)
            if (p < np) {
                mlv[p] = ml[p];
                ov[p] = wo[(int64_t)p * D];
            }
        float M = kMaxFloor;
#pragma unroll
        for (int p = 0; p < kReduceRegParts; ++p)
            if (p < np) M = fmaxf(M, mlv[p].x);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int p = 0; p < kReduceRegParts; ++p)
            if (p < np) {
                const float w = fast_exp2(mlv[p].x - M);
                L = fmaf(w, mlv[p].y, L);
                o = fmaf(w, ov[p], o);
            }
        if (active)
            *out = f32_to_bf16_bits(o / L);
        return;
    }

    // global max over the partitions: every thread of the head scans a slice, then LDS
    __shared__ float red[2][D];
    float M = kMaxFloor;
    for (int p = dd; p < np; p += D) M = fmaxf(M, ml[p].x);
    red[hh][dd] = M;
    __syncthreads();
    for (int w = D / 2; w > 0; w /= 2) {
        if (dd < w) red[hh][dd] = fmaxf(red[hh][dd], red[hh][dd + w]);
        __syncthreads();
    }
    M = red[hh][0];

    // weights 2^(m_p - M) staged in LDS, then independent loads of the partial rows
    __shared__ float2 wl[2][kReduceStage];
    float L = 0.f, o = 0.f;
    for (int p0 = 0; p0 < np; p0 += kReduceStage) {
        const int n = min(kReduceStage, np - p0);
        __syncthreads();
        for (int i = dd; i < n; i += D) {
            const float2 v = ml[p0 + i];
            wl[hh][i] = make_float2(fast_exp2(v.x - M), v.y);
        }
        __syncthreads();
#pragma unroll 8
        for (int i = 0; i < n; ++i) {
            const float2 w = wl[hh][i];
            L = fmaf(w.x, w.y, L);
            o = fmaf(w.x, wo[(int64_t)(p0 + i) * D], o);
        }
    }
    if (active)
        *out = f32_to_bf16_bits(o / L);
}

// every partition boundary is a multiple of `step` keys
bool partitions_aligned(const DecodeArgs &a, int step)
{
    return a.part_min ? 64 % step == 0 : a.part_tokens % step == 0;
}

template <int G, int U, bool FUSED>
void launch_split(const DecodeArgs &a, hipStream_t stream)
{
    // The partition index is the slowest grid dimension.  Workgroups go to the eight
    // XCDs round-robin by linear id, so XCD = (kvh + Hkv s + Hkv S p) mod 8: every XCD
    // gets every eighth (sequence, KV head) pair with all of its partitions.  With the
    // partition fastest, XCD = (p + n_part (kvh + Hkv s)) mod 8 puts all first partitions
    // (present in every sequence) on the same XCDs whenever n_part shares a factor with
    // 8, while later ones (long contexts only) land on others (measured on MI355X: 256
    // ragged contexts at Hkv 1 or 2 and four partitions ran at half the HBM rate).
    dim3 grid(a.num_kv_heads, a.num_seqs, a.n_part);
    if constexpr (G >= 8) {
        // one table lookup per step needs every 32-key step inside one block
        if (a.block_size % kMStep == 0 && partitions_aligned(a, kMStep))
            hipLaunchKernelGGL((decode_mfma_kernel<G, true, FUSED>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<G, false, FUSED>), grid, dim3(kThreads), 0, stream, a);
    } else {
        // one table lookup per iteration needs every 4U-key chunk inside one block
        if (a.block_size % (4 * U) == 0 && partitions_aligned(a, 4 * U))
            hipLaunchKernelGGL((decode_split_kernel<G, U, true, FUSED>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_split_kernel<G, U, false, FUSED>), grid, dim3(kThreads), 0, stream, a);
    }
}

template <int G, int U>
hipError_t launch_g(const DecodeArgs &a, int passes, hipStream_t stream)
{
    if (passes & 1) {
        if (a.slot_mapping)
            launch_split<G, U, true>(a, stream);
        else
            launch_split<G, U, false>(a, stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // with a single partition every row (empty contexts included) is final
    if ((passes & 2) && a.n_part > 1) {
        hipLaunchKernelGGL(decode_reduce_kernel, dim3((a.num_q_heads + 1) / 2, a.num_seqs),
                           dim3(kReduceThreads), 0, stream, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int passes, hipStream_t stream)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1, 16>(a, passes, stream);
    case 2: return launch_g<2, 16>(a, passes, stream);
    case 4: return launch_g<4, 8>(a, passes, stream);
    case 8: return launch_g<8, 8>(a, passes, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
