// decode.hip -- paged decode attention: one new query per sequence attends
// over its whole history through its block table ("Visual atlas" ch.21
// captions: one decode step; "nano-vLLM offline" course, THE IMPORTANT
// DETAILS item 02: logical blocks map to non-contiguous physical blocks).
//
// Memory-bound split-K design for gfx950:
//   * decode_split_kernel: one workgroup per (partition of part_tokens keys,
//     KV head, sequence).  The g = Hq/Hkv query heads of the group share every
//     K/V row the workgroup loads (GQA without a physical repeat, "Visual
//     atlas" ch.18).  A token's 256-byte K row is read by 16 lanes x 16 bytes,
//     so each wave64 load instruction moves four whole rows; a wave iteration
//     covers 4*U keys and keeps 2*U loads per lane in flight.  When the block
//     and partition sizes are multiples of 4*U the iteration's keys share one
//     block, found by one scalar table lookup.  Scores use v_dot2_f32_bf16 and a 4-step DPP row
//     reduction (groups of 8 Q heads: a 16x16x32 bf16 MFMA per 16 keys and 32
//     head-dim elements, the weights then broadcast from the score lanes to
//     their lane groups with DPP row broadcasts); weighted values use
//     v_dot2_f32_bf16 over pairs of keys, with
//     the weights rounded to bf16 (the same rounding the prefill MFMA applies).
//     The softmax runs online in the log2 domain with a lazily updated running
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

// value of lane h (0..7) of this lane's 16-lane row (DPP row_newbcast); h is a
// constant once the caller's loop is unrolled
__device__ __forceinline__ int row_bcast(int v, int h)
{
    switch (h) {
    case 0: return __builtin_amdgcn_update_dpp(0, v, 0x150, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0x151, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x152, 0xF, 0xF, false);
    case 3: return __builtin_amdgcn_update_dpp(0, v, 0x153, 0xF, 0xF, false);
    case 4: return __builtin_amdgcn_update_dpp(0, v, 0x154, 0xF, 0xF, false);
    case 5: return __builtin_amdgcn_update_dpp(0, v, 0x155, 0xF, 0xF, false);
    case 6: return __builtin_amdgcn_update_dpp(0, v, 0x156, 0xF, 0xF, false);
    default: return __builtin_amdgcn_update_dpp(0, v, 0x157, 0xF, 0xF, false);
    }
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

template <int G, int U, bool CHUNK_IN_BLOCK, bool FUSED_STORE>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a)
{
    const int p = blockIdx.x;
    const int kvh = blockIdx.y;
    const int s = blockIdx.z;
    const int ctx = a.context_lens[s];
    const int P = a.part_tokens;
    const int t_begin = p * P;
    if (t_begin >= ctx) {
        if (ctx <= 0 && p == 0) {   // empty context: a zero output row, defined by the C-ABI
            uint16_t *out = static_cast<uint16_t *>(a.out) + ((int64_t)s * a.num_q_heads + kvh * G) * D;
            for (int i = threadIdx.x; i < G * D; i += kThreads)
                out[i] = 0;
        }
        return;
    }
    const int t_end = min(ctx, t_begin + P);
    const int n_part_s = (ctx + P - 1) / P;
    // fused store: the partition holding position ctx-1 takes the new token's K/V
    // from k_new/v_new (and writes it to its slot) instead of reading the pool
    int new_slot = -1;
    if (FUSED_STORE && t_end == ctx)
        new_slot = a.slot_mapping[s];
    const int t_stop = new_slot >= 0 ? ctx - 1 : t_end;   // keys read from the pool

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int r = lane >> 4;   // lane group: which of the four rows a load instruction covers
    const int c = lane & 15;   // 8-element slice of the head dimension

    __shared__ float red_m[kWaves][G];
    __shared__ float red_l[kWaves][G];
    __shared__ float red_o[kWaves][G][D];

    const int bs = a.block_size, shift = a.bs_shift;
    const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int64_t row_elems = (int64_t)Hkv * D;

    const bf16 *q = static_cast<const bf16 *>(a.q);
    // q in the dot-product layout: lane c of every lane group holds q[8c .. 8c+8)
    uint32_t qw[G][4];
    auto load_qw = [&]() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 v = *reinterpret_cast<const uint4 *>(q + ((int64_t)s * Hq + kvh * G + h) * D + 8 * c);
            qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
        }
    };

    // groups of 8 Q heads: the scores are an MFMA, S = K Q^T with 16 keys (M) x 16
    // columns (N: the G heads, the rest zero) x 32 head-dim elements (K) per
    // instruction.  B operand: lane l holds Q[head l%16][32 kq + 8 (l/16) .. +8].
    // (Measured on MI355X: MQA step 135 -> 90 us.  For groups of 4 the dot-product
    // path stays: its K loads read 4 whole rows per instruction where the MFMA
    // layout reads 16 half lines, and the 16 x 32768 decode lost 2 % with it.)
    constexpr bool kMfmaQK = G >= 8;
    bf16x8 qt[4];
    if constexpr (!kMfmaQK) {
        load_qw();
    } else {
        const int hcol = lane & 15;
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
            qt[kq] = hcol < G ? *reinterpret_cast<const bf16x8 *>(
                                    q + ((int64_t)s * Hq + kvh * G + hcol) * D + 32 * kq + 8 * r)
                              : bf16x8{};
    }

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
        if constexpr (kMfmaQK) {
            static_assert(U == 8, "the MFMA score path takes 32-key chunks");
            // K as the MFMA A operand: for key half kb and head-dim chunk q4, lane l holds
            // K[key cs + 16 kb + l%16][32 q4 + 8 (l/16) .. +8] (one instruction reads 16 rows
            // x 64 contiguous bytes).  V in the weighting layout: lane group r owns keys
            // 4r + i and 16 + 4r + i (i < 4), the same keys the score accumulators of its
            // rows hold, so the weights move to it with row broadcasts.
            const int kl = lane & 15;
            uint4 kf[2][4], vr[8];
            auto vkey = [&](int u) { return (u & 3) + 4 * r + 16 * (u >> 2); };
            if (CHUNK_IN_BLOCK) {
                const int lb = __builtin_amdgcn_readfirstlane(shift >= 0 ? (cs >> shift) : (cs / bs));
                const int64_t row0 = (int64_t)__builtin_amdgcn_readfirstlane(bt_row[lb]) * bs + (cs - lb * bs);
                const bf16 *kb0 = kc + row0 * row_elems + kvh * D;
                const bf16 *vb0 = vc + row0 * row_elems + kvh * D + 8 * c;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        kf[kb][q4] = cs + 16 * kb + kl < t_stop
                                         ? ld(kb0 + (16 * kb + kl) * row_elems + 32 * q4 + 8 * r)
                                         : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    vr[u] = cs + vkey(u) < t_stop ? ld(vb0 + vkey(u) * row_elems) : make_uint4(0, 0, 0, 0);
            } else {
                auto row_of = [&](int j) {
                    const int lb = shift >= 0 ? (j >> shift) : (j / bs);
                    return ((int64_t)bt_row[lb] * bs + (j - lb * bs)) * row_elems + kvh * D;
                };
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int j = cs + 16 * kb + kl;
                    const int64_t o = j < t_stop ? row_of(j) : 0;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        kf[kb][q4] = j < t_stop ? ld(kc + o + 32 * q4 + 8 * r) : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = cs + vkey(u);
                    vr[u] = j < t_stop ? ld(vc + row_of(j) + 8 * c) : make_uint4(0, 0, 0, 0);
                }
            }

            // scores: lane l holds S[key cs + 16 kb + 4 (l/16) + i][head l%16], i < 4
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
                    if (cs + 16 * kb + 4 * r + i >= t_stop) sacc[kb][i] = -INFINITY;
                    mx = fmaxf(mx, sacc[kb][i]);
                }
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            // lanes h, h+16, h+32, h+48 now hold head h's chunk maximum
            bool grow_any = false;
            float mcand[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                mcand[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), h)) * sl2;
                grow_any |= mcand[h] > m[h] + kLazyTau;
            }
            if (grow_any) {   // wave-uniform: the maxima are read from lanes
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
            // weights in the score layout (this lane's head is l%16; columns past G unused),
            // rounded to bf16 in pairs of consecutive keys
            float mh = m[0];
#pragma unroll
            for (int h = 1; h < G; ++h) mh = kl == h ? m[h] : mh;
            uint32_t pw[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const float p0 = fast_exp2(fmaf(sacc[kb][2 * pr], sl2, -mh));
                    const float p1 = fast_exp2(fmaf(sacc[kb][2 * pr + 1], sl2, -mh));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    pw[kb][pr] = __builtin_bit_cast(uint32_t, pp);
                }
            // weighted values: keys (u, u+1) = (4 kb + 2 pr, +1) of this lane group; the
            // weights of head h come from lane h of the row (DPP row broadcast)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int u = 4 * kb + 2 * pr;
                    uint32_t vlo[4], vhi[4];
                    const uint32_t w0[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
                    const uint32_t w1[4] = {vr[u + 1].x, vr[u + 1].y, vr[u + 1].z, vr[u + 1].w};
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        vlo[w] = __builtin_amdgcn_perm(w1[w], w0[w], 0x05040100u);
                        vhi[w] = __builtin_amdgcn_perm(w1[w], w0[w], 0x07060302u);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const bf16x2 pp = __builtin_bit_cast(bf16x2, row_bcast((int)pw[kb][pr], h));
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
            continue;
        }
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
        if constexpr (kMfmaQK)
            load_qw();
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

constexpr int kReduceThreads = 256;   // two Q heads of one sequence per workgroup
constexpr int kReduceStage = 512;     // partitions staged in LDS per pass

__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeArgs a)
{
    const int hh = threadIdx.x / D;          // which of the workgroup's two heads
    const int dd = threadIdx.x % D;
    const bool active = 2 * (int)blockIdx.x + hh < a.num_q_heads;   // odd Hq: last half idles
    const int h = active ? 2 * blockIdx.x + hh : a.num_q_heads - 1;
    const int s = blockIdx.y;
    const int ctx = a.context_lens[s];
    const int np = (ctx + a.part_tokens - 1) / a.part_tokens;   // uniform over the workgroup
    if (np == 1)
        return;  // a single partition wrote the output itself
    uint16_t *out = static_cast<uint16_t *>(a.out) + ((int64_t)s * a.num_q_heads + h) * D + dd;
    if (np <= 0) {
        if (active)
            *out = 0;  // empty context: defined as a zero row
        return;
    }
    const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.n_part;
    const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + base;
    const float *wo = a.ws_o + base * D + dd;

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

template <int G, int U, bool FUSED>
void launch_split(const DecodeArgs &a, hipStream_t stream)
{
    dim3 grid(a.n_part, a.num_kv_heads, a.num_seqs);
    // one table lookup per iteration needs every 4U-key chunk inside one block
    if (a.block_size % (4 * U) == 0 && a.part_tokens % (4 * U) == 0)
        hipLaunchKernelGGL((decode_split_kernel<G, U, true, FUSED>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<G, U, false, FUSED>), grid, dim3(kThreads), 0, stream, a);
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
