// prefill.hip -- variable-length causal prefill attention with GQA and a
// position-offset mask, on bf16 MFMA (v_mfma_f32_32x32x16_bf16, gfx950).
//
// Problem ("Visual atlas" ch.16 captions: scores -> causal softmax -> weighted
// V, one probability row per query; ch.17: diagonal kept, and a cached chunk's
// [q_len, k_len] mask carries the offset k_len - q_len; ch.26: sequences are
// flattened through cu_seqlens and, after a prefix hit, read their keys from
// the cache).  Tiling with an online softmax follows the published
// FlashAttention idea the atlas' ch.22 caption describes (scores and
// probabilities never leave the chip); the gfx950 design below is our own.
//
// Workgroup = 4 waves, one KV head, BM = 128/g consecutive query positions of
// one sequence.  The g query heads of the group are packed along the MFMA N
// dimension, so each wave owns 32 (position, head) columns and every K/V tile
// staged in LDS serves all g heads.
//   S^T = K Q^T      A = K tile rows from LDS, B = Q^T held in registers
//   O^T += V^T P^T   A = V^T from LDS,        B = P^T straight from the S^T
//                    accumulators (no shuffle, see below)
// With S^T the accumulator layout gives each lane one query column and 16 keys
// of each 32-key half; the MFMA B operand wants 8 consecutive k-indices per
// lane.  The two agree up to swapping bits 2 and 3 of the key index inside
// each group of 16, so V^T is written to LDS with its key index permuted that
// way and P^T is converted to bf16 in place.  Softmax statistics are per lane
// (one column), with one cross-half exchange per tile.
// Key tiles beyond the last visible key of the workgroup are never loaded;
// rows past k_len are zero-filled, never read from memory.
#include "pa_common.h"

namespace pa {
namespace {

constexpr int D = 128;
constexpr int BN = 64;          // keys per tile
constexpr int kThreads = 256;
constexpr int KST = D + 8;      // LDS row stride of the K tile (bf16 elements)
constexpr int VST = BN + 8;     // LDS row stride of the V^T tile

__device__ __forceinline__ int swap_bits23(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int G, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a)
{
    constexpr int BM = 128 / G;
    __shared__ __attribute__((aligned(16))) bf16 k_lds[BN * KST];
    __shared__ __attribute__((aligned(16))) bf16 vt_lds[D * VST];

    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, S = a.num_seqs;
    const int n_qblk = (a.max_seqlen_q + BM - 1) / BM;
    int idx = blockIdx.x;
    const int kvh = idx % Hkv;
    idx /= Hkv;
    const int s = idx % S;
    const int qb = n_qblk - 1 - idx / S;   // heaviest query blocks are dispatched first

    const int q0 = a.cu_seqlens_q[s];
    const int q_len = a.cu_seqlens_q[s + 1] - q0;
    if (qb * BM >= q_len)
        return;
    const int k0 = a.cu_seqlens_k[s];
    const int k_len = a.cu_seqlens_k[s + 1] - k0;
    const int off = k_len - q_len;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int hl = lane >> 5;        // which half of the MFMA k-range this lane feeds
    const int col = lane & 31;       // this lane's column (query) inside the wave
    const int ccol = wave * 32 + col;
    const int qrow = qb * BM + ccol / G;
    const int head = kvh * G + ccol % G;
    const bool col_valid = qrow < q_len;
    const int kmax = off + qrow;     // last visible key of this column

    // Q^T operand: 8 k-steps of 16 head-dim elements, 8 per lane
    bf16x8 qreg[8];
    {
        const bf16 *qp = static_cast<const bf16 *>(a.q) + ((int64_t)(q0 + qrow) * Hq + head) * D + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (col_valid)
                qreg[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
            else
                qreg[ks] = bf16x8{};
        }
    }

    const int wg_last_key = off + min(q_len, (qb + 1) * BM) - 1;
    const int n_kt = wg_last_key / BN + 1;
    const int wave_min_kmax = off + qb * BM + (wave * 32) / G;

    const bf16 *ksrc = static_cast<const bf16 *>(PAGED ? a.k_cache : a.k);
    const bf16 *vsrc = static_cast<const bf16 *>(PAGED ? a.v_cache : a.v);
    const int32_t *bt_row = PAGED ? a.block_tables + (int64_t)s * a.max_blocks : nullptr;
    const int bs = a.block_size, shift = a.bs_shift;

    // element offset of key row `key` of this sequence / KV head
    auto row_off = [&](int key) -> int64_t {
        int64_t row;
        if (PAGED) {
            const int lb = shift >= 0 ? (key >> shift) : (key / bs);
            row = (int64_t)bt_row[lb] * bs + (key - lb * bs);
        } else {
            row = (int64_t)k0 + key;
        }
        return (row * Hkv + kvh) * D;
    };

    // loader mapping: K rows (tid>>4) + 16*pass, V keys 4*(tid>>4) .. +3; 8 dims each
    const int lrow = tid >> 4;
    const int lchunk = tid & 15;
    uint4 kbuf[4], vbuf[4];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
            const int key = kt * BN + lrow + 16 * ps;
            kbuf[ps] = key < k_len ? *reinterpret_cast<const uint4 *>(ksrc + row_off(key) + 8 * lchunk)
                                   : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kt * BN + 4 * lrow + i;
            vbuf[i] = key < k_len ? *reinterpret_cast<const uint4 *>(vsrc + row_off(key) + 8 * lchunk)
                                  : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
            *reinterpret_cast<uint4 *>(&k_lds[(lrow + 16 * ps) * KST + 8 * lchunk]) = kbuf[ps];
        const int pos0 = swap_bits23(4 * lrow);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t word = e < 2 ? vbuf[i].x : e < 4 ? vbuf[i].y : e < 6 ? vbuf[i].z : vbuf[i].w;
                w[i] = (e & 1) ? (word >> 16) : (word & 0xffffu);
            }
            uint2 pk;
            pk.x = w[0] | (w[1] << 16);
            pk.y = w[2] | (w[3] << 16);
            *reinterpret_cast<uint2 *>(&vt_lds[(8 * lchunk + e) * VST + pos0]) = pk;
        }
    };

    f32x16 acc_o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
    float m = kMaxFloor, l = 0.f;
    const float sl2 = a.scale_log2;

    load_tile(0);
    for (int kt = 0; kt < n_kt; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < n_kt)
            load_tile(kt + 1);

        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&k_lds[(32 * mt + col) * KST + 16 * ks + 8 * hl]);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sacc[mt], 0, 0, 0);
            }
        }

        const int kbase = kt * BN;
        if (kbase + BN - 1 > wave_min_kmax) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kbase + 32 * mt + 8 * (v >> 2) + 4 * hl + (v & 3);
                    if (key > kmax) sacc[mt][v] = -INFINITY;
                }
        }

        float tmax = sacc[0][0];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[mt][v]);
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const float mnew = fmaxf(m, tmax * sl2);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;

        bf16x8 pb[4];
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float pw = fast_exp2(fmaf(sacc[mt][v], sl2, -mnew));
                psum += pw;
                pb[2 * mt + (v >> 3)][v & 7] = (bf16)pw;
            }
        l = fmaf(l, alpha, psum);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;

#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
#pragma unroll
            for (int mtd = 0; mtd < 4; ++mtd) {
                const bf16x8 va = *reinterpret_cast<const bf16x8 *>(&vt_lds[(32 * mtd + col) * VST + 16 * qs + 8 * hl]);
                acc_o[mtd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qs], acc_o[mtd], 0, 0, 0);
            }
        }
    }

    l += shfl_xor_f(l, 32);
    if (col_valid) {
        const float inv = 1.f / l;
        uint16_t *op = static_cast<uint16_t *>(a.out) + ((int64_t)(q0 + qrow) * Hq + head) * D;
#pragma unroll
        for (int mtd = 0; mtd < 4; ++mtd)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * mtd + 8 * g4 + 4 * hl;
                uint2 pk;
                pk.x = pack_bf16x2(acc_o[mtd][4 * g4 + 0] * inv, acc_o[mtd][4 * g4 + 1] * inv);
                pk.y = pack_bf16x2(acc_o[mtd][4 * g4 + 2] * inv, acc_o[mtd][4 * g4 + 3] * inv);
                *reinterpret_cast<uint2 *>(op + d0) = pk;
            }
    }
}

template <int G>
hipError_t launch_g(const PrefillArgs &a, hipStream_t stream)
{
    constexpr int BM = 128 / G;
    const int64_t n_qblk = (a.max_seqlen_q + BM - 1) / BM;
    const int64_t grid = n_qblk * a.num_seqs * a.num_kv_heads;
    if (a.paged)
        hipLaunchKernelGGL((prefill_kernel<G, true>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_kernel<G, false>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
