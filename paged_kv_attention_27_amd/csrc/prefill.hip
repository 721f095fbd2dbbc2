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
//   S^T = K Q^T      A = K tile rows from LDS (ds_read_b128), B = Q^T in registers
//   O^T += V^T P^T   A = V^T read from the natural [key][d] V tile with the
//                    transposing ds_read_b64_tr_b16, B = P^T straight from the
//                    S^T accumulators
// The 32x32 accumulator layout gives each lane one query column and, for every
// 16 keys, keys {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); the B operand wants 8
// consecutive k-indices, which matches once bits 2 and 3 of the key index are
// swapped.  The two transposing reads fetch exactly that key order for V^T, so
// P^T needs no shuffle.  Softmax statistics are per lane (one column), with one
// cross-half exchange per tile.  The running maximum is updated lazily: the
// output is rescaled only when a column's maximum grows by more than 2^8, so
// weights stay <= 256 and most tiles skip the rescale entirely.
//
// K/V tiles of 64 keys are double-buffered in LDS (one barrier per tile) and
// prefetched into registers two tiles ahead.  Rows past k_len are zero-filled,
// never read.  When the block size is a multiple of 64 a tile lies inside one
// block: one table lookup per tile, otherwise one per row.  Heaviest query
// blocks are dispatched first; blockIdx mod Hkv = KV head keeps every block of a
// (sequence, KV head) on one XCD so its K/V stays in that L2.
#include "pa_common.h"

namespace pa {
namespace {

constexpr int D = 128;
constexpr int BN = 64;          // keys per tile
constexpr int kThreads = 256;
constexpr int KST = D + 8;      // K tile row stride (bf16): 272 B, conflict-free b128 reads
constexpr int VST = D + 32;     // V tile row stride (bf16): 320 B, conflict-free tr reads
constexpr int KBUF = BN * KST;
constexpr int VBUF = BN * VST;
constexpr float kLazyTau = 8.0f;   // log2 growth of a column max tolerated before rescaling

enum { kFlat = 0, kPagedTile = 1, kPagedRow = 2 };

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ bf16x8 read_vt(const bf16 *p0, const bf16 *p1) {
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p1));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

template <int G, int MODE>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a)
{
    constexpr int BM = 128 / G;
    __shared__ __attribute__((aligned(16))) bf16 k_lds[2 * KBUF];
    __shared__ __attribute__((aligned(16))) bf16 v_lds[2 * VBUF];

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
        for (int ks = 0; ks < 8; ++ks)
            qreg[ks] = col_valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * ks) : bf16x8{};
    }

    const int wg_last_key = off + min(q_len, (qb + 1) * BM) - 1;
    const int n_kt = wg_last_key / BN + 1;
    const int wave_min_kmax = off + qb * BM + (wave * 32) / G;

    const bf16 *ksrc = static_cast<const bf16 *>(MODE == kFlat ? a.k : a.k_cache);
    const bf16 *vsrc = static_cast<const bf16 *>(MODE == kFlat ? a.v : a.v_cache);
    const int32_t *bt_row = MODE == kFlat ? nullptr : a.block_tables + (int64_t)s * a.max_blocks;
    const int bs = a.block_size, shift = a.bs_shift;
    const int64_t row_elems = (int64_t)Hkv * D;

    // loader: thread owns rows lrow + 16*ps of each tile, 8 head-dim elements at 8*lchunk
    const int lrow = tid >> 4;
    const int lchunk = tid & 15;
    const int64_t lane_off = (int64_t)lrow * row_elems + kvh * D + 8 * lchunk;
    uint4 kbuf[4], vbuf[4];

    auto load_tile = [&](int kt) {
        const int key0 = kt * BN;
        if (MODE == kPagedRow) {
#pragma unroll
            for (int ps = 0; ps < 4; ++ps) {
                const int key = key0 + lrow + 16 * ps;
                if (key < k_len) {
                    const int lb = shift >= 0 ? (key >> shift) : (key / bs);
                    const int64_t e = ((int64_t)bt_row[lb] * bs + (key - lb * bs)) * row_elems + kvh * D + 8 * lchunk;
                    kbuf[ps] = *reinterpret_cast<const uint4 *>(ksrc + e);
                    vbuf[ps] = *reinterpret_cast<const uint4 *>(vsrc + e);
                } else {
                    kbuf[ps] = make_uint4(0, 0, 0, 0);
                    vbuf[ps] = make_uint4(0, 0, 0, 0);
                }
            }
        } else {
            int64_t base_row;
            if (MODE == kFlat) {
                base_row = (int64_t)k0 + key0;
            } else {
                const int lb = __builtin_amdgcn_readfirstlane(shift >= 0 ? (key0 >> shift) : (key0 / bs));
                base_row = (int64_t)__builtin_amdgcn_readfirstlane(bt_row[lb]) * bs + (key0 - lb * bs);
            }
            const bf16 *kb = ksrc + base_row * row_elems + lane_off;
            const bf16 *vb = vsrc + base_row * row_elems + lane_off;
#pragma unroll
            for (int ps = 0; ps < 4; ++ps) {
                const bool ok = key0 + lrow + 16 * ps < k_len;
                kbuf[ps] = ok ? *reinterpret_cast<const uint4 *>(kb + 16 * ps * row_elems) : make_uint4(0, 0, 0, 0);
                vbuf[ps] = ok ? *reinterpret_cast<const uint4 *>(vb + 16 * ps * row_elems) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf) {
        bf16 *kd = k_lds + buf * KBUF + lrow * KST + 8 * lchunk;
        bf16 *vd = v_lds + buf * VBUF + lrow * VST + 8 * lchunk;
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
            *reinterpret_cast<uint4 *>(kd + 16 * ps * KST) = kbuf[ps];
            *reinterpret_cast<uint4 *>(vd + 16 * ps * VST) = vbuf[ps];
        }
    };

    f32x16 acc_o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
    float m = kMaxFloor, l = 0.f;
    const float sl2 = a.scale_log2;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // V^T read pattern: 16-lane group g = lane/16 covers head-dim half (g & 1) and
    // key quarter (g >> 1); lane i of the group points at key row (i >> 2), dims 4*(i & 3)
    const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    load_tile(0);
    store_tile(0);
    if (n_kt > 1)
        load_tile(1);
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
        const int cur = kt & 1;
        const bf16 *kl = k_lds + cur * KBUF;
        const bf16 *vl = v_lds + cur * VBUF;

        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kl + (32 * mt + col) * KST + 16 * ks + 8 * hl);
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
        const float mcand = tmax * sl2;
        const bool grow = mcand > m + kLazyTau;
        if (__builtin_amdgcn_ballot_w64(grow)) {   // wave-uniform: rescale only when a max grew
            const float mnew = grow ? mcand : m;
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;
        }

        bf16x8 pb[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                pb[2 * mt + (v >> 3)][v & 7] = (bf16)fast_exp2(fmaf(sacc[mt][v], sl2, -m));
#pragma unroll
        for (int qs = 0; qs < 4; ++qs)
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const bf16x2 two = {pb[qs][2 * pr], pb[qs][2 * pr + 1]};
                l = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l, false);
            }

#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
            const bf16 *vrow = vl + (16 * qs + tr_row) * VST + tr_col;
#pragma unroll
            for (int mtd = 0; mtd < 4; ++mtd) {
                const bf16x8 va = read_vt(vrow + 32 * mtd, vrow + 8 * VST + 32 * mtd);
                acc_o[mtd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qs], acc_o[mtd], 0, 0, 0);
            }
        }

        if (kt + 1 < n_kt) {
            store_tile(cur ^ 1);
            if (kt + 2 < n_kt)
                load_tile(kt + 2);
        }
        __syncthreads();
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
    const dim3 grid((uint32_t)(n_qblk * a.num_seqs * a.num_kv_heads));
    if (!a.paged)
        hipLaunchKernelGGL((prefill_kernel<G, kFlat>), grid, dim3(kThreads), 0, stream, a);
    else if (a.block_size % BN == 0)
        hipLaunchKernelGGL((prefill_kernel<G, kPagedTile>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_kernel<G, kPagedRow>), grid, dim3(kThreads), 0, stream, a);
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
