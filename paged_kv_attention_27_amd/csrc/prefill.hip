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
// cross-half exchange (v_permlane32_swap) per tile.  The running maximum is
// updated lazily: the output is rescaled only when a column's maximum grows by
// more than 2^8, so weights stay <= 256 and most tiles skip the rescale.
//
// K/V tiles of 64 keys go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds, or global_load_lds_dwordx4 for per-row paging:
// lane i of an instruction fills the i-th 16-byte chunk of a 1 KB span, i.e. 4
// tile rows), double-buffered in two LDS stages: the copy of tile t+1 is
// issued between the S MFMAs of tile t and waited for at the end of the step,
// so it overlaps a whole tile of work and costs no registers.  Batches with
// more query blocks than two per CU run a persistent grid with a heavy-first
// schedule every workgroup derives from cu_seqlens_q (see
// prefill_persistent_kernel).  Rows are 256 B with no padding; the 16-byte chunk c of row r is
// stored at position c ^ swz(r mod 16), swz(r) = 4 (r mod 4) + (r div 4) mod 4,
// which keeps both the b128 K reads (16 rows, one chunk) and the transposing V
// reads (4 rows, 2-4 chunks) free of bank conflicts.  Rows past k_len load a
// copy of the last valid row, so every V value is finite and every key past
// k_len is removed by the causal mask.  The block tables are read one tile
// ahead with vector loads.  Heaviest query blocks go first; workgroups whose
// blockIdx agree mod 8 (one XCD) share a KV head when Hkv divides 8, so its K/V
// stays in that L2.
//
// A second, ping-pong form serves batches of at most one query block per CU
// whose keys span more than 16 tiles, and key-split batches: a workgroup of
// eight waves, two groups of four that hold the same 128 columns and take
// alternate key tiles through their own halves of the stages, one section apart
// with a workgroup barrier between sections, so that on every SIMD one wave runs
// MFMAs while the other runs its softmax; the two groups' softmax states are
// merged through LDS at the end (prefill_pp_kernel).  In key-split mode
// (pa_prefill_varlen_ws) each block's key range is also split between two such
// workgroups, whose partials are merged by the second to finish.
#include "pa_common.h"

#include <atomic>
#include <type_traits>

namespace pa {
namespace {

constexpr int D = 128;
constexpr int BN = 64;             // keys per tile
constexpr int kThreads = 256;     // four-wave form
constexpr int kPPThreads = 512;   // ping-pong form: two groups of four waves
constexpr int ROWB = 2 * D;        // bytes per tile row
constexpr int TILEB = BN * ROWB;   // 16 KB
constexpr int STAGEB = 2 * TILEB;  // K tile, then V tile
constexpr float kLazyTau = 8.0f;   // log2 growth of a column max tolerated before rescaling

enum { kFlat = 0, kPagedTile = 1, kPagedRow = 2 };

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

// position of 16-byte chunk c of tile row r is c ^ swz(r & 15)
__device__ __forceinline__ int swz(int r16) { return 4 * (r16 & 3) + (r16 >> 2); }

__device__ __forceinline__ bf16x8 read_vt(const char *p0, const char *p1) {
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p1));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// 16 bytes per lane from base + off into the LDS span at dst (lane i -> dst + 16 i).
// The buffer form (a descriptor built from the wave-uniform base) keeps the
// copy a pure vector-memory operation, so waits on LDS reads stay exact.
__device__ __forceinline__ void copy16_to_lds(const char *base, uint32_t off, char *dst)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, off, 0, 0, 0);
}

// value of x held by lane (lane xor 32)
__device__ __forceinline__ float other_half(float x, int hl) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(hl ? r[0] : r[1]);
}

// One work item: query block qb (BM = 128/g positions) of sequence s against KV
// head kvh, through the two LDS stages, output written here.  The caller guarantees
// qb * BM < q_len.  Every path that touches the stages ends with a workgroup
// barrier, so items can follow each other on the same stages.
template <int G, int MODE>
__device__ __forceinline__ void attend_block(const PrefillArgs &a, int s, int qb, int kvh,
                                             char *stage0, char *stage1)
{
    constexpr int BM = 128 / G;
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int q0 = a.cu_seqlens_q[s];
    const int q_len = a.cu_seqlens_q[s + 1] - q0;
    const int k0 = a.cu_seqlens_k[s];
    const int k_len = a.cu_seqlens_k[s + 1] - k0;
    const int off = k_len - q_len;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
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
    // key tiles of this item: [kt_begin, kt_end)
    const int kt_begin = 0;
    const int kt_end = n_kt;

    const bf16 *ksrc = static_cast<const bf16 *>(MODE == kFlat ? a.k : a.k_cache);
    const bf16 *vsrc = static_cast<const bf16 *>(MODE == kFlat ? a.v : a.v_cache);
    const int32_t *bt_row = MODE == kFlat ? nullptr : a.block_tables + (int64_t)s * a.max_blocks;
    const int bs = a.block_size, shift = a.bs_shift;
    const int64_t row_elems = (int64_t)Hkv * D;

    // copy mapping: instruction j (0..3) of this wave fills tile rows 16*wave + 4*j + lsub,
    // lane position lpos of the row; it fetches logical chunk lpos ^ swz(4*j + lsub)
    const int lsub = lane >> 4;
    const int lpos = lane & 15;
    const int n_blk = MODE == kFlat ? 0 : (k_len + bs - 1) / bs;

    // per-tile paging needs a power-of-two block size (launch condition), so a shift
    auto block_of = [&](int key) {
        return MODE == kPagedTile ? (key >> shift) : (shift >= 0 ? (key >> shift) : (key / bs));
    };
    // block-table entries the copy of tile t needs, read into registers one tile ahead
    auto load_tbl = [&](int t, int32_t (&tbl)[4]) {
        if (MODE == kPagedTile) {
            // a tile lies in one block; each lane reads a neighbouring entry (a vector load)
            // and the copy uses lane 0's
            tbl[0] = bt_row[min(block_of(t * BN) + lane, n_blk - 1)];
        } else if (MODE == kPagedRow) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tbl[j] = bt_row[block_of(min(t * BN + 16 * wave + 4 * j + lsub, k_len - 1))];
        }
    };
    // byte offset, from the tile's first row, of the 16 bytes lane copies in instruction j
    const uint32_t row_bytes = (uint32_t)row_elems * 2;
    uint32_t coff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        coff[j] = (uint32_t)(16 * wave + 4 * j + lsub) * row_bytes + kvh * ROWB + 16 * (lpos ^ (4 * lsub + j));
    auto issue_tile = [&](char *stage, int t, const int32_t (&tbl)[4]) {
        const int key0 = t * BN;
        const int last = k_len - 1 - key0;   // rows past it copy this row
        if (MODE == kPagedRow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = key0 + min(16 * wave + 4 * j + lsub, last);
                const int64_t row = (int64_t)tbl[j] * bs + (key - block_of(key) * bs);
                const int64_t e = row * row_elems + kvh * D + 8 * (lpos ^ (4 * lsub + j));
                char *dst = stage + (16 * wave + 4 * j) * ROWB;
                __builtin_amdgcn_global_load_lds((global_void *)(ksrc + e), (lds_void *)dst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds((global_void *)(vsrc + e), (lds_void *)(dst + TILEB), 16, 0, 0);
            }
            return;
        }
        // the tile's rows are consecutive pool rows: one scalar base plus 32-bit lane offsets
        int64_t tile_row0;
        if (MODE == kFlat) {
            tile_row0 = (int64_t)k0 + key0;
        } else {
            const int lb = block_of(key0);
            tile_row0 = (int64_t)__builtin_amdgcn_readfirstlane(tbl[0]) * bs + (key0 - lb * bs);
        }
        const char *kb = reinterpret_cast<const char *>(ksrc) + tile_row0 * row_bytes;
        const char *vb = reinterpret_cast<const char *>(vsrc) + tile_row0 * row_bytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // rows past the last key re-read it (< 64 rows; a 24-bit multiply runs at full rate)
            const uint32_t o = coff[j] - __umul24((uint32_t)max(16 * wave + 4 * j + lsub - last, 0), row_bytes);
            char *dst = stage + (16 * wave + 4 * j) * ROWB;
            copy16_to_lds(kb, o, dst);
            copy16_to_lds(vb, o, dst + TILEB);
        }
    };

    // LDS read offsets (bytes within a stage); mt adds 32 rows, qs adds 16 rows
    int koff[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        koff[ks] = col * ROWB + 16 * ((2 * ks + hl) ^ swz(col & 15));
    // V^T read pattern: 16-lane group g = lane/16 covers head-dim half (g & 1) and
    // key quarter (g >> 1); lane i of the group reads key row (i >> 2), dims 4*(i & 3)
    const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    int voff0[4], voff1[4];
#pragma unroll
    for (int mtd = 0; mtd < 4; ++mtd) {
        voff0[mtd] = TILEB + tr_row * ROWB + 16 * ((4 * mtd + tr_chunk) ^ swz(tr_row)) + 8 * (lane & 1);
        voff1[mtd] = TILEB + (tr_row + 8) * ROWB + 16 * ((4 * mtd + tr_chunk) ^ swz(tr_row + 8)) + 8 * (lane & 1);
    }

    f32x16 acc_o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
    float m = kMaxFloor, l = 0.f;
    const float sl2 = a.scale_log2;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    int32_t tbl[4] = {0, 0, 0, 0};
    load_tbl(kt_begin, tbl);
    issue_tile(stage0, kt_begin, tbl);
    if (kt_begin + 1 < kt_end)
        load_tbl(kt_begin + 1, tbl);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies have landed
    __syncthreads();

    // one tile: compute tile kt from stage ST while tile kt+1 streams into the other stage
    auto step = [&](auto st_c, int kt) {
        constexpr int ST = decltype(st_c)::value;
        const char *cur = ST == 0 ? stage0 : stage1;
        char *nxt = ST == 0 ? stage1 : stage0;
        // copy of the next tile (the last tile re-copies itself into the stage no step reads
        // again, which keeps this part branch-free so the copies interleave with the MFMAs)
        issue_tile(nxt, min(kt + 1, kt_end - 1), tbl);
        load_tbl(min(kt + 2, kt_end - 1), tbl);

        bf16x8 kf[2][8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                kf[mt][ks] = *reinterpret_cast<const bf16x8 *>(cur + koff[ks] + 32 * ROWB * mt);
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][ks], qreg[ks], sacc[mt], 0, 0, 0);
        // all 16 K reads are issued before the first MFMA, so their latencies overlap; the
        // next tile's copies are spread between the MFMAs so their issue never stalls the wave
        // every V^T operand of the tile is read right after the score MFMAs (into the
        // registers the K operands free), so the reads land during the softmax and the
        // weighted-value MFMAs below issue back to back
        bf16x8 va[4][4];
#pragma unroll
        for (int qs = 0; qs < 4; ++qs)
#pragma unroll
            for (int mtd = 0; mtd < 4; ++mtd)
                va[qs][mtd] = read_vt(cur + voff0[mtd] + 16 * ROWB * qs, cur + voff1[mtd] + 16 * ROWB * qs);
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);

        const int kbase = kt * BN;
        if (kbase + BN - 1 > wave_min_kmax) {
            // value v of block mt holds key kbase + 32 mt + 8 (v / 4) + 4 hl + v % 4: compare
            // its constant part with one per-lane limit
            const int lim = kmax - kbase - 4 * hl;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * mt + 8 * (v >> 2) + (v & 3) > lim) sacc[mt][v] = -INFINITY;
        }

        float tmax = sacc[0][0];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[mt][v]);
        tmax = fmaxf(tmax, other_half(tmax, hl));
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
        for (int qs = 0; qs < 4; ++qs)
#pragma unroll
            for (int mtd = 0; mtd < 4; ++mtd)
                acc_o[mtd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[qs][mtd], pb[qs], acc_o[mtd], 0, 0, 0);

        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): tile kt+1 has landed (this wave's part)
        __syncthreads();                      // ... and every wave's part; stage ST is free again
    };

    for (int kt = kt_begin; kt < kt_end; kt += 2) {
        step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < kt_end)
            step(std::integral_constant<int, 1>{}, kt + 1);
    }

    l += other_half(l, hl);
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

// One workgroup per work item; items in the order (qb descending, s, kvh), so
// the heaviest query blocks are dispatched first and blockIdx mod Hkv = kvh.
template <int G, int MODE>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a)
{
    constexpr int BM = 128 / G;
    __shared__ __attribute__((aligned(1024))) char stage0[STAGEB];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGEB];
    const int Hkv = a.num_kv_heads, S = a.num_seqs;
    const int n_qblk = (a.max_seqlen_q + BM - 1) / BM;
    int idx = blockIdx.x;
    const int kvh = idx % Hkv;
    idx /= Hkv;
    const int s = idx % S;
    const int qb = n_qblk - 1 - idx / S;
    if (qb * BM >= a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s])
        return;
    attend_block<G, MODE>(a, s, qb, kvh, stage0, stage1);
}

constexpr int kMaxLevels = 1024;   // query-block levels the persistent schedule supports

// Persistent form: a grid of P workgroups (a multiple of 8, about two per CU)
// walks the non-empty items in the same heavy-first order.  Level L holds the
// query blocks qb = L of every sequence with more than L blocks, L from the top
// down; within a level items go by sequence, then KV head.  The items whose rank
// is x mod 8 belong to the P/8 workgroups with blockIdx mod 8 = x (the
// dispatcher places those on one XCD, and for Hkv dividing 8 they share the KV
// head), dealt in a snake order: in round k the j-th workgroup of the class
// takes position k*P/8 + j when k is even and k*P/8 + P/8-1-j when k is odd,
// which balances the decreasing item costs.  Every workgroup derives the same
// schedule from cu_seqlens_q, so no state is shared between workgroups or calls.
template <int G, int MODE>
__global__ __launch_bounds__(kThreads, 2) void prefill_persistent_kernel(PrefillArgs a)
{
    constexpr int BM = 128 / G;
    __shared__ __attribute__((aligned(1024))) char stage0[STAGEB];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGEB];
    __shared__ int lvl_cnt[kMaxLevels];     // sequences with more than L query blocks
    __shared__ int lvl_start[kMaxLevels];   // rank of the first item of level L
    const int Hkv = a.num_kv_heads, S = a.num_seqs;
    const int n_lvl = (a.max_seqlen_q + BM - 1) / BM;   // <= kMaxLevels (checked by the host)
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    auto n_blocks = [&](int q) {
        const int len = a.cu_seqlens_q[q + 1] - a.cu_seqlens_q[q];
        return min((len + BM - 1) / BM, n_lvl);
    };
    // histogram of per-sequence query-block counts: lvl_cnt[i] = #{s : blocks(s) = i + 1}
    for (int i = tid; i < n_lvl; i += kThreads)
        lvl_cnt[i] = 0;
    __syncthreads();
    for (int q = tid; q < S; q += kThreads) {
        const int nb = n_blocks(q);
        if (nb > 0)
            atomicAdd(&lvl_cnt[nb - 1], 1);
    }
    __syncthreads();
    if (wave == 0) {
        // suffix sums over levels, lane i owning levels [i*C, i*C + C)
        const int C = (n_lvl + kWave - 1) / kWave;   // <= 16
        int cnt[16];
        int local = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int L = lane * C + c;
            cnt[c] = (c < C && L < n_lvl) ? lvl_cnt[L] : 0;
            local += cnt[c];
        }
        int suf = local;                             // inclusive suffix over lanes
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_down(suf, d, kWave);
            if (lane + d < kWave) suf += v;
        }
        int run = suf - local;                       // levels above this lane's chunk
#pragma unroll
        for (int c = 15; c >= 0; --c) {
            run += cnt[c];                           // cnt[c] is 0 outside the chunk
            cnt[c] = (c < C && lane * C + c < n_lvl) ? run : 0;   // sequences with more than L blocks
        }
        int local2 = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) local2 += cnt[c];
        int suf2 = local2;
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_down(suf2, d, kWave);
            if (lane + d < kWave) suf2 += v;
        }
        int run2 = suf2 - local2;
#pragma unroll
        for (int c = 15; c >= 0; --c) {
            const int L = lane * C + c;
            if (c < C && L < n_lvl) {
                lvl_cnt[L] = cnt[c];
                lvl_start[L] = run2 * Hkv;
            }
            run2 += cnt[c];
        }
    }
    __syncthreads();
    const int items = lvl_start[0] + lvl_cnt[0] * Hkv;      // non-empty items

    const int P8 = gridDim.x / 8, x = blockIdx.x % 8, j = blockIdx.x / 8;
    for (int k = 0;; ++k) {
        const int pos = k * P8 + ((k & 1) ? P8 - 1 - j : j);
        const int irank = 8 * pos + x;
        if (irank >= items)
            break;
        // level: the smallest L with lvl_start[L] <= irank
        int lo = 0, hi = n_lvl - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (lvl_start[mid] <= irank) hi = mid; else lo = mid + 1;
        }
        const int L = lo;
        const int within = irank - lvl_start[L];
        const int kvh = within % Hkv;
        int t = within / Hkv;                        // the t-th sequence with more than L blocks
        int s = -1;
        for (int base = 0; base < S; base += kWave) {
            const int q = base + lane;
            const bool f = q < S && n_blocks(q) > L;
            const uint64_t b = __builtin_amdgcn_ballot_w64(f);
            const int c = __builtin_popcountll(b);
            if (t < c) {
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
                const uint64_t me = __builtin_amdgcn_ballot_w64(f && below == t);
                s = base + __builtin_ctzll(me);
                break;
            }
            t -= c;
        }
        if (s < 0)   // cannot happen: the counts and the scan use the same block counts
            break;
        attend_block<G, MODE>(a, s, L, kvh, stage0, stage1);
    }
}

// Barrier between half-steps: no wait for this wave's copies in flight.  (A
// __syncthreads would wait for them, since its workgroup fence covers the LDS the
// copies write.)  The signal fences keep the compiler from moving memory accesses
// across it, the scheduling barriers keep any other instruction on its side.
__device__ __forceinline__ void bar_half()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Barrier after which every wave's LDS reads and writes are done (copies may still
// be in flight).
__device__ __forceinline__ void bar_lds()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Barrier after which every wave's copies have landed and its LDS reads are done.
__device__ __forceinline__ void bar_landed()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Group (0/1) and slot (0..3) of the calling wave.  The two waves that share a SIMD
// go to different groups (the hardware id of each wave names its SIMD), so the
// MFMA section of one overlaps the softmax of the other; if the waves do not sit
// two per SIMD, waves 0-3 form group 0.  Every wave gets the same answer for the
// whole workgroup; one barrier.
__device__ __forceinline__ void wave_roles(int *simd_of, int &grp, int &slot)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if ((threadIdx.x & (kWave - 1)) == 0)
        simd_of[wave] = (__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 4) & 3;   // HW_ID.SIMD_ID
    __syncthreads();
    int sid[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) sid[w] = __builtin_amdgcn_readfirstlane(simd_of[w]);
    int role[8];
    bool ok = true;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        int before = 0, same = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            before += (u < w && sid[u] == sid[w]) ? 1 : 0;
            same += sid[u] == sid[w] ? 1 : 0;
        }
        role[w] = before;
        ok = ok && same == 2;
    }
    int g = wave >> 2, r = wave & 3;
    if (ok) {
        g = role[0];
#pragma unroll
        for (int w = 1; w < 8; ++w) g = w == wave ? role[w] : g;
        r = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) r += (u < wave && role[u] == g) ? 1 : 0;
    }
    grp = __builtin_amdgcn_readfirstlane(g);
    slot = __builtin_amdgcn_readfirstlane(r);
}

// One work item: query block qb (BM = 128/g positions) of sequence s against KV
// head kvh, over key tiles [kt_begin, kt_end).  half = -1: the whole key range;
// half = 0 / 1 (key-split mode): an item with at least kPrefillMinSplitTiles key
// tiles is split at tile n/2, a smaller one is done whole by half 0 (half 1 then
// has nsteps = 0: nothing to do).  The two groups of waves split the key tiles:
// group g takes tiles kt_begin + 2j + g, j < nsteps; a tile past kt_end (group 1,
// odd count) sees no key.
struct Item {
    int s, qb, kvh, half;   // half: -1, or the key half computed (key-split mode)
    int q0, q_len, k0, k_len;
    int kt_begin, kt_end, nsteps;
};

template <int G>
__device__ __forceinline__ Item make_item(const PrefillArgs &a, int s, int qb, int kvh, int half)
{
    constexpr int BM = 128 / G;
    Item it;
    it.s = s;
    it.qb = qb;
    it.kvh = kvh;
    it.half = half;
    it.nsteps = 0;
    it.q0 = a.cu_seqlens_q[s];
    it.q_len = a.cu_seqlens_q[s + 1] - it.q0;
    it.k0 = a.cu_seqlens_k[s];
    it.k_len = a.cu_seqlens_k[s + 1] - it.k0;
    const int off = it.k_len - it.q_len;
    const int n_kt = (off + min(it.q_len, (qb + 1) * BM) - 1) / BN + 1;
    if (half >= 0 && n_kt < kPrefillMinSplitTiles) {
        if (half == 1)
            return it;   // the whole item belongs to half 0
        half = -1;
    }
    it.half = half;
    it.kt_begin = half == 1 ? n_kt / 2 : 0;
    it.kt_end = half == 0 ? n_kt / 2 : n_kt;
    it.nsteps = (it.kt_end - it.kt_begin + 1) / 2;
    return it;
}

// The K/V tile copies, block-table reads and Q loads of one wave.
template <int G, int MODE>
struct Tiles {
    const PrefillArgs &a;
    int grp, slot, lane, lsub, lpos;

    __device__ __forceinline__ Tiles(const PrefillArgs &a_, int grp_, int slot_) : a(a_), grp(grp_), slot(slot_)
    {
        lane = threadIdx.x & (kWave - 1);
        lsub = lane >> 4;
        lpos = lane & 15;
    }
    // tile copied at step j (clamped: a step past the last tile copies the last one)
    __device__ __forceinline__ int copied(const Item &it, int j) const
    {
        return min(it.kt_begin + 2 * j + grp, it.kt_end - 1);
    }
    // per-tile paging needs a power-of-two block size (launch condition), so a shift
    __device__ __forceinline__ int block_of(int key) const
    {
        const int shift = a.bs_shift;
        return MODE == kPagedTile ? (key >> shift) : (shift >= 0 ? (key >> shift) : (key / a.block_size));
    }
    // block-table entries the copy of tile t needs
    __device__ __forceinline__ void load_tbl(const Item &it, int t, int32_t (&tbl)[4]) const
    {
        if (MODE == kFlat)
            return;
        const int32_t *bt_row = a.block_tables + (int64_t)it.s * a.max_blocks;
        if (MODE == kPagedTile) {
            // a tile lies in one block; each lane reads a neighbouring entry (a vector load)
            // and the copy uses lane 0's
            const int n_blk = (it.k_len + a.block_size - 1) / a.block_size;
            tbl[0] = bt_row[min(block_of(t * BN) + lane, n_blk - 1)];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tbl[j] = bt_row[block_of(min(t * BN + 16 * slot + 4 * j + lsub, it.k_len - 1))];
        }
    }
    // copy of tile t into this group's half of a stage: instruction j (0..3) of this wave
    // fills tile rows 16*slot + 4*j + lsub, lane position lpos of the row, fetching logical
    // chunk lpos ^ swz(4*j + lsub); rows past the last key copy that key's row
    __device__ __forceinline__ void issue(const Item &it, char *stage, int t, const int32_t (&tbl)[4]) const
    {
        const bf16 *ksrc = static_cast<const bf16 *>(MODE == kFlat ? a.k : a.k_cache);
        const bf16 *vsrc = static_cast<const bf16 *>(MODE == kFlat ? a.v : a.v_cache);
        const int64_t row_elems = (int64_t)a.num_kv_heads * D;
        const uint32_t row_bytes = (uint32_t)row_elems * 2;
        const int key0 = t * BN;
        const int last = it.k_len - 1 - key0;
        if (MODE == kPagedRow) {
            const int bs = a.block_size;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = key0 + min(16 * slot + 4 * j + lsub, last);
                const int64_t row = (int64_t)tbl[j] * bs + (key - block_of(key) * bs);
                const int64_t e = row * row_elems + it.kvh * D + 8 * (lpos ^ (4 * lsub + j));
                char *dst = stage + (16 * slot + 4 * j) * ROWB;
                __builtin_amdgcn_global_load_lds((global_void *)(ksrc + e), (lds_void *)dst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds((global_void *)(vsrc + e), (lds_void *)(dst + TILEB), 16, 0, 0);
            }
            return;
        }
        // the tile's rows are consecutive pool rows: one scalar base plus 32-bit lane offsets
        int64_t tile_row0;
        if (MODE == kFlat) {
            tile_row0 = (int64_t)it.k0 + key0;
        } else {
            const int lb = block_of(key0);
            tile_row0 = (int64_t)__builtin_amdgcn_readfirstlane(tbl[0]) * a.block_size + (key0 - lb * a.block_size);
        }
        const char *kb = reinterpret_cast<const char *>(ksrc) + tile_row0 * row_bytes;
        const char *vb = reinterpret_cast<const char *>(vsrc) + tile_row0 * row_bytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // rows past the last key re-read it (< 64 rows; a 24-bit multiply runs at full rate)
            const uint32_t coff = (uint32_t)(16 * slot + 4 * j + lsub) * row_bytes + it.kvh * ROWB +
                                  16 * (lpos ^ (4 * lsub + j));
            const uint32_t o = coff - __umul24((uint32_t)max(16 * slot + 4 * j + lsub - last, 0), row_bytes);
            char *dst = stage + (16 * slot + 4 * j) * ROWB;
            copy16_to_lds(kb, o, dst);
            copy16_to_lds(vb, o, dst + TILEB);
        }
    }
    // Q^T operand of this wave's 32 columns: 8 k-steps of 16 head-dim elements, 8 per lane
    __device__ __forceinline__ void load_q(const Item &it, bf16x8 (&qreg)[8]) const
    {
        constexpr int BM = 128 / G;
        const int ccol = slot * 32 + (lane & 31);
        const int qrow = it.qb * BM + ccol / G;
        const int head = it.kvh * G + ccol % G;
        const bool col_valid = qrow < it.q_len;
        const bf16 *qp = static_cast<const bf16 *>(a.q) + ((int64_t)(it.q0 + qrow) * a.num_q_heads + head) * D +
                         8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qreg[ks] = col_valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * ks) : bf16x8{};
    }
};

// The steps of one item: the tiles of step 0 have landed in stage 0 (both groups),
// tbl holds the block-table entries of step 1.  A group's step j is an MFMA section
// (the weighted-value MFMAs of step j-1, the copy of step j+1, the score MFMAs of
// step j) followed by a softmax section (the V^T reads of step j, which land during
// it, then mask, running max, weights, row sums); group 1 runs one section behind
// group 0, with a workgroup barrier between sections, so on every SIMD one wave is
// in an MFMA section while the other is in a softmax section.  On return every
// wave is past the item's last barrier and no copy is in flight.
template <int G, int MODE>
__device__ __forceinline__ void run_steps(const PrefillArgs &a, const Tiles<G, MODE> &tl, const Item &it,
                                          char *stage0, char *stage1, const bf16x8 (&qreg)[8],
                                          int32_t (&tbl)[4], f32x16 (&acc_o)[4], float &m, float &l)
{
    constexpr int BM = 128 / G;
    const int grp = tl.grp, slot = tl.slot, lane = tl.lane;
    const int hl = lane >> 5;        // which half of the MFMA k-range this lane feeds
    const int col = lane & 31;       // this lane's column (query) inside the wave
    const int off = it.k_len - it.q_len;
    const int kmax = off + it.qb * BM + (slot * 32 + col) / G;   // last visible key of this column
    const int wave_min_kmax = off + it.qb * BM + (slot * 32) / G;
    const int goff = grp * STAGEB;   // this group's half of a stage
    const int nsteps = it.nsteps;

    // LDS read offsets (bytes within a stage); mt adds 32 rows, qs adds 16 rows
    int koff[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        koff[ks] = goff + col * ROWB + 16 * ((2 * ks + hl) ^ swz(col & 15));
    // V^T read pattern: 16-lane group g = lane/16 covers head-dim half (g & 1) and
    // key quarter (g >> 1); lane i of the group reads key row (i >> 2), dims 4*(i & 3)
    const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    int voff0[4], voff1[4];
#pragma unroll
    for (int mtd = 0; mtd < 4; ++mtd) {
        voff0[mtd] = goff + TILEB + tr_row * ROWB + 16 * ((4 * mtd + tr_chunk) ^ swz(tr_row)) + 8 * (lane & 1);
        voff1[mtd] = goff + TILEB + (tr_row + 8) * ROWB + 16 * ((4 * mtd + tr_chunk) ^ swz(tr_row + 8)) + 8 * (lane & 1);
    }

    const float sl2 = a.scale_log2;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    f32x16 sacc[2];
    bf16x8 va[4][4];   // V^T operands of the last softmax section
    bf16x8 pb[4];      // its weights

    auto msec = [&](auto st_c, auto pv_c, auto sc_c, int j) {
        constexpr int ST = decltype(st_c)::value;
        constexpr bool PV = decltype(pv_c)::value, SC = decltype(sc_c)::value;
        const char *cur = ST == 0 ? stage0 : stage1;
        char *nxt = (ST == 0 ? stage1 : stage0) + goff;
        if (PV) {
#pragma unroll
            for (int qs = 0; qs < 4; ++qs)
#pragma unroll
                for (int mtd = 0; mtd < 4; ++mtd)
                    acc_o[mtd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[qs][mtd], pb[qs], acc_o[mtd], 0, 0, 0);
        }
        if (SC) {
            tl.issue(it, nxt, tl.copied(it, j + 1), tbl);
            tl.load_tbl(it, tl.copied(it, j + 2), tbl);
            bf16x8 kf[2][8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    kf[mt][ks] = *reinterpret_cast<const bf16x8 *>(cur + koff[ks] + 32 * ROWB * mt);
            sacc[0] = f32x16{};
            sacc[1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][ks], qreg[ks], sacc[mt], 0, 0, 0);
            if (PV)
                __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);   // the PV MFMAs first
            __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };

    auto ssec = [&](auto st_c, int j) {
        constexpr int ST = decltype(st_c)::value;
        const char *cur = ST == 0 ? stage0 : stage1;
#pragma unroll
        for (int qs = 0; qs < 4; ++qs)
#pragma unroll
            for (int mtd = 0; mtd < 4; ++mtd)
                va[qs][mtd] = read_vt(cur + voff0[mtd] + 16 * ROWB * qs, cur + voff1[mtd] + 16 * ROWB * qs);
        const int t = it.kt_begin + 2 * j + grp;
        const int kbase = t * BN;
        if (t >= it.kt_end || kbase + BN - 1 > wave_min_kmax) {
            // value v of block mt holds key kbase + 32 mt + 8 (v / 4) + 4 hl + v % 4: compare
            // its constant part with one per-lane limit (below zero: every key masked)
            const int lim = t < it.kt_end ? kmax - kbase - 4 * hl : -1;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * mt + 8 * (v >> 2) + (v & 3) > lim) sacc[mt][v] = -INFINITY;
        }
        float tmax = sacc[0][0];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[mt][v]);
        tmax = fmaxf(tmax, other_half(tmax, hl));
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
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using T = std::true_type;
    using F = std::false_type;
    // group 1 idles while group 0 runs its first MFMA section, group 0 while group 1
    // runs its last
    if (grp == 1)
        bar_half();
    msec(I0{}, F{}, T{}, 0);
    bar_half();
    ssec(I0{}, 0);
    bar_landed();   // step 1 copied, step 0's V^T reads done: its stage half may be refilled
    int j = 1;
    for (; j + 1 < nsteps; j += 2) {
        msec(I1{}, T{}, T{}, j);
        bar_half();
        ssec(I1{}, j);
        bar_landed();
        msec(I0{}, T{}, T{}, j + 1);
        bar_half();
        ssec(I0{}, j + 1);
        bar_landed();
    }
    if (j < nsteps) {
        msec(I1{}, T{}, T{}, j);
        bar_half();
        ssec(I1{}, j);
        bar_landed();
    }
    msec(I0{}, T{}, F{}, nsteps);   // the last weighted-value MFMAs
    bar_half();
    if (grp == 0)
        bar_half();
    l += other_half(l, hl);
}

// Merge of the two groups' softmax states through LDS (log-sum-exp combination:
// rescale both to the larger running maximum).  Wave (grp, slot) keeps head-dim half
// grp (accumulator blocks 2 grp, 2 grp + 1) and hands the other half, with its max
// and sum, to wave (1 - grp, slot).  xo: [8 waves][8 chunks][64 lanes] of 16 bytes
// (64 KB), xs: [8 waves][64 lanes] of (max, sum).  o gets this wave's half of the
// unnormalised output, mm and lsum the item's column max and sum (the same bits in
// both groups).  Ends with every wave's LDS reads done.
__device__ __forceinline__ void merge_groups(int grp, int slot, const f32x16 (&acc_o)[4], float m, float l,
                                             float4 *xo, float2 *xs, f32x16 (&o)[2], float &mm, float &lsum)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int me = grp * 4 + slot, partner = (1 - grp) * 4 + slot;
    // (selects, not an index by grp: a runtime index would move acc_o out of registers)
    const f32x16 keep[2] = {grp == 0 ? acc_o[0] : acc_o[2], grp == 0 ? acc_o[1] : acc_o[3]};
    const f32x16 give[2] = {grp == 0 ? acc_o[2] : acc_o[0], grp == 0 ? acc_o[3] : acc_o[1]};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const f32x16 &g = give[c >> 2];
        const int v = 4 * (c & 3);
        xo[(partner * 8 + c) * 64 + lane] = make_float4(g[v], g[v + 1], g[v + 2], g[v + 3]);
    }
    xs[me * 64 + lane] = make_float2(m, l);
    bar_lds();
    const float2 ml = xs[partner * 64 + lane];
    // the same operands in the same order in both groups: group 0's state first
    const float m0 = grp == 0 ? m : ml.x, m1 = grp == 0 ? ml.x : m;
    const float l0 = grp == 0 ? l : ml.y, l1 = grp == 0 ? ml.y : l;
    mm = fmaxf(m0, m1);
    const float w0 = fast_exp2(m0 - mm), w1 = fast_exp2(m1 - mm);
    lsum = l0 * w0 + l1 * w1;
    const float w_me = grp == 0 ? w0 : w1, w_pa = grp == 0 ? w1 : w0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float4 p = xo[(me * 8 + c) * 64 + lane];
        const int i = c >> 2, v = 4 * (c & 3);
        o[i][v + 0] = keep[i][v + 0] * w_me + p.x * w_pa;
        o[i][v + 1] = keep[i][v + 1] * w_me + p.y * w_pa;
        o[i][v + 2] = keep[i][v + 2] * w_me + p.z * w_pa;
        o[i][v + 3] = keep[i][v + 3] * w_me + p.w * w_pa;
    }
}

// Output rows of this wave's columns, head-dim half grp: O / l in bf16.
template <int G>
__device__ __forceinline__ void store_out(const PrefillArgs &a, const Item &it, int grp, int slot,
                                          const f32x16 (&o)[2], float lsum)
{
    constexpr int BM = 128 / G;
    const int lane = threadIdx.x & (kWave - 1), hl = lane >> 5;
    const int ccol = slot * 32 + (lane & 31);
    const int qrow = it.qb * BM + ccol / G;
    const int head = it.kvh * G + ccol % G;
    if (qrow < it.q_len) {
        const float inv = 1.f / lsum;
        uint16_t *op = static_cast<uint16_t *>(a.out) + ((int64_t)(it.q0 + qrow) * a.num_q_heads + head) * D;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * (2 * grp + i) + 8 * g4 + 4 * hl;
                uint2 pk;
                pk.x = pack_bf16x2(o[i][4 * g4 + 0] * inv, o[i][4 * g4 + 1] * inv);
                pk.y = pack_bf16x2(o[i][4 * g4 + 2] * inv, o[i][4 * g4 + 3] * inv);
                *reinterpret_cast<uint2 *>(op + d0) = pk;
            }
    }
}

// Key-split half: store the partial (O / l, column max and sum, all fp32), count
// the arrival, and if second merge both halves (log-sum-exp combination) and write
// the output.  The partial and the counter use device-scope (coherent across XCDs)
// relaxed atomic stores and loads, which go through to the coherent level instead
// of staying in one XCD's L2; vmcnt(0) makes every store complete before the
// arrival is counted.  (A device-scope fence would instead write back and
// invalidate the whole L2 of the XCD, evicting the K/V tiles of every other
// workgroup there.)
template <int G>
__device__ __forceinline__ void split_tail(const PrefillArgs &a, const Item &it, int grp, int slot,
                                          const f32x16 (&o)[2], float mm, float lsum, int *arrival)
{
    constexpr int BM = 128 / G;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), hl = lane >> 5;
    const int Hkv = a.num_kv_heads;
    const int ccol = slot * 32 + (lane & 31);
    const int qrow = it.qb * BM + ccol / G;
    const int head = it.kvh * G + ccol % G;
    const int n_lvl = (a.max_seqlen_q + BM - 1) / BM;
    const int64_t item = ((int64_t)it.s * n_lvl + it.qb) * Hkv + it.kvh;
    constexpr int kWords = (int)(kPrefillPartBytes / 4);
    constexpr int kOWords = 4 * 64 * 64;
    uint32_t *mine = static_cast<uint32_t *>(a.ws_part) + (item * 2 + it.half) * kWords;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;   // a column may see no key of this half
    auto st = [](uint32_t *p, uint32_t v) {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto ldc = [](const uint32_t *p) {
        return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            st(mine + (slot * 64 + 16 * (2 * grp + i) + v) * 64 + lane, __float_as_uint(o[i][v] * inv));
    if (grp == 0) {
        st(mine + kOWords + (slot * 2 + 0) * 64 + lane, __float_as_uint(mm));
        st(mine + kOWords + (slot * 2 + 1) * 64 + lane, __float_as_uint(lsum));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
    __syncthreads();                      // ... and every wave's, before the arrival counts
    if (tid == 0)
        *arrival = __hip_atomic_fetch_add(&a.ws_cnt[item], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool second = *arrival == 1;
    __syncthreads();                      // *arrival is read by all before its next use
    if (!second)
        return;
    // the partner's partial is read only after its arrival was seen: no load below may
    // be moved above this point (the branch already orders them in the hardware, which
    // issues a wave's instructions in order)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t *other = static_cast<const uint32_t *>(a.ws_part) + (item * 2 + (1 - it.half)) * kWords;
    const float m1o = __uint_as_float(ldc(other + kOWords + (slot * 2 + 0) * 64 + lane));
    const float l1o = __uint_as_float(ldc(other + kOWords + (slot * 2 + 1) * 64 + lane));
    // both halves enter the merge as they are stored (O / l, max, sum) and in key order
    // (half 0 first), so the result does not depend on which half arrived second
    const bool h0 = it.half == 0;
    const float m0 = h0 ? mm : m1o, m1 = h0 ? m1o : mm;
    const float mmo = fmaxf(m0, m1);
    const float w0 = (h0 ? lsum : l1o) * fast_exp2(m0 - mmo);
    const float w1 = (h0 ? l1o : lsum) * fast_exp2(m1 - mmo);
    const float inv2 = 1.f / (w0 + w1);
    if (tid == 0)   // ready for the next call
        __hip_atomic_store(&a.ws_cnt[item], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (qrow < it.q_len) {
        uint16_t *op = static_cast<uint16_t *>(a.out) + ((int64_t)(it.q0 + qrow) * a.num_q_heads + head) * D;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int mtd = 2 * grp + i;
                const int d0 = 32 * mtd + 8 * g4 + 4 * hl;
                float ov[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float theirs = __uint_as_float(ldc(other + (slot * 64 + 16 * mtd + 4 * g4 + e) * 64 + lane));
                    const float own = o[i][4 * g4 + e] * inv;   // the bits this half stored
                    ov[e] = ((h0 ? own : theirs) * w0 + (h0 ? theirs : own) * w1) * inv2;
                }
                uint2 pk;
                pk.x = pack_bf16x2(ov[0], ov[1]);
                pk.y = pack_bf16x2(ov[2], ov[3]);
                *reinterpret_cast<uint2 *>(op + d0) = pk;
            }
    }
}

// One item from start to end, with its own prologue (Q, first tiles): the one-item
// kernel and key-split mode.
template <int G, int MODE>
__device__ __forceinline__ void attend_item(const PrefillArgs &a, const Tiles<G, MODE> &tl, const Item &it,
                                            char *stage0, char *stage1, float4 *xo, float2 *xs, int *arrival)
{
    if (it.nsteps == 0)
        return;
    bf16x8 qreg[8];
    tl.load_q(it, qreg);
    int32_t tbl[4] = {0, 0, 0, 0};
    tl.load_tbl(it, tl.copied(it, 0), tbl);
    tl.issue(it, stage0 + tl.grp * STAGEB, tl.copied(it, 0), tbl);
    tl.load_tbl(it, tl.copied(it, 1), tbl);
    bar_landed();   // step 0 of both groups is in LDS
    f32x16 acc_o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
    float m = kMaxFloor, l = 0.f;
    run_steps<G, MODE>(a, tl, it, stage0, stage1, qreg, tbl, acc_o, m, l);
    f32x16 o[2];
    float mm, lsum;
    merge_groups(tl.grp, tl.slot, acc_o, m, l, xo, xs, o, mm, lsum);
    if (it.half >= 0)
        split_tail<G>(a, it, tl.grp, tl.slot, o, mm, lsum, arrival);
    else
        store_out<G>(a, it, tl.grp, tl.slot, o, lsum);
    bar_lds();   // every wave's merge reads are done before the stages are reused
}

// Ping-pong form, one workgroup of eight waves per item (or per key half of an item in
// key-split mode), items in the order (qb descending, s, kvh) as in prefill_kernel;
// in key-split mode the two halves of an item take adjacent workgroups.  One
// workgroup per CU (133 KB of LDS).
template <int G, int MODE>
__global__ __launch_bounds__(kPPThreads, 1) void prefill_pp_kernel(PrefillArgs a)
{
    constexpr int BM = 128 / G;
    __shared__ __attribute__((aligned(1024))) char stage0[2 * STAGEB];
    __shared__ __attribute__((aligned(1024))) char stage1[2 * STAGEB];
    __shared__ float2 xs[8 * 64];
    __shared__ int simd_of[8];
    __shared__ int arrival;
    const int Hkv = a.num_kv_heads, S = a.num_seqs;
    const int n_qblk = (a.max_seqlen_q + BM - 1) / BM;
    int idx = a.split ? blockIdx.x >> 1 : blockIdx.x;
    const int half = a.split ? (int)(blockIdx.x & 1) : -1;
    const int kvh = idx % Hkv;
    idx /= Hkv;
    const int s = idx % S;
    const int qb = n_qblk - 1 - idx / S;
    if (qb * BM >= a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s])
        return;
    int grp, slot;
    wave_roles(simd_of, grp, slot);
    const Tiles<G, MODE> tl(a, grp, slot);
    const Item it = make_item<G>(a, s, qb, kvh, half);
    attend_item<G, MODE>(a, tl, it, stage0, stage1, reinterpret_cast<float4 *>(stage1), xs, &arrival);
}

// compute units of the current device (queried once per device; concurrent
// first calls store the same value)
int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace
int64_t prefill_split_items(int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t num_q_heads, int32_t num_kv_heads);
namespace {

// Which form runs a batch: the ping-pong form for key-split batches and for batches
// of at most one item per CU whose keys span more than 16 tiles (there each item's
// tiles are shared by two groups of waves, which halves the longest item; measured on
// MI355X, Hq16/Hkv8: 64 queries over 4096 keys 59 -> 47 us, 512 over 8192 96 -> 74,
// 4 x 512 over 4096 98 -> 78, 2048 over 4096 84 -> 72; a 1024-token prompt with no
// cache 25.5 -> 26.7, so short keys stay on the four-wave form); otherwise the
// four-wave form, one workgroup per item up to two items per CU, else persistent.
template <int G>
hipError_t launch_g(const PrefillArgs &a_in, hipStream_t stream)
{
    PrefillArgs a = a_in;
    if (a.split && prefill_split_items(a.num_seqs, a.max_seqlen_q, a.max_seqlen_k, a.num_q_heads,
                                       a.num_kv_heads) == 0)
        a.split = 0;
    constexpr int BM = 128 / G;
    const int64_t n_qblk = (a.max_seqlen_q + BM - 1) / BM;
    const int64_t items = n_qblk * a.num_seqs * a.num_kv_heads;
    const int64_t cus = device_cus();
    const bool pow2 = (a.block_size & (a.block_size - 1)) == 0;
    const int mode = !a.paged ? kFlat : (a.block_size % BN == 0 && pow2 ? kPagedTile : kPagedRow);
    if (a.split || (items <= cus && a.max_seqlen_k > 16 * BN)) {
        const dim3 grid((uint32_t)(a.split ? 2 * items : items));
        if (mode == kFlat)
            hipLaunchKernelGGL((prefill_pp_kernel<G, kFlat>), grid, dim3(kPPThreads), 0, stream, a);
        else if (mode == kPagedTile)
            hipLaunchKernelGGL((prefill_pp_kernel<G, kPagedTile>), grid, dim3(kPPThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_pp_kernel<G, kPagedRow>), grid, dim3(kPPThreads), 0, stream, a);
    } else if (items > 2 * cus && n_qblk <= kMaxLevels) {
        const dim3 grid((uint32_t)((2 * cus + 7) / 8 * 8));
        if (mode == kFlat)
            hipLaunchKernelGGL((prefill_persistent_kernel<G, kFlat>), grid, dim3(kThreads), 0, stream, a);
        else if (mode == kPagedTile)
            hipLaunchKernelGGL((prefill_persistent_kernel<G, kPagedTile>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_persistent_kernel<G, kPagedRow>), grid, dim3(kThreads), 0, stream, a);
    } else {
        const dim3 grid((uint32_t)items);
        if (mode == kFlat)
            hipLaunchKernelGGL((prefill_kernel<G, kFlat>), grid, dim3(kThreads), 0, stream, a);
        else if (mode == kPagedTile)
            hipLaunchKernelGGL((prefill_kernel<G, kPagedTile>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_kernel<G, kPagedRow>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

int64_t prefill_split_items(int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t num_q_heads, int32_t num_kv_heads)
{
    if (num_seqs < 1 || max_seqlen_q < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
        return 0;
    const int g = num_q_heads / num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return 0;
    const int64_t bm = 128 / g;
    const int64_t n_qblk = (max_seqlen_q + bm - 1) / bm;
    const int64_t items = n_qblk * num_seqs * num_kv_heads;
    // split only a batch of few, long items: at most one item per two CUs and at least
    // 2048 keys (32 key tiles) in the longest.  Measured on MI355X (Hq16/Hkv8, one
    // sequence): q 64 / k 4096 65 -> 46 us, q 512 / k 8192 127 -> 79 us, q 1024 /
    // k 4096 68 -> 51 us; with more items per CU (8 x U[100,1024] varlen, 4 x 512 over
    // 4096) or short keys (q = k = 1024) the merge costs more than the shorter
    // critical path saves.
    const bool few_long = items * 2 <= (int64_t)device_cus() && max_seqlen_k >= 2048;
    return (n_qblk <= kMaxLevels && few_long) ? items : 0;
}

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
