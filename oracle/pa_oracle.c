/*
 * pa_oracle.c -- plain fp64 CPU reference for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the package smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library: it is written from the pages' statement of the problem alone, in
 * the order the pages give the steps, with no tiling, fusion or reordering.
 *
 * Sources (web pages on nano-vLLM; titles abbreviated):
 *   [Atlas]  "Visual atlas" figure index (diomchen.github.io/reference/visual-atlas)
 *   [Course] "nano-vLLM offline" interactive course (3479845.xyz/nano-vllm)
 *   [Guide]  "nano-vLLM interactive guide: 13 chapters" (blog-mushroom.pages.dev)
 *   [Notes]  "Nano-vLLM reading notes, ch.1 overview" (wsj040303.github.io)
 *
 * Data conventions (fixed by the library's C-ABI, restated here so this file
 * stands alone):
 *   - bf16 values arrive as their 16-bit patterns (uint16_t) and are widened
 *     exactly to double; all arithmetic is in double.
 *   - q, k, v, out are [tokens, heads, head_dim], tokens of all sequences
 *     flattened back to back; cu_seqlens[s]..cu_seqlens[s+1] are sequence s's
 *     rows ([Atlas] figure index, flattening example cu_seqlens=[0,3,5]).
 *   - the pools are [num_blocks, block_size, kv_heads, head_dim]: physical
 *     block b, offset o inside it.
 *   - block_tables is [num_seqs, max_blocks]: logical block -> physical block
 *     ([Course] "THE IMPORTANT DETAILS" item 02; [Atlas] ch.25 captions).
 *
 * Readings taken where the pages leave a step open:
 *   - Q head h reads K/V head h / (Hq/Hkv): consecutive heads form a group
 *     ([Atlas] figure index GQA example and ch.18: several Q heads share one
 *     K/V head, without a physical copy).
 *   - For a query chunk of q_len rows against k_len keys (k_len >= q_len), the
 *     chunk is the last q_len positions, so row i sits at absolute position
 *     off + i with off = k_len - q_len and sees keys j <= off + i; the
 *     diagonal is visible ([Atlas] ch.17 captions: upper triangle masked,
 *     diagonal kept; a cached chunk's non-square mask carries the offset).
 *   - The scale multiplies q.k before the softmax ([Course] item 01 names the
 *     scaling step that its figures omit).
 *   - A slot value < 0 means "no token here" and is skipped by the store.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Slot of every new token.  Sequence s contributes q_len = cu_seqlens_q[s+1] -
 * cu_seqlens_q[s] new tokens, which are its last q_len positions out of
 * seqlens_k[s] in total.  For the token at logical position pos:
 *   logical block  = pos / block_size
 *   offset         = pos % block_size
 *   physical block = block_tables[s][logical block]
 *   slot           = physical block * block_size + offset
 * ([Atlas] figure index, slot example T=5, block_size=2, block_table=[3,0,4]:
 * per token, logical block, offset, physical block and slot.)
 * Returns 0, or -1 if a table entry needed is negative or past max_blocks.
 */
int oracle_slot_mapping(const int32_t *cu_seqlens_q, const int32_t *seqlens_k,
                        int32_t num_seqs, const int32_t *block_tables,
                        int32_t max_blocks, int32_t block_size, int32_t *slots)
{
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t q_len = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        int32_t first = seqlens_k[s] - q_len;
        for (int32_t i = 0; i < q_len; ++i) {
            int32_t pos = first + i;
            int32_t logical = pos / block_size;
            int32_t offset = pos % block_size;
            if (logical < 0 || logical >= max_blocks)
                return -1;
            int32_t physical = block_tables[(int64_t)s * max_blocks + logical];
            if (physical < 0)
                return -1;
            slots[cu_seqlens_q[s] + i] = physical * block_size + offset;
        }
    }
    return 0;
}

/*
 * KV-cache write: the K and V rows of token t go to the pool cell named by
 * slot_mapping[t] ([Guide] ch.08 "attention and cache writes"; [Course]
 * "ACCURACY & SCOPE": the input token's KV is written before sampling).
 * The copy is exact: bits in, bits out.
 */
void oracle_store(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
                  int32_t num_tokens, int32_t kv_heads, int32_t head_dim,
                  int32_t block_size, uint16_t *k_cache, uint16_t *v_cache)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int32_t slot = slot_mapping[t];
        if (slot < 0)
            continue;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        for (int32_t h = 0; h < kv_heads; ++h) {
            for (int32_t x = 0; x < head_dim; ++x) {
                int64_t src = ((int64_t)t * kv_heads + h) * head_dim + x;
                int64_t dst = ((block * block_size + offset) * kv_heads + h) * head_dim + x;
                k_cache[dst] = k[src];
                v_cache[dst] = v[src];
            }
        }
    }
}

/*
 * Key/value row j of sequence s for KV head h, widened to double.
 * Paged source: block_tables[s][j / block_size], offset j % block_size
 * ([Atlas] figure index slot example; [Course] item 02).
 * Flat source: row cu_seqlens_k[s] + j of k/v ([Atlas] flattening example).
 */
static void gather_row(const uint16_t *flat, const uint16_t *pool,
                       const int32_t *block_tables, int32_t max_blocks, int32_t block_size,
                       const int32_t *cu_seqlens_k, int32_t s, int32_t j,
                       int32_t kv_heads, int32_t h, int32_t head_dim, double *dst)
{
    const uint16_t *row;
    if (pool != NULL) {
        int64_t physical = block_tables[(int64_t)s * max_blocks + j / block_size];
        int64_t offset = j % block_size;
        row = pool + ((physical * block_size + offset) * kv_heads + h) * head_dim;
    } else {
        int64_t r = (int64_t)cu_seqlens_k[s] + j;
        row = flat + (r * kv_heads + h) * head_dim;
    }
    for (int32_t x = 0; x < head_dim; ++x)
        dst[x] = widen_bf16(row[x]);
}

/*
 * Causal attention of every query row against its sequence's keys.
 *
 * For sequence s with q_len query rows and k_len keys, Q head h, KV head
 * kvh = h / (Hq/Hkv), off = k_len - q_len, and query row i:
 *   visible keys   V_i = { j : 0 <= j <= off + i }
 *   score          S_ij = scale * sum_x q[i,h,x] * K[j,kvh,x]      (sum over d)
 *   max            m = max_{j in V_i} S_ij
 *   weight         p_ij = exp(S_ij - m)
 *   normaliser     l = sum_{j in V_i} p_ij
 *   output         out[i,h,x] = sum_{j in V_i} p_ij * V[j,kvh,x] / l  (sum over Tk)
 * ([Atlas] ch.16 captions: the three steps scores -> softmax -> weighted V,
 * one probability row per query; figure index single-head causal example: the
 * first sum runs over d, the second over Tk.)  Only visible keys enter the
 * sums: the mask is a set, not an additive -inf.
 *
 * Key source: if k_cache is non-NULL, keys come from the pools through
 * block_tables and k_len = seqlens_k[s]; otherwise from flat k/v through
 * cu_seqlens_k and k_len = cu_seqlens_k[s+1] - cu_seqlens_k[s].
 * Decode is the case q_len = 1 ([Atlas] ch.21 captions: one decode step).
 *
 * Returns 0, or -1 when a sequence has q_len > k_len or Hq % Hkv != 0.
 */
int oracle_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const uint16_t *k_cache, const uint16_t *v_cache,
                     const int32_t *block_tables, int32_t max_blocks, int32_t block_size,
                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                     const int32_t *seqlens_k, int32_t num_seqs,
                     int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                     double scale, double *out)
{
    if (kv_heads <= 0 || q_heads % kv_heads != 0)
        return -1;
    int32_t group = q_heads / kv_heads;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t q_len = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        int32_t k_len = k_cache ? seqlens_k[s] : cu_seqlens_k[s + 1] - cu_seqlens_k[s];
        if (q_len > k_len)
            return -1;
    }

    int64_t tasks = (int64_t)num_seqs * kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < tasks; ++task) {
        int32_t s = (int32_t)(task / kv_heads);
        int32_t kvh = (int32_t)(task % kv_heads);
        int32_t q_len = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        int32_t k_len = k_cache ? seqlens_k[s] : cu_seqlens_k[s + 1] - cu_seqlens_k[s];
        int32_t off = k_len - q_len;
        if (q_len == 0)
            continue;

        /* Gather this sequence's keys and values for KV head kvh. */
        double *K = malloc(sizeof(double) * (size_t)k_len * head_dim + 1);
        double *V = malloc(sizeof(double) * (size_t)k_len * head_dim + 1);
        double *S = malloc(sizeof(double) * (size_t)k_len + 1);
        double *qi = malloc(sizeof(double) * (size_t)head_dim);
        for (int32_t j = 0; j < k_len; ++j) {
            gather_row(k, k_cache, block_tables, max_blocks, block_size, cu_seqlens_k,
                       s, j, kv_heads, kvh, head_dim, K + (int64_t)j * head_dim);
            gather_row(v, v_cache, block_tables, max_blocks, block_size, cu_seqlens_k,
                       s, j, kv_heads, kvh, head_dim, V + (int64_t)j * head_dim);
        }

        for (int32_t h = kvh * group; h < (kvh + 1) * group; ++h) {
            for (int32_t i = 0; i < q_len; ++i) {
                int64_t row = (int64_t)cu_seqlens_q[s] + i;
                const uint16_t *qrow = q + (row * q_heads + h) * head_dim;
                for (int32_t x = 0; x < head_dim; ++x)
                    qi[x] = widen_bf16(qrow[x]);

                int32_t last = off + i; /* largest visible key index */

                /* scores over the visible keys: first sum, over d */
                for (int32_t j = 0; j <= last; ++j) {
                    double dot = 0.0;
                    for (int32_t x = 0; x < head_dim; ++x)
                        dot += qi[x] * K[(int64_t)j * head_dim + x];
                    S[j] = scale * dot;
                }
                /* softmax over the visible keys */
                double m = S[0];
                for (int32_t j = 1; j <= last; ++j)
                    if (S[j] > m)
                        m = S[j];
                double l = 0.0;
                for (int32_t j = 0; j <= last; ++j) {
                    S[j] = exp(S[j] - m);
                    l += S[j];
                }
                /* weighted values: second sum, over Tk */
                double *o = out + (row * q_heads + h) * head_dim;
                for (int32_t x = 0; x < head_dim; ++x) {
                    double acc = 0.0;
                    for (int32_t j = 0; j <= last; ++j)
                        acc += S[j] * V[(int64_t)j * head_dim + x];
                    o[x] = acc / l;
                }
            }
        }
        free(K);
        free(V);
        free(S);
        free(qi);
    }
    return 0;
}
