/*
 * pa.h -- C-ABI of libpa.so: attention over a paged KV cache on AMD MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * Sources (web pages on the nano-vLLM teaching engine; titles abbreviated):
 *   [Atlas]  "Visual atlas" figure index (diomchen.github.io/reference/visual-atlas)
 *   [Course] "nano-vLLM offline" interactive course (3479845.xyz/nano-vllm)
 *   [Guide]  "nano-vLLM interactive guide: 13 chapters" (blog-mushroom.pages.dev)
 *   [Notes]  "Nano-vLLM reading notes, ch.1 overview" (wsj040303.github.io)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Element types.  q, k, v, pools and out are bf16 (IEEE-754 binary32 with the
 *   low 16 bits dropped).  Index arrays are int32.  Arithmetic is fp32 with
 *   bf16 MFMA inputs; outputs are rounded to bf16 (nearest, ties to even).
 * Layouts (row-major, contiguous):
 *   q, out            [tokens, num_q_heads, head_dim]
 *   k, v              [tokens, num_kv_heads, head_dim]
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim]; the pool
 *                     row of slot s is element offset s * num_kv_heads * head_dim
 *   block_tables      [num_seqs, max_blocks_per_seq]; entry [s][b] is the physical
 *                     block holding sequence s's logical block b ([Course] "THE
 *                     IMPORTANT DETAILS" item 02; [Atlas] ch.25 captions)
 *   cu_seqlens_*      [num_seqs + 1] prefix sums of per-sequence lengths; sequence
 *                     s owns rows cu[s] .. cu[s+1]-1 ([Atlas] figure index,
 *                     flattening example cu_seqlens=[0,3,5])
 * Memory.  Pointers marked (device) are HIP device pointers, (host) are host
 *   pointers.  The caller owns every buffer: pools, metadata, workspace and
 *   outputs.  The library allocates no device memory and never synchronises,
 *   so every device entry point may be captured in a HIP graph; grid sizes
 *   come only from the host integers passed in, never from device data.
 * GQA.  Q head h reads KV head h / (num_q_heads / num_kv_heads): consecutive
 *   Q heads form a group sharing one K/V head, with no physical copy ([Atlas]
 *   figure index GQA example, ch.18 captions).
 * Errors.  Host-checkable problems (NULL pointers, inconsistent or unsupported
 *   sizes, a workspace too small) return a status before anything is launched.
 *   Device-resident values (slots, tables, lengths) are not validated: values
 *   outside the ranges stated below are undefined behaviour.  A failed launch
 *   returns PA_ERR_LAUNCH.
 * Threads.  The device entry points keep no state between calls (only each
 *   device's compute-unit count, read once) and are re-entrant; calls on one
 *   stream execute in order.  A block manager (pa_bm_*) belongs to one thread.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,        /* a required pointer is NULL                        */
    PA_ERR_SHAPE = 2,       /* sizes negative, zero where not allowed, or
                               inconsistent with each other                      */
    PA_ERR_UNSUPPORTED = 3, /* valid sizes this build has no kernel for           */
    PA_ERR_WORKSPACE = 4,   /* workspace_bytes smaller than required              */
    PA_ERR_LAUNCH = 5,      /* the HIP runtime reported a launch error            */
    PA_ERR_SCRATCH = 6,     /* the call needs more than the library's fixed device
                               scratch (pa_decode_noalloc)                       */
    PA_ERR_GRAPH = 7        /* the HIP runtime refused a graph capture,
                               instantiation or launch (pa_graph_*)              */
} pa_status;

/* Static, NUL-terminated description of a status code (never NULL). */
const char *pa_status_string(int status);

/*
 * Slot of every new token (host-side step metadata, as the model runner's
 * prefill/decode preparation builds it: [Notes] "key state and module
 * boundaries"; [Atlas] ch.29 captions).
 *
 * Sequence s has cu_seqlens_q[s+1] - cu_seqlens_q[s] new tokens, which are the
 * last ones of its seqlens_k[s] tokens.  The token at logical position pos
 * goes to
 *     slot = block_tables[s][pos / block_size] * block_size + pos % block_size
 * ([Atlas] figure index, slot example T=5, block_size=2, block_table=[3,0,4]).
 *
 * cu_seqlens_q  (host) [num_seqs+1], non-decreasing, cu_seqlens_q[0] == 0
 * seqlens_k     (host) [num_seqs], seqlens_k[s] >= its new-token count
 * block_tables  (host) [num_seqs, max_blocks_per_seq]
 * slot_mapping  (host, out) [num_tokens], num_tokens == cu_seqlens_q[num_seqs]
 * Returns PA_ERR_SHAPE if a position needs a table entry that is past
 * max_blocks_per_seq or negative; slot_mapping is then left partly written.
 */
int pa_slot_mapping(const int32_t *cu_seqlens_q, const int32_t *seqlens_k, int32_t num_seqs,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    int32_t block_size, int32_t *slot_mapping, int32_t num_tokens);

/*
 * KV-cache store: for every token t with slot_mapping[t] >= 0,
 *     k_cache row slot_mapping[t]  <-  k[t]      and the same for v,
 * copied bit for bit ([Guide] ch.08 "attention and cache writes"; [Course]
 * "ACCURACY & SCOPE": a token's K/V is written before sampling).  A negative
 * slot marks a padding token and is skipped.
 *
 * k, v          (device) [num_tokens, num_kv_heads, head_dim] bf16
 * k_cache/v_cache (device, in/out) [num_blocks, block_size, num_kv_heads, head_dim]
 * slot_mapping  (device) [num_tokens]; each slot < num_blocks * block_size and
 *               no two tokens share a slot
 * num_tokens may be 0 (nothing is launched).  head_dim * num_kv_heads must be
 * a multiple of 8.  k and v rows must not overlap the pools.
 */
int pa_store_kv(const void *k, const void *v, void *k_cache, void *v_cache,
                const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                hipStream_t stream);

/*
 * Placement of the two pools in one reservation.  The engine reserves the
 * whole KV pool once, up front, and afterwards only changes which blocks the
 * requests hold ([Course] "THE IMPORTANT DETAILS" item 02).  When k_cache and
 * v_cache share one allocation, this gives its size and where v_cache starts:
 * k_cache at byte 0, v_cache after it at an offset whose remainder modulo
 * 1024 bytes is 384.  The kernels read a token's K row and V row at the same
 * time; with the two pools at the same address modulo 1 KiB those reads land
 * in the same part of the HBM interleave and the decode loses bandwidth
 * (measured on MI355X: 256-sequence decode 383 -> 354 us, 16 x 32768-token
 * decode 359 -> 346 us).  Any other placement of 16-byte aligned pools is
 * equally correct for every entry point; only the speed changes.
 *
 * v_offset  (host, out) byte offset of v_cache from the start of the allocation
 * Returns the allocation size in bytes (k_cache bytes + padding + v_cache
 * bytes), or 0 with *v_offset untouched if v_offset is NULL, a size is not
 * positive, or the size does not fit in a size_t.
 */
size_t pa_kv_pool_layout(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, size_t *v_offset);

/*
 * Variable-length causal prefill attention.
 *
 * For sequence s: q_len = cu_seqlens_q[s+1] - cu_seqlens_q[s] query rows and
 * k_len = cu_seqlens_k[s+1] - cu_seqlens_k[s] keys, q_len <= k_len.  The
 * queries are the last q_len positions, so query row i (absolute position
 * k_len - q_len + i) sees keys j <= k_len - q_len + i: the causal mask keeps
 * the diagonal and, when a cached prefix precedes the chunk, is offset by the
 * cached length ([Atlas] ch.17 captions; ch.26: after a prefix hit the query
 * length differs from the key length).  With p_ij = exp(S_ij - max) over the
 * visible keys, S_ij = scale * q_i . k_j, the output row is
 * sum_j p_ij v_j / sum_j p_ij ([Atlas] ch.16 captions; figure index single-head
 * causal example: first sum over d, second over Tk).
 *
 * Key source:
 *   block_tables == NULL: keys are rows cu_seqlens_k[s] .. of flat k/v (no
 *     cache); k_cache/v_cache are ignored and may be NULL.
 *   block_tables != NULL: key j of sequence s is pool row
 *     block_tables[s][j / block_size] * block_size + j % block_size; k/v are
 *     ignored and may be NULL.  The chunk's own K/V must have been stored
 *     (pa_store_kv) before this call.  Table entries past the last block a
 *     sequence uses are never read.
 *
 * q        (device) [cu_seqlens_q[num_seqs], num_q_heads, head_dim] bf16
 * out      (device, out) same shape as q, bf16; rows of every sequence written
 * max_seqlen_q  >= every q_len (sizes the grid); max_seqlen_k >= every k_len
 * max_blocks_per_seq  row length of block_tables (paged source only)
 * block_size    any value >= 1 (paged source only)
 * Supported: head_dim == 128; num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 */
int pa_prefill_varlen(const void *q, const void *k, const void *v,
                      const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                      int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, float scale, void *out, hipStream_t stream);

/*
 * Bytes of device workspace pa_prefill_varlen_ws needs for these sizes on the
 * current device; 0 when such a batch is not split (then the workspace is
 * ignored and may be NULL) or the sizes are invalid.  A batch is split when it
 * has at most one (query block, sequence, KV head) item per two compute units
 * and max_seqlen_k >= 2048: few, long items, whose length then sets the time.
 */
size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);

/*
 * pa_prefill_varlen with a workspace: the same operation and arguments, plus
 * a key split for batches of few, long query blocks (see
 * pa_prefill_workspace_size; there the longest blocks set the time).  Each
 * query block with at least 4 key tiles of 64 keys is then computed as two
 * halves of its key range by two workgroups;
 * the second to finish merges the two partial softmax states, rescaling both
 * to the larger running maximum (the log-sum-exp combination that lets the
 * blocked computation of [Atlas] ch.22 avoid the full score matrix).  Results
 * differ from pa_prefill_varlen only by fp32 rounding (each half's partial
 * O / l, running max and sum are stored in fp32, so every bf16 value range is
 * covered), and they do not depend on which half finishes second: both halves
 * enter the merge in their stored form and in key order, so repeated calls
 * give the same bits.
 *
 * workspace  (device) >= pa_prefill_workspace_size(...) bytes (sized on the
 *            device the call runs on), 16-byte aligned, zero-filled before its
 *            first use.  It holds the partials and, at its end, one arrival
 *            counter per item; every call returns the counters to zero, so the
 *            buffer can be reused without clearing.  Calls that share a
 *            workspace must not overlap in time (issue them on one stream).
 * Errors as pa_prefill_varlen, plus PA_ERR_WORKSPACE (workspace_bytes too small)
 * and PA_ERR_NULL (workspace NULL while one is needed).
 */
int pa_prefill_varlen_ws(const void *q, const void *k, const void *v,
                         const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, int32_t max_blocks_per_seq,
                         const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                         int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, float scale, void *workspace,
                         size_t workspace_bytes, void *out, hipStream_t stream);

/*
 * Number of key partitions pa_decode splits the longest context into, for
 * the given partition_size (0 = the library's choice for these sizes, which
 * depends on the group size num_q_heads / num_kv_heads).
 * Returns 0 for invalid sizes.
 */
int32_t pa_decode_num_partitions(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * Bytes of device workspace pa_decode needs for these sizes (0 for invalid
 * sizes).  The workspace holds one fp32 partial output row plus its running
 * max and sum per (sequence, Q head, partition).
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len,
                                int32_t partition_size);

/*
 * Paged decode attention: one new query per sequence over its whole history
 * ([Atlas] ch.21 captions: a decode step's query attends over every cached
 * token; the newest token's K/V is written first, so context_lens counts it).
 *
 * For sequence s and Q head h: keys j < context_lens[s], key j at pool row
 * block_tables[s][j / block_size] * block_size + j % block_size; output
 * sum_j p_j v_j / sum_j p_j with p_j = exp(scale q.k_j - max).
 * The keys are split into partitions of partition_size tokens, each reduced
 * to a partial (running max, sum, unnormalised output) in the workspace, and
 * a second kernel combines the partials (log-sum-exp merge); with a single
 * partition the first kernel writes the output and the second is not
 * launched.  context_lens[s] == 0 yields a zero output row.
 *
 * q             (device) [num_seqs, num_q_heads, head_dim] bf16
 * k_cache/v_cache (device) pools as above
 * block_tables  (device) [num_seqs, max_blocks_per_seq]
 * context_lens  (device) [num_seqs], 0 <= context_lens[s] <= max_context_len
 * workspace     (device) >= pa_decode_workspace_size(...) bytes, any content
 * out           (device, out) [num_seqs, num_q_heads, head_dim] bf16
 * partition_size  0 (library's choice: one partition per sequence when
 *               num_seqs * num_kv_heads >= 1024, or >= 4096 when num_q_heads ==
 *               num_kv_heads; otherwise partitions of at most
 *               4096 keys that shrink toward the end of each sequence: counted
 *               from the end of the context rounded up to 64, 256, 256, 512, 512,
 *               1024, 1024, 2048, 2048, then 4096 keys, the first partition
 *               taking the rest; with num_q_heads / num_kv_heads == 8 the
 *               smallest are 512 keys: 512, 512, 1024, 1024, 2048, 2048, 4096s)
 *               or a multiple of 32: fixed partitions of that many keys
 * Supported: head_dim == 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 * num_seqs <= 65535 and at most 65535 partitions (max_context_len /
 * partition_size rounded up), else PA_ERR_UNSUPPORTED.
 */
int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, float scale, int32_t partition_size,
              void *workspace, size_t workspace_bytes, void *out, hipStream_t stream);

/*
 * Fused decode step: the KV-cache store of each sequence's new token and the
 * paged decode over its history, in one launch (plus the reduce pass when a
 * context is split into several partitions).  Equivalent to
 *     pa_store_kv(k_new, v_new, k_cache, v_cache, slot_mapping, num_seqs, ...)
 *     pa_decode(q, k_cache, v_cache, ...)
 * when slot_mapping[s] is the pool row of position context_lens[s] - 1 (as
 * pa_slot_mapping computes it): the workgroup that owns that position writes
 * the new K/V rows to the slot and attends to them from registers instead of
 * re-reading the pool ([Atlas] ch.21: the sampled token has no K/V until its
 * decode step; [Course] ACCURACY & SCOPE: the token's KV is written first).
 * A negative slot skips the store and the position is read from the pool.
 *
 * k_new, v_new  (device) [num_seqs, num_kv_heads, head_dim] bf16, 16-byte aligned
 * slot_mapping  (device) [num_seqs]
 * context_lens  (device) [num_seqs], >= 1 for every sequence with a new token
 * Other arguments as pa_decode; the outputs and pool contents equal the
 * unfused pair's up to fp32 summation order.
 */
int pa_decode_store(const void *q, const void *k_new, const void *v_new,
                    const int32_t *slot_mapping, void *k_cache, void *v_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, int32_t partition_size, void *workspace,
                    size_t workspace_bytes, void *out, hipStream_t stream);

/*
 * The two passes of pa_decode, for callers that schedule or time them apart.
 * Arguments are those of pa_decode.  pa_decode_split runs the partition pass:
 * it writes the final output row of every sequence whose context fits in one
 * partition, and the partials of the others into the workspace.
 * pa_decode_reduce then merges the partials (nothing to do when every
 * context fits one partition).  Calling pa_decode_split and then pa_decode_reduce on one stream
 * with the same arguments is exactly pa_decode.
 */
int pa_decode_split(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, int32_t partition_size,
                    void *workspace, size_t workspace_bytes, void *out, hipStream_t stream);
int pa_decode_reduce(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, float scale, int32_t partition_size,
                     void *workspace, size_t workspace_bytes, void *out, hipStream_t stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same operation, arguments (minus workspace) and
 * results as pa_decode: the partials of a split context go to a fixed device
 * array inside the library, PA_NOALLOC_SCRATCH_BYTES on each device, held
 * until the process ends.  The call allocates nothing; its first call on a
 * device looks up that device's copy of the array.
 *
 * Returns PA_ERR_SCRATCH, launching nothing, when
 * pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
 * max_context_len, partition_size) exceeds PA_NOALLOC_SCRATCH_BYTES (for
 * example 16 sequences x 32 Q heads x 32768 keys need 8.5 MB at the default
 * partition size).  Every call on one device shares that device's array:
 * calls that may overlap in time on one device (other streams, other host
 * threads) race and must not be issued; calls on one stream are ordered.
 * Nothing in the array needs to start at zero.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int pa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, float scale, int32_t partition_size, void *out,
                      hipStream_t stream);

/*
 * Host block manager with prefix caching.
 *
 * Owns the ids of a pool of num_blocks physical blocks (the pools themselves
 * stay the caller's device buffers) and hands them to sequences as block
 * tables.  The pool is reserved once; allocating and freeing only change
 * which ids a sequence holds ([Course] "THE IMPORTANT DETAILS" item 02).  It
 * keeps, per block, a reference count and, for a full block, a prefix key
 * ([Notes] "key state and module boundaries").
 *
 * Sharing rule ([Course] "ACCURACY & SCOPE"; [Atlas] ch.25, ch.28 captions):
 * only full blocks are shared, never the trailing partial block.  A full
 * block's key chains the key of the block before it, a caller salt (say, a
 * model or adapter id: requests with different salts never share), and its
 * tokens; a candidate hit is confirmed by comparing the stored tokens, so a
 * hash collision cannot share wrong data.  Once one block of a request
 * misses, every later block is fresh.  A block whose count drops to zero keeps
 * its key and content and can still be hit until it is handed out fresh;
 * fresh blocks are taken least-recently-freed first.
 *
 * The manager touches no GPU state and is not thread-safe: one thread (the
 * scheduler) owns a manager.  Token ids are opaque int32 values.
 */
typedef struct pa_block_manager pa_block_manager;

/* New manager over num_blocks blocks of block_size tokens (all free), or NULL
 * when a size is < 1 or memory runs out.  Release with pa_bm_destroy. */
pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager *bm);

/* Blocks with reference count 0 (cached or not); -1 for NULL. */
int32_t pa_bm_num_free(const pa_block_manager *bm);

/* Reference count of one block id; -1 for NULL or an id out of range. */
int32_t pa_bm_ref_count(const pa_block_manager *bm, int32_t block);

/* Free blocks pa_bm_allocate would take for this prompt now (a hit on a free
 * cached block counts, since it leaves the free pool); -1 on bad arguments. */
int32_t pa_bm_blocks_needed(const pa_block_manager *bm, const int32_t *tokens,
                            int32_t num_tokens, uint64_t salt);

/*
 * Block table for a new request whose prompt is tokens[0 .. num_tokens-1]
 * (all host memory).  Entries 0 .. ceil(num_tokens/block_size)-1 of
 * block_table [max_blocks] receive block ids, the rest -1.
 * *num_cached_tokens receives the length of the shared prefix (a multiple of
 * block_size): those positions already hold this prompt's K/V, so the prefill
 * stores and attends only positions from there on ([Atlas] ch.26: after a
 * prefix hit, the query covers the uncached tail and the keys the whole
 * prompt).  The block holding the last prompt token is never taken from the
 * cache, so num_cached_tokens < num_tokens for any non-empty prompt: the
 * prefill has at least one query row and writes only blocks that this request
 * holds alone.  Returns PA_ERR_WORKSPACE,
 * taking nothing, when fewer than pa_bm_blocks_needed blocks are free;
 * PA_ERR_SHAPE when the table is too short.
 */
int pa_bm_allocate(pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens,
                   uint64_t salt, int32_t *block_table, int32_t max_blocks,
                   int32_t *num_cached_tokens);

/*
 * One decode step of a running sequence: tokens[0 .. num_tokens-1] is its whole
 * token list including the token being appended (position num_tokens-1).
 * When that position opens a new block, a fresh block is taken into
 * block_table (PA_ERR_WORKSPACE, nothing changed, if none is free); when it
 * fills a block, that block is registered for later prefix hits.  Returns
 * PA_ERR_SHAPE for a table too short or inconsistent with num_tokens.
 */
int pa_bm_append(pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens,
                 uint64_t salt, int32_t *block_table, int32_t max_blocks);

/* Release a finished (or preempted) sequence's blocks: every id >= 0 among
 * block_table[0 .. num_blocks-1] loses one reference; blocks reaching zero
 * become free (most recent last).  PA_ERR_SHAPE for an id out of range or not
 * held; entries before it in reverse order may already have been released. */
int pa_bm_free(pa_block_manager *bm, const int32_t *block_table, int32_t num_blocks);

/*
 * Native HIP graphs of library calls, for a serving loop that replays the same
 * step with new values: the decode step is captured once and replayed, so a step
 * costs one graph launch instead of one host launch per kernel ([Course] "THE
 * IMPORTANT DETAILS" item 03: the decode loop runs under a captured graph;
 * [Atlas] ch.26 captions: a replay reads new values from the same preallocated
 * buffers, whose addresses and shapes the capture fixed).
 *
 * pa_graph_begin(stream) starts capturing the work issued on `stream`
 * (hipStreamBeginCapture, thread-local mode): calls on that stream from this
 * thread until pa_graph_end are recorded, not run.  Every device entry point of
 * this library can be captured (none allocates, synchronises or clears memory
 * with a memset node).  pa_graph_end(stream, &graph) ends the capture and
 * instantiates the result into *graph, an opaque handle the caller owns and
 * releases with pa_graph_destroy.  pa_graph_launch(graph, stream) enqueues one
 * replay on `stream`: the captured kernels run again with the captured pointers
 * and sizes, reading whatever the buffers hold when they run, in stream order with
 * the caller's other work on that stream.  A graph may be launched any number of
 * times, but replays that share buffers (a workspace in particular) must not
 * overlap in time: launch them on one stream.  pa_graph_node_counts reports what
 * was captured: *kernels receives the number of kernel nodes and *others the
 * number of nodes of any other kind.
 *
 * stream   a created stream (not the NULL stream)
 * Errors: PA_ERR_NULL (NULL stream, graph or out-pointer), PA_ERR_GRAPH (the
 * runtime refused the capture, the instantiation or the launch).  pa_graph_end
 * always ends the capture; on failure *graph is set to NULL.
 */
typedef struct pa_graph pa_graph;

int pa_graph_begin(hipStream_t stream);
int pa_graph_end(hipStream_t stream, pa_graph **graph);
int pa_graph_launch(const pa_graph *graph, hipStream_t stream);
int pa_graph_node_counts(const pa_graph *graph, size_t *kernels, size_t *others);
void pa_graph_destroy(pa_graph *graph);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
