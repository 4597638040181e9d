/*
 * mi_attn.h -- C ABI of an MI355X (gfx950) attention library: exact
 * scaled-dot-product attention computed FlashAttention-style, a paged-KV
 * decode with split-KV partitions and a merge pass, a fused RoPE + paged
 * KV-cache write, and the host-side block pool that hands out cache blocks.
 *
 * Source of the operations: the tutorial "Fast Attention Kernels and
 * Operator Fusion" (Machine Learning Mastery).  Section names below refer to
 * it.
 *
 * General conventions
 *   - Every pointer named *device* is device memory owned by the caller; the
 *     library never allocates, frees or keeps device memory.  Pool functions
 *     take host memory only.
 *   - Every launch function validates all arguments first.  On any error it
 *     returns a negative attn_status, records a message for attn_last_error()
 *     and makes no HIP call at all: nothing is launched or changed.
 *   - Launch functions enqueue on `stream` (NULL = the default stream) and
 *     return without synchronising.  They do not allocate and do not read
 *     device memory on the host, so a caller may capture them in a HIP graph
 *     (replay needs the same addresses and shapes).
 *   - Tensors are token-major with the head dimension contiguous.  Strides
 *     are in elements.  Device pointers must be 16-byte aligned and every
 *     stride a multiple of 8 elements (bf16) or 4 elements (f32).
 *   - Supported: head_dim 64 or 128; dtype F32 or BF16 (attn_decode_paged_rope:
 *     BF16 only); block_size 16; num_q_heads a multiple of num_kv_heads.
 *     Anything else returns ATTN_E_UNSUPPORTED.  BF16 runs on the matrix
 *     cores with fp32 accumulation; F32 runs full-precision VALU kernels
 *     (for parity work, not a performance path).
 *   - Paged cache layout (one pool per tensor):
 *       k_cache [num_blocks][num_kv_heads][16][head_dim]   (token-major)
 *       v_cache [num_blocks][num_kv_heads][head_dim][16]   (token-minor)
 *     Storing a value block token-minor lets the PV contraction read 4 or 8
 *     consecutive tokens of one channel with one load.
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* attn_stream_t; /* same handle as hipStream_t */

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* null pointer, bad size, misaligned pointer or stride */
  ATTN_E_UNSUPPORTED = -2, /* valid in principle, not supported by these kernels */
  ATTN_E_NOMEM = -3,       /* pool exhausted or workspace too small */
  ATTN_E_STATE = -4,       /* double free, refcount misuse */
  ATTN_E_DEVICE = -5       /* a HIP call failed */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Text of the last error on the calling thread ("" if none).  Valid until
 * that thread's next call into the library. */
ATTN_API const char* attn_last_error(void);

/* -------------------------------------------------------------------------
 * attn_prefill -- contiguous attention  O = softmax(Q K^T * scale + M) V.
 *
 * Defined by the attention equation of §FlashAttention-Style Kernels (an
 * additive mask M; d is the head dimension) and computed the way the same
 * section describes FlashAttention: per tile of queries, score blocks are
 * formed against tiles of keys, the running softmax statistics (row max and
 * row sum) are updated and the output is accumulated on chip; the Tq x Tk
 * score matrix never reaches device memory.
 *
 *   q   device [batch][seqlen_q][num_q_heads][head_dim]   (strides q_strides)
 *   k,v device [batch][seqlen_k][num_kv_heads][head_dim]  (k_strides, v_strides)
 *   o   device, same shape as q, written                  (o_strides)
 *   lse device float [batch][num_q_heads][seqlen_q], written if non-NULL:
 *       natural-log sum of exp of the scaled, masked scores of each row.
 *   *_strides[3]: element strides of the batch, token and head dimensions.
 *   Query head h reads key/value head h / (num_q_heads / num_kv_heads).
 *   scale: 0 means 1/sqrt(head_dim).
 *   causal: non-zero masks key j for query i unless j <= i + seqlen_k - seqlen_q
 *     (bottom-right aligned); requires seqlen_k >= seqlen_q.
 *   A query row that sees no key (only possible when seqlen_k == 0) gets O = 0.
 *   q, k, v, o must not overlap o.
 *   workspace    optional device scratch (256-byte aligned) of
 *                attn_prefill_workspace_size(...) bytes.  When that size is
 *                non-zero and a workspace is given, launches with too few
 *                query tiles to fill the GPU cut each query tile's keys into
 *                shares computed by separate workgroups, and a second kernel
 *                merges the shares' partial (max, sum, output) exactly, the
 *                recombination of the online softmax that §FlashAttention-
 *                Style Kernels describes.  NULL: one pass per query tile.  A
 *                non-NULL workspace smaller than the size returns
 *                ATTN_E_NOMEM.  Concurrent calls need separate workspaces.
 * ---------------------------------------------------------------------- */
ATTN_API size_t attn_prefill_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   attn_dtype dtype);
ATTN_API int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                 const int64_t q_strides[3], const int64_t k_strides[3],
                 const int64_t v_strides[3], const int64_t o_strides[3],
                 float scale, int32_t causal, attn_dtype dtype,
                 void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_prefill_masked -- attn_prefill with a general additive mask.
 *
 * §FlashAttention-Style Kernels writes attention as softmax(Q K^T / sqrt(d)
 * + M) V with an additive mask M; attn_prefill covers M = 0 and the causal
 * M.  Here M is given: element (b, h, i, j) (batch, query head, query row,
 * key) is mask[b*mask_strides[0] + h*mask_strides[1] + i*mask_strides[2] + j],
 * fp32, keys contiguous; a stride of 0 broadcasts that dimension (one
 * [Tq][Tk] mask for every batch and head, say).  Entries are finite or
 * -infinity; `causal` applies on top.  A row whose every key is masked
 * yields O = 0 (and LSE = -infinity).  Single pass (no workspace).
 *
 *   mask         device fp32, 16-byte aligned; strides >= 0 and multiples of
 *                4 elements
 *   every other argument as for attn_prefill.
 * ---------------------------------------------------------------------- */
ATTN_API int attn_prefill_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* mask, const int64_t mask_strides[3], int32_t batch,
                        int32_t seqlen_q, int32_t seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, const int64_t q_strides[3], const int64_t k_strides[3],
                        const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                        int32_t causal, attn_dtype dtype, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_prefill_paged -- prefill of new query chunks over a paged KV cache.
 *
 * The same computation as attn_prefill, with keys and values read through
 * a block table as §Paged Attention Kernels describes: logical token t of
 * sequence s lives in physical block block_table[s][t / 16] at offset t % 16;
 * K[t+1] is not assumed to follow K[t].
 *
 *   q            device [total_q][num_q_heads][head_dim], sequences packed
 *   k_cache,
 *   v_cache      device paged pools (layout in the header comment), q's dtype
 *   block_table  device int32 [num_seqs][max_blocks_per_seq]; entries past a
 *                sequence's last block are never read
 *   cu_seqlens_q device int32 [num_seqs + 1]; sequence s owns q rows
 *                cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 (at most max_seqlen_q)
 *   context_lens device int32 [num_seqs]; keys of sequence s, the new tokens
 *                included (they must already be in the cache); must be >= the
 *                sequence's query count
 *   o            device bf16, same shape as q, written
 *   Chunk row i of sequence s sits at position context_lens[s] - n_s + i and,
 *   when causal, sees keys 0 .. that position.
 *   max_context_len  the longest context_lens entry, or 0 for the bound
 *                max_blocks_per_seq * 16.  Only the split plan uses it: a
 *                longer context is still computed whole, by longer shares.
 *   workspace    optional device scratch of
 *                attn_prefill_paged_workspace_size(...) bytes (same meaning
 *                and rules as attn_prefill's).  F32 runs one pass per query
 *                tile and ignores the workspace and the flags below.
 * ---------------------------------------------------------------------- */
ATTN_API size_t attn_prefill_paged_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                         int32_t max_context_len, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim);
ATTN_API int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* cu_seqlens_q, const int32_t* context_lens,
                       void* o, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                       int32_t max_context_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks,
                       float scale, int32_t causal, attn_dtype dtype,
                       void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* attn_prefill_paged_ex -- attn_prefill_paged with a flags word (same
 * arguments otherwise; attn_prefill_paged is this with flags 0).  The
 * results do not depend on the flags: every query row is computed in the
 * same order either way, so the outputs are bit-identical.
 *
 *   ATTN_PREFILL_SHARE_CU  the launch runs while another kernel (a paged
 *                decode on another stream, the usual case in a serving step
 *                that mixes chunked prefill and decode) is given the rest of
 *                the GPU.  The prefill's workgroups then hold a deeper ring
 *                of value tiles in LDS, so that one fits per CU and leaves
 *                room beside it for a decode workgroup; by default two
 *                prefill workgroups share a CU and fill it.  Alone, the
 *                flagged launch is slower.
 *   Other bits: ATTN_E_INVALID.  The workspace size that
 *   attn_prefill_paged_workspace_size reports suffices for either tile. */
#define ATTN_PREFILL_SHARE_CU 1
ATTN_API int attn_prefill_paged_ex(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* context_lens,
                          void* o, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                          int32_t max_context_len,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks,
                          float scale, int32_t causal, attn_dtype dtype, int32_t flags,
                          void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_prefill_paged_masked -- attn_prefill_paged with a general additive
 * mask M (the attention equation of §FlashAttention-Style Kernels).
 *
 * Element (packed query row r, query head h, key position j) of M is
 * mask[r*mask_strides[0] + h*mask_strides[1] + j], fp32, keys contiguous, for
 * j < mask_keys; j counts the logical positions of the row's sequence
 * (0 .. context_lens[s]-1, cached tokens first).  A stride of 0 broadcasts
 * (one row for every head, say).  Entries are finite or -infinity; keys at
 * or past mask_keys are never read and count as masked (-infinity), so
 * mask_keys should be at least the longest context.  `causal` applies on
 * top.  A row whose every key is masked yields O = 0.  Single pass (no
 * workspace, no flags).
 *
 *   mask         device fp32, 16-byte aligned; strides >= 0 and multiples of
 *                4 elements
 *   every other argument as for attn_prefill_paged.
 * ---------------------------------------------------------------------- */
ATTN_API int attn_prefill_paged_masked(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* cu_seqlens_q, const int32_t* context_lens,
                              const float* mask, const int64_t mask_strides[2], int32_t mask_keys,
                              void* o, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                              int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                              int32_t causal, attn_dtype dtype, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_decode_paged -- one query token per sequence over its paged cache.
 *
 * §FlashAttention-Style Kernels: decode has one new query per request and is
 * dominated by reading the growing KV cache; §Paged Attention Kernels: the
 * kernel follows the block table.  Each sequence's context is cut into
 * partitions of `partition_size` tokens.  One workgroup per partition (and
 * kv head slice) computes the partition's running max m, sum l and
 * unnormalised output; the last of a sequence's workgroups to finish combines
 * the partitions exactly (each rescaled by exp(m_p - max_p m_p)).  A sequence
 * with one partition needs no combination.  One kernel launch per call.
 *
 *   q            device [num_seqs][num_q_heads][head_dim] (BF16 or F32; the
 *                caches and o share its dtype)
 *   block_table  device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                a sequence's last block (within its row) may be read, and
 *                are never used
 *   context_lens device int32 [num_seqs], 1 .. max_context_len (the new
 *                token included)
 *   o            device [num_seqs][num_q_heads][head_dim], written
 *   partition_size: 0 = automatic; else a multiple of 16 (whole blocks), at
 *                most 1024 for BF16 (one block-table entry per lane of a
 *                wavefront) and 65536 for F32.
 *   plan         optional device int32 [plan_items][2]: the (sequence,
 *                partition) pairs that attn_decode_paged_plan lists for the
 *                same context lengths, max_context_len, num_kv_heads and
 *                partition_size.  With a plan only those partitions are
 *                dispatched; NULL (plan_items 0): a padded grid of every
 *                sequence x the longest context's partitions, where the empty
 *                ones exit at once.  Entries out of range are skipped; a plan
 *                that omits a real partition leaves that part of the output
 *                unset.
 *   workspace    device scratch (256-byte aligned) of at least
 *                attn_decode_paged_workspace_size(...) bytes (same arguments),
 *                needed when that size is non-zero.  It begins with a block
 *                of arrival counters, one int32 for each (sequence, kv head
 *                slice) pair that a call with these numbers of query and kv
 *                heads may have (65535 sequences x kv heads x
 *                ceil(query heads per kv head / 16); 512 KiB at 2 kv heads),
 *                that must be ZERO before the first call that uses the
 *                workspace (fill it with zeros once after allocating); every
 *                completed call leaves them zero again, so the same
 *                workspace serves later calls with the same numbers of
 *                query and kv heads and any sequence count, contexts and
 *                partition size that fit.  (A call with other head numbers
 *                has a counter block of another size: zero the workspace
 *                again first.)  Calls that overlap on one workspace race; a
 *                plan that lists a partition twice corrupts the counters.
 * ---------------------------------------------------------------------- */
ATTN_API size_t attn_decode_paged_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t partition_size);
ATTN_API int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* context_lens, void* o,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t partition_size, float scale, attn_dtype dtype,
                      const int32_t* plan, int32_t plan_items,
                      void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without a
 * workspace, the same kernels and results bit for bit.  The split-KV
 * scratch (arrival counters, partial outputs and (m, l) pairs, laid out
 * like attn_decode_paged's workspace but with a 4 MiB counter block, room
 * for 65535 sequences x 16 kv head slices whatever the call's head
 * numbers) is a fixed 32 MiB device array of
 * the library's own, which every GPU the library runs on holds until the
 * process ends; the first call on a device finds its address there and
 * zero-fills it with a kernel on `stream`.  Nothing is allocated or freed.
 *   - A call whose partials and (m, l) pairs exceed the 28 MiB after the
 *     counter block, or whose kv head slices exceed 16, returns
 *     ATTN_E_NOMEM (launching nothing): about 140 sequences of 12 query
 *     heads at 32768 tokens with 1024-token partitions fit.
 *   - Every call on one GPU shares that GPU's array, and a completed call
 *     leaves its counters zero for the next, of any shape; calls that overlap on one GPU
 *     (other streams, other threads) race and corrupt each other's results.
 *     Serialise them on one stream.
 * ---------------------------------------------------------------------- */
ATTN_API int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens, void* o,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              int32_t partition_size, float scale, attn_dtype dtype,
                              const int32_t* plan, int32_t plan_items, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_decode_paged_rope -- the decode above, with each sequence's new token
 * rotated and written into the cache by the same launch.
 *
 * §Operator Fusion lists the rotary embedding of queries and keys and the
 * KV-cache update done while keys and values are transformed among the usual
 * fusions; here both are folded into the decode itself.  Equivalent to
 * attn_kv_cache_write_rope(q, k_new, v_new, positions, slot_mapping, ...)
 * (one token per sequence) followed by attn_decode_paged on the rotated q,
 * with the same rotation arithmetic bit for bit, except that q is not
 * modified: the rotated queries go to q_rot_out when it is non-NULL.
 *
 *   q_rot_out    device bf16 [num_seqs][num_q_heads][head_dim] or NULL; must
 *                not alias q (other workgroups of a sequence still read q)
 *   q            device bf16 [num_seqs][num_q_heads][head_dim], NOT rotated
 *   k_new, v_new device bf16 [num_seqs][num_kv_heads][head_dim]: the new
 *                token's key (not rotated) and value
 *   positions    device int32 [num_seqs]: the new token's position (the
 *                rotation angle); the attention itself follows context_lens
 *   slot_mapping device int32 [num_seqs]: the new token's slot, which must be
 *                the slot of logical position context_lens[s] - 1 under the
 *                sequence's block table; -1 (or a slot outside the pool)
 *                skips the write, and the cache's current contents are read
 *   rope_base    0 = no rotation (the write is a plain copy), else > 1
 *   all other arguments, the workspace contract and the errors as for
 *   attn_decode_paged; k_cache and v_cache are written.
 * ---------------------------------------------------------------------- */
ATTN_API int attn_decode_paged_rope(void* q_rot_out, const void* q, const void* k_new, const void* v_new,
                           const int32_t* positions, const int32_t* slot_mapping, float rope_base,
                           void* k_cache, void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, void* o, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                           int32_t partition_size, float scale, attn_dtype dtype, const int32_t* plan,
                           int32_t plan_items, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream);

/* Host-side plan of a decode launch (host memory only, no HIP call): the
 * (sequence, partition) pairs of the sequences' contexts, longest sequences
 * first, partitions in order, with the partition size attn_decode_paged
 * uses for the same arguments (partition_size 0, or a multiple of 16 up to
 * 65536; the decode call itself checks its dtype's rule).  context_lens: host int32 [num_seqs] (clamped
 * to max_context_len).  Returns the number of pairs; writes them to items
 * (int32 [count][2]) only when items is non-NULL and capacity (in pairs)
 * holds them all.  Negative attn_status on bad arguments. */
ATTN_API int64_t attn_decode_paged_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                               int32_t max_context_len, int32_t partition_size, int32_t* items,
                               int64_t capacity);

/* Partition size that attn_decode_paged uses when partition_size is 0. */
ATTN_API int32_t attn_decode_paged_auto_partition(int32_t num_seqs, int32_t num_kv_heads,
                                         int32_t max_context_len);

/* A partition size chosen from the contexts themselves (host int32
 * context_lens[num_seqs], no HIP call): the shortest of 128, 256, ..., 1024
 * tokens (multiples of 128, valid for every dtype) whose workgroups, one per
 * (sequence, partition) item, kv head and slice of 16 query heads, all fit on
 * the GPU at once (two per CU at head_dim 128, four at 64), so that the
 * longest item is as short as possible without a second round; 1024 when no
 * size fits.  Pass it to attn_decode_paged_plan and attn_decode_paged alike
 * (the automatic size of partition_size 0 sees only the longest context).
 * Negative attn_status on bad arguments. */
ATTN_API int32_t attn_decode_paged_partition_for(const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);

/* -------------------------------------------------------------------------
 * attn_prefill_decode_paged -- a chunked prefill and a decode over the same
 * paged cache in one launch.
 *
 * A serving step runs both regimes the tutorial separates, many queries per
 * request (prefill, bound by the matrix work) and one (decode, bound by
 * reading the cache) (§FlashAttention-Style Kernels, §Paged Attention
 * Kernels).  The two only read the cache (apart from the decode's own new
 * tokens) and write disjoint outputs, so one grid holds the workgroups of
 * both: no second stream, no join, and the CUs are shared in an order the
 * library chooses.  The results are those of attn_prefill_paged without a
 * workspace (prefill part, one pass per query tile) and attn_decode_paged,
 * or attn_decode_paged_rope when the decode part carries the new tokens,
 * bit for bit.
 *
 *   prefill   the chunked prefill: the arguments of attn_prefill_paged
 *             (num_seqs 0: no prefill part).  It runs on the default tile in
 *             one pass (no split-KV workspace, no mask).
 *   decode    the decode: the arguments of attn_decode_paged, its workspace
 *             and plan contract included (num_seqs 0: no decode part).  With
 *             k_new, v_new, positions and slot_mapping set (q_rot_out and
 *             rope_base as for attn_decode_paged_rope) the decode also
 *             rotates and writes each sequence's new token; all four NULL:
 *             the new tokens are already in the cache.  A new token's slot
 *             must not be one that the prefill part reads.
 *   k_cache, v_cache, num_q_heads, num_kv_heads, head_dim, block_size,
 *   num_blocks, scale: shared by both parts, as in those calls.
 *   dtype     BF16 only (ATTN_E_UNSUPPORTED otherwise).
 * Errors as for the two calls; nothing is launched unless both parts are
 * valid.  The launch allocates nothing and can be captured in a HIP graph.
 * ---------------------------------------------------------------------- */
typedef struct attn_paged_prefill_part {
  const void* q;                 /* [total_q][num_q_heads][head_dim] */
  const int32_t* block_table;    /* [num_seqs][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
  const int32_t* cu_seqlens_q;   /* [num_seqs + 1] */
  const int32_t* context_lens;   /* [num_seqs], new tokens included */
  void* o;                       /* [total_q][num_q_heads][head_dim] */
  int32_t num_seqs, total_q, max_seqlen_q, max_context_len;
  int32_t causal;
} attn_paged_prefill_part;

typedef struct attn_paged_decode_part {
  const void* q;                 /* [num_seqs][num_q_heads][head_dim] */
  const int32_t* block_table;    /* [num_seqs][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;   /* [num_seqs] */
  void* o;                       /* [num_seqs][num_q_heads][head_dim] */
  int32_t num_seqs, max_context_len, partition_size;
  const int32_t* plan;           /* optional, as for attn_decode_paged */
  int32_t plan_items;
  void* workspace;
  size_t workspace_bytes;
  /* optional fused write of each sequence's new token */
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
  const int32_t* slot_mapping;
  void* q_rot_out;
  float rope_base;
} attn_paged_decode_part;

ATTN_API int attn_prefill_decode_paged(const attn_paged_prefill_part* prefill,
                              const attn_paged_decode_part* decode, void* k_cache, void* v_cache,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, float scale, attn_dtype dtype,
                              attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_kv_cache_write_rope -- fused rotary embedding + paged cache write.
 *
 * This kernel performs in one pass two of the fusions §Operator Fusion
 * lists: the rotary embedding of queries and keys, and the KV-cache update
 * made as keys and values are transformed.  For token n with position
 * positions[n]: each pair (x[i], x[i + D/2]), i < D/2, of every query and key
 * head is rotated by angle positions[n] * rope_base^(-2i/D) (the angle is
 * formed and reduced modulo 2 pi in double precision, its sine and cosine
 * then taken in single precision); the rotated key and the unchanged
 * value are stored in slot slot_mapping[n] (block slot / 16, offset slot % 16);
 * slot -1 skips the cache write for that token.  Rotated queries overwrite q.
 *
 *   q            device [num_tokens][num_q_heads][head_dim], may be NULL
 *   k, v         device [num_tokens][num_kv_heads][head_dim]
 *   positions    device int32 [num_tokens], >= 0
 *   slot_mapping device int32 [num_tokens], -1 or 0 .. num_blocks*16-1
 *   rope_base    0 = no rotation (plain copy)
 *   dtype        BF16 or F32 (q, k, v and the caches share it)
 * ---------------------------------------------------------------------- */
ATTN_API int attn_kv_cache_write_rope(void* q, const void* k, const void* v, const int32_t* positions,
                             const int32_t* slot_mapping, void* k_cache, void* v_cache,
                             int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float rope_base, attn_dtype dtype, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * attn_residual_rms_norm -- fused residual add + RMS normalisation.
 *
 * §Operator Fusion counts the residual add followed by RMSNorm among the
 * common fusions and gives a definition of it: h = x + residual (stored in the
 * input dtype: the updated residual), y = h / sqrt(mean(h^2) + eps) * weight
 * row by row (mean over the hidden dimension); both y and h are returned.
 * One pass: x, residual and weight read once, y and h written once.
 *
 *   x, residual   device [rows][hidden]
 *   weight        device [hidden]
 *   y             device [rows][hidden], written; must not alias the others
 *   residual_out  device [rows][hidden], written with h; may be residual or
 *                 x itself (in place)
 *   hidden        a multiple of 8, 8 .. 8192; eps finite, >= 0 (the example
 *                 uses 1e-6); dtype BF16 or F32 (all tensors share it)
 * ---------------------------------------------------------------------- */
ATTN_API int attn_residual_rms_norm(const void* x, const void* residual, const void* weight, void* y,
                           void* residual_out, int32_t rows, int32_t hidden, float eps, attn_dtype dtype,
                           attn_stream_t stream);

/* -------------------------------------------------------------------------
 * Block pool (host only).  §Paged Attention Kernels: the cache is cut into
 * fixed-size blocks, handed out as requests grow, given back when a request
 * finishes, and possibly held by several sequences that begin with the same
 * tokens; a block table maps a sequence's logical blocks to physical ones.  The pool is a LIFO free list with a
 * reference count per block.  Not thread-safe: callers serialise access.
 * ---------------------------------------------------------------------- */
typedef struct attn_pool attn_pool;

/* num_blocks >= 1, block_size >= 1.  Fresh pools hand out ids 0, 1, 2, ... */
ATTN_API int attn_pool_create(int32_t num_blocks, int32_t block_size, attn_pool** out);
ATTN_API void attn_pool_destroy(attn_pool* pool);
/* Take n blocks (refcount 1) into out_ids[n].  All or nothing: NOMEM leaves
 * the pool unchanged. */
ATTN_API int attn_pool_alloc(attn_pool* pool, int32_t n, int32_t* out_ids);
/* Drop one reference of each id; a block whose count reaches 0 returns to the
 * free list (pushed in argument order).  Every id is checked first
 * (range, and enough references for repeated ids): on error nothing changes. */
ATTN_API int attn_pool_free(attn_pool* pool, const int32_t* ids, int32_t n);
/* Add one reference to each (allocated) id, for prefix sharing. */
ATTN_API int attn_pool_retain(attn_pool* pool, const int32_t* ids, int32_t n);
ATTN_API int32_t attn_pool_num_free(const attn_pool* pool);
ATTN_API int32_t attn_pool_num_blocks(const attn_pool* pool);
/* Reference count of id (0 = free), or ATTN_E_INVALID. */
ATTN_API int attn_pool_refcount(const attn_pool* pool, int32_t id);

/* Grow a sequence from cur_len to cur_len + n_new tokens.  Blocks the new
 * length needs beyond ceil(cur_len / block_size) are allocated (all or
 * nothing) and appended to block_table_row (host, max_blocks entries); the
 * slot of each new token, block_table_row[t / bs] * bs + t % bs, is written to
 * slot_mapping_out[n_new] (may be NULL). */
ATTN_API int attn_seq_reserve(attn_pool* pool, int32_t* block_table_row, int32_t max_blocks,
                     int32_t cur_len, int32_t n_new, int32_t* slot_mapping_out);

/* Prefix sharing.  §Paged Attention Kernels: sequences that begin with the
 * same tokens may hold the same blocks.  attn_seq_fork gives child_row (host,
 * max_blocks entries) the first ceil(len / block_size) entries of parent_row,
 * each block retained once more; parent and child then read the same
 * physical blocks.  On error nothing changes. */
ATTN_API int attn_seq_fork(attn_pool* pool, const int32_t* parent_row, int32_t len, int32_t* child_row,
                  int32_t max_blocks);
/* attn_seq_reserve for a row whose blocks may be shared: when the first new
 * token falls into a partly filled block (cur_len % block_size != 0) that
 * another sequence still references (refcount > 1), the sequence first gets
 * a fresh block in its place (the shared one loses this reference) and
 * copy_pair_out (host int32[2]) = {shared id, fresh id}: the caller copies
 * the block's contents (attn_copy_blocks) before writing the new tokens.
 * Otherwise copy_pair_out = {-1, -1}.  All or nothing: NOMEM (the fresh
 * block and the growth together) changes nothing. */
ATTN_API int attn_seq_reserve_cow(attn_pool* pool, int32_t* block_table_row, int32_t max_blocks,
                         int32_t cur_len, int32_t n_new, int32_t* slot_mapping_out,
                         int32_t* copy_pair_out);

/* -------------------------------------------------------------------------
 * attn_copy_blocks -- copy whole cache blocks, both pools, every kv head:
 * for each pair p, block pairs[p][1] of k_cache and of v_cache becomes a
 * copy of block pairs[p][0] (the copy-on-write step of prefix sharing).
 *
 *   k_cache, v_cache  device, [num_blocks][num_kv_heads][block_size][D] and
 *                     [num_blocks][num_kv_heads][D][block_size]
 *   pairs             device int32 [num_pairs][2] (src, dst); a pair with an
 *                     id outside [0, num_blocks) or src == dst is skipped.
 *                     Destinations must be distinct and no destination may be
 *                     a source of the same call.
 *   dtype             BF16 or F32
 * ---------------------------------------------------------------------- */
ATTN_API int attn_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     attn_dtype dtype, attn_stream_t stream);

/* -------------------------------------------------------------------------
 * Debug library.  Every kernel keeps its accesses inside the buffers whatever
 * the device-side inputs hold: block-table entries outside the pool read
 * block 0, slots and copy pairs outside the pool are skipped, lengths are cut
 * to what the block-table row and the launch cover.  The release library
 * does this silently.  The debug library (libmi_attn_debug.so, built from the
 * same sources with MI_ATTN_DEBUG=1; the Python binding loads it instead of
 * libmi_attn.so when the environment variable MI_ATTN_DEBUG is 1) also
 * records, per device, which kinds of malformed input the kernels met:
 * ---------------------------------------------------------------------- */
#define ATTN_DEBUG_BLOCK_ID 1u  /* a block-table entry a kernel needed lies outside [0, num_blocks) */
#define ATTN_DEBUG_SLOT 2u      /* a slot_mapping entry below -1 or at or past num_blocks * block_size */
#define ATTN_DEBUG_CONTEXT 4u   /* a context length below 0, or beyond the block-table row
                                   (max_blocks_per_seq * block_size) or the decode launch
                                   (max_context_len rounded up to the partition) */
#define ATTN_DEBUG_COPY_PAIR 8u /* an attn_copy_blocks pair with an id outside [0, num_blocks) */
#define ATTN_DEBUG_SEQLENS 16u  /* cu_seqlens_q not starting at 0, falling, or past total_q */

/* Debug library: waits for the current device (hipDeviceSynchronize), ORs
 * the recorded bits of that device into *flags_out (host) and, when
 * clear != 0, forgets them.  Release library: *flags_out = 0 and
 * ATTN_E_UNSUPPORTED.  ATTN_E_INVALID for a NULL flags_out, ATTN_E_DEVICE
 * if a HIP call fails. */
ATTN_API int attn_debug_flags(uint32_t* flags_out, int clear);

#ifdef __cplusplus
}
#endif
#endif /* MI_ATTN_H */
