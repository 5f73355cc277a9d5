/*
 * pa.h -- paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * The method: the KV cache of every sequence lives in fixed-size blocks of
 * block_size token positions scattered through one pool, and a per-sequence
 * block table maps logical positions to physical blocks ("Serving"
 * (transformers-and-math module 23), section 23.4 Paged Attention; the
 * "Paged Attention: Managing the KV Cache Like Virtual Memory" summary on the
 * inference-serving tag page).  A decode step writes each sequence's new
 * token into its slot, then reads the whole cached K/V of every sequence for
 * one query token per sequence ("Serving", section 23.2 Prefill and Decode).
 * The attention is scaled dot-product softmax attention; grouped-query
 * attention lets gqa_group consecutive query heads share one KV head
 * ("Serving", section 23.1: 8 KV heads for 32 query heads in LLaMA-3 8B).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers are DEVICE pointers owned by the caller unless stated otherwise.
 *   The GPU entry points never allocate or free memory.  State they keep:
 *   a note of each of the first 64 devices' CU count and of how many work
 *   groups of the attention kernel fit on one CU (filled on first use,
 *   thread-safe; later devices are queried on every call); the fixed device array of pa_decode_step_noalloc (one per device,
 *   shared by that entry point's calls, see there); and the two events set
 *   by pa_time_next_attention, per host thread, until the launch that uses
 *   them.  Apart from pa_decode_step_noalloc, calls on different streams or
 *   threads are independent.
 *   The host-side block pool (pa_pool_*, pa_block_hashes, at the end) works
 *   on HOST memory: a pool is an object the caller creates and destroys.
 * - All arrays are dense and row-major, with the shapes given below, and
 *   every array pointer is 16-byte aligned.
 * - q, pools and out share one element type (dtype); partition workspace is
 *   always float32.  Accumulation is float32; outputs are rounded to dtype
 *   with round-to-nearest-even.
 * - Pool layout: [n_blocks, n_kv_heads, block_size, d_head].  Position t of
 *   sequence b lives in block block_table[b * max_blocks + t / block_size] at
 *   offset t % block_size.  Flat slot of a position: block * block_size +
 *   offset.
 * - Supported: d_head in {64, 128}; block_size in {8, 16, 32, 64} (a power of
 *   two, multiple of 8); dtype PA_F32, PA_F16, PA_BF16; gqa_group >= 1.
 * - Each call checks its host-side arguments, enqueues its kernels on
 *   `stream` (a hipStream_t; NULL = the default stream) and returns without
 *   waiting.  Calls on one stream run in order, so a cache write followed by
 *   a decode on the same stream sees the written token.
 * - Return value: PA_OK, or a negative status (pa_strerror gives text).  A
 *   failed argument check enqueues nothing.  PA_ERR_HIP reports a launch
 *   error; faults inside a kernel surface at the caller's next sync.
 * - Contract violations found on the device never cause out-of-bounds
 *   accesses: a sequence whose context length is negative or exceeds
 *   max_blocks * block_size (or the workspace), or whose table names a block
 *   outside [0, n_blocks) for a used position, gets NaN in every output
 *   element of that sequence; a cache-write slot outside
 *   [0, n_blocks * block_size) is skipped.
 * - batch == 0 (or n_tokens == 0) is a no-op returning PA_OK.
 */
#ifndef PA_H_
#define PA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_F32 = 0,  /* IEEE binary32 */
  PA_F16 = 1,  /* IEEE binary16 */
  PA_BF16 = 2  /* bfloat16 (upper half of a binary32) */
} pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is negative or inconsistent */
  PA_ERR_UNSUPPORTED = -3, /* d_head, block_size or dtype not supported */
  PA_ERR_WORKSPACE = -4,   /* max_partitions < 1 */
  PA_ERR_PARTITION = -5,   /* partition_size not a positive multiple of block_size */
  PA_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  PA_ERR_ALIGN = -7,       /* an array pointer is not 16-byte aligned */
  PA_ERR_NOSPACE = -8,     /* the block pool has too few free blocks */
  PA_ERR_SCRATCH = -9      /* pa_decode_step_noalloc: the workspace would not
                              fit the fixed scratch buffer */
};

/*
 * pa_cache_write -- put each new token's key and value into its pool slot.
 *
 * The cache grows token by token into blocks allocated as the sequence grows
 * ("Serving", section 23.4).  For i < n_tokens with s = slot_mapping[i]:
 *   k_pool[s / block_size, h, s % block_size, :] = key[i, h, :]   for all h
 *   v_pool[...]                                  = value[i, h, :]
 * A bit copy (no rounding).  s < 0 skips token i.  Slots must be distinct;
 * with duplicates the surviving value is unspecified.
 *
 *   key, value     [n_tokens, n_kv_heads, d_head]           dtype, read
 *   k_pool, v_pool [n_blocks, n_kv_heads, block_size, d_head] dtype, written
 *   slot_mapping   [n_tokens] int32                           read
 */
int pa_cache_write(const void* key, const void* value, void* k_pool,
                   void* v_pool, const int32_t* slot_mapping, int32_t n_tokens,
                   int32_t n_kv_heads, int32_t d_head, int32_t block_size,
                   int32_t n_blocks, int32_t dtype, void* stream);

/*
 * pa_copy_blocks -- copy whole physical blocks within both pools, so that a
 * block shared by several sequences can be duplicated before one of them
 * writes into it (copy-on-write sharing of the paged cache: the "Paged
 * Attention" summary on the inference-serving tag page; sequences sharing a
 * prefix share its blocks, "Serving" section 23.4).
 *
 * For i < n_pairs with s = block_pairs[2i], d = block_pairs[2i + 1]:
 *   k_pool[d, :, :, :] = k_pool[s, :, :, :]   and   v_pool[d] = v_pool[s]
 * A bit copy.  Every pair reads the pools as they were before the call:
 * destinations must be distinct and must not be the source of any pair
 * (otherwise the result is unspecified).  A pair naming a block outside
 * [0, n_blocks) is skipped.  The caller updates its block tables.
 *
 *   k_pool, v_pool [n_blocks, n_kv_heads, block_size, d_head] dtype, read and
 *                  written
 *   block_pairs    [n_pairs, 2] int32 (source, destination)       read
 */
int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs,
                   int32_t n_pairs, int32_t n_kv_heads, int32_t d_head,
                   int32_t block_size, int32_t n_blocks, int32_t dtype,
                   void* stream);

/*
 * pa_read_ceiling -- a measurement aid, not part of the decode path: reads
 * n_tiles tiles of tile_bytes bytes from buf (tile ids tile_order[i], or
 * 0 .. n_tiles - 1 in address order when tile_order is NULL) with the
 * non-temporal 16-byte loads the attention kernels use, and nothing else.
 * Timed on its own it gives the device's achievable HBM read rate for that
 * access pattern -- sequential, or a gather of 4 KiB tiles scattered like
 * the cache's (block, KV head) tiles -- the ceiling the attention kernels'
 * rates are compared with (the decode path itself is bound by HBM reads:
 * "Serving" section 23.2).  Tile ids outside the buffer are skipped.  sink
 * is written only in the (practically impossible) case that the folded
 * bytes equal a fixed constant; it keeps the loads from being removed.
 *
 *   buf         [buf_bytes] bytes, 16-byte aligned, read
 *   tile_order  [n_tiles] int32, or NULL (then n_tiles <= buf_bytes / tile_bytes)
 *   tile_bytes  a positive multiple of 16 (PA_ERR_SHAPE otherwise)
 *   sink        one uint32
 */
int pa_read_ceiling(const void* buf, int64_t buf_bytes, const int32_t* tile_order,
                    int64_t n_tiles, int32_t tile_bytes, uint32_t* sink,
                    void* stream);

/*
 * pa_time_next_attention -- a measurement aid, not part of the decode path:
 * the attention kernel launched next by a decode call on this thread (any
 * of pa_decode, pa_decode_partitioned, pa_decode_partitioned_vector,
 * pa_decode_step, pa_decode_split, pa_decode_shared_prefix,
 * pa_decode_multi), or the read kernel of the next pa_read_ceiling call,
 * records its own start in
 * start_event and its end in stop_event (hipEvent_t handles the caller
 * created with timing enabled; either may be NULL).  hipEventElapsedTime
 * of the two is then the kernel's execution time, without the gaps between
 * launches that events recorded around the call also measure.  The events
 * are consumed by that one launch; NULL, NULL cancels.  Host-side only.
 */
int pa_time_next_attention(void* start_event, void* stop_event);

/*
 * pa_decode -- one query token per sequence attends over all its cached
 * positions, in one pass per (sequence, KV head).
 *
 * For query head h of sequence b, with kvh = h / gqa_group and n =
 * context_lens[b] (the token written this step included):
 *   s_t = scale * <q[b, h, :], K_t>            t = 0 .. n-1
 *   out[b, h, :] = sum_t softmax(s)_t * V_t
 * where K_t, V_t are row t of KV head kvh read through the block table.
 * n == 0 gives a zero row.
 *
 *   out            [batch, n_kv_heads * gqa_group, d_head]   dtype, written
 *   q              [batch, n_kv_heads * gqa_group, d_head]   dtype, read
 *   k_pool, v_pool [n_blocks, n_kv_heads, block_size, d_head] dtype, read
 *   block_table    [batch, max_blocks] int32                  read
 *   context_lens   [batch] int32                              read
 */
int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_table, int32_t max_blocks,
              const int32_t* context_lens, int32_t batch, int32_t n_kv_heads,
              int32_t gqa_group, int32_t d_head, int32_t block_size,
              int32_t n_blocks, float scale, int32_t dtype, void* stream);

/*
 * pa_decode_partitioned -- the same attention split along the context into
 * partitions of partition_size positions, each reduced to softmax statistics
 * that pa_reduce combines (log-sum-exp merge).  The pages do not describe
 * this split: it is an exact rearrangement of the attention of pa_decode
 * (rounding aside) that lets a long context, or a small batch, spread over
 * the whole GPU; the decode it serves reads the whole cache and is bound by
 * memory reads ("Serving", section 23.2).  Partition p of sequence b
 * covers positions [p * P, min((p + 1) * P, n)).  For each non-empty
 * partition and query head, with s_t as in pa_decode:
 *   max_logits[b, h, p] = m, a reference logit within 8 ln 2 below the
 *                         partition's largest s_t (and not above it)
 *   exp_sums[b, h, p]   = sum_t exp(s_t - m)
 *   tmp_out[b, h, p, :] = sum_t exp(s_t - m) V_t / exp_sums[b, h, p]
 * Entries of empty partitions (p * P >= n) are not written.
 *
 *   max_logits, exp_sums [batch, n_q_heads, max_partitions] float32, written
 *   tmp_out   [batch, n_q_heads, max_partitions, d_head]     float32, written
 *   max_partitions must be >= ceil(max_b context_lens[b] / partition_size);
 *   sequences that need more get NaN outputs from pa_reduce.
 *   Other arguments as in pa_decode.
 */
int pa_decode_partitioned(float* max_logits, float* exp_sums, float* tmp_out,
                          int32_t partition_size, int32_t max_partitions,
                          const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* context_lens,
                          int32_t batch, int32_t n_kv_heads, int32_t gqa_group,
                          int32_t d_head, int32_t block_size, int32_t n_blocks,
                          float scale, int32_t dtype, void* stream);

/*
 * pa_decode_partitioned_vector -- pa_decode_partitioned computed by the
 * vector-ALU kernel (the one fp32 caches use) for every dtype, where
 * pa_decode_partitioned runs fp16 and bf16 on the matrix cores.  A
 * measurement aid: decode reads each cached byte once and spends only a
 * multiply-add or two on it ("Serving", section 23.2), and this entry
 * point times the two engines on the same batch.  Arguments, outputs,
 * layout, errors and NaN rules are those of pa_decode_partitioned; the
 * values agree with it to rounding (the sums run in another order).
 */
int pa_decode_partitioned_vector(float* max_logits, float* exp_sums,
                                 float* tmp_out, int32_t partition_size,
                                 int32_t max_partitions, const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_table,
                                 int32_t max_blocks,
                                 const int32_t* context_lens, int32_t batch,
                                 int32_t n_kv_heads, int32_t gqa_group,
                                 int32_t d_head, int32_t block_size,
                                 int32_t n_blocks, float scale, int32_t dtype,
                                 void* stream);

/*
 * pa_decode_step -- a whole decode step for the partitioned path: the cache
 * write of each sequence's new token folded into pa_decode_partitioned.
 * For every sequence with n = context_lens[b] >= 1 whose table entry for
 * position n - 1 lies in the pool, key_new[b] / value_new[b] are stored at
 * position n - 1 (block block_table[b][(n-1) / block_size], offset
 * (n-1) % block_size), every KV head, as a bit copy; then the attention and
 * the workspace are exactly those of pa_decode_partitioned over the written
 * cache (pa_reduce finishes).  The result equals pa_cache_write with the
 * slots of positions n - 1 followed by pa_decode_partitioned, bit for bit,
 * in one launch: the work item that covers position n - 1 writes the row
 * and uses it directly.  fp32 runs the write as a separate kernel first.
 * The write also happens for a sequence that needs more than max_partitions
 * partitions (whose output pa_reduce reports as NaN), so a caller that
 * retries with a larger workspace finds the token in the cache.
 *
 *   key_new, value_new [batch, n_kv_heads, d_head] dtype, read
 *   k_pool, v_pool     written at position n - 1 of each sequence, read
 *   Other arguments as in pa_decode_partitioned.
 */
int pa_decode_step(float* max_logits, float* exp_sums, float* tmp_out,
                   int32_t partition_size, int32_t max_partitions,
                   const void* key_new, const void* value_new, const void* q,
                   void* k_pool, void* v_pool, const int32_t* block_table,
                   int32_t max_blocks, const int32_t* context_lens,
                   int32_t batch, int32_t n_kv_heads, int32_t gqa_group,
                   int32_t d_head, int32_t block_size, int32_t n_blocks,
                   float scale, int32_t dtype, void* stream);

/*
 * pa_decode_step_noalloc -- pa_decode_step followed by pa_reduce, with the
 * partition workspace in a fixed buffer inside the library instead of
 * caller memory: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * It allocates and frees nothing.
 *
 * max_partitions is ceil(max_blocks * block_size / partition_size), enough
 * for any valid context; the workspace is n_q_heads * batch *
 * max_partitions * (d_head + 2) * 4 bytes and must fit the buffer's
 * 32 MiB (PA_ERR_SCRATCH otherwise, nothing enqueued): e.g. the LLaMA-3-8B
 * batch (B 128, 32 query heads, d 128, 8192-position tables) at partition
 * 3072 needs 6.4 MB.  The buffer is one per GPU, kept until the process
 * ends; every call on a GPU uses the same one, so calls that overlap on one
 * GPU (different streams or threads) race.  Nothing in it needs to start
 * at zero: every entry pa_reduce reads is first written by the attention.
 * The result -- pools and out -- is bit-identical to pa_decode_step +
 * pa_reduce with that max_partitions.
 *
 *   out            [batch, n_kv_heads * gqa_group, d_head] dtype, written
 *   Other arguments as in pa_decode_step.
 */
int pa_decode_step_noalloc(void* out, int32_t partition_size,
                           const void* key_new, const void* value_new,
                           const void* q, void* k_pool, void* v_pool,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* context_lens, int32_t batch,
                           int32_t n_kv_heads, int32_t gqa_group,
                           int32_t d_head, int32_t block_size,
                           int32_t n_blocks, float scale, int32_t dtype,
                           void* stream);

/*
 * pa_decode_shared_prefix -- pa_decode_partitioned (key_new == NULL) or
 * pa_decode_step (key_new != NULL) for a batch whose sequences share the
 * physical blocks of a common prefix, a shared prompt for instance
 * ("Serving", section 23.4: sequences with a common prefix can share its
 * blocks).  The workspace it writes is the one those calls define, read by
 * pa_reduce; the values differ from theirs only by rounding order.
 *
 * Stated by the caller: positions [0, prefix_len) of every sequence map to
 * the same physical blocks (the first ceil(prefix_len / block_size) table
 * entries are equal in every row).  The first floor(prefix_len /
 * partition_size) partitions -- fewer if some sequence with a valid length
 * ends in or before them -- are then computed for several sequences in one
 * work item: each K/V tile of the prefix is read once for 16 / gqa_group
 * sequences (at least one) instead of once per sequence.
 *
 * Contract violations have defined results:
 * - a sequence whose table entries for such a shared partition differ from
 *   those of the first sequence of its work item gets NaN in every output
 *   element (the item reads one table for all its sequences and checks the
 *   others against it); out-of-pool block ids give NaN, never an
 *   out-of-bounds read;
 * - with key_new != NULL, a sequence whose new token would land inside the
 *   shared positions (n - 1 < prefix_len, so the write would change a block
 *   other sequences read) is not written and gets NaN in every output
 *   element.  This holds on every path, including the fallbacks below.
 * A valid length is one of 1 .. max_blocks * block_size that does not break
 * the second rule.  With batch > 1024, fp32, or a device too small for one
 * work group per KV head no work item is shared: the call computes what
 * pa_decode_partitioned / pa_decode_step compute, with the second rule.
 *
 *   prefix_len >= 0 (PA_ERR_SHAPE otherwise)
 *   key_new, value_new  both NULL, or both [batch, n_kv_heads, d_head] dtype
 *                       (one NULL: PA_ERR_NULL); the write of pa_decode_step
 *   Other arguments as in pa_decode_step.
 */
int pa_decode_shared_prefix(float* max_logits, float* exp_sums, float* tmp_out,
                            int32_t partition_size, int32_t max_partitions,
                            const void* key_new, const void* value_new,
                            const void* q, void* k_pool, void* v_pool,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* context_lens, int32_t batch,
                            int32_t n_kv_heads, int32_t gqa_group,
                            int32_t d_head, int32_t block_size,
                            int32_t n_blocks, int32_t prefix_len, float scale,
                            int32_t dtype, void* stream);

/*
 * pa_decode_split -- the decode step (the write of pa_decode_step when
 * key_new != NULL, none when NULL) with the context cut into pieces by
 * work rather than by position, for batches whose lengths are uneven or
 * too few to fill the GPU evenly with fixed partitions.  Like the
 * partition split, this is not on the pages: an exact rearrangement of the
 * attention of pa_decode (rounding aside); the decode reads the whole cache
 * and is bound by memory reads ("Serving", section 23.2), so the work is
 * what each part reads.
 *
 * All sequences' 16-position tiles, in sequence order, are cut into equal
 * runs, one run per work group; a sequence is cut where a run ends.  Slot j
 * of a row holds the statistics of the sequence's j-th piece (positions in
 * order): max_logits, exp_sums and tmp_out as pa_decode_partitioned
 * defines them for a partition, over the piece's positions.  Slots past the
 * sequence's last piece get exp_sums = 0 (and max_logits = -inf; tmp_out is
 * not written).  No sequence is cut into more than max_partitions pieces
 * (the runs are lengthened if needed), so max_partitions >= 2 is the only
 * requirement (PA_ERR_WORKSPACE otherwise); more slots allow a more even
 * split.  pa_reduce with partition_size = 0 merges the pieces.  A
 * sequence with an invalid length gets NaN in every slot.  fp16 and bf16
 * only (PA_ERR_UNSUPPORTED for fp32).
 *
 *   max_logits, exp_sums [batch, n_q_heads, max_partitions] float32, written
 *   tmp_out   [batch, n_q_heads, max_partitions, d_head]     float32, written
 *   key_new, value_new  both NULL, or both [batch, n_kv_heads, d_head]
 *   Other arguments as in pa_decode_step.
 */
int pa_decode_split(float* max_logits, float* exp_sums, float* tmp_out,
                    int32_t max_partitions, const void* key_new,
                    const void* value_new, const void* q, void* k_pool,
                    void* v_pool, const int32_t* block_table,
                    int32_t max_blocks, const int32_t* context_lens,
                    int32_t batch, int32_t n_kv_heads, int32_t gqa_group,
                    int32_t d_head, int32_t block_size, int32_t n_blocks,
                    float scale, int32_t dtype, void* stream);

/*
 * pa_decode_multi -- several query tokens per sequence: the last n_queries
 * positions of each sequence, causal among themselves, as in the one pass
 * in which the target model checks all drafted tokens of speculative
 * decoding ("Serving", section 23.5).  Their keys and values are already in
 * the cache, and context_lens[b] = n counts them.  Query token j < n_queries
 * of head h sees the positions t < n - n_queries + j + 1:
 *   s_t = scale * <q[b, j, h, :], K_t>,  out[b, j, h, :] = sum_t softmax(s)_t V_t
 * A token that sees no position gives a zero row.  Computed like
 * pa_decode_partitioned, with n_queries * n_q_heads rows per sequence, row
 * j * n_q_heads + h; pa_reduce with n_q_heads = n_queries * n_kv_heads *
 * gqa_group merges them into out viewed as [batch, n_queries * n_q_heads,
 * d_head].  The KV bytes are read once for all n_queries tokens.
 *
 *   q              [batch, n_queries, n_kv_heads * gqa_group, d_head] dtype
 *   max_logits, exp_sums [batch, n_queries * n_q_heads, max_partitions] f32
 *   tmp_out   [batch, n_queries * n_q_heads, max_partitions, d_head]    f32
 *   A (row, partition) that the token's causal limit leaves empty gets
 *   exp_sums = 0 and tmp_out = 0.  fp16 and bf16 only (PA_ERR_UNSUPPORTED
 *   for fp32 with n_queries > 1).  Other arguments as in
 *   pa_decode_partitioned.
 */
int pa_decode_multi(float* max_logits, float* exp_sums, float* tmp_out,
                    int32_t partition_size, int32_t max_partitions,
                    const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, int32_t max_blocks,
                    const int32_t* context_lens, int32_t batch,
                    int32_t n_queries, int32_t n_kv_heads, int32_t gqa_group,
                    int32_t d_head, int32_t block_size, int32_t n_blocks,
                    float scale, int32_t dtype, void* stream);

/*
 * pa_reduce -- merge per-partition statistics into the attention output:
 * the second half of the split of pa_decode_partitioned (not on the pages;
 * an exact identity of softmax: each partition's weights are rescaled to a
 * common maximum and the partial outputs averaged by their denominators).
 * With n_p = ceil(n / partition_size), M = max_{p<n_p} m_p and
 * w_p = l_p * exp(m_p - M):
 *   out[b, h, :] = sum_p w_p tmp_out[b, h, p, :] / sum_p w_p
 * n == 0 gives a zero row (and so does a row whose partitions all have
 * exp_sums = 0).  A partition with exp_sums = 0 adds nothing and its
 * tmp_out is not read.  partition_size = 0 merges a pa_decode_split
 * workspace: every slot (pieces, not partitions) of rows with n >= 1.
 * Arrays as in pa_decode_partitioned; out as in pa_decode.
 */
int pa_reduce(void* out, const float* max_logits, const float* exp_sums,
              const float* tmp_out, const int32_t* context_lens, int32_t batch,
              int32_t n_q_heads, int32_t d_head, int32_t partition_size,
              int32_t max_partitions, int32_t dtype, void* stream);

/*
 * Host-side block pool and prefix cache (HOST pointers; no GPU work).
 *
 * The allocator behind the paged cache: blocks are handed out as sequences
 * grow and shared by sequences with a common prefix ("Serving", section
 * 23.4), with reference counts so a shared block is released only by its
 * last user (copy it with pa_copy_blocks before writing into it).  Prefix
 * caching names each full block by a hash of its tokens chained with the
 * hash of the block before it (the block-and-hash-chain scheme of the
 * prompt-caching articles on the pagedattention tag page), so a request
 * whose leading blocks hash alike reuses their physical blocks, and one
 * changed token renames every later block.
 *
 * Policy (fixed, so results are reproducible): a fresh block is the
 * lowest-numbered free block holding no cached prefix, else the cached free
 * block released longest ago (its hash is then forgotten).  A block whose
 * reference count drops to zero is free; if it carries a hash it stays
 * findable until it is reused.  A pool is not thread-safe.
 */
typedef struct pa_block_pool pa_block_pool;

/*
 * pa_block_hashes -- chained hashes of the full blocks of a token sequence.
 * With h_{-1} = parent (0 at the start of a sequence), block i (tokens
 * [i * block_size, (i + 1) * block_size)) gets
 *   h_i = FNV-1a-64(8 bytes of h_{i-1}, little endian, then the block's
 *                   token ids as 4-byte little-endian integers)
 * (FNV-1a: offset basis 14695981039346656037, prime 1099511628211).
 * Writes n_full = n_tokens / block_size hashes.
 *   tokens [n_tokens] int32, hashes [n_tokens / block_size] uint64 (host)
 */
int pa_block_hashes(const int32_t* tokens, int32_t n_tokens,
                    int32_t block_size, uint64_t parent, uint64_t* hashes,
                    int32_t* n_full);

/* A pool of n_blocks physical block ids, all free; NULL if n_blocks < 1 or
 * out of memory.  pa_pool_destroy(NULL) is allowed. */
pa_block_pool* pa_pool_create(int32_t n_blocks);
void pa_pool_destroy(pa_block_pool* pool);

/* Blocks that can be handed out now (free, cached or not). */
int32_t pa_pool_available(const pa_block_pool* pool);

/* Reference count of one block (0 = free). */
int32_t pa_pool_refcount(const pa_block_pool* pool, int32_t block);

/* n fresh blocks with reference count 1 into ids[n]; PA_ERR_NOSPACE (and no
 * change) if fewer than n are available. */
int pa_pool_alloc(pa_block_pool* pool, int32_t n, int32_t* ids);

/* One more reference to each listed block (a sequence starts sharing it);
 * PA_ERR_SHAPE (and no change) if any is out of range or free. */
int pa_pool_fork(pa_block_pool* pool, const int32_t* ids, int32_t n);

/* One reference fewer for each listed block (a block may be listed as many
 * times as it has references); PA_ERR_SHAPE (and no change) otherwise. */
int pa_pool_release(pa_block_pool* pool, const int32_t* ids, int32_t n);

/*
 * pa_pool_map_prefix -- physical blocks for a request's full blocks, given
 * their chained hashes.  The longest leading run of hashes found in the
 * cache reuses those blocks (one more reference each; *n_hit = its length);
 * every later block is fresh and is entered in the cache under its hash.
 * PA_ERR_NOSPACE (and no change) if the fresh blocks are not available.
 *   hashes [n] uint64, ids [n] int32 (written), n_hit (written); host
 */
int pa_pool_map_prefix(pa_block_pool* pool, const uint64_t* hashes, int32_t n,
                       int32_t* ids, int32_t* n_hit);

/*
 * pa_pool_simulate -- requests growing token by token in a pool of n_blocks
 * blocks of block_size tokens, under one of two policies: the contrast of
 * the widget of "Serving" section 23.4 (a 96-block pool and eight requests:
 * reserving each request's worst case lets four run at once, paging lets
 * every request start when it arrives) and of the utilisation figures in
 * the "Paged Attention" summary on the inference-serving tag page.  Blocks
 * are real ids drawn from and returned to a pa_block_pool.
 *
 * Request i arrives at step arrivals[i] holding prompt_lens[i] tokens.  At
 * each step: arrived requests join a queue in arrival order (ties by index);
 * the head of the queue starts while the blocks it needs are free --
 *   PA_SIM_RESERVE: ceil(max_len / block_size) blocks, held to the end;
 *   PA_SIM_PAGED:   ceil(prompt / block_size) blocks, one more each time its
 *                   tokens pass the blocks it holds;
 * then the step is counted (running[step] = requests running; the step's
 * stored tokens and held capacity, blocks * block_size, are added to
 * *util_tokens and *util_capacity); then each running request finishes if
 * it holds final_lens[i] tokens (finish[i] = step, its blocks freed) or
 * gains one token.  The simulation ends after the step in which the last
 * request finishes; *n_steps = that step + 1.  Utilisation is
 * *util_tokens / *util_capacity.
 *
 *   arrivals, prompt_lens, final_lens [n_requests] int32, host, read
 *   start, finish [n_requests] int32, host, written
 *   running [max_steps] int32, host, written (the first min(n_steps,
 *           max_steps) entries)
 * Errors: PA_ERR_SHAPE for a negative arrival, a prompt < 1, a final length
 * below the prompt (or above max_len when reserving), or a trace longer than
 * max_steps (the other outputs are still complete); PA_ERR_NOSPACE if some
 * request needs more blocks than the pool has to start, or (paging) the
 * pool runs out while requests grow.
 */
enum { PA_SIM_RESERVE = 0, PA_SIM_PAGED = 1 };
int pa_pool_simulate(const int32_t* arrivals, const int32_t* prompt_lens,
                     const int32_t* final_lens, int32_t n_requests,
                     int32_t n_blocks, int32_t block_size, int32_t policy,
                     int32_t max_len, int32_t* start, int32_t* finish,
                     int32_t* running, int32_t max_steps, int32_t* n_steps,
                     int64_t* util_tokens, int64_t* util_capacity);

/* Static text for a status code; never NULL. */
const char* pa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
