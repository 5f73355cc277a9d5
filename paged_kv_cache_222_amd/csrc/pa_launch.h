// Host-side launch interface between the C ABI (pa_api.hip) and the kernel
// translation units.  Not part of the public header.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Arguments of the attention kernel.  partition_size == 0 selects the
// single-pass mode (one work item covers a sequence's whole context and
// writes `out`); otherwise each work item covers one partition and writes
// max_logits / exp_sums / tmp_out.
struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* out;
  float* max_logits;
  float* exp_sums;
  float* tmp_out;
  // Partitioned decode with the step's cache write folded in: each
  // sequence's new key/value row [n_kv_heads, d_head] goes to position
  // context_len - 1 (null: no write).
  const void* key_new;
  const void* value_new;
  int32_t max_blocks;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t gqa_group;
  int32_t n_hchunks;   // query-head chunks per KV head
  int32_t heads_per_chunk;
  int32_t block_shift; // log2(block_size)
  int32_t n_blocks;
  int32_t partition_size;
  int32_t max_partitions;
  int32_t persistent;  // partitioned launch sized to the GPU, items planned in-kernel
  int32_t n_queries;   // query tokens per sequence (the last n_queries positions)
  // Shared prefix (persistent partitioned launches, n_queries == 1): the
  // first prefix_parts partitions lie in blocks every table row shares, and
  // one work item computes such a partition for prefix_seqs consecutive
  // sequences at once (columns = (sequence, head) pairs).  0: off.
  int32_t prefix_parts;
  int32_t prefix_seqs;
  // With a folded write into a batch whose positions [0, shared_len) sit in
  // blocks every row shares: a sequence whose new token falls there would
  // write into a shared block, so it is a contract violation -- no write,
  // NaN outputs.  0: no such positions.
  int32_t shared_len;
  // pa_decode_split: work groups take equal runs of the tiles of all
  // sequences, writing one workspace slot per sequence piece
  // (partition_size is 0).
  int32_t split;
  // Persistent partitioned launches (not split) with two work groups on
  // every CU: deal the plan's items over CUs rather than work groups (the
  // kernel's item loop says how).  0: deal over work groups; 1: a CU's
  // rounds alternate between its two work groups; 2: pairs of rounds do
  // (launches with shared items, whose list alternates shared and private
  // items).
  int32_t cu_deal;
  // With cu_deal 1, when half the grid is a multiple of 8 * columns: spread
  // every column over the eight XCDs (see the kernel).  0: column =
  // block % columns.
  int32_t xcd_spread;
  float scale_log2;    // scale * log2(e)
};

// partition_size == 0: the workspace of pa_decode_split (every slot merged,
// empty ones -- exp_sums 0 -- skipped).
struct ReduceArgs {
  void* out;
  const float* max_logits;
  const float* exp_sums;
  const float* tmp_out;
  const int32_t* context_lens;
  int32_t batch;
  int32_t n_q_heads;
  int32_t partition_size;
  int32_t max_partitions;
};

struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* k_pool;
  void* v_pool;
  const int32_t* slot_mapping;
  int32_t n_tokens;
  int32_t n_kv_heads;
  int32_t row_bytes;   // d_head * element size
  int32_t block_shift;
  int32_t n_blocks;
};

struct AppendArgs {
  const void* key;      // [batch, n_kv_heads, d_head]
  const void* value;
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t batch;
  int32_t max_blocks;
  int32_t n_kv_heads;
  int32_t row_bytes;
  int32_t block_shift;
  int32_t n_blocks;
  int32_t shared_len;   // as in AttnArgs: a new token before it is not written
};

constexpr int kCopyThreads = 256;
#ifndef PA_COPY_UNROLL
#define PA_COPY_UNROLL 4
#endif
constexpr int kCopyUnroll = PA_COPY_UNROLL;  // 16-byte loads in flight per thread
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * 16 * kCopyUnroll;  // bytes per work group

struct CopyBlocksArgs {
  void* k_pool;
  void* v_pool;
  const int32_t* block_pairs;  // [n_pairs, 2]: source, destination
  int32_t n_pairs;
  int32_t n_blocks;
  int64_t block_bytes;         // n_kv_heads * block_size * d_head * element size
};

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;   // tiles whose loads are in flight together

struct ReadCeilingArgs {
  const void* buf;
  const int32_t* tile_order;  // null: tiles in address order
  uint32_t* sink;
  int64_t n_tiles;            // tiles to read
  int64_t buf_tiles;          // tiles in the buffer (ids outside are skipped)
  int64_t tile_bytes;         // a multiple of 16
};

// Measurement aid behind pa_time_next_attention: if events were set on
// this thread, hand them over (and clear them) so that the attention launch
// records its own start and end in them.
bool take_attention_events(hipEvent_t* start, hipEvent_t* stop);

// A kernel launch that records its start and end in the events set by
// pa_time_next_attention, if any (the timestamps of the dispatch itself),
// and is an ordinary launch otherwise.
template <typename F, typename... Args>
void launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (take_attention_events(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// Each returns a hipError_t from the launch.
hipError_t launch_attention_f32(const AttnArgs& a, int d_head, int heads_per_chunk,
                                unsigned grid, hipStream_t s);
hipError_t launch_attention_vector_f16(const AttnArgs& a, int d_head, int heads_per_chunk,
                                       unsigned grid, hipStream_t s);
hipError_t launch_attention_vector_bf16(const AttnArgs& a, int d_head, int heads_per_chunk,
                                        unsigned grid, hipStream_t s);
hipError_t launch_attention_mfma_f16(const AttnArgs& a, int d_head, unsigned grid,
                                     hipStream_t s);
hipError_t launch_attention_mfma_bf16(const AttnArgs& a, int d_head, unsigned grid,
                                      hipStream_t s);
// Work groups of the matrix-core attention kernel that fit on one CU.
int attention_mfma_occupancy(int dtype, int d_head);
hipError_t launch_reduce(const ReduceArgs& a, int dtype, int d_head, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
hipError_t launch_read_ceiling(const ReadCeilingArgs& a, unsigned grid, hipStream_t s);

constexpr int kAttnThreads = 256;  // four waves per work item
constexpr int kMfmaHeads = 16;     // columns (query token, head pairs) per matrix-core work item
constexpr int kPlanBatch = 1024;   // largest batch the in-kernel partition plan handles

}  // namespace pa
