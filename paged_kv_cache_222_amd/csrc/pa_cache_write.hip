// Cache write: each new token's K and V rows go to their pool slot.
//
// The cache grows position by position into fixed-size blocks ("Serving"
// section 23.4).  Flat slot s names block s >> block_shift, offset
// s & (block_size - 1).  A bit copy, no conversion.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kWriteThreads = 256;

// One thread per 16-byte chunk of a (token, KV head) row: it copies that
// chunk of K and of V.  Consecutive threads cover consecutive bytes of a
// token's rows, so both the reads and the writes are whole lines.
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(CacheWriteArgs a) {
  const int cpr = a.row_bytes >> 4;                 // chunks per row
  const int64_t per_tok = (int64_t)a.n_kv_heads * cpr;
  const int64_t gid = (int64_t)blockIdx.x * kWriteThreads + threadIdx.x;
  if (gid >= per_tok * a.n_tokens) return;
  const int tok = (int)(gid / per_tok);
  const int rem = (int)(gid - (int64_t)tok * per_tok);
  const int h = rem / cpr;
  const int c = rem - h * cpr;
  const int slot = a.slot_mapping[tok];
  const int64_t n_slots = (int64_t)a.n_blocks << a.block_shift;
  if (slot < 0 || (int64_t)slot >= n_slots) return;
  const int64_t blk = slot >> a.block_shift;
  const int off = slot & ((1 << a.block_shift) - 1);
  const int64_t src = gid * 16;
  const int64_t dst = (((blk * a.n_kv_heads + h) << a.block_shift) + off) * a.row_bytes + c * 16;
  const u32x4 kv = *(const u32x4*)((const char*)a.key + src);
  const u32x4 vv = *(const u32x4*)((const char*)a.value + src);
  *(u32x4*)((char*)a.k_pool + dst) = kv;
  *(u32x4*)((char*)a.v_pool + dst) = vv;
}

// The same copy with the slot taken from the block table: each sequence's
// new row goes to position context_lens[b] - 1 (a sequence with no position,
// whose table entry lies outside the pool, or whose new position lies in the
// shared positions [0, shared_len) is skipped).
__global__ __launch_bounds__(kWriteThreads) void append_kernel(AppendArgs a) {
  const int cpr = a.row_bytes >> 4;
  const int64_t per_seq = (int64_t)a.n_kv_heads * cpr;
  const int64_t gid = (int64_t)blockIdx.x * kWriteThreads + threadIdx.x;
  if (gid >= per_seq * a.batch) return;
  const int b = (int)(gid / per_seq);
  const int rem = (int)(gid - (int64_t)b * per_seq);
  const int h = rem / cpr;
  const int c = rem - h * cpr;
  const int ctx = a.context_lens[b];
  if (ctx < 1 || (int64_t)ctx > ((int64_t)a.max_blocks << a.block_shift)) return;
  const int pos = ctx - 1;
  if (pos < a.shared_len) return;
  const int blk = a.block_table[(int64_t)b * a.max_blocks + (pos >> a.block_shift)];
  if (blk < 0 || blk >= a.n_blocks) return;
  const int off = pos & ((1 << a.block_shift) - 1);
  const int64_t dst = ((((int64_t)blk * a.n_kv_heads + h) << a.block_shift) + off) * a.row_bytes + c * 16;
  const u32x4 kv = *(const u32x4*)((const char*)a.key + gid * 16);
  const u32x4 vv = *(const u32x4*)((const char*)a.value + gid * 16);
  *(u32x4*)((char*)a.k_pool + dst) = kv;
  *(u32x4*)((char*)a.v_pool + dst) = vv;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t chunks = (int64_t)a.batch * a.n_kv_heads * (a.row_bytes >> 4);
  const unsigned grid = (unsigned)((chunks + kWriteThreads - 1) / kWriteThreads);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(kWriteThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s) {
  const int64_t chunks = (int64_t)a.n_tokens * a.n_kv_heads * (a.row_bytes >> 4);
  const unsigned grid = (unsigned)((chunks + kWriteThreads - 1) / kWriteThreads);
  hipLaunchKernelGGL(cache_write_kernel, dim3(grid), dim3(kWriteThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
