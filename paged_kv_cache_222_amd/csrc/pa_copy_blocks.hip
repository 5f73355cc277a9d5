// Block copy for copy-on-write sharing of the paged cache.
//
// Sequences that share a prefix can share its physical blocks ("Serving"
// section 23.4); a shared block is copied before one of its sharers writes
// into it (copy-on-write sharing, named in the "Paged Attention" summary on
// the inference-serving tag page).  A block is one slice of each pool's
// first dimension: every KV head, position and dimension, bit for bit.
#include "pa_device.h"
#include "pa_launch.h"

#ifndef PA_COPY_NT_STORE
#define PA_COPY_NT_STORE 0
#endif
#ifndef PA_COPY_NT_LOAD
#define PA_COPY_NT_LOAD 1
#endif

namespace pa {

// Work group x copies chunk x % cpb of pool (x / cpb) % 2 of pair
// x / (2 cpb), cpb chunks per block.  Each thread moves up to kCopyUnroll
// 16-byte pieces, 4 KiB apart, all loads issued before any store; the copy
// is read once and written once, so both go non-temporal.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int64_t cpb = (a.block_bytes + kCopyChunk - 1) / kCopyChunk;
  const int64_t x = blockIdx.x;
  const int64_t pair = x / (2 * cpb);
  const int pool = (int)((x / cpb) & 1);
  const int64_t chunk = x % cpb;
  const __attribute__((address_space(4))) int32_t* pairs =
      (const __attribute__((address_space(4))) int32_t*)a.block_pairs;
  const int src = pairs[2 * pair];
  const int dst = pairs[2 * pair + 1];
  if (src < 0 || src >= a.n_blocks || dst < 0 || dst >= a.n_blocks) return;
  char* base = (char*)(pool ? a.v_pool : a.k_pool);
  const u32x4* from = (const u32x4*)(base + (int64_t)src * a.block_bytes + chunk * kCopyChunk);
  u32x4* to = (u32x4*)(base + (int64_t)dst * a.block_bytes + chunk * kCopyChunk);
  const int64_t n16 = min(kCopyChunk, a.block_bytes - chunk * kCopyChunk) >> 4;
  u32x4 r[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = threadIdx.x + u * kCopyThreads;
    if (i < n16) {
#if PA_COPY_NT_LOAD
      r[u] = __builtin_nontemporal_load(from + i);
#else
      r[u] = from[i];
#endif
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = threadIdx.x + u * kCopyThreads;
    if (i < n16) {
#if PA_COPY_NT_STORE
      __builtin_nontemporal_store(r[u], to + i);
#else
      to[i] = r[u];
#endif
    }
  }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  const int64_t cpb = (a.block_bytes + kCopyChunk - 1) / kCopyChunk;
  const unsigned grid = (unsigned)((int64_t)a.n_pairs * 2 * cpb);  // checked by the caller
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
