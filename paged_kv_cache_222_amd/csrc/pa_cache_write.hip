// Cache write: each new token's K and V rows go to their pool slot.
//
// The cache grows position by position into fixed-size blocks ("Serving"
// section 23.4).  Flat slot s names block s >> block_shift, offset
// s & (block_size - 1).  One wave per token copies its n_kv_heads rows of K and
// of V with 16-byte loads and stores; a bit copy, no conversion.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kWriteWaves = 4;

__global__ __launch_bounds__(kWave* kWriteWaves) void cache_write_kernel(CacheWriteArgs a) {
  const int tok = blockIdx.x * kWriteWaves + (int)(threadIdx.x / kWave);
  if (tok >= a.n_tokens) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int slot = a.slot_mapping[tok];
  const int64_t n_slots = (int64_t)a.n_blocks << a.block_shift;
  if (slot < 0 || (int64_t)slot >= n_slots) return;
  const int64_t blk = slot >> a.block_shift;
  const int off = slot & ((1 << a.block_shift) - 1);
  const int RB = a.row_bytes;
  const int total = a.n_kv_heads * RB;
  const char* ks = (const char*)a.key + (int64_t)tok * total;
  const char* vs = (const char*)a.value + (int64_t)tok * total;
  char* kd = (char*)a.k_pool;
  char* vd = (char*)a.v_pool;
  for (int x = lane * 16; x < total; x += kWave * 16) {
    const int h = x / RB;
    const int w = x - h * RB;
    const int64_t dst = (((blk * a.n_kv_heads + h) << a.block_shift) + off) * RB + w;
    const u32x4 kv = *(const u32x4*)(ks + x);
    const u32x4 vv = *(const u32x4*)(vs + x);
    *(u32x4*)(kd + dst) = kv;
    *(u32x4*)(vd + dst) = vv;
  }
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n_tokens + kWriteWaves - 1) / kWriteWaves);
  hipLaunchKernelGGL(cache_write_kernel, dim3(grid), dim3(kWave * kWriteWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
