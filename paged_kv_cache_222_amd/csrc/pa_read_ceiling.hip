// Read-bandwidth calibration: the rate at which the device streams a buffer
// from HBM, sequentially or as a gather of fixed-size tiles in a given order
// (the access pattern of the attention kernels: one 4 KiB tile per block
// and KV head, blocks scattered through the pool).  Its result is the
// achievable ceiling the attention kernels' HBM rates are compared with.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Work group x reads the tiles [x * span, (x + 1) * span) of the order
// (kReadUnroll tiles per round, every load of a round issued before any is
// used; the tile ids come 64 at a time, one per lane, the next 64 loaded
// while the current ones are read).  Thread i reads the 16-byte pieces
// i, i + 256, ... of each tile, non-temporal.  The bytes are folded into one
// word that is stored only if it equals a fixed constant, which keeps the
// loads without writing anything in practice.
__global__ __launch_bounds__(kReadThreads) void read_ceiling_kernel(ReadCeilingArgs a) {
  const int64_t per_tile = a.tile_bytes >> 4;   // 16-byte pieces per tile
  const u32x4* buf = (const u32x4*)a.buf;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t span = (a.n_tiles + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * span;
  const int64_t hi = min(lo + span, a.n_tiles);
  auto ids = [&](int64_t base) -> int {   // lane l: tile id of position base + l
    const int64_t t = base + lane;
    if (t >= hi) return -1;
    return a.tile_order ? a.tile_order[t] : (int)t;
  };
  uint32_t acc = 0;
  int next = lo < hi ? ids(lo) : -1;
  for (int64_t base = lo; base < hi; base += kWave) {
    const int cur = next;
    if (base + kWave < hi) next = ids(base + kWave);
    const int nb = (int)min((int64_t)kWave, hi - base);
    for (int j = 0; j < nb; j += kReadUnroll) {
      for (int64_t c = threadIdx.x; c < per_tile; c += kReadThreads) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int k = 0; k < kReadUnroll; ++k) {
          const int tile = __builtin_amdgcn_readlane(cur, min(j + k, kWave - 1));
          const bool ok = j + k < nb && tile >= 0 && tile < a.buf_tiles;
          v[k] = ok ? __builtin_nontemporal_load(buf + (int64_t)tile * per_tile + c)
                    : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
      }
    }
  }
  if (acc == 0x9E3779B9u) a.sink[0] = acc;
}

hipError_t launch_read_ceiling(const ReadCeilingArgs& a, unsigned grid, hipStream_t s) {
  launch_timed(read_ceiling_kernel, dim3(grid), dim3(kReadThreads), s, a);
  return hipGetLastError();
}

}  // namespace pa
