// Matrix-core attention kernels instantiated for fp16 and bf16.
#include "pa_attention_mfma.h"

namespace pa {

hipError_t launch_attention_mfma_f16(const AttnArgs& a, int d_head, unsigned grid,
                                     hipStream_t s) {
  return launch_attention_mfma<Dt::F16>(a, d_head, grid, s);
}

hipError_t launch_attention_mfma_bf16(const AttnArgs& a, int d_head, unsigned grid,
                                      hipStream_t s) {
  return launch_attention_mfma<Dt::BF16>(a, d_head, grid, s);
}

int attention_mfma_occupancy(int dtype, int d_head) {
  return dtype == 1 ? attention_mfma_blocks_per_cu<Dt::F16>(d_head)
                    : attention_mfma_blocks_per_cu<Dt::BF16>(d_head);
}

}  // namespace pa

#ifdef PA_TIMELINE
// The timeline's host side (measurement build only; not in include/pa.h).
extern "C" int pa_timeline_copy(void* dst, size_t bytes) {
  if (bytes > sizeof(pa::g_timeline)) return -2;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(pa::g_timeline), bytes, 0, hipMemcpyDeviceToHost) ==
                 hipSuccess
             ? 0
             : -1;
}
extern "C" int pa_timeline_clear() {
  static unsigned long long zero[pa::kTimelineGroups * pa::kTimelineSlots];
  return hipMemcpyToSymbol(HIP_SYMBOL(pa::g_timeline), zero, sizeof(zero), 0,
                           hipMemcpyHostToDevice) == hipSuccess
             ? 0
             : -1;
}
#endif
