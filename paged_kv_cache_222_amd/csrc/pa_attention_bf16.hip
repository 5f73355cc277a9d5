// Attention kernels instantiated for the bf16 element type.
#include "pa_attention.h"

namespace pa {

hipError_t launch_attention_bf16(const AttnArgs& a, int d_head, int heads_per_chunk,
                                 unsigned grid, hipStream_t s) {
  return launch_attention_dt<Dt::BF16>(a, d_head, heads_per_chunk, grid, s);
}

}  // namespace pa
