// The vector-ALU attention kernel (the one fp32 caches use) instantiated for
// the 16-bit element types.  16-bit caches normally run on the matrix cores;
// this form is reached only through pa_decode_partitioned_vector, which
// exists to time the two engines on the same batch.
#include "pa_attention.h"

namespace pa {

hipError_t launch_attention_vector_f16(const AttnArgs& a, int d_head, int heads_per_chunk,
                                       unsigned grid, hipStream_t s) {
  return launch_attention_dt<Dt::F16>(a, d_head, heads_per_chunk, grid, s);
}

hipError_t launch_attention_vector_bf16(const AttnArgs& a, int d_head, int heads_per_chunk,
                                        unsigned grid, hipStream_t s) {
  return launch_attention_dt<Dt::BF16>(a, d_head, heads_per_chunk, grid, s);
}

}  // namespace pa
