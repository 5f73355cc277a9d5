// Merge of per-partition softmax statistics (log-sum-exp rule).
//
// Partition p of a sequence holds (m_p, l_p, o_p) with l_p = sum exp(s - m_p)
// and o_p the normalised partial output.  Then l_p exp(m_p) is that
// partition's softmax denominator, and attention over the whole context is
// the mean of the o_p weighted by w_p = l_p exp(m_p - M), M = max_p m_p.
// One wave per (sequence, query head), four per work group; lanes own
// d_head/64 output elements.
//
// With partition_size == 0 the workspace holds the pieces of a split launch
// (pa_decode_split): every slot is merged, and a slot with l = 0 (a piece
// the sequence does not have) is skipped -- its o is never read into the
// sum, so it need not be written.  Skipping l = 0 leaves the partitioned
// results unchanged: there such a slot (a verify-pass token that sees
// nothing) holds o = 0 and adds nothing.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Workspaces of at most kFewParts partitions: every load of the row (its
// context length, all m_p, l_p and this lane's o_p elements) is issued at
// once, then the partitions past the sequence's end are masked, so the row
// costs one memory round trip instead of three.
constexpr int kFewParts = 8;
// (sequence, query head) rows per work group, one wave each: fewer, larger
// work groups are dispatched faster than one 64-thread group per row.
#ifndef PA_REDUCE_ROWS
#define PA_REDUCE_ROWS 4
#endif
constexpr int kRedRows = PA_REDUCE_ROWS;

template <Dt DT, int D, int FEW>
__global__ __launch_bounds__(kWave * kRedRows) void reduce_few_kernel(ReduceArgs a) {
  constexpr int DPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t bh64 = (int64_t)blockIdx.x * kRedRows + threadIdx.x / kWave;
  if (bh64 >= (int64_t)a.batch * a.n_q_heads) return;
  const int bh = (int)bh64;
  const int b = bh / a.n_q_heads;
  const int PM = a.max_partitions;  // <= FEW
  const float* ml = a.max_logits + (int64_t)bh * PM;
  const float* es = a.exp_sums + (int64_t)bh * PM;
  const float* to = a.tmp_out + (int64_t)bh * PM * D + lane * DPL;
  const int ctx = a.context_lens[b];
  float m[FEW], l[FEW], o[FEW][DPL];
#pragma unroll
  for (int p = 0; p < FEW; ++p) {
    if (p < PM) {
      m[p] = ml[p];
      l[p] = es[p];
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[p][k] = to[(int64_t)p * D + k];
    }
  }
  const int64_t orow = (int64_t)bh * D;
  const int P = a.partition_size;
  const int64_t np64 = ctx > 0 ? (P > 0 ? ((int64_t)ctx + P - 1) / P : PM) : 0;
  if (ctx < 0 || np64 > PM || np64 == 0) {
    const float v = (np64 == 0 && ctx == 0) ? 0.0f : __builtin_nanf("");
#pragma unroll
    for (int k = 0; k < DPL; ++k) store_elem<DT>(a.out, orow + lane * DPL + k, v);
    return;
  }
  const int np = (int)np64;
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int p = 0; p < FEW; ++p)
    if (p < np) M = fmaxf(M, m[p]);
  float W = 0.0f, acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.0f;
#pragma unroll
  for (int p = 0; p < FEW; ++p) {
    if (p < np && l[p] != 0.0f) {
      const float w = l[p] * exp2_fast((m[p] - M) * kLog2e);
      W += w;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = __builtin_fmaf(w, o[p][k], acc[k]);
    }
  }
  // W = 0: a query token that sees no position (multi-token queries only);
  // a NaN W (a partition flagged bad) stays NaN
#pragma unroll
  for (int k = 0; k < DPL; ++k)
    store_elem<DT>(a.out, orow + lane * DPL + k, W == 0.0f ? 0.0f : acc[k] / W);
}

template <Dt DT, int D>
__global__ __launch_bounds__(kWave * kRedRows) void reduce_kernel(ReduceArgs a) {
  constexpr int DPL = D / kWave;  // output elements per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t bh64 = (int64_t)blockIdx.x * kRedRows + threadIdx.x / kWave;
  if (bh64 >= (int64_t)a.batch * a.n_q_heads) return;
  const int bh = (int)bh64;  // b * n_q_heads + h
  const int b = bh / a.n_q_heads;
  const int ctx = a.context_lens[b];
  const int P = a.partition_size;
  const int64_t orow = (int64_t)bh * D;
  const int64_t np64 = ctx > 0 ? (P > 0 ? ((int64_t)ctx + P - 1) / P : a.max_partitions) : 0;
  if (ctx < 0 || np64 > a.max_partitions || np64 == 0) {
    const float v = (np64 == 0 && ctx == 0) ? 0.0f : __builtin_nanf("");
#pragma unroll
    for (int k = 0; k < DPL; ++k) store_elem<DT>(a.out, orow + lane * DPL + k, v);
    return;
  }
  const int np = (int)np64;
  const float* ml = a.max_logits + (int64_t)bh * a.max_partitions;
  const float* es = a.exp_sums + (int64_t)bh * a.max_partitions;
  const float* to = a.tmp_out + (int64_t)bh * a.max_partitions * D + lane * DPL;

  // M over all partitions (lane p reads partitions p, p + 64, ...)
  float M = -__builtin_huge_valf();
  for (int p = lane; p < np; p += kWave) M = fmaxf(M, ml[p]);
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) M = fmaxf(M, shfl_xor_f(M, s));

  float W = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.0f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    // the weights of 64 partitions at once, one per lane
    const int pl = p0 + lane;
    const float w = pl < np ? es[pl] * exp2_fast((ml[pl] - M) * kLog2e) : 0.0f;
    float ws = w;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) ws += shfl_xor_f(ws, s);
    W += ws;
    const int n = min(kWave, np - p0);
    int j = 0;
    for (; j + 4 <= n; j += 4) {
      float wj[4], oj[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wj[u] = as_f(__builtin_amdgcn_readlane((int)as_u(w), j + u));
#pragma unroll
        for (int k = 0; k < DPL; ++k) oj[u][k] = to[(int64_t)(p0 + j + u) * D + k];
      }
      // a zero weight (an empty slot) is skipped: its o may be unwritten
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < DPL; ++k)
          acc[k] = wj[u] != 0.0f ? __builtin_fmaf(wj[u], oj[u][k], acc[k]) : acc[k];
    }
    for (; j < n; ++j) {
      const float wj = as_f(__builtin_amdgcn_readlane((int)as_u(w), j));
      if (wj == 0.0f) continue;
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        acc[k] = __builtin_fmaf(wj, to[(int64_t)(p0 + j) * D + k], acc[k]);
    }
  }
#pragma unroll
  // W = 0: a query token that sees no position (multi-token queries only);
  // a NaN W (a partition flagged bad) stays NaN
  for (int k = 0; k < DPL; ++k)
    store_elem<DT>(a.out, orow + lane * DPL + k, W == 0.0f ? 0.0f : acc[k] / W);
}

template <Dt DT>
static hipError_t launch_reduce_dt(const ReduceArgs& a, int d_head, hipStream_t s) {
  const unsigned grid = (unsigned)(((int64_t)a.batch * a.n_q_heads + kRedRows - 1) / kRedRows);
  const bool few = a.max_partitions <= kFewParts;
  // split workspaces of up to 16 pieces also take one round trip (for
  // partitioned workspaces of 9-16 the general loop measured faster)
  const bool few16 = !few && a.partition_size == 0 && a.max_partitions <= 2 * kFewParts;
  const dim3 g(grid), t(kWave * kRedRows);
  if (d_head == 64) {
    if (few)
      hipLaunchKernelGGL((reduce_few_kernel<DT, 64, kFewParts>), g, t, 0, s, a);
    else if (few16)
      hipLaunchKernelGGL((reduce_few_kernel<DT, 64, 2 * kFewParts>), g, t, 0, s, a);
    else
      hipLaunchKernelGGL((reduce_kernel<DT, 64>), g, t, 0, s, a);
  } else if (d_head == 128) {
    if (few)
      hipLaunchKernelGGL((reduce_few_kernel<DT, 128, kFewParts>), g, t, 0, s, a);
    else if (few16)
      hipLaunchKernelGGL((reduce_few_kernel<DT, 128, 2 * kFewParts>), g, t, 0, s, a);
    else
      hipLaunchKernelGGL((reduce_kernel<DT, 128>), g, t, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int dtype, int d_head, hipStream_t s) {
  switch (dtype) {
    case 0: return launch_reduce_dt<Dt::F32>(a, d_head, s);
    case 1: return launch_reduce_dt<Dt::F16>(a, d_head, s);
    case 2: return launch_reduce_dt<Dt::BF16>(a, d_head, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
