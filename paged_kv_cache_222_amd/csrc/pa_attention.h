// Decode attention over a paged KV cache: the kernel template.
//
// What is computed (one query token per sequence, "Serving" section 23.2;
// blocks + per-sequence table, section 23.4): for query head h of sequence b,
// out = softmax(scale * q K^T) V over the sequence's cached positions, K and V
// read through the block table.  The GQA group of query heads that share a KV
// head ("Serving" section 23.1) is processed by one work item, so every K/V
// byte is read from HBM once per step.
//
// Work item: (sequence b, KV head, chunk of <= 8 query heads[, partition]).
// A work group of four waves shares the item; the item's positions are cut
// into passes of 8 consecutive positions (a pass never crosses a block, since
// block sizes are multiples of 8) and pass k goes to wave k % 4.
//
// Lane layout inside a pass: lane = 8 * r + c handles position r of the pass
// and the 16-byte chunks at byte c*16 + 128*i (i < NC) of that position's
// row.  One load instruction thus covers 8 rows x 128 contiguous bytes, i.e.
// whole 128-byte lines.  The 8 lanes of a position reduce <q, k> with three
// DPP adds; each lane then keeps its own online-softmax state (m, l, o over its
// D/8 output elements) for the positions it sees.  The state is rescaled only
// when a logit exceeds the running maximum by more than kTau (log2 units):
// exp2(x - m) <= 2^kTau stays far from fp32 overflow, and the rescale branch
// is almost never taken after the first pass.  At the end the 8 row groups of
// a wave and the 4 waves are merged with the log-sum-exp rule.
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kPassTokens = 8;
constexpr float kTau = 8.0f;

template <Dt DT, int D>
struct Geo {
  static constexpr int EB = DtInfo<DT>::bytes;  // bytes per element
  static constexpr int RB = D * EB;             // bytes per (position, head) row
  static constexpr int NC = RB / 128;           // 16-byte chunks per lane per row
  static constexpr int EPC = 16 / EB;           // elements per chunk
  static constexpr int EPL = NC * EPC;          // elements per lane per row
  static constexpr int ECHUNK = 128 / EB;       // elements between a lane's chunks
  static_assert(RB % 128 == 0 && NC >= 1, "row must be a multiple of 128 bytes");
};

template <Dt DT, int D, int GC, int U>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(AttnArgs a) {
  using GE = Geo<DT, D>;
  constexpr int NC = GE::NC, EPC = GE::EPC, EPL = GE::EPL, RB = GE::RB, EB = GE::EB;
  constexpr int NW = kAttnThreads / kWave;

  __shared__ float s_m[NW][GC];
  __shared__ float s_l[NW][GC];
  __shared__ float s_o[NW][GC][D];
  __shared__ int s_bad[NW];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane >> 3;
  const int c = lane & 7;

  // ---- which work item: block ids run (row, kv head, head chunk) with the
  // KV head fastest, so with 8 | n_kv_heads every item of one KV head lands
  // on the same XCD (block id mod 8) and shares its L2.
  const int cols = a.n_kv_heads * a.n_hchunks;
  const int col = blockIdx.x % cols;
  const int rowi = blockIdx.x / cols;
  const int kvh = col / a.n_hchunks;
  const int hc = col - kvh * a.n_hchunks;
  const bool parts = a.partition_size > 0;
  int b, jrow = 0;
  if (parts) {
    jrow = rowi / a.batch;
    b = rowi - jrow * a.batch;
  } else {
    b = rowi;
  }
  const int ctx = a.context_lens[b];
  const int bs = 1 << a.block_shift;
  const int G = a.gqa_group;
  const int Hq = a.n_kv_heads * G;
  const int h0 = kvh * G + hc * GC;
  const int gv = min(GC, G - hc * GC);
  // invalid length, or a new token written into the shared positions
  const bool bad_ctx = ctx < 0 || (int64_t)ctx > ((int64_t)a.max_blocks << a.block_shift) ||
                       (ctx >= 1 && ctx - 1 < a.shared_len);

  int t0 = 0, t1 = ctx, p = 0;
  if (parts) {
    const int P = a.partition_size;
    const int64_t np64 = ctx > 0 ? ((int64_t)ctx + P - 1) / P : 0;
    // np > max_partitions (and ctx < 0) are reported as NaN by pa_reduce;
    // the fp32 step's cache write is a kernel of its own and still happens.
    if (np64 > a.max_partitions) return;
    const int np = (int)np64;
    // Rows are dispatched in order; row j holds partition np - PMAX + j, so
    // the last rows carry every sequence's final (partial) partition and the
    // dispatcher fills the tail of the launch with the smallest items.
    p = np - a.max_partitions + jrow;
    if (p < 0) return;
    if (bad_ctx) {
      const float qnan = __builtin_nanf("");
      for (int idx = threadIdx.x; idx < gv * D; idx += kAttnThreads) {
        const int g = idx / D, d = idx - g * D;
        const int64_t prow = (int64_t)(b * Hq + h0 + g) * a.max_partitions + p;
        a.tmp_out[prow * D + d] = qnan;
        if (d == 0) {
          a.max_logits[prow] = qnan;
          a.exp_sums[prow] = qnan;
        }
      }
      return;
    }
    t0 = p * P;
    t1 = min(t0 + P, ctx);
  } else if (bad_ctx || ctx == 0) {
    const float v = bad_ctx ? __builtin_nanf("") : 0.0f;
    for (int idx = threadIdx.x; idx < gv * D; idx += kAttnThreads) {
      const int g = idx / D, d = idx - g * D;
      store_elem<DT>(a.out, (int64_t)(b * Hq + h0 + g) * D + d, v);
    }
    return;
  }

  // ---- this lane's slice of the chunk's queries (raw storage bits)
  u32x4 qv[GC][NC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const char* qrow = (const char*)a.q + (int64_t)(b * Hq + h0 + g) * RB;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (g < gv)
        qv[g][i] = *(const u32x4*)(qrow + i * 128 + c * 16);
      else
        qv[g][i] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int ntok = t1 - t0;
  const int npass = (ntok + kPassTokens - 1) / kPassTokens;
  const int my_n = npass > wave ? (npass - 1 - wave) / NW + 1 : 0;
  const int64_t tile_bytes = (int64_t)bs * RB;            // one (block, head)
  const int64_t blk_bytes = tile_bytes * a.n_kv_heads;    // one block
  const char* kbase = (const char*)a.k_pool + kvh * tile_bytes;
  const char* vbase = (const char*)a.v_pool + kvh * tile_bytes;
  const uint32_t lane_off = (uint32_t)(r * RB + c * 16);
  // The table row is read with scalar loads (constant address space): they
  // are counted apart from the vector loads, so waiting for a block id never
  // waits for K/V data in flight.
  const __attribute__((address_space(4))) int32_t* trow =
      (const __attribute__((address_space(4))) int32_t*)(a.block_table +
                                                         (int64_t)b * a.max_blocks);
  bool bad = false;

  // Pass idx of this wave (clamped: past the end it repeats the last pass,
  // which keeps the number of loads in flight static).
  auto pass_of = [&](int idx) { return wave + min(idx, my_n - 1) * NW; };
  auto fetch_ids = [&](int idx0, int (&ph)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      ph[u] = trow[(t0 + pass_of(idx0 + u) * kPassTokens) >> a.block_shift];
  };
  auto issue = [&](int idx0, const int (&ph)[U], u32x4 (&kc)[U][NC], u32x4 (&vc)[U][NC]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pass = pass_of(idx0 + u);
      const bool ok = ph[u] >= 0 && ph[u] < a.n_blocks;
      bad |= !ok;
      const int64_t phys = ok ? ph[u] : 0;
      const int off0 = (t0 + pass * kPassTokens) & (bs - 1);
      const int64_t boff = phys * blk_bytes + (int64_t)off0 * RB;
      const char* kp = kbase + boff;
      const char* vp = vbase + boff;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        kc[u][i] = *(const u32x4*)(kp + lane_off + i * 128);
        vc[u][i] = *(const u32x4*)(vp + lane_off + i * 128);
      }
    }
  };

  float m[GC], l[GC], o[GC][EPL];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = -__builtin_huge_valf();
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.0f;
  }
  const float sl2 = a.scale_log2;

  // One pass: logits of this lane's position for the GC heads, online
  // softmax update, V accumulation.  All branches are wave-uniform; the
  // partial last pass masks its invalid positions with selects.
  auto compute_pass = [&](int idx, const u32x4 (&kc)[NC], const u32x4 (&vc)[NC]) {
    const int tok0 = t0 + (wave + idx * NW) * kPassTokens;
    const bool full = tok0 + kPassTokens <= t1;
    const bool valid = tok0 + r < t1;
    float x[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NC; ++i) acc = dot_chunk<DT>(kc[i], qv[g][i], acc);
      x[g] = sum8(acc) * sl2;
      if (!full) x[g] = valid ? x[g] : -__builtin_huge_valf();
    }
    bool need = false;
#pragma unroll
    for (int g = 0; g < GC; ++g) need |= x[g] > m[g] + kTau;
    if (__ballot(need)) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        const float mn = fmaxf(m[g], x[g]);
        const float al = (m[g] == mn) ? 1.0f : exp2_fast(m[g] - mn);
        l[g] *= al;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] *= al;
        m[g] = mn;
      }
    }
    float vf[EPL];
#pragma unroll
    for (int i = 0; i < NC; ++i) Unpack<DT>::run(vc[i], vf + i * EPC);
    if (!full) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[e] = valid ? vf[e] : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float pg = exp2_fast(x[g] - m[g]);
      if (!full) pg = valid ? pg : 0.0f;
      l[g] += pg;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = __builtin_fmaf(pg, vf[e], o[g][e]);
    }
  };

  if (my_n > 0) {
    u32x4 ka[U][NC], va[U][NC], kb[U][NC], vb[U][NC];
    int pa_[U], pb_[U];
    fetch_ids(0, pa_);
    issue(0, pa_, ka, va);
    fetch_ids(U, pb_);
    for (int base = 0; base < my_n; base += 2 * U) {
      issue(base + U, pb_, kb, vb);
      fetch_ids(base + 2 * U, pa_);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (base + u < my_n) compute_pass(base + u, ka[u], va[u]);
      if (base + U >= my_n) break;
      issue(base + 2 * U, pa_, ka, va);
      fetch_ids(base + 3 * U, pb_);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (base + U + u < my_n) compute_pass(base + U + u, kb[u], vb[u]);
    }
  }

  // ---- merge the 8 row groups of this wave (lanes 8r + c, fixed c)
  auto merge_with = [&](auto partner) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float mo = partner(m[g]);
      const float lo = partner(l[g]);
      const float M = fmaxf(m[g], mo);
      const float a1 = (m[g] == -__builtin_huge_valf()) ? 0.0f : exp2_fast(m[g] - M);
      const float a2 = (mo == -__builtin_huge_valf()) ? 0.0f : exp2_fast(mo - M);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = o[g][e] * a1 + partner(o[g][e]) * a2;
      m[g] = M;
    }
  };
  merge_with([](float v) { return xor8(v); });
  merge_with([](float v) { return shfl_xor_f(v, 16); });
  merge_with([](float v) { return shfl_xor_f(v, 32); });

  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g)
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int j = 0; j < EPC; ++j)
          s_o[wave][g][i * GE::ECHUNK + c * EPC + j] = o[g][i * EPC + j];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      s_m[wave][g] = m[g];
      s_l[wave][g] = l[g];
    }
    s_bad[wave] = bad ? 1 : 0;
  }
  __syncthreads();

  // ---- merge the waves and write
  bool anybad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) anybad |= s_bad[w] != 0;
  const float qnan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < gv * D; idx += kAttnThreads) {
    const int g = idx / D, d = idx - g * D;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][g];
      const float aw = (mw == -__builtin_huge_valf()) ? 0.0f : exp2_fast(mw - M);
      L += aw * s_l[w][g];
      O += aw * s_o[w][g][d];
    }
    const int h = h0 + g;
    if (parts) {
      const int64_t prow = (int64_t)(b * Hq + h) * a.max_partitions + p;
      a.tmp_out[prow * D + d] = anybad ? qnan : O / L;
      if (d == 0) {
        a.max_logits[prow] = anybad ? qnan : M * kLn2;
        a.exp_sums[prow] = anybad ? qnan : L;
      }
    } else {
      const float v = anybad ? qnan : (L > 0.0f ? O / L : 0.0f);
      store_elem<DT>(a.out, (int64_t)(b * Hq + h) * D + d, v);
    }
  }
  (void)EB;
}

template <Dt DT, int D, int GC>
hipError_t launch_gc(const AttnArgs& a, unsigned grid, hipStream_t s) {
  constexpr int U = GC <= 4 ? 2 : 1;
  launch_timed(attention_kernel<DT, D, GC, U>, dim3(grid), dim3(kAttnThreads), s, a);
  return hipGetLastError();
}

template <Dt DT, int D>
hipError_t launch_d(const AttnArgs& a, int gc, unsigned grid, hipStream_t s) {
  switch (gc) {
    case 1: return launch_gc<DT, D, 1>(a, grid, s);
    case 2: return launch_gc<DT, D, 2>(a, grid, s);
    case 3: return launch_gc<DT, D, 3>(a, grid, s);
    case 4: return launch_gc<DT, D, 4>(a, grid, s);
    case 5: return launch_gc<DT, D, 5>(a, grid, s);
    case 6: return launch_gc<DT, D, 6>(a, grid, s);
    case 7: return launch_gc<DT, D, 7>(a, grid, s);
    case 8: return launch_gc<DT, D, 8>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <Dt DT>
hipError_t launch_attention_dt(const AttnArgs& a, int d_head, int gc, unsigned grid,
                               hipStream_t s) {
  switch (d_head) {
    case 64: return launch_d<DT, 64>(a, gc, grid, s);
    case 128: return launch_d<DT, 128>(a, gc, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
