// Decode attention over a paged KV cache on the matrix cores (fp16/bf16).
//
// Computes, for every query head h of sequence b, softmax(scale * q K^T) V
// over the sequence's cached positions read through its block table
// ("Serving" section 23.2: decode reads the whole cached K/V of a sequence for
// one query token; section 23.4: fixed-size blocks and a per-sequence table).
// The G query heads that share a KV head (section 23.1) are one work item, so
// each K/V byte is read from HBM once per step.  With n_queries > 1 the
// columns of a work item are (query token, head) pairs of the last
// n_queries positions, causal among themselves (the verify pass of
// speculative decoding, section 23.5), still one read of each K/V byte.
//
// Tiles of 16 consecutive positions.  For a tile:
//   S = K Q^T       v_mfma_f32_16x16x32: A = K rows (lane l: position l%16,
//                   16 bytes at dims 32j + 8(l/16)); B = the queries (lane l:
//                   column l%16, zero past the chunk); C = S (lane l:
//                   positions 4(l/16)+i, column l%16)
//   P = exp2(S*scale*log2e - m), rounded to the storage type
//   O += P V        v_mfma_f32_16x16x16: A = P, which is exactly the C layout
//                   of S; B = V (lane l: positions 4(l/16)..+3 of dim l%16).
// K and V tiles are copied HBM -> LDS with global_load_lds (non-temporal);
// K is read back with ds_read_b128 (16-byte chunks swizzled per row against
// bank conflicts), V transposed with ds_read_b64_tr_b16.
// The running maximum m is per column and shared by the four lanes holding
// it; it is raised only when a tile's maximum exceeds it by more than kTau
// (log2 units), so exp2(S - m) <= 2^kTau.  The normaliser l sums the rounded
// P, so the weights applied to V are exactly the ones summed.
//
// Work items are (sequence, KV head, chunk of <= 16 columns[, partition])
// and four waves share one item, taking its tiles round-robin, each wave
// double-buffering its own two slots; their states are merged in LDS with
// the log-sum-exp rule at the end of the item.  Partitioned launches are
// persistent: every work group derives the same item list from the context
// lengths (full partitions, then final partitions longest first) and takes
// its items in a back-and-forth deal over the work groups of its column.
// No work group is launched for an empty partition.  With a shared prefix
// (blocks every table row shares) its partitions are items of their own,
// each for up to 16 / G sequences -- columns (sequence, head) pairs -- so a
// prefix tile is read once per such group rather than once per sequence.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// A timeline of every work group, in a measurement build only (built with
// -DPA_TIMELINE; bench.py --op timeline reads it): thread 0 of work group g
// stores 64-bit words at g * kTimelineSlots + slot of g_timeline, with
// vector stores -- slot 0 the start (s_memrealtime, a 100 MHz counter), 1
// the end of the plan, 2 the end, 3 the number of items completed, 60 the
// XCC id << 32 | HW_ID, and for item k < kTimelineItems: 4 + 3k its start,
// 5 + 3k its end, 6 + 3k its tiles | shared << 20 | sequence << 32; in the
// partition plan also 58 (context lengths in), 59 (after the scans) and 61
// (after the rank).  In the product build the macros are empty.
constexpr int kTimelineGroups = 4096;
constexpr int kTimelineSlots = 64;
constexpr int kTimelineItems = 18;
#ifdef PA_TIMELINE
__device__ unsigned long long g_timeline[kTimelineGroups * kTimelineSlots];
#define PA_TL(slot, v)                                                        \
  do {                                                                        \
    if (threadIdx.x == 0 && blockIdx.x < kTimelineGroups)                     \
      g_timeline[blockIdx.x * kTimelineSlots + (slot)] = (unsigned long long)(v); \
  } while (0)
#define PA_TL_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define PA_TL(slot, v) \
  do {                 \
  } while (0)
#define PA_TL_NOW() 0ull
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMfmaTau = 8;          // lazy-rescale threshold, log2 units
// Cache policy of the K/V copies: non-temporal ("nt"), since each byte is
// read once per step.
#ifndef PA_KV_NT
#define PA_KV_NT 1
#endif
constexpr int kNonTemporal = PA_KV_NT ? 2 : 0;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }
constexpr int kPlanMaxBatch = kPlanBatch;

template <Dt DT>
struct Mfma;

template <>
struct Mfma<Dt::BF16> {
  __device__ __forceinline__ static f32x4_t qk(u32x4 a, u32x4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t pv(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
  }
  // Round p to bf16 (nearest even); returns the bits, and the rounded value.
  __device__ __forceinline__ static uint32_t round(float p, float& r) {
    const __bf16 h = (__bf16)p;  // round to nearest even
    const uint32_t bits = (uint32_t)__builtin_bit_cast(uint16_t, h);
    r = as_f(bits << 16);
    return bits;
  }
};

template <>
struct Mfma<Dt::F16> {
  __device__ __forceinline__ static f32x4_t qk(u32x4 a, u32x4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t pv(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t round(float p, float& r) {
    const _Float16 h = (_Float16)p;
    r = (float)h;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
  }
};

// LDS reads issued from inline assembly: the compiler would otherwise wait
// for every outstanding HBM->LDS copy (vmcnt(0)) before any LDS read in a
// loop, including copies into the other buffer.  The kernel orders the
// copies with explicit vmcnt waits instead; lds_wait() then waits for these
// reads and ties their results to the wait, so no use is scheduled earlier.
//
// Why this is safe although the compiler takes an asm output as written the
// moment the asm statement issues (the hardware writes it only when the LDS
// read returns): every call site issues a group of these reads and then, in
// the same basic block with nothing in between, the lds_wait() that names
// every one of their destinations as a read-write operand.  So (1) each
// destination stays live, and is not handed to another value, until the
// wait; (2) no instruction reads a destination before the wait, since its
// only use before then is the wait itself; (3) the volatile statements keep
// their order.  A read whose destination is not passed to the wait that
// follows it, or any code placed between the reads and the wait, breaks this.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&k)[N]) {
  if constexpr (N == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k[0]), "+v"(k[1])::"memory");
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3])::"memory");
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x2_t (&v)[N]) {
  if constexpr (N == 4)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])::"memory");
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                   "+v"(v[6]), "+v"(v[7])::"memory");
}
template <int KQ, int ND, int TILE, int SLOT, int I>
struct ReadTile {
  __device__ __forceinline__ static void k(const uint32_t (&ka)[KQ], u32x4 (&kop)[KQ]) {
    kop[I] = lds_read_b128<2 * SLOT * TILE>(ka[I]);
    if constexpr (I + 1 < KQ) ReadTile<KQ, ND, TILE, SLOT, I + 1>::k(ka, kop);
  }
  __device__ __forceinline__ static void v(uint32_t va, u32x2_t (&vop)[ND]) {
    vop[I] = lds_read_tr16<(2 * SLOT + 1) * TILE + 32 * I>(va);
    if constexpr (I + 1 < ND) ReadTile<KQ, ND, TILE, SLOT, I + 1>::v(va, vop);
  }
};

// Work-group barrier after this wave's LDS accesses completed; unlike
// __syncthreads it does not wait for vector-memory operations in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ int shfl_xor_i(int x, int m) {
  return __builtin_amdgcn_ds_bpermute((__lane_id() ^ m) << 2, x);
}
__device__ __forceinline__ float shfl_from(float x, int src_lane) {
  return as_f(__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)as_u(x)));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute((lane - d) << 2, x);
    if (lane >= d) x += y;
  }
  return x;
}

// Largest i in [0, n) with pre[i] <= r, for a non-decreasing pre with
// pre[0] <= r < pre[n].  pre lives in LDS; every lane computes the same i.
__device__ __forceinline__ int plan_search(const int* pre, int n, int r) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= r)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Launch modes, each its own instantiation so that a launch carries no code
// of the others (the split and shared-prefix paths in the plain kernel cost
// 52 more spilled scalar registers and ~2 us on a 35 us launch).
enum AttnMode : int {
  kModePlain = 0,   // single pass, or partitions (with or without the plan)
  kModePrefix = 1,  // partitions with shared-prefix items
  kModeSplit = 2,   // pa_decode_split: pieces of equal runs of tiles
};

template <Dt DT, int D, int MODE>
#ifndef PA_MFMA_MIN_BLOCKS
#define PA_MFMA_MIN_BLOCKS 2  // work groups per CU the register budget must allow
#endif
__global__ __launch_bounds__(kAttnThreads, PA_MFMA_MIN_BLOCKS) void attention_mfma_kernel(AttnArgs a) {
  constexpr int RB = D * 2;                // bytes per (position, head) row
  constexpr int NW = kAttnThreads / kWave;
  constexpr int KQ = D / 32;               // QK MFMAs per tile
  constexpr int ND = D / 16;               // PV MFMAs per tile
  constexpr int TILE = 16 * RB;            // bytes of one 16-position tile
  constexpr int NVI = TILE / 1024;         // 1 KiB copies per V tile
  constexpr int CPR = RB / 16;             // 16-byte chunks per row
  static_assert(NW * 16 * D * 4 <= NW * 4 * TILE, "merge buffer must fit the rings");

  // Per wave, two slots (double buffer) of a K tile and a V tile; after the
  // tiles of an item the same bytes hold the per-wave partial outputs.
  __shared__ __attribute__((aligned(16))) char s_ring[NW * 4 * TILE];
  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];
  __shared__ int s_bad[NW];
  // Shared-prefix launches: bit b set if sequence b's context length is
  // invalid (negative or longer than its table, or its new token would be
  // written into the shared positions); its columns of a shared item are
  // written as NaN.
  __shared__ uint32_t s_inval[kPlanBatch / 32];
  // Partitioned plan: exclusive prefix of the full partitions per sequence
  // (and the total), then the sequences in the order their final partitions
  // are dealt.  While it is built, the rings hold each sequence's sort key
  // and rank.
  __shared__ int s_plan[2 * (kPlanMaxBatch + 1)];
  int* s_key = reinterpret_cast<int*>(s_ring);
  int* s_rank = s_key + kPlanMaxBatch;
  static_assert(2 * kPlanMaxBatch * 4 <= NW * 4 * TILE, "plan keys must fit the rings");

  PA_TL(0, PA_TL_NOW());
#ifdef PA_TIMELINE
  {
    // hardware register ids 20 (XCC_ID) and 4 (HW_ID), 16 and 32 bits
    const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11));
    const unsigned hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
    PA_TL(60, ((unsigned long long)xcc << 32) | hw);
  }
#endif
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int bs = 1 << a.block_shift;
  const int G = a.gqa_group;
  const int Hq = a.n_kv_heads * G;
  const int NQ = a.n_queries;  // query tokens per sequence, the last NQ positions
  // Columns of a KV head's work: pairs (query token j, head g of the group),
  // column c = j * G + g, in chunks of 16.  Column c of sequence b reads and
  // writes row (b * NQ + j) * Hq + kvh * G + g of q / out / the workspace,
  // and sees positions t < ctx - NQ + j + 1 (causal among the NQ tokens).
  const int K = a.n_kv_heads * a.n_hchunks;
  // Split launches (pa_decode_split): the workspace holds pieces of equal
  // runs of tiles instead of fixed partitions (see the plan below).
  constexpr bool split = MODE == kModeSplit;
  const bool parts = a.partition_size > 0 || split;
  const bool plan = parts && a.persistent;
  const int P = a.partition_size;
  const int64_t max_ctx = (int64_t)a.max_blocks << a.block_shift;

  static_assert(kPlanMaxBatch == 4 * kAttnThreads && kPlanMaxBatch % 16 == 0,
                "the plan gives each thread 4 sequences");
  // ---- item list
  int n_items, n_full = 0;
  // Shared-prefix items: partitions p < npp of every sequence, prefix_seqs
  // sequences (a group) per item, p-major, so the work groups of a column
  // read the same prefix tiles at about the same time; in the plan they
  // alternate with the full private partitions.
  int npp = 0, n_pre = 0, n_groups = 0;
  // Split plan: the tiles of a column are every sequence's 16-position
  // tiles in sequence order (s_plan[b] = tiles before sequence b, s_plan[B]
  // = all of them); work group jw of the column takes the run
  // [jw * R, (jw + 1) * R) and writes one workspace slot per sequence the run
  // touches: slot jw - s_plan[b] / R of sequence b.  R is the even share,
  // raised where needed so that no sequence is cut into more than
  // max_partitions pieces.  b_cur: the next sequence this work group visits.
  int64_t sp_lo = 0, sp_hi = 0;
  int sp_R = 1, b_cur = 0;
  if (plan && split) {
    const int B = a.batch;
    int tl[4], ts = 0, tm = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = threadIdx.x * 4 + j;
      const int c = b < B ? a.context_lens[b] : 0;
      // an invalid length gets one tile: its piece is written as NaN
      tl[j] = b >= B ? 0 : (c >= 1 && (int64_t)c <= max_ctx) ? (c + 15) >> 4 : (c == 0 ? 0 : 1);
      ts += tl[j];
      tm = max(tm, tl[j]);
    }
    const int fi = wave_incl_scan(ts);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) tm = max(tm, shfl_xor_i(tm, d));
    if (lane == kWave - 1) {
      s_m[wave][0] = __builtin_bit_cast(float, fi);
      s_l[wave][0] = __builtin_bit_cast(float, tm);
    }
    __syncthreads();
    int fo = 0, ftot = 0, tmax = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int fw = __builtin_bit_cast(int, s_m[w][0]);
      if (w < wave) fo += fw;
      ftot += fw;
      tmax = max(tmax, __builtin_bit_cast(int, s_l[w][0]));
    }
    int fx = fo + fi - ts;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = threadIdx.x * 4 + j;
      if (b < B) s_plan[b] = fx;
      fx += tl[j];
    }
    if (threadIdx.x == 0) s_plan[B] = ftot;
    __syncthreads();
    const int Wc = (int)gridDim.x / K, jwc = (int)blockIdx.x / K;
    const int PM = a.max_partitions;   // >= 2 (checked on the host)
    sp_R = __builtin_amdgcn_readfirstlane(
        max(max((ftot + Wc - 1) / Wc, (tmax + PM - 2) / (PM - 1)), 1));
    sp_lo = (int64_t)jwc * sp_R;
    sp_hi = min(sp_lo + sp_R, (int64_t)ftot);
    b_cur = sp_lo < sp_hi ? plan_search(s_plan, B, (int)sp_lo) : B;
    b_cur = __builtin_amdgcn_readfirstlane(b_cur);
    n_items = 0;   // unused: the run decides
  } else if (plan) {
    // Thread t owns sequences 4t..4t+3.  full(b) = partitions before b's
    // last one (and past the shared prefix), tail(b) = 1 if b has any; the
    // exclusive prefix sum of full(b), and the rank of b's final partition
    // among all final partitions by decreasing length (ties by sequence).
    const int B = a.batch;
    int fl[4], tl[4], key[4], cs[4], fs = 0, ts = 0;
    static_assert((int64_t)((1 << 20) - 1) * kPlanMaxBatch + kPlanMaxBatch < INT32_MAX, "plan keys fit 31 bits");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = threadIdx.x * 4 + j;
      cs[j] = b < B ? a.context_lens[b] : 0;
    }
    if (MODE == kModePrefix && a.prefix_parts > 0) {
      if (threadIdx.x < kPlanBatch / 32) s_inval[threadIdx.x] = 0u;
      // Only partitions before every valid sequence's final one are shared
      // items, so each sequence's final partition (the one holding the new
      // token) stays its own item and no shared item needs a mask.
      int cmin = INT32_MAX;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (cs[j] >= 1 && (int64_t)cs[j] <= max_ctx && cs[j] - 1 >= a.shared_len)
          cmin = min(cmin, cs[j]);
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) cmin = min(cmin, shfl_xor_i(cmin, d));
      if (lane == 0) s_bad[wave] = cmin;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NW; ++w) cmin = min(cmin, s_bad[w]);
      // uniform: keep the item decode below scalar
      npp = __builtin_amdgcn_readfirstlane(
          cmin == INT32_MAX ? 0 : min(min(a.prefix_parts, a.max_partitions), (cmin - 1) / P));
      n_groups = (B + a.prefix_seqs - 1) / a.prefix_seqs;
      n_pre = npp * n_groups;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = threadIdx.x * 4 + j;
        if (b < B && (cs[j] < 0 || (int64_t)cs[j] > max_ctx ||
                      (cs[j] >= 1 && cs[j] - 1 < a.shared_len)))
          atomicOr(&s_inval[b >> 5], 1u << (b & 31));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = threadIdx.x * 4 + j;
      int np = 0;
      const int c = cs[j];
      if (b < B) {
        // more than max_partitions is an error reported by pa_reduce; the
        // cap keeps the item count in range
        np = c > 0 ? (int)min(((int64_t)c + P - 1) / P, (int64_t)a.max_partitions + 1) : 0;
      }
      fl[j] = np > npp ? np - 1 - npp : 0;
      tl[j] = np > npp ? 1 : 0;
      // final-partition length (capped at 2^20 - 1), ties broken by sequence:
      // distinct keys, larger first; no final partition or padding: below all
      const int64_t len = np > npp ? min((int64_t)c - (int64_t)(np - 1) * P, (int64_t)(1 << 20) - 1) : -1;
      key[j] = len >= 0 ? (int)(len * kPlanMaxBatch + (kPlanMaxBatch - 1 - b)) : -1 - (b >= B);
      s_key[b] = key[j];
      s_rank[b] = 0;
      fs += fl[j];
      ts += tl[j];
    }
    PA_TL(58, PA_TL_NOW());   // thread 0 has its context lengths
    const int fi = wave_incl_scan(fs), ti = wave_incl_scan(ts);
    if (lane == kWave - 1) {
      s_m[wave][0] = __builtin_bit_cast(float, fi);
      s_l[wave][0] = __builtin_bit_cast(float, ti);
    }
    __syncthreads();
    PA_TL(59, PA_TL_NOW());   // after the scans' barrier
    int fo = 0, ftot = 0, ttot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int fw = __builtin_bit_cast(int, s_m[w][0]), tw = __builtin_bit_cast(int, s_l[w][0]);
      if (w < wave) fo += fw;
      ftot += fw;
      ttot += tw;
    }
    // rank(b) = number of keys above b's.  A group of tps consecutive
    // threads counts for 4 consecutive sequences (their keys in registers),
    // each thread over every tps-th block of 4 keys, so each key read serves
    // 16 comparisons; the group sums its counts with lane exchanges.  tps =
    // 1024 / B (B rounded up to a power of two, at least 16) gives one pass
    // over all sequences.  The threads of a wave read at most tps key
    // addresses at once (LDS broadcast).  Integer counts: the result does
    // not depend on the order.  (Summing (sequence, 16 keys) units with LDS
    // atomics took ~9 us at B = 256; one thread per sequence, ~3.8 us.)
    {
      const int4* keys4 = reinterpret_cast<const int4*>(s_key);
      const int nk4 = (B + 3) >> 2;   // keys past B are padding, below all
      int bp = 16;
      while (bp < B) bp <<= 1;
      const int tps = min(kWave, kPlanMaxBatch / bp);
      const int part = threadIdx.x & (tps - 1);
      for (int grp = threadIdx.x / tps; 4 * grp < B; grp += kAttnThreads / tps) {
        const int4 kb = keys4[grp];
        int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll 4
        for (int g = part; g < nk4; g += tps) {
          const int4 k4 = keys4[g];
          c0 += (k4.x > kb.x) + (k4.y > kb.x) + (k4.z > kb.x) + (k4.w > kb.x);
          c1 += (k4.x > kb.y) + (k4.y > kb.y) + (k4.z > kb.y) + (k4.w > kb.y);
          c2 += (k4.x > kb.z) + (k4.y > kb.z) + (k4.z > kb.z) + (k4.w > kb.z);
          c3 += (k4.x > kb.w) + (k4.y > kb.w) + (k4.z > kb.w) + (k4.w > kb.w);
        }
        // the group's lanes are all in this iteration (same grp)
        for (int d = 1; d < tps; d <<= 1) {
          c0 += shfl_xor_i(c0, d);
          c1 += shfl_xor_i(c1, d);
          c2 += shfl_xor_i(c2, d);
          c3 += shfl_xor_i(c3, d);
        }
        if (part == 0) {
          const int b0 = 4 * grp;
          s_rank[b0] = c0;   // b0 < B
          if (b0 + 1 < B) s_rank[b0 + 1] = c1;
          if (b0 + 2 < B) s_rank[b0 + 2] = c2;
          if (b0 + 3 < B) s_rank[b0 + 3] = c3;
        }
      }
    }
    __syncthreads();
    PA_TL(61, PA_TL_NOW());   // after the rank's barrier
    int fx = fo + fi - fs;  // exclusive offset of b = 4t
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = threadIdx.x * 4 + j;
      if (b < B) {
        s_plan[b] = fx;
        if (tl[j]) s_plan[kPlanMaxBatch + 1 + s_rank[b]] = b;
      }
      fx += fl[j];
    }
    if (threadIdx.x == 0) s_plan[B] = ftot;
    __syncthreads();
    n_full = ftot;
    n_items = n_pre + ftot + ttot;  // per column
  } else if (parts && !split) {
    n_items = K * a.batch * a.max_partitions;
  } else {
    n_items = K * a.batch;   // single pass, or a split launch without the plan
  }

  PA_TL(1, PA_TL_NOW());
  int tl_k = 0;   // items completed (timeline build)
  (void)tl_k;
  const float sl2 = a.scale_log2;
  const float qnan = __builtin_nanf("");
  float* s_o = reinterpret_cast<float*>(s_ring);  // [NW][16][D] after the tiles

  // Persistent launches: the grid is W work groups per column (a KV head and
  // head chunk), and work group j of a column takes its column's items
  // j, 2W-1-j, 2W+j, 4W-1-j, ... of the plan (full partitions, then final
  // partitions longest first): dealt back and forth, so the work groups of
  // a column end with nearly equal loads.  With cu_deal the grid is two
  // work groups per CU, and work groups j and j + W/2 of a column share one
  // (blocks b and b + gridDim.x/2 are dispatched to the same CU): the items
  // are dealt back and forth over the W/2 CUs instead, the CU's rounds
  // alternating between its two work groups.  The two work groups of a CU
  // share its memory pipeline, so the CU's total sets its end: on the
  // LLaMA-3-8B batch dealing over work groups left the CUs' totals 373-447
  // tiles apart, dealing over CUs 406-436, and the launch went from 145.6
  // to 143.9 us.  Other launches take every gridDim.x-th (item, column)
  // pair.
  const int W = plan ? (int)gridDim.x / K : 0;
  // This work group's column and its index jw among the column's W work
  // groups.  Blocks are dispatched to the eight XCDs round-robin (block b
  // to XCD b % 8), so column = b % K keeps each column on one XCD.  With
  // xcd_spread, block b = h * R + r (R = gridDim.x / 2, h the CU half)
  // takes column (r / 8) % K and jw = h * R/K + (r / 8K) * 8 + r % 8: each
  // column's work groups sit on all eight XCDs, and blocks b and b + R keep
  // one column and slots jw and jw + W/2, as the CU deal needs.  On the
  // LLaMA-3-8B batch every XCD then reads every KV head's tiles, and the
  // launch went from 142.4-142.7 to 140.8-141.0 us (three alternating runs
  // on one box; the odd XCDs stay the slower, by less).
  int col_wg = plan ? (int)blockIdx.x % K : 0;
  int jw = plan ? (int)blockIdx.x / K : 0;
  if (plan && a.xcd_spread) {
    const int R = (int)gridDim.x >> 1, r = (int)blockIdx.x % R, h = (int)blockIdx.x / R;
    col_wg = (r >> 3) % K;
    jw = h * (R / K) + (r / (8 * K)) * 8 + (r & 7);
  }
  for (int it = 0;; ++it) {
    // ---- decode the item
    int kh, rr;
    // split launches: the piece's tile range [u0, u1) within the sequence,
    // whether it is the sequence's last piece, and the sequence's piece count
    int u0 = 0, u1 = 0, n_pieces = 1;
    bool last_piece = true;
    if (split && plan) {
      kh = blockIdx.x % K;
      rr = 0;
      if (b_cur >= a.batch) break;
      const int Sb = s_plan[b_cur];
      if ((int64_t)Sb >= sp_hi) break;
      const int Tb = s_plan[b_cur + 1] - Sb;
      u0 = (int)max(sp_lo - Sb, (int64_t)0);
      u1 = (int)min(sp_hi - Sb, (int64_t)Tb);
      last_piece = (int64_t)Sb + Tb <= sp_hi;
      n_pieces = (Sb + Tb - 1) / sp_R - Sb / sp_R + 1;
    } else if (plan) {
      kh = col_wg;
      if (a.cu_deal) {
        // round t of CU cu: position cu (t even) or C-1-cu (t odd).  The
        // CU's first work group takes its even rounds and the second its odd
        // ones; or (cu_deal 2) the first takes rounds 0, 1, 4, 5, ... and the
        // second 2, 3, 6, 7, ...: with shared items the list alternates
        // shared and private items, and alternating single rounds would give
        // one work group of a CU only shared items and the other only
        // private ones (shared-prefix batch, P 512: 612.0/612.3 us that way,
        // 606.7/608.6 with the work-group deal, 604.3/605.2 with pairs of
        // rounds)
        const int C = W >> 1, cu = jw % C, h = jw / C;
        const int t = a.cu_deal == 2 ? 4 * (it >> 1) + 2 * h + (it & 1) : 2 * it + h;
        rr = t * C + ((t & 1) ? C - 1 - cu : cu);
      } else {
        rr = it * W + ((it & 1) ? W - 1 - jw : jw);
      }
      if (rr >= n_items) break;
    } else {
      const int item = blockIdx.x + it * gridDim.x;
      if (item >= n_items) break;
      kh = item % K;
      rr = item / K;
    }
    if (tl_k < kTimelineItems) PA_TL(4 + 3 * tl_k, PA_TL_NOW());
    const int kvh = kh / a.n_hchunks;
    const int hc = kh - kvh * a.n_hchunks;
    // pre: a shared-prefix item; b is then the group of sequences
    // b * prefix_seqs .. + prefix_seqs - 1 (columns (sequence, head) pairs)
    int b, p = 0;
    bool pre = false;
    int rp = 0, r2 = rr;   // index among shared items / among the rest
    if (n_pre > 0) {
      // shared items alternate with full partitions, so the L2-bound shared
      // reads overlap the HBM-bound private ones (all shared items first:
      // 609 instead of 590 us on the shared-prefix batch, P 2048)
      const int m2 = min(n_pre, n_full);
      if (rr < 2 * m2) {
        pre = (rr & 1) == 0;
        rp = rr >> 1;
        r2 = rr >> 1;
      } else if (rr < n_pre + n_full) {
        pre = n_pre > n_full;
        rp = rr - m2;
        r2 = rr - m2;
      } else {
        pre = false;
        r2 = rr - n_pre;
      }
    }
    if (split && plan) {
      b = b_cur;
      p = jw - s_plan[b_cur] / sp_R;
      // the next sequence with tiles
      int nb = b_cur + 1;
      while (nb < a.batch && s_plan[nb + 1] == s_plan[nb]) ++nb;
      b_cur = __builtin_amdgcn_readfirstlane(nb);
    } else if (split) {
      b = rr;        // the whole sequence in one piece
      u1 = INT32_MAX;
    } else if (pre) {
      p = rp / n_groups;
      b = rp - p * n_groups;
    } else if (plan) {
      if (r2 < n_full) {
        b = plan_search(s_plan, a.batch, r2);
        p = r2 - s_plan[b] + npp;
      } else {
        b = s_plan[kPlanMaxBatch + 1 + r2 - n_full];
        p = s_plan[b + 1] - s_plan[b] + npp;  // b's full partitions, then its tail
      }
    } else if (parts) {
      const int j = rr / a.batch;
      b = rr - j * a.batch;
    } else {
      b = rr;
    }
    b = __builtin_amdgcn_readfirstlane(b);
    p = __builtin_amdgcn_readfirstlane(p);
    // first sequence of the item (its table row is the one read)
    const int bseq = pre ? b * a.prefix_seqs : b;
    // a scalar read (the table and lengths are not written by this kernel);
    // a shared-prefix item's partition lies before every sequence's end
    const int ctx = pre ? (p + 1) * P
                        : ((const __attribute__((address_space(4))) int32_t*)a.context_lens)[b];
    // an invalid length, or (a folded write into a batch with shared
    // positions) a new token that would land in a shared block
    const bool bad_ctx = ctx < 0 || (int64_t)ctx > max_ctx ||
                         (!pre && ctx >= 1 && ctx - 1 < a.shared_len);
    // columns per head of the group: query tokens, or a prefix item's sequences
    const int nq = pre ? a.prefix_seqs : NQ;
    const int nq_valid = pre ? min(nq, a.batch - bseq) : NQ;
    const int c0 = hc * 16;                      // first column of the chunk
    const int gv = min(16, G * nq_valid - c0);   // columns in the chunk
    // row of column c0 + g (see above; a prefix item's column c is head
    // c % G of sequence bseq + c / G)
    auto row_of = [&](int g) -> int64_t {
      const int c = c0 + g;
      return (int64_t)(b * nq + c / G) * Hq + kvh * G + c % G;
    };
    int t0 = 0, t1 = ctx;
    if (pre) {
      t0 = p * P;
    } else if (split) {
      if (bad_ctx) {
        // every slot of the row NaN (the piece's o too), so pa_reduce
        // gives NaN whatever the slots held before
        for (int idx = threadIdx.x; idx < gv * D; idx += kAttnThreads) {
          const int g = idx / D, d = idx - g * D;
          a.tmp_out[(row_of(g) * a.max_partitions + p) * D + d] = qnan;
        }
        for (int idx = threadIdx.x; idx < gv * a.max_partitions; idx += kAttnThreads) {
          const int g = idx / a.max_partitions, q = idx - g * a.max_partitions;
          a.max_logits[row_of(g) * a.max_partitions + q] = qnan;
          a.exp_sums[row_of(g) * a.max_partitions + q] = qnan;
        }
        continue;
      }
      t0 = u0 * 16;
      t1 = (int)min((int64_t)u1 * 16, (int64_t)ctx);
    } else if (parts) {
      const int64_t np = ctx > 0 ? ((int64_t)ctx + P - 1) / P : 0;
      if (np > a.max_partitions) {
        // The workspace cannot hold this sequence: no attention (pa_reduce
        // reports NaN), but the folded cache write still happens, done by
        // the item that would hold the final partition -- the last row of
        // the grid, or the plan's tail item of the sequence.
        // (The plan caps a sequence at max_partitions + 1 partitions, so its
        // tail item has p == max_partitions.)
        const bool writer = plan ? p == a.max_partitions
                                 : rr / a.batch == a.max_partitions - 1;
        if (a.key_new != nullptr && writer && !bad_ctx && wave == 0 && lane < CPR) {
          const int tn = ctx - 1;
          const int pblk = a.block_table[(int64_t)b * a.max_blocks + (tn >> a.block_shift)];
          if (pblk >= 0 && pblk < a.n_blocks) {
            const int64_t head_bytes = (int64_t)bs * RB;
            const int64_t src = (int64_t)(b * a.n_kv_heads + kvh) * RB + lane * 16;
            const int64_t dst = ((int64_t)pblk * a.n_kv_heads + kvh) * head_bytes +
                                (int64_t)(tn & (bs - 1)) * RB + lane * 16;
            *(u32x4*)((char*)a.k_pool + dst) = *(const u32x4*)((const char*)a.key_new + src);
            *(u32x4*)((char*)a.v_pool + dst) = *(const u32x4*)((const char*)a.value_new + src);
          }
        }
        continue;
      }
      if (!plan) {
        // one work group per (row, sequence): row j holds partition
        // np - PMAX + j, so final partitions are dispatched last
        p = (int)np - a.max_partitions + rr / a.batch;
        if (p < 0) continue;
      }
      if (bad_ctx) {
        for (int idx = threadIdx.x; idx < gv * D; idx += kAttnThreads) {
          const int g = idx / D, d = idx - g * D;
          const int64_t prow = row_of(g) * a.max_partitions + p;
          a.tmp_out[prow * D + d] = qnan;
          if (d == 0) {
            a.max_logits[prow] = qnan;
            a.exp_sums[prow] = qnan;
          }
        }
        continue;
      }
      t0 = p * P;
      t1 = min(t0 + P, ctx);
    } else if (bad_ctx || ctx == 0) {
      const float v = bad_ctx ? qnan : 0.0f;
      for (int idx = threadIdx.x; idx < gv * D; idx += kAttnThreads) {
        const int g = idx / D, d = idx - g * D;
        store_elem<DT>(a.out, row_of(g) * D + d, v);
      }
      continue;
    }

    // ---- queries of the chunk: B operand of S = K Q^T (zero past the group)
    u32x4 qop[KQ];
    {
      const char* qrow = (const char*)a.q + row_of(min(l16, gv - 1)) * RB + lg * 16;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk)
        qop[kk] = l16 < gv ? *(const u32x4*)(qrow + kk * 64) : u32x4{0u, 0u, 0u, 0u};
    }

    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    const int ntile = (t1 - t0 + 15) >> 4;
    // Shared items: the pairs (sequence bseq + sq, block j of the item), sq
    // >= 1, numbered idx = (sq - 1) * nbi + j; thread t loads the first
    // sequence's and sequence sq's entries of pairs t and t + 256 here, after
    // the queries and before the first tile's copies, so the wait for that
    // tile (loads complete in issue order) covers them and nothing in the
    // tile loop waits for them; they are compared after the loop.  Pairs
    // past 512 (only with more than 512 / nbi sequences per item) are
    // compared there too, loaded then.
    int mis_e0[2] = {0, 0}, mis_e1[2] = {0, 0};
    int nbi = 0, n_pairs = 0;
    const int32_t* mis_row = a.block_table + (int64_t)bseq * a.max_blocks + (t0 >> a.block_shift);
    if (pre) {
      nbi = (t1 - t0 + bs - 1) >> a.block_shift;
      n_pairs = (nq_valid - 1) * nbi;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int idx = threadIdx.x + k * kAttnThreads;
        if (idx < n_pairs) {
          const int sq = 1 + idx / nbi, j = idx - (sq - 1) * nbi;
          mis_e0[k] = mis_row[j];
          mis_e1[k] = mis_row[(int64_t)sq * a.max_blocks + j];
        }
      }
    }
    // The folded cache write (decode only): the work item holding position
    // ctx - 1 -- the sequence's final partition -- stores the new row of its
    // KV head in the pool, and the wave that owns that position's tile
    // patches it into the tile in LDS after the tile's copy lands (the copy
    // may predate the store), so the attention reads the new row either way.
    const bool append = a.key_new != nullptr && t1 == ctx && ctx > 0 && !pre;
    const int tn = ctx - 1;
    const int ti_new = (tn - t0) >> 4;                     // its tile in the item
    const int wave_new = ti_new % NW, i_new = ti_new / NW, r_new = (tn - t0) & 15;
    u32x4 knew = u32x4{0u, 0u, 0u, 0u}, vnew = u32x4{0u, 0u, 0u, 0u};
    if (append && wave == wave_new && lane < CPR) {
      const int64_t src = (int64_t)(b * a.n_kv_heads + kvh) * RB + lane * 16;
      knew = *(const u32x4*)((const char*)a.key_new + src);
      vnew = *(const u32x4*)((const char*)a.value_new + src);
    }
    const int lim_min = ctx - NQ + 1;                      // of the first query token
    const int lim_lane = lim_min + (c0 + l16) / G;         // of this lane's column
    const int my_n = __builtin_amdgcn_readfirstlane(ntile > wave ? (ntile - 1 - wave) / NW + 1 : 0);
    const int64_t head_bytes = (int64_t)bs * RB;        // one (block, KV head) tile
    const int64_t blk_bytes = head_bytes * a.n_kv_heads;
    const char* kbase = (const char*)a.k_pool + kvh * head_bytes;
    const char* vbase = (const char*)a.v_pool + kvh * head_bytes;
    const __attribute__((address_space(4))) int32_t* trow =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table +
                                                           (int64_t)bseq * a.max_blocks);
    char* my_ring = s_ring + wave * 4 * TILE;  // slot x: K at 2x*TILE, V at (2x+1)*TILE
    bool bad = false;
    // A shared item reads the first sequence's table for the whole group:
    // bit s is set when sequence bseq + s names other blocks for the item's
    // positions (the rows do not share the prefix as stated), and that
    // sequence's columns are written as NaN.  The entries are loaded at the
    // item's start (see mis_load) and compared after its tiles.
    uint32_t mis = 0u;

    // Byte offsets (in a KV head's view of a pool) of a tile's rows 0-7 and
    // rows 8-15 (row r lives at base + r * RB).  With blocks of 16 or more
    // positions a tile lies in one block and the two are equal; 8-position
    // blocks give two blocks.
    struct TileBase {
      int64_t lo, hi;
    };
    auto tile_base = [&](int i) -> TileBase {
      const int tok = __builtin_amdgcn_readfirstlane(t0 + (wave + i * NW) * 16);
      // rows 8-15 past the end (tok + 8 >= t1) alias rows 0-7: in bounds,
      // and masked out of the result
      const int tok_hi = tok + 8 < t1 ? tok + 8 : tok;
      const int bl0 = tok >> a.block_shift;
      const int bl1 = tok_hi >> a.block_shift;
      const int p0 = trow[bl0];
      const int p1 = trow[bl1];
      const bool ok0 = p0 >= 0 && p0 < a.n_blocks;
      const bool ok1 = p1 >= 0 && p1 < a.n_blocks;
      bad |= !(ok0 && ok1);
      TileBase t;
      t.lo = (ok0 ? (int64_t)p0 : 0) * blk_bytes + (int64_t)(tok & (bs - 1)) * RB;
      t.hi = (ok1 ? (int64_t)p1 : 0) * blk_bytes + (int64_t)(tok_hi & (bs - 1)) * RB - 8 * RB;
      return t;
    };
    // Copies HBM -> LDS, 1 KiB per instruction (16 bytes per lane).  The
    // V tile is stored row-major (read back transposed); the K tile stores
    // chunk c of row r at chunk c ^ (r % CPR) of that row, so the 16 lanes
    // that read one column of 16 rows hit 16 different banks.
    auto issue = [&](int i, int slot) {
      const TileBase t = tile_base(i);
      char* kd = my_ring + (2 * slot) * TILE;
      char* vd = kd + TILE;
#pragma unroll
      for (int v = 0; v < NVI; ++v) {
        const int sidx = v * 64 + lane;   // 16-byte slot in the tile
        const int row = sidx / CPR;
        const int64_t base = row >= 8 ? t.hi : t.lo;
        const int kc = (sidx % CPR) ^ (row % CPR);
        // A shared item's tiles are read again by the other groups of
        // sequences: ordinary loads keep them in L2 (non-temporal: 590
        // instead of 580 us on the shared-prefix batch at P 2048).
        if (pre) {
          __builtin_amdgcn_global_load_lds(kbase + base + row * RB + kc * 16,
                                           (__attribute__((address_space(3))) void*)(kd + v * 1024),
                                           16, 0, 0);
          __builtin_amdgcn_global_load_lds(vbase + base + sidx * 16,
                                           (__attribute__((address_space(3))) void*)(vd + v * 1024),
                                           16, 0, 0);
        } else {
          __builtin_amdgcn_global_load_lds(kbase + base + row * RB + kc * 16,
                                           (__attribute__((address_space(3))) void*)(kd + v * 1024),
                                           16, 0, kNonTemporal);
          __builtin_amdgcn_global_load_lds(vbase + base + sidx * 16,
                                           (__attribute__((address_space(3))) void*)(vd + v * 1024),
                                           16, 0, kNonTemporal);
        }
      }
    };

    f32x4_t O[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n) O[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // running max (log2 units) of column l16; a finite floor, so a column
    // with no visible position yet gives exp2(-inf - m) = 0, not NaN
    float m = -1e30f;
    float lsum = 0.0f;                 // this lane's share of the normaliser
    // LDS byte addresses of this lane's reads in slot 0 (slot 1 adds an
    // immediate offset): K as the A operand (row l16, chunk 4kk + lg of the
    // swizzled row), V transposed (rows 4lg..4lg+3, dims 4(l16%4).. of each
    // 16-dim column block).
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)my_ring;
    uint32_t k_addr[KQ];
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      k_addr[kk] = ring_lds + l16 * RB + (((kk * 4 + lg) ^ (l16 % CPR)) * 16);
    const uint32_t v_addr = ring_lds + (lg * 4 + (l16 >> 2)) * RB + (l16 & 3) * 8;

    // After tile i's copy has landed: the folded cache write (see above).
    auto patch_new_row = [&](int i, int slot) {
      if (!append || wave != wave_new || i != i_new) return;
      const int pblk = trow[tn >> a.block_shift];
      if (lane < CPR) {
        char* kd = my_ring + (2 * slot) * TILE;
        *(u32x4*)(kd + r_new * RB + ((lane ^ (r_new % CPR)) * 16)) = knew;
        *(u32x4*)(kd + TILE + r_new * RB + lane * 16) = vnew;
        if (pblk >= 0 && pblk < a.n_blocks) {
          const int64_t dst = (int64_t)pblk * blk_bytes + (int64_t)(tn & (bs - 1)) * RB + lane * 16;
          *(u32x4*)((char*)kbase + dst) = knew;
          *(u32x4*)((char*)vbase + dst) = vnew;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the LDS stores are done
      asm volatile("" ::: "memory");       // and ordered before the tile's reads
    };

    auto compute = [&](int i, auto slot_tag) {
      constexpr int SLOT = decltype(slot_tag)::value;
      const int tok = __builtin_amdgcn_readfirstlane(t0 + (wave + i * NW) * 16);
      const int nvalid = min(16, t1 - tok);
      u32x4 kop[KQ];
      ReadTile<KQ, ND, TILE, SLOT, 0>::k(k_addr, kop);
      lds_wait(kop);
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) s = Mfma<DT>::qk(kop[kk], qop[kk], s);
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = s[j] * sl2;
      if (nvalid < 16 || tok + 16 > lim_min) {
        // past the item's end, or past this column's causal limit
        const int nv = min(nvalid, lim_lane - tok);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (lg * 4 + j < nv) ? x[j] : -__builtin_huge_valf();
      }
      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = fmaxf(bm, shfl_xor_f(bm, 16));
      bm = fmaxf(bm, shfl_xor_f(bm, 32));
      if (__ballot(bm > m + (float)kMfmaTau)) {
        const float mn = fmaxf(m, bm);
        const float al = (m == mn) ? 1.0f : exp2_fast(m - mn);
        lsum *= al;
        m = mn;
        // O rows are heads 4*lg + j: fetch their factors from lanes 4*lg + j.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = shfl_from(al, lg * 4 + j);
#pragma unroll
          for (int n = 0; n < ND; ++n) O[n][j] *= aj;
        }
      }
      uint32_t pb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float r;
        pb[j] = Mfma<DT>::round(exp2_fast(x[j] - m), r);
        lsum += r;
      }
      const u32x2_t pa = u32x2_t{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
      u32x2_t vop[ND];
      ReadTile<KQ, ND, TILE, SLOT, 0>::v(v_addr, vop);
      lds_wait(vop);
      uint32_t vm0 = 0xFFFFFFFFu, vm1 = 0xFFFFFFFFu;
      if (nvalid < 16) {
        // zero V of positions past the end (they may hold NaN)
        const int r0 = lg * 4;
        vm0 = (r0 + 0 < nvalid ? 0x0000FFFFu : 0u) | (r0 + 1 < nvalid ? 0xFFFF0000u : 0u);
        vm1 = (r0 + 2 < nvalid ? 0x0000FFFFu : 0u) | (r0 + 3 < nvalid ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        u32x2_t vb = vop[n];
        vb[0] &= vm0;
        vb[1] &= vm1;
        O[n] = Mfma<DT>::pv(pa, vb, O[n]);
      }
    };

    if (my_n > 0) {
      // Tile i + 1 is copied while tile i is computed.  Loads (and these
      // copies) complete in issue order, so "at most 2 * NVI outstanding"
      // right after tile i + 1's copies are issued means tile i, and
      // anything issued before it, has landed.  The slots are compile-time offsets, which lets
      // the compiler see that reading one slot does not wait for copies
      // into the other.
      issue(0, 0);
      for (int i = 0; i < my_n; i += 2) {
        if (i + 1 < my_n) {
          issue(i + 1, 1);
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NVI));
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        patch_new_row(i, 0);
        compute(i, std::integral_constant<int, 0>{});
        if (i + 1 >= my_n) break;
        if (i + 2 < my_n) {
          issue(i + 2, 0);
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NVI));
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        patch_new_row(i + 1, 1);
        compute(i + 1, std::integral_constant<int, 1>{});
      }
    }

    if (pre) {
      uint32_t lm = 0u;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int idx = threadIdx.x + k * kAttnThreads;
        if (idx < n_pairs && mis_e0[k] != mis_e1[k]) lm |= 1u << (1 + idx / nbi);
      }
      for (int idx = threadIdx.x + 2 * kAttnThreads; idx < n_pairs; idx += kAttnThreads) {
        const int sq = 1 + idx / nbi, j = idx - (sq - 1) * nbi;
        if (mis_row[j] != mis_row[(int64_t)sq * a.max_blocks + j]) lm |= 1u << sq;
      }
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) lm |= (uint32_t)shfl_xor_i((int)lm, d);
      mis = __builtin_amdgcn_readfirstlane(lm);
    }

    // ---- merge the waves
    float lh = lsum + shfl_xor_f(lsum, 16);
    lh += shfl_xor_f(lh, 32);
    // The merge's barriers wait for LDS work only: __syncthreads would also
    // wait for every vector-memory operation in flight, the previous item's
    // output stores included.
    lds_barrier();  // every wave is done with its ring
    if (lane < 16) {
      s_m[wave][lane] = m;
      s_l[wave][lane] = lh;
    }
    if (lane == 0) s_bad[wave] = (int)(mis | (bad ? 1u : 0u));  // mis never has bit 0
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = lg * 4 + j;
      if (h < gv) {
#pragma unroll
        for (int n = 0; n < ND; ++n) s_o[(wave * 16 + h) * D + n * 16 + l16] = O[n][j];
      }
    }
    lds_barrier();
    bool anybad = false;
    uint32_t allmis = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      anybad |= (s_bad[w] & 1) != 0;
      allmis |= (uint32_t)s_bad[w] & ~1u;
    }
    // Thread (column g, dims d..d+3) of pass j: 4 outputs per thread, so a
    // 16-column chunk takes NP passes of the work group.  Every LDS read of
    // the merge comes before its first store: the compiler orders reads of
    // the rings after all vector-memory operations in flight (the copies
    // into them), and a read after a store would wait for that store.
    constexpr int D4 = D / 4;
    constexpr int NP = (16 * D4 + kAttnThreads - 1) / kAttnThreads;
    float mw[NP][NW], lw[NP][NW];
    f32x4_t ow[NP][NW];
    bool colbad[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int idx = threadIdx.x + j * kAttnThreads;
      colbad[j] = anybad;
      if (idx < gv * D4) {
        const int g = idx / D4, d = (idx - g * D4) * 4;
        if (pre) {
          const int sq = (c0 + g) / G;
          const int sb = bseq + sq;
          colbad[j] |= ((s_inval[sb >> 5] >> (sb & 31)) & 1u) != 0u;
          colbad[j] |= ((allmis >> sq) & 1u) != 0u;
        }
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          mw[j][w] = s_m[w][g];
          lw[j][w] = s_l[w][g];
          ow[j][w] = *reinterpret_cast<const f32x4_t*>(&s_o[(w * 16 + g) * D + d]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int idx = threadIdx.x + j * kAttnThreads;
      if (idx >= gv * D4) break;
      const int g = idx / D4, d = (idx - g * D4) * 4;
      float M = -__builtin_huge_valf();
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[j][w]);
      float L = 0.0f;
      f32x4_t Ov = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float aw = exp2_fast(mw[j][w] - M);  // waves without positions have l = 0
        L += aw * lw[j][w];
#pragma unroll
        for (int k = 0; k < 4; ++k) Ov[k] += aw * ow[j][w][k];
      }
      // a column with no visible position in the partition: l = 0, o = 0
      f32x4_t r;
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = colbad[j] ? qnan : (L > 0.0f ? Ov[k] / L : 0.0f);
      if (parts) {
        const int64_t prow = row_of(g) * a.max_partitions + p;
        // With shared items the prefix tiles live in L2, and the partial
        // outputs are written at system scope (sc0 sc1): they pass L2 by
        // instead of evicting the prefix, and the reduce that follows finds
        // them in the memory-side cache.  Shared-prefix batch, P 512:
        // non-temporal stores 621 us, sc0 sc1 617 us (and its reduce 15.6
        // -> 13.2 us), where ordinary stores had cost ~5 % more than
        // non-temporal ones; P 2048 unchanged at 556 us.  Without
        // shared items ordinary stores are the fastest (LLaMA-3 batch 146
        // us against 148 us with sc0 sc1).  A vector store; gfx9 counts it
        // in vmcnt, and vector memory operations complete in issue order,
        // so the waits the compiler places for its own loads stay correct.
        if (n_pre > 0) {
          float* sp = &a.tmp_out[prow * D + d];
          asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" : : "v"(sp), "v"(r) : "memory");
        } else {
          *reinterpret_cast<f32x4_t*>(&a.tmp_out[prow * D + d]) = r;
        }
        if (d == 0) {
          a.max_logits[prow] = colbad[j] ? qnan : M * kLn2;
          a.exp_sums[prow] = colbad[j] ? qnan : L;
          if (split && last_piece) {
            // the sequence's unused slots: empty (exp_sums 0, pa_reduce
            // skips them)
            const int64_t r0 = row_of(g) * a.max_partitions;
            for (int q = n_pieces; q < a.max_partitions; ++q) {
              a.max_logits[r0 + q] = -__builtin_huge_valf();
              a.exp_sums[r0 + q] = 0.0f;
            }
          }
        }
      } else {
        const int64_t o = row_of(g) * D + d;
#pragma unroll
        for (int k = 0; k < 4; ++k) store_elem<DT>(a.out, o + k, r[k]);
      }
    }
    lds_barrier();  // the merge buffer is the next item's rings
    if (tl_k < kTimelineItems) {
      PA_TL(5 + 3 * tl_k, PA_TL_NOW());
      PA_TL(6 + 3 * tl_k, (unsigned long long)ntile | ((unsigned long long)pre << 20) |
                              ((unsigned long long)(unsigned)b << 32));
    }
    ++tl_k;
  }
  PA_TL(2, PA_TL_NOW());
  PA_TL(3, tl_k);
}

template <Dt DT, int D>
hipError_t launch_attention_mfma_d(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if (a.split)
    launch_timed(attention_mfma_kernel<DT, D, kModeSplit>, dim3(grid), dim3(kAttnThreads), s, a);
  else if (a.prefix_parts > 0)
    launch_timed(attention_mfma_kernel<DT, D, kModePrefix>, dim3(grid), dim3(kAttnThreads), s, a);
  else
    launch_timed(attention_mfma_kernel<DT, D, kModePlain>, dim3(grid), dim3(kAttnThreads), s, a);
  return hipGetLastError();
}

template <Dt DT>
hipError_t launch_attention_mfma(const AttnArgs& a, int d_head, unsigned grid, hipStream_t s) {
  if (d_head == 64) return launch_attention_mfma_d<DT, 64>(a, grid, s);
  if (d_head == 128) return launch_attention_mfma_d<DT, 128>(a, grid, s);
  return hipErrorInvalidValue;
}

// Work groups per CU, the fewest over the three modes (all are built for two).
template <Dt DT, int D>
int attention_mfma_blocks_per_cu_d() {
  int n = 1 << 30;
  for (int m = 0; m < 3; ++m) {
    int k = 0;
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &k,
        m == 0 ? attention_mfma_kernel<DT, D, kModePlain>
               : m == 1 ? attention_mfma_kernel<DT, D, kModePrefix>
                        : attention_mfma_kernel<DT, D, kModeSplit>,
        kAttnThreads, 0);
    n = std::min(n, k);
  }
  return n > 0 ? n : 1;
}

template <Dt DT>
int attention_mfma_blocks_per_cu(int d_head) {
  return d_head == 64 ? attention_mfma_blocks_per_cu_d<DT, 64>()
                      : attention_mfma_blocks_per_cu_d<DT, 128>();
}

}  // namespace pa
