// Device-side helpers shared by the paged-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

template <Dt T>
struct DtInfo;
template <>
struct DtInfo<Dt::F32> {
  static constexpr int bytes = 4;
};
template <>
struct DtInfo<Dt::F16> {
  static constexpr int bytes = 2;
};
template <>
struct DtInfo<Dt::BF16> {
  static constexpr int bytes = 2;
};

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
// Reinterpret a dword as two 16-bit lanes.  Takes the dword by value: with a
// vector-element operand (v[j]) __builtin_bit_cast reads element 0 whatever j
// is (seen with clang 22 for gfx950), so every caller passes a plain scalar.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the 8 consecutive lanes [8k, 8k+8): quad swaps of 1 and 2, then
// the half-row mirror pairs each quad with the other.  Every lane of the
// group ends with the full sum.  Must run with all 8 lanes active.
__device__ __forceinline__ float sum8(float x) {
  x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0xB1, 0xF, 0xF, false));
  x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x4E, 0xF, 0xF, false));
  x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x141, 0xF, 0xF, false));
  return x;
}

// Value held by lane (lane ^ 8): a rotate by 8 inside each 16-lane row.
__device__ __forceinline__ float xor8(float x) {
  return as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
  const int lane = __lane_id();
  return as_f(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)as_u(x)));
}

// <k, q> over one 16-byte chunk, accumulated into acc in fp32.
template <Dt T>
__device__ __forceinline__ float dot_chunk(u32x4 k, u32x4 q, float acc);

template <>
__device__ __forceinline__ float dot_chunk<Dt::BF16>(u32x4 k, u32x4 q, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k[j]), as_bf16x2(q[j]), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot_chunk<Dt::F16>(u32x4 k, u32x4 q, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2(as_f16x2(k[j]), as_f16x2(q[j]), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot_chunk<Dt::F32>(u32x4 k, u32x4 q, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(as_f(k[j]), as_f(q[j]), acc);
  return acc;
}

// Elements of one 16-byte chunk as floats (exact conversions).
template <Dt T>
struct Unpack;

template <>
struct Unpack<Dt::BF16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(u32x4 v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = as_f(v[j] << 16);
      f[2 * j + 1] = as_f(v[j] & 0xFFFF0000u);
    }
  }
};

template <>
struct Unpack<Dt::F16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(u32x4 v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2 h = as_f16x2(v[j]);
      f[2 * j] = (float)h[0];
      f[2 * j + 1] = (float)h[1];
    }
  }
};

template <>
struct Unpack<Dt::F32> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void run(u32x4 v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = as_f(v[j]);
  }
};

// fp32 -> storage element, round to nearest even; NaN stays NaN.
template <Dt T>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x);

template <>
__device__ __forceinline__ void store_elem<Dt::F32>(void* base, int64_t idx, float x) {
  reinterpret_cast<float*>(base)[idx] = x;
}

template <>
__device__ __forceinline__ void store_elem<Dt::F16>(void* base, int64_t idx, float x) {
  reinterpret_cast<_Float16*>(base)[idx] = (_Float16)x;
}

template <>
__device__ __forceinline__ void store_elem<Dt::BF16>(void* base, int64_t idx, float x) {
  uint32_t u = as_u(x);
  uint16_t r;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    r = 0x7FC0;
  } else {
    u += 0x7FFFu + ((u >> 16) & 1u);
    r = (uint16_t)(u >> 16);
  }
  reinterpret_cast<uint16_t*>(base)[idx] = r;
}

}  // namespace pa
