// Shared device helpers for the gfx950 kernels: vector types for the bf16
// MFMA operands, bf16 conversion, SiLU, and the relative-bias bucket functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Work item of the attention kernels: one (sequence, head, query tile), with
// the sequence's start and length (clamped offsets; T < 2^27, so they fit in
// 32 bits) and its first query tile in the list's per-sequence numbering, so
// that a workgroup needs a single 16-byte load to begin.
struct WorkItem {
  int32_t seq0;
  int32_t n;
  int32_t packed;  // q_tile | head << 20
  int32_t tile_base;
};
__device__ __forceinline__ int item_qtile(WorkItem w) { return w.packed & 0xFFFFF; }
__device__ __forceinline__ int item_head(WorkItem w) { return w.packed >> 20; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// SiLU(x) = x / (1 + 2^(-x log2 e)). For x below about -88 the power is +inf,
// its reciprocal 0 and the product -0, the correctly rounded limit.
__device__ __forceinline__ float silu_f32(float x) {
  float e = __builtin_amdgcn_exp2f(-x * kLog2e);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Variant for the fp32 path: the device library's expf (not the fast
// __expf) and an IEEE division.
__device__ __forceinline__ float silu_f32_accurate(float x) {
  return x / (1.0f + expf(-x));
}

// Relative position bucket: min(i - j, nb - 1) for i - j >= 0.
__device__ __forceinline__ int pos_bucket(int delta, int nb) { return min(max(delta, 0), nb - 1); }

// Relative time bucket: min(floor(log2(1 + max(dt, 0))), nb - 1), exact in
// integers: floor(log2(x)) of a positive 64-bit x is 63 - (leading zeros).
// Gaps are clamped below 2^62 so that 1 + dt cannot overflow.
__device__ __forceinline__ int time_bucket64(int64_t dt, int nb) {
  dt = dt < 0 ? 0 : (dt > (int64_t(1) << 62) ? (int64_t(1) << 62) : dt);
  int c = 63 - __clzll(static_cast<unsigned long long>(dt + 1));
  return min(c, nb - 1);
}

// The same bucket of the gap t_late - t_early when that gap is known to fit
// in int32: the wrapped difference of the low words is then the gap itself.
// (Any other input still yields a bucket in [0, nb - 1].)
__device__ __forceinline__ int time_bucket_narrow(int64_t t_late, int64_t t_early, int nb) {
  const int gap = static_cast<int>(static_cast<unsigned>(t_late) - static_cast<unsigned>(t_early));
  return min(31 - __builtin_clz(static_cast<unsigned>(max(gap, 0)) + 1u), nb - 1);
}

}  // namespace hstu
