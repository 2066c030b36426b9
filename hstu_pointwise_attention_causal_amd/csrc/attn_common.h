// Device helpers shared by the bf16 attention kernels (forward and backward):
// direct HBM -> LDS loads through buffer resources, LDS transpose reads, the
// tile barrier, vmcnt waits, and the swizzle of tiles that are read both by
// rows and by transposed columns.
#pragma once

#include "common.h"

namespace hstu {

constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit dwords, no swizzle

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ lds_ptr_t to_lds(void* p) { return (lds_ptr_t)(p); }

// ds_read_b64_tr_b16: in every 16-lane group, lane 4k + m names 4 consecutive
// bf16 of one LDS row and lane i receives element (i % 4) of the addresses of
// lanes 4k + i/4, k = 0..3 -- one column of 4 rows.
__device__ __forceinline__ bf16x4_t tr_read(const char* p) {
  s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(bf16x4_t, r);
}

__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes));
}

// Buffer resource over `bytes` bytes from p (reads past the end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(clamp_records(bytes)),
                                          kRsrcFlags);
}

// One 16-byte-per-lane direct load into LDS: lane l lands at lds + 16 l.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 16, voff, 0, 0, 0);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Workgroup barrier of a tile loop. __syncthreads() would add a release
// fence, i.e. wait for every outstanding memory operation of the wave --
// including the direct loads of tiles that are meant to stay in flight. Here
// the caller waits for exactly the loads it needs (wait_vmcnt), this function
// waits for the wave's own LDS operations (their buffer is refilled after the
// barrier) and the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) (no wait on the other counters) for a wave-uniform n.
__device__ __forceinline__ void wait_vmcnt(int n) {
#define HSTU_VMCNT(c) __builtin_amdgcn_s_waitcnt(((c) & 15) | 0x70 | 0xF00 | (((c) >> 4) << 14))
  switch (n) {
    case 0: HSTU_VMCNT(0); break;
    case 1: HSTU_VMCNT(1); break;
    case 2: HSTU_VMCNT(2); break;
    case 3: HSTU_VMCNT(3); break;
    case 4: HSTU_VMCNT(4); break;
    case 5: HSTU_VMCNT(5); break;
    case 6: HSTU_VMCNT(6); break;
    case 7: HSTU_VMCNT(7); break;
    case 8: HSTU_VMCNT(8); break;
    case 9: HSTU_VMCNT(9); break;
    case 10: HSTU_VMCNT(10); break;
    case 11: HSTU_VMCNT(11); break;
    case 12: HSTU_VMCNT(12); break;
    case 13: HSTU_VMCNT(13); break;
    case 14: HSTU_VMCNT(14); break;
    case 15: HSTU_VMCNT(15); break;
    default: HSTU_VMCNT(0); break;
  }
#undef HSTU_VMCNT
}

// XOR mask of the 16-byte chunk index for row r of a tile with CH chunks per
// row that is read both ways: by rows (ds_read_b128 of an MFMA A operand: 16
// lanes, 16 consecutive rows, one logical chunk) and by transposed columns
// (ds_read_b64_tr_b16: 4 consecutive rows x one aligned group of 4 chunks per
// 16 lanes). With s = the row's index in units of 256 bytes (64 banks), the
// mask permutes the bits of s so that both patterns cover distinct banks.
template <int CH>
__device__ __forceinline__ int swz_dual(int r) {
  static_assert(CH == 4 || CH == 8 || CH == 16, "chunks per row");
  if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (CH == 8) return ((r >> 1) & 1) << 2 | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}

// SiLU in log2 units, shared by the attention kernels: with x' = log2(e) x,
// g(x') = log2(e) SiLU(x) = x' / (1 + 2^-x'). Both forms return 2 g(x') (the
// factor 2 is exact and removed in the output scale): exactly x' / (1/2 +
// 2^-x' / 2) -- an exp2 and a reciprocal, both quarter rate -- or, when |x'|
// is known to stay within kPolyBound, x' + y 2P(y) with y = x'^2 and a quadratic
// P fitted on |x| <= 2 (max error 3.3e-4 in x' units; where |g| > 0.05 the
// relative error is at most 1.1e-3, below the bf16 half-ulp of 2^-9 that P is
// rounded to anyway; coefficients from gen_silu_poly.py): four FMA-class
// operations.
constexpr float kPolyC0 = 1.724344390e-01f, kPolyC1 = -6.268887826e-03f, kPolyC2 = 1.697165370e-04f;
constexpr float kPolyBound = 1.95f * kLog2e;   // in x' units; fit range is 2 log2(e)

__device__ __forceinline__ float silu2_exact(float x) {
  return x * __builtin_amdgcn_rcpf(fmaf(__builtin_amdgcn_exp2f(-x), 0.5f, 0.5f));
}
__device__ __forceinline__ float silu2_poly(float x) {
  const float y = x * x;
  float p = fmaf(y, 2.0f * kPolyC2, 2.0f * kPolyC1);
  p = fmaf(y, p, 2.0f * kPolyC0);
  return fmaf(y, p, x);
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// Largest / smallest value over the wave as a wave-uniform (scalar) value: a
// DPP reduction inside each row of 16 lanes, then the four row results read
// back with v_readlane. fmaxf / fminf drop a NaN operand: a caller that must
// see NaN tests for it separately.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = fmaxf(v, dpp_row<0xB1>(v));    // quad [1,0,3,2]
  v = fmaxf(v, dpp_row<0x4E>(v));    // quad [2,3,0,1]
  v = fmaxf(v, dpp_row<0x141>(v));   // half-row mirror
  v = fmaxf(v, dpp_row<0x140>(v));   // row mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_min_uniform(float v) {
  v = fminf(v, dpp_row<0xB1>(v));
  v = fminf(v, dpp_row<0x4E>(v));
  v = fminf(v, dpp_row<0x141>(v));
  v = fminf(v, dpp_row<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fminf(fminf(r0, r1), fminf(r2, r3));
}

}  // namespace hstu
