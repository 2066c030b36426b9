// Offsets of a jagged batch as the attention kernels read them.
//
// The caller's seq_offsets live in device memory and the host never reads
// them, so the library cannot reject a malformed array. Instead the first
// kernel of a call writes a clamped copy, and every later kernel of the call
// reads only that copy:
//     c(-1) = 0,   c(b) = min(max(off[b], c(b-1)), T)      b = 0 .. B
// i.e. each offset is clamped into [0, T] and the sequence is made
// non-decreasing. Then every sequence lies inside the T tokens and the
// lengths c(b+1) - c(b) are >= 0 and sum to at most T, which is what the
// work-list capacity and every buffer bound assume. A well-formed array
// (off[0] = 0, non-decreasing, off[B] = T) is left unchanged.
//
// Unrolled, c(b) = min(max(0, off[0], ..., off[b]), T): a prefix maximum and
// one clamp, which is how the builder computes it in parallel
// (clamp_offset(inclusive prefix max inside a chunk, running max of the
// earlier chunks, T)).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define HSTU_HD __host__ __device__
#else
#define HSTU_HD
#endif

namespace hstu {

// One step of the recurrence above: raw raised to at least floor_, then capped at T.
HSTU_HD inline int64_t clamp_offset(int64_t raw, int64_t floor_, int64_t T) {
  const int64_t x = raw < floor_ ? floor_ : raw;
  return x > T ? T : x;
}

}  // namespace hstu
