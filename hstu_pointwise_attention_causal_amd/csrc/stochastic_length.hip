// Stochastic Length: random shortening of long training histories (named in
// the briansu.co explainer, section 6 "Why it works"; the pages give no
// procedure). Reading: a sequence of n <= L tokens is kept whole; a longer one
// keeps the L tokens whose (key, position) pairs are smallest, in their
// original order, where the caller passes one uniform 32-bit key per token --
// a uniformly random L-subset.
//
//   sl_offsets_kernel   new_offsets = exclusive scan of min(n_b, L) (one block)
//   sl_select_kernel    one block per sequence: the L-th smallest key by a
//                       three-pass radix select (11 + 11 + 10 bits, LDS
//                       histograms), then a compaction in position order (per-
//                       wave ballot counts, one barrier, a placing walk) that
//                       keeps keys below it and the first ones equal to it,
//                       writing the kept tokens' input positions; a
//                       sequence of up to 16384 tokens works on an LDS copy
//                       of its keys
//   gather_rows_kernel  dst row r = src row index[r] (a wave per wide row, a
//                       thread per narrow one)
#include "stochastic_length.h"

#include <algorithm>

#include "common.h"
#include "timing.h"

namespace hstu {

namespace {

// Sequence b's token range, clamped to [0, T] and non-decreasing, so that a
// malformed offsets array cannot move a read or a write out of bounds.
__device__ __forceinline__ void seq_range(const SlArgs& a, int b, int64_t& s, int64_t& e) {
  const int64_t T = a.total_tokens;
  s = min(max(a.seq_offsets[b], int64_t(0)), T);
  e = min(max(a.seq_offsets[b + 1], s), T);
}

__global__ __launch_bounds__(1024) void sl_offsets_kernel(SlArgs a) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t carry = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int64_t len = 0;
    if (b < a.num_seqs) {
      int64_t s, e;
      seq_range(a, b, s, e);
      len = min(e - s, a.max_len);
    }
    int64_t v = len;   // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t u = __shfl_up(v, o, 64);
      if (lane >= o) v += u;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    int64_t before = 0, total = 0;
    for (int i = 0; i < 16; ++i) {
      before += i < w ? wsum[i] : 0;
      total += wsum[i];
    }
    if (b < a.num_seqs) a.new_offsets[b] = carry + before + v - len;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) a.new_offsets[a.num_seqs] = carry;
}

constexpr int kSelThreads = 1024;
constexpr int kBinsPerThread = 2048 / kSelThreads;

// Exclusive prefix over the block of per-thread counts, and the block total
// (kSelThreads / 64 wave totals in LDS).
__device__ __forceinline__ uint32_t block_excl(uint32_t v, uint32_t* wtot, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    before += i < w ? wtot[i] : 0;
    total += wtot[i];
  }
  __syncthreads();   // wtot is reused by the next call
  return before + incl - v;
}

constexpr int kSelLdsKeys = 16384;   // sequences up to this long are selected from a copy of their keys in LDS

// The cap-th smallest key of key[0, nn) and the compaction of the kept
// positions into out[base ...]. `key` is a sequence's keys in global memory or
// their LDS copy; each call site is inlined with its own address space.
__device__ __forceinline__ void select_compact(const uint32_t* __restrict__ key, int nn, uint32_t cap,
                                               int64_t s, int64_t base, int64_t T, int64_t* __restrict__ out,
                                               uint32_t* hist, uint32_t* wtot, uint32_t* sel) {
  const int tid = threadIdx.x;
  // ---- the cap-th smallest key: rank k among the keys that match the digits so far
  uint32_t prefix = 0, mask = 0, k = cap;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dm = pass < 2 ? 2047u : 1023u;
    for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nn; i += kSelThreads) {
      const uint32_t kv = key[i];
      if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & dm], 1u);
    }
    __syncthreads();
    uint32_t c[kBinsPerThread], sum = 0;
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) {
      c[j] = hist[kBinsPerThread * tid + j];
      sum += c[j];
    }
    uint32_t total;
    uint32_t run = block_excl(sum, wtot, total);
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) {
      if (run < k && run + c[j] >= k) {   // exactly one bin crosses rank k
        sel[0] = kBinsPerThread * tid + j;
        sel[1] = run;
      }
      run += c[j];
    }
    __syncthreads();
    k -= sel[1];
    prefix |= sel[0] << shift;
    mask |= dm << shift;
    __syncthreads();
  }
  // keys below `prefix` are kept; of the keys equal to it, the first k by position
  const uint32_t kstar = prefix, take_eq = k;

  // ---- compaction in position order. A kept token's output position is the
  // number of keys below kstar before it plus min(equal keys before it,
  // take_eq). Wave w owns a contiguous run of positions: it counts its keys
  // below and equal to kstar (ballots), one barrier publishes the per-wave
  // counts, and a second walk over the run places each kept token from its
  // wave's starting counts and the ballot bits of the lanes before it.
  const int lane = tid & 63, w = tid >> 6;
  constexpr int kWaves = kSelThreads / 64;
  const int per = (((nn + kWaves - 1) / kWaves) + 63) & ~63;
  const int lo = min(nn, w * per), hi = min(nn, lo + per);
  uint32_t nlt = 0, neq = 0;
  for (int i0 = lo; i0 < hi; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t kv = i < hi ? key[i] : 0u;
    nlt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < hi && kv < kstar));
    neq += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < hi && kv == kstar));
  }
  if (lane == 0) {
    wtot[w] = nlt;
    wtot[kWaves + w] = neq;
  }
  __syncthreads();
  uint32_t lt_run = 0, eq_run = 0;
  for (int j = 0; j < w; ++j) {
    lt_run += wtot[j];
    eq_run += wtot[kWaves + j];
  }
  for (int i0 = lo; i0 < hi; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t kv = i < hi ? key[i] : 0u;
    const bool lt = i < hi && kv < kstar, eq = i < hi && kv == kstar;
    const uint64_t bl = __builtin_amdgcn_ballot_w64(lt), be = __builtin_amdgcn_ballot_w64(eq);
    const uint32_t lt_before = lt_run + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bl >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bl), 0u));
    const uint32_t eq_before = eq_run + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(be >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(be), 0u));
    if (lt || (eq && eq_before < take_eq)) {
      const int64_t pos = static_cast<int64_t>(lt_before) + min(eq_before, take_eq);
      if (base + pos < T) out[base + pos] = s + i;
    }
    lt_run += __builtin_popcountll(bl);
    eq_run += __builtin_popcountll(be);
  }
}

__global__ __launch_bounds__(kSelThreads) void sl_select_kernel(SlArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[2 * (kSelThreads / 64)];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t skeys[kSelLdsKeys];
  const int b = blockIdx.x, tid = threadIdx.x;
  int64_t s, e;
  seq_range(a, b, s, e);
  const int64_t n = e - s, T = a.total_tokens;
  const int64_t base = a.new_offsets[b];
  int64_t* out = a.gather_index;
  if (n <= a.max_len) {   // kept whole
    for (int64_t i = tid; i < n; i += kSelThreads)
      if (base + i < T) out[base + i] = s + i;
    return;
  }
  if (a.max_len == 0) return;
  const uint32_t* key = a.keys + s;
  const int nn = static_cast<int>(n);   // n < T < 2^31
  const uint32_t cap = static_cast<uint32_t>(a.max_len);   // < n
  if (nn <= kSelLdsKeys) {
    // one read of the keys from memory (every load in flight before the
    // first LDS store); the passes over them then run from LDS
    constexpr int kPer = kSelLdsKeys / kSelThreads;
    uint32_t kr[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * kSelThreads;
      kr[j] = i < nn ? key[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * kSelThreads;
      if (i < nn) skeys[i] = kr[j];
    }
    __syncthreads();
    select_compact(skeys, nn, cap, s, base, T, out, hist, wtot, sel);
  } else {
    select_compact(key, nn, cap, s, base, T, out, hist, wtot, sel);
  }
}

// Wide rows: one wave per row, lanes over 16/8/4-byte chunks. Narrow rows
// (fewer than 16 chunks): one thread per row.
template <typename V, bool WIDE>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherArgs a) {
  const int64_t rows = max(int64_t(0), min(*a.count, a.max_rows));
  const int64_t cpr = a.row_bytes / static_cast<int64_t>(sizeof(V));
  const char* src = static_cast<const char*>(a.src);
  char* dst = static_cast<char*>(a.dst);
  if (WIDE) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
    for (int64_t r = wave; r < rows; r += nwaves) {
      const int64_t sr = a.index[r];
      if (sr < 0 || sr >= a.src_rows) continue;
      const V* sp = reinterpret_cast<const V*>(src + sr * a.src_stride);
      V* dp = reinterpret_cast<V*>(dst + r * a.dst_stride);
      for (int64_t c = lane; c < cpr; c += 64) dp[c] = sp[c];
    }
  } else {
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; r < rows;
         r += static_cast<int64_t>(gridDim.x) * 256) {
      const int64_t sr = a.index[r];
      if (sr < 0 || sr >= a.src_rows) continue;
      const V* sp = reinterpret_cast<const V*>(src + sr * a.src_stride);
      V* dp = reinterpret_cast<V*>(dst + r * a.dst_stride);
      for (int64_t c = 0; c < cpr; ++c) dp[c] = sp[c];
    }
  }
}

template <typename V>
hipError_t launch_gather_v(const GatherArgs& a, hipStream_t stream) {
  const int64_t cpr = a.row_bytes / static_cast<int64_t>(sizeof(V));
  if (cpr >= 16) {
    const int64_t blocks = std::min<int64_t>((a.max_rows + 3) / 4, 8192);
    hipLaunchKernelGGL((gather_rows_kernel<V, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  } else {
    const int64_t blocks = std::min<int64_t>((a.max_rows + 255) / 256, 8192);
    hipLaunchKernelGGL((gather_rows_kernel<V, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

bool aligned_to(int64_t v, int64_t al) { return v % al == 0; }

}  // namespace

hipError_t launch_stochastic_length(const SlArgs& a, hipStream_t stream) {
  TimedScope timed(kTimedSlSelect, stream);
  hipLaunchKernelGGL(sl_offsets_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_seqs == 0) return e;
  hipLaunchKernelGGL(sl_select_kernel, dim3(static_cast<unsigned>(a.num_seqs)), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const GatherArgs& a, hipStream_t stream) {
  if (a.max_rows <= 0 || a.row_bytes <= 0) return hipSuccess;
  const int64_t s = static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.src));
  const int64_t d = static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.dst));
  auto all = [&](int64_t al) {
    return aligned_to(s, al) && aligned_to(d, al) && aligned_to(a.src_stride, al) && aligned_to(a.dst_stride, al) &&
           aligned_to(a.row_bytes, al);
  };
  TimedScope timed(kTimedGather, stream);
  if (all(16)) return launch_gather_v<u32x4_t>(a, stream);
  if (all(8)) return launch_gather_v<u32x2_t>(a, stream);
  if (all(4)) return launch_gather_v<uint32_t>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace hstu
