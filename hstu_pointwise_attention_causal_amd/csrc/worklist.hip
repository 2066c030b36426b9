// Per-tile work list of the jagged attention kernels.
//
// A work item is one (sequence b, head h, query tile qt) with qt < ceil(n_b/BM).
// Key tiles above the diagonal of a query tile are never visited by the
// attention kernels (their loop stops at the diagonal), so fully masked
// upper-triangle tiles cost nothing. Items are emitted longest-first: the cost
// of query tile qt is proportional to qt + 1 key tiles, so the list is ordered
// by qt descending ("levels"). The hardware dispatcher hands blocks to compute
// units in block order, which makes this a longest-processing-time-first
// schedule over a dynamic pool of compute units.
//
// The builder runs as ONE workgroup, on the stream of the attention call,
// entirely on device: the host never reads the offsets. It also writes the
// clamped copy of the offsets (offsets.h) that every later kernel of the call
// reads instead of the caller's array.
#include "common.h"
#include "launch.h"
#include "offsets.h"

namespace hstu {

namespace {

constexpr int kBuildThreads = 1024;

// Inclusive scan over the block (kBuildThreads threads); returns the inclusive
// prefix of `v` and writes the block total to *total.
__device__ int block_inclusive_scan(int v, int* total) {
  __shared__ int wave_sums[kBuildThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kBuildThreads / 64 ? wave_sums[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < kBuildThreads / 64) wave_sums[lane] = s;
  }
  __syncthreads();
  int prefix = wave > 0 ? wave_sums[wave - 1] : 0;
  *total = wave_sums[kBuildThreads / 64 - 1];
  __syncthreads();
  return x + prefix;
}

// Inclusive max-scan of int64 values over the block; writes the block's
// maximum to *total.
__device__ int64_t block_inclusive_max(int64_t v, int64_t* total) {
  __shared__ int64_t wave_max[kBuildThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x = y > x ? y : x;
  }
  if (lane == 63) wave_max[wave] = x;
  __syncthreads();
  int64_t before = INT64_MIN, all = INT64_MIN;
  for (int i = 0; i < kBuildThreads / 64; ++i) {
    const int64_t m = wave_max[i];
    if (i < wave) before = m > before ? m : before;
    all = m > all ? m : all;
  }
  *total = all;
  __syncthreads();
  return before > x ? before : x;
}

// Counters and scans of the builder live in LDS when the levels and the
// sequences fit (LDS atomics and reads instead of global-memory round trips in
// every phase); tile_base is also copied out, for the attention kernels.
constexpr int kLdsLevels = 4096;   // num_levels + 1 entries per array
constexpr int kLdsSeqs = 4096;     // B + 1 entries

template <bool LDS>
__global__ __launch_bounds__(kBuildThreads) void build_worklist_kernel(
    const int64_t* __restrict__ off_in, int64_t T, int B, int H, int BM, int num_levels,
    int64_t* __restrict__ off, int* __restrict__ hdr, int* __restrict__ hist_g, int* __restrict__ level_start_g,
    int* __restrict__ fill_g, int* __restrict__ tile_base_g, WorkItem* __restrict__ items) {
  __shared__ int lds_hist[LDS ? kLdsLevels : 1], lds_level_start[LDS ? kLdsLevels : 1],
      lds_fill[LDS ? kLdsLevels : 1], lds_tile_base[LDS ? kLdsSeqs : 1];
  int* hist = LDS ? lds_hist : hist_g;
  int* level_start = LDS ? lds_level_start : level_start_g;
  int* fill = LDS ? lds_fill : fill_g;
  int* tile_base = LDS ? lds_tile_base : tile_base_g;
  const int tid = threadIdx.x;
  for (int i = tid; i <= num_levels; i += kBuildThreads) {
    hist[i] = 0;
    fill[i] = 0;
  }

  // 0. the clamped offsets: c(b) = min(max(0, off[0..b]), T)
  int64_t run = 0;   // max(0, off[0 .. b0 - 1])
  for (int b0 = 0; b0 <= B; b0 += kBuildThreads) {
    const int b = b0 + tid;
    int64_t chunk_max;
    const int64_t m = block_inclusive_max(b <= B ? off_in[b] : INT64_MIN, &chunk_max);
    if (b <= B) off[b] = clamp_offset(m, run, T);
    run = chunk_max > run ? chunk_max : run;
  }
  __syncthreads();

  // 1. tiles per sequence, histogram of tile counts, and the exclusive scan of
  //    tile counts over sequences (tile_base) for the flat pass below.
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += kBuildThreads) {
    int b = b0 + tid;
    int nt = 0;
    if (b < B) {
      const int64_t n = off[b + 1] - off[b];   // >= 0, sum over b <= T
      nt = n <= 0 ? 0 : static_cast<int>((n + BM - 1) / BM);
      nt = min(nt, num_levels);
      atomicAdd(&hist[nt], 1);
    }
    int chunk_total;
    int incl = block_inclusive_scan(nt, &chunk_total);
    if (b < B) tile_base[b] = carry + incl - nt;
    carry += chunk_total;
  }
  const int total_tiles = carry;
  if (tid == 0) tile_base[B] = total_tiles;
  __syncthreads();

  // 2. cnt[qt] = #sequences with more than qt tiles = sum_{m > qt} hist[m];
  //    level_start[qt] = H * sum_{qt' > qt} cnt[qt'] (levels laid out from the
  //    top level down). Two suffix scans, done as prefix scans over the
  //    reversed level index r = num_levels - 1 - qt.
  carry = 0;
  for (int r0 = 0; r0 < num_levels; r0 += kBuildThreads) {
    int r = r0 + tid;
    int qt = num_levels - 1 - r;
    int h = (r < num_levels)
                ? __hip_atomic_load(&hist[qt + 1], __ATOMIC_RELAXED,
                                    LDS ? __HIP_MEMORY_SCOPE_WORKGROUP : __HIP_MEMORY_SCOPE_AGENT)
                : 0;
    int chunk_total;
    int incl = block_inclusive_scan(h, &chunk_total);
    if (r < num_levels) level_start[qt] = carry + incl;  // cnt[qt], stored temporarily
    carry += chunk_total;
  }
  __syncthreads();
  carry = 0;
  for (int r0 = 0; r0 < num_levels; r0 += kBuildThreads) {
    int r = r0 + tid;
    int qt = num_levels - 1 - r;
    int c = (r < num_levels) ? level_start[qt] : 0;
    int chunk_total;
    int incl = block_inclusive_scan(c, &chunk_total);
    __syncthreads();
    if (r < num_levels) level_start[qt] = H * (carry + incl - c);
    carry += chunk_total;
  }
  __syncthreads();

  // 3. flat pass over all (sequence, tile) pairs: place the H items of each.
  for (int f = tid; f < total_tiles; f += kBuildThreads) {
    int lo = 0, hi = B;  // largest b with tile_base[b] <= f
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (tile_base[mid] <= f) lo = mid; else hi = mid;
    }
    // skip empty sequences that share tile_base with the next one
    int b = lo;
    int qt = f - tile_base[b];
    int slot = atomicAdd(&fill[qt], 1);
    int base = level_start[qt] + slot * H;
    const int64_t s0 = off[b];
    const int n = static_cast<int>(off[b + 1] - s0);
    const int tb = tile_base[b];
    for (int h = 0; h < H; ++h) {
      WorkItem w;
      w.seq0 = static_cast<int32_t>(s0);
      w.n = n;
      w.packed = qt | (h << 20);
      w.tile_base = tb;
      items[base + h] = w;
    }
  }
  if (LDS)
    for (int i = tid; i <= B; i += kBuildThreads) tile_base_g[i] = tile_base[i];
  if (tid == 0) {
    hdr[0] = total_tiles * H;
    hdr[1] = 0;
  }
}

}  // namespace

WorklistLayout worklist_layout(int B, int64_t T, int H, int BM) {
  WorklistLayout L;
  int64_t levels = (T + BM - 1) / BM + 1;
  int64_t cap_tiles = (T + static_cast<int64_t>(B) * (BM - 1)) / BM + 1;
  L.num_levels = static_cast<int>(levels);
  L.capacity = cap_tiles * H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  L.hdr_off = take(16);
  L.offc_off = take(sizeof(int64_t) * (static_cast<size_t>(B) + 1));
  L.hist_off = take(sizeof(int) * (levels + 1));
  L.level_start_off = take(sizeof(int) * (levels + 1));
  L.fill_off = take(sizeof(int) * (levels + 1));
  L.tile_base_off = take(sizeof(int) * (static_cast<size_t>(B) + 1));
  L.items_off = take(sizeof(WorkItem) * static_cast<size_t>(L.capacity));
  L.meta_blocks = kMetaPerTile * cap_tiles + 2;   // +2: a key tile's pair of blocks may run past the last
  L.meta_off = take(sizeof(BlockMeta) * static_cast<size_t>(L.meta_blocks) * static_cast<size_t>(H));
  L.bytes = off;
  return L;
}

hipError_t launch_build_worklist(const int64_t* off, int64_t T, int B, int H, int BM, const WorklistLayout& L,
                                 char* ws, hipStream_t stream) {
  int64_t* offc = reinterpret_cast<int64_t*>(ws + L.offc_off);
  int* hdr = reinterpret_cast<int*>(ws + L.hdr_off);
  int* hist = reinterpret_cast<int*>(ws + L.hist_off);
  int* level_start = reinterpret_cast<int*>(ws + L.level_start_off);
  int* fill = reinterpret_cast<int*>(ws + L.fill_off);
  int* tile_base = reinterpret_cast<int*>(ws + L.tile_base_off);
  WorkItem* items = reinterpret_cast<WorkItem*>(ws + L.items_off);
  if (L.num_levels + 1 <= kLdsLevels && B + 1 <= kLdsSeqs)
    hipLaunchKernelGGL(build_worklist_kernel<true>, dim3(1), dim3(kBuildThreads), 0, stream, off, T, B, H, BM,
                       L.num_levels - 1, offc, hdr, hist, level_start, fill, tile_base, items);
  else
    hipLaunchKernelGGL(build_worklist_kernel<false>, dim3(1), dim3(kBuildThreads), 0, stream, off, T, B, H, BM,
                       L.num_levels - 1, offc, hdr, hist, level_start, fill, tile_base, items);
  return hipGetLastError();
}

}  // namespace hstu
