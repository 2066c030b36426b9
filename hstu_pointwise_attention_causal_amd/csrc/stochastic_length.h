// Internal launch interface of the Stochastic Length kernels (random
// shortening of long training histories; briansu.co explainer, section 6
// "Why it works"): new offsets, the kept tokens' gather index, row gathers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

struct SlArgs {
  const int64_t* seq_offsets;  // [B+1], clamped to [0, T] and made non-decreasing on read
  int64_t total_tokens;        // T: keys and gather_index hold T entries
  int num_seqs;
  int64_t max_len;             // L >= 0
  const uint32_t* keys;        // [T] one random key per token
  int64_t* new_offsets;        // [B+1] out
  int64_t* gather_index;       // [T] out; entries past new_offsets[B] untouched
};

// new_offsets = exclusive scan of min(n_b, L); then per sequence the kept
// tokens' input positions, in order, at gather_index[new_offsets[b] ...].
hipError_t launch_stochastic_length(const SlArgs& a, hipStream_t stream);

struct GatherArgs {
  const int64_t* index;   // [>= min(*count, max_rows)]
  const int64_t* count;   // device: rows to copy (e.g. new_offsets + B)
  int64_t max_rows;       // host bound: at most this many rows are copied
  int64_t src_rows;       // rows of src; rows whose index falls outside are left unwritten
  const void* src;
  int64_t src_stride;     // bytes
  void* dst;
  int64_t dst_stride;     // bytes
  int64_t row_bytes;
};

// dst row r = src row index[r] for r < min(*count, max_rows). Row bytes,
// strides and base addresses must share an alignment of 4, 8 or 16 bytes.
hipError_t launch_gather_rows(const GatherArgs& a, hipStream_t stream);

}  // namespace hstu
