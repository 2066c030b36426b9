// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hstu {

// ---------------------------------------------------------------- work list
struct WorklistLayout {
  int num_levels = 0;   // ceil(T/BM) + 1
  int64_t capacity = 0; // upper bound on the number of items
  size_t offc_off = 0;  // int64 [B+1]: the clamped offsets (offsets.h) every kernel reads
  size_t hdr_off = 0, hist_off = 0, level_start_off = 0, fill_off = 0, tile_base_off = 0,
         items_off = 0;
  // per-(head, 32-key block) metadata of the bf16 forward: 4 blocks per query tile
  size_t meta_off = 0;
  int64_t meta_blocks = 0;   // blocks per head (row stride of the metadata array)
  size_t bytes = 0;
};

WorklistLayout worklist_layout(int B, int64_t T, int H, int BM);
// Writes the clamped offsets and the work list into ws (laid out by L).
hipError_t launch_build_worklist(const int64_t* off, int64_t T, int B, int H, int BM, const WorklistLayout& L,
                                 char* ws, hipStream_t stream);

// Query-tile height shared by every attention kernel and the work list.
constexpr int kAttnBM = 128;
// 32-key metadata blocks per query tile
constexpr int kMetaPerTile = kAttnBM / 32;

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t ldq, ldk, ldv;
  void* o;         // forward output
  int64_t ldo;
  const int64_t* off;       // the clamped copy written by the work-list builder
  const int64_t* ts;        // may be NULL
  const float* pos_table;   // may be NULL
  int pos_buckets;
  const float* time_table;  // may be NULL
  int time_buckets;
  float alpha;
  float divisor;
  int num_heads;
  const void* items;        // WorkItem list
  const int* item_count;
  int64_t capacity;
  const int* tile_base;     // [B+1] exclusive scan of query tiles per sequence
  void* meta;               // BlockMeta [H][meta_blocks]
  int64_t meta_blocks;
};

// Metadata of one 32-key block of one head: the largest key norm and the
// timestamp range of the keys inside the sequence (32 bytes, DMA-friendly).
struct BlockMeta {
  float kmax;
  float pad0;
  int64_t tmin;
  int64_t tmax;
  int64_t pad1;
};
static_assert(sizeof(BlockMeta) == 32, "BlockMeta layout");

// Candidate scoring against a cached history (M-FALCON reading): candidates
// [T_c, H, d] with cand_off, history keys / values [T_h, H, d] with hist_off.
struct CandArgs {
  const void* q_c;
  const void* k_c;
  const void* v_c;
  int64_t ldq, ldk, ldv;
  const void* k_h;
  const void* v_h;
  int64_t ldkh, ldvh;
  void* o;
  int64_t ldo;
  const int64_t* hist_off_in;   // the caller's offsets, read once by the chunk-scan kernel
  const int64_t* cand_off_in;
  int64_t* hist_off;        // workspace: their clamped copies (offsets.h), read by every other kernel
  int64_t* cand_off;
  int64_t hist_tokens, cand_tokens;
  const int64_t* ts_h;      // history timestamps, NULL without a time table
  const int64_t* ts_c;      // candidate timestamps, NULL without a time table
  const float* pos_table;
  int pos_buckets;
  const float* time_table;
  int time_buckets;
  float alpha;
  float divisor;
  int num_heads;
  int num_seqs;
  int max_candidates;      // candidates past it in a sequence are not scored
  int64_t* chunk_base;     // workspace: [num_seqs + 1] first history chunk of each sequence
  float* partial;          // workspace: fp32 [chunks][max_candidates][H][d] partial outputs
  int64_t chunk_limit;     // chunks the partial buffer holds (set by the launcher)
};
// History keys per chunk of candidate scoring: a sequence's history splits
// into max(1, ceil(n / kCandChunk)) chunks, each one workgroup's key range.
constexpr int kCandChunk = 2048;
// Workspace of launch_attn_cand_bf16: chunk bases, then (at
// cand_partial_offset) the partial outputs.
size_t cand_partial_offset(int num_seqs);
size_t cand_workspace_bytes(int64_t hist_tokens, int num_seqs, int max_candidates, int num_heads, int d);
// Chunk bases, the chunked scoring, then the sum of the partials of
// multi-chunk sequences, all on `stream`.
hipError_t launch_attn_cand_bf16(const CandArgs& a, int d, int64_t hist_tokens, int64_t cand_tokens,
                                 hipStream_t stream);

hipError_t launch_attn_block_meta(const AttnArgs& a, int dqk, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int dqk, int dv, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, int dqk, int dv, hipStream_t stream);

// ---------------------------------------------------------------- backward
// Position-table entries the backward keeps (values and gradients) in LDS;
// larger tables are rejected by the C ABI.
constexpr int kBwdPosMax = 1024;
// Time buckets that int64 gaps can reach (0..62), rounded up.
constexpr int kBwdTimeSlots = 64;

struct AttnBwdArgs {
  AttnArgs f;               // forward inputs, work list and block metadata
  const void* d_o;
  int64_t lddo;
  void* dq;
  int64_t lddq;
  void* dk;
  int64_t lddk;
  void* dv;
  int64_t lddv;
  float* d_pos;             // [H][Bp] or NULL
  float* d_time;            // [H][Bt] or NULL
  float* partial;           // [H][tile_rows][grad_stride]: bias-gradient sums of one key tile
  int grad_stride;          // (Bp if pos) + (kBwdTimeSlots if time)
  int64_t tile_rows;        // rows per head of `partial` (>= total query tiles)
  int num_seqs;
};

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, int dqk, int dv, hipStream_t stream);
// x[0 .. n) = value (a kernel, so that the call can be captured in a graph)
hipError_t launch_fill_f32(float* x, int64_t n, float value, hipStream_t stream);

}  // namespace hstu
