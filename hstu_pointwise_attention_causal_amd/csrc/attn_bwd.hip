// Causal pointwise aggregated attention, backward, on gfx950.
//
// Gradients of sum(O * dO) for the forward of attn_fwd.hip. With x the
// pre-activation of a pair (j <= i of one sequence), sig = 1/(1 + e^-x) and
// SiLU'(x) = sig (1 + x (1 - sig)):
//     dA_ij = dO_i . v_j            dS_ij = dA_ij SiLU'(x_ij) / N
//     dv_j  = sum_i A_ij dO_i       dk_j  = alpha sum_i dS_ij q_i
//     dq_i  = alpha sum_j dS_ij k_j
//     dP[h][b], dTt[h][b] = sum of dS_ij over the pairs that read entry b.
// (Derived from the forward of the neurarch model card, "Exported PyTorch",
// HSTUBlock aggregation, and the relative biases of the briansu.co explainer,
// section 3; the pages train every position generatively, daiwk reproduction
// notes, core formula.)
//
// Two passes over the same work list, both without atomics to global memory,
// so every result is the same from run to run:
//
//   key pass (attn_bwd_kv_kernel): a work item owns 128 keys (32 per wave) and
//   walks the query tiles from the diagonal to the end of the sequence. K and V
//   of the wave's keys stay in registers as MFMA B operands; Q and dO tiles
//   stream through LDS:
//     S[i][j]  = Q K^T,  dA[i][j] = dO V^T     A = Q / dO rows (LDS)
//     dV[j][c] += P^T dO, dK[j][d] += dS^T Q   A = P / dS straight from the
//                                              S / dA accumulators, B = dO / Q
//                                              read transposed from LDS
//   The accumulator of S leaves each lane one key (column) and 16 query rows,
//   which is the A-operand layout of the two updates when the rows of a 16-row
//   step are taken in the order {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); the
//   transposed reads of dO and Q use the same order. Bias-table gradients are
//   summed per gradient wave in LDS (one table per wave, so no two waves race)
//   and written as one partial row per key tile.
//
//   query pass (attn_bwd_q_kernel): a work item owns 128 query rows, as in the
//   forward, and recomputes S^T = K Q^T and dA^T = V dO^T per key block to
//   form dQ[i][d] += dS K with K read transposed from LDS.
//
//   Both passes run eight waves per workgroup in two roles on each SIMD: a
//   score wave (S, the bias, SiLU and SiLU' of every pair, one block ahead)
//   and a gradient wave (the tile loads, the block classes, dA, dS and the
//   products that use them); SiLU' and the classes pass between the two
//   through LDS (see each kernel's comment).
//
//   bias reduction (attn_bwd_bias_reduce_kernel): sums the partial rows of
//   each head in tile order.
//
// Scores are kept in x' = log2(e) x units as in the forward (one exp2 and one
// reciprocal per pair); P is stored to bf16 as log2(e) SiLU(x) and the output
// scales remove the factor.
#include <type_traits>

#include "attn_common.h"
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace hstu {

namespace {

constexpr int kBW = kAttnBM / 32;     // waves per workgroup, 32 rows (keys or queries) each
constexpr int kBThreads = kBW * 64;
constexpr int kBBN = 64;              // rows of a streamed tile
constexpr float kLn2 = 0.6931471805599453f;

// log2(e) SiLU(x) and SiLU'(x) from x' = log2(e) x.
__device__ __forceinline__ void silu_and_grad(float xl, float& pl, float& dsilu) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-xl));
  pl = xl * sg;
  dsilu = sg * fmaf(xl * kLn2, 1.0f - sg, 1.0f);
}

// Bias class of one (32 query rows, 32 keys) block; both blocks start at
// multiples of 32 inside one sequence.
//   kBUniform  - every pair reads the same position and time buckets;
//   kBTwoTime  - one position bucket and time buckets tlo, tlo + 1: a pair
//                takes tlo + 1 exactly when t_i - t_j >= 2^(tlo+1) - 1;
//   kBGeneral  - per-pair buckets and the causal / sequence-end mask.
enum BPath { kBUniform = 0, kBTwoTime = 1, kBGeneral = 2 };
struct BlockClass {
  int path;
  int tlo;
  float clo, chi;   // x'-unit bias of the pairs in bucket tlo / tlo + 1
};

__device__ __forceinline__ BlockClass classify_block(int qa, int ka, int n, bool has_pos, int Bp, bool has_time,
                                                     int Bt, int64_t tq_min, int64_t tq_max, int64_t tk_min,
                                                     int64_t tk_max, float pos_last, const float* stime) {
  BlockClass c{kBGeneral, 0, 0.f, 0.f};
  const bool need_mask = (ka + 31 > qa) || (qa + 31 >= n) || (ka + 31 >= n);
  const bool pos_uniform = !has_pos || (qa - (ka + 31) >= Bp - 1);
  if (need_mask || !pos_uniform) return c;
  c.clo = c.chi = pos_last;
  if (!has_time) {
    c.path = kBUniform;
    return c;
  }
  const int blo = time_bucket64(tq_min - tk_max, Bt), bhi = time_bucket64(tq_max - tk_min, Bt);
  if (blo == bhi) {
    c.path = kBUniform;
    c.tlo = blo;
    c.clo = c.chi = pos_last + stime[blo];
  } else if (bhi == blo + 1) {
    c.path = kBTwoTime;
    c.tlo = blo;
    c.clo = pos_last + stime[blo];
    c.chi = pos_last + stime[bhi];
  }
  return c;
}

// Time buckets of a block whose pairs need per-pair work (mask or varying
// position buckets). Every valid pair's gap lies in [gmin, gmax] (from the
// blocks' timestamp ranges), so its bucket lies in [lo, hi]; when that gap
// range fits in int32 the wrapped difference of the timestamps' low words is
// the gap itself.
struct TimeSpan {
  int lo, hi;
  bool narrow;
};

__device__ __forceinline__ TimeSpan time_span(int64_t gmin, int64_t gmax, int Bt) {
  TimeSpan t;
  t.lo = time_bucket64(gmin, Bt);
  t.hi = time_bucket64(gmax, Bt);
  t.narrow = gmax <= int64_t(INT32_MAX) - 1 && gmin >= int64_t(INT32_MIN);
  return t;
}

// Direct HBM -> LDS loads of one 64-row tile of two row-major matrices (A with
// ACH, B with BCH 16-byte chunks per row), the rows' timestamps and the two
// 32-row metadata records. Instruction i of a matrix is issued by wave i % kBW;
// wave 0 loads the timestamps, wave 1 the metadata. Rows past the sequence
// (and metadata past its last block) arrive as zeros.
template <int ACH, int BCH>
__device__ __forceinline__ void issue_rows_tile(const char* abase, const char* bbase, int64_t lda, int64_t ldb,
                                                const int64_t* tsbase, const BlockMeta* mbase, int n, int r0,
                                                int w, int lane, const uint32_t* aoff, const uint32_t* boff,
                                                char* sa, char* sb, int64_t* st, BlockMeta* sm) {
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase + static_cast<int64_t>(r0) * lda * 2,
                                              static_cast<int64_t>(n - r0) * lda * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bbase + static_cast<int64_t>(r0) * ldb * 2,
                                              static_cast<int64_t>(n - r0) * ldb * 2);
#pragma unroll
  for (int j = 0; j < (ACH + kBW - 1) / kBW; ++j) {
    const int i = w + j * kBW;
    if (i < ACH) load_lds16(ra, sa + i * 1024, aoff[j]);
  }
#pragma unroll
  for (int j = 0; j < (BCH + kBW - 1) / kBW; ++j) {
    const int i = w + j * kBW;
    if (i < BCH) load_lds16(rb, sb + i * 1024, boff[j]);
  }
  if (w == 0 && lane < kBBN / 2) {
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tsbase ? tsbase + r0 : nullptr,
                                                tsbase ? static_cast<int64_t>(n - r0) * 8 : 0);
    load_lds16(rt, reinterpret_cast<char*>(st), lane * 16);
  }
  if (w == 1 % kBW && lane < 4) {
    const int blk0 = r0 / 32, nblk = (n + 31) / 32;
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mbase + blk0, static_cast<int64_t>(nblk - blk0) * 32);
    load_lds16(rm, reinterpret_cast<char*>(sm), lane * 16);
  }
}

// Per-lane global byte offsets of the direct loads of a 64-row tile with CH
// chunks per row, stored with the dual-read swizzle.
template <int CH>
__device__ __forceinline__ void tile_load_offsets(int w, int lane, int64_t ld, uint32_t* off) {
#pragma unroll
  for (int j = 0; j < (CH + kBW - 1) / kBW; ++j) {
    const int s = (w + j * kBW) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz_dual<CH>(r);
    off[j] = static_cast<uint32_t>(r * ld * 2 + c * 16);
  }
}

// LDS byte offset of this lane's A-operand row read (row lr, k-step kb).
template <int CH>
__device__ __forceinline__ uint32_t row_read_offset(int lr, int lh, int kb) {
  return static_cast<uint32_t>((lr * CH + ((2 * kb + lh) ^ swz_dual<CH>(lr))) * 16);
}

// LDS byte offsets of this lane's two transposed reads (rows r1 and r1 + 8 of
// a 16-row step, 32-column group nb) of the B operand.
template <int CH>
__device__ __forceinline__ void tr_read_offsets(int lane, int nb, uint32_t& o0, uint32_t& o1) {
  const int lh = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
  const int r1 = 4 * lh + (i16 >> 2);
  const int c = nb * 4 + (g16 & 1) * 2 + ((i16 & 3) >> 1);
  const int half = (i16 & 1) * 8;
  o0 = static_cast<uint32_t>((r1 * CH + (c ^ swz_dual<CH>(r1))) * 16 + half);
  o1 = static_cast<uint32_t>(((r1 + 8) * CH + (c ^ swz_dual<CH>(r1 + 8))) * 16 + half);
}

template <int ACH, int BCH>
__device__ __forceinline__ int rows_tile_loads(int w) {
  int c = 0;
  for (int i = w; i < ACH; i += kBW) ++c;
  for (int i = w; i < BCH; i += kBW) ++c;
  return c + (w == 0 ? 1 : 0) + (w == 1 % kBW ? 1 : 0);
}

template <int DQK, int DV>
struct BwdSmem {
  __attribute__((aligned(16))) char a[2][kBBN * DQK * 2];   // Q (key pass) or K (query pass)
  __attribute__((aligned(16))) char b[2][kBBN * DV * 2];    // dO (key pass) or V (query pass)
  __attribute__((aligned(16))) int64_t t[2][kBBN];
  __attribute__((aligned(16))) BlockMeta m[2][2];
  float pos[kBwdPosMax];        // log2(e) P[h][.]
  float time[kBwdTimeSlots];    // log2(e) Tt[h][.]
};

// LDS float add without a return value; lanes that hit one address are all
// applied. Written as asm: the compiler's atomic carries no alias scope, so
// it would first wait for every tile load in flight. The compiler does not
// count it among the outstanding LDS operations: a reader on another wave
// waits for it explicitly (lgkmcnt(0) before the barrier), see below.
__device__ __forceinline__ void lds_add_f32(float* p, float v) {
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(to_lds(p)));
  asm volatile("ds_add_f32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Diagonal sums of a 32 x 32 block held as an MFMA accumulator: lane
// (lr, lh), element r holds row i' = 8(r/4) + 4 lh + r%4, column lr, on
// diagonal i' - lr. Element r of lane m of each half is rotated to the column
// (i' - m) mod 32 of the same row, whose diagonal is m (no wrap) or m - 32.
// On return lanes lr of both halves hold dpos = the sum of diagonal lr and
// dneg = the sum of diagonal lr - 32 (zero for lr = 0), each over the whole
// block; the order of the additions is fixed. All 16 rotations are issued
// before the first sum, so their LDS latencies overlap. The split by sign of
// i' - lr is a bit mask of each rotated value, computed from a lane value the
// compiler cannot hoist out of the caller's loop: hoisted, the 16 compares
// became 64-bit lane masks held across the block loop, which spilled to VGPR
// lanes and cost two v_readlane per select (measured on the key pass of 32
// sequences of 64-2048 tokens: 0.180 -> 0.171 ms).
__device__ __forceinline__ void diagonal_sums(const float* v, int lr, int lh, float& dpos, float& dneg) {
  const int t0 = 4 * lh - lr, hbase = lh << 5;
  float y[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int d = 8 * (r >> 2) + (r & 3) + t0;   // i' - lr
    y[r] = __int_as_float(__builtin_amdgcn_ds_bpermute((hbase | (d & 31)) << 2, __float_as_int(v[r])));
  }
  float sp = 0.f, sn = 0.f;
  int tm = t0;
  asm volatile("" : "+v"(tm));   // the masks below are recomputed per call, not kept as lane masks
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int neg = (8 * (r >> 2) + (r & 3) + tm) >> 31;   // all ones where i' - lr < 0
    const int yb = __float_as_int(y[r]);
    sp += __int_as_float(yb & ~neg);
    sn += __int_as_float(yb & neg);
  }
  dpos = sp + __shfl_xor(sp, 32, 64);
  dneg = sn + __shfl_xor(sn, 32, 64);
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// ============================================================================
// key pass: dK, dV and the bias-table gradients
//
// A work item owns 128 keys and walks the 32-row query blocks from the
// diagonal to the end of the sequence. Waves w and w + 4 of the workgroup run
// on one SIMD and share a group of 32 keys (kw = k0 + 32 (w & 3), one key per
// lane as the column of S), in two roles:
//   score wave (w < 4)      S = Q K^T one block ahead (its products spread
//                           over the current block's per-pair loop), the
//                           bias, P = SiLU(x) and SiLU'(x) of every pair
//                           (masked pairs: 0), dV += P^T dO;
//   gradient wave (w >= 4)  the tile loads, the block classes (64 blocks at a
//                           time, one per lane), and one block behind the
//                           score wave: dA = dO V^T, dS = dA SiLU'(x), the
//                           bias-table gradients and dK += dS^T Q.
// SiLU'(x) (fp16), each pair's time bucket and the block classes pass
// through LDS. Each role's registers fit two waves per SIMD, and the work
// that does not depend on the per-pair arithmetic runs on the gradient wave.
// K (score) and V (gradient) of the lane's key stay in registers as MFMA B
// operands; Q, dO, the timestamps and the metadata of block t + 2 load into
// a ring of four LDS slots while block t is processed, one barrier per block.
// ============================================================================
constexpr int kKW = 8;                // waves of a key-pass workgroup
constexpr int kKThreads = kKW * 64;
constexpr int kKRing = 4;             // 32-row block slots (Q, dO, timestamps, metadata)
constexpr int kKIssue = 4;            // waves that issue the tile loads (the gradient waves)
constexpr int kGFast = 32;            // time buckets summed in lane-private columns

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Class of a (query block, key group) pair, written by the gradient waves
// for 64 blocks at a time: the path (bits 0-1), the low time bucket of a one-
// or two-bucket block (bits 8-15), and flags.
constexpr int kInfoFastTime = 1 << 16;   // every time bucket of the block is below kGFast
constexpr int kInfoMasked = 1 << 17;     // causal or sequence-end mask inside the block
constexpr int kInfoNarrow = 1 << 18;     // every gap of the block fits in int32
struct KvClass {
  int info;
  float clo, chi;   // x'-unit bias of the pairs in bucket tlo / tlo + 1
  int pad;
};

template <int DQK, int DV>
struct KvLds {
  __attribute__((aligned(16))) char q[kKRing][32 * DQK * 2];
  __attribute__((aligned(16))) char d[kKRing][32 * DV * 2];
  __attribute__((aligned(16))) int64_t t[kKRing][32];
  __attribute__((aligned(16))) BlockMeta m[kKRing];
  f16x8_t xg[2][4][2][64];      // SiLU' of a block: [buffer][key group][r / 8][lane]
  u32x4_t xb[2][4][64];         // time bucket of pair r in byte r % 4 of word r / 4: [buffer][key group][lane]
  KvClass cls[2][4][64];        // [(block / 64) % 2][key group][block % 64]
  // Bias-table gradients, one table per gradient wave. Position buckets:
  // plain adds of diagonal sums. Time buckets below kGFast: one column per
  // lane ([wave][bucket][lane]), as most pairs of a block near the diagonal
  // share a bucket; larger buckets (gaps of 2^32 - 1 and more): per-wave sums.
  float gpos[4][kBwdPosMax];
  float gtime[4][kGFast][64];
  float gslow[4][kBwdTimeSlots];
  float pos[kBwdPosMax];        // log2(e) P[h][.] (one 0 without the table)
  float time[kBwdTimeSlots];    // log2(e) Tt[h][.] (one 0 without the table)
};

// Direct loads of one 32-row block of a row-major matrix with CH 16-byte
// chunks per row, stored with the dual-read swizzle: instruction i fills LDS
// slots [64 i, 64 i + 64) and is issued by gradient wave i % kKIssue. Rows
// past the sequence arrive as zeros.
template <int CH>
__device__ __forceinline__ void block_load_offsets(int wi, int lane, int64_t ld, uint32_t* off) {
  constexpr int NI = CH / 2;
#pragma unroll
  for (int j = 0; j < (NI + kKIssue - 1) / kKIssue; ++j) {
    const int s = (wi + j * kKIssue) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz_dual<CH>(r);
    off[j] = static_cast<uint32_t>(r * ld * 2 + c * 16);
  }
}

template <int CH>
__device__ __forceinline__ void issue_block(const char* base, int64_t ld, int n, int r0, int wi, const uint32_t* off,
                                            char* dst) {
  constexpr int NI = CH / 2;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + static_cast<int64_t>(r0) * ld * 2,
                                              static_cast<int64_t>(n - r0) * ld * 2);
#pragma unroll
  for (int j = 0; j < (NI + kKIssue - 1) / kKIssue; ++j) {
    const int i = wi + j * kKIssue;
    if (i < NI) load_lds16(rs, dst + i * 1024, off[j]);
  }
}

// The 32 timestamps (gradient wave 2; zeros without timestamps) and the
// metadata record (gradient wave 3) of the query block at row r0.
__device__ __forceinline__ void issue_block_extras(const int64_t* tsbase, const BlockMeta* mbase, int n, int r0,
                                                   int wi, int lane, int64_t* st, BlockMeta* sm) {
  if (wi == kKIssue - 2 && lane < 16) {
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tsbase ? tsbase + r0 : nullptr,
                                                tsbase ? static_cast<int64_t>(n - r0) * 8 : 0);
    load_lds16(rt, reinterpret_cast<char*>(st), lane * 16);
  }
  if (wi == kKIssue - 1 && lane < 2) {
    const int blk = r0 / 32, nblk = (n + 31) / 32;
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mbase + blk, static_cast<int64_t>(nblk - blk) * 32);
    load_lds16(rm, reinterpret_cast<char*>(sm), lane * 16);
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(kKThreads, 1) void attn_bwd_kv_kernel(AttnBwdArgs g) {
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  const AttnArgs& a = g.f;
  constexpr int KB = DQK / 16, VB = DV / 16;       // k-steps of S and dA
  constexpr int NQ = DQK / 32, NV = DV / 32;       // 32-column groups of dK and dV
  constexpr int QCH = DQK / 8, DCH = DV / 8;       // 16-byte chunks per Q / dO row
  constexpr int QI = (QCH / 2 + kKIssue - 1) / kKIssue, DI = (DCH / 2 + kKIssue - 1) / kKIssue;
  static_assert(KB <= 16, "at most one product per pair");

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int h = item_head(item);
  const int64_t seq0 = item.seq0;
  const int n = item.n;
  // the list orders tiles by query-pass cost (tile index + 1); the key pass
  // costs (tiles - key tile), so tile qt of the list is key tile tiles-1-qt
  const int ntl = (n + kAttnBM - 1) / kAttnBM;
  const int kt = ntl - 1 - item_qtile(item);
  const int k0 = kt * kAttnBM;

  __shared__ KvLds<DQK, DV> lds;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int grp = w & 3;
  const int kw = k0 + 32 * grp;   // first key of this wave's group
  const int key = kw + lr;        // this lane's key (column of S)
  const bool has_time = a.time_table != nullptr, has_pos = a.pos_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;
  // index bounds of the staged tables (a missing table is one zero entry)
  const int pos_hi = has_pos ? Bp - 1 : 0, time_nb = has_time ? min(Bt, kBwdTimeSlots) : 1;
  const BlockMeta* meta_row =
      static_cast<const BlockMeta*>(a.meta) + h * a.meta_blocks + static_cast<int64_t>(kMetaPerTile) * item.tile_base;

  // ---- prologue: every global load is issued before the first wait (a
  // work item's set-up is exposed: one workgroup fills a compute unit)
  const int qb0 = k0 / 32;                   // first query block: key group 0's diagonal
  const int nqb = (n + 31) / 32 - qb0;       // >= 1
  // a block's pairs are all masked when its last row precedes the group's first key
  auto block_active = [&](int t) __attribute__((always_inline)) { return kw < n && (qb0 + t) * 32 + 31 >= kw; };

  // K (score waves) or V (gradient waves) rows of this lane's key: the MFMA
  // B operands of S = Q K^T and dA = dO V^T
  static_assert(KB == VB, "one fragment count for both roles");
  bf16x8_t frag[KB];
  {
    const __bf16* src = w < 4 ? static_cast<const __bf16*>(a.k) + (seq0 + key) * a.ldk + h * DQK
                              : static_cast<const __bf16*>(a.v) + (seq0 + key) * a.ldv + h * DV;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      frag[kb] = key < n ? *reinterpret_cast<const bf16x8_t*>(src + kb * 16 + lh * 8) : bf16x8_t{};
  }
  const int64_t tk = (has_time && key < n) ? a.ts[seq0 + key] : 0;
  int64_t tk_min = 0, tk_max = 0;
  if (has_time && kw < n) {
    tk_min = uniform_i64(meta_row[kw / 32].tmin);
    tk_max = uniform_i64(meta_row[kw / 32].tmax);
  }
  const float pos_last = has_pos ? kLog2e * a.pos_table[h * Bp + Bp - 1] : 0.f;
  // the bias tables (up to kBwdPosMax = 2 kKThreads and kBwdTimeSlots entries)
  static_assert(kBwdPosMax <= 2 * kKThreads && kBwdTimeSlots <= kKThreads, "two table loads per thread");
  // (buffer loads, zero past the table: no branch, so the wait for them is
  // not placed right after each load)
  const __amdgpu_buffer_rsrc_t rpos = make_rsrc(has_pos ? a.pos_table + h * Bp : nullptr, has_pos ? Bp * 4 : 0);
  const __amdgpu_buffer_rsrc_t rtim = make_rsrc(has_time ? a.time_table + h * Bt : nullptr, has_time ? time_nb * 4 : 0);
  const float pos0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rpos, tid * 4, 0, 0));
  const float pos1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rpos, (tid + kKThreads) * 4, 0, 0));
  const float time0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rtim, tid * 4, 0, 0));
  // (gradient waves) the metadata of query block qb0 + lane, for the first classes
  int64_t cq_min = 0, cq_max = 0;
  if (w >= kKIssue && has_time && lane < nqb) {
    cq_min = meta_row[qb0 + lane].tmin;
    cq_max = meta_row[qb0 + lane].tmax;
  }

  // (gradient waves) the loads of the blocks in order, block t into ring
  // slot t % kKRing; the buffer descriptors advance by one block per call
  const int wi = w - kKIssue;
  uint32_t qoff[QI], doff[DI];
  const int64_t qstep = int64_t(32) * a.ldq * 2, dstep = int64_t(32) * g.lddo * 2;
  const char* qnext = static_cast<const char*>(a.q) + ((seq0 + qb0 * 32) * a.ldq + h * DQK) * 2;
  const char* dnext = static_cast<const char*>(g.d_o) + ((seq0 + qb0 * 32) * g.lddo + h * DV) * 2;
  const int64_t* tnext = has_time ? a.ts + seq0 + qb0 * 32 : nullptr;
  const BlockMeta* mnext = meta_row + qb0;
  int64_t qleft = int64_t(n - qb0 * 32) * a.ldq * 2, dleft = int64_t(n - qb0 * 32) * g.lddo * 2;
  int64_t rows_left = n - qb0 * 32, blocks_left = (n + 31) / 32 - qb0;
  int issued = 0;
  auto issue_next = [&](char* nq, char* nd, int64_t* nt, BlockMeta* nm) __attribute__((always_inline)) {
    if (issued < nqb) {
      constexpr int NQI = QCH / 2, NDI = DCH / 2;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(qnext, qleft), rd = make_rsrc(dnext, dleft);
#pragma unroll
      for (int j = 0; j < QI; ++j)
        if (wi + j * kKIssue < NQI) load_lds16(rq, nq + (wi + j * kKIssue) * 1024, qoff[j]);
#pragma unroll
      for (int j = 0; j < DI; ++j)
        if (wi + j * kKIssue < NDI) load_lds16(rd, nd + (wi + j * kKIssue) * 1024, doff[j]);
      if (wi == kKIssue - 2 && lane < 16)
        load_lds16(make_rsrc(tnext, tnext ? rows_left * 8 : 0), reinterpret_cast<char*>(nt), lane * 16);
      if (wi == kKIssue - 1 && lane < 2)
        load_lds16(make_rsrc(mnext, blocks_left * 32), reinterpret_cast<char*>(nm), lane * 16);
      qnext += qstep;
      dnext += dstep;
      qleft -= qstep;
      dleft -= dstep;
      if (tnext) tnext += 32;
      rows_left -= 32;
      ++mnext;
      --blocks_left;
      ++issued;
    }
  };
  // (gradient waves) classes of blocks [c0, c0 + 64) for this key group, one
  // block per lane (tq_min, tq_max: its query block's timestamp range), into
  // out[block - c0]
  auto classify_chunk = [&](int c0, int64_t tq_min, int64_t tq_max, const float* stime, KvClass* out)
                            __attribute__((always_inline)) {
    const int t = c0 + lane;
    if (t >= nqb) return;
    const int qa = (qb0 + t) * 32;
    const BlockClass c =
        classify_block(qa, kw, n, has_pos, Bp, has_time, Bt, tq_min, tq_max, tk_min, tk_max, pos_last, stime);
    int info = c.path | (c.tlo << 8);
    if (c.path == kBGeneral) {
      if (!has_time || time_bucket64(tq_max - tk_min, Bt) < kGFast) info |= kInfoFastTime;
      if (kw + 31 > qa || qa + 31 >= n || kw + 31 >= n) info |= kInfoMasked;
      if (!has_time || (tq_max - tk_min <= int64_t(INT32_MAX) - 1 && tq_min - tk_max >= int64_t(INT32_MIN)))
        info |= kInfoNarrow;
    }
    out[lane] = KvClass{info, c.clo, c.chi, 0};
  };

  if (w >= kKIssue) {
    block_load_offsets<QCH>(wi, lane, a.ldq, qoff);
    block_load_offsets<DCH>(wi, lane, g.lddo, doff);
    issue_next(lds.q[0], lds.d[0], lds.t[0], &lds.m[0]);
    issue_next(lds.q[1], lds.d[1], lds.t[1], &lds.m[1]);
  }
  for (int i = tid; i < 4 * kBwdPosMax; i += kKThreads) (&lds.gpos[0][0])[i] = 0.f;
  for (int i = tid; i < 4 * kGFast * 64; i += kKThreads) (&lds.gtime[0][0][0])[i] = 0.f;
  for (int i = tid; i < 4 * kBwdTimeSlots; i += kKThreads) (&lds.gslow[0][0])[i] = 0.f;
  wait_vmcnt(0);
  if (tid <= pos_hi) lds.pos[tid] = kLog2e * pos0;   // one 0 without the table
  if (tid + kKThreads <= pos_hi) lds.pos[tid + kKThreads] = kLog2e * pos1;
  if (tid < time_nb) lds.time[tid] = kLog2e * time0;
  __syncthreads();   // the staged tables (read by the classification)
  if (w >= kKIssue) classify_chunk(0, cq_min, cq_max, lds.time, &lds.cls[0][grp][0]);
  __syncthreads();   // also publishes the first classes and the zeroed gradient tables

  const float inv_n = a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n);

  if (w < 4) {
    // ======================= score wave =======================
    const bf16x8_t* kf = frag;
    const float alpha_l = a.alpha * kLog2e;
    uint32_t q_row[KB], d_tr0[NV], d_tr1[NV];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) q_row[kb] = row_read_offset<QCH>(lr, lh, kb);
#pragma unroll
    for (int nb = 0; nb < NV; ++nb) tr_read_offsets<DCH>(lane, nb, d_tr0[nb], d_tr1[nb]);
    f32x16_t dva[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) dva[i] = f32x16_t{};
    // S of block t (computed one step earlier)
    f32x16_t s_cur = f32x16_t{};

    // One block per step. The products of S of block t + 1 are spread over
    // the per-pair loop, one after each pair, so they run under the
    // arithmetic (an unused S past the sequence or when block t + 1 is masked
    // entirely); dV += P^T dO of block t follows the loop. Every LDS buffer
    // comes in through a __restrict__ parameter, so the compiler does not
    // wait for the loads in flight before reading LDS.
    auto step = [&](const char* __restrict__ rq1, const char* __restrict__ rd, const int64_t* __restrict__ rt,
                    const KvClass* __restrict__ rc, f16x8_t* __restrict__ xg, u32x4_t* __restrict__ xb,
                    const float* __restrict__ spos, const float* __restrict__ stime, int t)
                    __attribute__((always_inline)) {
      const f32x16_t s = s_cur;
      f32x16_t sn = f32x16_t{};
      auto mf = [&](int k) __attribute__((always_inline)) {
        if (k < KB) {
          const bf16x8_t qf = *reinterpret_cast<const bf16x8_t*>(rq1 + q_row[k]);
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[k], sn, 0, 0, 0);
        }
      };
      if (!block_active(t)) {
#pragma unroll
        for (int k = 0; k < KB; ++k) mf(k);
        s_cur = sn;
        return;
      }
      const int qa = (qb0 + t) * 32;
      // s[4g+e]: query row qa + 8g + 4lh + e, key `key`
      const int info = __builtin_amdgcn_readfirstlane(rc->info);
      const int path = info & 3, tlo = (info >> 8) & 255;
      const float clo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rc->clo)));
      const float chi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rc->chi)));
      // per pair r: SiLU' (fp16) and P (bf16) packed eight at a time, the
      // time bucket into byte r % 4 of word r / 4
      bf16x8_t pa[2];
      f16x8_t gq;
      u32x4_t tw = u32x4_t{0u, 0u, 0u, 0u};
      auto emit = [&](int r, float pl, float dl) __attribute__((always_inline)) {
        pa[r >> 3][r & 7] = static_cast<__bf16>(pl);
        gq[r & 7] = static_cast<_Float16>(dl);
        if ((r & 7) == 7) xg[(r >> 3) * 64 + lane] = gq;
      };
      auto emit_tb = [&](int r, int tbr) __attribute__((always_inline)) {
        tw[r >> 2] |= static_cast<uint32_t>(tbr) << (8 * (r & 3));
      };
      // the pairs of a block with varying position buckets or a mask: a
      // bucket per pair, the time bucket from the timestamps' low words when
      // the block's gaps fit in int32 (zero tables stand in for missing ones)
      auto general = [&](auto masked_c, auto narrow_c) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value, NARROW = decltype(narrow_c)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 8 * (r >> 2) + 4 * lh + (r & 3);
          const int i = qa + il, d = i - key;
          int tbr;
          if constexpr (NARROW) tbr = time_bucket_narrow(rt[il], tk, time_nb);
          else tbr = time_bucket64(rt[il] - tk, time_nb);
          const int pb = MASKED ? min(max(d, 0), pos_hi) : min(d, pos_hi);
          float pl, dl;
          silu_and_grad(fmaf(s[r], alpha_l, spos[pb] + stime[tbr]), pl, dl);
          if constexpr (MASKED) {
            const bool valid = d >= 0 && i < n && key < n;
            emit(r, valid ? pl : 0.f, valid ? dl : 0.f);
            // a masked pair adds 0 to bucket 0: a key past the sequence end
            // reads timestamp 0, and its bucket is not bounded by the block's
            emit_tb(r, valid ? tbr : 0);
          } else {
            emit(r, pl, dl);
            emit_tb(r, tbr);
          }
          mf(r);
        }
      };
      if (path == kBUniform) {
        // one bias for every pair; the gradient wave needs no buckets
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pl, dl;
          silu_and_grad(fmaf(s[r], alpha_l, clo), pl, dl);
          emit(r, pl, dl);
          mf(r);
        }
      } else if (path == kBTwoTime) {
        const int64_t lim = tk + ((int64_t(1) << (tlo + 1)) - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool hi = rt[il] >= lim;
          float pl, dl;
          silu_and_grad(fmaf(s[r], alpha_l, hi ? chi : clo), pl, dl);
          emit(r, pl, dl);
          emit_tb(r, tlo + (hi ? 1 : 0));
          mf(r);
        }
      } else if (!(info & kInfoMasked) && (info & kInfoNarrow)) {
        general(std::false_type{}, std::true_type{});
      } else if (info & kInfoNarrow) {
        general(std::true_type{}, std::true_type{});
      } else {
        general(std::true_type{}, std::false_type{});
      }
      if (path != kBUniform) xb[lane] = tw;
      // dV += P^T dO over the block's 32 query rows (two 16-row steps)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const char* dst = rd + kk * 16 * DCH * 16;
        bf16x8_t ob[NV];   // every fragment of the step read before the first product
#pragma unroll
        for (int nb = 0; nb < NV; ++nb)
          ob[nb] = __builtin_shufflevector(tr_read(dst + d_tr0[nb]), tr_read(dst + d_tr1[nb]), 0, 1, 2, 3, 4, 5, 6, 7);
        __builtin_amdgcn_sched_barrier(0);   // keeps the reads ahead: the scheduler sank each to its product
#pragma unroll
        for (int nb = 0; nb < NV; ++nb) dva[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], ob[nb], dva[nb], 0, 0, 0);
      }
      s_cur = sn;
    };

    if (block_active(0)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(lds.q[0] + q_row[kb]),
                                                        kf[kb], s_cur, 0, 0, 0);
    }
    for (int t = 0; t < nqb; ++t) {
      const int sl = t % kKRing;
      step(lds.q[(t + 1) % kKRing], lds.d[sl], lds.t[sl], &lds.cls[(t >> 6) & 1][grp][t & 63], &lds.xg[t & 1][grp][0][0],
           &lds.xb[t & 1][grp][0], lds.pos, lds.time, t);
      tile_barrier();
    }

    // ---- dV: accumulator [i][r] holds key kw + 8(r/4) + 4 lh + r%4, column 32 i + lr
    const float sv = inv_n / kLog2e;
    __bf16* dvp = static_cast<__bf16*>(g.dv) + (seq0 + kw) * g.lddv + h * DV + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * lh + (r & 3);
      if (kw + kr < n) {
#pragma unroll
        for (int nb = 0; nb < NV; ++nb) dvp[kr * g.lddv + nb * 32] = static_cast<__bf16>(dva[nb][r] * sv);
      }
    }
  } else {
    // ====================== gradient wave ======================
    const bf16x8_t* vf = frag;
    uint32_t d_row[VB], q_tr0[NQ], q_tr1[NQ];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) d_row[vb] = row_read_offset<DCH>(lr, lh, vb);
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb) tr_read_offsets<QCH>(lane, nb, q_tr0[nb], q_tr1[nb]);
    f32x16_t dka[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) dka[i] = f32x16_t{};
    float far_acc = 0.f;   // dS' of the pairs that read position bucket Bp - 1
    float* gpos = lds.gpos[grp];
    float* gtime = &lds.gtime[grp][0][lane];
    float* gslow = lds.gslow[grp];

    // Step t: the loads of block t + 2, at t = 64 k + 1 the classes of blocks
    // [64 (k + 1), 64 (k + 2)) (into the table half that held blocks
    // [64 (k - 1), 64 k), whose last reader was step 64 k), then block t - 1
    // (its SiLU' was written before
    // the last barrier): dA, dS, the gradient-table updates and dK. Every LDS
    // buffer comes in through a __restrict__ parameter (as in the score
    // wave's step).
    auto step = [&](const char* __restrict__ rd, const char* __restrict__ rq, const f16x8_t* __restrict__ xg,
                    const u32x4_t* __restrict__ xb, const KvClass* __restrict__ rc, KvClass* __restrict__ wc,
                    char* __restrict__ nq, char* __restrict__ nd, int64_t* __restrict__ nt,
                    BlockMeta* __restrict__ nm, const float* __restrict__ stime, float* __restrict__ gp,
                    float* __restrict__ gt, float* __restrict__ gsl, int t) __attribute__((always_inline)) {
      issue_next(nq, nd, nt, nm);
      if ((t & 63) == 1 && t + 63 < nqb) {
        int64_t q_min = 0, q_max = 0;
        if (has_time && t + 63 + lane < nqb) {
          q_min = meta_row[qb0 + t + 63 + lane].tmin;
          q_max = meta_row[qb0 + t + 63 + lane].tmax;
        }
        classify_chunk(t + 63, q_min, q_max, stime, wc);
      }
      const int tb_ = t - 1;
      if (tb_ < 0 || !block_active(tb_)) return;
      const int qa = (qb0 + tb_) * 32;
      bf16x8_t dfr[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) dfr[vb] = *reinterpret_cast<const bf16x8_t*>(rd + d_row[vb]);
      f32x16_t da = f32x16_t{};
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr[vb], vf[vb], da, 0, 0, 0);
      const int info = __builtin_amdgcn_readfirstlane(rc->info);
      const int path = info & 3, tlo = (info >> 8) & 255;
      float ds[16];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const f16x8_t v = xg[h8 * 64 + lane];
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[8 * h8 + e] = da[8 * h8 + e] * static_cast<float>(v[e]);
      }
      if (g.grad_stride > 0) {
        if (path == kBUniform) {
          // every pair reads position bucket Bp - 1 and time bucket tlo
          float sl = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) sl += ds[r];
          if (has_pos) far_acc += sl;
          if (has_time) {
            if (tlo < kGFast) {
              gt[64 * tlo] += sl;
            } else {
              const float s0 = wave_sum(sl);
              if (lane == 0) gsl[tlo] += s0;
            }
          }
        } else if (path == kBTwoTime) {
          // every pair reads position bucket Bp - 1 and time bucket tlo or tlo + 1
          const u32x4_t tw = xb[lane];
          float slo = 0.f, shi = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool hi = ((tw[r >> 2] >> (8 * (r & 3))) & 255) != static_cast<uint32_t>(tlo);
            slo += hi ? 0.f : ds[r];
            shi += hi ? ds[r] : 0.f;
          }
          if (has_pos) far_acc += slo + shi;
          if (has_time) {
            if (tlo + 1 < kGFast) {
              gt[64 * tlo] += slo;
              gt[64 * (tlo + 1)] += shi;
            } else {
              const float s0 = wave_sum(slo), s1 = wave_sum(shi);
              if (lane == 0) {
                gsl[tlo] += s0;
                gsl[tlo + 1] += s1;
              }
            }
          }
        } else {
          const u32x4_t tw = xb[lane];
          if (has_time) {
            if (info & kInfoFastTime) {
#pragma unroll
              for (int r = 0; r < 16; ++r) gt[64 * ((tw[r >> 2] >> (8 * (r & 3))) & 255)] += ds[r];
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int tbr = (tw[r >> 2] >> (8 * (r & 3))) & 255;
                if (tbr < kGFast) gt[64 * tbr] += ds[r];
                else lds_add_f32(&gsl[tbr], ds[r]);
              }
            }
          }
          // position buckets: a valid pair of the block reads bucket
          // min(i - key, Bp - 1) = min(qa - kw + d, Bp - 1) with d = i' - lr
          // its diagonal (masked pairs hold dS = 0)
          if (has_pos) {
            if (qa - (kw + 31) >= Bp - 1) {
#pragma unroll
              for (int r = 0; r < 16; ++r) far_acc += ds[r];
            } else {
              float dpos, dneg;
              diagonal_sums(ds, lr, lh, dpos, dneg);
              if (lh == 0) {
                const int bpos = qa - kw + lr, bneg = bpos - 32;
                if (bpos < Bp - 1) gp[bpos] += dpos;
                else far_acc += dpos;
                if (bneg >= Bp - 1) far_acc += dneg;
                else if (bneg >= 0) gp[bneg] += dneg;
              }
            }
          }
        }
      }
      // dK += dS^T Q over the block's 32 query rows (two 16-row steps)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t sa;
#pragma unroll
        for (int i = 0; i < 8; ++i) sa[i] = static_cast<__bf16>(ds[kk * 8 + i]);
        const char* qst = rq + kk * 16 * QCH * 16;
        bf16x8_t qt[NQ];   // every fragment of the step read before the first product
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb)
          qt[nb] = __builtin_shufflevector(tr_read(qst + q_tr0[nb]), tr_read(qst + q_tr1[nb]), 0, 1, 2, 3, 4, 5, 6, 7);
        __builtin_amdgcn_sched_barrier(0);   // keeps the reads ahead: the scheduler sank each to its product
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) dka[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, qt[nb], dka[nb], 0, 0, 0);
      }
    };

    for (int t = 0; t <= nqb; ++t) {
      // slots: block t - 1 (dO, Q), t + 2 (loads)
      const int pv = (t + kKRing - 1) % kKRing, n2 = (t + 2) % kKRing;
      const int tp = t > 0 ? t - 1 : 0;
      step(lds.d[pv], lds.q[pv], &lds.xg[(t + 1) & 1][grp][0][0], &lds.xb[(t + 1) & 1][grp][0],
           &lds.cls[(tp >> 6) & 1][grp][tp & 63], &lds.cls[((t >> 6) + 1) & 1][grp][0], lds.q[n2], lds.d[n2],
           lds.t[n2], &lds.m[n2], lds.time, gpos, gtime, gslow, t);
      wait_vmcnt(0);
      if (t < nqb) tile_barrier();
    }

    // ---- dK: accumulator [i][r] holds key kw + 8(r/4) + 4 lh + r%4, column 32 i + lr
    const float sk = a.alpha * inv_n;
    __bf16* dkp = static_cast<__bf16*>(g.dk) + (seq0 + kw) * g.lddk + h * DQK + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * lh + (r & 3);
      if (kw + kr < n) {
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) dkp[kr * g.lddk + nb * 32] = static_cast<__bf16>(dka[nb][r] * sk);
      }
    }
    if (g.grad_stride > 0 && has_pos) {
      const float f = wave_sum(far_acc);
      if (lane == 0) gpos[Bp - 1] += f;
    }
  }

  // ---- bias-table gradients of this key tile
  if (g.grad_stride > 0) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the asm adds have landed
    __syncthreads();
    float* prow = g.partial + (static_cast<int64_t>(h) * g.tile_rows + item.tile_base + kt) * g.grad_stride;
    if (has_pos)
      for (int i = tid; i < Bp; i += kKThreads) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) s += lds.gpos[ww][i];
        prow[i] = s * inv_n;
      }
    if (has_time) {
      // bucket tid / 8: thread part = tid % 8 sums half part % 2 of gradient
      // wave part / 2's lane columns, then the 8 threads (adjacent lanes)
      // combine in a fixed order
      static_assert(kKThreads == 8 * kBwdTimeSlots, "one bucket per 8 threads");
      float* trow = prow + (has_pos ? Bp : 0);
      const int tb = tid >> 3, part = tid & 7, ww = part >> 1, half = part & 1;
      float s = 0.f;
      if (tb < kGFast) {
        const f32x4_t* col = reinterpret_cast<const f32x4_t*>(&lds.gtime[ww][tb][half * 32]);
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
          const f32x4_t v4 = col[c4];
          s += (v4[0] + v4[1]) + (v4[2] + v4[3]);
        }
      }
      if (half == 0) s += lds.gslow[ww][tb];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (part == 0) trow[tb] = s * inv_n;
    }
  }
}

// ============================================================================
// query pass: dQ
//
// A work item owns 128 query rows and walks the 32-key blocks from the
// sequence start to its last row. Waves w and w + 4 run on one SIMD and share
// a group of 32 query rows (qa = q0 + 32 (w & 3), one query per lane as the
// column of S^T), in two roles as in the key pass:
//   score wave (w < 4)      S^T = K Q^T one block ahead (its products spread
//                           over the current block's per-pair loop), the bias
//                           and SiLU'(x) of every pair (masked pairs: 0);
//   gradient wave (w >= 4)  the tile loads, the block classes (64 blocks at a
//                           time, one per lane), and one block behind the
//                           score wave: dA^T = V dO^T, dS = dA SiLU'(x) and
//                           dQ += dS K.
// SiLU'(x) passes through LDS as fp16. Q (score) and dO (gradient) of the
// lane's query stay in registers as MFMA B operands; K, V and the key
// timestamps of block t + 2 load into a ring of four LDS
// slots while block t is processed, one barrier per block.
// ============================================================================
template <int DQK, int DV>
struct QLds {
  __attribute__((aligned(16))) char k[kKRing][32 * DQK * 2];
  __attribute__((aligned(16))) char v[kKRing][32 * DV * 2];
  __attribute__((aligned(16))) int64_t t[kKRing][32];
  f16x8_t xg[2][4][2][64];      // SiLU' of a block: [buffer][query group][r / 8][lane]
  KvClass cls[2][4][64];        // [(block / 64) % 2][query group][block % 64]
  float pos[kBwdPosMax];        // log2(e) P[h][.] (one 0 without the table)
  float time[kBwdTimeSlots];    // log2(e) Tt[h][.] (one 0 without the table)
};

template <int DQK, int DV>
__global__ __launch_bounds__(kKThreads, 1) void attn_bwd_q_kernel(AttnBwdArgs g) {
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  const AttnArgs& a = g.f;
  constexpr int KB = DQK / 16, VB = DV / 16;       // k-steps of S^T and dA^T
  constexpr int NQ = DQK / 32;                     // 32-column groups of dQ
  constexpr int KCH = DQK / 8, VCH = DV / 8;       // 16-byte chunks per K / V row
  constexpr int KI = (KCH / 2 + kKIssue - 1) / kKIssue, VI = (VCH / 2 + kKIssue - 1) / kKIssue;
  static_assert(KB <= 16 && KB == VB, "at most one product per pair; one fragment count for both roles");

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = item.seq0;
  const int n = item.n;
  const int q0 = qt * kAttnBM;

  __shared__ QLds<DQK, DV> lds;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int grp = w & 3;
  const int qa = q0 + 32 * grp;   // first query row of this wave's group
  const int qrow = qa + lr;       // this lane's query (column of S^T)
  const bool has_time = a.time_table != nullptr, has_pos = a.pos_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;
  const int pos_hi = has_pos ? Bp - 1 : 0, time_nb = has_time ? min(Bt, kBwdTimeSlots) : 1;
  const BlockMeta* meta_row =
      static_cast<const BlockMeta*>(a.meta) + h * a.meta_blocks + static_cast<int64_t>(kMetaPerTile) * item.tile_base;

  // ---- prologue: every global load is issued before the first wait
  const int kv_end = min(n, q0 + kAttnBM);
  const int nkb = (kv_end + 31) / 32;        // key blocks of the walk (>= 1)
  // a block's pairs are all masked when its first key follows the group's last row
  auto block_active = [&](int t) __attribute__((always_inline)) { return qa < n && 32 * t <= qa + 31; };

  // Q (score waves) or dO (gradient waves) row of this lane's query: the MFMA
  // B operands of S^T = K Q^T and dA^T = V dO^T
  bf16x8_t frag[KB];
  {
    const __bf16* src = w < 4 ? static_cast<const __bf16*>(a.q) + (seq0 + qrow) * a.ldq + h * DQK
                              : static_cast<const __bf16*>(g.d_o) + (seq0 + qrow) * g.lddo + h * DV;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      frag[kb] = qrow < n ? *reinterpret_cast<const bf16x8_t*>(src + kb * 16 + lh * 8) : bf16x8_t{};
  }
  const int64_t tq = (has_time && qrow < n) ? a.ts[seq0 + qrow] : 0;
  int64_t tq_min = 0, tq_max = 0;
  if (has_time && qa < n) {
    tq_min = uniform_i64(meta_row[qa / 32].tmin);
    tq_max = uniform_i64(meta_row[qa / 32].tmax);
  }
  const float pos_last = has_pos ? kLog2e * a.pos_table[h * Bp + Bp - 1] : 0.f;
  static_assert(kBwdPosMax <= 2 * kKThreads && kBwdTimeSlots <= kKThreads, "two table loads per thread");
  const __amdgpu_buffer_rsrc_t rpos = make_rsrc(has_pos ? a.pos_table + h * Bp : nullptr, has_pos ? Bp * 4 : 0);
  const __amdgpu_buffer_rsrc_t rtim = make_rsrc(has_time ? a.time_table + h * Bt : nullptr, has_time ? time_nb * 4 : 0);
  const float pos0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rpos, tid * 4, 0, 0));
  const float pos1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rpos, (tid + kKThreads) * 4, 0, 0));
  const float time0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rtim, tid * 4, 0, 0));
  // (gradient waves) the metadata of key block lane, for the first classes
  int64_t ck_min = 0, ck_max = 0;
  if (w >= kKIssue && has_time && lane < nkb) {
    ck_min = meta_row[lane].tmin;
    ck_max = meta_row[lane].tmax;
  }

  // (gradient waves) the loads of the key blocks in order, block t into ring
  // slot t % kKRing; the buffer descriptors advance by one block per call
  const int wi = w - kKIssue;
  uint32_t koff[KI], voff[VI];
  const int64_t kstep = int64_t(32) * a.ldk * 2, vstep = int64_t(32) * a.ldv * 2;
  const char* knext = static_cast<const char*>(a.k) + (seq0 * a.ldk + h * DQK) * 2;
  const char* vnext = static_cast<const char*>(a.v) + (seq0 * a.ldv + h * DV) * 2;
  const int64_t* tnext = has_time ? a.ts + seq0 : nullptr;
  int64_t kleft = int64_t(n) * a.ldk * 2, vleft = int64_t(n) * a.ldv * 2;
  int64_t rows_left = n;
  int issued = 0;
  auto issue_next = [&](char* nk, char* nv, int64_t* nt) __attribute__((always_inline)) {
    if (issued < nkb) {
      constexpr int NKI = KCH / 2, NVI = VCH / 2;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(knext, kleft), rv = make_rsrc(vnext, vleft);
#pragma unroll
      for (int j = 0; j < KI; ++j)
        if (wi + j * kKIssue < NKI) load_lds16(rk, nk + (wi + j * kKIssue) * 1024, koff[j]);
#pragma unroll
      for (int j = 0; j < VI; ++j)
        if (wi + j * kKIssue < NVI) load_lds16(rv, nv + (wi + j * kKIssue) * 1024, voff[j]);
      if (wi == kKIssue - 2 && lane < 16)
        load_lds16(make_rsrc(tnext, tnext ? rows_left * 8 : 0), reinterpret_cast<char*>(nt), lane * 16);
      knext += kstep;
      vnext += vstep;
      kleft -= kstep;
      vleft -= vstep;
      if (tnext) tnext += 32;
      rows_left -= 32;
      ++issued;
    }
  };
  // (gradient waves) classes of key blocks [c0, c0 + 64) for this query
  // group, one block per lane (tk_min, tk_max: its timestamp range), into
  // out[block - c0]
  auto classify_chunk = [&](int c0, int64_t tk_min, int64_t tk_max, const float* stime, KvClass* out)
                            __attribute__((always_inline)) {
    const int t = c0 + lane;
    if (t >= nkb) return;
    const int ka = 32 * t;
    const BlockClass c =
        classify_block(qa, ka, n, has_pos, Bp, has_time, Bt, tq_min, tq_max, tk_min, tk_max, pos_last, stime);
    int info = c.path | (c.tlo << 8);
    if (c.path == kBGeneral) {
      if (ka + 31 > qa || qa + 31 >= n || ka + 31 >= n) info |= kInfoMasked;
      if (!has_time || (tq_max - tk_min <= int64_t(INT32_MAX) - 1 && tq_min - tk_max >= int64_t(INT32_MIN)))
        info |= kInfoNarrow;
    }
    out[lane] = KvClass{info, c.clo, c.chi, 0};
  };

  if (w >= kKIssue) {
    block_load_offsets<KCH>(wi, lane, a.ldk, koff);
    block_load_offsets<VCH>(wi, lane, a.ldv, voff);
    issue_next(lds.k[0], lds.v[0], lds.t[0]);
    issue_next(lds.k[1], lds.v[1], lds.t[1]);
  }
  wait_vmcnt(0);
  if (tid <= pos_hi) lds.pos[tid] = kLog2e * pos0;   // one 0 without the table
  if (tid + kKThreads <= pos_hi) lds.pos[tid + kKThreads] = kLog2e * pos1;
  if (tid < time_nb) lds.time[tid] = kLog2e * time0;
  __syncthreads();   // the staged tables (read by the classification)
  if (w >= kKIssue) classify_chunk(0, ck_min, ck_max, lds.time, &lds.cls[0][grp][0]);
  __syncthreads();   // also publishes the first classes

  if (w < 4) {
    // ======================= score wave =======================
    const bf16x8_t* qf = frag;
    const float alpha_l = a.alpha * kLog2e;
    uint32_t k_row[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) k_row[kb] = row_read_offset<KCH>(lr, lh, kb);
    // S^T of block t (computed one step earlier)
    f32x16_t s_cur = f32x16_t{};

    // One block per step; the products of S^T of block t + 1 (unused past
    // the walk or when block t + 1 is masked entirely) are spread over the
    // per-pair loop; a block masked entirely ends the wave's work. Every LDS buffer comes in through a __restrict__
    // parameter, so the compiler does not wait for the loads in flight.
    auto step = [&](const char* __restrict__ rk1, const int64_t* __restrict__ rt, const KvClass* __restrict__ rc,
                    f16x8_t* __restrict__ xg, const float* __restrict__ spos, const float* __restrict__ stime,
                    int t) __attribute__((always_inline)) {
      const f32x16_t s = s_cur;
      f32x16_t sn = f32x16_t{};
      auto mf = [&](int k) __attribute__((always_inline)) {
        if (k < KB) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(rk1 + k_row[k]);
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], sn, 0, 0, 0);
        }
      };
      if (!block_active(t)) return;   // and every later block
      const int ka = 32 * t;
      // s[4g+e]: key ka + 8g + 4lh + e, query qrow
      const int info = __builtin_amdgcn_readfirstlane(rc->info);
      const int path = info & 3, tlo = (info >> 8) & 255;
      const float clo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rc->clo)));
      const float chi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rc->chi)));
      // SiLU' (fp16) packed eight at a time
      f16x8_t gq;
      auto emit = [&](int r, float dl) __attribute__((always_inline)) {
        gq[r & 7] = static_cast<_Float16>(dl);
        if ((r & 7) == 7) xg[(r >> 3) * 64 + lane] = gq;
      };
      // pairs with varying position buckets or a mask: a bucket per pair, the
      // time bucket from the timestamps' low words when the block's gaps fit
      // in int32 (zero tables stand in for missing ones)
      auto general = [&](auto masked_c, auto narrow_c) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value, NARROW = decltype(narrow_c)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 8 * (r >> 2) + 4 * lh + (r & 3);
          const int kv = ka + il, d = qrow - kv;
          int tbr;
          if constexpr (NARROW) tbr = time_bucket_narrow(tq, rt[il], time_nb);
          else tbr = time_bucket64(tq - rt[il], time_nb);
          const int pb = MASKED ? min(max(d, 0), pos_hi) : min(d, pos_hi);
          float pl, dl;
          silu_and_grad(fmaf(s[r], alpha_l, spos[pb] + stime[tbr]), pl, dl);
          if constexpr (MASKED) {
            // the mask is opaque to the compiler, which otherwise moved each
            // pair's bucket lookups and SiLU' into a branch of its own (one
            // exec-masked region per pair, its LDS reads serialised)
            int keep = (d >= 0 && kv < n && qrow < n) ? -1 : 0;
            asm("" : "+v"(keep));
            emit(r, __int_as_float(__float_as_int(dl) & keep));
          } else {
            emit(r, dl);
          }
          mf(r);
        }
      };
      if (path == kBUniform) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pl, dl;
          silu_and_grad(fmaf(s[r], alpha_l, clo), pl, dl);
          emit(r, dl);
          mf(r);
        }
      } else if (path == kBTwoTime) {
        // the key's timestamp at most tq - (2^(tlo+1) - 1): bucket tlo + 1
        const int64_t lim = tq - ((int64_t(1) << (tlo + 1)) - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool hi = rt[il] <= lim;
          float pl, dl;
          silu_and_grad(fmaf(s[r], alpha_l, hi ? chi : clo), pl, dl);
          emit(r, dl);
          mf(r);
        }
      } else if (!(info & kInfoMasked) && (info & kInfoNarrow)) {
        general(std::false_type{}, std::true_type{});
      } else if (info & kInfoNarrow) {
        general(std::true_type{}, std::true_type{});
      } else {
        general(std::true_type{}, std::false_type{});
      }
      s_cur = sn;
    };

    if (block_active(0)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(lds.k[0] + k_row[kb]),
                                                        qf[kb], s_cur, 0, 0, 0);
    }
    for (int t = 0; t < nkb; ++t) {
      step(lds.k[(t + 1) % kKRing], lds.t[t % kKRing], &lds.cls[(t >> 6) & 1][grp][t & 63],
           &lds.xg[t & 1][grp][0][0], lds.pos, lds.time, t);
      tile_barrier();
    }
  } else {
    // ====================== gradient wave ======================
    const bf16x8_t* df = frag;
    uint32_t v_row[VB], k_tr0[NQ], k_tr1[NQ];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) v_row[vb] = row_read_offset<VCH>(lr, lh, vb);
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb) tr_read_offsets<KCH>(lane, nb, k_tr0[nb], k_tr1[nb]);
    f32x16_t dqa[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) dqa[i] = f32x16_t{};

    // Step t: the loads of block t + 2, at t = 64 k + 1 the classes of blocks
    // [64 (k + 1), 64 (k + 2)) (into the table half whose last reader was
    // step 64 k), then block t - 1 (its SiLU' was written before the last
    // barrier): dA^T, dS and dQ += dS K. Every LDS buffer comes in through a
    // __restrict__ parameter (as in the score wave's step).
    auto step = [&](const char* __restrict__ rk, const char* __restrict__ rv, const f16x8_t* __restrict__ xg,
                    KvClass* __restrict__ wc, char* __restrict__ nk, char* __restrict__ nv,
                    int64_t* __restrict__ nt, const float* __restrict__ stime,
                    int t) __attribute__((always_inline)) {
      issue_next(nk, nv, nt);
      if ((t & 63) == 1 && t + 63 < nkb) {
        int64_t k_min = 0, k_max = 0;
        if (has_time && t + 63 + lane < nkb) {
          k_min = meta_row[t + 63 + lane].tmin;
          k_max = meta_row[t + 63 + lane].tmax;
        }
        classify_chunk(t + 63, k_min, k_max, stime, wc);
      }
      const int tb_ = t - 1;
      if (tb_ < 0 || !block_active(tb_)) return;
      bf16x8_t vfr[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) vfr[vb] = *reinterpret_cast<const bf16x8_t*>(rv + v_row[vb]);
      f32x16_t da = f32x16_t{};
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[vb], df[vb], da, 0, 0, 0);
      // dQ += dS K over the block's 32 keys (two 16-key steps)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8_t gv = xg[kk * 64 + lane];
        bf16x8_t sa;
#pragma unroll
        for (int i = 0; i < 8; ++i) sa[i] = static_cast<__bf16>(da[kk * 8 + i] * static_cast<float>(gv[i]));
        const char* kst = rk + kk * 16 * KCH * 16;
        bf16x8_t kb16[NQ];   // every fragment of the step read before the first product
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb)
          kb16[nb] = __builtin_shufflevector(tr_read(kst + k_tr0[nb]), tr_read(kst + k_tr1[nb]), 0, 1, 2, 3, 4, 5, 6, 7);
        __builtin_amdgcn_sched_barrier(0);   // keeps the reads ahead: the scheduler sank each to its product
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) dqa[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, kb16[nb], dqa[nb], 0, 0, 0);
      }
    };

    for (int t = 0; t <= nkb; ++t) {
      // slots: block t - 1 (K, V), t + 2 (loads)
      const int pv = (t + kKRing - 1) % kKRing, n2 = (t + 2) % kKRing;
      step(lds.k[pv], lds.v[pv], &lds.xg[(t + 1) & 1][grp][0][0], &lds.cls[((t >> 6) + 1) & 1][grp][0], lds.k[n2],
           lds.v[n2], lds.t[n2], lds.time, t);
      wait_vmcnt(0);
      if (t < nkb) tile_barrier();
    }

    // ---- dQ: accumulator [i][r] holds query qa + 8(r/4) + 4 lh + r%4, column 32 i + lr
    const float inv_n = a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n);
    const float sq = a.alpha * inv_n;
    __bf16* dqp = static_cast<__bf16*>(g.dq) + (seq0 + qa) * g.lddq + h * DQK + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = 8 * (r >> 2) + 4 * lh + (r & 3);
      if (qa + qr < n) {
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) dqp[qr * g.lddq + nb * 32] = static_cast<__bf16>(dqa[nb][r] * sq);
      }
    }
  }
}

// ============================================================================
// bias-table gradients: per-head sums of the key tiles' partial rows. One
// workgroup per (64 consecutive partial-row slots, head): lane l of wave g
// sums slot l over tiles g, g + 16, g + 32, ... (four independent chains),
// then wave 0 adds the 16 group sums in order -- a fixed summation order.
// ============================================================================
constexpr int kReduceGroups = 16;

__global__ __launch_bounds__(kReduceGroups * 64) void attn_bwd_bias_reduce_kernel(AttnBwdArgs g) {
  const AttnArgs& a = g.f;
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int slot = blockIdx.x * 64 + lane;
  const int tiles = a.tile_base[g.num_seqs];
  const int stride = g.grad_stride;
  // time buckets past the reachable ones (>= kBwdTimeSlots) receive no pair
  if (blockIdx.x == 0 && g.d_time)
    for (int j = kBwdTimeSlots + threadIdx.x; j < a.time_buckets; j += blockDim.x)
      g.d_time[h * a.time_buckets + j] = 0.f;
  const float* col = g.partial + static_cast<int64_t>(h) * g.tile_rows * stride + slot;
  __shared__ float part[kReduceGroups][64];
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  if (slot < stride) {
    int t = grp;
    for (; t + 3 * kReduceGroups < tiles; t += 4 * kReduceGroups) {
      s0 += col[static_cast<int64_t>(t) * stride];
      s1 += col[static_cast<int64_t>(t + kReduceGroups) * stride];
      s2 += col[static_cast<int64_t>(t + 2 * kReduceGroups) * stride];
      s3 += col[static_cast<int64_t>(t + 3 * kReduceGroups) * stride];
    }
    for (; t < tiles; t += kReduceGroups) s0 += col[static_cast<int64_t>(t) * stride];
  }
  part[grp][lane] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  if (grp != 0 || slot >= stride) return;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kReduceGroups; ++i) s += part[i][lane];
  const int Bp = a.pos_buckets, Bt = a.time_buckets;
  const int pos_slots = g.d_pos ? Bp : 0;
  if (slot < pos_slots) {
    g.d_pos[h * Bp + slot] = s;
  } else if (g.d_time) {
    const int tb = slot - pos_slots;   // < kBwdTimeSlots
    if (tb < Bt) g.d_time[h * Bt + tb] = s;
  }
}

template <typename K>
hipError_t launch_bwd_items(K kernel, int threads, const AttnBwdArgs& g, hipStream_t stream) {
  if (g.f.capacity <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(g.f.capacity)), dim3(threads), 0, stream, g);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_dims(const AttnBwdArgs& g, hipStream_t stream) {
  hipError_t e;
  {
    TimedScope timed(kTimedAttnBwdKv, stream);
    e = launch_bwd_items(attn_bwd_kv_kernel<D, D>, kKThreads, g, stream);
  }
  if (e != hipSuccess) return e;
  {
    TimedScope timed(kTimedAttnBwdQ, stream);
    e = launch_bwd_items(attn_bwd_q_kernel<D, D>, kKThreads, g, stream);
  }
  if (e != hipSuccess) return e;
  if (g.grad_stride > 0) {
    hipLaunchKernelGGL(attn_bwd_bias_reduce_kernel,
                       dim3(static_cast<unsigned>((g.grad_stride + 63) / 64), static_cast<unsigned>(g.f.num_heads)),
                       dim3(kReduceGroups * 64), 0, stream, g);
    e = hipGetLastError();
  }
  return e;
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* x, int64_t n, float value) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) x[i] = value;
}

}  // namespace

hipError_t launch_fill_f32(float* x, int64_t n, float value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     stream, x, n, value);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& g, int dqk, int dv, hipStream_t stream) {
  if (dqk != dv) return hipErrorInvalidValue;
  hipError_t e = launch_attn_block_meta(g.f, dqk, stream);
  if (e != hipSuccess) return e;
  if (dqk == 128) return launch_bwd_dims<128>(g, stream);
  if (dqk == 64) return launch_bwd_dims<64>(g, stream);
  if (dqk == 32) return launch_bwd_dims<32>(g, stream);
  return hipErrorInvalidValue;
}

}  // namespace hstu
