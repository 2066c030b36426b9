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
//   summed per wave in LDS (one table per wave, so no two waves race) and
//   written as one partial row per key tile.
//
//   query pass (attn_bwd_q_kernel): a work item owns 128 query rows, as in the
//   forward, and recomputes S^T = K Q^T and dA^T = V dO^T per key tile to form
//   dQ[i][d] += dS K with K read transposed from LDS.
//
//   bias reduction (attn_bwd_bias_reduce_kernel): sums the partial rows of
//   each head in tile order.
//
// Scores are kept in x' = log2(e) x units as in the forward (one exp2 and one
// reciprocal per pair); P is stored to bf16 as log2(e) SiLU(x) and the output
// scales remove the factor.
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

// Bias-table gradients of one key tile, summed in LDS. Position buckets: one
// table per wave (its lanes' pairs rarely share a bucket within one add).
// Time buckets: one column per lane of each wave ([wave][bucket][lane]) --
// near the diagonal most pairs of a block share a bucket, and lane-private
// columns keep those adds free of same-address serialization (and of atomics:
// plain read-modify-write measured faster than conflict-free LDS atomics).
struct BwdGradSmem {
  float gpos[kBW][kBwdPosMax];
  float gtime[kBW][kBwdTimeSlots][64];
};

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// ============================================================================
// key pass: dK, dV and the bias-table gradients
// ============================================================================
template <int DQK, int DV>
__global__ __launch_bounds__(kBThreads, 1) void attn_bwd_kv_kernel(AttnBwdArgs g) {
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  const AttnArgs& a = g.f;
  constexpr int KB = DQK / 16, VB = DV / 16;       // k-steps of S and dA
  constexpr int NQ = DQK / 32, NV = DV / 32;       // 32-column groups of dK and dV
  constexpr int QCH = DQK / 8, DCH = DV / 8;       // 16-byte chunks per Q / dO row
  constexpr int QI = (QCH + kBW - 1) / kBW, DI = (DCH + kBW - 1) / kBW;

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int b = item.seq, h = item_head(item);
  const int64_t seq0 = a.off[b];
  const int n = static_cast<int>(a.off[b + 1] - seq0);
  // the list orders tiles by query-pass cost (tile index + 1); the key pass
  // costs (tiles - key tile), so tile qt of the list is key tile tiles-1-qt
  const int ntl = (n + kAttnBM - 1) / kAttnBM;
  const int kt = ntl - 1 - item_qtile(item);
  const int k0 = kt * kAttnBM;

  __shared__ BwdSmem<DQK, DV> sm;
  __shared__ BwdGradSmem gs;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int kw = k0 + 32 * w;     // first key of this wave
  const int key = kw + lr;        // this lane's key (column of S)
  const bool has_time = a.time_table != nullptr, has_pos = a.pos_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;
  const BlockMeta* meta_row =
      static_cast<const BlockMeta*>(a.meta) + h * a.meta_blocks + static_cast<int64_t>(kMetaPerTile) * a.tile_base[b];

  if (has_pos)
    for (int i = tid; i < Bp; i += kBThreads) sm.pos[i] = kLog2e * a.pos_table[h * Bp + i];
  if (has_time)
    for (int i = tid; i < min(Bt, kBwdTimeSlots); i += kBThreads) sm.time[i] = kLog2e * a.time_table[h * Bt + i];
  for (int i = tid; i < kBW * kBwdPosMax; i += kBThreads) (&gs.gpos[0][0])[i] = 0.f;
  for (int i = tid; i < kBW * kBwdTimeSlots * 64; i += kBThreads) (&gs.gtime[0][0][0])[i] = 0.f;
  const float pos_last = has_pos ? kLog2e * a.pos_table[h * Bp + Bp - 1] : 0.f;

  // K and V rows of this lane's key: B operands of S = Q K^T and dA = dO V^T
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);
  bf16x8_t kf[KB], vf[VB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    kf[kb] = key < n ? *reinterpret_cast<const bf16x8_t*>(kp + (seq0 + key) * a.ldk + h * DQK + kb * 16 + lh * 8)
                     : bf16x8_t{};
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
    vf[vb] = key < n ? *reinterpret_cast<const bf16x8_t*>(vp + (seq0 + key) * a.ldv + h * DV + vb * 16 + lh * 8)
                     : bf16x8_t{};
  const int64_t tk = (has_time && key < n) ? a.ts[seq0 + key] : 0;
  int64_t tk_min = 0, tk_max = 0;
  if (has_time && kw < n) {
    tk_min = uniform_i64(meta_row[kw / 32].tmin);
    tk_max = uniform_i64(meta_row[kw / 32].tmax);
  }
  const float alpha_l = a.alpha * kLog2e;

  f32x16_t dva[NV], dka[NQ];
#pragma unroll
  for (int i = 0; i < NV; ++i) dva[i] = f32x16_t{};
#pragma unroll
  for (int i = 0; i < NQ; ++i) dka[i] = f32x16_t{};
  float far_acc = 0.f;   // dS' of the blocks whose pairs all read position bucket Bp - 1

  uint32_t qoff[QI], doff[DI];
  tile_load_offsets<QCH>(w, lane, a.ldq, qoff);
  tile_load_offsets<DCH>(w, lane, g.lddo, doff);
  const char* qbase = static_cast<const char*>(a.q) + (seq0 * a.ldq + h * DQK) * 2;
  const char* dbase = static_cast<const char*>(g.d_o) + (seq0 * g.lddo + h * DV) * 2;
  const int64_t* tsbase = has_time ? a.ts + seq0 : nullptr;
  uint32_t q_row[KB], d_row[VB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) q_row[kb] = row_read_offset<QCH>(lr, lh, kb);
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) d_row[vb] = row_read_offset<DCH>(lr, lh, vb);
  uint32_t q_tr0[NQ], q_tr1[NQ], d_tr0[NV], d_tr1[NV];
#pragma unroll
  for (int nb = 0; nb < NQ; ++nb) tr_read_offsets<QCH>(lane, nb, q_tr0[nb], q_tr1[nb]);
#pragma unroll
  for (int nb = 0; nb < NV; ++nb) tr_read_offsets<DCH>(lane, nb, d_tr0[nb], d_tr1[nb]);

  const int tq0 = k0 / kBBN;                       // first query tile: holds the diagonal
  const int ntq = (n + kBBN - 1) / kBBN - tq0;     // >= 1
  float* gpos = gs.gpos[w];
  float* gtime = &gs.gtime[w][0][lane];   // bucket b of this lane: gtime[64 b]

  // dV += P^T dO and dK += dS^T Q of a block run one block late: they are
  // issued right after the next block's S and dA products, so they execute
  // while that block's P and dS are computed. Carried between blocks: the
  // packed P and dS and the block's transposed dO and Q fragments (read before
  // the barrier that may recycle their tile). Zero-initialized, the first
  // block's late products add nothing.
  bf16x8_t pa_prev[2], sa_prev[2], ob_prev[2 * NV], qt_prev[2 * NQ];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) pa_prev[kk] = sa_prev[kk] = bf16x8_t{};
#pragma unroll
  for (int i = 0; i < 2 * NV; ++i) ob_prev[i] = bf16x8_t{};
#pragma unroll
  for (int i = 0; i < 2 * NQ; ++i) qt_prev[i] = bf16x8_t{};
  auto late_products = [&] __device__() __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int nb = 0; nb < NV; ++nb)
        dva[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_prev[kk], ob_prev[kk * NV + nb], dva[nb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < NQ; ++nb)
        dka[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa_prev[kk], qt_prev[kk * NQ + nb], dka[nb], 0, 0, 0);
    }
  };

  auto step = [&] __device__(const char* __restrict__ rq, const char* __restrict__ rd,
                             const int64_t* __restrict__ rt, const BlockMeta* __restrict__ rm,
                             char* __restrict__ nq, char* __restrict__ nd, int64_t* __restrict__ nt,
                             BlockMeta* __restrict__ nm, const float* __restrict__ spos,
                             const float* __restrict__ stime, int t) __attribute__((always_inline)) {
    const int i0 = (tq0 + t) * kBBN;
    if (t + 1 < ntq)
      issue_rows_tile<QCH, DCH>(qbase, dbase, a.ldq, g.lddo, tsbase, meta_row, n, i0 + kBBN, w, lane, qoff, doff, nq,
                                nd, nt, nm);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qa = i0 + 32 * qb;
      const bool active = kw < n && qa < n && qa + 31 >= kw;
      f32x16_t s = f32x16_t{}, da = f32x16_t{};
      const char* qblk = rq + qb * 32 * QCH * 16;
      const char* dblk = rd + qb * 32 * DCH * 16;
      // all A fragments first (their reads overlap), then the two chains
      bf16x8_t qfr[KB], dfr[VB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qfr[kb] = *reinterpret_cast<const bf16x8_t*>(qblk + q_row[kb]);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) dfr[vb] = *reinterpret_cast<const bf16x8_t*>(dblk + d_row[vb]);
#pragma unroll
      for (int kb = 0; kb < (KB > VB ? KB : VB); ++kb) {
        if (kb < KB) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr[kb], kf[kb], s, 0, 0, 0);
        if (kb < VB) da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr[kb], vf[kb], da, 0, 0, 0);
      }
      // the previous block's dV, dK products, then this block's transposed
      // fragments for its own (one block later)
      late_products();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const char* dst = dblk + kk * 16 * DCH * 16;
        const char* qst = qblk + kk * 16 * QCH * 16;
#pragma unroll
        for (int nb = 0; nb < NV; ++nb)
          ob_prev[kk * NV + nb] =
              __builtin_shufflevector(tr_read(dst + d_tr0[nb]), tr_read(dst + d_tr1[nb]), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb)
          qt_prev[kk * NQ + nb] =
              __builtin_shufflevector(tr_read(qst + q_tr0[nb]), tr_read(qst + q_tr1[nb]), 0, 1, 2, 3, 4, 5, 6, 7);
      }
      __builtin_amdgcn_sched_barrier(0);   // the products above go out before the P / dS arithmetic
      // s[4g+e], da[4g+e]: query row qa + 8g + 4lh + e, key `key`
      float p[16], ds[16];
      if (!active) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = ds[r] = 0.f;
      } else {
        int64_t tq_min = 0, tq_max = 0;
        if (has_time) {
          tq_min = uniform_i64(rm[qb].tmin);
          tq_max = uniform_i64(rm[qb].tmax);
        }
        const BlockClass c =
            classify_block(qa, kw, n, has_pos, Bp, has_time, Bt, tq_min, tq_max, tk_min, tk_max, pos_last, stime);
        if (c.path != kBGeneral) {
          const int64_t lim = tk + ((int64_t(1) << (c.tlo + 1)) - 1);
          float slo = 0.f, shi = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int il = qb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const bool hi = c.path == kBTwoTime && rt[il] >= lim;
            const float x = fmaf(s[r], alpha_l, hi ? c.chi : c.clo);
            float dsl;
            silu_and_grad(x, p[r], dsl);
            ds[r] = da[r] * dsl;
            if (hi) shi += ds[r];
            else slo += ds[r];
          }
          if (has_pos) far_acc += slo + shi;
          if (has_time) {
            gtime[64 * c.tlo] += slo;
            if (c.path == kBTwoTime) gtime[64 * (c.tlo + 1)] += shi;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int il = qb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const int i = i0 + il;
            const bool valid = i >= key && i < n && key < n;
            const int pb = min(max(i - key, 0), Bp - 1);
            float cb = 0.f;
            if (has_pos) cb = spos[pb];
            int tb = 0;
            if (has_time) {
              tb = time_bucket64(rt[il] - tk, Bt);
              cb += stime[tb];
            }
            const float x = fmaf(s[r], alpha_l, cb);
            float pl, dsl;
            silu_and_grad(x, pl, dsl);
            p[r] = valid ? pl : 0.f;
            ds[r] = valid ? da[r] * dsl : 0.f;
            // masked pairs add nothing; pairs in the last position bucket go
            // to the register sum of the far pairs
            if (has_pos && valid) {
              if (pb < Bp - 1) atomicAdd(&gpos[pb], ds[r]);
              else far_acc += ds[r];
            }
            if (has_time) gtime[64 * tb] += ds[r];
          }
        }
      }
      // P and dS of this block's 32 query rows (two 16-row steps), for the
      // late products
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pa_prev[kk][i] = static_cast<__bf16>(p[kk * 8 + i]);
          sa_prev[kk][i] = static_cast<__bf16>(ds[kk * 8 + i]);
        }
    }
  };

  issue_rows_tile<QCH, DCH>(qbase, dbase, a.ldq, g.lddo, tsbase, meta_row, n, tq0 * kBBN, w, lane, qoff, doff,
                            sm.a[0], sm.b[0], sm.t[0], sm.m[0]);
  wait_vmcnt(0);
  __syncthreads();   // also publishes the staged tables and the zeroed gradient tables
  for (int t = 0; t < ntq; ++t) {
    const int buf = t & 1;
    step(sm.a[buf], sm.b[buf], sm.t[buf], sm.m[buf], sm.a[buf ^ 1], sm.b[buf ^ 1], sm.t[buf ^ 1], sm.m[buf ^ 1],
         sm.pos, sm.time, t);
    wait_vmcnt(0);
    tile_barrier();
  }

  late_products();   // the last block's

  // ---- dK, dV: accumulator [i][r] holds key kw + 8(r/4) + 4 lh + r%4, column 32 i + lr
  const float inv_n = a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n);
  const float sv = inv_n / kLog2e, sk = a.alpha * inv_n;
  __bf16* dvp = static_cast<__bf16*>(g.dv) + (seq0 + kw) * g.lddv + h * DV + lr;
  __bf16* dkp = static_cast<__bf16*>(g.dk) + (seq0 + kw) * g.lddk + h * DQK + lr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = 8 * (r >> 2) + 4 * lh + (r & 3);
    if (kw + kr < n) {
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) dvp[kr * g.lddv + nb * 32] = static_cast<__bf16>(dva[nb][r] * sv);
#pragma unroll
      for (int nb = 0; nb < NQ; ++nb) dkp[kr * g.lddk + nb * 32] = static_cast<__bf16>(dka[nb][r] * sk);
    }
  }

  // ---- bias-table gradients of this key tile
  if (g.grad_stride > 0) {
    if (has_pos) {
      const float f = wave_sum(far_acc);
      if (lane == 0) gpos[Bp - 1] += f;
    }
    __syncthreads();
    float* prow = g.partial + (static_cast<int64_t>(h) * g.tile_rows + a.tile_base[b] + kt) * g.grad_stride;
    if (has_pos)
      for (int i = tid; i < Bp; i += kBThreads) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < kBW; ++ww) s += gs.gpos[ww][i];
        prow[i] = s * inv_n;
      }
    if (has_time) {
      // bucket tid / 4: thread (tid & 3) sums wave (tid & 3)'s 64 lane columns,
      // then the 4 threads (adjacent lanes) combine, in a fixed order
      static_assert(kBThreads == 4 * kBwdTimeSlots && kBW == 4, "one bucket per 4 threads");
      float* trow = prow + (has_pos ? Bp : 0);
      const int tb = tid >> 2, ww = tid & 3;
      const f32x4_t* col = reinterpret_cast<const f32x4_t*>(&gs.gtime[ww][tb][0]);
      float s = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < 16; ++c4) {
        const f32x4_t v4 = col[c4];
        s += (v4[0] + v4[1]) + (v4[2] + v4[3]);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (ww == 0) trow[tb] = s * inv_n;
    }
  }
}

// ============================================================================
// query pass: dQ
// ============================================================================
template <int DQK, int DV>
__global__ __launch_bounds__(kBThreads, 2) void attn_bwd_q_kernel(AttnBwdArgs g) {
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  const AttnArgs& a = g.f;
  constexpr int KB = DQK / 16, VB = DV / 16;       // k-steps of S^T and dA^T
  constexpr int NQ = DQK / 32;                     // 32-column groups of dQ
  constexpr int KCH = DQK / 8, VCH = DV / 8;
  constexpr int KI = (KCH + kBW - 1) / kBW, VI = (VCH + kBW - 1) / kBW;

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int b = item.seq, qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = a.off[b];
  const int n = static_cast<int>(a.off[b + 1] - seq0);
  const int q0 = qt * kAttnBM;

  __shared__ BwdSmem<DQK, DV> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int qa = q0 + 32 * w;
  const int qrow = qa + lr;
  const bool has_time = a.time_table != nullptr, has_pos = a.pos_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;
  const BlockMeta* meta_row =
      static_cast<const BlockMeta*>(a.meta) + h * a.meta_blocks + static_cast<int64_t>(kMetaPerTile) * a.tile_base[b];

  if (has_pos)
    for (int i = tid; i < Bp; i += kBThreads) sm.pos[i] = kLog2e * a.pos_table[h * Bp + i];
  if (has_time)
    for (int i = tid; i < min(Bt, kBwdTimeSlots); i += kBThreads) sm.time[i] = kLog2e * a.time_table[h * Bt + i];
  const float pos_last = has_pos ? kLog2e * a.pos_table[h * Bp + Bp - 1] : 0.f;

  // Q and dO rows of this lane's query: B operands of S^T = K Q^T, dA^T = V dO^T
  const __bf16* qp = static_cast<const __bf16*>(a.q);
  const __bf16* dop = static_cast<const __bf16*>(g.d_o);
  bf16x8_t qf[KB], df[VB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qf[kb] = qrow < n ? *reinterpret_cast<const bf16x8_t*>(qp + (seq0 + qrow) * a.ldq + h * DQK + kb * 16 + lh * 8)
                      : bf16x8_t{};
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
    df[vb] = qrow < n ? *reinterpret_cast<const bf16x8_t*>(dop + (seq0 + qrow) * g.lddo + h * DV + vb * 16 + lh * 8)
                      : bf16x8_t{};
  const int64_t tq = (has_time && qrow < n) ? a.ts[seq0 + qrow] : 0;
  int64_t tq_min = 0, tq_max = 0;
  if (has_time && qa < n) {
    tq_min = uniform_i64(meta_row[qa / 32].tmin);
    tq_max = uniform_i64(meta_row[qa / 32].tmax);
  }
  const float alpha_l = a.alpha * kLog2e;

  f32x16_t dqa[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dqa[i] = f32x16_t{};

  uint32_t koff[KI], voff[VI];
  tile_load_offsets<KCH>(w, lane, a.ldk, koff);
  tile_load_offsets<VCH>(w, lane, a.ldv, voff);
  const char* kbase = static_cast<const char*>(a.k) + (seq0 * a.ldk + h * DQK) * 2;
  const char* vbase = static_cast<const char*>(a.v) + (seq0 * a.ldv + h * DV) * 2;
  const int64_t* tsbase = has_time ? a.ts + seq0 : nullptr;
  uint32_t k_row[KB], v_row[VB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) k_row[kb] = row_read_offset<KCH>(lr, lh, kb);
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) v_row[vb] = row_read_offset<VCH>(lr, lh, vb);
  uint32_t k_tr0[NQ], k_tr1[NQ];
#pragma unroll
  for (int nb = 0; nb < NQ; ++nb) tr_read_offsets<KCH>(lane, nb, k_tr0[nb], k_tr1[nb]);

  const int kv_end = min(n, q0 + kAttnBM);
  const int ntk = (kv_end + kBBN - 1) / kBBN;

  auto step = [&] __device__(const char* __restrict__ rk, const char* __restrict__ rv,
                             const int64_t* __restrict__ rt, const BlockMeta* __restrict__ rm,
                             char* __restrict__ nk, char* __restrict__ nv, int64_t* __restrict__ nt,
                             BlockMeta* __restrict__ nm, const float* __restrict__ spos,
                             const float* __restrict__ stime, int t) {
    const int k0 = t * kBBN;
    if (t + 1 < ntk)
      issue_rows_tile<KCH, VCH>(kbase, vbase, a.ldk, a.ldv, tsbase, meta_row, n, k0 + kBBN, w, lane, koff, voff, nk,
                                nv, nt, nm);
#pragma unroll
    for (int kvb = 0; kvb < 2; ++kvb) {
      const int ka = k0 + 32 * kvb;
      const bool active = qa < n && ka < n && ka <= qa + 31;
      f32x16_t s = f32x16_t{}, da = f32x16_t{};
      const char* kblk = rk + kvb * 32 * KCH * 16;
      const char* vblk = rv + kvb * 32 * VCH * 16;
#pragma unroll
      for (int kb = 0; kb < (KB > VB ? KB : VB); ++kb) {
        if (kb < KB)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(kblk + k_row[kb]), qf[kb], s,
                                                      0, 0, 0);
        if (kb < VB)
          da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(vblk + v_row[kb]), df[kb],
                                                       da, 0, 0, 0);
      }
      // s[4g+e], da[4g+e]: key ka + 8g + 4lh + e, query qrow
      float ds[16];
      if (!active) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = 0.f;
      } else {
        int64_t tk_min = 0, tk_max = 0;
        if (has_time) {
          tk_min = uniform_i64(rm[kvb].tmin);
          tk_max = uniform_i64(rm[kvb].tmax);
        }
        const BlockClass c =
            classify_block(qa, ka, n, has_pos, Bp, has_time, Bt, tq_min, tq_max, tk_min, tk_max, pos_last, stime);
        if (c.path != kBGeneral) {
          const int64_t lim = tq - ((int64_t(1) << (c.tlo + 1)) - 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = kvb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const bool hi = c.path == kBTwoTime && rt[kl] <= lim;
            const float x = fmaf(s[r], alpha_l, hi ? c.chi : c.clo);
            float pl, dsl;
            silu_and_grad(x, pl, dsl);
            ds[r] = da[r] * dsl;
          }
        } else {
          // Per-pair buckets in two halves of 8 pairs, each issuing all its
          // lookups before the first is used; one or two time buckets across
          // the block's valid pairs take a compare-and-select instead (as in
          // the key pass).
          TimeSpan tsp{0, 0, false};
          if (has_time) tsp = time_span(tq_min - tk_max, tq_max - tk_min, Bt);
          const int64_t lim = tq - ((int64_t(1) << (tsp.lo + 1)) - 1);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float cb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * hf + e;
              const int kv = k0 + kvb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
              cb[e] = has_pos ? spos[min(max(qrow - kv, 0), Bp - 1)] : 0.f;
            }
            if (has_time) {
              if (tsp.hi - tsp.lo <= 1) {
                const float vlo = stime[tsp.lo], vhi = stime[tsp.hi];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const int r = 8 * hf + e;
                  cb[e] += tsp.hi > tsp.lo && rt[kvb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)] <= lim ? vhi : vlo;
                }
              } else if (tsp.narrow) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const int r = 8 * hf + e;
                  cb[e] += stime[time_bucket_narrow(tq, rt[kvb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)], Bt)];
                }
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const int r = 8 * hf + e;
                  cb[e] += stime[time_bucket64(tq - rt[kvb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)], Bt)];
                }
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * hf + e;
              const int kv = k0 + kvb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
              const bool valid = kv <= qrow && kv < n && qrow < n;
              const float x = fmaf(s[r], alpha_l, cb[e]);
              float pl, dsl;
              silu_and_grad(x, pl, dsl);
              ds[r] = valid ? da[r] * dsl : 0.f;
            }
          }
        }
      }
      // dQ += dS K over the block's 32 keys (two 16-key steps)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t sa;
#pragma unroll
        for (int i = 0; i < 8; ++i) sa[i] = static_cast<__bf16>(ds[kk * 8 + i]);
        const char* kst = kblk + kk * 16 * KCH * 16;
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) {
          const bf16x8_t kb16 = __builtin_shufflevector(tr_read(kst + k_tr0[nb]), tr_read(kst + k_tr1[nb]), 0, 1, 2,
                                                        3, 4, 5, 6, 7);
          dqa[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, kb16, dqa[nb], 0, 0, 0);
        }
      }
    }
  };

  if (ntk > 0)
    issue_rows_tile<KCH, VCH>(kbase, vbase, a.ldk, a.ldv, tsbase, meta_row, n, 0, w, lane, koff, voff, sm.a[0],
                              sm.b[0], sm.t[0], sm.m[0]);
  wait_vmcnt(0);
  __syncthreads();
  for (int t = 0; t < ntk; ++t) {
    const int buf = t & 1;
    step(sm.a[buf], sm.b[buf], sm.t[buf], sm.m[buf], sm.a[buf ^ 1], sm.b[buf ^ 1], sm.t[buf ^ 1], sm.m[buf ^ 1],
         sm.pos, sm.time, t);
    wait_vmcnt(0);
    tile_barrier();
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
hipError_t launch_bwd_items(K kernel, const AttnBwdArgs& g, hipStream_t stream) {
  if (g.f.capacity <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(g.f.capacity)), dim3(kBThreads), 0, stream, g);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_dims(const AttnBwdArgs& g, hipStream_t stream) {
  hipError_t e;
  {
    TimedScope timed(kTimedAttnBwdKv, stream);
    e = launch_bwd_items(attn_bwd_kv_kernel<D, D>, g, stream);
  }
  if (e != hipSuccess) return e;
  {
    TimedScope timed(kTimedAttnBwdQ, stream);
    e = launch_bwd_items(attn_bwd_q_kernel<D, D>, g, stream);
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
