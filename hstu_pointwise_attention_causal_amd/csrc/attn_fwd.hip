// Causal pointwise aggregated attention, forward, on gfx950.
//
// For one work item (sequence b, head h, query tile of kAttnBM rows) the kernel
// walks the key/value tiles from the sequence start up to the diagonal only
// (fully masked upper-triangle tiles are never touched) and accumulates
//     O_i += sum_j [j <= i] SiLU(alpha q_i.k_j + P[h][pos] + Tt[h][time]) v_j
// then scales by 1/N (neurarch model card, "Exported PyTorch", HSTUBlock
// aggregation; briansu.co explainer section 3 for the two relative biases).
// There is no softmax, hence no running row maximum and no rescaling.
//
// bf16 kernel (MFMA): 4 waves, each owning 32 query rows. Per 64-key tile:
//   S^T[kv][q] = K Q^T       v_mfma_f32_32x32x16_bf16, A = K tile (LDS),
//                            B = Q^T (registers, loaded once per item)
//   P = mask(SiLU(S + bias)) in fp32 registers, packed to bf16
//   O[q][dv] += P V          v_mfma_f32_32x32x16_bf16, A = P straight from the
//                            S^T accumulator registers, B = V^T (LDS)
// Computing S^T instead of S leaves every lane holding one query column and 16
// key rows of the 32x32 block, which is the A-operand layout of the P.V
// product once the 16 keys of a k-block are read in the permuted order
// {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); V^T is read from LDS in the same
// order with transposing reads (ds_read_b64_tr_b16), so no LDS round trip or
// cross-lane shuffle is needed between the two products.
//
// Short work lists (fewer items than two per compute unit) run the same code
// with eight waves per workgroup: two groups of four split each item's key
// range and add their sums through LDS (see attn_fwd_bf16_kernel).
//
// fp32 kernel (VALU): one thread per query row, fp32 throughout, for the
// fp32 workload and as a precision reference path.
#include <type_traits>

#include "attn_common.h"
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace hstu {

namespace {

constexpr int kBN = 64;            // keys per LDS tile
constexpr int kWaves = kAttnBM / 32;   // 32 query rows each
constexpr int kThreads = kWaves * 64;
constexpr int kBufs = 2;           // K/V tiles in flight (2 workgroups per CU fit in LDS)
constexpr int kPosLds = 1024;      // position-table entries staged in LDS
constexpr int kTimeLds = 64;       // time buckets reachable with int64 gaps: 0..62
constexpr int64_t kFwdSplitItemBound = 512;   // work-list bound below which the key-range-split kernel runs

struct BiasLds {
  float pos[kPosLds];
  float time[kTimeLds];
};

__device__ __forceinline__ void stage_bias_tables(BiasLds& s, const AttnArgs& a, int h) {
  if (a.pos_table) {
    const int n = min(a.pos_buckets, kPosLds);
    for (int i = threadIdx.x; i < n; i += blockDim.x) s.pos[i] = a.pos_table[h * a.pos_buckets + i];
  }
  if (a.time_table) {
    const int n = min(a.time_buckets, kTimeLds);
    for (int i = threadIdx.x; i < n; i += blockDim.x) s.time[i] = a.time_table[h * a.time_buckets + i];
  }
}

__device__ __forceinline__ float pos_bias(const BiasLds& s, const AttnArgs& a, int h, int delta) {
  int b = pos_bucket(delta, a.pos_buckets);
  return b < kPosLds ? s.pos[b] : a.pos_table[h * a.pos_buckets + b];
}

__device__ __forceinline__ float time_bias(const BiasLds& s, const AttnArgs& a, int64_t dt) {
  return s.time[time_bucket64(dt, a.time_buckets)];
}

// ============================================================================
// bf16 MFMA kernel
// ============================================================================
//
// Data movement. K and V tiles go from HBM straight into LDS with
// buffer_load ... lds (16 bytes per lane, no VGPR staging); a buffer resource
// per tile bounds the reads to the sequence, so rows past its end arrive as
// zeros. K rows are stored with their 16-byte chunks XOR-swizzled by the row
// index (conflict-free ds_read_b128 of the MFMA A operand). V stays row-major,
// chunks XOR-swizzled by 4 (row mod 4) so that the 4 rows x 4 chunks read by
// 32 lanes fall in 16 distinct bank groups, and the B operand of P.V is read with
// ds_read_b64_tr_b16: in each 16-lane group, lane 4k+q names 4 consecutive
// dims of key row k and lane i receives that column (dim i) of all 4 rows, so
// one transpose read yields 4 keys of one output column per lane.
//
// Relative bias per (wave, 32-key block). The wave's 32 query rows and the
// block's 32 keys bound every pair's distance i - j and timestamp gap, so the
// wave classifies the block from per-block metadata before touching scores:
//   kUniform  - one position bucket and one time bucket: a constant bias;
//   kTwoTime  - one position bucket, time buckets c and c+1: bucket c+1
//               exactly when t_i - t_j >= 2^(c+1) - 1 (compare and select);
//   kGeneral  - per-pair buckets looked up in LDS, plus the causal / sequence
//               mask (diagonal and near-diagonal blocks, sequence tails).
// All paths add the same fp32 bias value to the same fp32 score.
//
// SiLU. Scores and bias are pre-multiplied by log2(e): with x' = log2(e) x
// the kernel needs g(x') = log2(e) SiLU(x) = x' / (1 + 2^-x'). Exactly, that
// is one exp2 and one reciprocal (both quarter-rate on gfx950). When a row's
// scores in an unmasked block are provably small -- |alpha| |q_i| max_j |k_j|
// + max |bias table| <= 1.95 (Cauchy-Schwarz) -- the kernel evaluates
// 2 g = x' + y 2P(y), y = x'^2, with a quadratic P fitted on |x| <= 2 (max
// error 3.3e-4 in x' units; where |g| > 0.05 the relative error is at most
// 1.1e-3, below the bf16 half-ulp that P is rounded to): four FMA-class
// operations instead (silu2_poly in attn_common.h). The choice is made per
// query row from that row's own norm, the norms of keys before it and a bound
// over the whole bias table, so a row's result never depends on later tokens.
enum BlockPath { kUniform = 0, kTwoTime = 1, kGeneral = 2 };

constexpr int kPosLdsFast = 1024;

// Direct HBM -> LDS loads of one key tile (K, V and key timestamps). Kept out
// of the kernel body as a device-only function (the LDS address-space
// pointers have no host meaning). A tile of KCH (VCH) 1 KB instructions is
// spread over the waves, instruction i issued by wave i % kWaves; wave 0 also
// loads the timestamps. Every tile issues the same instructions, also a tile
// past the sequence (all lanes out of range: zeros), so each wave's count of
// loads per tile is a constant.
template <int KCH, int VCH>
__device__ __forceinline__ void issue_tile_loads(const char* kbase, const char* vbase, const int64_t* tsbase,
                                                 int64_t ldk, int64_t ldv, int n, int k0, int w, int lane,
                                                 char* sk, char* sv, int64_t* st) {
  __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(kbase + static_cast<int64_t>(k0) * ldk * 2), 0,
      static_cast<int>(clamp_records(static_cast<int64_t>(n - k0) * ldk * 2)), kRsrcFlags);
  __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(vbase + static_cast<int64_t>(k0) * ldv * 2), 0,
      static_cast<int>(clamp_records(static_cast<int64_t>(n - k0) * ldv * 2)), kRsrcFlags);
  // Per-lane source offsets are recomputed here rather than kept live across
  // the tile loop: instruction i fills LDS slots [64 i, 64 i + 64) of the tile,
  // slot s holding chunk (s % CH) ^ swizzle(row) of row s / CH.
#pragma unroll
  for (int j = 0; j < (KCH + kWaves - 1) / kWaves; ++j) {
    const int i = w + j * kWaves;
    if (KCH % kWaves == 0 || i < KCH) {
      const int sl = i * 64 + lane, r = sl / KCH, c = (sl % KCH) ^ (r & (KCH - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(sk + i * 1024), 16,
                                               static_cast<uint32_t>(r * ldk * 2 + c * 16), 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < (VCH + kWaves - 1) / kWaves; ++j) {
    const int i = w + j * kWaves;
    if (VCH % kWaves == 0 || i < VCH) {
      const int sl = i * 64 + lane, r = sl / VCH, c = (sl % VCH) ^ ((4 * r) & (VCH - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(sv + i * 1024), 16,
                                               static_cast<uint32_t>(r * ldv * 2 + c * 16), 0, 0, 0);
    }
  }
  if (w == 0 && lane < kBN / 2) {
    __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int64_t*>(tsbase + k0), 0,
        tsbase ? static_cast<int>(clamp_records(static_cast<int64_t>(n - k0) * 8)) : 0, kRsrcFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_ptr_t)(st), 16, lane * 16, 0, 0, 0);
  }
}

// HALVES: 2 for the key-range-split kernel (one tile pipeline per half)
template <int DQK, int DV, int HALVES>
struct FwdSmem {
  __attribute__((aligned(16))) char k[HALVES][kBufs][kBN * DQK * 2];
  __attribute__((aligned(16))) char v[HALVES][kBufs][kBN * DV * 2];
  __attribute__((aligned(16))) int64_t t[HALVES][kBufs][kBN];
  float pos[kPosLdsFast];   // log2(e) * P[h][0 .. min(Bp, 1024))
  float time[kTimeLds];     // log2(e) * Tt[h][0 .. min(Bt, 64))
};

// Per-(wave, 32-key block) bias record. A wave classifies 64 key blocks at
// once (one per lane) and each tile reads its two records back into scalar
// registers with v_readlane, so the tile loop carries no LDS or memory round
// trip for the classification. info bits: [1:0] BlockPath, [2] polynomial SiLU
// valid for every row of the wave, [8:3] lower time bucket of a kTwoTime block.
constexpr int kInfoPolyAll = 4;
constexpr int kInfoMasked = 1 << 9;
constexpr int kInfoExactAll = 1 << 10;   // no row of the wave qualifies for the polynomial
constexpr int kInfoNarrowTime = 1 << 11; // every gap t_i - t_j of the block's pairs fits in int32
constexpr int kInfoEmpty = 1 << 12;      // no pair of the block is causal and inside the sequence

// SPLIT: eight waves per workgroup. Waves 0-3 take key tiles [0, qt + 1) of
// the item and waves 4-7 the rest up to the diagonal, each group with its own
// double-buffered tiles; the groups run the same number of steps (the second
// group's spare step, if any, lies past the diagonal and does no work), and
// the second group's fp32 sums are added to the first group's through LDS, in
// that order, before the store. For short work lists, where one workgroup per
// compute unit would leave one wave per SIMD.
template <int DQK, int DV, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 2 * kThreads : kThreads, SPLIT ? 1 : 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  constexpr int KB = DQK / 16;            // k-blocks of QK^T
  constexpr int NB = DV / 32;             // 32-wide column blocks of O
  constexpr int KCH = DQK / 8;            // 16-byte chunks per K row
  constexpr int VCH = DV / 8;             // 16-byte chunks per V row
  using Smem = FwdSmem<DQK, DV, SPLIT ? 2 : 1>;
  constexpr int kT = SPLIT ? 2 * kThreads : kThreads;

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = item.seq0;
  const int n = item.n;
  const int q0 = qt * kAttnBM;

  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(SPLIT ? (tid >> 6) & (kWaves - 1) : tid >> 6);   // query wave of its group
  const int half = SPLIT ? __builtin_amdgcn_readfirstlane(tid >> 8) : 0;      // key-range group
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int qa = q0 + 32 * w;                 // first query row of this wave
  const int qrow = qa + lr;                   // this lane's query column of S^T
  const bool has_time = a.time_table != nullptr;
  const bool has_pos = a.pos_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;
  const bool pos_in_lds = Bp <= kPosLdsFast;
  // metadata row of (head h, the item's sequence): its 32-key blocks start at
  // kMetaPerTile times the sequence's first query tile in the list numbering
  const BlockMeta* meta_row =
      static_cast<const BlockMeta*>(a.meta) + h * a.meta_blocks + static_cast<int64_t>(kMetaPerTile) * item.tile_base;

  // The loads of the prologue go out first, so that their latencies overlap
  // with the table staging and the reductions below: key tile 0 and this
  // lane's Q row.
  const int kv_end = min(n, q0 + kAttnBM);
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const int kt_begin = SPLIT && half == 1 ? qt + 1 : 0;   // this group's first key tile
  const int nsteps = SPLIT ? qt + 1 : ntiles;          // steps of every group
  const char* kbase = static_cast<const char*>(a.k) + (seq0 * a.ldk + h * DQK) * 2;
  const char* vbase = static_cast<const char*>(a.v) + (seq0 * a.ldv + h * DV) * 2;
  auto issue_tile = [&] __device__(int kt, char* dk, char* dv, int64_t* dt) {
    issue_tile_loads<KCH, VCH>(kbase, vbase, has_time ? a.ts + seq0 : nullptr, a.ldk, a.ldv, n, kt * kBN, w, lane,
                               dk, dv, dt);
  };
  if (ntiles > 0) issue_tile(kt_begin, sm.k[half][0], sm.v[half][0], sm.t[half][0]);

  const __bf16* qp = static_cast<const __bf16*>(a.q);
  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qf[kb] = qrow < n ? *reinterpret_cast<const bf16x8_t*>(qp + (seq0 + qrow) * a.ldq + h * DQK + kb * 16 + lh * 8)
                      : bf16x8_t{};

  // (issued before the table staging below, whose wait then covers them)
  const int64_t tq = (has_time && qrow < n) ? a.ts[seq0 + qrow] : 0;
  int64_t wq_min = 0, wq_max = 0;   // timestamps of this wave's query rows (metadata of its block)
  if (has_time && qa < n) {
    wq_min = uniform_i64(meta_row[qa / 32].tmin);
    wq_max = uniform_i64(meta_row[qa / 32].tmax);
  }
  if (has_pos) {
    for (int i = tid; i < min(Bp, kPosLdsFast); i += kT) sm.pos[i] = kLog2e * a.pos_table[h * Bp + i];
  }
  if (has_time) {
    for (int i = tid; i < min(Bt, kTimeLds); i += kT) sm.time[i] = kLog2e * a.time_table[h * Bt + i];
  }
  const float pos_last = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(
      has_pos ? kLog2e * a.pos_table[h * Bp + Bp - 1] : 0.f)));   // bias of far pairs
  __syncthreads();   // the staged tables
  // |bias| <= cmax for every pair: max |L P[h][.]| + max |L Tt[h][.]| (NaN
  // propagates), from the staged tables (and the position entries past them)
  const int np_lds = has_pos ? min(Bp, kPosLdsFast) : 0, nt_lds = has_time ? min(Bt, kTimeLds) : 0;
  float pmax = 0.f, tmax_ = 0.f;
  bool bad = false;
  for (int i = lane; i < np_lds; i += 64) {
    const float x = fabsf(sm.pos[i]);
    pmax = fmaxf(pmax, x);
    bad |= !(x == x);
  }
  if (has_pos)
    for (int i = kPosLdsFast + lane; i < Bp; i += 64) {
      const float x = fabsf(kLog2e * a.pos_table[h * Bp + i]);
      pmax = fmaxf(pmax, x);
      bad |= !(x == x);
    }
  for (int i = lane; i < nt_lds; i += 64) {
    const float x = fabsf(sm.time[i]);
    tmax_ = fmaxf(tmax_, x);
    bad |= !(x == x);
  }
  // wave-uniform values live in scalar registers
  const float cmax = __builtin_amdgcn_ballot_w64(bad) ? __builtin_nanf("")
                                                      : wave_max_uniform(pmax) + wave_max_uniform(tmax_);

  float qsq = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) qsq = fmaf(static_cast<float>(qf[kb][i]), static_cast<float>(qf[kb][i]), qsq);
  qsq += __shfl_xor(qsq, 32, 64);
  const float alpha_l = a.alpha * kLog2e;
  const float qbound = fabsf(alpha_l) * __builtin_sqrtf(qsq);   // |alpha| log2(e) |q_i|
  const float qbound_max =
      __builtin_amdgcn_ballot_w64(qbound != qbound) ? __builtin_nanf("") : wave_max_uniform(qbound);
  const float qbound_min = wave_min_uniform(qrow < n ? qbound : __builtin_inff());   // smallest row bound

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};


  // ---- LDS byte offsets of this lane's operand fragments inside one buffer
  uint32_t k_lds[KB];                       // K row (kvb*32 + lr): + kvb * 32 * KCH * 16
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) k_lds[kb] = (lr * KCH + ((2 * kb + lh) ^ (lr & (KCH - 1)))) * 16;
  const int g16 = lane >> 4, i16 = lane & 15;
  uint32_t v_lds[NB];                       // V row r1 = 4 lh + i16/4 (+ kvb*32 + kk*16, + 8 for the 2nd read)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r1 = 4 * lh + (i16 >> 2);
    const int c = nb * 4 + (g16 & 1) * 2 + ((i16 & 3) >> 1);
    v_lds[nb] = (r1 * VCH + (c ^ ((4 * r1) & (VCH - 1)))) * 16 + (i16 & 1) * 8;
  }

  // S^T of both 32-key blocks of a tile; the two accumulation chains are
  // interleaved (a dependent MFMA waits for its predecessor's result).
  auto qk_tile = [&] __device__(const char* kbuf, f32x16_t& s0, f32x16_t& s1) {
    s0 = f32x16_t{};
    s1 = f32x16_t{};
    const char* kb1 = kbuf + 32 * KCH * 16;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8_t k0f = *reinterpret_cast<const bf16x8_t*>(kbuf + k_lds[kb]);
      const bf16x8_t k1f = *reinterpret_cast<const bf16x8_t*>(kb1 + k_lds[kb]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f, qf[kb], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f, qf[kb], s1, 0, 0, 0);
    }
  };
  auto pack_p = [&] __device__(const float* p, bf16x8_t* pa) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) pa[kk][i] = static_cast<__bf16>(p[kk * 8 + i]);
  };
  // V^T fragments of block kvb (B operands of P.V, keys in the permuted order):
  // vf[kk * NB + nb] for the 16-key step kk and output column group nb.
  auto read_v = [&] __device__(const char* vbuf, int kvb, bf16x8_t* vf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* vb0 = vbuf + (kvb * 32 + kk * 16) * VCH * 16;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x4_t v0 = tr_read(vb0 + v_lds[nb]);
        const bf16x4_t v1 = tr_read(vb0 + v_lds[nb] + 8 * VCH * 16);
        vf[kk * NB + nb] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  auto pv_mfma = [&] __device__(const bf16x8_t* vf, const bf16x8_t* pp) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pp[kk], vf[kk * NB + nb], oacc[nb], 0, 0, 0);
  };
  // K fragments (A operands of S^T) of both blocks of a tile: kf[2 kb + kvb].
  auto read_k = [&] __device__(const char* kbuf, bf16x8_t* kf) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int kvb = 0; kvb < 2; ++kvb)
        kf[2 * kb + kvb] = *reinterpret_cast<const bf16x8_t*>(kbuf + kvb * 32 * KCH * 16 + k_lds[kb]);
  };

  // ---- classification of 64 key blocks (one per lane) for this wave's rows
  int rec_info = kGeneral;
  float rec_clo = 0.f, rec_chi = 0.f, rec_kmax = 0.f;
  auto classify_window = [&] __device__(int win, const float* stime) {
    const int ka = (win * 64 + lane) * 32;
    int info = kGeneral | kInfoMasked | kInfoEmpty;   // no pair for this wave: P is zero
    float clo = 0.f, chi = 0.f, km = 0.f;
    if (ka < n && ka <= qa + 31) {
      const BlockMeta m = meta_row[win * 64 + lane];
      km = m.kmax;
      const bool need_mask = (ka + 31 > qa) || (ka + 31 >= n);
      const bool pos_uniform = !has_pos || (qa - (ka + 31) >= Bp - 1);
      int path = kGeneral, blo = 0;
      clo = chi = pos_last;
      if (!need_mask && pos_uniform) {
        if (!has_time) {
          path = kUniform;
        } else {
          blo = time_bucket64(wq_min - m.tmax, Bt);
          const int bhi = time_bucket64(wq_max - m.tmin, Bt);
          if (blo == bhi) {
            path = kUniform;
            clo = chi = pos_last + stime[blo];
          } else if (bhi == blo + 1) {
            path = kTwoTime;
            clo = pos_last + stime[blo];
            chi = pos_last + stime[bhi];
          }
        }
      }
      const bool polyall = !need_mask && fmaf(qbound_max, km, cmax) <= kPolyBound;
      // every row fails the bound when the smallest one does (fma is monotone in it)
      const bool exactall = !need_mask && fmaf(qbound_min, km, cmax) > kPolyBound;
      // gaps of valid pairs lie in [wq_min - tmax, wq_max - tmin]; inside int32 the
      // low words' wrapped difference is exact (and max(gap, 0) + 1 cannot overflow)
      const bool narrow = has_time && qa < n && wq_max - m.tmin <= int64_t(INT32_MAX) - 1 &&
                          wq_min - m.tmax >= int64_t(INT32_MIN);
      info = path | (polyall ? kInfoPolyAll : 0) | (exactall ? kInfoExactAll : 0) | (blo << 3) |
             (need_mask ? kInfoMasked : 0) | (narrow ? kInfoNarrowTime : 0);
    }
    rec_info = info;
    rec_clo = clo;
    rec_chi = chi;
    rec_kmax = km;
  };

  // P of one block from its scores, for every block the common case does not
  // cover: diagonal and sequence-end blocks, blocks with two time buckets or
  // per-pair buckets, and blocks whose rows differ in SiLU form. The bias of
  // each pair is computed one of three ways (constant, compare-and-select
  // between two time buckets, per-pair lookups: always the same fp32 sum of
  // the same table values), then SiLU is evaluated in the form each row's own
  // bound allows, and the causal / sequence mask zeroes pairs past the row or
  // the sequence (which also covers a block with no work for this wave).
  auto general_block = [&] __device__(const f32x16_t& sc, int l, int k0, int kvb, const int64_t* rt,
                                      const float* spos, const float* stime, bf16x8_t* pa) {
    const int info = __builtin_amdgcn_readlane(rec_info, l);
    if (info & kInfoEmpty) {   // past the wave's last row or the sequence end
      pa[0] = bf16x8_t{};
      pa[1] = bf16x8_t{};
      return;
    }
    const int path = info & 3;
    float x[16];
    if (path == kUniform) {
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec_clo), l));
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = fmaf(sc[j], alpha_l, c);
    } else if (path == kTwoTime) {
      const float clo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec_clo), l));
      const float chi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec_chi), l));
      const int64_t lim = tq - ((int64_t(1) << (((info >> 3) & 63) + 1)) - 1);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        x[j] = fmaf(sc[j], alpha_l, rt[kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)] <= lim ? chi : clo);
    } else {
      // Per-pair buckets. Every branch below is uniform over the wave and taken
      // once per block, and each loop issues all 16 lookups before the first
      // is used, so the LDS latencies overlap.
      float c[16];
      if (has_pos && pos_in_lds) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kv = k0 + kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
          c[j] = spos[min(max(qrow - kv, 0), Bp - 1)];
        }
      } else if (has_pos) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kv = k0 + kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
          const int pb = min(max(qrow - kv, 0), Bp - 1);
          c[j] = pb < kPosLdsFast ? spos[pb] : kLog2e * a.pos_table[h * Bp + pb];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) c[j] = 0.f;
      }
      if (has_time) {
        float tb[16];
        if (info & kInfoNarrowTime) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            tb[j] = stime[time_bucket_narrow(tq, rt[kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)], Bt)];
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kvl = kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
            tb[j] = stime[time_bucket64(tq - rt[kvl], Bt)];
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) c[j] += tb[j];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = fmaf(sc[j], alpha_l, c[j]);
    }
    float p[16];
    if (info & kInfoPolyAll) {
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = silu2_poly(x[j]);
    } else if (info & (kInfoExactAll | kInfoMasked)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = silu2_exact(x[j]);
    } else {
      // rows differ: each takes the form its own bound allows
      const float km = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec_kmax), l));
      const bool poly_row = fmaf(qbound, km, cmax) <= kPolyBound;
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = poly_row ? silu2_poly(x[j]) : silu2_exact(x[j]);
    }
    if (info & kInfoMasked) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kv = k0 + kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
        p[j] = (kv <= qrow && kv < n) ? p[j] : 0.0f;
      }
    }
    pack_p(p, pa);
  };

  constexpr int kFast = kUniform | kInfoPolyAll;
  // Block 1 of the previous tile: its V fragments and P, whose products run
  // at the start of the next step, while that step's K reads are in flight.
  bf16x8_t vf1[2 * NB], p1[2];
  bool prev_active = false;

  // One step, entered right after the barrier that publishes tile kt:
  //   loads of tile kt + 1 into the buffer tile kt - 1 has released; K
  //   fragments of tile kt (their latency hidden by block 1's products of tile
  //   kt - 1); S^T of both blocks; V of block 0 read while P is computed;
  //   block 0's products; V of block 1 read; barrier.
  // Every LDS buffer comes in through a __restrict__ parameter: the step only
  // reads tile kt's buffers and only fills tile kt + 1's, so the compiler does
  // not wait for the in-flight loads before reading LDS.
  //
  // Both products are straight-line code; one branch per tile chooses how P
  // is computed, so only the packed P values cross a branch merge. The common
  // case -- both blocks unmasked, each with one constant bias, every row on
  // the polynomial -- is a few FMA-class operations per pair.
  auto tile_step = [&] __device__(const char* __restrict__ rk, const char* __restrict__ rv,
                                  const int64_t* __restrict__ rt, char* __restrict__ dk, char* __restrict__ dv,
                                  int64_t* __restrict__ dt, const float* __restrict__ spos,
                                  const float* __restrict__ stime, int kt) {
    const int k0 = kt * kBN;
    // tile kt + 1 reuses the buffer of tile kt - 1, released by the last barrier
    issue_tile(kt + 1, dk, dv, dt);
    if ((SPLIT && kt == kt_begin) || (kt & 31) == 0) classify_window(kt >> 5, stime);
    const bool active = qa < n && k0 <= qa + 31 && (!SPLIT || kt < ntiles);
    bf16x8_t kf[2 * KB];
    if (active) read_k(rk, kf);
    if (prev_active) pv_mfma(vf1, p1);
    if (active) {
      const int l0 = (2 * kt) & 63;
      f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * kb], qf[kb], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * kb + 1], qf[kb], s1, 0, 0, 0);
      }
      bf16x8_t vf0[2 * NB];
      read_v(rv, 0, vf0);
      const int i0 = __builtin_amdgcn_readlane(rec_info, l0), i1 = __builtin_amdgcn_readlane(rec_info, l0 + 1);
      bf16x8_t p0[2];
      if ((i0 & (7 | kInfoMasked)) == kFast && (i1 & (7 | kInfoMasked)) == kFast && k0 + 32 <= qa) {
        const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec_clo), l0));
        const float c1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec_clo), l0 + 1));
        float q0[16], q1[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          q0[j] = silu2_poly(fmaf(s0[j], alpha_l, c0));
          q1[j] = silu2_poly(fmaf(s1[j], alpha_l, c1));
        }
        pack_p(q0, p0);
        pack_p(q1, p1);
      } else {
        general_block(s0, l0, k0, 0, rt, spos, stime, p0);
        general_block(s1, l0 + 1, k0, 1, rt, spos, stime, p1);
      }
      pv_mfma(vf0, p0);
      read_v(rv, 1, vf1);
    }
    prev_active = active;
    wait_vmcnt(0);    // this wave's loads of tile kt + 1 have landed
    tile_barrier();   // ... and every other wave's; tile kt's buffers are free
  };

  // tile 0 (in flight since the prologue) lands
  wait_vmcnt(0);
  __syncthreads();   // also publishes the bias tables staged with ordinary LDS stores

  for (int kt = kt_begin; kt < kt_begin + nsteps; ++kt) {
    const int buf = (kt - kt_begin) % kBufs, nxt = (kt - kt_begin + 1) % kBufs;
    tile_step(sm.k[half][buf], sm.v[half][buf], sm.t[half][buf], sm.k[half][nxt], sm.v[half][nxt],
              sm.t[half][nxt], sm.pos, sm.time, kt);
  }
  if (prev_active) pv_mfma(vf1, p1);
  wait_vmcnt(0);

  if constexpr (SPLIT) {
    // the second group's sums, through its own (now idle) tile buffers: 16
    // floats x NB x 64 lanes per wave, two waves in the K buffers, two in V
    __syncthreads();   // every wave's loads have landed; no wave reads a tile buffer any more
    float* red = reinterpret_cast<float*>(w < 2 ? &sm.k[1][0][0] : &sm.v[1][0][0]) + (w & 1) * (NB * 16 * 64);
    if (half == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(red + ((nb * 4 + g) * 64 + lane) * 4) =
              make_float4(oacc[nb][4 * g], oacc[nb][4 * g + 1], oacc[nb][4 * g + 2], oacc[nb][4 * g + 3]);
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 x = *reinterpret_cast<const float4*>(red + ((nb * 4 + g) * 64 + lane) * 4);
        oacc[nb][4 * g] += x.x;
        oacc[nb][4 * g + 1] += x.y;
        oacc[nb][4 * g + 2] += x.z;
        oacc[nb][4 * g + 3] += x.w;
      }
  }

  // ---- epilogue: oacc[nb][j] = 2 log2(e) * N * O[qa + 8(j/4) + 4 lh + j%4][nb*32 + lr]
  const float scale = (a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n)) / (2.0f * kLog2e);
  __bf16* op = static_cast<__bf16*>(a.o) + (seq0 + qa) * a.ldo + h * DV + lr;
  if (qa + 31 < n) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        op[(8 * (j >> 2) + 4 * lh + (j & 3)) * a.ldo + nb * 32] = static_cast<__bf16>(oacc[nb][j] * scale);
  } else if (qa < n) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 8 * (j >> 2) + 4 * lh + (j & 3);
        if (qa + r < n) op[r * a.ldo + nb * 32] = static_cast<__bf16>(oacc[nb][j] * scale);
      }
  }
}

// ============================================================================
// per-(head, 32-key block) metadata: max |k_j| and the timestamp range
// ============================================================================
template <int DQK>
__global__ __launch_bounds__(kMetaPerTile * 64) void attn_block_meta_kernel(AttnArgs a) {
  const int item_idx = blockIdx.x;
  // the entry is read together with the count (the grid is the list's
  // capacity, so the read stays inside the list); the empty asm keeps the
  // compiler from sinking the entry's load below the branch
  const int count = *a.item_count;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  asm volatile("" ::"s"(item.seq0), "s"(item.n), "s"(item.packed), "s"(item.tile_base));
  if (item_idx >= count) return;
  const int qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = item.seq0;
  const int n = item.n;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int jb = qt * kMetaPerTile + w;       // 32-key block of this wave
  if (jb * 32 >= n) return;
  // Each load instruction covers RPI whole key rows (16-byte chunk lane % CPR
  // of row lane / CPR), so every instruction reads contiguous row segments;
  // a row's sum of squares is then reduced over its CPR lanes.
  constexpr int CPR = DQK / 8, RPI = 64 / CPR, NI = 32 / RPI;
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "key row of 4, 8 or 16 chunks");
  const int c = lane % CPR, rsub = lane / CPR;
  bf16x8_t x[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int key = jb * 32 + i * RPI + rsub;
    x[i] = key < n ? *reinterpret_cast<const bf16x8_t*>(static_cast<const __bf16*>(a.k) + (seq0 + key) * a.ldk +
                                                        h * DQK + c * 8)
                   : bf16x8_t{};
  }
  float kn = 0.f;
  bool nan_seen = false;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq = fmaf(static_cast<float>(x[i][e]), static_cast<float>(x[i][e]), sq);
    sq += dpp_row<0xB1>(sq);                         // quad [1,0,3,2]
    sq += dpp_row<0x4E>(sq);                         // quad [2,3,0,1]
    if constexpr (CPR >= 8) sq += dpp_row<0x141>(sq);   // half-row mirror
    if constexpr (CPR >= 16) sq += dpp_row<0x140>(sq);  // row mirror
    nan_seen |= sq != sq;
    kn = fmaxf(kn, __builtin_sqrtf(sq));
  }
  for (int o = CPR; o < 64; o <<= 1) kn = fmaxf(kn, __shfl_xor(kn, o, 64));
  // a NaN norm must keep the polynomial path off: max() drops NaN, so propagate it explicitly
  if (__builtin_amdgcn_ballot_w64(nan_seen)) kn = __builtin_nanf("");
  const int key = jb * 32 + (lane >> 1);
  const bool inside = key < n;
  int64_t tmin = INT64_MAX, tmax = INT64_MIN;
  if (a.ts) {
    const int64_t t = inside ? a.ts[seq0 + key] : 0;
    tmin = inside ? t : INT64_MAX;
    tmax = inside ? t : INT64_MIN;
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y0 = __shfl_xor(tmin, o, 64), y1 = __shfl_xor(tmax, o, 64);
      tmin = y0 < tmin ? y0 : tmin;
      tmax = y1 > tmax ? y1 : tmax;
    }
  }
  if (lane == 0) {
    BlockMeta m;
    m.kmax = kn;
    m.pad0 = 0.f;
    m.tmin = tmin;
    m.tmax = tmax;
    m.pad1 = 0;
    static_cast<BlockMeta*>(a.meta)[h * a.meta_blocks + static_cast<int64_t>(kMetaPerTile) * item.tile_base + jb] = m;
  }
}

// ============================================================================
// fp32 VALU kernel: one thread per query row
// ============================================================================
constexpr int kF32Threads = kAttnBM;
constexpr int kF32BN = 32;

template <int DQK, int DV>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32_kernel(AttnArgs a) {
  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = item.seq0;
  const int n = item.n;
  const int q0 = qt * kAttnBM;
  const float inv_div = a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n);

  __shared__ float sK[kF32BN][DQK];
  __shared__ float sV[kF32BN][DV];
  __shared__ int64_t sT[kF32BN];
  __shared__ BiasLds sB;

  const int tid = threadIdx.x;
  const int qrow = q0 + tid;
  stage_bias_tables(sB, a, h);

  const float* qp = static_cast<const float*>(a.q);
  const float* kp = static_cast<const float*>(a.k);
  const float* vp = static_cast<const float*>(a.v);

  float qr[DQK];
  float acc[DV];
#pragma unroll
  for (int d = 0; d < DQK; ++d) qr[d] = qrow < n ? qp[(seq0 + qrow) * a.ldq + h * DQK + d] : 0.f;
#pragma unroll
  for (int d = 0; d < DV; ++d) acc[d] = 0.f;
  const bool has_time = a.time_table != nullptr;
  const bool has_pos = a.pos_table != nullptr;
  const int64_t tq = (has_time && qrow < n) ? a.ts[seq0 + qrow] : 0;

  const int kv_end = min(n, q0 + kAttnBM);
  for (int k0 = 0; k0 < kv_end; k0 += kF32BN) {
    __syncthreads();
    for (int c = tid; c < kF32BN * DQK; c += kF32Threads) {
      const int r = c / DQK, d = c % DQK;
      sK[r][d] = (k0 + r < n) ? kp[(seq0 + k0 + r) * a.ldk + h * DQK + d] : 0.f;
    }
    for (int c = tid; c < kF32BN * DV; c += kF32Threads) {
      const int r = c / DV, d = c % DV;
      sV[r][d] = (k0 + r < n) ? vp[(seq0 + k0 + r) * a.ldv + h * DV + d] : 0.f;
    }
    if (has_time && tid < kF32BN) sT[tid] = (k0 + tid < n) ? a.ts[seq0 + k0 + tid] : 0;
    __syncthreads();
    for (int r = 0; r < kF32BN; ++r) {
      const int kv = k0 + r;
      if (kv > qrow || kv >= n) break;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DQK; ++d) s = fmaf(qr[d], sK[r][d], s);
      float x = a.alpha * s;
      if (has_pos) x += pos_bias(sB, a, h, qrow - kv);
      if (has_time) x += time_bias(sB, a, tq - sT[r]);
      const float pa = silu_f32_accurate(x);
#pragma unroll
      for (int d = 0; d < DV; ++d) acc[d] = fmaf(pa, sV[r][d], acc[d]);
    }
  }
  if (qrow < n) {
    float* op = static_cast<float*>(a.o);
#pragma unroll
    for (int d = 0; d < DV; ++d) op[(seq0 + qrow) * a.ldo + h * DV + d] = acc[d] * inv_div;
  }
}

template <typename K>
hipError_t launch_items(K kernel, const AttnArgs& a, int threads, hipStream_t stream) {
  if (a.capacity <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(a.capacity)), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_block_meta(const AttnArgs& a, int dqk, hipStream_t stream) {
  if (dqk == 128) return launch_items(attn_block_meta_kernel<128>, a, kMetaPerTile * 64, stream);
  if (dqk == 64) return launch_items(attn_block_meta_kernel<64>, a, kMetaPerTile * 64, stream);
  if (dqk == 32) return launch_items(attn_block_meta_kernel<32>, a, kMetaPerTile * 64, stream);
  return hipErrorInvalidValue;
}

template <int DQK, int DV>
hipError_t launch_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  // A work list that fits the chip at one workgroup per compute unit (or
  // little more) runs the key-range-split kernel: two waves per SIMD instead
  // of one, and half the longest item's chain.
  if (a.capacity < kFwdSplitItemBound) return launch_items(attn_fwd_bf16_kernel<DQK, DV, true>, a, 2 * kThreads, stream);
  return launch_items(attn_fwd_bf16_kernel<DQK, DV, false>, a, kThreads, stream);
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int dqk, int dv, hipStream_t stream) {
  hipError_t e = launch_attn_block_meta(a, dqk, stream);
  if (e != hipSuccess) return e;
  TimedScope timed(kTimedAttnFwd, stream);
  if (dqk == 128 && dv == 128) return launch_fwd_bf16<128, 128>(a, stream);
  if (dqk == 64 && dv == 64) return launch_fwd_bf16<64, 64>(a, stream);
  if (dqk == 32 && dv == 32) return launch_fwd_bf16<32, 32>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 128 && dv == 128) return launch_items(attn_fwd_f32_kernel<128, 128>, a, kF32Threads, stream);
  if (dqk == 64 && dv == 64) return launch_items(attn_fwd_f32_kernel<64, 64>, a, kF32Threads, stream);
  if (dqk == 32 && dv == 32) return launch_items(attn_fwd_f32_kernel<32, 32>, a, kF32Threads, stream);
  return hipErrorInvalidValue;
}

}  // namespace hstu
