// Candidate scoring against a history with cached keys and values (M-FALCON,
// "micro-batched candidate scoring with KV reuse": briansu.co explainer,
// section 6 "Why it works"). Candidate c of sequence b, whose history has n
// tokens, is scored as if it alone were appended at position n:
//     O_c = ( sum_{j<n} SiLU(S_cj) v_j + SiLU(S_cc) v_c ) / N,   N = n + 1 (or the divisor)
//     S_cj = alpha q_c.k_j + P[h][min(n - j, Bp-1)] + Tt[h][bucket(t_c - t_j)]
//     S_cc = alpha q_c.k_c + P[h][0] + Tt[h][0]
// (the forward's pointwise aggregation of the neurarch model card, "Exported
// PyTorch", with the relative biases of the briansu.co explainer, section 3).
// Candidates never see each other, so one pass over the history's K and V
// serves a whole micro-batch of candidates.
//
// Long histories are split into chunks of kCandChunk keys so that the
// workgroups carry similar work whatever the history lengths: a workgroup
// holds 128 candidates of one (sequence, head) against one chunk, 4 waves of
// 32. A sequence with one chunk writes its output directly; otherwise each
// chunk writes an fp32 partial (no softmax, so partials simply add) and
// attn_cand_reduce_kernel sums them in chunk order and scales. The chunk-0
// workgroup also takes the candidates' own keys.
// History K / V / timestamp tiles of 64 keys go HBM -> LDS with direct loads,
// double-buffered. Per 32-key block: S^T = K Q^T on v_mfma_f32_32x32x16_bf16
// (Q in registers), P = SiLU(S + bias) in fp32, O += P V with P straight from
// the S^T accumulators and V^T read transposed from LDS (the operand layouts
// of the forward kernel). Bias per block: a constant position term when every
// key is at least Bp-1 positions back, else one lookup per key (all
// candidates share position n); a constant time term when the block's bucket
// range is one bucket, else one per pair. The candidates' own keys come last,
// as one 32-key block per wave whose mask keeps the diagonal only.
#include "attn_common.h"
#include "common.h"
#include "launch.h"
#include "offsets.h"
#include "timing.h"

namespace hstu {

namespace {

constexpr int kCWaves = 4;
constexpr int kCBM = 32 * kCWaves;   // candidates per workgroup
constexpr int kCBN = 64;             // keys per LDS tile
constexpr int kCPosLds = 1024;
constexpr int kCTimeLds = 64;

template <int D>
struct CandSmem {
  __attribute__((aligned(16))) char k[2][kCBN * D * 2];
  __attribute__((aligned(16))) char v[2][kCBN * D * 2];
  __attribute__((aligned(16))) int64_t t[2][kCBN];
  float pos[kCPosLds];    // log2(e) P[h][.]
  float time[kCTimeLds];  // log2(e) Tt[h][.]
};

// Direct loads of 64 rows of D bf16 (row stride ld) from `base`; rows past
// `rows_left` read as zeros. Instruction i (of CH) is issued by wave i % 4 and
// fills LDS slots [64 i, 64 i + 64); slot s holds chunk (s % CH) ^ swz(row) of
// row s / CH: swz = row mod CH for K (row reads), 4 row mod CH for V
// (transposed reads).
template <int CH, bool VSWZ>
__device__ __forceinline__ void issue_rows64(const char* base, int64_t ld, int rows_left, int w, int lane,
                                             char* __restrict__ dst) {
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(base, rows_left > 0 ? static_cast<int64_t>(rows_left - 1) * ld * 2 + CH * 16 : 0);
#pragma unroll
  for (int j = 0; j < (CH + kCWaves - 1) / kCWaves; ++j) {
    const int i = w + kCWaves * j;
    if (CH % kCWaves == 0 || i < CH) {
      const int sl = i * 64 + lane, r = sl / CH;
      const int c = (sl % CH) ^ (VSWZ ? ((4 * r) & (CH - 1)) : (r & (CH - 1)));
      load_lds16(rs, dst + i * 1024, static_cast<uint32_t>(r * ld * 2 + c * 16));
    }
  }
}

// Smallest / largest int over each row of 16 lanes (every lane of the row
// gets it): DPP quad permutations, then the half-row and row mirrors.
template <int CTRL>
__device__ __forceinline__ int dpp_int(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_int<0xB1>(v));
  v = min(v, dpp_int<0x4E>(v));
  v = min(v, dpp_int<0x141>(v));
  return min(v, dpp_int<0x140>(v));
}
__device__ __forceinline__ int row16_max(int v) {
  v = max(v, dpp_int<0xB1>(v));
  v = max(v, dpp_int<0x4E>(v));
  v = max(v, dpp_int<0x141>(v));
  return max(v, dpp_int<0x140>(v));
}

// Sequence whose chunk range holds global chunk g: the last b with base[b] <= g.
__device__ __forceinline__ int chunk_seq(const int64_t* base, int num_seqs, int64_t g) {
  int lo = 0, hi = num_seqs;   // base[lo] <= g < base[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (base[mid] <= g) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Block-wide scans of the one-workgroup kernel below (1024 threads, 16 waves):
// inclusive sum and inclusive max of int64 values; *total gets the block's
// sum / maximum.
__device__ int64_t block_scan_i64(int64_t v, bool is_max, int64_t* total) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(v, o, 64);
    if (lane >= o) v = is_max ? (u > v ? u : v) : v + u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int64_t before = is_max ? INT64_MIN : 0, all = is_max ? INT64_MIN : 0;
  for (int i = 0; i < 16; ++i) {
    const int64_t x = wsum[i];
    if (i < w) before = is_max ? (x > before ? x : before) : before + x;
    all = is_max ? (x > all ? x : all) : all + x;
  }
  *total = all;
  __syncthreads();
  return is_max ? (before > v ? before : v) : before + v;
}

// Clamped copy of a batch's offsets (offsets.h): out[b] = min(max(0, in[0..b]), T).
__device__ void clamp_offsets(const int64_t* in, int num_seqs, int64_t T, int64_t* out) {
  int64_t run = 0;
  for (int c0 = 0; c0 <= num_seqs; c0 += 1024) {
    const int b = c0 + static_cast<int>(threadIdx.x);
    int64_t chunk_max;
    const int64_t m = block_scan_i64(b <= num_seqs ? in[b] : INT64_MIN, true, &chunk_max);
    if (b <= num_seqs) out[b] = clamp_offset(m, run, T);
    run = chunk_max > run ? chunk_max : run;
  }
}

// One workgroup: the clamped history and candidate offsets, which every later
// kernel of the call reads, then base[b] = sum over earlier sequences of
// max(1, ceil(n / kCandChunk)).
__global__ __launch_bounds__(1024) void cand_chunk_scan_kernel(CandArgs a) {
  const int tid = threadIdx.x;
  clamp_offsets(a.hist_off_in, a.num_seqs, a.hist_tokens, a.hist_off);
  clamp_offsets(a.cand_off_in, a.num_seqs, a.cand_tokens, a.cand_off);
  __syncthreads();
  int64_t carry = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int64_t cnt = 0;
    if (b < a.num_seqs) {
      const int64_t n = a.hist_off[b + 1] - a.hist_off[b];   // >= 0, sum over b <= hist_tokens
      cnt = max(int64_t(1), (n + kCandChunk - 1) / kCandChunk);
    }
    int64_t total;
    const int64_t incl = block_scan_i64(cnt, false, &total);
    if (b < a.num_seqs) a.chunk_base[b] = carry + incl - cnt;
    carry += total;
  }
  if (tid == 0) a.chunk_base[a.num_seqs] = carry;
}

template <int D>
__global__ __launch_bounds__(kCWaves * 64, 2) void attn_cand_kernel(CandArgs a) {
  static_assert(D % 32 == 0, "head dim");
  constexpr int KB = D / 16, NB = D / 32, CH = D / 8;
  const int64_t g = blockIdx.x;
  if (g >= a.chunk_base[a.num_seqs]) return;
  const int b = chunk_seq(a.chunk_base, a.num_seqs, g), h = blockIdx.y;
  const int chunk = static_cast<int>(g - a.chunk_base[b]);
  const bool single = a.chunk_base[b + 1] - a.chunk_base[b] == 1;
  const int64_t h0 = a.hist_off[b], c0 = a.cand_off[b];
  const int n = static_cast<int>(a.hist_off[b + 1] - h0);
  const int m = min(static_cast<int>(a.cand_off[b + 1] - c0), a.max_candidates);
  const int ct0 = blockIdx.z * kCBM;
  if (ct0 >= m) return;

  __shared__ CandSmem<D> sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int cw = ct0 + 32 * w;       // first candidate of this wave
  const int crow = cw + lr;          // this lane's candidate (column of S^T)
  const bool has_pos = a.pos_table != nullptr, has_time = a.time_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;

  if (has_pos)
    for (int i = tid; i < min(Bp, kCPosLds); i += kCWaves * 64) sm.pos[i] = kLog2e * a.pos_table[h * Bp + i];
  if (has_time)
    for (int i = tid; i < min(Bt, kCTimeLds); i += kCWaves * 64) sm.time[i] = kLog2e * a.time_table[h * Bt + i];
  const float pos_far = has_pos ? kLog2e * a.pos_table[h * Bp + Bp - 1] : 0.f;
  const float pos_self = has_pos ? kLog2e * a.pos_table[h * Bp] : 0.f;
  const float time_self = has_time ? kLog2e * a.time_table[h * Bt] : 0.f;
  const float alpha_l = a.alpha * kLog2e;

  // Q fragments of the wave's candidates (B operands of S^T = K Q^T)
  const __bf16* qp = static_cast<const __bf16*>(a.q_c);
  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qf[kb] = crow < m ? *reinterpret_cast<const bf16x8_t*>(qp + (c0 + crow) * a.ldq + h * D + kb * 16 + lh * 8)
                      : bf16x8_t{};
  const int64_t tc = (has_time && crow < m) ? a.ts_c[c0 + crow] : 0;
  // the wave's candidate timestamp range (over its valid candidates)
  int64_t tc_min = crow < m ? tc : INT64_MAX, tc_max = crow < m ? tc : INT64_MIN;
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y0 = __shfl_xor(tc_min, o, 64), y1 = __shfl_xor(tc_max, o, 64);
    tc_min = y0 < tc_min ? y0 : tc_min;
    tc_max = y1 > tc_max ? y1 : tc_max;
  }
  tc_min = uniform_i64(tc_min);
  tc_max = uniform_i64(tc_max);

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};

  // LDS byte offsets of this lane's fragments inside one tile buffer
  uint32_t k_lds[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) k_lds[kb] = (lr * CH + ((2 * kb + lh) ^ (lr & (CH - 1)))) * 16;
  const int g16 = lane >> 4, i16 = lane & 15;
  uint32_t v_lds[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r1 = 4 * lh + (i16 >> 2);
    const int c = nb * 4 + (g16 & 1) * 2 + ((i16 & 3) >> 1);
    v_lds[nb] = (r1 * CH + (c ^ ((4 * r1) & (CH - 1)))) * 16 + (i16 & 1) * 8;
  }

  auto scores = [&] __device__(const char* kbuf, int kvb) __attribute__((always_inline)) {
    f32x16_t s = f32x16_t{};
    const char* kb0 = kbuf + kvb * 32 * CH * 16;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(kb0 + k_lds[kb]), qf[kb], s,
                                                  0, 0, 0);
    return s;
  };
  auto pv = [&] __device__(const char* vbuf, int kvb, const float* p) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t pa;
#pragma unroll
      for (int i = 0; i < 8; ++i) pa[i] = static_cast<__bf16>(p[kk * 8 + i]);
      const char* vb0 = vbuf + (kvb * 32 + kk * 16) * CH * 16;
      bf16x8_t vf[NB];   // every fragment of the step read before the first product
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vf[nb] = __builtin_shufflevector(tr_read(vb0 + v_lds[nb]), tr_read(vb0 + v_lds[nb] + 8 * CH * 16), 0, 1, 2, 3,
                                         4, 5, 6, 7);
      __builtin_amdgcn_sched_barrier(0);   // keeps the reads ahead: the scheduler sank each to its product
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vf[nb], oacc[nb], 0, 0, 0);
    }
  };

  const char* khb = static_cast<const char*>(a.k_h) + (h0 * a.ldkh + h * D) * 2;
  const char* vhb = static_cast<const char*>(a.v_h) + (h0 * a.ldvh + h * D) * 2;
  const int64_t* thb = has_time ? a.ts_h + h0 : nullptr;
  auto issue_hist = [&] __device__(int t, char* dk, char* dv, int64_t* dt) __attribute__((always_inline)) {
    const int k0 = t * kCBN;
    issue_rows64<CH, false>(khb + static_cast<int64_t>(k0) * a.ldkh * 2, a.ldkh, n - k0, w, lane, dk);
    issue_rows64<CH, true>(vhb + static_cast<int64_t>(k0) * a.ldvh * 2, a.ldvh, n - k0, w, lane, dv);
    if (w == 0 && lane < kCBN / 2) {
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(thb ? thb + k0 : nullptr, thb ? static_cast<int64_t>(n - k0) * 8 : 0);
      load_lds16(rt, reinterpret_cast<char*>(dt), lane * 16);
    }
  };

  // ---- history chunk: every key is visible to every candidate (all sit at position n)
  const int t_begin = chunk * (kCandChunk / kCBN);
  const int ntiles = min((n + kCBN - 1) / kCBN, t_begin + kCandChunk / kCBN);
  if (t_begin < ntiles) issue_hist(t_begin, sm.k[0], sm.v[0], sm.t[0]);
  wait_vmcnt(0);
  __syncthreads();   // also publishes the staged bias tables
  auto tile_step = [&] __device__(const char* __restrict__ rk, const char* __restrict__ rv,
                                  const int64_t* __restrict__ rt, char* __restrict__ dk, char* __restrict__ dv,
                                  int64_t* __restrict__ dt, const float* __restrict__ spos,
                                  const float* __restrict__ stime, int t) __attribute__((always_inline)) {
    if (t + 1 < ntiles) issue_hist(t + 1, dk, dv, dt);
    // timestamp range of each 32-key block (lanes 0-31: block 0, 32-63:
    // block 1). When every key of the tile is within 2^31 of its first key,
    // as offsets from that key in 32-bit DPP reductions; otherwise 64-bit
    // cross-lane reductions.
    int64_t bmin2[2] = {INT64_MAX, INT64_MAX}, bmax2[2] = {INT64_MIN, INT64_MIN};
    if (has_time) {
      const bool valid = t * kCBN + lane < n;
      const int64_t tv = valid ? rt[lane] : 0;
      const int64_t base = uniform_i64(rt[0]);   // key t * kCBN, inside the history
      const int64_t d = tv - base;
      const bool near = !valid || (d >= int64_t(INT32_MIN) && d <= int64_t(INT32_MAX));
      if (__builtin_amdgcn_ballot_w64(!near) == 0) {
        const int mn = row16_min(valid ? static_cast<int>(d) : INT32_MAX);
        const int mx = row16_max(valid ? static_cast<int>(d) : INT32_MIN);
#pragma unroll
        for (int kvb = 0; kvb < 2; ++kvb) {
          bmin2[kvb] = base + min(__builtin_amdgcn_readlane(mn, 32 * kvb), __builtin_amdgcn_readlane(mn, 32 * kvb + 16));
          bmax2[kvb] = base + max(__builtin_amdgcn_readlane(mx, 32 * kvb), __builtin_amdgcn_readlane(mx, 32 * kvb + 16));
        }
      } else {
        int64_t kmin = valid ? tv : INT64_MAX, kmax = valid ? tv : INT64_MIN;
        for (int o = 1; o < 32; o <<= 1) {
          const int64_t y0 = __shfl_xor(kmin, o, 64), y1 = __shfl_xor(kmax, o, 64);
          kmin = y0 < kmin ? y0 : kmin;
          kmax = y1 > kmax ? y1 : kmax;
        }
#pragma unroll
        for (int kvb = 0; kvb < 2; ++kvb) {
          bmin2[kvb] = uniform_i64(__shfl(kmin, 32 * kvb, 64));
          bmax2[kvb] = uniform_i64(__shfl(kmax, 32 * kvb, 64));
        }
      }
    }
#pragma unroll
    for (int kvb = 0; kvb < 2; ++kvb) {
      const int ka = t * kCBN + kvb * 32;   // first history key of the block
      if (ka >= n) break;
      const f32x16_t s = scores(rk, kvb);
      // position term: constant when every key of the block is >= Bp-1 back
      const bool pos_const = !has_pos || (n - (ka + 31) >= Bp - 1);
      // time term: constant when the block's bucket range is one bucket
      int tlo = 0, thi = 0;
      bool time_const = true, narrow = false;
      if (has_time) {
        const int64_t bmin = bmin2[kvb], bmax = bmax2[kvb];
        tlo = __builtin_amdgcn_readfirstlane(time_bucket64(tc_min - bmax, Bt));
        thi = __builtin_amdgcn_readfirstlane(time_bucket64(tc_max - bmin, Bt));
        time_const = tlo == thi;
        // gaps of valid pairs lie in [tc_min - bmax, tc_max - bmin]
        narrow = tc_max - bmin <= int64_t(INT32_MAX) - 1 && tc_min - bmax >= int64_t(INT32_MIN);
      }
      const bool tail = ka + 31 >= n;   // keys past the history: masked
      float p[16];
      if (pos_const && time_const && !tail) {
        const float c = (has_pos ? pos_far : 0.f) + (has_time ? stime[tlo] : 0.f);
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = silu2_exact(fmaf(s[j], alpha_l, c));
      } else {
        // Per-pair terms. Each branch is uniform over the wave and taken once
        // per block, and each loop issues all its lookups before the first is
        // used. Keys j of this lane: t * kCBN + kvb * 32 + 8 (j / 4) + 4 lh + j % 4.
        float c[16];
        if (has_pos && !pos_const && Bp <= kCPosLds) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            c[j] = spos[min(max(n - (t * kCBN + kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)), 0), Bp - 1)];
        } else if (has_pos && !pos_const) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int pb = min(max(n - (t * kCBN + kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)), 0), Bp - 1);
            c[j] = pb < kCPosLds ? spos[pb] : kLog2e * a.pos_table[h * Bp + pb];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) c[j] = has_pos ? pos_far : 0.f;
        }
        if (has_time) {
          if (time_const) {
            const float v = stime[tlo];
#pragma unroll
            for (int j = 0; j < 16; ++j) c[j] += v;
          } else if (thi == tlo + 1) {
            // bucket thi exactly when tc - t_j >= 2^(tlo+1) - 1
            const int64_t lim = tc - ((int64_t(1) << (tlo + 1)) - 1);
            const float vlo = stime[tlo], vhi = stime[thi];
#pragma unroll
            for (int j = 0; j < 16; ++j) c[j] += rt[kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)] <= lim ? vhi : vlo;
          } else if (narrow) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
              c[j] += stime[time_bucket_narrow(tc, rt[kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)], Bt)];
          } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
              c[j] += stime[time_bucket64(tc - rt[kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)], Bt)];
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = t * kCBN + kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
          p[j] = key < n ? silu2_exact(fmaf(s[j], alpha_l, c[j])) : 0.f;
        }
      }
      pv(rv, kvb, p);
    }
    wait_vmcnt(0);
    tile_barrier();
  };
  for (int t = t_begin; t < ntiles; ++t) {
    const int buf = (t - t_begin) & 1, nxt = buf ^ 1;
    tile_step(sm.k[buf], sm.v[buf], sm.t[buf], sm.k[nxt], sm.v[nxt], sm.t[nxt], sm.pos, sm.time, t);
  }

  // ---- each candidate's own key (chunk 0 only): the workgroup's 128
  //      candidates as two 64-key tiles; wave w reads its 32 from tile w / 2,
  //      half w % 2
  if (chunk == 0) {
    const char* kcb = static_cast<const char*>(a.k_c) + (c0 * a.ldk + h * D) * 2;
    const char* vcb = static_cast<const char*>(a.v_c) + (c0 * a.ldv + h * D) * 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = ct0 + u * kCBN;
      issue_rows64<CH, false>(kcb + static_cast<int64_t>(r0) * a.ldk * 2, a.ldk, m - r0, w, lane, sm.k[u]);
      issue_rows64<CH, true>(vcb + static_cast<int64_t>(r0) * a.ldv * 2, a.ldv, m - r0, w, lane, sm.v[u]);
    }
    wait_vmcnt(0);
    __syncthreads();
    const char* kbuf = sm.k[w >> 1];
    const char* vbuf = sm.v[w >> 1];
    const int kvb = w & 1;
    const f32x16_t s = scores(kbuf, kvb);
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kk = 8 * (j >> 2) + 4 * lh + (j & 3);   // candidate key within the wave's 32
      p[j] = (kk == lr && crow < m) ? silu2_exact(fmaf(s[j], alpha_l, pos_self + time_self)) : 0.f;
    }
    pv(vbuf, kvb, p);
  }

  // ---- epilogue: oacc[nb][j] = 2 log2(e) N O[cw + 8(j/4) + 4 lh + j%4][nb*32 + lr]
  //      (this chunk's share of it when the history has several chunks)
  if (single) {
    const float scale = (a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n + 1)) / (2.0f * kLog2e);
    __bf16* op = static_cast<__bf16*>(a.o) + (c0 + cw) * a.ldo + h * D + lr;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 8 * (j >> 2) + 4 * lh + (j & 3);
        if (cw + r < m) op[r * a.ldo + nb * 32] = static_cast<__bf16>(oacc[nb][j] * scale);
      }
  } else {
    float* pp = a.partial + ((g * a.max_candidates + cw) * a.num_heads + h) * D + lr;
    const int64_t rs = static_cast<int64_t>(a.num_heads) * D;   // floats per candidate row
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 8 * (j >> 2) + 4 * lh + (j & 3);
        if (cw + r < m) pp[r * rs + nb * 32] = oacc[nb][j];
      }
  }
}

// Candidate rows of sequences with several history chunks: the partials of
// the sequence's chunks summed in chunk order, scaled, rounded to bf16. One
// workgroup per candidate, four consecutive features per thread.
__global__ __launch_bounds__(256) void attn_cand_reduce_kernel(CandArgs a, int d) {
  const int64_t r = blockIdx.x;   // candidate token
  const int b = chunk_seq(a.cand_off, a.num_seqs, r);
  const int64_t c0 = a.cand_off[b];
  const int64_t cl = r - c0;
  const int64_t g0 = a.chunk_base[b], g1 = min(a.chunk_base[b + 1], a.chunk_limit);
  // past the last sequence (clamped offsets may end before cand_tokens), a
  // single-chunk sequence, or a candidate past max_candidates: nothing to sum
  if (r >= a.cand_off[b + 1] || a.chunk_base[b + 1] - g0 <= 1 || cl >= a.max_candidates) return;
  const int n = static_cast<int>(a.hist_off[b + 1] - a.hist_off[b]);
  const float scale = (a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n + 1)) / (2.0f * kLog2e);
  const int width = a.num_heads * d;
  __bf16* op = static_cast<__bf16*>(a.o) + r * a.ldo;
  for (int i = threadIdx.x * 4; i < width; i += blockDim.x * 4) {
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int64_t gg = g0; gg < g1; ++gg)
      s += *reinterpret_cast<const f32x4_t*>(a.partial + (gg * a.max_candidates + cl) * width + i);
    bf16x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(s[e] * scale);
    *reinterpret_cast<bf16x4_t*>(op + i) = o;
  }
}

}  // namespace

namespace {
int64_t chunk_bound(int64_t hist_tokens, int num_seqs) {   // >= sum over sequences of max(1, ceil(n / C))
  return (hist_tokens + kCandChunk - 1) / kCandChunk + num_seqs;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

// Workspace: chunk bases, the clamped history offsets and the clamped
// candidate offsets (int64 [num_seqs + 1] each), then the partial outputs.
size_t cand_partial_offset(int num_seqs) { return align256(3 * static_cast<size_t>(num_seqs + 1) * 8); }

size_t cand_workspace_bytes(int64_t hist_tokens, int num_seqs, int max_candidates, int num_heads, int d) {
  if (num_seqs <= 0 || max_candidates <= 0) return 0;
  return cand_partial_offset(num_seqs) +
         static_cast<size_t>(chunk_bound(hist_tokens, num_seqs)) * max_candidates * num_heads * d * 4;
}

hipError_t launch_attn_cand_bf16(const CandArgs& a_in, int d, int64_t hist_tokens, int64_t cand_tokens,
                                 hipStream_t stream) {
  if (a_in.num_seqs <= 0 || a_in.max_candidates <= 0 || cand_tokens <= 0) return hipSuccess;
  if (d != 128 && d != 64 && d != 32) return hipErrorInvalidValue;
  CandArgs a = a_in;
  a.chunk_limit = chunk_bound(hist_tokens, a.num_seqs);
  a.hist_tokens = hist_tokens;
  a.cand_tokens = cand_tokens;
  a.hist_off = a.chunk_base + (a.num_seqs + 1);
  a.cand_off = a.hist_off + (a.num_seqs + 1);
  const dim3 grid(static_cast<unsigned>(a.chunk_limit), static_cast<unsigned>(a.num_heads),
                  static_cast<unsigned>((a.max_candidates + kCBM - 1) / kCBM));
  TimedScope timed(kTimedAttnCand, stream);
  hipLaunchKernelGGL(cand_chunk_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  if (d == 128) hipLaunchKernelGGL(attn_cand_kernel<128>, grid, dim3(kCWaves * 64), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(attn_cand_kernel<64>, grid, dim3(kCWaves * 64), 0, stream, a);
  else hipLaunchKernelGGL(attn_cand_kernel<32>, grid, dim3(kCWaves * 64), 0, stream, a);
  hipLaunchKernelGGL(attn_cand_reduce_kernel, dim3(static_cast<unsigned>(cand_tokens)), dim3(256), 0, stream, a, d);
  return hipGetLastError();
}

}  // namespace hstu
