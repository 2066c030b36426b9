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
// order, so no LDS round trip or cross-lane shuffle is needed between the two
// products. V is transposed once per tile while it is staged into LDS.
//
// fp32 kernel (VALU): one thread per query row, fp32 throughout, for the
// fp32 workload and as a precision reference path.
#include "common.h"
#include "launch.h"

namespace hstu {

namespace {

constexpr int kBN = 64;            // keys per LDS tile
constexpr int kWaves = 4;          // 32 query rows each
constexpr int kThreads = kWaves * 64;
constexpr int kPosLds = 1024;      // position-table entries staged in LDS
constexpr int kTimeLds = 64;       // time buckets reachable with int64 gaps: 0..62

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
// Relative bias per (wave, 32-key block). The wave's 32 query rows and the
// block's 32 keys bound every pair's distance i - j and timestamp gap
// t_i - t_j, so before touching the 1024 scores the wave classifies the block:
//   kUniform  - one position bucket and one time bucket for every pair: the
//               bias is a single constant c (most blocks away from the diagonal);
//   kTwoTime  - one position bucket, time buckets c and c+1 only: bucket c+1
//               exactly when t_i - t_j >= 2^(c+1) - 1, a compare and select;
//   kGeneral  - per-pair position and time buckets looked up in LDS (blocks
//               near the diagonal, the diagonal itself and sequence tails).
// Every path adds the same fp32 bias value to the same fp32 score, so the
// choice of path never changes a result bit (bitwise causality holds).
// Scores and bias tables are pre-multiplied by log2(e) so that the SiLU is
// x' / (1 + 2^-x') with one exp2 and one reciprocal; the factor is removed in
// the output scale.
enum BlockPath { kUniform = 0, kTwoTime = 1, kGeneral = 2, kGeneral64 = 3 };

constexpr int kPosLdsFast = 1024;
constexpr int kInt32Max = 0x7fffffff;

struct TileTime {
  int32_t rel[kBN];         // min(t_k - kvmin(block of k), 2^31 - 1); 0 past the sequence
  int64_t raw[kBN];         // t_k (for the 64-bit fallback)
  int64_t kmin[kBN / 32];   // per 32-key block, over keys inside the sequence
  int64_t kmax[kBN / 32];
};

__device__ __forceinline__ int64_t wave_min64(int64_t x, int width) {
  for (int o = width / 2; o > 0; o >>= 1) {
    int64_t y = __shfl_xor(x, o, width);
    x = y < x ? y : x;
  }
  return x;
}
__device__ __forceinline__ int64_t wave_max64(int64_t x, int width) {
  for (int o = width / 2; o > 0; o >>= 1) {
    int64_t y = __shfl_xor(x, o, width);
    x = y > x ? y : x;
  }
  return x;
}
__device__ __forceinline__ int uniform_int(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int DQK, int DV>
struct FwdSmem {
  static constexpr int KLD = DQK + 8;   // K row stride (bf16): rows shift by 16 B
  static constexpr int VLD = kBN + 4;   // V^T row stride (bf16): rows shift by 8 B
  __bf16 k[2][kBN * KLD];
  __bf16 vt[2][DV * VLD];
  TileTime tt[2];
  float pos[kPosLdsFast];   // log2(e) * P[h][0 .. min(Bp, 1024))
  float time[kTimeLds];     // log2(e) * Tt[h][0 .. min(Bt, 64))
};

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  constexpr int KB = DQK / 16;   // k-blocks of the QK^T product
  constexpr int NB = DV / 32;    // 32-wide column blocks of O
  using Smem = FwdSmem<DQK, DV>;
  constexpr int KLD = Smem::KLD, VLD = Smem::VLD;
  constexpr int KCH = DQK / 8;                   // 16-byte chunks per K row
  constexpr int KCH_PER_THREAD = kBN * KCH / kThreads;
  constexpr int VCH = (kBN / 4) * (DV / 8);      // (4 keys x 8 dims) chunks of V
  static_assert(kBN * KCH % kThreads == 0, "K tile split");
  static_assert(VCH <= kThreads, "V tile split");

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int b = item.seq, qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = a.off[b];
  const int n = static_cast<int>(a.off[b + 1] - seq0);
  const int q0 = qt * kAttnBM;

  __shared__ __align__(16) Smem sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 31, lh = l >> 5;
  const int qa = q0 + w * 32;                 // first query row of this wave
  const int qrow = qa + lr;                   // this lane's query column of S^T
  const int wave_qmax = qa + 31;
  const bool has_time = a.time_table != nullptr;
  const bool has_pos = a.pos_table != nullptr;
  const int Bp = a.pos_buckets, Bt = a.time_buckets;

  // bias tables of head h, pre-multiplied by log2(e)
  if (has_pos) {
    for (int i = tid; i < min(Bp, kPosLdsFast); i += kThreads) sm.pos[i] = kLog2e * a.pos_table[h * Bp + i];
  }
  if (has_time) {
    for (int i = tid; i < min(Bt, kTimeLds); i += kThreads) sm.time[i] = kLog2e * a.time_table[h * Bt + i];
  }

  const __bf16* qp = static_cast<const __bf16*>(a.q);
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);

  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    qf[kb] = qrow < n ? *reinterpret_cast<const bf16x8_t*>(qp + (seq0 + qrow) * a.ldq + h * DQK + kb * 16 + lh * 8)
                      : bf16x8_t{};
  }
  // query timestamps: this lane's, and the wave's min / max over rows inside the sequence
  int64_t tq = 0, wq_min = 0, wq_max = 0;
  if (has_time) {
    tq = qrow < n ? a.ts[seq0 + qrow] : 0;
    wq_min = wave_min64(qrow < n ? tq : INT64_MAX, 64);
    wq_max = wave_max64(qrow < n ? tq : INT64_MIN, 64);
    wq_min = uniform_i64(wq_min);
    wq_max = uniform_i64(wq_max);
  }

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};

  const float alpha_l = a.alpha * kLog2e;
  const int kv_end = min(n, q0 + kAttnBM);
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- register staging of one K/V tile (global -> registers -> LDS)
  bf16x8_t kreg[KCH_PER_THREAD];
  bf16x8_t vreg[4];
  int64_t treg = 0;
  auto load_tile = [&](int kt) {
    const int k0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < KCH_PER_THREAD; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / KCH, c8 = c % KCH;
      kreg[i] = (k0 + r < n) ? *reinterpret_cast<const bf16x8_t*>(kp + (seq0 + k0 + r) * a.ldk + h * DQK + c8 * 8)
                             : bf16x8_t{};
    }
    if (tid < VCH) {
      const int kq = tid % (kBN / 4), d0 = (tid / (kBN / 4)) * 8;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kv = k0 + kq * 4 + r;
        vreg[r] = kv < n ? *reinterpret_cast<const bf16x8_t*>(vp + (seq0 + kv) * a.ldv + h * DV + d0) : bf16x8_t{};
      }
    }
    if (has_time && tid < kBN) treg = (k0 + tid < n) ? a.ts[seq0 + k0 + tid] : 0;
  };
  auto store_tile = [&](int kt, int buf) {
    const int k0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < KCH_PER_THREAD; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / KCH, c8 = c % KCH;
      *reinterpret_cast<bf16x8_t*>(&sm.k[buf][r * KLD + c8 * 8]) = kreg[i];
    }
    if (tid < VCH) {
      const int kq = tid % (kBN / 4), d0 = (tid / (kBN / 4)) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bf16x4_t col = {vreg[0][i], vreg[1][i], vreg[2][i], vreg[3][i]};
        *reinterpret_cast<bf16x4_t*>(&sm.vt[buf][(d0 + i) * VLD + kq * 4]) = col;
      }
    }
    if (has_time && tid < kBN) {  // wave 0: one key per lane, 32-key blocks = lane halves
      const bool inside = k0 + tid < n;
      const int64_t kmin = wave_min64(inside ? treg : INT64_MAX, 32);
      const int64_t kmax = wave_max64(inside ? treg : INT64_MIN, 32);
      const int64_t rel = treg - kmin;
      sm.tt[buf].rel[tid] = inside ? static_cast<int32_t>(rel < kInt32Max ? rel : kInt32Max) : 0;
      sm.tt[buf].raw[tid] = treg;
      if ((tid & 31) == 0) {
        sm.tt[buf].kmin[tid >> 5] = kmin;
        sm.tt[buf].kmax[tid >> 5] = kmax;
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const int k0 = kt * kBN;
    if (kt + 1 < ntiles) load_tile(kt + 1);

    if (qa < n && k0 <= wave_qmax) {
#pragma unroll
      for (int kvb = 0; kvb < kBN / 32; ++kvb) {
        const int ka = k0 + kvb * 32;
        if (ka > wave_qmax || ka >= n) break;

        // ---- classify the block (wave-uniform)
        int path = kUniform;
        float c_lo = 0.f, c_hi = 0.f;
        int32_t lim = 0;      // kTwoTime: key rel <= lim  <=>  gap >= threshold
        int32_t tq_rel = 0;   // kGeneral: clamp(t_q - kvmin, -1, 2^31 - 1)
        int64_t kvmin = 0;
        const bool need_mask = (ka + 31 > qa) || (ka + 31 >= n);
        const bool pos_uniform = !has_pos || (qa - (ka + 31) >= Bp - 1);
        if (has_pos) c_lo = (Bp - 1 < kPosLdsFast) ? sm.pos[Bp - 1] : kLog2e * a.pos_table[h * Bp + Bp - 1];
        c_hi = c_lo;
        if (has_time) {
          kvmin = sm.tt[buf].kmin[kvb];
          const int64_t kvmax = sm.tt[buf].kmax[kvb];
          const int64_t dlo = wq_min - kvmax, dhi = wq_max - kvmin;
          const int blo = time_bucket64(dlo, Bt), bhi = time_bucket64(dhi, Bt);
          if (!pos_uniform || need_mask) {
            path = dhi < int64_t(kInt32Max) - 1 ? kGeneral : kGeneral64;
          } else if (blo == bhi) {
            path = kUniform;
            c_lo += sm.time[blo];
            c_hi = c_lo;
          } else if (bhi == blo + 1) {
            path = kTwoTime;
            const float base = c_lo;
            c_lo = base + sm.time[blo];
            c_hi = base + sm.time[bhi];
            const int64_t thr = (int64_t(1) << (blo + 1)) - 1;     // gap >= thr <=> bucket bhi
            const int64_t lim64 = tq - kvmin - thr;                  // per lane
            lim = static_cast<int32_t>(lim64 < -1 ? -1 : (lim64 > kInt32Max - 1 ? kInt32Max - 1 : lim64));
          } else {
            path = dhi < int64_t(kInt32Max) - 1 ? kGeneral : kGeneral64;
          }
          const int64_t trel = tq - kvmin;
          tq_rel = static_cast<int32_t>(trel < -1 ? -1 : (trel > kInt32Max ? kInt32Max : trel));
        } else if (!pos_uniform || need_mask) {
          path = kGeneral;
        }
        path = uniform_int(path);

        // ---- S^T block = K Q^T
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&sm.k[buf][(kvb * 32 + lr) * KLD + kb * 16 + lh * 8]);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], s, 0, 0, 0);
        }
        // s[j] = S^T[key ka + 8(j/4) + 4 lh + j%4][query qrow]
        float p[16];
        if (path == kUniform) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float x = fmaf(s[j], alpha_l, c_lo);
            p[j] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x));
          }
        } else if (path == kTwoTime) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int4 rk = *reinterpret_cast<const int4*>(&sm.tt[buf].rel[kvb * 32 + 8 * g + 4 * lh]);
            const int32_t rr[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float c = rr[e] <= lim ? c_hi : c_lo;
              const float x = fmaf(s[4 * g + e], alpha_l, c);
              p[4 * g + e] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x));
            }
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            int32_t rr[4] = {0, 0, 0, 0};
            if (has_time) {
              const int4 rk = *reinterpret_cast<const int4*>(&sm.tt[buf].rel[kvb * 32 + 8 * g + 4 * lh]);
              rr[0] = rk.x; rr[1] = rk.y; rr[2] = rk.z; rr[3] = rk.w;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int kvl = kvb * 32 + 8 * g + 4 * lh + e;
              const int kv = k0 + kvl;
              float c = 0.f;
              if (has_pos) {
                const int pb = min(max(qrow - kv, 0), Bp - 1);
                c = pb < kPosLdsFast ? sm.pos[pb] : kLog2e * a.pos_table[h * Bp + pb];
              }
              if (has_time) {
                int tb;
                if (path == kGeneral) {
                  const int32_t dt = max(tq_rel - rr[e], 0);
                  tb = min(31 - __clz(dt + 1), Bt - 1);
                } else {
                  tb = time_bucket64(tq - sm.tt[buf].raw[kvl], Bt);
                }
                c += sm.time[tb];
              }
              const float x = fmaf(s[4 * g + e], alpha_l, c);
              const float pv = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x));
              p[4 * g + e] = (kv <= qrow && kv < n) ? pv : 0.0f;
            }
          }
        }

        // ---- O += P V  (A = P from the S^T registers, B = V^T from LDS)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8_t pa;
#pragma unroll
          for (int i = 0; i < 8; ++i) pa[i] = static_cast<__bf16>(p[kk * 8 + i]);
          const int kbase = kvb * 32 + kk * 16;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const __bf16* vrow = &sm.vt[buf][(nb * 32 + lr) * VLD + kbase + 4 * lh];
            const bf16x4_t v0 = *reinterpret_cast<const bf16x4_t*>(vrow);
            const bf16x4_t v1 = *reinterpret_cast<const bf16x4_t*>(vrow + 8);
            const bf16x8_t vb = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, oacc[nb], 0, 0, 0);
          }
        }
      }
    }
    if (kt + 1 < ntiles) store_tile(kt + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: oacc[nb][j] = log2(e) * N * O[qa + 8(j/4) + 4 lh + j%4][nb*32 + lr]
  const float scale = (a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n)) / kLog2e;
  __bf16* op = static_cast<__bf16*>(a.o);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int qpos = qa + 8 * (j >> 2) + 4 * lh + (j & 3);
      if (qpos < n) op[(seq0 + qpos) * a.ldo + h * DV + nb * 32 + lr] = static_cast<__bf16>(oacc[nb][j] * scale);
    }
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
  const int b = item.seq, qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = a.off[b];
  const int n = static_cast<int>(a.off[b + 1] - seq0);
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

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 128 && dv == 128) return launch_items(attn_fwd_bf16_kernel<128, 128>, a, kThreads, stream);
  if (dqk == 64 && dv == 64) return launch_items(attn_fwd_bf16_kernel<64, 64>, a, kThreads, stream);
  if (dqk == 32 && dv == 32) return launch_items(attn_fwd_bf16_kernel<32, 32>, a, kThreads, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 128 && dv == 128) return launch_items(attn_fwd_f32_kernel<128, 128>, a, kF32Threads, stream);
  if (dqk == 64 && dv == 64) return launch_items(attn_fwd_f32_kernel<64, 64>, a, kF32Threads, stream);
  if (dqk == 32 && dv == 32) return launch_items(attn_fwd_f32_kernel<32, 32>, a, kF32Threads, stream);
  return hipErrorInvalidValue;
}

}  // namespace hstu
