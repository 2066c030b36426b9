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
template <int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  constexpr int KB = DQK / 16;   // k-blocks of the QK^T product
  constexpr int NB = DV / 32;    // 32-wide column blocks of O
  constexpr int KLD = DQK + 8;   // LDS row stride of K (bf16): 16 B shift per row
  constexpr int VLD = kBN + 4;   // LDS row stride of V^T (bf16): 8 B shift per row

  const int item_idx = blockIdx.x;
  if (item_idx >= *a.item_count) return;
  const WorkItem item = reinterpret_cast<const WorkItem*>(a.items)[item_idx];
  const int b = item.seq, qt = item_qtile(item), h = item_head(item);
  const int64_t seq0 = a.off[b];
  const int n = static_cast<int>(a.off[b + 1] - seq0);
  const int q0 = qt * kAttnBM;
  const float inv_div = a.divisor > 0.f ? 1.0f / a.divisor : 1.0f / static_cast<float>(n);

  __shared__ __align__(16) __bf16 sK[kBN * KLD];
  __shared__ __align__(16) __bf16 sVt[DV * VLD];
  __shared__ int64_t sT[kBN];
  __shared__ BiasLds sB;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 31, lh = l >> 5;
  const int qrow = q0 + w * 32 + lr;          // this lane's query column of S^T
  const int wave_qmax = q0 + w * 32 + 31;

  stage_bias_tables(sB, a, h);

  const __bf16* qp = static_cast<const __bf16*>(a.q);
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);

  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (qrow < n) {
      qf[kb] = *reinterpret_cast<const bf16x8_t*>(qp + (seq0 + qrow) * a.ldq + h * DQK + kb * 16 +
                                                  lh * 8);
    } else {
      qf[kb] = bf16x8_t{};
    }
  }
  const bool has_time = a.time_table != nullptr;
  const bool has_pos = a.pos_table != nullptr;
  const int64_t tq = (has_time && qrow < n) ? a.ts[seq0 + qrow] : 0;

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};

  const int kv_end = min(n, q0 + kAttnBM);
  const int ntiles = (kv_end + kBN - 1) / kBN;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * kBN;
    __syncthreads();  // previous tile fully consumed
    // ---- K tile [kBN][DQK] -> LDS, row-major, zero-filled past the sequence
    constexpr int KCH = DQK / 8;  // 16-byte chunks per row
    for (int c = tid; c < kBN * KCH; c += kThreads) {
      const int r = c / KCH, c8 = c % KCH;
      bf16x8_t val = bf16x8_t{};
      if (k0 + r < n) val = *reinterpret_cast<const bf16x8_t*>(kp + (seq0 + k0 + r) * a.ldk + h * DQK + c8 * 8);
      *reinterpret_cast<bf16x8_t*>(&sK[r * KLD + c8 * 8]) = val;
    }
    // ---- V tile -> LDS transposed (V^T [DV][kBN]): each thread takes 4 keys x 8 dims
    constexpr int VCH = (kBN / 4) * (DV / 8);
    for (int c = tid; c < VCH; c += kThreads) {
      const int kq = c % (kBN / 4), d0 = (c / (kBN / 4)) * 8;
      bf16x8_t rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kv = k0 + kq * 4 + r;
        rows[r] = kv < n ? *reinterpret_cast<const bf16x8_t*>(vp + (seq0 + kv) * a.ldv + h * DV + d0)
                         : bf16x8_t{};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bf16x4_t col = {rows[0][i], rows[1][i], rows[2][i], rows[3][i]};
        *reinterpret_cast<bf16x4_t*>(&sVt[(d0 + i) * VLD + kq * 4]) = col;
      }
    }
    if (has_time) {
      for (int r = tid; r < kBN; r += kThreads) sT[r] = (k0 + r < n) ? a.ts[seq0 + k0 + r] : 0;
    }
    __syncthreads();

    if (k0 > wave_qmax) continue;  // every key of this tile is after every row of this wave

#pragma unroll
    for (int kvb = 0; kvb < kBN / 32; ++kvb) {
      if (k0 + kvb * 32 > wave_qmax) break;
      f32x16_t s = f32x16_t{};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&sK[(kvb * 32 + lr) * KLD + kb * 16 + lh * 8]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], s, 0, 0, 0);
      }
      // s[j] = S^T[key = k0 + kvb*32 + 8(j/4) + 4 lh + j%4][query = qrow]
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kvl = kvb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
        const int kv = k0 + kvl;
        float x = a.alpha * s[j];
        if (has_pos) x += pos_bias(sB, a, h, qrow - kv);
        if (has_time) x += time_bias(sB, a, tq - sT[kvl]);
        const bool valid = (kv <= qrow) && (kv < n);
        p[j] = valid ? silu_f32(x) : 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t pa;
#pragma unroll
        for (int i = 0; i < 8; ++i) pa[i] = static_cast<__bf16>(p[kk * 8 + i]);
        const int kbase = kvb * 32 + kk * 16;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const __bf16* vrow = &sVt[(nb * 32 + lr) * VLD + kbase + 4 * lh];
          bf16x4_t v0 = *reinterpret_cast<const bf16x4_t*>(vrow);
          bf16x4_t v1 = *reinterpret_cast<const bf16x4_t*>(vrow + 8);
          bf16x8_t vb = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, oacc[nb], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: oacc[nb][j] = O[q0 + 32w + 8(j/4) + 4 lh + j%4][nb*32 + lr]
  __bf16* op = static_cast<__bf16*>(a.o);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int qpos = q0 + w * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
      if (qpos < n) {
        op[(seq0 + qpos) * a.ldo + h * DV + nb * 32 + lr] = static_cast<__bf16>(oacc[nb][j] * inv_div);
      }
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
