// Row kernels of the HSTU layer's backward (the chain rule through the layer
// of the daiwk reproduction notes' flowchart and core formula, in reverse):
//
//   ln_bwd_kernel<W, GATE>    gradient of y = LN(x; gamma, beta) [* gate] for
//                             upstream dy, one wave per row: dx (+ a residual
//                             gradient), d gate = dy * LN(x), and per-wave
//                             partial sums of dy_ln * xhat and dy_ln (the
//                             gamma / beta gradients), with dy_ln = dy [* gate]
//   silu_bwd_colsum_kernel    dZ = dG * SiLU'(Z) in place, plus per-block
//                             column partial sums of dZ (the bias gradient);
//                             without Z only the column sums of dG
//   sum_rows_kernel           fixed-order sums of partial rows (two levels)
//
// With xhat = (x - mean) / sqrt(var + eps) and g = dy_ln * gamma:
//     dx = (g - mean(g) - xhat * mean(g * xhat)) / sqrt(var + eps).
// Every reduction runs in a fixed order, so the gradients repeat bitwise.
#include "common.h"
#include "layer.h"

namespace hstu {

namespace {

constexpr int kLnWaves = 4;

__device__ __forceinline__ float wave_allsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void load8(const __bf16* p, float* x) {
  const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(v[i]);
}

__device__ __forceinline__ void store8(__bf16* p, const float* x) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<__bf16>(x[i]);
  *reinterpret_cast<bf16x8_t*>(p) = v;
}

// Lane `lane` owns features c * 512 + 8 lane + i (c < W / 512, i < 8).
template <int W, bool GATE>
__global__ __launch_bounds__(kLnWaves * 64) void ln_bwd_kernel(LnBwdArgs a) {
  constexpr int PER = W / 64, NC = W / 512;
  static_assert(W % 512 == 0, "row width");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float acc_g[PER], acc_b[PER], gam[PER], bet[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    acc_g[i] = acc_b[i] = 0.f;
    const int f = (i / 8) * 512 + lane * 8 + (i % 8);
    gam[i] = a.gamma[f];
    bet[i] = GATE ? a.beta[f] : 0.f;
  }
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * a.rows_per_block;
  const int64_t r1 = min(a.rows, r0 + a.rows_per_block);
  for (int64_t row = r0 + w; row < r1; row += kLnWaves) {
    const __bf16* xp = static_cast<const __bf16*>(a.x) + row * a.ldx;
    const __bf16* dyp = static_cast<const __bf16*>(a.dy) + row * a.lddy;
    float x[PER], dyl[PER];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      load8(xp + c * 512 + lane * 8, x + 8 * c);
      load8(dyp + c * 512 + lane * 8, dyl + 8 * c);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += x[i];
    const float mean = wave_allsum(s) * (1.0f / W);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      x[i] -= mean;
      q = fmaf(x[i], x[i], q);
    }
    const float rstd = rsqrtf(wave_allsum(q) * (1.0f / W) + a.eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] *= rstd;   // xhat
    if (GATE) {
      // y = LN(x) * gate: d gate = dy * LN(x), and the norm sees dy * gate
      const __bf16* gp = static_cast<const __bf16*>(a.gate) + row * a.ldg;
      __bf16* dgp = static_cast<__bf16*>(a.dgate) + row * a.lddg;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float gv[8], dg[8];
        load8(gp + c * 512 + lane * 8, gv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = 8 * c + i;
          dg[i] = dyl[k] * fmaf(x[k], gam[k], bet[k]);
          dyl[k] *= gv[i];
        }
        store8(dgp + c * 512 + lane * 8, dg);
      }
    }
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      acc_g[i] = fmaf(dyl[i], x[i], acc_g[i]);
      acc_b[i] += dyl[i];
      const float g = dyl[i] * gam[i];
      dyl[i] = g;
      m1 += g;
      m2 = fmaf(g, x[i], m2);
    }
    m1 = wave_allsum(m1) * (1.0f / W);
    m2 = wave_allsum(m2) * (1.0f / W);
    __bf16* dxp = static_cast<__bf16*>(a.dx) + row * a.lddx;
    const __bf16* rp = a.resid ? static_cast<const __bf16*>(a.resid) + row * a.ldr : nullptr;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float o[8], rv[8];
      if (rp) load8(rp + c * 512 + lane * 8, rv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 8 * c + i;
        o[i] = (dyl[k] - m1 - x[k] * m2) * rstd + (rp ? rv[i] : 0.f);
      }
      store8(dxp + c * 512 + lane * 8, o);
    }
  }
  // partial row of this wave: [d gamma (W) | d beta (W)]
  float* pr = a.partial + (static_cast<int64_t>(blockIdx.x) * kLnWaves + w) * (2 * W);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int f0 = c * 512 + lane * 8;
    *reinterpret_cast<f32x4_t*>(pr + f0) = f32x4_t{acc_g[8 * c], acc_g[8 * c + 1], acc_g[8 * c + 2], acc_g[8 * c + 3]};
    *reinterpret_cast<f32x4_t*>(pr + f0 + 4) =
        f32x4_t{acc_g[8 * c + 4], acc_g[8 * c + 5], acc_g[8 * c + 6], acc_g[8 * c + 7]};
    *reinterpret_cast<f32x4_t*>(pr + W + f0) =
        f32x4_t{acc_b[8 * c], acc_b[8 * c + 1], acc_b[8 * c + 2], acc_b[8 * c + 3]};
    *reinterpret_cast<f32x4_t*>(pr + W + f0 + 4) =
        f32x4_t{acc_b[8 * c + 4], acc_b[8 * c + 5], acc_b[8 * c + 6], acc_b[8 * c + 7]};
  }
}

// SiLU'(z) = sig (1 + z (1 - sig)), sig = 1 / (1 + e^-z).
__device__ __forceinline__ float silu_grad(float z) {
  const float sg = 1.0f / (1.0f + __expf(-z));
  return sg * fmaf(z, 1.0f - sg, 1.0f);
}

// A block covers `rows_per_block` rows. Thread t owns 8 columns: column group
// (t % CT) + CT y with CT = min(256, N / 8) column threads, and row lane t / CT
// of 256 / CT lanes that take every (256 / CT)-th row, four rows in flight.
// The row lanes are summed in LDS in a fixed order: one partial row per block.
__global__ __launch_bounds__(256) void silu_bwd_colsum_kernel(ColGradArgs a) {
  const int ct = min(256, a.N / 8), lanes = 256 / ct;
  const int cg = threadIdx.x % ct, rl = threadIdx.x / ct;
  const int col = (blockIdx.y * ct + cg) * 8;
  const bool live = col < a.N && rl < lanes;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * a.rows_per_block;
  const int64_t r1 = min(a.rows, r0 + a.rows_per_block);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto one_row = [&](int64_t row) {
    __bf16* gp = static_cast<__bf16*>(a.dg) + row * a.ldg + col;
    float g[8];
    load8(gp, g);
    if (a.z) {
      float z[8];
      load8(static_cast<const __bf16*>(a.z) + row * a.ldz + col, z);
      bf16x8_t o;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 d = static_cast<__bf16>(g[i] * silu_grad(z[i]));
        o[i] = d;
        g[i] = static_cast<float>(d);   // the bias gradient sums the stored dZ
      }
      *reinterpret_cast<bf16x8_t*>(gp) = o;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += g[i];
  };
  if (live) {
    int64_t row = r0 + rl;
    for (; row + 3 * lanes < r1; row += 4 * lanes) {
#pragma unroll
      for (int u = 0; u < 4; ++u) one_row(row + u * lanes);
    }
    for (; row < r1; row += lanes) one_row(row);
  }
  __shared__ f32x4_t red[256][2];
  red[threadIdx.x][0] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
  red[threadIdx.x][1] = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  __syncthreads();
  if (rl == 0 && col < a.N) {
    f32x4_t lo = red[cg][0], hi = red[cg][1];
    for (int l = 1; l < lanes; ++l) {
      lo += red[l * ct + cg][0];
      hi += red[l * ct + cg][1];
    }
    float* pr = a.partial + static_cast<int64_t>(blockIdx.x) * a.N + col;
    *reinterpret_cast<f32x4_t*>(pr) = lo;
    *reinterpret_cast<f32x4_t*>(pr + 4) = hi;
  }
}

// One level of the partial-row sums: block (x, y) takes columns
// [64 x, 64 x + 64) of rows [G y, G y + G); its 4 row slices take every
// fourth row, then combine in LDS in a fixed order:
// out[y * W + c] = scale * sum of in[p * ld + c] over the block's rows.
__global__ __launch_bounds__(256) void sum_rows_kernel(const float* __restrict__ in, int64_t P, int64_t W,
                                                       int64_t ld, int G, float scale, float* __restrict__ out) {
  const int cl = threadIdx.x & 63, sl = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + cl;
  const int64_t p0 = static_cast<int64_t>(blockIdx.y) * G, p1 = min(P, p0 + G);
  float s = 0.f;
  if (c < W)
    for (int64_t p = p0 + sl; p < p1; p += 4) s += in[p * ld + c];
  __shared__ float red[4][64];
  red[sl][cl] = s;
  __syncthreads();
  if (sl == 0 && c < W) out[static_cast<int64_t>(blockIdx.y) * W + c] = (((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl]) * scale;
}

constexpr int kSumGroup = 64;

}  // namespace

int64_t ln_bwd_partial_rows(int64_t rows, int rows_per_block) {
  return ((rows + rows_per_block - 1) / rows_per_block) * kLnWaves;
}

hipError_t launch_ln_bwd(const LnBwdArgs& a, int width, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.rows_per_block < 1) return hipErrorInvalidValue;
  const bool gate = a.gate != nullptr;
  const dim3 grid(static_cast<unsigned>((a.rows + a.rows_per_block - 1) / a.rows_per_block));
#define HSTU_LN_BWD(W)                                                                          \
  if (width == W) {                                                                             \
    if (gate) hipLaunchKernelGGL((ln_bwd_kernel<W, true>), grid, dim3(kLnWaves * 64), 0, stream, a); \
    else hipLaunchKernelGGL((ln_bwd_kernel<W, false>), grid, dim3(kLnWaves * 64), 0, stream, a);     \
    return hipGetLastError();                                                                   \
  }
  HSTU_LN_BWD(512)
  HSTU_LN_BWD(1024)
  HSTU_LN_BWD(2048)
  HSTU_LN_BWD(4096)
#undef HSTU_LN_BWD
  return hipErrorInvalidValue;
}

int64_t colsum_partial_rows(int64_t rows, int rows_per_block) {
  return (rows + rows_per_block - 1) / rows_per_block;
}

hipError_t launch_silu_bwd_colsum(const ColGradArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.N % 8 != 0 || a.rows_per_block < 1) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((a.rows + a.rows_per_block - 1) / a.rows_per_block),
                  static_cast<unsigned>((a.N / 8 + 255) / 256));
  hipLaunchKernelGGL(silu_bwd_colsum_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

int64_t sum_rows_scratch_floats(int64_t P, int64_t W) {
  // levels of 64 rows each, ping-ponging between two halves
  int64_t need = 0;
  for (int64_t p = P; p > kSumGroup; p = (p + kSumGroup - 1) / kSumGroup) need = max(need, (p + kSumGroup - 1) / kSumGroup);
  return 2 * need * W;
}

hipError_t launch_sum_rows(const float* in, int64_t P, int64_t W, int64_t ld, float scale, float* out, float* scratch,
                           hipStream_t stream) {
  if (W <= 0) return hipSuccess;
  const unsigned cols = static_cast<unsigned>((W + 63) / 64);
  const int64_t half = sum_rows_scratch_floats(P, W) / 2;
  const float* src = in;
  int64_t rows = P, src_ld = ld;
  int flip = 0;
  // levels: 64 rows into one, until at most 64 rows are left
  while (rows > kSumGroup) {
    const int64_t groups = (rows + kSumGroup - 1) / kSumGroup;
    float* dst = scratch + flip * half;
    hipLaunchKernelGGL(sum_rows_kernel, dim3(cols, static_cast<unsigned>(groups)), dim3(256), 0, stream, src, rows, W,
                       src_ld, kSumGroup, 1.0f, dst);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    src = dst;
    rows = groups;
    src_ld = W;
    flip ^= 1;
  }
  hipLaunchKernelGGL(sum_rows_kernel, dim3(cols, 1), dim3(256), 0, stream, src, rows, W, src_ld,
                     static_cast<int>(kSumGroup), scale, out);
  return hipGetLastError();
}

}  // namespace hstu
