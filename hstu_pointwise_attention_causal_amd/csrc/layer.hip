// Kernels of one HSTU layer around the attention (daiwk reproduction notes,
// flowchart and core formula; briansu.co explainer, section 3):
//   G  = SiLU(LN(X) W_uvqk^T + b_uvqk)         ln_rows_kernel + gemm_nt_kernel<kEpiSilu>
//   Y  = LN(O) * U                              ln_rows_kernel (gated)
//   X' = X + Y W_out^T + b_out                  gemm_nt_kernel<kEpiResidual>
//
// GEMM. C[M,N] = A[M,K] B[N,K]^T: A holds tokens, B is a weight matrix in the
// nn.Linear [out, in] layout of the neurarch exported block, so both MFMA
// operands are contiguous along K and no transpose is ever needed. A 128x128
// output tile per workgroup, 4 waves of 64x64 (2x2 blocks of
// v_mfma_f32_32x32x16_bf16), K in steps of 64. A and B tiles go HBM -> LDS with
// buffer_load ... lds (rows past M / N arrive as zeros), 16-byte chunks of each
// row XOR-swizzled by the row index so the ds_read_b128 of 32 consecutive rows
// hits distinct banks; two stages in flight.
//
// LayerNorm. One wave per token row; the row lives in registers (8 features
// per lane per 512), mean and variance by wave butterflies (two passes, fp32),
// output rounded to bf16.
#include "common.h"
#include "layer.h"
#include "timing.h"

namespace hstu {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kRsrcFlags = 0x00020000;

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kChunks = GBK / 8;   // 16-byte chunks per tile row

__device__ __forceinline__ uint32_t clamp_u32(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes));
}

// One K-step of A and B tiles, direct to LDS. Instruction i (of 16 per operand)
// fills LDS slots [64 i, 64 i + 64): wave w issues i = w, w + 4, w + 8, w + 12.
__device__ __forceinline__ void gemm_issue(const char* abase, int64_t lda, uint32_t arecs, const char* bbase,
                                           int64_t ldb, uint32_t brecs, int k0, int w, const uint32_t* aoff,
                                           const uint32_t* boff, char* __restrict__ sa, char* __restrict__ sb) {
  __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(abase + k0 * 2), 0,
                                                                 static_cast<int>(arecs), kRsrcFlags);
  __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(bbase + k0 * 2), 0,
                                                                 static_cast<int>(brecs), kRsrcFlags);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = w + 4 * j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(sa + i * 1024), 16, aoff[j], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(sb + i * 1024), 16, boff[j], 0, 0, 0);
  }
}

// One K-step: MFMAs on stage (rs_a, rs_b) while the next step's tiles stream
// into (ds_a, ds_b). All four buffers arrive as __restrict__ pointers, so the
// compiler knows the reads never touch the stage being filled and does not
// wait for the in-flight loads before reading LDS.
__device__ __forceinline__ void gemm_step(const GemmArgs& g, const char* __restrict__ rs_a,
                                          const char* __restrict__ rs_b, char* __restrict__ ds_a,
                                          char* __restrict__ ds_b, bool issue_next, int k_next,
                                          const char* abase, uint32_t arecs, const char* bbase, uint32_t brecs,
                                          int w, const uint32_t* aoff, const uint32_t* boff,
                                          const uint32_t (&a_lds)[2][4], const uint32_t (&b_lds)[2][4],
                                          f32x16_t (&acc)[2][2]) {
  if (issue_next) gemm_issue(abase, g.lda, arecs, bbase, g.ldb, brecs, k_next, w, aoff, boff, ds_a, ds_b);
#pragma unroll
  for (int k16 = 0; k16 < 4; ++k16) {
    bf16x8_t af[2], bfr[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      af[mb] = *reinterpret_cast<const bf16x8_t*>(rs_a + a_lds[mb][k16]);
      bfr[mb] = *reinterpret_cast<const bf16x8_t*>(rs_b + b_lds[mb][k16]);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);   // next stage landed, this stage's reads done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_nt_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char sa[2][GBM * GBK * 2];
  __shared__ __attribute__((aligned(16))) char sb[2][GBN * GBK * 2];

  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = (w + 4 * j) * 64 + lane;
    const int r = s / kChunks, c = (s % kChunks) ^ (r & 7);
    aoff[j] = static_cast<uint32_t>(r * g.lda * 2 + c * 16);
    boff[j] = static_cast<uint32_t>(r * g.ldb * 2 + c * 16);
  }
  const char* abase = static_cast<const char*>(g.a) + static_cast<int64_t>(m0) * g.lda * 2;
  const char* bbase = static_cast<const char*>(g.b) + static_cast<int64_t>(n0) * g.ldb * 2;
  // rows past M (N) are out of range: records end right after the last valid row's K range
  const uint32_t arecs = g.M > m0 ? clamp_u32(static_cast<int64_t>(g.M - m0 - 1) * g.lda * 2 + g.K * 2) : 0u;
  const uint32_t brecs = g.N > n0 ? clamp_u32(static_cast<int64_t>(g.N - n0 - 1) * g.ldb * 2 + g.K * 2) : 0u;

  f32x16_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16_t{};

  uint32_t a_lds[2][4], b_lds[2][4];   // byte offsets of this lane's fragments in a stage
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int k16 = 0; k16 < 4; ++k16) {
      const int ra = wm * 64 + mb * 32 + lr, rb = wn * 64 + mb * 32 + lr, c = 2 * k16 + lh;
      a_lds[mb][k16] = (ra * kChunks + (c ^ (ra & 7))) * 16;
      b_lds[mb][k16] = (rb * kChunks + (c ^ (rb & 7))) * 16;
    }

  gemm_issue(abase, g.lda, arecs, bbase, g.ldb, brecs, 0, w, aoff, boff, sa[0], sb[0]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nsteps = g.K / GBK;
  for (int kt = 0; kt < nsteps; kt += 2) {   // stages alternate statically: 0 -> 1 -> 0 ...
    gemm_step(g, sa[0], sb[0], sa[1], sb[1], kt + 1 < nsteps, (kt + 1) * GBK, abase, arecs, bbase, brecs, w,
              aoff, boff, a_lds, b_lds, acc);
    if (kt + 1 < nsteps)
      gemm_step(g, sa[1], sb[1], sa[0], sb[0], kt + 2 < nsteps, (kt + 2) * GBK, abase, arecs, bbase, brecs, w,
                aoff, boff, a_lds, b_lds, acc);
  }

  // epilogue: acc[mb][nb][j] = C[m0 + 64 wm + 32 mb + 8(j/4) + 4 lh + j%4][n0 + 64 wn + 32 nb + lr]
  __bf16* cp = static_cast<__bf16*>(g.c);
  const __bf16* rp = static_cast<const __bf16*>(g.r);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = n0 + wn * 64 + nb * 32 + lr;
    if (n >= g.N) continue;
    const float bias = g.bias ? g.bias[n] : 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = m0 + wm * 64 + mb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
        if (m >= g.M) continue;
        float x = acc[mb][nb][j] + bias;
        if (EPI == kEpiSilu) x = x / (1.0f + __expf(-x));
        if (EPI == kEpiResidual) x += static_cast<float>(rp[static_cast<int64_t>(m) * g.ldr + n]);
        cp[static_cast<int64_t>(m) * g.ldc + n] = static_cast<__bf16>(x);
      }
  }
}

// ----------------------------------------------------------------------------
// LayerNorm over a token row (optionally times a gate row), one wave per row.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void ln_rows_kernel(LnArgs a) {
  constexpr int PER = D / 64;          // features per lane
  static_assert(D % 512 == 0, "row width");
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const __bf16* xp = static_cast<const __bf16*>(a.x) + row * a.ldx;
  float x[PER];
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(xp + c * 512 + lane * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[c * 8 + i] = static_cast<float>(v[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += x[i];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  const float mean = s * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float d = x[i] - mean;
    q = fmaf(d, d, q);
  }
  for (int o = 32; o > 0; o >>= 1) q += __shfl_xor(q, o, 64);
  const float rstd = rsqrtf(q * (1.0f / D) + a.eps);
  __bf16* yp = static_cast<__bf16*>(a.y) + row * a.ldy;
  const __bf16* gp = a.gate ? static_cast<const __bf16*>(a.gate) + row * a.ldg : nullptr;
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    const int f0 = c * 512 + lane * 8;
    bf16x8_t gv;
    if (gp) gv = *reinterpret_cast<const bf16x8_t*>(gp + f0);
    bf16x8_t out;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y = (x[c * 8 + i] - mean) * rstd * a.gamma[f0 + i] + a.beta[f0 + i];
      if (gp) y *= static_cast<float>(gv[i]);
      out[i] = static_cast<__bf16>(y);
    }
    *reinterpret_cast<bf16x8_t*>(yp + f0) = out;
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmArgs& g, int epi, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tiles = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
  TimedScope timed(epi == kEpiResidual ? kTimedGemmOut : kTimedGemmUvqk, stream);
  if (epi == kEpiSilu)
    hipLaunchKernelGGL(gemm_nt_kernel<kEpiSilu>, dim3(tiles), dim3(kGemmThreads), 0, stream, g);
  else if (epi == kEpiResidual)
    hipLaunchKernelGGL(gemm_nt_kernel<kEpiResidual>, dim3(tiles), dim3(kGemmThreads), 0, stream, g);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<kEpiNone>, dim3(tiles), dim3(kGemmThreads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_ln_rows(const LnArgs& a, int width, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.rows + 3) / 4));
  TimedScope timed(kTimedLayerNorm, stream);
  switch (width) {
    case 512: hipLaunchKernelGGL(ln_rows_kernel<512>, grid, dim3(256), 0, stream, a); break;
    case 1024: hipLaunchKernelGGL(ln_rows_kernel<1024>, grid, dim3(256), 0, stream, a); break;
    case 2048: hipLaunchKernelGGL(ln_rows_kernel<2048>, grid, dim3(256), 0, stream, a); break;
    case 4096: hipLaunchKernelGGL(ln_rows_kernel<4096>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hstu
