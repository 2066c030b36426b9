// Internal launch interface of the layer kernels (GEMM with epilogues, LayerNorm).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

enum GemmEpilogue { kEpiSilu = 0, kEpiResidual = 1, kEpiNone = 2 };

// C[M,N] (bf16, ldc) = epi(A[M,K] B[N,K]^T + bias[N]); A, B bf16 row-major.
// kEpiSilu: SiLU; kEpiResidual: + R[M,N] (bf16, ldr). K must be a multiple of
// 64, N, ldc and ldr multiples of 8, C and R 16-byte aligned (else
// hipErrorInvalidValue).
struct GemmArgs {
  const void* a;
  int64_t lda;
  const void* b;
  int64_t ldb;
  void* c;
  int64_t ldc;
  const float* bias;   // [N] or NULL
  const void* r;       // residual (kEpiResidual)
  int64_t ldr;
  int M, N, K;
};

// y = LN(x) * gamma + beta (optionally * gate), rows of `width` features, bf16 in/out.
struct LnArgs {
  const void* x;
  int64_t ldx;
  const void* gate;    // NULL or bf16 rows (ldg)
  int64_t ldg;
  void* y;
  int64_t ldy;
  const float* gamma;
  const float* beta;
  float eps;
  int64_t rows;
};

hipError_t launch_gemm_nt(const GemmArgs& g, int epi, hipStream_t stream);
hipError_t launch_ln_rows(const LnArgs& a, int width, hipStream_t stream);

}  // namespace hstu
