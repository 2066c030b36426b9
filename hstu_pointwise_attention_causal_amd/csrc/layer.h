// Internal launch interface of the layer kernels (GEMM with epilogues, LayerNorm).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

enum GemmEpilogue { kEpiSilu = 0, kEpiResidual = 1, kEpiNone = 2, kEpiSiluPair = 3, kEpiF32 = 4 };

// C[M,N] = epi(op(A) op(B)^T + bias[N]), bf16 operands, fp32 accumulation.
// op(A) is A[M,K] (row-major, lda) or, K-major, the transpose of A[K,M]
// (lda = its row stride); likewise op(B) is B[N,K] or the transpose of B[K,N].
// Epilogues (C bf16 unless noted):
//   kEpiSilu      SiLU(x)
//   kEpiResidual  x + R[M,N] (bf16, ldr)
//   kEpiNone      x
//   kEpiSiluPair  C = SiLU(x) and C2 = x (bf16, ldc2): the activation and its input
//   kEpiF32       x in fp32 (no bias); with K split over `splits` workgroup
//                 columns, split s writes its partial sum at C + s * split_stride
// Row-major operands need K a multiple of 64; N, ldc, ldr, ldc2 multiples of 8
// (ldc of 4 for fp32), C, R, C2 16-byte aligned; else hipErrorInvalidValue.
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
  void* c2;            // second output (kEpiSiluPair)
  int64_t ldc2;
  int64_t split_stride;   // elements between split partials (kEpiF32)
  int M, N, K;
  int group_m;         // > 1: tile order in bands of group_m tile rows, column by column
  int blocks;          // > 0: that many workgroups (a multiple of 8), each looping over tiles; 0: one per tile
  int stream_out;      // set by launch_gemm: large SiLU outputs stored with the non-temporal hint
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

// Backward of y = LN(x; gamma, beta) [* gate] for upstream dy, rows of
// `width` features (bf16 rows, fp32 gamma / beta): dx = LN-backward [+ resid],
// dgate = dy * LN(x) (when gate != NULL), and per-wave partial rows
// [d gamma | d beta] (2 * width fp32 each) at partial; ln_bwd_partial_rows
// gives their count.
struct LnBwdArgs {
  const void* x;
  int64_t ldx;
  const void* gate;    // NULL: no gate
  int64_t ldg;
  const void* dy;
  int64_t lddy;
  const void* resid;   // NULL or a gradient added to dx
  int64_t ldr;
  void* dx;
  int64_t lddx;
  void* dgate;         // written when gate != NULL
  int64_t lddg;
  const float* gamma;
  const float* beta;
  float eps;
  int64_t rows;
  float* partial;
  int rows_per_block;
};

// dZ = dG * SiLU'(Z) in place over rows x N (bf16), and per-block partial rows
// of its column sums (colsum_partial_rows of N fp32); with z == NULL, dG is
// left as is and only its column sums are taken.
struct ColGradArgs {
  void* dg;
  int64_t ldg;
  const void* z;
  int64_t ldz;
  int64_t rows;
  int N;
  float* partial;
  int rows_per_block;
};

hipError_t launch_gemm(const GemmArgs& g, int epi, bool a_kmajor, bool b_kmajor, int splits, hipStream_t stream);
hipError_t launch_ln_bwd(const LnBwdArgs& a, int width, hipStream_t stream);
int64_t ln_bwd_partial_rows(int64_t rows, int rows_per_block);
hipError_t launch_silu_bwd_colsum(const ColGradArgs& a, hipStream_t stream);
int64_t colsum_partial_rows(int64_t rows, int rows_per_block);
// out[c] = scale * sum over p < P of in[p * ld + c] (c < W), in a fixed order;
// scratch holds sum_rows_scratch_floats(P, W) floats (none for P <= 64).
hipError_t launch_sum_rows(const float* in, int64_t P, int64_t W, int64_t ld, float scale, float* out, float* scratch,
                           hipStream_t stream);
int64_t sum_rows_scratch_floats(int64_t P, int64_t W);
hipError_t launch_gemm_nt(const GemmArgs& g, int epi, hipStream_t stream);
hipError_t launch_ln_rows(const LnArgs& a, int width, hipStream_t stream);

// y = x / sqrt(mean(x^2) + eps) * gamma (gamma NULL: ones; beta and gate unused),
// width 512 or 1024.
hipError_t launch_rms_rows(const LnArgs& a, int width, hipStream_t stream);

// The retrieval head's C = A B^T (kEpiNone, row-major operands, no bias),
// timed on its own.
hipError_t launch_head_gemm(const GemmArgs& g, hipStream_t stream);

}  // namespace hstu
