// Kernels of one HSTU layer around the attention (daiwk reproduction notes,
// flowchart and core formula; briansu.co explainer, section 3):
//   G  = SiLU(LN(X) W_uvqk^T + b_uvqk)         ln_rows_kernel + gemm_nt_kernel<kEpiSilu>
//   Y  = LN(O) * U                              ln_rows_kernel (gated)
//   X' = X + Y W_out^T + b_out                  gemm_nt_kernel<kEpiResidual>
//
// GEMM. C[M,N] = A[M,K] B[N,K]^T: A holds tokens, B is a weight matrix in the
// nn.Linear [out, in] layout of the neurarch exported block, so both MFMA
// operands are contiguous along K and no transpose is ever needed. Wide
// outputs (N >= 1024) take 256x256 tiles of 8 waves with 128x64 each, narrow
// ones 128x128 tiles of 4 waves with 64x64 each (blocks of
// v_mfma_f32_32x32x16_bf16), K in steps of 64. A and B tiles go HBM -> LDS with
// buffer_load ... lds (rows past M / N arrive as zeros), 16-byte chunks of each
// row XOR-swizzled by the row index so the ds_read_b128 of 32 consecutive rows
// hits distinct banks; the next stage loads while the current one multiplies.
// The epilogue (bias, SiLU or residual) stages each wave's results through LDS
// so that every global access is a row-contiguous 16-byte one.
//
// LayerNorm. One wave per token row; the row lives in registers (8 features
// per lane per 512), mean and variance by wave butterflies (two passes, fp32),
// output rounded to bf16.
#include "attn_common.h"
#include "common.h"
#include "layer.h"
#include "timing.h"

namespace hstu {

namespace {

constexpr int GBK = 64;            // K per stage of K-major operands, and the K granularity of row-major ones
constexpr int kStoreNonTemporal = 2;   // buffer store cache policy: the nt bit
// SiLU outputs (G of the UVQK projection) at least this large are stored with
// the non-temporal hint. Measured on the jagged layer (49404 tokens, 200 MB of
// G): its UVQK GEMM 162 -> 146 us and the layer 5% faster; on the 8192-token
// stack (34 MB of G, which the attention then reads back) the hint made the
// layer 1% slower, so smaller outputs keep the default policy, as do the other
// epilogues (the residual projection's output is smaller than G, split
// partials are read back at once by their sum).
constexpr int64_t kStreamOutBytes = int64_t(96) << 20;

// One 16-byte store, with the non-temporal hint when NT.
template <bool NT, class V>
__device__ __forceinline__ void store16(V* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

__device__ __forceinline__ uint32_t clamp_u32(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes));
}

// s_waitcnt vmcnt(n) lgkmcnt(0) for a small compile-time n.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);   // lgkmcnt(0), expcnt not waited
}

// GEMM tile shape: BM x BN outputs per workgroup, WM x WN per wave
// ((WM/32) x (WN/32) blocks of v_mfma_f32_32x32x16_bf16), `ST` K stages of BK
// in LDS. AT / BT: the operand is stored K-major ([K][M] / [K][N], i.e. the
// product uses its transpose); its stage tile is then 64 K-rows of BM (BN)
// columns, read back with transposed LDS reads. BK = 32 (row-major operands
// only) halves a stage, so twice as many stages fit and more loads stay in
// flight when K is short.
template <int BM, int BN, int WM, int WN, int ST, bool AT, bool BT, int BK = 64>
struct GemmShape {
  static constexpr int kBK = BK, kChunks = BK / 8;   // 16-byte chunks per row-major tile row
  static constexpr int kWavesM = BM / WM, kWavesN = BN / WN, kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int kAInst = BM * kChunks / 64;   // 1 KB direct loads per stage
  static constexpr int kBInst = BN * kChunks / 64;
  static constexpr int kAPer = kAInst / kWaves, kBPer = kBInst / kWaves;
  static constexpr int kLoadsPerStage = kAPer + kBPer;   // per wave
  static constexpr int kStagesAhead = ST - 1;
  static constexpr int ACH = AT ? BM / 8 : kChunks;     // 16-byte chunks per LDS row of a stage tile
  static constexpr int BCH = BT ? BN / 8 : kChunks;
  static constexpr bool kAT = AT, kBT = BT;
  static_assert(kAInst % kWaves == 0 && kBInst % kWaves == 0, "loads spread evenly over the waves");
  static_assert(ST >= 2 && ST <= 4, "stages");
  static_assert(BK == 64 || (BK == 32 && !AT && !BT), "K-major operands take 64-deep stages");
};

// Swizzle of the 16-byte chunks of one LDS row of a stage tile. The LDS
// serves a ds_read_b128 16 lanes at a time from 64 four-byte banks (256
// bytes), and the fragment reads give those 16 lanes 16 consecutive rows at
// the same logical chunk. Row-major (K-contiguous) rows of 8 chunks (128 B,
// two rows per 256 B): chunk ^ ((row >> 1) & 7) puts the 16 rows in 16
// distinct bank slots; rows of 4 chunks (four per 256 B): chunk ^ ((row >> 2)
// & 3). K-major tiles: chunk ^ (4 row mod CH) for the transposed reads of 4
// rows x 4 chunks per 16 lanes.
template <bool KMAJOR, int CH>
__device__ __forceinline__ int stage_swizzle(int r) {
  if constexpr (KMAJOR) return (4 * r) & (CH - 1);
  else if constexpr (CH == 4) return (r >> 2) & 3;
  else return (r >> 1) & 7;
}

// Direct loads of one operand's stage tile: instruction i fills LDS slots
// [64 i, 64 i + 64); slot s holds chunk (s % CH) ^ swizzle(row) of row s / CH.
template <class S, bool KMAJOR, int CH, int PER>
__device__ __forceinline__ void issue_operand(__amdgpu_buffer_rsrc_t rs, int64_t ld, int w, int lane,
                                              char* __restrict__ dst) {
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = w + S::kWaves * j, sl = i * 64 + lane, r = sl / CH,
              c = (sl % CH) ^ stage_swizzle<KMAJOR, CH>(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + i * 1024), 16,
                                             static_cast<uint32_t>(r * ld * 2 + c * 16), 0, 0, 0);
  }
}

// Buffer resource over an operand's stage tile at K offset k0. Row-major: the
// tile's rows start at `base` (row m0 of the operand), K offset k0; rows past
// the operand's end read as zeros. K-major: rows k0 .. k_end-1 of the operand,
// columns from the tile's first one; rows past k_end and columns past the last
// row's end read as zeros.
template <bool KMAJOR>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const char* base, int64_t ld, int rows_left,
                                                               int cols_left, int k0, int k_end, int K) {
  if constexpr (!KMAJOR) {
    const int64_t bytes = rows_left > 0 ? static_cast<int64_t>(rows_left - 1) * ld * 2 + (K - k0) * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + k0 * 2), 0,
                                             static_cast<int>(clamp_u32(bytes)), kRsrcFlags);
  } else {
    const int64_t bytes =
        (k_end > k0 && cols_left > 0) ? static_cast<int64_t>(k_end - k0 - 1) * ld * 2 + cols_left * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + static_cast<int64_t>(k0) * ld * 2), 0,
                                             static_cast<int>(clamp_u32(bytes)), kRsrcFlags);
  }
}

// One operand's fragment geometry. Row-major: one ds_read_b128 of the lane's
// row, chunk 2 k16 + lh (the row's swizzle folded into `o0`). K-major: two
// transposed reads (K rows 8 lh + i16/4 and + 4 of the 16-row step) of the
// lane's column; each lane gets the same 8 consecutive K of its column as the
// row-major read would.
template <bool KMAJOR, int CH>
struct Frag {
  uint32_t o0, o1;
  __device__ __forceinline__ void init(int col0, int lane) {   // col0: first row (column) of the 32-block
    const int lr = lane & 31, lh = lane >> 5;
    if constexpr (!KMAJOR) {
      const int r = col0 + lr;
      o0 = static_cast<uint32_t>(r * CH * 16 + (stage_swizzle<false, CH>(r) << 4));
      o1 = 0;
    } else {
      const int g16 = lane >> 4, i16 = lane & 15;
      const int r1 = 8 * lh + (i16 >> 2);
      const int c = col0 / 8 + 2 * (g16 & 1) + ((i16 & 3) >> 1);
      const int half = (i16 & 1) * 8;
      o0 = static_cast<uint32_t>((r1 * CH + (c ^ stage_swizzle<true, CH>(r1))) * 16 + half);
      o1 = static_cast<uint32_t>(((r1 + 4) * CH + (c ^ stage_swizzle<true, CH>(r1 + 4))) * 16 + half);
    }
  }
  __device__ __forceinline__ bf16x8_t read(const char* stage, int k16, int lh) const {
    if constexpr (!KMAJOR) {
      return *reinterpret_cast<const bf16x8_t*>(stage + (o0 ^ static_cast<uint32_t>((2 * k16 + lh) * 16)));
    } else {
      // 16 K rows further keeps the swizzle (it depends on row mod CH / 4 <= 16)
      const char* p = stage + k16 * 16 * CH * 16;
      return __builtin_shufflevector(tr_read(p + o0), tr_read(p + o1), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
};

// The fragments of one 16-deep K slice of a stage: MB of op(A), NB of op(B).
template <class S>
struct FragSet {
  bf16x8_t a[S::MB], b[S::NB];
};

template <class S>
__device__ __forceinline__ void read_frags(FragSet<S>& f, const char* __restrict__ sa_, const char* __restrict__ sb_,
                                           int k16, int lh, const Frag<S::kAT, S::ACH> (&af_)[S::MB],
                                           const Frag<S::kBT, S::BCH> (&bf_)[S::NB]) {
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) f.a[mb] = af_[mb].read(sa_, k16, lh);
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) f.b[nb] = bf_[nb].read(sb_, k16, lh);
}

// One K step on stage (rs_a, rs_b), entered with the fragments of its first
// 16-deep slice in `cur`. The loads of the stage ST - 1 steps ahead go into
// (ds_a, ds_b) first. Each slice's MFMAs run while the next slice's fragments
// are read: within the stage, or -- after waiting for the next stage
// (nx_a, nx_b) to land and a barrier -- the next stage's first slice, so the
// step leaves `cur` holding it. Scheduling fences keep the reads ahead of the
// products they overlap (the compiler would otherwise sink each read to its
// first use). All buffers arrive as __restrict__ pointers, so the compiler
// knows the reads never touch the stage being filled.
//
// With `pre` (the overlapped epilogue of the previous tile requested this
// tile's first two stages, then issued its MB * 4 stores), step 0 issues no
// loads and waits for stage 1 with those stores still allowed in flight.
template <class S>
__device__ __forceinline__ void gemm_step(const GemmArgs& g, const char* __restrict__ rs_a,
                                          const char* __restrict__ rs_b, char* __restrict__ ds_a,
                                          char* __restrict__ ds_b, const char* __restrict__ nx_a,
                                          const char* __restrict__ nx_b, int kt, int nsteps, int kbase_elems,
                                          int k_end, const char* abase, int arows, const char* bbase, int brows,
                                          int w, int lane, const Frag<S::kAT, S::ACH> (&af_)[S::MB],
                                          const Frag<S::kBT, S::BCH> (&bf_)[S::NB], FragSet<S>& cur,
                                          f32x16_t (&acc)[S::MB][S::NB], bool pre = false) {
  const bool pre0 = pre && kt == 0;
  if (kt + S::kStagesAhead < nsteps && !pre0) {
    const int k0 = kbase_elems + (kt + S::kStagesAhead) * S::kBK;
    issue_operand<S, S::kAT, S::ACH, S::kAPer>(operand_rsrc<S::kAT>(abase, g.lda, arows, arows, k0, k_end, g.K),
                                              g.lda, w, lane, ds_a);
    issue_operand<S, S::kBT, S::BCH, S::kBPer>(operand_rsrc<S::kBT>(bbase, g.ldb, brows, brows, k0, k_end, g.K),
                                              g.ldb, w, lane, ds_b);
  }
  const int lh = lane >> 5;
  constexpr int KS = S::kBK / 16;
#pragma unroll
  for (int k16 = 0; k16 < KS; ++k16) {
    FragSet<S> nxt;
    if (k16 + 1 < KS) {
      read_frags<S>(nxt, rs_a, rs_b, k16 + 1, lh, af_, bf_);
    } else {
      // The next stage must have landed; the ones issued since may stay in flight.
      asm volatile("" ::: "memory");
      const int ahead = nsteps - 1 - (kt + 1);   // stages issued beyond the next one, capped below
      if (pre0) {
        wait_vm_lgkm0<S::MB * 4>();
      } else if (ahead >= S::kStagesAhead - 1) {
        if constexpr (S::kStagesAhead == 3) wait_vm_lgkm0<2 * S::kLoadsPerStage>();
        else if constexpr (S::kStagesAhead == 2) wait_vm_lgkm0<S::kLoadsPerStage>();
        else wait_vm_lgkm0<0>();
      } else if (S::kStagesAhead == 3 && ahead == 1) {
        wait_vm_lgkm0<S::kLoadsPerStage>();
      } else {
        wait_vm_lgkm0<0>();
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + 1 < nsteps) read_frags<S>(nxt, nx_a, nx_b, 0, lh, af_, bf_);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[nb], cur.a[mb], acc[mb][nb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  }
}

template <int EPI, int BM, int BN, int WM, int WN, int ST, bool AT, bool BT, int BK, bool OVL, bool NT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 2) void gemm_kernel(GemmArgs g) {
  using S = GemmShape<BM, BN, WM, WN, ST, AT, BT, BK>;
  // OVL (looping workgroups, bf16 outputs rounded once): the epilogue stages
  // bf16 values in an area of its own, so the stage buffers are free once the
  // last K step has passed its barrier. The next tile's first stage is then
  // requested before this tile's epilogue, and the barrier that publishes it
  // waits for those loads only (vmcnt counts the epilogue's stores, issued
  // after them, as still in flight): the epilogue hides the load latency and
  // the stores drain under the next tile's first products.
  static_assert(!OVL || ((EPI == kEpiNone || EPI == kEpiSilu) && !AT && !BT && ST == 2 && WN == 64),
                "overlapped epilogue: row-major operands, two stages, bf16 output rounded once");
  __shared__ __attribute__((aligned(16))) char sa[ST][BM * BK * 2];
  __shared__ __attribute__((aligned(16))) char sb[ST][BN * BK * 2];
  __shared__ __attribute__((aligned(16))) char so[OVL ? S::kWaves * 32 * WN * 2 : 16];

  // Workgroups are dealt to the 8 XCDs in turn (block b to XCD b % 8). Tile t
  // of the row-major tile order goes to a block on XCD t / ceil-share, so each
  // XCD's L2 serves a contiguous band of A rows against all of B.
  // With group_m > 1 the order walks bands of group_m tile rows column by
  // column instead, so the workgroups resident on one XCD share a short band
  // of A rows and a few B tiles (for outputs far wider than tall).
  // A grid smaller than the tile count (a multiple of 8 workgroups) loops:
  // workgroup b takes virtual blocks b, b + grid, ..., each mapped as above, so
  // a tile's stores drain while the next tile's products run.
  const int tiles_n = (g.N + BN - 1) / BN;
  const int tiles = ((g.M + BM - 1) / BM) * tiles_n, q = tiles / 8, r = tiles % 8;
  auto tile_origin = [&](int vb_, int& m0_, int& n0_) __attribute__((always_inline)) {
    const int xcd = vb_ % 8;
    const int t = xcd * q + min(xcd, r) + vb_ / 8;
    int tm, tn;
    if (g.group_m > 1) {
      const int tiles_m = (g.M + BM - 1) / BM;
      const int band = t / (g.group_m * tiles_n), idx = t - band * g.group_m * tiles_n;
      const int rows = min(g.group_m, tiles_m - band * g.group_m);
      tm = band * g.group_m + idx % rows;
      tn = idx / rows;
    } else {
      tm = t / tiles_n;
      tn = t % tiles_n;
    }
    m0_ = tm * BM;
    n0_ = tn * BN;
  };
  bool stage0_ready = false;   // OVL: this tile's first stage was requested and has landed
  for (int vb = blockIdx.x; vb < tiles; vb += gridDim.x) {
  int m0, n0;
  tile_origin(vb, m0, n0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wm = w / S::kWavesN, wn = w % S::kWavesN;

  // K range of this split (blockIdx.y of gridDim.y); only K-major operands split K
  const int ksteps_all = (g.K + BK - 1) / BK;
  const int per = (ksteps_all + gridDim.y - 1) / gridDim.y;
  const int ks0 = blockIdx.y * per;
  const int nsteps = max(0, min(per, ksteps_all - ks0));
  const int kbase_elems = ks0 * BK, k_end = min(g.K, (ks0 + nsteps) * BK);

  // operand bases: row-major -> first row of the tile; K-major -> first column of the tile
  const char* abase = static_cast<const char*>(g.a) + (AT ? static_cast<int64_t>(m0) * 2 : static_cast<int64_t>(m0) * g.lda * 2);
  const char* bbase = static_cast<const char*>(g.b) + (BT ? static_cast<int64_t>(n0) * 2 : static_cast<int64_t>(n0) * g.ldb * 2);
  const int arows = g.M - m0, brows = g.N - n0;   // rows (row-major) or columns (K-major) left

  f32x16_t acc[S::MB][S::NB];
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) acc[mb][nb] = f32x16_t{};

  Frag<AT, S::ACH> af_[S::MB];
  Frag<BT, S::BCH> bf_[S::NB];
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) af_[mb].init(wm * WM + mb * 32, lane);
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) bf_[nb].init(wn * WN + nb * 32, lane);

  if (!stage0_ready) {
    // stages 0 .. ST-2 in flight, wait for stage 0
#pragma unroll
    for (int s_ = 0; s_ < ST - 1; ++s_)
      if (s_ < nsteps) {
        const int k0 = kbase_elems + s_ * BK;
        issue_operand<S, AT, S::ACH, S::kAPer>(operand_rsrc<AT>(abase, g.lda, arows, arows, k0, k_end, g.K), g.lda,
                                              w, lane, sa[s_]);
        issue_operand<S, BT, S::BCH, S::kBPer>(operand_rsrc<BT>(bbase, g.ldb, brows, brows, k0, k_end, g.K), g.ldb,
                                              w, lane, sb[s_]);
      }
    // wait for stage 0 only; the later ones stay in flight
    if (nsteps >= ST - 1) wait_vm_lgkm0<(ST - 2) * S::kLoadsPerStage>();
    else wait_vm_lgkm0<0>();
    __syncthreads();
  }
  // stages rotate statically; step t reads stage t % ST, fills (t + ST - 1) % ST
  // and ends with the first fragments of stage (t + 1) % ST in registers
  FragSet<S> cur;
  if (nsteps > 0) read_frags<S>(cur, sa[0], sb[0], 0, lane >> 5, af_, bf_);
  for (int kt = 0; kt < nsteps; kt += ST) {
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      if (kt + u >= nsteps) break;
      gemm_step<S>(g, sa[u], sb[u], sa[(u + ST - 1) % ST], sb[(u + ST - 1) % ST], sa[(u + 1) % ST],
                   sb[(u + 1) % ST], kt + u, nsteps, kbase_elems, k_end, abase, arows, bbase, brows, w, lane, af_,
                   bf_, cur, acc, OVL && stage0_ready);
    }
  }

  if constexpr (OVL) {
    // (the bias loads go out before the next stage's, so that waiting for
    // them does not wait for the stage)
    float bias[S::NB][4][4];
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int n = n0 + wn * WN + nb * 32 + 8 * jq + 4 * lh;
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[nb][jq][i] = (g.bias && n + i < g.N) ? g.bias[n + i] : 0.f;
      }
    // The last K step ended with a barrier after every wave's final fragment
    // reads, so both stage buffers are free: request the next tile's first two
    // stages now, stage s into buffer s. (An odd step count would leave the
    // first stage in buffer 1: those tiles take the plain prologue.)
    const int vn = vb + static_cast<int>(gridDim.x);
    stage0_ready = vn < tiles && nsteps > 0 && nsteps % ST == 0;
    if (stage0_ready) {
      int m1, n1;
      tile_origin(vn, m1, n1);
      const char* a1 = static_cast<const char*>(g.a) + static_cast<int64_t>(m1) * g.lda * 2;
      const char* b1 = static_cast<const char*>(g.b) + static_cast<int64_t>(n1) * g.ldb * 2;
#pragma unroll
      for (int s_ = 0; s_ < ST; ++s_) {
        const int k0 = kbase_elems + s_ * BK;
        issue_operand<S, false, S::ACH, S::kAPer>(
            operand_rsrc<false>(a1, g.lda, g.M - m1, g.M - m1, k0, k_end, g.K), g.lda, w, lane, sa[s_]);
        issue_operand<S, false, S::BCH, S::kBPer>(
            operand_rsrc<false>(b1, g.ldb, g.N - n1, g.N - n1, k0, k_end, g.K), g.ldb, w, lane, sb[s_]);
      }
    }
    // Epilogue: acc[mb][nb][4 jq + i] holds C[m][n + i] for m = 32 mb + lr,
    // n = 32 nb + 8 jq + 4 lh (wave-tile coordinates; the products ran as
    // B A^T). Each 32-row slice is rounded to bf16 once, staged in the wave's
    // 32 x 64 area (8-byte pieces, 16-byte chunks XOR-swizzled by row / 2) and
    // read back as one 16-byte chunk per lane, 8 rows per store. The stores
    // are buffer stores, issued by every lane (an index outside the tile's
    // rows or columns is past the resource and dropped), so each wave issues
    // exactly MB * 4 of them, which the wait below counts. With NT they
    // carry the non-temporal hint: the retrieval head's logits are written
    // once and not read back here, and without the hint they drained 22%
    // slower.
    char* stg = so + w * (32 * WN * 2);
    const int rows_here = min(BM, g.M - m0);
    const int64_t span = static_cast<int64_t>(rows_here - 1) * g.ldc * 2 + static_cast<int64_t>(g.N) * 2;
    const uint32_t oob = clamp_u32(span);
    const __amdgpu_buffer_rsrc_t rc_out = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(g.c) + static_cast<int64_t>(m0) * g.ldc * 2, 0, static_cast<int>(oob), kRsrcFlags);
    const int rr = lane >> 3, rc = lane & 7;
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          bf16x4_t x;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acc[mb][nb][4 * jq + i] + bias[nb][jq][i];
            if (EPI == kEpiSilu) v = silu_f32(v);
            x[i] = static_cast<__bf16>(v);
          }
          const int c16 = nb * 4 + jq;
          *reinterpret_cast<bf16x4_t*>(stg + lr * (WN * 2) + ((c16 ^ ((lr >> 1) & 7)) << 4) + lh * 8) = x;
        }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = rr + 8 * it;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + row * (WN * 2) + ((rc ^ ((row >> 1) & 7)) << 4));
        const int ml = wm * WM + mb * 32 + row, n = n0 + wn * WN + 8 * rc;
        const uint32_t off = (ml < rows_here && n < g.N)
                                 ? static_cast<uint32_t>((static_cast<int64_t>(ml) * g.ldc + n) * 2)
                                 : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v, rc_out, off, 0, NT ? kStoreNonTemporal : 0);
      }
    }
    if (stage0_ready) {
      // the next tile's first stage has landed (its second stage and the
      // stores may stay in flight); the barrier publishes it
      wait_vm_lgkm0<S::MB * 4 + S::kLoadsPerStage>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    continue;
  }

  // Epilogue. The products ran as B A^T, so acc[mb][nb][4 jq + i] holds
  // C[m][n + i] for m = 32 mb + lr, n = 32 nb + 8 jq + 4 lh (wave-tile
  // coordinates). Each 32-row slice (one mb) goes through a wave-private fp32
  // staging area of 32 rows x WN columns in the (now idle) A stage buffers,
  // 16-byte chunks XOR-swizzled by row, and leaves as row-contiguous stores
  // of 8 values per lane (one instruction covers 8 rows). Bias and SiLU apply
  // before staging, the residual after it; bf16 rounding happens once.
  constexpr int kRowChunks = WN / 4;             // 16-byte fp32 chunks per staged row
  static_assert(kRowChunks == 16, "staging swizzle assumes 64-column wave tiles");
  static_assert(S::kWaves * 32 * WN * 4 <= sizeof(sa), "staging fits in the A stage buffers");
  char* stage = &sa[0][0] + w * (32 * WN * 4);
  float bias[S::NB][4][4];
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int n = n0 + wn * WN + nb * 32 + 8 * jq + 4 * lh;
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[nb][jq][i] = (EPI != kEpiF32 && g.bias && n + i < g.N) ? g.bias[n + i] : 0.f;
    }
  char* cp = static_cast<char*>(g.c);
  const char* rp = static_cast<const char*>(g.r);
  const int rr = lane >> 3, rc = lane & 7;   // read-back: row rr (+ 8 it), chunk pair rc
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        f32x4_t x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[mb][nb][4 * jq + i] + bias[nb][jq][i];
          if (EPI == kEpiSilu) v = silu_f32(v);
          x[i] = v;
        }
        const int chunk = nb * 8 + 2 * jq + lh;
        *reinterpret_cast<f32x4_t*>(stage + lr * (WN * 4) + ((chunk ^ (lr & 15)) << 4)) = x;
      }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = rr + 8 * it;
      const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(stage + row * (WN * 4) + (((2 * rc) ^ (row & 15)) << 4));
      const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(stage + row * (WN * 4) + (((2 * rc + 1) ^ (row & 15)) << 4));
      const int m = m0 + wm * WM + mb * 32 + row, n = n0 + wn * WN + 8 * rc;
      if (m >= g.M || n >= g.N) continue;
      if constexpr (EPI == kEpiF32) {
        float* op = reinterpret_cast<float*>(cp) + static_cast<int64_t>(blockIdx.y) * g.split_stride +
                    static_cast<int64_t>(m) * g.ldc + n;
        store16<NT>(reinterpret_cast<f32x4_t*>(op), lo);
        store16<NT>(reinterpret_cast<f32x4_t*>(op + 4), hi);
        continue;
      }
      float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (EPI == kEpiResidual) {
        const bf16x8_t rv = *reinterpret_cast<const bf16x8_t*>(rp + (static_cast<int64_t>(m) * g.ldr + n) * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] += static_cast<float>(rv[i]);
      }
      bf16x8_t out;
      if (EPI == kEpiSiluPair) {
        bf16x8_t pre;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pre[i] = static_cast<__bf16>(x[i]);
          out[i] = static_cast<__bf16>(silu_f32(x[i]));
        }
        store16<NT>(reinterpret_cast<bf16x8_t*>(static_cast<char*>(g.c2) + (static_cast<int64_t>(m) * g.ldc2 + n) * 2),
                    pre);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = static_cast<__bf16>(x[i]);
      }
      store16<NT>(reinterpret_cast<bf16x8_t*>(cp + (static_cast<int64_t>(m) * g.ldc + n) * 2), out);
    }
  }
  // the staging area (A stage buffers) is read back before the next tile's loads refill it
  if (vb + static_cast<int>(gridDim.x) < tiles) __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// LayerNorm over a token row (optionally times a gate row), one wave per row.
// ----------------------------------------------------------------------------
// RMS: y = x / sqrt(mean(x^2) + eps) * gamma (gamma NULL: ones), no mean, no shift.
template <int D, bool RMS>
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
  float mean = 0.f;
  if (!RMS) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += x[i];
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    mean = s * (1.0f / D);
  }
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
      float y;
      if (RMS)
        y = x[c * 8 + i] * rstd * (a.gamma ? a.gamma[f0 + i] : 1.0f);
      else
        y = (x[c * 8 + i] - mean) * rstd * a.gamma[f0 + i] + a.beta[f0 + i];
      if (gp) y *= static_cast<float>(gv[i]);
      out[i] = static_cast<__bf16>(y);
    }
    *reinterpret_cast<bf16x8_t*>(yp + f0) = out;
  }
}

}  // namespace

namespace {
template <int EPI, int BM, int BN, int WM, int WN, int ST, bool AT, bool BT, int BK = 64, bool OVL = false,
          bool NT = false>
hipError_t launch_gemm_shape(const GemmArgs& g, int splits, hipStream_t stream) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int grid = g.blocks > 0 && g.blocks < tiles ? g.blocks : tiles;
  hipLaunchKernelGGL((gemm_kernel<EPI, BM, BN, WM, WN, ST, AT, BT, BK, OVL, NT>), dim3(grid, splits),
                     dim3((BM / WM) * (BN / WN) * 64), 0, stream, g);
  return hipGetLastError();
}
template <int EPI, bool AT, bool BT>
hipError_t launch_gemm_epi(const GemmArgs& g, int splits, hipStream_t stream) {
  // wide outputs: 256 x 256 tiles, 8 waves of 128 x 64; narrow ones: 128 x 128, 4 waves of 64 x 64.
  // Large SiLU outputs (the forward UVQK projection's G) take the non-temporal stores.
  if constexpr (EPI == kEpiSilu && !AT && !BT)
    if (g.N >= 1024 && g.stream_out)
      return launch_gemm_shape<EPI, 256, 256, 128, 64, 2, AT, BT, 64, false, true>(g, splits, stream);
  if (g.N >= 1024) return launch_gemm_shape<EPI, 256, 256, 128, 64, 2, AT, BT>(g, splits, stream);
  return launch_gemm_shape<EPI, 128, 128, 64, 64, 2, AT, BT>(g, splits, stream);
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
}  // namespace

namespace {
hipError_t check_gemm(const GemmArgs& g, int epi, bool a_kmajor, bool b_kmajor, int splits) {
  // a row-major operand steps through K in whole stages; K-major ones take any K
  if ((!a_kmajor || !b_kmajor) && g.K % GBK != 0) return hipErrorInvalidValue;
  if (splits < 1 || (splits > 1 && epi != kEpiF32) || g.K <= 0) return hipErrorInvalidValue;
  // 16-byte epilogue accesses: eight-column groups, 16-byte aligned rows
  if (g.N % 8 != 0 || !aligned(g.c, 16)) return hipErrorInvalidValue;
  if (epi == kEpiF32) {
    if (g.ldc % 4 != 0 || (splits > 1 && g.split_stride % 4 != 0)) return hipErrorInvalidValue;
  } else if (g.ldc % 8 != 0) {
    return hipErrorInvalidValue;
  }
  if (epi == kEpiResidual && (g.ldr % 8 != 0 || !aligned(g.r, 16))) return hipErrorInvalidValue;
  if (epi == kEpiSiluPair && (g.ldc2 % 8 != 0 || !aligned(g.c2, 16))) return hipErrorInvalidValue;
  if (g.group_m < 0 || g.blocks < 0 || g.blocks % 8 != 0) return hipErrorInvalidValue;
  return hipSuccess;
}
}  // namespace

hipError_t launch_gemm(const GemmArgs& g_in, int epi, bool a_kmajor, bool b_kmajor, int splits, hipStream_t stream) {
  if (g_in.M <= 0 || g_in.N <= 0) return hipSuccess;
  if (hipError_t e = check_gemm(g_in, epi, a_kmajor, b_kmajor, splits); e != hipSuccess) return e;
  GemmArgs g = g_in;
  g.stream_out = epi == kEpiSilu && static_cast<int64_t>(g.M) * g.N * 2 >= kStreamOutBytes;
  TimedScope timed(epi == kEpiResidual ? kTimedGemmOut : kTimedGemmUvqk, stream);
  if (!a_kmajor && !b_kmajor) {
    switch (epi) {
      case kEpiSilu: return launch_gemm_epi<kEpiSilu, false, false>(g, splits, stream);
      case kEpiResidual: return launch_gemm_epi<kEpiResidual, false, false>(g, splits, stream);
      case kEpiNone: return launch_gemm_epi<kEpiNone, false, false>(g, splits, stream);
      case kEpiSiluPair: return launch_gemm_epi<kEpiSiluPair, false, false>(g, splits, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (!a_kmajor && b_kmajor && epi == kEpiNone) return launch_gemm_epi<kEpiNone, false, true>(g, splits, stream);
  if (a_kmajor && b_kmajor && epi == kEpiF32) return launch_gemm_epi<kEpiF32, true, true>(g, splits, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_nt(const GemmArgs& g, int epi, hipStream_t stream) {
  return launch_gemm(g, epi, false, false, 1, stream);
}

hipError_t launch_head_gemm(const GemmArgs& g_in, hipStream_t stream) {
  if (g_in.M <= 0 || g_in.N <= 0) return hipSuccess;
  if (hipError_t e = check_gemm(g_in, kEpiNone, false, false, 1); e != hipSuccess) return e;
  GemmArgs g = g_in;
  g.stream_out = static_cast<int64_t>(g.M) * g.N * 2 >= kStreamOutBytes;
  TimedScope timed(kTimedHeadGemm, stream);
  // wide outputs loop over 256 x 256 tiles with the overlapped epilogue
  if (g.N >= 1024 && g.blocks > 0 && g.ldc <= (int64_t(1) << 22))
    return launch_gemm_shape<kEpiNone, 256, 256, 128, 64, 2, false, false, 64, true, true>(g, 1, stream);
  return launch_gemm_epi<kEpiNone, false, false>(g, 1, stream);
}

hipError_t launch_rms_rows(const LnArgs& a, int width, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.rows + 3) / 4));
  TimedScope timed(kTimedRmsNorm, stream);
  switch (width) {
    case 512: hipLaunchKernelGGL((ln_rows_kernel<512, true>), grid, dim3(256), 0, stream, a); break;
    case 1024: hipLaunchKernelGGL((ln_rows_kernel<1024, true>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ln_rows(const LnArgs& a, int width, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.rows + 3) / 4));
  TimedScope timed(kTimedLayerNorm, stream);
  switch (width) {
    case 512: hipLaunchKernelGGL((ln_rows_kernel<512, false>), grid, dim3(256), 0, stream, a); break;
    case 1024: hipLaunchKernelGGL((ln_rows_kernel<1024, false>), grid, dim3(256), 0, stream, a); break;
    case 2048: hipLaunchKernelGGL((ln_rows_kernel<2048, false>), grid, dim3(256), 0, stream, a); break;
    case 4096: hipLaunchKernelGGL((ln_rows_kernel<4096, false>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hstu
