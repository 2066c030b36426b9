/*
 * hstu.h -- C ABI of the MI355X (gfx950) HSTU hot-path library (libhstu.so).
 *
 * What is computed (by page title and section):
 *   - neurarch "HSTU (Generative Recommender)" model card, "Exported PyTorch",
 *     HSTUBlock: one fused linear map to u|v|q|k (in that order), per-head
 *     views, and pointwise aggregation: SiLU(q.k^T) divided by the sequence
 *     length, masked to j <= i after the SiLU, times v. No softmax.
 *   - briansu.co "HSTU: Hierarchical Sequential Transduction Units", section 3
 *     "How it works": relative position and relative time biases enter the
 *     pointwise SiLU attention; a layer is projection, aggregation, gated
 *     transformation.
 *   - daiwk.github.io HSTU reproduction notes, "core formula" and flowchart:
 *     U,V,Q,K = SiLU(Norm(X) W_uvqk); causal pointwise aggregation with
 *     relative bias; post-pooling normalisation; U gate; output projection
 *     with residual.
 *
 * For sequence b (tokens off[b] .. off[b+1]-1, length n), head h and
 * positions i, j inside the sequence:
 *     S_ij = qk_scale * q_i.k_j + P[h][min(i-j, Bp-1)]
 *            + Tt[h][min(floor(log2(1 + max(t_i - t_j, 0))), Bt-1)]
 *     A_ij = SiLU(S_ij) / N  (j <= i),  0 (j > i);   O_i = sum_j A_ij v_j
 * with N = n (divisor <= 0) or N = divisor (divisor > 0).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer (HBM of the current HIP
 *     device); descriptors and the size out-parameters are HOST memory.
 *   - Token-major tensors are row-major [T, H, d]: token t of head h starts at
 *     element t*ld + h*d, the d elements of a head are contiguous, ld is the
 *     row stride in elements (ld >= H*d). q, k, v, u may therefore be column
 *     views of one packed [T, H(2dv+2dqk)] buffer.
 *   - The caller owns every buffer, including the workspace; the library
 *     allocates no device memory and keeps no per-call state.
 *   - Calls are enqueued on `hip_stream` (a hipStream_t, NULL = default
 *     stream) and return without synchronising. A non-OK status means nothing
 *     was enqueued, except HSTU_E_HIP (a launch failed; hstu_last_error()
 *     has the HIP message). Device faults surface at the caller's next sync.
 *   - No exception or abort crosses the ABI. Calls on distinct streams with
 *     distinct workspaces and outputs are independent and thread-safe.
 *   - Outputs must not alias inputs (HSTU_E_ALIAS when the ranges overlap).
 *   - Alignment: base pointers 16-byte aligned; ld a multiple of 8 elements
 *     (bf16) or 4 elements (fp32) (HSTU_E_ALIGN).
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_E_NULL = 1,        /* a required pointer is NULL */
  HSTU_E_SHAPE = 2,       /* inconsistent or negative sizes */
  HSTU_E_DTYPE = 3,       /* dtype not supported by this entry point */
  HSTU_E_ALIGN = 4,       /* pointer or row stride misaligned */
  HSTU_E_UNSUPPORTED = 5, /* head dims / bucket counts outside what is built */
  HSTU_E_WORKSPACE = 6,   /* workspace smaller than *_workspace_size reports */
  HSTU_E_ALIAS = 7,       /* an output overlaps an input */
  HSTU_E_HIP = 8          /* a HIP call or kernel launch failed */
} hstu_status_t;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype_t;

/* A jagged batch of B sequences packed along the token axis.
 *
 * seq_offsets lives in device memory and the host never reads it. Each call's
 * first kernel writes a clamped copy, c(b) = min(max(0, off[0], ..., off[b]),
 * T), and every later kernel of the call reads only that copy. A well-formed
 * array (off[0] = 0, non-decreasing, off[B] = T) is unchanged by it. A
 * malformed one cannot make a kernel read or write outside the T tokens: it
 * is computed as the batch of the clamped offsets. Offsets past T are cut to
 * T, a decreasing step becomes an empty sequence, and tokens past c(B) belong
 * to no sequence and their outputs are not written. (hstu_stochastic_length
 * clamps its offsets per sequence instead; see there.) */
typedef struct {
  int32_t num_seqs;           /* B >= 0 */
  int64_t total_tokens;       /* T: the tokens every [T, ...] tensor holds */
  const int64_t* seq_offsets; /* device [B+1]: off[0] = 0, non-decreasing, off[B] = T; empty sequences allowed */
  const int64_t* timestamps;  /* device [T] int64 seconds, or NULL (then no time bias);
                                 pairwise gaps must fit in int64 */
} hstu_jagged_t;

/* Relative-attention bias tables (fp32, per head). Either may be NULL. */
typedef struct {
  const float* pos_table;     /* device [H, Bp] row-major; bucket min(i-j, Bp-1) */
  int32_t pos_buckets;        /* Bp >= 1 when pos_table != NULL */
  const float* time_table;    /* device [H, Bt]; bucket min(floor(log2(1+max(dt,0))), Bt-1);
                                 needs hstu_jagged_t.timestamps */
  int32_t time_buckets;       /* Bt >= 1 when time_table != NULL */
} hstu_bias_t;

typedef struct {
  int32_t num_heads;          /* H >= 1 */
  int32_t dqk;                /* attn_dim of the pages; built: 32, 64, 128 */
  int32_t dv;                 /* linear_dim of the pages; built: dv == dqk */
  hstu_dtype_t dtype;         /* element type of q, k, v, o (and dO, dq, dk, dv) */
  float qk_scale;             /* alpha on q.k^T (1.0 in the pages' exported block) */
  float divisor;              /* <= 0: divide sequence b's rows by its length n_b;
                                 > 0: divide every row by this constant */
} hstu_attn_desc_t;

/* ---------------------------------------------------------------------------
 * hstu_attn_workspace_size -- device workspace bytes needed by
 * hstu_attn_fwd (is_bwd = 0) or hstu_attn_bwd (is_bwd != 0) for this shape.
 * `bytes` is a host pointer. Depends only on (desc, num_seqs, total_tokens,
 * bias bucket counts), never on device data. Errors: HSTU_E_NULL, HSTU_E_SHAPE.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_attn_workspace_size(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag,
                                       const hstu_bias_t* bias, int is_bwd, size_t* bytes);

/* ---------------------------------------------------------------------------
 * hstu_attn_fwd -- causal pointwise aggregated attention over a jagged batch
 * (neurarch model card, "Exported PyTorch", HSTUBlock.forward aggregation;
 * briansu.co explainer section 3 for the relative position / time biases).
 *
 *   q [T,H,dqk] (row stride ldq), k [T,H,dqk] (ldk), v [T,H,dv] (ldv): inputs,
 *   o [T,H,dv] (ldo): output, fully overwritten for every token of every
 *   sequence; dtype per desc->dtype (HSTU_BF16: bf16 inputs, fp32 accumulate,
 *   bf16 output; HSTU_F32: fp32 throughout). bias may be NULL (no bias).
 *   workspace: device scratch of at least hstu_attn_workspace_size(...,0,...)
 *   bytes (holds the per-tile work list); contents on entry are ignored.
 * Results are deterministic run to run. A row's bf16 output does not depend on
 * later tokens of its sequence. With fewer than 512 work items in the bound
 * (H times the query tiles the batch can hold), the bf16 path sums each
 * query tile's two key-range halves separately and adds them, so the same
 * sequence in a batch of a different size may differ in the last bit.
 * Errors: HSTU_E_NULL, HSTU_E_SHAPE, HSTU_E_DTYPE, HSTU_E_ALIGN,
 *   HSTU_E_UNSUPPORTED, HSTU_E_WORKSPACE, HSTU_E_ALIAS, HSTU_E_HIP.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_attn_fwd(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag,
                            const hstu_bias_t* bias,
                            const void* q, int64_t ldq, const void* k, int64_t ldk,
                            const void* v, int64_t ldv, void* o, int64_t ldo,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_attn_fwd_noalloc -- hstu_attn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, arguments and errors as
 * hstu_attn_fwd, without the workspace. Its workspace lives in a fixed 16 MiB
 * array of device memory that the library holds on each GPU it runs on until
 * the process ends; the first call on a device looks up that device's copy.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * A batch whose hstu_attn_workspace_size(..., 0, ...) exceeds 16 MiB
 * (T x H above about 15 million token-heads) returns HSTU_E_UNSUPPORTED; use
 * hstu_attn_fwd with a workspace for it. Every call on a GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other
 * host threads) race on it and may corrupt each other's outputs. Nothing in
 * the array needs clearing between calls (the first kernel of a call
 * initialises what the later ones read).
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_attn_fwd_noalloc(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag,
                                    const hstu_bias_t* bias,
                                    const void* q, int64_t ldq, const void* k, int64_t ldk,
                                    const void* v, int64_t ldv, void* o, int64_t ldo, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_attn_bwd -- gradients of sum(O * dO) for hstu_attn_fwd with the same
 * inputs: with sig = 1/(1+e^-S), SiLU'(S) = sig (1 + S (1 - sig)), over pairs
 * j <= i: dA_ij = dO_i.v_j, dS_ij = dA_ij SiLU'(S_ij)/N, dv_j = sum_i A_ij dO_i,
 * dq_i = alpha sum_j dS_ij k_j, dk_j = alpha sum_i dS_ij q_i, and each bias
 * table entry receives the sum of dS over the pairs that read it. (Derived from
 * the forward definition above; the pages train all positions generatively,
 * daiwk reproduction notes, core formula.)
 *
 *   d_o [T,H,dv] (lddo): upstream gradient (dtype per desc).
 *   dq [T,H,dqk] (lddq), dk (lddk), dv [T,H,dv] (lddv): overwritten.
 *   d_pos_table [H,Bp], d_time_table [H,Bt]: fp32, overwritten (not
 *   accumulated); each must be non-NULL exactly when its table is.
 *   workspace: at least hstu_attn_workspace_size(...,1,...) bytes.
 * Errors: as hstu_attn_fwd. Results are deterministic run to run.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_attn_bwd(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag,
                            const hstu_bias_t* bias,
                            const void* q, int64_t ldq, const void* k, int64_t ldk,
                            const void* v, int64_t ldv, const void* d_o, int64_t lddo,
                            void* dq, int64_t lddq, void* dk, int64_t lddk,
                            void* dv, int64_t lddv,
                            float* d_pos_table, float* d_time_table,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_attn_fwd_candidates -- candidate scoring against a history whose keys
 * and values are cached (M-FALCON, "micro-batched candidate scoring with KV
 * reuse": briansu.co explainer, section 6 "Why it works"; the pages give no
 * formula, the reading here): candidate c of sequence b, whose history has n
 * tokens, is scored exactly as if it alone were appended at position n --
 *   O_c = ( sum_{j<n} SiLU(S_cj) v_j + SiLU(S_cc) v_c ) / N,  N = n + 1
 *         (divisor <= 0) or the divisor,
 *   S_cj = qk_scale q_c.k_j + P[h][min(n-j, Bp-1)] + Tt[h][bucket(t_c - t_j)],
 *   S_cc = qk_scale q_c.k_c + P[h][0] + Tt[h][0];
 * candidates never attend to each other.
 *   hist: history batch (offsets; timestamps when there is a time table).
 *   cand: candidate batch, same num_seqs (offsets; candidate timestamps).
 *   max_candidates: host upper bound on any sequence's candidate count; it
 *     sizes the grid -- candidates past it in a sequence are not scored.
 *   k_hist, v_hist [T_h,H,d] (ldkh, ldvh): the history's cached keys / values.
 *   q, k, v [T_c,H,d]: the candidates' projections. o [T_c,H,d]: output.
 *   workspace: at least hstu_attn_cand_workspace_size(...) bytes, 16-byte
 *     aligned, not overlapping any argument (long histories are scored in
 *     chunks whose fp32 partial outputs it holds; they are summed in a fixed
 *     order, so results repeat bitwise).
 * bf16 only (dqk == dv in {32, 64, 128}). Errors: as hstu_attn_fwd.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_attn_fwd_candidates(const hstu_attn_desc_t* desc, const hstu_jagged_t* hist,
                                       const hstu_jagged_t* cand, int32_t max_candidates,
                                       const hstu_bias_t* bias,
                                       const void* k_hist, int64_t ldkh, const void* v_hist, int64_t ldvh,
                                       const void* q, int64_t ldq, const void* k, int64_t ldk,
                                       const void* v, int64_t ldv, void* o, int64_t ldo,
                                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_attn_cand_workspace_size -- device workspace bytes for
 * hstu_attn_fwd_candidates: about (T_h / 2048 + num_seqs) x max_candidates x
 * H x d x 4 bytes. Host function; desc, hist and bytes are host pointers.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_attn_cand_workspace_size(const hstu_attn_desc_t* desc, const hstu_jagged_t* hist,
                                            int32_t max_candidates, size_t* bytes);

/* Parameters of one HSTU layer (bf16 weights, fp32 norms and biases). Weight
 * matrices use the nn.Linear layout [out_features, in_features] of the
 * neurarch exported block (row-major, contiguous). */
typedef struct {
  int32_t embed_dim;          /* D; built: D % 64 == 0, D <= 4096 */
  hstu_attn_desc_t attn;      /* dtype must be HSTU_BF16; dqk == dv == 128 built */
  float ln_eps;               /* epsilon of both LayerNorms (1e-6 in the workloads) */
  const float* ln_in_gamma;   /* device [D] */
  const float* ln_in_beta;    /* device [D] */
  const void* w_uvqk;         /* device bf16 [H(2dv+2dqk), D]; rows u | v | q | k, head-major inside */
  const float* b_uvqk;        /* device [H(2dv+2dqk)] or NULL */
  const float* ln_out_gamma;  /* device [H dv] */
  const float* ln_out_beta;   /* device [H dv] */
  const void* w_out;          /* device bf16 [D, H dv] */
  const float* b_out;         /* device [D] or NULL */
  hstu_bias_t bias;           /* this layer's relative-bias tables */
} hstu_layer_params_t;

/* ---------------------------------------------------------------------------
 * hstu_layer_workspace_size -- device workspace bytes for hstu_layer_fwd.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_layer_workspace_size(const hstu_layer_params_t* params,
                                        const hstu_jagged_t* jag, size_t* bytes);

/* ---------------------------------------------------------------------------
 * hstu_layer_fwd -- one HSTU layer over a jagged batch (daiwk reproduction
 * notes, flowchart and core formula; briansu.co explainer section 3):
 *   G = SiLU(LN(X) W_uvqk^T + b_uvqk) split u|v|q|k;  O = attention(q,k,v);
 *   Y = LN(O) * u (norm over the H dv features of a token);
 *   X' = X + Y W_out^T + b_out.
 *   x [T,D] bf16 (contiguous): input. y [T,D] bf16: output, must not alias x.
 *   uvqk_out: optional bf16 [T, H(2dv+2dqk)] copy of G, or NULL.
 *   o_out: optional bf16 [T, H dv] copy of O, or NULL.
 *   workspace: at least hstu_layer_workspace_size bytes.
 * Errors: as hstu_attn_fwd.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_layer_fwd(const hstu_layer_params_t* params, const hstu_jagged_t* jag,
                             const void* x, void* y, void* uvqk_out, void* o_out,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* Parameter gradients of one layer (device fp32, row-major, overwritten -- not
 * accumulated). Shapes follow hstu_layer_params_t; d_pos_table [H, Bp] and
 * d_time_table [H, Bt] must be non-NULL exactly when the layer has that table. */
typedef struct {
  float* d_ln_in_gamma;       /* [D] */
  float* d_ln_in_beta;        /* [D] */
  float* d_w_uvqk;            /* [H(2dv+2dqk), D] */
  float* d_b_uvqk;            /* [H(2dv+2dqk)] (written also when b_uvqk is NULL) */
  float* d_ln_out_gamma;      /* [H dv] */
  float* d_ln_out_beta;       /* [H dv] */
  float* d_w_out;             /* [D, H dv] */
  float* d_b_out;             /* [D] (written also when b_out is NULL) */
  float* d_pos_table;         /* [H, Bp] or NULL */
  float* d_time_table;        /* [H, Bt] or NULL */
} hstu_layer_grads_t;

/* ---------------------------------------------------------------------------
 * hstu_layer_bwd_workspace_size -- device workspace bytes for hstu_layer_bwd.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_layer_bwd_workspace_size(const hstu_layer_params_t* params,
                                            const hstu_jagged_t* jag, size_t* bytes);

/* ---------------------------------------------------------------------------
 * hstu_layer_bwd -- gradients of sum(X' * d_out) for hstu_layer_fwd with the
 * same parameters and input: the chain rule through the layer's steps in
 * reverse (daiwk reproduction notes, flowchart and core formula; the pages
 * train every position generatively). The forward is recomputed from x
 * inside the call (nothing is kept between calls).
 *   x [T,D] bf16: the layer input. d_out [T,D] bf16: gradient of the output X'.
 *   dx [T,D] bf16: overwritten with the input gradient; must not alias x or d_out.
 *   grads: fp32 parameter gradients (hstu_layer_grads_t), 16-byte aligned.
 *   workspace: at least hstu_layer_bwd_workspace_size bytes.
 * Built for bf16 with at most 1024 position buckets (as hstu_attn_bwd).
 * Results are deterministic run to run. Errors: as hstu_layer_fwd.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_layer_bwd(const hstu_layer_params_t* params, const hstu_jagged_t* jag,
                             const void* x, const void* d_out, void* dx,
                             const hstu_layer_grads_t* grads,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_head_workspace_size -- device workspace bytes for hstu_head_fwd
 * (rows x dim bf16: the normalised rows).
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_head_workspace_size(int64_t rows, int32_t dim, size_t* bytes);

/* ---------------------------------------------------------------------------
 * hstu_head_fwd -- catalogue logits of the retrieval head over token rows
 * (neurarch HSTU model card, section "Structure": rows "RMSNorm" and
 * "Retrieval Head", and its exported code's bias-free linear map; the
 * neurarch graph JSON of the model: "norm" node, eps 1e-6, and "head" node,
 * tied weights):
 *   Y = X / sqrt(mean over the dim features of X^2 + eps) * gamma
 *   logits[t, i] = sum_d Y[t, d] table[i, d]     (Y rounded to bf16)
 *   rows, dim: token rows and features (dim 512 or 1024 built).
 *   vocab: items scored, a multiple of 8.
 *   x: bf16 [rows, dim], row stride ldx elements.
 *   gamma: fp32 [dim], or NULL for ones.
 *   table: bf16 [vocab, dim], row stride ldt: the item table -- with tied
 *     weights, the token-embedding table itself.
 *   logits: bf16 [rows, vocab], row stride ldl >= vocab; must not overlap x,
 *     gamma or the table.
 *   workspace: at least hstu_head_workspace_size(rows, dim) bytes, not
 *     overlapping any argument.
 * Pointers are device pointers, 16-byte aligned; row strides are multiples
 * of 8 elements. Nothing is allocated. rows or vocab 0: nothing is launched.
 * Errors: HSTU_E_NULL, HSTU_E_SHAPE, HSTU_E_ALIGN, HSTU_E_ALIAS,
 * HSTU_E_WORKSPACE, HSTU_E_UNSUPPORTED (dim not built, vocab not a multiple
 * of 8, rows or vocab at or above 2^31), HSTU_E_HIP (a launch failed).
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_head_fwd(int64_t rows, int32_t dim, int64_t vocab, float eps,
                            const void* x, int64_t ldx, const float* gamma,
                            const void* table, int64_t ldt, void* logits, int64_t ldl,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_stochastic_length -- random shortening of long training histories
 * (Stochastic Length: briansu.co explainer, section 6 "Why it works"; the
 * pages give no procedure, the reading here): a sequence of n <= max_len
 * tokens is kept whole; a longer one keeps the max_len tokens whose
 * (key, position in the sequence) pairs are smallest, in their original
 * order. With independent uniform keys that is a uniformly random subset.
 *   num_seqs, seq_offsets: the input batch (device int64 [B+1]); offsets are
 *     clamped to [0, total_tokens] and made non-decreasing on read.
 *   total_tokens: T (host), the tokens that keys and gather_index cover.
 *   keys: device uint32 [T], one random key per token (drawn by the caller).
 *   new_offsets: device int64 [B+1], overwritten with the shortened batch's
 *     offsets (new_offsets[B] = T', the kept tokens).
 *   gather_index: device int64 [T] capacity; entry r < T' is the input token
 *     of output token r; entries from T' on are not written.
 * Outputs must not overlap the inputs or each other. Deterministic: the
 * result depends on the keys alone. Nothing is allocated.
 * Errors: HSTU_E_NULL, HSTU_E_SHAPE (negative sizes), HSTU_E_ALIGN (offsets
 * and gather_index 8-byte, keys 4-byte), HSTU_E_ALIAS, HSTU_E_UNSUPPORTED
 * (T >= 2^31), HSTU_E_HIP.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_stochastic_length(int32_t num_seqs, const int64_t* seq_offsets, int64_t total_tokens,
                                     int64_t max_len, const uint32_t* keys, int64_t* new_offsets,
                                     int64_t* gather_index, void* hip_stream);

/* ---------------------------------------------------------------------------
 * hstu_gather_rows -- dst row r = src row index[r] for r < min(*count,
 * max_rows): moves a batch's per-token rows (embeddings, timestamps, ids)
 * into the shortened batch of hstu_stochastic_length.
 *   index: device int64 (e.g. its gather_index). count: device int64, the
 *     rows to copy (e.g. new_offsets + num_seqs), read by the kernel so the
 *     host need not wait for it. max_rows: host bound on the rows copied.
 *   src [src_rows rows of row_bytes, stride src_stride bytes]; rows whose
 *     index lies outside [0, src_rows) are left unwritten.
 *   dst [max_rows rows, stride dst_stride bytes]; must not overlap src,
 *     index or count.
 * Bases, strides and row_bytes 4-byte aligned (16-byte alignment takes the
 * widest copies); index and count 8-byte aligned. Nothing is allocated.
 * Errors: HSTU_E_NULL, HSTU_E_SHAPE, HSTU_E_ALIGN, HSTU_E_ALIAS, HSTU_E_HIP.
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_gather_rows(const int64_t* index, const int64_t* count, int64_t max_rows, const void* src,
                               int64_t src_rows, int64_t src_stride, void* dst, int64_t dst_stride,
                               int64_t row_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Kernel timing for measurement tools. While enabled (process-wide), every
 * launch of a timed kernel is bracketed by two HIP events recorded on the
 * caller's stream, which adds a small gap between launches; off by default.
 * hstu_timing_read waits for the recorded events of all kernels, returns the
 * number of launches of `kernel` and their summed duration in milliseconds
 * since the last read of that kernel, and resets that kernel's totals.
 * Kernel names: "attn_fwd", "attn_bwd_kv", "attn_bwd_q", "layer_gemm_uvqk",
 * "layer_gemm_out", "layer_norm", "attn_cand", "head_rms_norm", "head_gemm",
 * "sl_select", "gather_rows".
 * Host pointers. Errors: HSTU_E_NULL,
 * HSTU_E_SHAPE (unknown name), HSTU_E_HIP (an event failed).
 * ------------------------------------------------------------------------- */
hstu_status_t hstu_timing_enable(int enable);
hstu_status_t hstu_timing_read(const char* kernel, int64_t* launches, double* total_ms);

/* Static English text of a status code. */
const char* hstu_status_string(hstu_status_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* hstu_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t hstu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
