// C ABI of libhstu.so: argument validation, workspace carving and kernel
// dispatch. Every check runs on the host from the descriptors alone (the
// host never reads device memory), so a non-OK status means nothing was
// enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/hstu.h"
#include "api_internal.h"
#include "launch.h"
#include "layer.h"
#include "stochastic_length.h"

namespace {

thread_local std::string g_last_error;

hstu_status_t fail(hstu_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hstu_status_t ok() { return HSTU_OK; }

}  // namespace

hstu_status_t hstu::api_fail(hstu_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

namespace {

hstu_status_t hip_fail(hipError_t e, const char* what) {
  return fail(HSTU_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(hstu_dtype_t t) { return t == HSTU_BF16 ? 2 : 4; }

bool supported_dims(int dqk, int dv) { return dqk == dv && (dqk == 32 || dqk == 64 || dqk == 128); }

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
};

// Byte range touched by a [T, H, d] view with row stride ld.
Range view_range(const void* p, int64_t T, int64_t ld, int64_t width, size_t es) {
  Range r;
  if (!p || T <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + static_cast<uintptr_t>(((T - 1) * ld + width) * static_cast<int64_t>(es));
  return r;
}

bool overlaps(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hstu_status_t check_view(const char* name, const void* p, int64_t ld, int64_t width, int64_t T,
                         hstu_dtype_t dt) {
  if (T > 0 && !p) return fail(HSTU_E_NULL, "%s is NULL", name);
  if (ld < width) return fail(HSTU_E_SHAPE, "%s: row stride %lld < H*d = %lld", name, (long long)ld,
                              (long long)width);
  const int64_t mult = dt == HSTU_BF16 ? 8 : 4;
  if (T > 0 && (!aligned16(p) || ld % mult != 0))
    return fail(HSTU_E_ALIGN, "%s: base must be 16-byte aligned and the row stride a multiple of %lld elements",
                name, (long long)mult);
  return ok();
}

hstu_status_t check_attn_common(const hstu_attn_desc_t* d, const hstu_jagged_t* j, const hstu_bias_t* bias) {
  if (!d || !j) return fail(HSTU_E_NULL, "descriptor or jagged batch is NULL");
  if (j->num_seqs < 0 || j->total_tokens < 0) return fail(HSTU_E_SHAPE, "negative num_seqs or total_tokens");
  if (j->num_seqs > 0 && !j->seq_offsets) return fail(HSTU_E_NULL, "seq_offsets is NULL");
  if (d->num_heads < 1 || d->num_heads > 1024) return fail(HSTU_E_SHAPE, "num_heads must be in [1, 1024]");
  if (d->dtype != HSTU_BF16 && d->dtype != HSTU_F32) return fail(HSTU_E_DTYPE, "unknown dtype %d", (int)d->dtype);
  if (!supported_dims(d->dqk, d->dv))
    return fail(HSTU_E_UNSUPPORTED, "head dims dqk=%d dv=%d not built (dqk == dv in {32, 64, 128})", d->dqk, d->dv);
  if (j->total_tokens >= (int64_t(1) << 27))
    return fail(HSTU_E_UNSUPPORTED, "total_tokens must be below 2^27");
  if (bias) {
    if (bias->pos_table && bias->pos_buckets < 1) return fail(HSTU_E_SHAPE, "pos_buckets must be >= 1");
    if (bias->time_table && bias->time_buckets < 1) return fail(HSTU_E_SHAPE, "time_buckets must be >= 1");
    if (bias->time_table && !j->timestamps && j->total_tokens > 0) return fail(HSTU_E_NULL, "time_table given without timestamps");
    if ((bias->pos_table && !aligned16(bias->pos_table)) || (bias->time_table && !aligned16(bias->time_table)))
      return fail(HSTU_E_ALIGN, "bias tables must be 16-byte aligned");
  }
  return ok();
}

hstu::AttnArgs make_args(const hstu_attn_desc_t* d, const hstu_jagged_t* j, const hstu_bias_t* bias,
                         const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv) {
  hstu::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.off = nullptr;   // set by bind_worklist: the kernels read the clamped copy
  a.ts = j->timestamps;
  a.pos_table = bias ? bias->pos_table : nullptr;
  a.pos_buckets = bias && bias->pos_table ? bias->pos_buckets : 0;
  a.time_table = bias ? bias->time_table : nullptr;
  a.time_buckets = bias && bias->time_table ? bias->time_buckets : 0;
  a.alpha = d->qk_scale;
  a.divisor = d->divisor;
  a.num_heads = d->num_heads;
  return a;
}

// Points the kernels at the work list, the block metadata and the clamped
// offsets that the builder writes into the workspace ws (laid out by L).
void bind_worklist(hstu::AttnArgs& a, const hstu::WorklistLayout& L, char* ws) {
  a.off = reinterpret_cast<const int64_t*>(ws + L.offc_off);
  a.items = ws + L.items_off;
  a.item_count = reinterpret_cast<const int*>(ws + L.hdr_off);
  a.capacity = L.capacity;
  a.tile_base = reinterpret_cast<const int*>(ws + L.tile_base_off);
  a.meta = ws + L.meta_off;
  a.meta_blocks = L.meta_blocks;
}


// Backward support beyond the forward's: bf16 only, and position tables that
// fit the kernels' LDS copy.
hstu_status_t check_bwd_support(const hstu_attn_desc_t* d, const hstu_bias_t* bias) {
  if (d->dtype != HSTU_BF16) return fail(HSTU_E_UNSUPPORTED, "the backward is built for bf16 only");
  if (bias && bias->pos_table && bias->pos_buckets > hstu::kBwdPosMax)
    return fail(HSTU_E_UNSUPPORTED, "the backward supports at most %d position buckets", hstu::kBwdPosMax);
  return ok();
}

// Workspace of the backward: the forward's work list and block metadata, then
// one row of bias-gradient partial sums per (head, key tile).
struct BwdLayout {
  size_t partial_off = 0, bytes = 0;
  int grad_stride = 0;
  int64_t tile_rows = 0;
};

BwdLayout bwd_layout(const hstu::WorklistLayout& L, const hstu_attn_desc_t* d, const hstu_bias_t* bias) {
  BwdLayout B;
  B.grad_stride = (bias && bias->pos_table ? bias->pos_buckets : 0) + (bias && bias->time_table ? hstu::kBwdTimeSlots : 0);
  B.tile_rows = d->num_heads > 0 ? L.capacity / d->num_heads : 0;
  B.partial_off = (L.bytes + 255) & ~size_t(255);
  B.bytes = B.partial_off + sizeof(float) * static_cast<size_t>(L.capacity) * static_cast<size_t>(B.grad_stride);
  if (B.grad_stride == 0) B.bytes = L.bytes;
  return B;
}

}  // namespace

extern "C" {

hstu_status_t hstu_attn_workspace_size(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag,
                                       const hstu_bias_t* bias, int is_bwd, size_t* bytes) {
  if (!bytes) return fail(HSTU_E_NULL, "bytes is NULL");
  hstu_status_t st = check_attn_common(desc, jag, bias);
  if (st != HSTU_OK) return st;
  hstu::WorklistLayout L =
      hstu::worklist_layout(jag->num_seqs, jag->total_tokens, desc->num_heads, hstu::kAttnBM);
  size_t total = L.bytes;
  if (is_bwd) {
    if ((st = check_bwd_support(desc, bias)) != HSTU_OK) return st;
    total = bwd_layout(L, desc, bias).bytes;
  }
  *bytes = total;
  return ok();
}

hstu_status_t hstu_attn_fwd(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag, const hstu_bias_t* bias,
                            const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                            void* o, int64_t ldo, void* workspace, size_t workspace_bytes, void* hip_stream) {
  hstu_status_t st = check_attn_common(desc, jag, bias);
  if (st != HSTU_OK) return st;
  const int64_t T = jag->total_tokens, H = desc->num_heads;
  const hstu_dtype_t dt = desc->dtype;
  if ((st = check_view("q", q, ldq, H * desc->dqk, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("k", k, ldk, H * desc->dqk, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("v", v, ldv, H * desc->dv, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("o", o, ldo, H * desc->dv, T, dt)) != HSTU_OK) return st;
  const size_t es = elem_size(dt);
  Range ro = view_range(o, T, ldo, H * desc->dv, es);
  if (overlaps(ro, view_range(q, T, ldq, H * desc->dqk, es)) ||
      overlaps(ro, view_range(k, T, ldk, H * desc->dqk, es)) ||
      overlaps(ro, view_range(v, T, ldv, H * desc->dv, es)))
    return fail(HSTU_E_ALIAS, "o overlaps q, k or v");
  hstu::WorklistLayout L = hstu::worklist_layout(jag->num_seqs, T, (int)H, hstu::kAttnBM);
  if (workspace_bytes < L.bytes || (L.bytes > 0 && !workspace))
    return fail(HSTU_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes,
                L.bytes);
  if (jag->num_seqs == 0 || T == 0) return ok();
  if (!aligned16(workspace)) return fail(HSTU_E_ALIGN, "workspace must be 16-byte aligned");

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = hstu::launch_build_worklist(jag->seq_offsets, T, jag->num_seqs, (int)H, hstu::kAttnBM, L, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "work-list launch");
  hstu::AttnArgs a = make_args(desc, jag, bias, q, ldq, k, ldk, v, ldv);
  bind_worklist(a, L, ws);
  a.o = o;
  a.ldo = ldo;
  e = dt == HSTU_BF16 ? hstu::launch_attn_fwd_bf16(a, desc->dqk, desc->dv, stream)
                      : hstu::launch_attn_fwd_f32(a, desc->dqk, desc->dv, stream);
  if (e != hipSuccess) return hip_fail(e, "attention forward launch");
  return ok();
}

hstu_status_t hstu_attn_bwd(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag, const hstu_bias_t* bias,
                            const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                            const void* d_o, int64_t lddo, void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv,
                            int64_t lddv, float* d_pos_table, float* d_time_table, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
  hstu_status_t st = check_attn_common(desc, jag, bias);
  if (st != HSTU_OK) return st;
  if ((st = check_bwd_support(desc, bias)) != HSTU_OK) return st;
  const int64_t T = jag->total_tokens, H = desc->num_heads;
  const int64_t wq = H * desc->dqk, wv = H * desc->dv;
  const hstu_dtype_t dt = desc->dtype;
  if ((st = check_view("q", q, ldq, wq, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("k", k, ldk, wq, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("v", v, ldv, wv, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("d_o", d_o, lddo, wv, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("dq", dq, lddq, wq, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("dk", dk, lddk, wq, T, dt)) != HSTU_OK) return st;
  if ((st = check_view("dv", dv, lddv, wv, T, dt)) != HSTU_OK) return st;
  const bool has_pos = bias && bias->pos_table, has_time = bias && bias->time_table;
  if (has_pos != (d_pos_table != nullptr))
    return fail(HSTU_E_NULL, "d_pos_table must be given exactly when the position table is");
  if (has_time != (d_time_table != nullptr))
    return fail(HSTU_E_NULL, "d_time_table must be given exactly when the time table is");
  const size_t es = elem_size(dt);
  const Range rq = view_range(q, T, ldq, wq, es), rk = view_range(k, T, ldk, wq, es),
              rv = view_range(v, T, ldv, wv, es), rdo = view_range(d_o, T, lddo, wv, es);
  const Range outs[3] = {view_range(dq, T, lddq, wq, es), view_range(dk, T, lddk, wq, es),
                         view_range(dv, T, lddv, wv, es)};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], rq) || overlaps(outs[i], rk) || overlaps(outs[i], rv) || overlaps(outs[i], rdo))
      return fail(HSTU_E_ALIAS, "dq, dk and dv must not overlap q, k, v or d_o");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return fail(HSTU_E_ALIAS, "dq, dk and dv must not overlap each other");
  }
  hstu::WorklistLayout L = hstu::worklist_layout(jag->num_seqs, T, (int)H, hstu::kAttnBM);
  const BwdLayout BL = bwd_layout(L, desc, bias);
  if (workspace_bytes < BL.bytes || (BL.bytes > 0 && !workspace))
    return fail(HSTU_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes,
                BL.bytes);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (jag->num_seqs == 0 || T == 0) {
    // no pairs: the table gradients are zero
    hipError_t e = hipSuccess;
    if (has_pos) e = hstu::launch_fill_f32(d_pos_table, H * bias->pos_buckets, 0.f, stream);
    if (e == hipSuccess && has_time) e = hstu::launch_fill_f32(d_time_table, H * bias->time_buckets, 0.f, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "zeroing the bias gradients");
  }
  if (!aligned16(workspace)) return fail(HSTU_E_ALIGN, "workspace must be 16-byte aligned");

  char* ws = static_cast<char*>(workspace);
  hipError_t e = hstu::launch_build_worklist(jag->seq_offsets, T, jag->num_seqs, (int)H, hstu::kAttnBM, L, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "work-list launch");
  hstu::AttnBwdArgs g{};
  g.f = make_args(desc, jag, bias, q, ldq, k, ldk, v, ldv);
  bind_worklist(g.f, L, ws);
  g.d_o = d_o;
  g.lddo = lddo;
  g.dq = dq;
  g.lddq = lddq;
  g.dk = dk;
  g.lddk = lddk;
  g.dv = dv;
  g.lddv = lddv;
  g.d_pos = d_pos_table;
  g.d_time = d_time_table;
  g.partial = BL.grad_stride > 0 ? reinterpret_cast<float*>(ws + BL.partial_off) : nullptr;
  g.grad_stride = BL.grad_stride;
  g.tile_rows = BL.tile_rows;
  g.num_seqs = jag->num_seqs;
  e = hstu::launch_attn_bwd_bf16(g, desc->dqk, desc->dv, stream);
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return ok();
}

hstu_status_t hstu_attn_cand_workspace_size(const hstu_attn_desc_t* desc, const hstu_jagged_t* hist,
                                            int32_t max_candidates, size_t* bytes) {
  if (!bytes) return fail(HSTU_E_NULL, "bytes is NULL");
  if (!desc || !hist) return fail(HSTU_E_NULL, "descriptor or history batch is NULL");
  if (hist->num_seqs < 0 || hist->total_tokens < 0 || max_candidates < 0 || desc->num_heads < 1)
    return fail(HSTU_E_SHAPE, "negative sizes or no heads");
  *bytes = hstu::cand_workspace_bytes(hist->total_tokens, hist->num_seqs, max_candidates, desc->num_heads,
                                      desc->dqk);
  return ok();
}

hstu_status_t hstu_attn_fwd_candidates(const hstu_attn_desc_t* desc, const hstu_jagged_t* hist,
                                       const hstu_jagged_t* cand, int32_t max_candidates, const hstu_bias_t* bias,
                                       const void* k_hist, int64_t ldkh, const void* v_hist, int64_t ldvh,
                                       const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                       int64_t ldv, void* o, int64_t ldo, void* workspace, size_t workspace_bytes,
                                       void* hip_stream) {
  hstu_status_t st = check_attn_common(desc, hist, bias);
  if (st != HSTU_OK) return st;
  if (!cand) return fail(HSTU_E_NULL, "candidate batch is NULL");
  if (desc->dtype != HSTU_BF16) return fail(HSTU_E_UNSUPPORTED, "candidate scoring is built for bf16 only");
  if (cand->num_seqs != hist->num_seqs) return fail(HSTU_E_SHAPE, "history and candidates differ in num_seqs");
  if (cand->total_tokens < 0 || max_candidates < 0) return fail(HSTU_E_SHAPE, "negative candidate counts");
  if (cand->num_seqs > 0 && !cand->seq_offsets) return fail(HSTU_E_NULL, "candidate offsets are NULL");
  if (cand->total_tokens >= (int64_t(1) << 27)) return fail(HSTU_E_UNSUPPORTED, "too many candidates");
  if (cand->num_seqs > 65535) return fail(HSTU_E_UNSUPPORTED, "at most 65535 sequences");
  const bool has_time = bias && bias->time_table;
  if (has_time && cand->total_tokens > 0 && !cand->timestamps)
    return fail(HSTU_E_NULL, "time_table given without candidate timestamps");
  const int64_t Th = hist->total_tokens, Tc = cand->total_tokens, H = desc->num_heads, d = desc->dqk;
  const hstu_dtype_t dt = desc->dtype;
  if ((st = check_view("k_hist", k_hist, ldkh, H * d, Th, dt)) != HSTU_OK) return st;
  if ((st = check_view("v_hist", v_hist, ldvh, H * d, Th, dt)) != HSTU_OK) return st;
  if ((st = check_view("q", q, ldq, H * d, Tc, dt)) != HSTU_OK) return st;
  if ((st = check_view("k", k, ldk, H * d, Tc, dt)) != HSTU_OK) return st;
  if ((st = check_view("v", v, ldv, H * d, Tc, dt)) != HSTU_OK) return st;
  if ((st = check_view("o", o, ldo, H * d, Tc, dt)) != HSTU_OK) return st;
  const Range ro = view_range(o, Tc, ldo, H * d, 2);
  const Range ins[5] = {view_range(k_hist, Th, ldkh, H * d, 2), view_range(v_hist, Th, ldvh, H * d, 2),
                        view_range(q, Tc, ldq, H * d, 2), view_range(k, Tc, ldk, H * d, 2),
                        view_range(v, Tc, ldv, H * d, 2)};
  for (const Range& r : ins)
    if (overlaps(ro, r)) return fail(HSTU_E_ALIAS, "o overlaps an input");
  if (cand->num_seqs == 0 || Tc == 0 || max_candidates == 0) return ok();
  const size_t need = hstu::cand_workspace_bytes(Th, cand->num_seqs, max_candidates, static_cast<int>(H),
                                                 static_cast<int>(d));
  if (workspace_bytes < need || !workspace)
    return fail(HSTU_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(HSTU_E_ALIGN, "workspace must be 16-byte aligned");
  const Range rw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  if (overlaps(rw, ro)) return fail(HSTU_E_ALIAS, "workspace overlaps o");
  for (const Range& r : ins)
    if (overlaps(rw, r)) return fail(HSTU_E_ALIAS, "workspace overlaps an input");
  hstu::CandArgs a{};
  a.num_seqs = cand->num_seqs;
  a.max_candidates = max_candidates;
  a.chunk_base = static_cast<int64_t*>(workspace);
  a.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + hstu::cand_partial_offset(cand->num_seqs));
  a.q_c = q; a.k_c = k; a.v_c = v; a.ldq = ldq; a.ldk = ldk; a.ldv = ldv;
  a.k_h = k_hist; a.v_h = v_hist; a.ldkh = ldkh; a.ldvh = ldvh;
  a.o = o; a.ldo = ldo;
  a.hist_off_in = hist->seq_offsets; a.cand_off_in = cand->seq_offsets;
  a.ts_h = has_time ? hist->timestamps : nullptr;
  a.ts_c = has_time ? cand->timestamps : nullptr;
  a.pos_table = bias ? bias->pos_table : nullptr;
  a.pos_buckets = bias && bias->pos_table ? bias->pos_buckets : 0;
  a.time_table = has_time ? bias->time_table : nullptr;
  a.time_buckets = has_time ? bias->time_buckets : 0;
  a.alpha = desc->qk_scale; a.divisor = desc->divisor; a.num_heads = static_cast<int>(H);
  hipError_t e = hstu::launch_attn_cand_bf16(a, static_cast<int>(d), Th, Tc, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "candidate scoring launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// layer
// ---------------------------------------------------------------------------
namespace {

struct LayerLayout {
  hstu::WorklistLayout attn;
  size_t xn_off = 0, g_off = 0, o_off = 0, y_off = 0, bytes = 0;
};

LayerLayout layer_layout(const hstu_layer_params_t* p, const hstu_jagged_t* j) {
  LayerLayout L;
  const int64_t T = j->total_tokens, H = p->attn.num_heads, D = p->embed_dim;
  const int64_t n1 = H * (2 * p->attn.dv + 2 * p->attn.dqk), hv = H * p->attn.dv;
  L.attn = hstu::worklist_layout(j->num_seqs, T, static_cast<int>(H), hstu::kAttnBM);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  take(L.attn.bytes);
  L.xn_off = take(static_cast<size_t>(T * D * 2));
  L.g_off = take(static_cast<size_t>(T * n1 * 2));
  L.o_off = take(static_cast<size_t>(T * hv * 2));
  L.y_off = take(static_cast<size_t>(T * hv * 2));
  L.bytes = off;
  return L;
}

bool ln_width_ok(int64_t w) { return w == 512 || w == 1024 || w == 2048 || w == 4096; }

hstu_status_t check_layer(const hstu_layer_params_t* p, const hstu_jagged_t* j) {
  if (!p || !j) return fail(HSTU_E_NULL, "layer parameters or jagged batch is NULL");
  hstu_status_t st = check_attn_common(&p->attn, j, &p->bias);
  if (st != HSTU_OK) return st;
  if (p->attn.dtype != HSTU_BF16) return fail(HSTU_E_DTYPE, "the layer runs in bf16");
  const int64_t H = p->attn.num_heads;
  if (!ln_width_ok(p->embed_dim) || !ln_width_ok(H * p->attn.dv))
    return fail(HSTU_E_UNSUPPORTED, "embed_dim and H*dv must be one of 512, 1024, 2048, 4096 (got %d, %lld)",
                p->embed_dim, (long long)(H * p->attn.dv));
  if (!p->ln_in_gamma || !p->ln_in_beta || !p->ln_out_gamma || !p->ln_out_beta || !p->w_uvqk || !p->w_out)
    return fail(HSTU_E_NULL, "a LayerNorm parameter or weight matrix is NULL");
  if (!aligned16(p->w_uvqk) || !aligned16(p->w_out)) return fail(HSTU_E_ALIGN, "weights must be 16-byte aligned");
  return ok();
}

// Backward of one layer: rows per block of the LayerNorm-backward and
// column-sum kernels (their partial rows are summed in a fixed order), and the
// K splits of the two weight-gradient GEMMs (K = tokens).
constexpr int kLnBwdRows = 16;
constexpr int kColSumRows = 16;
// Head GEMM tile order: bands of 8 tile rows (2048 token rows, 2 MB of
// normalised rows at dim 512) walked column by column, so the 32 workgroups
// resident on an XCD share that band in L2 and read each table tile together.
constexpr int kHeadGroupRows = 8;

// Workgroups of the head GEMM: one per compute unit of the current device (its
// 256 x 256 tiles take a unit's LDS), rounded down to a multiple of 8, each
// looping over tiles so that one tile's logit stores drain while the next
// tile's products run. 0 (one workgroup per tile) if the count is unknown.
int head_gemm_blocks() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int blocks = cus / 8 * 8;
  if (dev >= 0 && dev < 64) cached[dev] = blocks;
  return blocks;
}

int weight_grad_splits(int64_t M, int64_t N, int64_t T) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t ksteps = (T + 63) / 64;
  int64_t s = (512 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, ksteps / 8));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 64)));
}

struct LayerBwdLayout {
  hstu::WorklistLayout attn;
  BwdLayout abwd;
  size_t xn_off = 0, z_off = 0, g_off = 0, o_off = 0, y_off = 0, dyy_off = 0, do_off = 0, dg_off = 0, dxn_off = 0;
  size_t part_off = 0, scratch_off = 0, bytes = 0;
  int splits_uvqk = 1, splits_out = 1;
};

LayerBwdLayout layer_bwd_layout(const hstu_layer_params_t* p, const hstu_jagged_t* j) {
  LayerBwdLayout L;
  const int64_t T = j->total_tokens, H = p->attn.num_heads, D = p->embed_dim;
  const int64_t n1 = H * (2 * p->attn.dv + 2 * p->attn.dqk), hv = H * p->attn.dv;
  L.attn = hstu::worklist_layout(j->num_seqs, T, static_cast<int>(H), hstu::kAttnBM);
  L.abwd = bwd_layout(L.attn, &p->attn, &p->bias);
  L.splits_uvqk = weight_grad_splits(n1, D, T);
  L.splits_out = weight_grad_splits(D, hv, T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  take(L.abwd.bytes);   // the attention's work list, metadata and bias partials first
  L.xn_off = take(static_cast<size_t>(T * D * 2));
  L.z_off = take(static_cast<size_t>(T * n1 * 2));
  L.g_off = take(static_cast<size_t>(T * n1 * 2));
  L.o_off = take(static_cast<size_t>(T * hv * 2));
  L.y_off = take(static_cast<size_t>(T * hv * 2));
  L.dyy_off = take(static_cast<size_t>(T * hv * 2));
  L.do_off = take(static_cast<size_t>(T * hv * 2));
  L.dg_off = take(static_cast<size_t>(T * n1 * 2));
  L.dxn_off = take(static_cast<size_t>(T * D * 2));
  // fp32 partial rows, reused stage by stage (stream order), and the sums' scratch
  const int64_t pl = hstu::ln_bwd_partial_rows(T, kLnBwdRows), pc = hstu::colsum_partial_rows(T, kColSumRows);
  const int64_t part = std::max({pl * 2 * hv, pl * 2 * D, pc * n1, pc * D, L.splits_uvqk * n1 * D,
                                 static_cast<int64_t>(L.splits_out) * D * hv});
  const int64_t scratch = std::max({hstu::sum_rows_scratch_floats(pl, 2 * hv), hstu::sum_rows_scratch_floats(pl, 2 * D),
                                    hstu::sum_rows_scratch_floats(pc, n1), hstu::sum_rows_scratch_floats(pc, D),
                                    hstu::sum_rows_scratch_floats(L.splits_uvqk, n1 * D),
                                    hstu::sum_rows_scratch_floats(L.splits_out, D * hv)});
  L.part_off = take(static_cast<size_t>(part) * 4);
  L.scratch_off = take(static_cast<size_t>(std::max<int64_t>(scratch, 1)) * 4);
  L.bytes = off;
  return L;
}

hstu_status_t check_layer_grads(const hstu_layer_params_t* p, const hstu_layer_grads_t* g) {
  if (!g) return fail(HSTU_E_NULL, "gradient outputs are NULL");
  if (!g->d_ln_in_gamma || !g->d_ln_in_beta || !g->d_w_uvqk || !g->d_b_uvqk || !g->d_ln_out_gamma ||
      !g->d_ln_out_beta || !g->d_w_out || !g->d_b_out)
    return fail(HSTU_E_NULL, "a parameter gradient output is NULL");
  const bool has_pos = p->bias.pos_table != nullptr, has_time = p->bias.time_table != nullptr;
  if (has_pos != (g->d_pos_table != nullptr) || has_time != (g->d_time_table != nullptr))
    return fail(HSTU_E_NULL, "a table gradient must be given exactly when its table is");
  const float* outs[] = {g->d_ln_in_gamma, g->d_ln_in_beta, g->d_w_uvqk, g->d_b_uvqk, g->d_ln_out_gamma,
                         g->d_ln_out_beta, g->d_w_out, g->d_b_out};
  for (const float* o : outs)
    if (!aligned16(o)) return fail(HSTU_E_ALIGN, "parameter gradients must be 16-byte aligned");
  return ok();
}

}  // namespace

extern "C" {

hstu_status_t hstu_layer_workspace_size(const hstu_layer_params_t* params, const hstu_jagged_t* jag, size_t* bytes) {
  if (!bytes) return fail(HSTU_E_NULL, "bytes is NULL");
  hstu_status_t st = check_layer(params, jag);
  if (st != HSTU_OK) return st;
  *bytes = layer_layout(params, jag).bytes;
  return ok();
}

hstu_status_t hstu_layer_fwd(const hstu_layer_params_t* p, const hstu_jagged_t* jag, const void* x, void* y,
                             void* uvqk_out, void* o_out, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
  hstu_status_t st = check_layer(p, jag);
  if (st != HSTU_OK) return st;
  const int64_t T = jag->total_tokens, H = p->attn.num_heads, D = p->embed_dim;
  const int64_t dqk = p->attn.dqk, dv = p->attn.dv;
  const int64_t n1 = H * (2 * dv + 2 * dqk), hv = H * dv;
  if (T > 0 && (!x || !y)) return fail(HSTU_E_NULL, "x or y is NULL");
  if (T > 0 && (!aligned16(x) || !aligned16(y))) return fail(HSTU_E_ALIGN, "x and y must be 16-byte aligned");
  if ((uvqk_out && !aligned16(uvqk_out)) || (o_out && !aligned16(o_out)))
    return fail(HSTU_E_ALIGN, "uvqk_out and o_out must be 16-byte aligned");
  const Range rx = view_range(x, T, D, D, 2), ry = view_range(y, T, D, D, 2);
  if (overlaps(rx, ry)) return fail(HSTU_E_ALIAS, "y overlaps x");
  if (overlaps(view_range(uvqk_out, T, n1, n1, 2), rx) || overlaps(view_range(uvqk_out, T, n1, n1, 2), ry) ||
      overlaps(view_range(o_out, T, hv, hv, 2), rx) || overlaps(view_range(o_out, T, hv, hv, 2), ry))
    return fail(HSTU_E_ALIAS, "uvqk_out or o_out overlaps x or y");
  const LayerLayout L = layer_layout(p, jag);
  if (workspace_bytes < L.bytes || (L.bytes > 0 && !workspace))
    return fail(HSTU_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, L.bytes);
  if (T == 0 || jag->num_seqs == 0) return ok();
  if (!aligned16(workspace)) return fail(HSTU_E_ALIGN, "workspace must be 16-byte aligned");

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  void* xn = ws + L.xn_off;
  void* g = uvqk_out ? uvqk_out : static_cast<void*>(ws + L.g_off);
  void* o = o_out ? o_out : static_cast<void*>(ws + L.o_off);
  void* yy = ws + L.y_off;
  hipError_t e;

  // 1. Xn = LN(X; gamma1, beta1)
  hstu::LnArgs ln{};
  ln.x = x; ln.ldx = D; ln.gate = nullptr; ln.ldg = 0; ln.y = xn; ln.ldy = D;
  ln.gamma = p->ln_in_gamma; ln.beta = p->ln_in_beta; ln.eps = p->ln_eps; ln.rows = T;
  if ((e = hstu::launch_ln_rows(ln, static_cast<int>(D), stream)) != hipSuccess) return hip_fail(e, "input LayerNorm");

  // 2. G = SiLU(Xn W_uvqk^T + b_uvqk), columns u | v | q | k
  hstu::GemmArgs g1{};
  g1.a = xn; g1.lda = D; g1.b = p->w_uvqk; g1.ldb = D; g1.c = g; g1.ldc = n1; g1.bias = p->b_uvqk;
  g1.M = static_cast<int>(T); g1.N = static_cast<int>(n1); g1.K = static_cast<int>(D);
  if ((e = hstu::launch_gemm_nt(g1, hstu::kEpiSilu, stream)) != hipSuccess) return hip_fail(e, "UVQK projection");

  // 3. O = attention(q, k, v) on column views of G
  const __bf16* gb = static_cast<const __bf16*>(g);
  hstu::WorklistLayout WL = L.attn;
  if ((e = hstu::launch_build_worklist(jag->seq_offsets, T, jag->num_seqs, static_cast<int>(H), hstu::kAttnBM, WL,
                                       ws, stream)) != hipSuccess)
    return hip_fail(e, "work-list launch");
  hstu::AttnArgs a = make_args(&p->attn, jag, &p->bias, gb + 2 * hv, n1, gb + 2 * hv + H * dqk, n1, gb + hv, n1);
  bind_worklist(a, WL, ws);
  a.o = o;
  a.ldo = hv;
  if ((e = hstu::launch_attn_fwd_bf16(a, static_cast<int>(dqk), static_cast<int>(dv), stream)) != hipSuccess)
    return hip_fail(e, "attention forward launch");

  // 4. Y = LN(O; gamma2, beta2) * U
  hstu::LnArgs lo{};
  lo.x = o; lo.ldx = hv; lo.gate = g; lo.ldg = n1; lo.y = yy; lo.ldy = hv;
  lo.gamma = p->ln_out_gamma; lo.beta = p->ln_out_beta; lo.eps = p->ln_eps; lo.rows = T;
  if ((e = hstu::launch_ln_rows(lo, static_cast<int>(hv), stream)) != hipSuccess) return hip_fail(e, "post-pooling LayerNorm");

  // 5. X' = X + Y W_out^T + b_out
  hstu::GemmArgs g2{};
  g2.a = yy; g2.lda = hv; g2.b = p->w_out; g2.ldb = hv; g2.c = y; g2.ldc = D; g2.bias = p->b_out;
  g2.r = x; g2.ldr = D; g2.M = static_cast<int>(T); g2.N = static_cast<int>(D); g2.K = static_cast<int>(hv);
  if ((e = hstu::launch_gemm_nt(g2, hstu::kEpiResidual, stream)) != hipSuccess) return hip_fail(e, "output projection");
  return ok();
}

hstu_status_t hstu_layer_bwd_workspace_size(const hstu_layer_params_t* params, const hstu_jagged_t* jag,
                                            size_t* bytes) {
  if (!bytes) return fail(HSTU_E_NULL, "bytes is NULL");
  hstu_status_t st = check_layer(params, jag);
  if (st != HSTU_OK) return st;
  if ((st = check_bwd_support(&params->attn, &params->bias)) != HSTU_OK) return st;
  *bytes = layer_bwd_layout(params, jag).bytes;
  return ok();
}

hstu_status_t hstu_layer_bwd(const hstu_layer_params_t* p, const hstu_jagged_t* jag, const void* x,
                             const void* d_out, void* dx, const hstu_layer_grads_t* grads, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  hstu_status_t st = check_layer(p, jag);
  if (st != HSTU_OK) return st;
  if ((st = check_bwd_support(&p->attn, &p->bias)) != HSTU_OK) return st;
  if ((st = check_layer_grads(p, grads)) != HSTU_OK) return st;
  const int64_t T = jag->total_tokens, H = p->attn.num_heads, D = p->embed_dim;
  const int64_t dqk = p->attn.dqk, dv = p->attn.dv;
  const int64_t n1 = H * (2 * dv + 2 * dqk), hv = H * dv;
  if (T > 0 && (!x || !d_out || !dx)) return fail(HSTU_E_NULL, "x, d_out or dx is NULL");
  if (T > 0 && (!aligned16(x) || !aligned16(d_out) || !aligned16(dx)))
    return fail(HSTU_E_ALIGN, "x, d_out and dx must be 16-byte aligned");
  const Range rdx = view_range(dx, T, D, D, 2);
  if (overlaps(rdx, view_range(x, T, D, D, 2)) || overlaps(rdx, view_range(d_out, T, D, D, 2)))
    return fail(HSTU_E_ALIAS, "dx overlaps x or d_out");
  const LayerBwdLayout L = layer_bwd_layout(p, jag);
  if (workspace_bytes < L.bytes || (L.bytes > 0 && !workspace))
    return fail(HSTU_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, L.bytes);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (T == 0 || jag->num_seqs == 0) {
    // no tokens: every parameter gradient is zero
    const std::pair<float*, int64_t> z[] = {
        {grads->d_ln_in_gamma, D}, {grads->d_ln_in_beta, D}, {grads->d_w_uvqk, n1 * D}, {grads->d_b_uvqk, n1},
        {grads->d_ln_out_gamma, hv}, {grads->d_ln_out_beta, hv}, {grads->d_w_out, D * hv}, {grads->d_b_out, D},
        {grads->d_pos_table, p->bias.pos_table ? H * p->bias.pos_buckets : 0},
        {grads->d_time_table, p->bias.time_table ? H * p->bias.time_buckets : 0}};
    for (const auto& pr : z)
      if (pr.first && pr.second > 0 && (e = hstu::launch_fill_f32(pr.first, pr.second, 0.f, stream)) != hipSuccess)
        return hip_fail(e, "zeroing the parameter gradients");
    return ok();
  }
  if (!aligned16(workspace)) return fail(HSTU_E_ALIGN, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  auto bf = [&](size_t o) { return static_cast<void*>(ws + o); };
  void *xn = bf(L.xn_off), *z = bf(L.z_off), *g = bf(L.g_off), *o = bf(L.o_off), *yy = bf(L.y_off);
  void *dyy = bf(L.dyy_off), *dob = bf(L.do_off), *dg = bf(L.dg_off), *dxn = bf(L.dxn_off);
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  float* scratch = reinterpret_cast<float*>(ws + L.scratch_off);
  const int64_t pl = hstu::ln_bwd_partial_rows(T, kLnBwdRows), pc = hstu::colsum_partial_rows(T, kColSumRows);

  // ---- forward again, keeping Z = LN(X) W_uvqk^T + b beside G = SiLU(Z)
  hstu::LnArgs ln{};
  ln.x = x; ln.ldx = D; ln.y = xn; ln.ldy = D;
  ln.gamma = p->ln_in_gamma; ln.beta = p->ln_in_beta; ln.eps = p->ln_eps; ln.rows = T;
  if ((e = hstu::launch_ln_rows(ln, static_cast<int>(D), stream)) != hipSuccess) return hip_fail(e, "input LayerNorm");
  hstu::GemmArgs g1{};
  g1.a = xn; g1.lda = D; g1.b = p->w_uvqk; g1.ldb = D; g1.c = g; g1.ldc = n1; g1.bias = p->b_uvqk;
  g1.c2 = z; g1.ldc2 = n1; g1.M = static_cast<int>(T); g1.N = static_cast<int>(n1); g1.K = static_cast<int>(D);
  if ((e = hstu::launch_gemm(g1, hstu::kEpiSiluPair, false, false, 1, stream)) != hipSuccess)
    return hip_fail(e, "UVQK projection");
  if ((e = hstu::launch_build_worklist(jag->seq_offsets, T, jag->num_seqs, static_cast<int>(H), hstu::kAttnBM,
                                       L.attn, ws, stream)) != hipSuccess)
    return hip_fail(e, "work-list launch");
  const __bf16* gb = static_cast<const __bf16*>(g);
  const void *uq = gb + 2 * hv, *uk = gb + 2 * hv + H * dqk, *uv = gb + hv;
  hstu::AttnArgs a = make_args(&p->attn, jag, &p->bias, uq, n1, uk, n1, uv, n1);
  bind_worklist(a, L.attn, ws);
  a.o = o;
  a.ldo = hv;
  if ((e = hstu::launch_attn_fwd_bf16(a, static_cast<int>(dqk), static_cast<int>(dv), stream)) != hipSuccess)
    return hip_fail(e, "attention forward launch");
  hstu::LnArgs lo{};
  lo.x = o; lo.ldx = hv; lo.gate = g; lo.ldg = n1; lo.y = yy; lo.ldy = hv;
  lo.gamma = p->ln_out_gamma; lo.beta = p->ln_out_beta; lo.eps = p->ln_eps; lo.rows = T;
  if ((e = hstu::launch_ln_rows(lo, static_cast<int>(hv), stream)) != hipSuccess)
    return hip_fail(e, "post-pooling LayerNorm");

  // ---- X' = X + Y W_out^T + b_out: d_b_out, d_W_out = d_out^T Y, dY = d_out W_out
  hstu::ColGradArgs cs{};
  cs.dg = const_cast<void*>(d_out); cs.ldg = D; cs.z = nullptr; cs.rows = T; cs.N = static_cast<int>(D);
  cs.partial = part; cs.rows_per_block = kColSumRows;
  if ((e = hstu::launch_silu_bwd_colsum(cs, stream)) != hipSuccess) return hip_fail(e, "output-bias gradient");
  if ((e = hstu::launch_sum_rows(part, pc, D, D, 1.0f, grads->d_b_out, scratch, stream)) != hipSuccess)
    return hip_fail(e, "output-bias gradient sum");
  hstu::GemmArgs gw{};
  gw.a = d_out; gw.lda = D; gw.b = yy; gw.ldb = hv; gw.c = part; gw.ldc = hv; gw.split_stride = D * hv;
  gw.M = static_cast<int>(D); gw.N = static_cast<int>(hv); gw.K = static_cast<int>(T);
  if ((e = hstu::launch_gemm(gw, hstu::kEpiF32, true, true, L.splits_out, stream)) != hipSuccess)
    return hip_fail(e, "output-projection weight gradient");
  if ((e = hstu::launch_sum_rows(part, L.splits_out, D * hv, D * hv, 1.0f, grads->d_w_out, scratch, stream)) != hipSuccess)
    return hip_fail(e, "output-projection weight gradient sum");
  hstu::GemmArgs gd{};
  gd.a = d_out; gd.lda = D; gd.b = p->w_out; gd.ldb = hv; gd.c = dyy; gd.ldc = hv;
  gd.M = static_cast<int>(T); gd.N = static_cast<int>(hv); gd.K = static_cast<int>(D);
  if ((e = hstu::launch_gemm(gd, hstu::kEpiNone, false, true, 1, stream)) != hipSuccess)
    return hip_fail(e, "gradient through the output projection");

  // ---- Y = LN(O) * u: dO, du (into dG's u columns), d gamma2, d beta2
  hstu::LnBwdArgs lb{};
  lb.x = o; lb.ldx = hv; lb.gate = g; lb.ldg = n1; lb.dy = dyy; lb.lddy = hv; lb.dx = dob; lb.lddx = hv;
  lb.dgate = dg; lb.lddg = n1; lb.gamma = p->ln_out_gamma; lb.beta = p->ln_out_beta; lb.eps = p->ln_eps;
  lb.rows = T; lb.partial = part; lb.rows_per_block = kLnBwdRows;
  if ((e = hstu::launch_ln_bwd(lb, static_cast<int>(hv), stream)) != hipSuccess)
    return hip_fail(e, "post-pooling LayerNorm backward");
  if ((e = hstu::launch_sum_rows(part, pl, hv, 2 * hv, 1.0f, grads->d_ln_out_gamma, scratch, stream)) != hipSuccess ||
      (e = hstu::launch_sum_rows(part + hv, pl, hv, 2 * hv, 1.0f, grads->d_ln_out_beta, scratch, stream)) != hipSuccess)
    return hip_fail(e, "post-pooling LayerNorm parameter gradient sum");

  // ---- attention backward: dv, dq, dk into dG's columns, bias-table gradients
  hstu::AttnBwdArgs ab{};
  ab.f = a;
  ab.d_o = dob; ab.lddo = hv;
  __bf16* dgb = static_cast<__bf16*>(dg);
  ab.dv = dgb + hv; ab.lddv = n1;
  ab.dq = dgb + 2 * hv; ab.lddq = n1;
  ab.dk = dgb + 2 * hv + H * dqk; ab.lddk = n1;
  ab.d_pos = grads->d_pos_table;
  ab.d_time = grads->d_time_table;
  ab.partial = L.abwd.grad_stride > 0 ? reinterpret_cast<float*>(ws + L.abwd.partial_off) : nullptr;
  ab.grad_stride = L.abwd.grad_stride;
  ab.tile_rows = L.abwd.tile_rows;
  ab.num_seqs = jag->num_seqs;
  if ((e = hstu::launch_attn_bwd_bf16(ab, static_cast<int>(dqk), static_cast<int>(dv), stream)) != hipSuccess)
    return hip_fail(e, "attention backward launch");

  // ---- G = SiLU(Z): dZ in place, d_b_uvqk, d_W_uvqk = dZ^T LN(X), d LN(X) = dZ W_uvqk
  hstu::ColGradArgs sb{};
  sb.dg = dg; sb.ldg = n1; sb.z = z; sb.ldz = n1; sb.rows = T; sb.N = static_cast<int>(n1);
  sb.partial = part; sb.rows_per_block = kColSumRows;
  if ((e = hstu::launch_silu_bwd_colsum(sb, stream)) != hipSuccess) return hip_fail(e, "SiLU backward");
  if ((e = hstu::launch_sum_rows(part, pc, n1, n1, 1.0f, grads->d_b_uvqk, scratch, stream)) != hipSuccess)
    return hip_fail(e, "projection-bias gradient sum");
  hstu::GemmArgs gu{};
  gu.a = dg; gu.lda = n1; gu.b = xn; gu.ldb = D; gu.c = part; gu.ldc = D; gu.split_stride = n1 * D;
  gu.M = static_cast<int>(n1); gu.N = static_cast<int>(D); gu.K = static_cast<int>(T);
  if ((e = hstu::launch_gemm(gu, hstu::kEpiF32, true, true, L.splits_uvqk, stream)) != hipSuccess)
    return hip_fail(e, "projection weight gradient");
  if ((e = hstu::launch_sum_rows(part, L.splits_uvqk, n1 * D, n1 * D, 1.0f, grads->d_w_uvqk, scratch, stream)) != hipSuccess)
    return hip_fail(e, "projection weight gradient sum");
  hstu::GemmArgs gx{};
  gx.a = dg; gx.lda = n1; gx.b = p->w_uvqk; gx.ldb = D; gx.c = dxn; gx.ldc = D;
  gx.M = static_cast<int>(T); gx.N = static_cast<int>(D); gx.K = static_cast<int>(n1);
  if ((e = hstu::launch_gemm(gx, hstu::kEpiNone, false, true, 1, stream)) != hipSuccess)
    return hip_fail(e, "gradient through the projection");

  // ---- Xn = LN(X): dX = d_out + LN backward, d gamma1, d beta1
  hstu::LnBwdArgs li{};
  li.x = x; li.ldx = D; li.gate = nullptr; li.dy = dxn; li.lddy = D; li.resid = d_out; li.ldr = D;
  li.dx = dx; li.lddx = D; li.gamma = p->ln_in_gamma; li.beta = p->ln_in_beta; li.eps = p->ln_eps;
  li.rows = T; li.partial = part; li.rows_per_block = kLnBwdRows;
  if ((e = hstu::launch_ln_bwd(li, static_cast<int>(D), stream)) != hipSuccess)
    return hip_fail(e, "input LayerNorm backward");
  if ((e = hstu::launch_sum_rows(part, pl, D, 2 * D, 1.0f, grads->d_ln_in_gamma, scratch, stream)) != hipSuccess ||
      (e = hstu::launch_sum_rows(part + D, pl, D, 2 * D, 1.0f, grads->d_ln_in_beta, scratch, stream)) != hipSuccess)
    return hip_fail(e, "input LayerNorm parameter gradient sum");
  return ok();
}

// ---------------------------------------------------------------------------
// final RMSNorm + retrieval head
// ---------------------------------------------------------------------------
hstu_status_t hstu_head_workspace_size(int64_t rows, int32_t dim, size_t* bytes) {
  if (!bytes) return fail(HSTU_E_NULL, "bytes is NULL");
  if (rows < 0 || dim < 1) return fail(HSTU_E_SHAPE, "negative rows or dim < 1");
  *bytes = static_cast<size_t>(rows) * static_cast<size_t>(dim) * 2;
  return ok();
}

hstu_status_t hstu_head_fwd(int64_t rows, int32_t dim, int64_t vocab, float eps, const void* x, int64_t ldx,
                            const float* gamma, const void* table, int64_t ldt, void* logits, int64_t ldl,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (rows < 0 || vocab < 0) return fail(HSTU_E_SHAPE, "negative rows or vocab");
  if (dim != 512 && dim != 1024) return fail(HSTU_E_UNSUPPORTED, "dim must be 512 or 1024 (got %d)", dim);
  if (!(eps >= 0.f)) return fail(HSTU_E_SHAPE, "eps must be >= 0");
  if (rows == 0 || vocab == 0) return ok();
  if (!x || !table || !logits) return fail(HSTU_E_NULL, "x, table or logits is NULL");
  if (ldx < dim || ldt < dim || ldl < vocab) return fail(HSTU_E_SHAPE, "a row stride is below its row width");
  if (vocab % 8 != 0) return fail(HSTU_E_UNSUPPORTED, "vocab must be a multiple of 8 (got %lld)", (long long)vocab);
  const int64_t tiles = ((rows + 255) / 256) * ((vocab + 255) / 256);
  if (rows >= (int64_t(1) << 31) || vocab >= (int64_t(1) << 31) || tiles >= (int64_t(1) << 31))
    return fail(HSTU_E_UNSUPPORTED, "rows x vocab too large for one launch");
  if (!aligned16(x) || !aligned16(table) || !aligned16(logits) || (gamma && !aligned16(gamma)) ||
      ldx % 8 != 0 || ldt % 8 != 0 || ldl % 8 != 0)
    return fail(HSTU_E_ALIGN, "x, table, logits and gamma must be 16-byte aligned and row strides multiples of 8");
  const Range rl = view_range(logits, rows, ldl, vocab, 2);
  if (overlaps(rl, view_range(x, rows, ldx, dim, 2)) || overlaps(rl, view_range(table, vocab, ldt, dim, 2)) ||
      overlaps(rl, view_range(gamma, 1, dim, dim, 4)))
    return fail(HSTU_E_ALIAS, "logits overlap x, gamma or the table");
  const size_t need = static_cast<size_t>(rows) * static_cast<size_t>(dim) * 2;
  if (!workspace || workspace_bytes < need)
    return fail(HSTU_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(HSTU_E_ALIGN, "workspace must be 16-byte aligned");
  const Range rw = view_range(workspace, rows, dim, dim, 2);
  if (overlaps(rw, rl) || overlaps(rw, view_range(x, rows, ldx, dim, 2)) ||
      overlaps(rw, view_range(table, vocab, ldt, dim, 2)) || overlaps(rw, view_range(gamma, 1, dim, dim, 4)))
    return fail(HSTU_E_ALIAS, "workspace overlaps an argument");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  hstu::LnArgs rn{};
  rn.x = x; rn.ldx = ldx; rn.y = workspace; rn.ldy = dim; rn.gamma = gamma; rn.eps = eps; rn.rows = rows;
  if ((e = hstu::launch_rms_rows(rn, dim, stream)) != hipSuccess) return hip_fail(e, "RMSNorm launch");
  hstu::GemmArgs g{};
  g.a = workspace; g.lda = dim; g.b = table; g.ldb = ldt; g.c = logits; g.ldc = ldl;
  g.M = static_cast<int>(rows); g.N = static_cast<int>(vocab); g.K = dim;
  g.group_m = kHeadGroupRows;
  g.blocks = head_gemm_blocks();
  if ((e = hstu::launch_head_gemm(g, stream)) != hipSuccess) return hip_fail(e, "head GEMM launch");
  return ok();
}

// ---------------------------------------------------------------------------
// Stochastic Length and row gathers
// ---------------------------------------------------------------------------
hstu_status_t hstu_stochastic_length(int32_t num_seqs, const int64_t* seq_offsets, int64_t total_tokens,
                                     int64_t max_len, const uint32_t* keys, int64_t* new_offsets,
                                     int64_t* gather_index, void* hip_stream) {
  if (num_seqs < 0 || total_tokens < 0) return fail(HSTU_E_SHAPE, "negative num_seqs or total_tokens");
  if (max_len < 0) return fail(HSTU_E_SHAPE, "max_len must be >= 0");
  if (total_tokens >= (int64_t(1) << 31)) return fail(HSTU_E_UNSUPPORTED, "total_tokens must be below 2^31");
  if (!new_offsets) return fail(HSTU_E_NULL, "new_offsets is NULL");
  if (num_seqs > 0 && !seq_offsets) return fail(HSTU_E_NULL, "seq_offsets is NULL");
  if (total_tokens > 0 && (!keys || !gather_index)) return fail(HSTU_E_NULL, "keys or gather_index is NULL");
  if ((reinterpret_cast<uintptr_t>(new_offsets) | reinterpret_cast<uintptr_t>(gather_index) |
       reinterpret_cast<uintptr_t>(seq_offsets)) & 7u || reinterpret_cast<uintptr_t>(keys) & 3u)
    return fail(HSTU_E_ALIGN, "offsets and gather_index must be 8-byte aligned, keys 4-byte aligned");
  const Range ro = view_range(new_offsets, 1, num_seqs + 1, num_seqs + 1, 8);
  const Range ri = view_range(gather_index, 1, total_tokens, total_tokens, 8);
  const Range ins[] = {view_range(seq_offsets, 1, num_seqs + 1, num_seqs + 1, 8),
                       view_range(keys, 1, total_tokens, total_tokens, 4)};
  for (const Range& r : ins)
    if (overlaps(ro, r) || overlaps(ri, r)) return fail(HSTU_E_ALIAS, "an output overlaps seq_offsets or keys");
  if (overlaps(ro, ri)) return fail(HSTU_E_ALIAS, "new_offsets overlaps gather_index");
  hstu::SlArgs a{};
  a.seq_offsets = seq_offsets; a.total_tokens = total_tokens; a.num_seqs = num_seqs; a.max_len = max_len;
  a.keys = keys; a.new_offsets = new_offsets; a.gather_index = gather_index;
  const hipError_t e = hstu::launch_stochastic_length(a, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "stochastic length launch");
}

hstu_status_t hstu_gather_rows(const int64_t* index, const int64_t* count, int64_t max_rows, const void* src,
                               int64_t src_rows, int64_t src_stride, void* dst, int64_t dst_stride,
                               int64_t row_bytes, void* hip_stream) {
  if (max_rows < 0 || src_rows < 0 || row_bytes < 0) return fail(HSTU_E_SHAPE, "negative size");
  if (max_rows == 0 || row_bytes == 0) return ok();
  if (!index || !count || !dst || (src_rows > 0 && !src)) return fail(HSTU_E_NULL, "a pointer is NULL");
  if (src_stride < row_bytes || dst_stride < row_bytes) return fail(HSTU_E_SHAPE, "a row stride is below row_bytes");
  const auto al4 = [](int64_t v) { return (v & 3) == 0; };
  if (!al4(static_cast<int64_t>(reinterpret_cast<uintptr_t>(src))) ||
      !al4(static_cast<int64_t>(reinterpret_cast<uintptr_t>(dst))) || !al4(src_stride) || !al4(dst_stride) ||
      !al4(row_bytes) || (reinterpret_cast<uintptr_t>(index) & 7u) || (reinterpret_cast<uintptr_t>(count) & 7u))
    return fail(HSTU_E_ALIGN, "rows, strides and bases must be 4-byte aligned; index and count 8-byte aligned");
  const Range rd = view_range(dst, max_rows, dst_stride, row_bytes, 1);
  if (overlaps(rd, view_range(src, src_rows, src_stride, row_bytes, 1)) ||
      overlaps(rd, view_range(index, 1, max_rows, max_rows, 8)) || overlaps(rd, view_range(count, 1, 1, 1, 8)))
    return fail(HSTU_E_ALIAS, "dst overlaps src, index or count");
  hstu::GatherArgs g{};
  g.index = index; g.count = count; g.max_rows = max_rows; g.src_rows = src_rows; g.src = src;
  g.src_stride = src_stride; g.dst = dst; g.dst_stride = dst_stride; g.row_bytes = row_bytes;
  const hipError_t e = hstu::launch_gather_rows(g, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "row gather launch");
}

const char* hstu_status_string(hstu_status_t s) {
  switch (s) {
    case HSTU_OK: return "ok";
    case HSTU_E_NULL: return "null pointer";
    case HSTU_E_SHAPE: return "bad shape";
    case HSTU_E_DTYPE: return "unsupported dtype";
    case HSTU_E_ALIGN: return "misaligned pointer or stride";
    case HSTU_E_UNSUPPORTED: return "unsupported configuration";
    case HSTU_E_WORKSPACE: return "workspace too small";
    case HSTU_E_ALIAS: return "output aliases an input";
    case HSTU_E_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* hstu_last_error(void) { return g_last_error.c_str(); }

int32_t hstu_version(void) { return 100; }

}  // extern "C"
