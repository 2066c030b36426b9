// C ABI of libhstu.so: argument validation, workspace carving and kernel
// dispatch. Every check runs on the host from the descriptors alone (the
// host never reads device memory), so a non-OK status means nothing was
// enqueued.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/hstu.h"
#include "launch.h"

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
  a.off = j->seq_offsets;
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
    return fail(HSTU_E_UNSUPPORTED, "backward not built yet");
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
  hipError_t e = hstu::launch_build_worklist(jag->seq_offsets, jag->num_seqs, (int)H, hstu::kAttnBM, L, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "work-list launch");
  hstu::AttnArgs a = make_args(desc, jag, bias, q, ldq, k, ldk, v, ldv);
  a.o = o;
  a.ldo = ldo;
  a.items = ws + L.items_off;
  a.item_count = reinterpret_cast<const int*>(ws + L.hdr_off);
  a.capacity = L.capacity;
  a.tile_base = reinterpret_cast<const int*>(ws + L.tile_base_off);
  a.meta = ws + L.meta_off;
  a.meta_blocks = L.meta_blocks;
  e = dt == HSTU_BF16 ? hstu::launch_attn_fwd_bf16(a, desc->dqk, desc->dv, stream)
                      : hstu::launch_attn_fwd_f32(a, desc->dqk, desc->dv, stream);
  if (e != hipSuccess) return hip_fail(e, "attention forward launch");
  return ok();
}

hstu_status_t hstu_attn_bwd(const hstu_attn_desc_t*, const hstu_jagged_t*, const hstu_bias_t*, const void*,
                            int64_t, const void*, int64_t, const void*, int64_t, const void*, int64_t, void*,
                            int64_t, void*, int64_t, void*, int64_t, float*, float*, void*, size_t, void*) {
  return fail(HSTU_E_UNSUPPORTED, "backward not built yet");
}

hstu_status_t hstu_layer_workspace_size(const hstu_layer_params_t*, const hstu_jagged_t*, size_t*) {
  return fail(HSTU_E_UNSUPPORTED, "layer not built yet");
}

hstu_status_t hstu_layer_fwd(const hstu_layer_params_t*, const hstu_jagged_t*, const void*, void*, void*, void*,
                             void*, size_t, void*) {
  return fail(HSTU_E_UNSUPPORTED, "layer not built yet");
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
