// Per-kernel launch timing (see timing.h).
#include "timing.h"

#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/hstu.h"

namespace hstu {

namespace {

const char* const kNames[kNumTimed] = {"attn_fwd", "attn_bwd_kv", "attn_bwd_q",
                                       "layer_gemm_uvqk", "layer_gemm_out", "layer_norm", "attn_cand",
                                       "head_rms_norm", "head_gemm", "sl_select", "gather_rows"};

struct Pending {
  int kernel;
  hipEvent_t start, stop;
};

struct TimerState {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  long long launches[kNumTimed] = {};
  double ms[kNumTimed] = {};
};

TimerState& state() {
  static TimerState s;
  return s;
}

hipEvent_t take_event(TimerState& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Folds every finished bracket into the totals (caller holds the lock).
hipError_t drain(TimerState& s) {
  hipError_t err = hipSuccess;
  for (const Pending& p : s.pending) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(p.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, p.start, p.stop);
    if (e == hipSuccess) {
      s.launches[p.kernel] += 1;
      s.ms[p.kernel] += t;
    } else {
      err = e;
    }
    s.pool.push_back(p.start);
    s.pool.push_back(p.stop);
  }
  s.pending.clear();
  return err;
}

}  // namespace

TimedScope::TimedScope(int kernel, hipStream_t stream) : kernel_(kernel), stream_(stream) {
  TimerState& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  if (!s.enabled) return;
  start_ = take_event(s);
  stop_ = take_event(s);
  if (!start_ || !stop_ || hipEventRecord(start_, stream_) != hipSuccess) {
    if (start_) s.pool.push_back(start_);
    if (stop_) s.pool.push_back(stop_);
    start_ = stop_ = nullptr;
  }
}

TimedScope::~TimedScope() {
  if (!start_) return;
  TimerState& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    s.pending.push_back({kernel_, start_, stop_});
  } else {
    s.pool.push_back(start_);
    s.pool.push_back(stop_);
  }
}

}  // namespace hstu

extern "C" {

hstu_status_t hstu_timing_enable(int enable) {
  hstu::TimerState& s = hstu::state();
  std::lock_guard<std::mutex> lock(s.mu);
  s.enabled = enable != 0;
  return HSTU_OK;
}

hstu_status_t hstu_timing_read(const char* kernel, int64_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return HSTU_E_NULL;
  int k = -1;
  for (int i = 0; i < hstu::kNumTimed; ++i)
    if (std::strcmp(kernel, hstu::kNames[i]) == 0) k = i;
  if (k < 0) return HSTU_E_SHAPE;
  hstu::TimerState& s = hstu::state();
  std::lock_guard<std::mutex> lock(s.mu);
  const hipError_t e = hstu::drain(s);
  *launches = s.launches[k];
  *total_ms = s.ms[k];
  s.launches[k] = 0;
  s.ms[k] = 0.0;
  return e == hipSuccess ? HSTU_OK : HSTU_E_HIP;
}

}  // extern "C"
