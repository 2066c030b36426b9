// Per-kernel launch timing for measurement tools (hstu_timing_enable /
// hstu_timing_read in the C ABI). While timing is on, a TimedScope brackets
// one kernel launch with two HIP events on the launch's stream; reading the
// totals waits for those events.
#pragma once

#include <hip/hip_runtime.h>

namespace hstu {

enum TimedKernel : int {
  kTimedAttnFwd = 0,
  kTimedAttnBwdKv,
  kTimedAttnBwdQ,
  kTimedGemmUvqk,
  kTimedGemmOut,
  kTimedLayerNorm,
  kTimedAttnCand,
  kTimedRmsNorm,
  kTimedHeadGemm,
  kTimedSlSelect,
  kTimedGather,
  kNumTimed
};

class TimedScope {
 public:
  TimedScope(int kernel, hipStream_t stream);
  ~TimedScope();
  TimedScope(const TimedScope&) = delete;
  TimedScope& operator=(const TimedScope&) = delete;

 private:
  int kernel_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

}  // namespace hstu
