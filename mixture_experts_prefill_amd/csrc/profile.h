// RAII event pair around one kernel launch, active only while profiling is on.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {
class ProfileScope {
  public:
    // attached = false: events are recorded on the stream before the launch
    // and after it (when the scope ends).  attached = true: the launch site
    // hands start() and stop() to hipExtLaunchKernel, which stamps them with
    // the kernel's own start and end, so no marker packets go into the
    // stream between kernels.
    ProfileScope(int phase, hipStream_t s, bool attached = false);
    ~ProfileScope();
    hipEvent_t start() const { return a_; }
    hipEvent_t stop() const { return b_; }

  private:
    int phase_;
    hipStream_t s_;
    bool attached_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};
}  // namespace moe
