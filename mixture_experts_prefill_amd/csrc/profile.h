// RAII event pair around one kernel launch, active only while profiling is on.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {
class ProfileScope {
  public:
    ProfileScope(int phase, hipStream_t s);
    ~ProfileScope();

  private:
    int phase_;
    hipStream_t s_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};
}  // namespace moe
