// Optional per-kernel timing. While enabled on the calling thread, every kernel a
// library call launches is bracketed by two HIP events recorded on that call's
// stream; oomb_profile_collect() reads and releases them. Disabled (the default),
// a launch costs one thread-local flag test.
#pragma once

#include <hip/hip_runtime.h>

namespace oomb {

bool profiling_on();
void profile_push(const char* name, hipEvent_t start, hipEvent_t stop);

class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s) : name_(name), s_(s) {
    if (profiling_on() && hipEventCreate(&a_) == hipSuccess && hipEventCreate(&b_) == hipSuccess) {
      active_ = hipEventRecord(a_, s_) == hipSuccess;
    }
  }
  ~ProfScope() {
    if (active_ && hipEventRecord(b_, s_) == hipSuccess) profile_push(name_, a_, b_);
  }

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool active_ = false;
};

}  // namespace oomb

// Launch `kernel` and, when profiling is on, time it under `name`.
#define OOMB_LAUNCH(name, kernel, grid, block, shmem, stream, ...)         \
  do {                                                                     \
    ::oomb::ProfScope oomb_prof_scope_(name, stream);                      \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);   \
  } while (0)
