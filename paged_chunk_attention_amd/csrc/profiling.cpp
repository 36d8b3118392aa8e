// Thread-local store of the kernel timing events (see profiling.hpp).
#include "profiling.hpp"

#include <vector>

#include "oomb.h"

namespace oomb {
namespace {
struct Rec {
  const char* name;
  hipEvent_t start, stop;
};
thread_local bool g_on = false;
thread_local std::vector<Rec> g_recs;
}  // namespace

bool profiling_on() { return g_on; }

void profile_push(const char* name, hipEvent_t start, hipEvent_t stop) {
  g_recs.push_back(Rec{name, start, stop});
}

}  // namespace oomb

extern "C" {

int oomb_profile_enable(int on) {
  oomb::g_on = on != 0;
  return OOMB_OK;
}

int oomb_profile_collect(const char** names, float* ms, int max) {
  int n = 0;
  for (auto& r : oomb::g_recs) {
    float t = -1.0f;
    if (hipEventSynchronize(r.stop) == hipSuccess) hipEventElapsedTime(&t, r.start, r.stop);
    if (n < max && names != nullptr && ms != nullptr) {
      names[n] = r.name;
      ms[n] = t;
    }
    ++n;
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
  }
  oomb::g_recs.clear();
  return n < max ? n : max;
}

}  // extern "C"
