// Optional per-kernel timing: HIP event pairs recorded on the launch stream.
#include <vector>

#include "common.h"

namespace {

struct Rec {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};

std::vector<Rec> g_pool;  // created by mamba2_timing_enable
size_t g_used = 0;
bool g_on = false;
const char* g_pending = nullptr;

void destroy_pool() {
  for (Rec& r : g_pool) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_pool.clear();
  g_used = 0;
}

}  // namespace

namespace m2 {

void timing_before(hipStream_t st, const char* name) {
  g_pending = nullptr;
  if (!g_on || g_used >= g_pool.size()) return;
  g_pending = name;
  (void)hipEventRecord(g_pool[g_used].start, st);
}

void timing_after(hipStream_t st) {
  if (!g_pending) return;
  g_pool[g_used].name = g_pending;
  (void)hipEventRecord(g_pool[g_used].stop, st);
  ++g_used;
  g_pending = nullptr;
}

}  // namespace m2

extern "C" {

mamba2_status mamba2_timing_enable(int32_t capacity) {
  destroy_pool();
  g_on = false;
  if (capacity <= 0) return MAMBA2_OK;
  g_pool.resize((size_t)capacity);
  for (Rec& r : g_pool) {
    r.name = nullptr;
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
      g_pool.clear();
      return MAMBA2_HIP_ERROR;
    }
  }
  g_on = true;
  return MAMBA2_OK;
}

int32_t mamba2_timing_collect(mamba2_kernel_time* out, int32_t max) {
  if (!g_on) return 0;
  int32_t n = 0;
  for (size_t i = 0; i < g_used; ++i) {
    if (hipEventSynchronize(g_pool[i].stop) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_pool[i].start, g_pool[i].stop) != hipSuccess) return -1;
    if (out && n < max) {
      out[n].name = g_pool[i].name;
      out[n].ms = ms;
      ++n;
    }
  }
  g_used = 0;
  return n;
}

}  // extern "C"
