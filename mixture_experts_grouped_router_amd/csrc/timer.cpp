// Per-kernel timing records (see timer.hpp).
#include "timer.hpp"

namespace moe {

thread_local KernelTimer* tl_timer = nullptr;

KernelTimer::~KernelTimer() {
  reset();
  for (hipEvent_t e : pool_) (void)hipEventDestroy(e);
}

hipEvent_t KernelTimer::take() {
  if (!pool_.empty()) {
    hipEvent_t e = pool_.back();
    pool_.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void KernelTimer::begin(const char* name, hipStream_t s) {
  open_ = take();
  open_name_ = name;
  if (open_) (void)hipEventRecord(open_, s);
}

void KernelTimer::end(hipStream_t s) {
  if (!open_) return;
  hipEvent_t b = take();
  if (!b) {
    pool_.push_back(open_);
    open_ = nullptr;
    return;
  }
  (void)hipEventRecord(b, s);
  recs_.push_back({open_name_, open_, b});
  open_ = nullptr;
}

hipError_t KernelTimer::query(const char* name, int64_t* launches,
                              double* ms) {
  int64_t n = 0;
  double sum = 0.0;
  for (const Rec& r : recs_) {
    if (r.name != name) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return e;
    float t = 0.0f;
    e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return e;
    ++n;
    sum += t;
  }
  *launches = n;
  *ms = sum;
  return hipSuccess;
}

void KernelTimer::reset() {
  for (const Rec& r : recs_) {
    (void)hipEventSynchronize(r.b);
    pool_.push_back(r.a);
    pool_.push_back(r.b);
  }
  recs_.clear();
}

}  // namespace moe
