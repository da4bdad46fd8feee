// Per-kernel timing of libmoe launches (off unless a context enables it).
// While a call runs with timing on, every kernel launch is bracketed by two
// HIP events recorded on the launch stream; the host reads the summed
// durations per kernel name afterwards.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace moe {

class KernelTimer {
 public:
  ~KernelTimer();
  void begin(const char* name, hipStream_t s);
  void end(hipStream_t s);
  // launches and summed milliseconds of every record named `name`
  // (synchronises on the recorded events)
  hipError_t query(const char* name, int64_t* launches, double* ms);
  void reset();

 private:
  struct Rec {
    std::string name;
    hipEvent_t a, b;
  };
  hipEvent_t take();
  std::vector<Rec> recs_;
  std::vector<hipEvent_t> pool_;
  std::string open_name_;
  hipEvent_t open_ = nullptr;
};

// timer of the library call in progress on this host thread (null: off)
extern thread_local KernelTimer* tl_timer;

// RAII bracket around one kernel launch
struct KernelScope {
  hipStream_t s;
  bool on;
  KernelScope(const char* name, hipStream_t st)
      : s(st), on(tl_timer != nullptr) {
    if (on) tl_timer->begin(name, s);
  }
  ~KernelScope() {
    if (on) tl_timer->end(s);
  }
};

}  // namespace moe
