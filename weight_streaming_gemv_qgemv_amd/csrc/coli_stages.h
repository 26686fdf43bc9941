// coli_stages.h -- scoped stage timer used by the entry points (coli_stages.hip).
#ifndef COLI_STAGES_H
#define COLI_STAGES_H

#include <hip/hip_runtime.h>

namespace coli {

enum Stage { kStRouter = 0, kStGroup = 1, kStGateUp = 2, kStDown = 3, kStCombine = 4, kStQgemv = 5,
             kStPrep = 6, kStNorm = 7 };

// Records a start event on construction and an end event on destruction
// when stage timing is enabled; does nothing otherwise.  A stage that is one
// kernel launch (one_kernel) instead hands its two events to that launch
// (take_kernel_events), which records them at the kernel's own start and end
// (hipExtLaunchKernelGGL): the stage time is then the kernel's duration,
// without the gap between an event and the dispatch that follows it.
class StageTimer {
  public:
    StageTimer(int stage, hipStream_t st, bool one_kernel = false);
    ~StageTimer();
    StageTimer(const StageTimer &) = delete;
    StageTimer &operator=(const StageTimer &) = delete;

  private:
    int stage_;
    hipStream_t st_;
    void *a_ = nullptr;
    void *b_ = nullptr;
    bool one_ = false;
};

// The start/stop events of the enclosing one-kernel stage, once (both null
// when stage timing is off or the stage records its own events).
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
KernelEvents take_kernel_events();

}  // namespace coli

#endif
