// coli_stages.h -- scoped stage timer used by the entry points (coli_stages.hip).
#ifndef COLI_STAGES_H
#define COLI_STAGES_H

#include <hip/hip_runtime.h>

namespace coli {

enum Stage { kStRouter = 0, kStGroup = 1, kStGateUp = 2, kStDown = 3, kStCombine = 4, kStQgemv = 5,
             kStPrep = 6, kStNorm = 7 };

// Records a start event on construction and an end event on destruction
// when stage timing is enabled; does nothing otherwise.
class StageTimer {
  public:
    StageTimer(int stage, hipStream_t st);
    ~StageTimer();
    StageTimer(const StageTimer &) = delete;
    StageTimer &operator=(const StageTimer &) = delete;

  private:
    int stage_;
    hipStream_t st_;
    void *a_ = nullptr;
    void *b_ = nullptr;
};

}  // namespace coli

#endif
