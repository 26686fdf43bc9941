// coli_stages.hip -- optional per-stage GPU timing of the MoE calls.
//
// Off by default.  When enabled, each MoE call records a hipEvent on its
// stream before and after every stage (router, grouping, matrix-core
// preparation, gate/up, down, combine, qgemv); coli_stage_times() waits for the recorded events and adds
// up the elapsed times.  This is the only state the library keeps between
// calls, and it exists for measurement: the pages time the same phases of
// their MoE block (expert-matmul, setup, kernel and scatter time).
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "coli.h"
#include "coli_stages.h"

namespace coli {

namespace {

struct Rec {
    int stage;
    hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_pending;
std::vector<hipEvent_t> g_pool;
double g_ms[COLI_NSTAGES] = {};
int64_t g_calls[COLI_NSTAGES] = {};

hipEvent_t take_event()
{
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

const char *const kNames[COLI_NSTAGES] = {"router", "group", "gate_up", "down", "combine", "qgemv", "prep", "norm"};

}  // namespace

namespace {
// the events a one-kernel stage offers its launch, and whether it took them
thread_local KernelEvents t_offer;
thread_local bool t_taken = false;
}  // namespace

KernelEvents take_kernel_events()
{
    KernelEvents e = t_offer;
    t_offer = KernelEvents{};
    if (e.start) t_taken = true;
    return e;
}

StageTimer::StageTimer(int stage, hipStream_t st, bool one_kernel) : stage_(stage), st_(st)
{
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_on) return;
    a_ = take_event();
    b_ = take_event();
    if (!a_ || !b_) return;
    one_ = one_kernel;
    if (one_) {
        t_offer = KernelEvents{(hipEvent_t)a_, (hipEvent_t)b_};
        t_taken = false;
    } else {
        (void)hipEventRecord((hipEvent_t)a_, st_);
    }
}

StageTimer::~StageTimer()
{
    std::lock_guard<std::mutex> g(g_mu);
    if (!a_ || !b_) return;
    if (one_) {
        const bool used = t_taken;
        t_offer = KernelEvents{};
        t_taken = false;
        if (!used) {   // no launch took them (an error path): nothing to time
            g_pool.push_back((hipEvent_t)a_);
            g_pool.push_back((hipEvent_t)b_);
            return;
        }
    } else {
        (void)hipEventRecord((hipEvent_t)b_, st_);
    }
    g_pending.push_back(Rec{stage_, (hipEvent_t)a_, (hipEvent_t)b_});
}

}  // namespace coli

using namespace coli;

extern "C" int coli_stage_timing(int enable)
{
    std::lock_guard<std::mutex> g(g_mu);
    g_on = enable != 0;
    return COLI_OK;
}

extern "C" int coli_stage_times(double *ms, int64_t *calls, int reset)
{
    std::lock_guard<std::mutex> g(g_mu);
    int rc = COLI_OK;
    for (const Rec &r : g_pending) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            rc = COLI_EDEVICE;
        g_ms[r.stage] += t;
        g_calls[r.stage] += 1;
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_pending.clear();
    for (int i = 0; i < COLI_NSTAGES; ++i) {
        if (ms) ms[i] = g_ms[i];
        if (calls) calls[i] = g_calls[i];
        if (reset) {
            g_ms[i] = 0.0;
            g_calls[i] = 0;
        }
    }
    return rc;
}

extern "C" const char *coli_stage_name(int stage)
{
    return (stage >= 0 && stage < COLI_NSTAGES) ? kNames[stage] : "unknown";
}
