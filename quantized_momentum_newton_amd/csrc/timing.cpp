// Launch timing recorder behind qm_timing_enable / qm_timing_read.
//
// A pool of HIP event pairs is reused across enable cycles; each Timed scope
// takes the next pair, and the scope's launches carry it on their dispatches
// (launch.h).  Reading waits on the stop events and sums
// hipEventElapsedTime per kernel class.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"

namespace qm {
namespace {

struct Rec {
    int cls = 0;
    hipEvent_t start = nullptr, stop = nullptr;
};

std::mutex g_mu;
std::vector<Rec> g_pool;   // events are created once and reused
size_t g_used = 0;         // records of the current cycle: g_pool[0 .. g_used)
std::atomic<bool> g_on{false};

}  // namespace

bool timing_on() { return g_on.load(std::memory_order_relaxed); }

TimedScope *&timed_current() {
    static thread_local TimedScope *cur = nullptr;
    return cur;
}

int timing_begin(int cls, void **start, void **stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return -1;
    if (g_used == g_pool.size()) {
        Rec r;
        if (hipEventCreate(&r.start) != hipSuccess) return -1;
        if (hipEventCreate(&r.stop) != hipSuccess) {
            (void)hipEventDestroy(r.start);
            return -1;
        }
        g_pool.push_back(r);
    }
    Rec &r = g_pool[g_used];
    r.cls = cls;
    *start = r.start;
    *stop = r.stop;
    return (int)g_used++;
}

void timing_end(int token, bool launched) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (token < 0 || (size_t)token >= g_used) return;
    if (!launched) g_pool[(size_t)token].cls = -1;   // no kernel carried the events
}

}  // namespace qm

using namespace qm;

extern "C" qm_status qm_timing_enable(int32_t on) {
    clear_error();
    if (on < 0 || on > 2) return fail(QM_E_ARG, "timing mode %d (0 stop, 1 start, 2 resume)", (int)on);
    std::lock_guard<std::mutex> lk(g_mu);
    if (on == 1) g_used = 0;
    g_on = on != 0;
    return QM_OK;
}

extern "C" qm_status qm_timing_read(int32_t kernel_class, double *total_ms, int64_t *launches) {
    clear_error();
    if (kernel_class < 0 || kernel_class >= QM_K_CLASSES) return fail(QM_E_ARG, "kernel class %d out of range", kernel_class);
    if (!total_ms || !launches) return fail(QM_E_ARG, "null output");
    std::lock_guard<std::mutex> lk(g_mu);
    double sum = 0.0;
    int64_t n = 0;
    for (size_t i = 0; i < g_used; i++) {
        const Rec &r = g_pool[i];
        if (r.cls != kernel_class) continue;
        if (hipEventSynchronize(r.stop) != hipSuccess) return fail(QM_E_HIP, "event wait failed");
        float ms = 0.0f;
        const hipError_t e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return fail(QM_E_HIP, "elapsed time: %s", hipGetErrorString(e));
        sum += ms;
        n++;
    }
    *total_ms = sum;
    *launches = n;
    return QM_OK;
}
