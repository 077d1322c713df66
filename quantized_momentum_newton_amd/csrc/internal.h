// Host-side helpers shared by the library's translation units.
#pragma once
#include <stdarg.h>
#include <stdint.h>

#include "qmuon.h"

namespace qm {

// Records a per-thread message for qm_last_error() and returns `s`.
qm_status fail(qm_status s, const char *fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();

// Reads and checks a host plan blob; nullptr on error (message recorded).
struct PlanHeader;
const PlanHeader *plan_header(const void *host_blob, qm_status *st);

// Launch timing: while qm_timing_enable(1) is in effect, a Timed object
// opens a record of kernel class `cls`: a pair of HIP events.  The launches
// of its scope made through launch() (launch.h) carry the events on their
// dispatches (the start event on the first, the stop event on every one, so
// it ends up on the last), which puts no separate event packets between the
// kernels on the stream.  A scope that launched nothing leaves no record.
// The innermost open scope of the calling thread takes the launches.
struct TimedScope {
    void *start = nullptr, *stop = nullptr;   // hipEvent_t
    int token = -1;
    bool started = false;
    TimedScope *outer = nullptr;
};
TimedScope *&timed_current();
bool timing_on();
int timing_begin(int cls, void **start, void **stop);
void timing_end(int token, bool launched);
struct Timed {
    TimedScope sc;
    Timed(void * /*stream*/, int cls) {
        if (timing_on()) sc.token = timing_begin(cls, &sc.start, &sc.stop);
        if (sc.token >= 0) {
            sc.outer = timed_current();
            timed_current() = &sc;
        }
    }
    ~Timed() {
        if (sc.token >= 0) {
            timed_current() = sc.outer;
            timing_end(sc.token, sc.started);
        }
    }
    Timed(const Timed &) = delete;
    Timed &operator=(const Timed &) = delete;
};

inline bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace qm
