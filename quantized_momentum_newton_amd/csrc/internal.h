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
// records a HIP event on `stream` when built and another when destroyed,
// bracketing the launches of its scope under kernel class `cls`.
bool timing_on();
int timing_begin(void *stream, int cls);
void timing_end(void *stream, int token);
struct Timed {
    void *stream;
    int token;
    Timed(void *s, int cls) : stream(s), token(timing_on() ? timing_begin(s, cls) : -1) {}
    ~Timed() {
        if (token >= 0) timing_end(stream, token);
    }
    Timed(const Timed &) = delete;
    Timed &operator=(const Timed &) = delete;
};

inline bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace qm
