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

inline bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace qm
