// Kernel launch that carries the open timing record's events (internal.h,
// Timed) on the dispatch itself, through hipExtLaunchKernel, when timing is
// on; a plain launch otherwise.  Errors are left for hipGetLastError, as
// after a triple-chevron launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

#include "internal.h"

namespace qm {

template <typename... KArgs, typename... Args>
void launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream, Args &&...args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    TimedScope *t = timed_current();
    if (!t) {
        kern<<<grid, block, lds, stream>>>(std::forward<Args>(args)...);
        return;
    }
    std::tuple<KArgs...> vals{std::forward<Args>(args)...};
    void *ptrs[sizeof...(KArgs)];
    std::apply([&](auto &...v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    hipEvent_t start = t->started ? nullptr : static_cast<hipEvent_t>(t->start);
    t->started = true;
    (void)hipExtLaunchKernel(reinterpret_cast<const void *>(kern), grid, block, ptrs, lds, stream, start,
                             static_cast<hipEvent_t>(t->stop), 0);
}

}  // namespace qm
