// Measurement aid: a plain HBM copy with the access pattern of the q8 update
// kernel (16-byte non-temporal loads and stores, each wave instruction
// covering one contiguous 1 KiB span), so the achievable read + write rate of
// the memory system can be measured next to the kernels it bounds, and so a
// kernel of exactly known traffic can calibrate the profiler's HBM byte
// counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "qmuon.h"

namespace qm {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kThreads = 256;
// 16-byte units per thread, one pass per wave: measured fastest among 1, 2, 4
// and 8 units per lane and grids of 1024 to 8192 looping workgroups (one unit:
// 6.53 TB/s for 1.3 GB, four: 6.23)
constexpr int kUnitsPerThread = 1;

__global__ __launch_bounds__(kThreads) void hbm_stream_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                              int64_t units) {
    const int64_t base = (int64_t)blockIdx.x * kThreads * kUnitsPerThread + threadIdx.x;
    u32x4 v[kUnitsPerThread];
#pragma unroll
    for (int k = 0; k < kUnitsPerThread; k++) {
        const int64_t u = base + (int64_t)k * kThreads;
        if (u < units) v[k] = __builtin_nontemporal_load(src + u);
    }
#pragma unroll
    for (int k = 0; k < kUnitsPerThread; k++) {
        const int64_t u = base + (int64_t)k * kThreads;
        if (u < units) __builtin_nontemporal_store(v[k], dst + u);
    }
}

}  // namespace
}  // namespace qm

using namespace qm;

extern "C" qm_status qm_hbm_stream_copy(const void *src, void *dst, size_t bytes, qm_stream_t stream) {
    clear_error();
    if (!src || !dst) return fail(QM_E_ARG, "src and dst must not be null");
    if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16) return fail(QM_E_ALIGN, "16-byte alignment and size");
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return fail(QM_E_ARG, "src and dst overlap");
    if (bytes == 0) return QM_OK;
    const int64_t units = (int64_t)(bytes / 16);
    const int64_t per_wg = (int64_t)kThreads * kUnitsPerThread;
    const int64_t grid = (units + per_wg - 1) / per_wg;
    if (grid > INT32_MAX) return fail(QM_E_UNSUPPORTED, "copy too large");
    hbm_stream_kernel<<<(unsigned)grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), units);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "stream copy launch: %s", hipGetErrorString(e));
    return QM_OK;
}
