// Byte layout of a norm-plan blob.  The host encoder writes it; the caller
// copies it verbatim to the device; the update kernels read it there.
//
// A plan is what "Quantized Muon Momentum" (section "Grouped QKV And
// Sharding") builds once and reuses: one group id per 256-element block,
// plus, here, the tensor table (device pointers baked in, so a step needs no
// per-call metadata copy) and the work decomposition of the kernels:
//   task  = up to 4 consecutive blocks of one tensor, processed by one wave64;
//           the task index space lists the tensors grouped by grad dtype
//           (fp32, bf16, f16), so each dtype's tasks are one contiguous
//           range that a dtype-specialised kernel covers;
//   run   = up to kRunMax consecutive blocks of one group, summed by one lane
//           in the group reduction;
//   chunk = up to kChunkRuns runs of one group, reduced by one workgroup to
//           one partial; a group's sum adds its chunks' partials in order.
#pragma once
#include <stdint.h>

namespace qm {

constexpr uint32_t kPlanMagic = 0x4e4c5051u;  // "QPLN"
constexpr uint32_t kPlanVersion = 4;
constexpr int kBlock = 256;
constexpr int kBlocksPerTask = 4;
constexpr int kTaskElems = kBlock * kBlocksPerTask;  // 1024
constexpr int kRunMax = 16;
constexpr int kChunkRuns = 256;

struct PlanHeader {
    uint32_t magic, version;
    int32_t n_tensors, n_groups;
    int64_t n_blocks, n_tasks, n_runs, total_numel;
    int64_t n_chunks;
    int64_t off_tensors;       // PlanTensor[n_tensors]
    int64_t off_task_offsets;  // int64[n_tensors + 1], in task order
    int64_t off_block_group;   // int32[n_blocks]
    int64_t off_run_offsets;   // int64[n_groups + 1]
    int64_t off_runs;          // PlanRun[n_runs]
    int64_t off_chunk_offsets; // int64[n_groups + 1]
    int64_t off_chunk_group;   // int32[n_chunks]
    int64_t off_task_tensor;   // int32[n_tensors]: tensor table index of the k-th tensor in task order
    int64_t dt_task_lo[3], dt_task_hi[3];  // task range of each grad dtype (qm_dtype), possibly empty
    int64_t total_bytes;
};

struct PlanTensor {
    uint64_t codes, absmax, grad;  // device addresses
    int64_t numel;
    int64_t block_offset;          // global index of the tensor's first block
    int64_t task_offset;           // index of the tensor's first task (dtype-grouped order)
    int32_t dtype;                 // qm_dtype
    int32_t group_lo, group_hi;    // smallest / largest group id it touches
    int32_t pad;
    int64_t grad_cols, grad_ld;    // grad rows (0: contiguous) and their pitch, elements
};

struct PlanRun {
    int64_t start_block;           // global block index
    int32_t count;                 // 1 .. kRunMax
    int32_t pad;
};

static_assert(sizeof(PlanHeader) == 176, "plan header layout");
static_assert(sizeof(PlanTensor) == 80, "plan tensor layout");
static_assert(sizeof(PlanRun) == 16, "plan run layout");

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
constexpr int64_t align_up_const(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

}  // namespace qm
