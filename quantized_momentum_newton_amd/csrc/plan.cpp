// Host side of the norm plan: validation and encoding (no HIP calls), plus
// the library's error reporting.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "internal.h"
#include "plan_layout.h"
#include "qmuon.h"

namespace qm {

static thread_local char g_err[512];

qm_status fail(qm_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = 0; }

const PlanHeader *plan_header(const void *host_blob, qm_status *st) {
    if (!host_blob) {
        *st = fail(QM_E_ARG, "host plan is null");
        return nullptr;
    }
    if (!aligned(host_blob, 8)) {
        *st = fail(QM_E_ALIGN, "host plan must be 8-byte aligned");
        return nullptr;
    }
    const PlanHeader *h = static_cast<const PlanHeader *>(host_blob);
    if (h->magic != kPlanMagic || h->version != kPlanVersion) {
        *st = fail(QM_E_PLAN, "not a plan blob of version %u", kPlanVersion);
        return nullptr;
    }
    if (h->n_tensors <= 0 || h->n_groups <= 0 || h->n_blocks <= 0 || h->n_tasks <= 0) {
        *st = fail(QM_E_PLAN, "plan blob has empty tables");
        return nullptr;
    }
    *st = QM_OK;
    return h;
}

namespace {

struct Layout {
    int64_t off_tensors, off_task, off_bg, off_ro, off_runs, off_co, off_cg, off_tt, total;
};

Layout layout_for(int32_t nt, int32_t ng, int64_t nb, int64_t nr, int64_t nc) {
    Layout L;
    int64_t o = align_up(sizeof(PlanHeader), 64);
    L.off_tensors = o;  o = align_up(o + (int64_t)nt * sizeof(PlanTensor), 64);
    L.off_task = o;     o = align_up(o + (int64_t)(nt + 1) * 8, 64);
    L.off_bg = o;       o = align_up(o + nb * 4, 64);
    L.off_ro = o;       o = align_up(o + (int64_t)(ng + 1) * 8, 64);
    L.off_runs = o;     o = align_up(o + nr * (int64_t)sizeof(PlanRun), 64);
    L.off_co = o;       o = align_up(o + (int64_t)(ng + 1) * 8, 64);
    L.off_cg = o;       o = align_up(o + nc * 4, 64);
    L.off_tt = o;       o = align_up(o + (int64_t)nt * 4, 64);
    L.total = o;
    return L;
}

int64_t nblocks(int64_t numel) { return (numel + kBlock - 1) / kBlock; }

// Bytes [lo, hi) a buffer touches: all of them (pitch 0), or, for a strided
// grad, rows of `row` bytes every `pitch` bytes starting at lo.
struct Region {
    uintptr_t lo, hi, pitch, row;
};

// Whether two regions whose spans intersect share a byte.  Exact for two
// strided regions of one pitch (their rows occupy fixed column ranges modulo
// the pitch, e.g. column slices of one fused buffer); any other pair with
// intersecting spans counts as overlapping.
bool regions_overlap(const Region &x, const Region &y) {
    if (x.hi <= y.lo || y.hi <= x.lo) return false;
    if (!x.pitch || !y.pitch || x.pitch != y.pitch) return true;
    const uintptr_t P = x.pitch;
    const uintptr_t a = x.lo % P, b = y.lo % P;   // row starts modulo the pitch
    auto hits = [&](uintptr_t s0, uintptr_t l0, uintptr_t s1, uintptr_t l1) {
        // [s0, s0 + l0) and [s1, s1 + l1) on a circle of length P (l0, l1 <= P)
        const uintptr_t d = (s1 + P - s0) % P;
        return d < l0 || (P - d) % P < l1;
    };
    return hits(a, x.row, b, y.row);
}

}  // namespace
}  // namespace qm

using namespace qm;

extern "C" qm_status qm_plan_encode(const qm_q8_tensor *tensors, int32_t n_tensors,
                                    const qm_norm_segment *segments, int32_t n_segments,
                                    int32_t n_groups, void *host_blob,
                                    size_t *inout_blob_bytes) {
    clear_error();
    if (!tensors || n_tensors <= 0) return fail(QM_E_ARG, "no tensors");
    if (!segments || n_segments <= 0) return fail(QM_E_ARG, "no segments");
    if (n_groups <= 0) return fail(QM_E_ARG, "n_groups must be positive");
    if (!inout_blob_bytes) return fail(QM_E_ARG, "inout_blob_bytes is null");

    // ---- tensors
    std::vector<Region> spans;
    int64_t nb_total = 0, total_numel = 0;
    for (int32_t i = 0; i < n_tensors; i++) {
        const qm_q8_tensor &t = tensors[i];
        if (!t.codes || !t.absmax || !t.grad)
            return fail(QM_E_ARG, "tensor %d: null pointer", i);
        if (t.numel <= 0) return fail(QM_E_ARG, "tensor %d: numel must be positive", i);
        if (t.reserved != 0) return fail(QM_E_ARG, "tensor %d: reserved field must be 0", i);
        if (t.grad_dtype != QM_F32 && t.grad_dtype != QM_BF16 && t.grad_dtype != QM_F16)
            return fail(QM_E_DTYPE, "tensor %d: unknown grad dtype %d", i, t.grad_dtype);
        if (!aligned(t.codes, 16) || !aligned(t.grad, 16) || !aligned(t.absmax, 4))
            return fail(QM_E_ALIGN, "tensor %d: codes/grad need 16-byte, absmax 4-byte alignment", i);
        const int64_t esz = t.grad_dtype == QM_F32 ? 4 : 2;
        int64_t gspan = t.numel;  // elements from grad to one past its last element
        if (t.grad_cols != 0) {
            if (t.grad_cols < 0 || t.numel % t.grad_cols != 0)
                return fail(QM_E_SHAPE, "tensor %d: grad_cols must be positive and divide numel", i);
            if (t.grad_ld < t.grad_cols) return fail(QM_E_SHAPE, "tensor %d: grad_ld < grad_cols", i);
            if (t.grad_cols % 8 != 0 || t.grad_ld % 8 != 0)
                return fail(QM_E_ALIGN, "tensor %d: grad_cols and grad_ld must be multiples of 8", i);
            if (t.numel >= (int64_t)1 << 32)
                return fail(QM_E_UNSUPPORTED, "tensor %d: strided grad too large", i);
            gspan = (t.numel / t.grad_cols - 1) * t.grad_ld + t.grad_cols;
        }
        const uintptr_t c = (uintptr_t)t.codes, a = (uintptr_t)t.absmax, g = (uintptr_t)t.grad;
        spans.push_back({c, c + (uintptr_t)t.numel, 0, 0});
        spans.push_back({a, a + (uintptr_t)(nblocks(t.numel) * 4), 0, 0});
        if (t.grad_cols != 0)
            spans.push_back({g, g + (uintptr_t)(gspan * esz), (uintptr_t)(t.grad_ld * esz), (uintptr_t)(t.grad_cols * esz)});
        else
            spans.push_back({g, g + (uintptr_t)(gspan * esz), 0, 0});
        nb_total += nblocks(t.numel);
        total_numel += t.numel;
    }
    std::sort(spans.begin(), spans.end(), [](const Region &x, const Region &y) { return x.lo < y.lo; });
    for (size_t k = 0; k < spans.size(); k++)
        for (size_t j = k + 1; j < spans.size() && spans[j].lo < spans[k].hi; j++)
            if (regions_overlap(spans[k], spans[j])) return fail(QM_E_ARG, "state/grad buffers overlap");

    // ---- segments -> one group id per block
    std::vector<int64_t> boff(n_tensors + 1, 0);
    for (int32_t i = 0; i < n_tensors; i++) boff[i + 1] = boff[i] + nblocks(tensors[i].numel);
    std::vector<int32_t> bg(nb_total, -1);
    for (int32_t s = 0; s < n_segments; s++) {
        const qm_norm_segment &g = segments[s];
        if (g.tensor_index < 0 || g.tensor_index >= n_tensors)
            return fail(QM_E_ARG, "segment %d: tensor index out of range", s);
        if (g.group_id < 0 || g.group_id >= n_groups)
            return fail(QM_E_ARG, "segment %d: group id out of range", s);
        const int64_t n = tensors[g.tensor_index].numel;
        if (g.start < 0 || g.length <= 0 || g.start > n - g.length)
            return fail(QM_E_ARG, "segment %d: outside its tensor", s);
        const int64_t end = g.start + g.length;
        if (g.start % kBlock != 0 || (end % kBlock != 0 && end != n))
            return fail(QM_E_ALIGN, "segment %d: boundaries must lie on 256-element blocks "
                                    "(or end at the tensor's end)", s);
        const int64_t b0 = boff[g.tensor_index] + g.start / kBlock;
        const int64_t b1 = boff[g.tensor_index] + nblocks(end);
        for (int64_t b = b0; b < b1; b++) {
            if (bg[b] != -1) return fail(QM_E_SHAPE, "segment %d overlaps another segment", s);
            bg[b] = g.group_id;
        }
    }
    for (int32_t i = 0; i < n_tensors; i++)
        for (int64_t b = boff[i]; b < boff[i + 1]; b++)
            if (bg[b] < 0)
                return fail(QM_E_SHAPE, "tensor %d block %lld is in no segment", i,
                            (long long)(b - boff[i]));

    // ---- group runs (ascending global block order, split at kRunMax)
    std::vector<std::vector<PlanRun>> gruns(n_groups);
    for (int64_t b = 0; b < nb_total; b++) {
        auto &v = gruns[bg[b]];
        if (!v.empty() && v.back().start_block + v.back().count == b && v.back().count < kRunMax)
            v.back().count++;
        else
            v.push_back(PlanRun{b, 1, 0});
    }
    int64_t n_runs = 0, n_chunks = 0;
    for (auto &v : gruns) {
        n_runs += (int64_t)v.size();
        n_chunks += ((int64_t)v.size() + kChunkRuns - 1) / kChunkRuns;
    }
    for (int32_t g = 0; g < n_groups; g++)
        if (gruns[g].empty()) return fail(QM_E_SHAPE, "group %d has no blocks", g);

    const Layout L = layout_for(n_tensors, n_groups, nb_total, n_runs, n_chunks);
    if (!host_blob) {
        *inout_blob_bytes = (size_t)L.total;
        return QM_OK;
    }
    if (*inout_blob_bytes < (size_t)L.total)
        return fail(QM_E_ARG, "blob buffer too small: need %lld bytes", (long long)L.total);
    if (!aligned(host_blob, 8)) return fail(QM_E_ALIGN, "host blob must be 8-byte aligned");

    char *base = static_cast<char *>(host_blob);
    memset(base, 0, (size_t)L.total);
    PlanHeader *h = reinterpret_cast<PlanHeader *>(base);
    PlanTensor *pt = reinterpret_cast<PlanTensor *>(base + L.off_tensors);
    int64_t *task = reinterpret_cast<int64_t *>(base + L.off_task);
    int32_t *pbg = reinterpret_cast<int32_t *>(base + L.off_bg);
    int64_t *ro = reinterpret_cast<int64_t *>(base + L.off_ro);
    PlanRun *runs = reinterpret_cast<PlanRun *>(base + L.off_runs);
    int64_t *co = reinterpret_cast<int64_t *>(base + L.off_co);
    int32_t *cg = reinterpret_cast<int32_t *>(base + L.off_cg);
    int32_t *tt = reinterpret_cast<int32_t *>(base + L.off_tt);

    // Task order: tensors grouped by grad dtype (stable), so that each
    // dtype's tasks form one range; the tensor table keeps the caller's order.
    std::vector<int32_t> order(n_tensors);
    for (int32_t i = 0; i < n_tensors; i++) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t x, int32_t y) { return tensors[x].grad_dtype < tensors[y].grad_dtype; });
    for (int d = 0; d < 3; d++) h->dt_task_lo[d] = h->dt_task_hi[d] = 0;
    int64_t toff = 0;
    for (int32_t k = 0; k < n_tensors; k++) {
        const int32_t i = order[k];
        const qm_q8_tensor &t = tensors[i];
        const int64_t nb = nblocks(t.numel);
        pt[i].codes = (uint64_t)(uintptr_t)t.codes;
        pt[i].absmax = (uint64_t)(uintptr_t)t.absmax;
        pt[i].grad = (uint64_t)(uintptr_t)t.grad;
        pt[i].numel = t.numel;
        pt[i].block_offset = boff[i];
        pt[i].task_offset = toff;
        pt[i].dtype = t.grad_dtype;
        pt[i].grad_cols = t.grad_cols;
        pt[i].grad_ld = t.grad_cols ? t.grad_ld : 0;
        int32_t lo = n_groups, hi = -1;
        for (int64_t b = boff[i]; b < boff[i + 1]; b++) {
            lo = std::min(lo, bg[b]);
            hi = std::max(hi, bg[b]);
        }
        pt[i].group_lo = lo;
        pt[i].group_hi = hi;
        task[k] = toff;
        tt[k] = i;
        const int d = t.grad_dtype;
        if (h->dt_task_hi[d] == 0) h->dt_task_lo[d] = toff;
        toff += (nb + kBlocksPerTask - 1) / kBlocksPerTask;
        h->dt_task_hi[d] = toff;
    }
    task[n_tensors] = toff;
    memcpy(pbg, bg.data(), (size_t)nb_total * 4);
    int64_t r = 0, c = 0;
    for (int32_t g = 0; g < n_groups; g++) {
        ro[g] = r;
        co[g] = c;
        for (const PlanRun &x : gruns[g]) runs[r++] = x;
        const int64_t nch = ((int64_t)gruns[g].size() + kChunkRuns - 1) / kChunkRuns;
        for (int64_t k = 0; k < nch; k++) cg[c++] = g;
    }
    ro[n_groups] = r;
    co[n_groups] = c;

    h->magic = kPlanMagic;
    h->version = kPlanVersion;
    h->n_tensors = n_tensors;
    h->n_groups = n_groups;
    h->n_blocks = nb_total;
    h->n_tasks = toff;
    h->n_runs = n_runs;
    h->n_chunks = n_chunks;
    h->total_numel = total_numel;
    h->off_tensors = L.off_tensors;
    h->off_task_offsets = L.off_task;
    h->off_block_group = L.off_bg;
    h->off_run_offsets = L.off_ro;
    h->off_runs = L.off_runs;
    h->off_chunk_offsets = L.off_co;
    h->off_chunk_group = L.off_cg;
    h->off_task_tensor = L.off_tt;
    h->total_bytes = L.total;
    *inout_blob_bytes = (size_t)L.total;
    return QM_OK;
}

extern "C" qm_status qm_plan_info(const void *host_blob, int32_t *n_tensors, int32_t *n_groups,
                                  int64_t *n_blocks, int64_t *total_numel) {
    clear_error();
    qm_status st;
    const PlanHeader *h = plan_header(host_blob, &st);
    if (!h) return st;
    if (n_tensors) *n_tensors = h->n_tensors;
    if (n_groups) *n_groups = h->n_groups;
    if (n_blocks) *n_blocks = h->n_blocks;
    if (total_numel) *total_numel = h->total_numel;
    return QM_OK;
}

// Workspace of the grouped update: per-block fp64 sums, fp64 chunk partials,
// fp64 group sums, fp32 inverse norms, each section 256-byte aligned.
extern "C" size_t qm_update_workspace_bytes(const void *host_blob) {
    qm_status st;
    const PlanHeader *h = plan_header(host_blob, &st);
    if (!h) return 0;
    return (size_t)(align_up(h->n_blocks * 8, 256) + align_up(h->n_chunks * 8, 256) +
                    align_up((int64_t)h->n_groups * 8, 256) + align_up((int64_t)h->n_groups * 4, 256));
}

extern "C" const char *qm_status_string(qm_status s) {
    switch (s) {
        case QM_OK: return "ok";
        case QM_E_ARG: return "invalid argument";
        case QM_E_ALIGN: return "alignment violated";
        case QM_E_DTYPE: return "unsupported dtype";
        case QM_E_SHAPE: return "inconsistent shape";
        case QM_E_WORKSPACE: return "workspace too small";
        case QM_E_HIP: return "HIP runtime error";
        case QM_E_UNSUPPORTED: return "unsupported request";
        case QM_E_PLAN: return "malformed plan";
    }
    return "unknown status";
}

extern "C" const char *qm_last_error(void) { return g_err; }

extern "C" int qm_abi_version(void) { return QM_ABI_VERSION; }
