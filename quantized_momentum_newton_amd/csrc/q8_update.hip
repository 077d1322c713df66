// Blockwise-int8 momentum update for gfx950 (wave64), compiled with
// -ffp-contract=off so every binary32 expression keeps one rounding per
// operation in the order written: codes and absmax then match a CPU run of
// the same operations bit for bit.
//
// "Quantized Muon Momentum" (cppmega docs), sections "What Exists",
// "Algorithm" and "Grouped QKV And Sharding" define what is computed:
// dequantise the int8 state with its per-256-element absmax, the beta-EMA
// with the grad in fp32, m back into the grad buffer, a new block absmax,
// symmetric nearest requantisation to [-127, 127], and per-block / per-group
// sums of m*m for the Frobenius normalisation that feeds Newton-Schulz.
//
// Layout on the MI355X (not the page's 64 threads x 4 elements): one wave64
// owns a task of 4 consecutive blocks (1024 elements).  For 16-bit grads a
// lane holds 8 elements in each of two halves of the task, so every load and
// store instruction of the wave covers one contiguous 1 KiB (grads) or 512 B
// (codes) span; a block is 32 lanes of one half and its absmax and sum are
// butterfly reductions over those 32 lanes.  fp32 grads use 4 elements per
// lane and 4 quarters, one block per quarter.  Tasks of all tensors form one
// grid-stride index space, so one launch covers the whole tensor list.
#include <hip/hip_runtime.h>

#include <atomic>
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "launch.h"
#include "plan_layout.h"
#include "q8_internal.h"
#include "qmuon.h"

namespace qm {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWG = kThreads / 64;

// ------------------------------------------------------------ global pointers

// A device address as a pointer the compiler knows points to global memory.
// The tensor addresses the plan holds, and the pointers inside argument
// structs, are otherwise generic, and their accesses compile to flat
// instructions: a 64-bit address per lane, and both the vector-memory and
// the LDS counters, so each wait for a lane shuffle's result also waits for
// the outstanding loads and stores.
template <typename T> __device__ __forceinline__ T *gmem(uint64_t a) {
    return (T *)(__attribute__((address_space(1))) T *)a;
}
template <typename T> __device__ __forceinline__ T *gmem(T *p) { return gmem<T>((uint64_t)p); }

// ------------------------------------------------------------ lane exchange

// Lane l's value from lane l ^ k.  For k < 32 (inside l's 32-lane half) a
// ds_swizzle in bit-mask mode, which needs no lane-address register, unlike
// the generic shuffle used for k = 32.  Every lane must be active.
__device__ __forceinline__ int xor_lanes(int v, int k) {
    switch (k) {
        case 1: return __builtin_amdgcn_ds_swizzle(v, 0x041f);
        case 2: return __builtin_amdgcn_ds_swizzle(v, 0x081f);
        case 4: return __builtin_amdgcn_ds_swizzle(v, 0x101f);
        case 8: return __builtin_amdgcn_ds_swizzle(v, 0x201f);
        case 16: return __builtin_amdgcn_ds_swizzle(v, 0x401f);
        default: return __shfl_xor(v, k);
    }
}
__device__ __forceinline__ float xor_lanes(float v, int k) { return __int_as_float(xor_lanes(__float_as_int(v), k)); }
__device__ __forceinline__ double xor_lanes(double v, int k) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)xor_lanes((int)(uint32_t)u, k), hi = (uint32_t)xor_lanes((int)(uint32_t)(u >> 32), k);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ------------------------------------------------------------ requantisation scale

// x = (m * s) * inv: s = 2^64 for a block so small (0 < amax < 2^-64) that
// 127 / amax could overflow, else 1; inv = 127 / (amax * s), 0 for an
// all-zero block.  Scaling by a power of two is exact, so x is
// m * (127 / amax) wherever that quotient is finite; in the tiny range the
// codes stay those of nearest rounding (a zero element stays 0 instead of
// 0 * inf).
__device__ __forceinline__ float requant_inv(float amax, float &s) {
    s = amax > 0.0f && amax < 0x1p-64f ? 0x1p64f : 1.0f;
    return amax == 0.0f ? 0.0f : 127.0f / (amax * s);
}

// ------------------------------------------------------------ conversions

// Two fp32 values to packed bf16 (a in the low half), round to nearest even,
// a NaN kept quiet with its sign and top payload bits: gfx950's
// v_cvt_pk_bf16_f32, one instruction for the pair.  It gives the same bits as
// the integer form (add 0x7fff plus the kept lsb, shift; NaN: top half | 0x40)
// for every fp32 input, subnormals and NaNs included (checked exhaustively
// on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return (uint16_t)bf16x2_rne(f, 0.0f); }
__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f16_rne(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_val(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Four E4M3 bytes (1 sign bit, 4 exponent bits biased by 7, 3 mantissa
// bits, subnormals below 2^-6, largest finite 448, no infinities) of x[0..3],
// byte j from x[j]: round to nearest even, magnitudes past 448 saturate to
// 448.  gfx950's v_cvt_pk_fp8_f32 converts to this format with round to
// nearest even; the clamp in front gives the saturation (a NaN passes through
// and comes out as a NaN byte).
__device__ __forceinline__ uint32_t e4m3x4_rne_sat(const float *x) {
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; j++) c[j] = x[j] != x[j] ? x[j] : fminf(fmaxf(x[j], -448.0f), 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
}

template <int DT> struct Elem;
template <> struct Elem<QM_F32> {
    static constexpr int kEpl = 4;  // elements per lane per part
    static constexpr int kSize = 4;
};
template <> struct Elem<QM_BF16> {
    static constexpr int kEpl = 8;
    static constexpr int kSize = 2;
};
template <> struct Elem<QM_F16> {
    static constexpr int kEpl = 8;
    static constexpr int kSize = 2;
};

template <int DT> __device__ __forceinline__ float widen(const void *p, int64_t i) {
    if constexpr (DT == QM_F32) return static_cast<const float *>(p)[i];
    else if constexpr (DT == QM_BF16) return bf16_val(static_cast<const uint16_t *>(p)[i]);
    else return f16_val(static_cast<const uint16_t *>(p)[i]);
}
template <int DT> __device__ __forceinline__ void narrow(void *p, int64_t i, float v) {
    if constexpr (DT == QM_F32) static_cast<float *>(p)[i] = v;
    else if constexpr (DT == QM_BF16) static_cast<uint16_t *>(p)[i] = bf16_rne(v);
    else static_cast<uint16_t *>(p)[i] = f16_rne(v);
}

// Vector load/store of kEpl grad elements at element offset e (16 bytes).
// Grads and codes are streamed: each byte is read once and written once per
// step, so their loads and stores carry the non-temporal hint and do not
// displace what other work keeps in the caches.  Measured: back-to-back
// update calls 8-11 % faster (Llama-8B layer, 28-layer set), the 28-layer
// grouped update with its normalisation 5 %, the update inside a full Muon step
// about 1 %.  The hint needs plain vector types.
typedef unsigned ntv4 __attribute__((ext_vector_type(4)));
typedef unsigned ntv2 __attribute__((ext_vector_type(2)));
template <int DT> __device__ __forceinline__ void load_grad_vec(const void *g, int64_t e, float *out) {
    const ntv4 v = __builtin_nontemporal_load(reinterpret_cast<const ntv4 *>(static_cast<const char *>(g) + e * Elem<DT>::kSize));
    if constexpr (DT == QM_F32) {
        out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            if constexpr (DT == QM_BF16) {
                out[2 * k] = bf16_val((uint16_t)(w[k] & 0xffffu));
                out[2 * k + 1] = bf16_val((uint16_t)(w[k] >> 16));
            } else {
                out[2 * k] = f16_val((uint16_t)(w[k] & 0xffffu));
                out[2 * k + 1] = f16_val((uint16_t)(w[k] >> 16));
            }
        }
    }
}
template <int DT> __device__ __forceinline__ void store_grad_vec(void *g, int64_t e, const float *in) {
    uint4 v;
    if constexpr (DT == QM_F32) {
        v.x = __float_as_uint(in[0]); v.y = __float_as_uint(in[1]);
        v.z = __float_as_uint(in[2]); v.w = __float_as_uint(in[3]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            if constexpr (DT == QM_BF16) w[k] = bf16x2_rne(in[2 * k], in[2 * k + 1]);
            else w[k] = (uint32_t)f16_rne(in[2 * k]) | ((uint32_t)f16_rne(in[2 * k + 1]) << 16);
        }
        v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    }
    ntv4 nv = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(nv, reinterpret_cast<ntv4 *>(static_cast<char *>(g) + e * Elem<DT>::kSize));
}

// kEpl int8 codes at element offset e (8 or 4 bytes, naturally aligned).
template <int N> __device__ __forceinline__ void load_codes_vec(const int8_t *c, int64_t e, int8_t *q) {
    if constexpr (N == 8) {
        const ntv2 v = __builtin_nontemporal_load(reinterpret_cast<const ntv2 *>(c + e));
#pragma unroll
        for (int k = 0; k < 4; k++) { q[k] = (int8_t)(v.x >> (8 * k)); q[4 + k] = (int8_t)(v.y >> (8 * k)); }
    } else {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(c + e);
#pragma unroll
        for (int k = 0; k < 4; k++) q[k] = (int8_t)(v >> (8 * k));
    }
}
// Four codes from the low bytes of a, b, c, d (a in the lowest byte): three
// byte permutes.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);   // a.0, b.0, 0, 0
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);   // c.0, d.0, 0, 0
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);              // a.0, b.0, c.0, d.0
}
// N codes, each the low byte of q[j], stored at element offset e.
template <int N> __device__ __forceinline__ void store_codes_vec(int8_t *c, int64_t e, const uint32_t *q) {
    if constexpr (N == 8) {
        ntv2 nv = {pack_low_bytes(q[0], q[1], q[2], q[3]), pack_low_bytes(q[4], q[5], q[6], q[7])};
        __builtin_nontemporal_store(nv, reinterpret_cast<ntv2 *>(c + e));
    } else {
        *reinterpret_cast<uint32_t *>(c + e) = pack_low_bytes(q[0], q[1], q[2], q[3]);
    }
}

// Element offset in the grad buffer of logical element e: e itself for a
// contiguous grad, row-major position in rows of grad_cols with pitch
// grad_ld otherwise (numel < 2^32 there, so 32-bit division suffices).
__device__ __forceinline__ int64_t gpos(const PlanTensor &T, int64_t e) {
    if (T.grad_cols == 0) return e;
    const uint32_t c = (uint32_t)T.grad_cols, ue = (uint32_t)e;
    const uint32_t r = ue / c;
    return (int64_t)r * T.grad_ld + (int64_t)(ue - r * c);
}

// Largest i with task_offsets[i] <= task (every tensor owns >= 1 task): the
// position of the task's tensor in task order.
__device__ __forceinline__ int find_tensor(const int64_t *task_offsets, int n, int64_t task) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (task_offsets[mid] <= task) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Position in task order of the tensor holding `task`, for a wave whose
// tasks only increase: a binary search for its first task (pos < 0), then a
// forward scan from the previous position, usually zero or one step.
__device__ __forceinline__ int tensor_pos(const int64_t *task_offsets, int n, int pos, int64_t task) {
    if (pos < 0) return find_tensor(task_offsets, n, task);
    while (pos + 1 < n && task_offsets[pos + 1] <= task) pos++;
    return pos;
}

// ------------------------------------------------------------ K1: update

// Stochastic rounding: Philox4x32-10 ("Parallel random numbers: as easy as
// 1, 2, 3", Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds, each
// multiplying counter words 0 and 2 by two fixed constants and mixing the
// high halves with the other words and the key, the key advanced by the two
// Weyl constants between rounds.  Counter (e / 4 as 64 bits, offset, tensor),
// key (seed); word e % 4 serves element e.
struct SrParams {
    uint64_t seed;
    uint32_t offset;
};

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t *out) {
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        // each 64-bit product as one v_mad_u64_u32 (both halves), not a
        // separate high and low multiply (32-bit integer multiplies issue at
        // a quarter of the VALU rate)
        const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// Random words of elements e .. e+3 (e a multiple of 4) of tensor `tensor`.
__device__ __forceinline__ void sr_words(int64_t e, const SrParams &sr, uint32_t tensor, uint32_t *out) {
    const uint64_t q = (uint64_t)e >> 2;
    philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), sr.offset, tensor, (uint32_t)sr.seed,
                  (uint32_t)(sr.seed >> 32), out);
}

// MXFP8 carrier output ("Quantized Muon Momentum", section "Wave18B MXFP8
// Carrier Probe"): instead of m in the grad buffer, E4M3 bytes of m / s and
// one E8M0 byte per 32 elements, s = 2^(floor(log2 max|m|) - 8) with the
// exponent clamped at -127 (the OCP Microscaling rule for E4M3).  The arrays
// hold every tensor of the plan: tensor t's bytes start at element
// 256 * (its first block).
struct CarrierOut {
    uint8_t *data;
    uint8_t *scale;
    uint64_t skip;   // tensors (index < 64) whose carrier another kernel writes (K1T): K1 leaves them alone
};

// What one update launch writes.
//  kOutM:    codes, absmax and m into the grad buffer (the update as defined).
//  kOutNorm: codes, absmax and m * (its group's inverse norm) into the grad
//            buffer: the second pass of the normalising update, after a
//            sums pass (q8_sums_kernel) and the group reduction.  m is
//            recomputed from the same inputs with the same operations, so it
//            has the sums pass's bits, and the value written is what an
//            in-place scale of the stored m makes of it: m rounded to the
//            grad dtype, times the inverse norm in fp32, rounded again.
// The two passes move 9.05 bytes per bf16 element (grad, codes and absmax
// read twice, written once) where the update followed by a scale pass moves
// 10.03: re-reading the state costs less than re-reading and rewriting m.
enum { kOutM = 0, kOutNorm = 1 };
struct NormIn {
    const int32_t *block_group;   // group of every block of the plan
    const float *inv;             // inverse norm of every group
};

// m as the grad buffer stores it, widened back to fp32
template <int DT> __device__ __forceinline__ float stored(float v) {
    if constexpr (DT == QM_F32) return v;
    else if constexpr (DT == QM_BF16) return bf16_val(bf16_rne(v));
    else return f16_val(f16_rne(v));
}

// One task's inputs as a lane holds them, still packed as loaded (all of a
// task's loads are issued before any arithmetic): per part, its kEpl codes
// (four per word) and grads (16 bytes), zero past the tensor's end, and its
// block's step absmax / 127.
template <int DT> struct TaskIn {
    static constexpr int EPL = Elem<DT>::kEpl;
    static constexpr int PARTS = kTaskElems / (64 * EPL);
    uint32_t qw[PARTS][EPL / 4];
    uint32_t gw[PARTS][4];
    float step[PARTS];
    int nvalid;   // elements of the task inside the tensor
};

// Element j of a lane's 16 grad bytes, widened to fp32.
template <int DT> __device__ __forceinline__ float grad_elem(const uint32_t *gw, int j) {
    if constexpr (DT == QM_F32) return __uint_as_float(gw[j]);
    else {
        const uint16_t h = (uint16_t)(gw[j / 2] >> (16 * (j % 2)));
        return DT == QM_BF16 ? bf16_val(h) : f16_val(h);
    }
}

// DEFER: the block maxima are loaded with the codes and grads and divided
// only once all of the task's loads are in flight (a lane past the tensor's
// end reads its task's last valid block and keeps step 0); otherwise each
// part's step is formed before its codes and grads are loaded.  Measured:
// deferring makes the grid-stride sums pass about 2 % faster and the
// one-task-per-wave update kernels up to 6 % slower.
template <int DT, bool DEFER>
__device__ __forceinline__ void load_task(const PlanTensor &T, int64_t lt, int lane, TaskIn<DT> &in) {
    constexpr int EPL = TaskIn<DT>::EPL, PARTS = TaskIn<DT>::PARTS, ES = Elem<DT>::kSize;
    const int64_t e_task = lt * kTaskElems;
    const int64_t rem = T.numel - e_task;
    const int nvalid = rem < kTaskElems ? (int)rem : kTaskElems;
    in.nvalid = nvalid;
    const int8_t *codes = gmem<const int8_t>(T.codes) + e_task;
    const float *absmax = gmem<const float>(T.absmax) + lt * kBlocksPerTask;
    const char *grad = gmem<const char>(T.grad);   // addressed through gpos
    float am[PARTS];
    if constexpr (DEFER)
#pragma unroll
        for (int p = 0; p < PARTS; p++) {
            const int e0 = p * 64 * EPL + lane * EPL;
            am[p] = absmax[(e0 < nvalid ? e0 : nvalid - 1) / kBlock];
        }
#pragma unroll
    for (int p = 0; p < PARTS; p++) {
        const int e0 = p * 64 * EPL + lane * EPL;
        if constexpr (!DEFER) in.step[p] = e0 < nvalid ? absmax[e0 / kBlock] / 127.0f : 0.0f;
        if (e0 + EPL <= nvalid) {
            const ntv4 v = __builtin_nontemporal_load(reinterpret_cast<const ntv4 *>(grad + gpos(T, e_task + e0) * ES));
            in.gw[p][0] = v.x; in.gw[p][1] = v.y; in.gw[p][2] = v.z; in.gw[p][3] = v.w;
            if constexpr (EPL == 8) {
                const ntv2 c = __builtin_nontemporal_load(reinterpret_cast<const ntv2 *>(codes + e0));
                in.qw[p][0] = c.x; in.qw[p][1] = c.y;
            } else {
                in.qw[p][0] = *reinterpret_cast<const uint32_t *>(codes + e0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; k++) in.gw[p][k] = 0u;
#pragma unroll
            for (int k = 0; k < EPL / 4; k++) in.qw[p][k] = 0u;
#pragma unroll
            for (int j = 0; j < EPL; j++) {
                if (e0 + j >= nvalid) continue;
                in.qw[p][j / 4] |= (uint32_t)(uint8_t)codes[e0 + j] << (8 * (j % 4));
                const char *gp = grad + gpos(T, e_task + e0 + j) * ES;
                if constexpr (DT == QM_F32) in.gw[p][j] = *reinterpret_cast<const uint32_t *>(gp);
                else in.gw[p][j / 2] |= (uint32_t)*reinterpret_cast<const uint16_t *>(gp) << (16 * (j % 2));
            }
        }
    }
    if constexpr (DEFER)
#pragma unroll
        for (int p = 0; p < PARTS; p++) in.step[p] = p * 64 * EPL + lane * EPL < nvalid ? am[p] / 127.0f : 0.0f;
}

// m = beta (q step) + (1 - beta) g: two rounded products and a rounded sum
__device__ __forceinline__ float ema1(int8_t q, float step, float g, float beta, float omb) {
    const float old = (float)q * step;
    const float t1 = beta * old;
    const float t2 = omb * g;
    return t1 + t2;
}

// m of part p of a loaded task
template <int DT>
__device__ __forceinline__ void ema_part(const TaskIn<DT> &in, int p, float beta, float omb, float *m) {
#pragma unroll
    for (int j = 0; j < TaskIn<DT>::EPL; j++)
        m[j] = ema1((int8_t)(in.qw[p][j / 4] >> (8 * (j % 4))), in.step[p], grad_elem<DT>(in.gw[p], j), beta, omb);
}

// Sum of m*m over one block: the lane's kEpl squares in fp64 in order, then
// a butterfly over the block's lanes (every lane of the block gets the sum).
template <int DT> __device__ __forceinline__ double block_sum(const float *mp) {
    constexpr int EPL = Elem<DT>::kEpl, LPB = kBlock / EPL;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        const double d = (double)mp[j];
        s += d * d;
    }
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) s += xor_lanes(s, off);
    return s;
}

template <int DT, bool SUMS, bool SR, bool CAR, int OUT>
__device__ __forceinline__ void update_task(const PlanTensor &T, int64_t lt, float beta, float omb,
                                            double *block_sums, int lane, const SrParams &sr, uint32_t tensor,
                                            const CarrierOut &co, const NormIn &nz) {
    static_assert(OUT != kOutNorm || (!SUMS && !CAR), "the normalising pass writes no sums and no carrier");
    constexpr int EPL = Elem<DT>::kEpl;
    constexpr int PARTS = kTaskElems / (64 * EPL);
    constexpr int LPB = kBlock / EPL;  // lanes per block
    constexpr int LPX = 32 / EPL;      // lanes per 32-element carrier block
    const int64_t e_task = lt * kTaskElems;
    int8_t *codes = gmem<int8_t>(T.codes) + e_task;
    float *absmax = gmem<float>(T.absmax) + lt * kBlocksPerTask;
    void *grad = gmem<void>(T.grad);   // addressed through gpos

    const int64_t rem = T.numel - e_task;
    const int nvalid = rem < kTaskElems ? (int)rem : kTaskElems;
    float m[PARTS][EPL];
    float gscale[PARTS];   // kOutNorm: the inverse norm of each part's block
    {
        // kOutNorm: each part's group (one group: wave-uniform, else the
        // block's entry) is looked up first, so that its inverse norm, which
        // depends on it, can be loaded while the task's loads are in flight
        int grp[PARTS];
#pragma unroll
        for (int p = 0; p < PARTS; p++) {
            const int e0 = p * 64 * EPL + lane * EPL;
            grp[p] = -1;
            if constexpr (OUT == kOutNorm)
                if (e0 < nvalid)
                    grp[p] = T.group_lo == T.group_hi
                                 ? T.group_lo
                                 : gmem(nz.block_group)[T.block_offset + lt * kBlocksPerTask + e0 / kBlock];
        }
        TaskIn<DT> in;
        load_task<DT, false>(T, lt, lane, in);   // every load of the task before any arithmetic
#pragma unroll
        for (int p = 0; p < PARTS; p++) {
            gscale[p] = 0.0f;
            if constexpr (OUT == kOutNorm)
                if (grp[p] >= 0) gscale[p] = gmem(nz.inv)[grp[p]];
        }
#pragma unroll
        for (int p = 0; p < PARTS; p++) ema_part<DT>(in, p, beta, omb, m[p]);
    }

#pragma unroll
    for (int p = 0; p < PARTS; p++) {
        const int e0 = p * 64 * EPL + lane * EPL;
        const int kb = e0 / kBlock;
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < EPL; j++) amax = fmaxf(amax, fabsf(m[p][j]));
        // the first butterfly stages reduce over the lanes of one 32-element
        // carrier block, the rest over the 256-element block
#pragma unroll
        for (int off = 1; off < LPX; off <<= 1) amax = fmaxf(amax, xor_lanes(amax, off));
        const float xmax = amax;
#pragma unroll
        for (int off = LPX; off < LPB; off <<= 1) amax = fmaxf(amax, xor_lanes(amax, off));
        float sc;
        const float inv = requant_inv(amax, sc);
        float mx[EPL];   // m, scaled by sc only when some lane of the wave has a tiny block
#pragma unroll
        for (int j = 0; j < EPL; j++) mx[j] = m[p][j];
        if (__any(sc != 1.0f))
#pragma unroll
            for (int j = 0; j < EPL; j++) mx[j] = m[p][j] * sc;
        uint32_t q[EPL];   // codes in the low bytes
        if constexpr (SR) {
            // floor(x) + 1 with probability frac(x); u = top 24 bits * 2^-24
            uint32_t w[EPL];
#pragma unroll
            for (int k = 0; k < EPL; k += 4) sr_words(e_task + e0 + k, sr, tensor, w + k);
#pragma unroll
            for (int j = 0; j < EPL; j++) {
                const float x = mx[j] * inv;
                const float fl = floorf(x);
                const float u = (float)(w[j] >> 8) * 0x1p-24f;
                float r = u < x - fl ? fl + 1.0f : fl;
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                q[j] = (uint32_t)(int)r;
            }
        } else {
            // clamped, then rounded to nearest even by adding 1.5 * 2^23, whose
            // ulp is 1: the sum's low byte is the code in two's complement.
            // The same codes as rounding first and clamping after (|x| <= 127
            // but for rounding; a NaN clamps to -127 either way).
#pragma unroll
            for (int j = 0; j < EPL; j++)
                q[j] = __float_as_uint(fminf(fmaxf(mx[j] * inv, -127.0f), 127.0f) + 0x1.8p23f);
        }
        if constexpr (CAR) {
            // E8M0 byte: biased exponent of xmax minus 8, 0 for zero / tiny blocks
            const uint32_t xe = __float_as_uint(xmax) >> 23;
            const uint32_t sb = xe > 8u ? xe - 8u : 0u;
            // lane l (l % 4 LPX == 0) collects the bytes of the four carrier
            // blocks from l on, stored as one word (all lanes take part)
            uint32_t sb4 = sb;
#pragma unroll
            for (int k = 1; k < 4; k++) sb4 |= (uint32_t)__shfl_down((int)sb, k * LPX) << (8 * k);
            // numel is a multiple of 32, so a carrier block is all valid or all past the end
            if (e0 < nvalid) {
                store_codes_vec<EPL>(codes, e0, q);
                const float inv_s = __uint_as_float((254u - sb) << 23);   // 2^(127 - sb), exact
                uint32_t w[EPL / 4];
#pragma unroll
                for (int k = 0; k < EPL / 4; k++) {
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; j++) x[j] = m[p][4 * k + j] * inv_s;   // exact: a power of two
                    w[k] = e4m3x4_rne_sat(x);
                }
                const int64_t ce = T.block_offset * kBlock + e_task + e0;
                if constexpr (EPL == 8)
                    *reinterpret_cast<uint2 *>(gmem(co.data) + ce) = make_uint2(w[0], w[1]);
                else
                    *reinterpret_cast<uint32_t *>(gmem(co.data) + ce) = w[0];
                if ((lane % (4 * LPX)) == 0) {
                    const int nb = (nvalid - e0) / 32;   // carrier blocks of the four inside the tensor
                    if (nb >= 4)
                        *reinterpret_cast<uint32_t *>(gmem(co.scale) + ce / 32) = sb4;   // ce / 32 is a multiple of 4
                    else
                        for (int k = 0; k < nb; k++) gmem(co.scale)[ce / 32 + k] = (uint8_t)(sb4 >> (8 * k));
                }
            }
        } else {
            // kOutNorm: the product is pinned to an fp32 register (empty asm)
            // before it is narrowed, or the f16 path fuses it into one
            // v_fma_mixlo_f16 and skips the product's fp32 rounding
            float y[EPL];
#pragma unroll
            for (int j = 0; j < EPL; j++) {
                if constexpr (OUT == kOutNorm) {
                    y[j] = stored<DT>(m[p][j]) * gscale[p];
                    asm volatile("" : "+v"(y[j]));
                } else {
                    y[j] = m[p][j];
                }
            }
            if (e0 + EPL <= nvalid) {
                store_codes_vec<EPL>(codes, e0, q);
                store_grad_vec<DT>(grad, gpos(T, e_task + e0), y);
            } else {
#pragma unroll
                for (int j = 0; j < EPL; j++)
                    if (e0 + j < nvalid) {
                        codes[e0 + j] = (int8_t)q[j];
                        narrow<DT>(grad, gpos(T, e_task + e0 + j), y[j]);
                    }
            }
        }
        double s = 0.0;
        if constexpr (SUMS) s = block_sum<DT>(m[p]);
        if ((lane % LPB) == 0 && kb * kBlock < nvalid) {
            absmax[kb] = amax;
            if constexpr (SUMS) block_sums[T.block_offset + lt * kBlocksPerTask + kb] = s;
        }
    }
}

// One launch per grad dtype present, over that dtype's task range (the plan
// orders the task space by dtype), so each kernel carries one element path.
// Specialised, the kernels fit 7-8 waves per SIMD (60-72 VGPRs) without
// spills; the launch bound asks for at least 8 on the 16-bit paths and 6 on
// the fp32 and stochastic-rounding ones (the kernel with all three element
// paths took 112 VGPRs, i.e. 4 waves).  Counters put the bf16 update near
// the VALU's limit as well as the memory's (about 415 VALU instructions per
// 1024-element task, 72 % of the VALU's cycles, before the last cuts), so
// per-element instructions matter: the hardware bf16 conversion, rounding by
// an added constant, byte permutes for the code words, swizzles for the
// butterflies, global rather than flat accesses.
template <int DT, bool SR> constexpr int update_wgs_per_cu() { return DT == QM_F32 || SR ? 6 : 8; }

template <int DT, bool SUMS, bool SR, bool CAR, int OUT>
__global__ __launch_bounds__(kThreads, (update_wgs_per_cu<DT, SR>())) void q8_update_kernel(
    const PlanTensor *__restrict__ tensors, const int64_t *__restrict__ task_offsets,
    const int32_t *__restrict__ task_tensor, int n_tensors, int64_t task_lo, int64_t task_hi, float beta,
    double *__restrict__ block_sums, SrParams sr, CarrierOut co, NormIn nz) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float omb = 1.0f - beta;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerWG;
    int pos = -1;
    for (int64_t task = task_lo + (int64_t)blockIdx.x * kWavesPerWG + wave; task < task_hi; task += stride) {
        pos = tensor_pos(task_offsets, n_tensors, pos, task);
        const int ti = task_tensor[pos];
        if constexpr (CAR) {
            if (ti < 64 && ((co.skip >> ti) & 1u)) continue;   // updated by the tall-carrier kernel
        }
        const PlanTensor T = tensors[ti];
        update_task<DT, SUMS, SR, CAR, OUT>(T, task - T.task_offset, beta, omb, block_sums, lane, sr, (uint32_t)ti, co,
                                            nz);
    }
}

// ------------------------------------------------ sums pass (normalising update)
// Block sums of m only, nothing else written; m and its sums are computed
// exactly as the update computes them.  A read-only stream runs fastest with
// a moderate grid whose waves sweep the data together (grid-stride): about 8
// workgroups per CU (measured 7.1 TB/s for a plain 16-byte read stream at
// that size, 5.5 with one task per wave).  Each wave finds its next tensor by
// a forward scan from the last one.
constexpr int kSumsGrid = 2048;

template <int DT>
__global__ __launch_bounds__(kThreads, (update_wgs_per_cu<DT, false>())) void q8_sums_kernel(
    const PlanTensor *__restrict__ tensors, const int64_t *__restrict__ task_offsets,
    const int32_t *__restrict__ task_tensor, int n_tensors, int64_t task_lo, int64_t task_hi, float beta,
    double *__restrict__ block_sums) {
    constexpr int EPL = Elem<DT>::kEpl, PARTS = TaskIn<DT>::PARTS, LPB = kBlock / EPL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float omb = 1.0f - beta;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerWG;
    int pos = -1;
    for (int64_t task = task_lo + (int64_t)blockIdx.x * kWavesPerWG + wave; task < task_hi; task += stride) {
        pos = tensor_pos(task_offsets, n_tensors, pos, task);
        const PlanTensor T = tensors[task_tensor[pos]];
        const int64_t lt = task - T.task_offset;
        TaskIn<DT> in;
        load_task<DT, true>(T, lt, lane, in);
        const int64_t boff = T.block_offset + lt * kBlocksPerTask;
#pragma unroll
        for (int p = 0; p < PARTS; p++) {
            const int e0 = p * 64 * EPL + lane * EPL;
            const int kb = e0 / kBlock;
            float m[EPL];
            ema_part<DT>(in, p, beta, omb, m);
            const double s = block_sum<DT>(m);
            if ((lane % LPB) == 0 && kb * kBlock < in.nvalid) block_sums[boff + kb] = s;
        }
    }
}

// ------------------------------------ K1T: tall matrices, carrier of m^T
// A tall rows x cols tensor (rows % kTallRows == 0, cols % 256 == 0) whose
// carrier goes to Newton-Schulz transposed: data (cols, rows) with byte
// [c][r] coding m[r][c], one E8M0 byte per 32 consecutive rows of a column.
// One workgroup per kTallRows x 256 tile, in passes of 32 rows.  Every row of
// the tile is one whole 256-element quantisation block, updated exactly as
// K1 does (codes, absmax, block sums of the same binary32 m) and, as in K1's
// 16-bit path, by 32 lanes of 8 consecutive elements: in step i of a pass,
// wave w's lane half h takes row 8 w + 4 h + i, lane l % 32 columns
// 8 (l % 32) .. + 7, so after four steps a lane holds four consecutive rows of
// eight columns.  The pass's 256 column-block maxima go through LDS, each lane
// encodes its 4 x 8 elements (one E4M3 word of four rows per column) and the
// words collect, transposed, in LDS; at the end every thread stores its
// column's kTallRows bytes and kTallRows / 32 scale bytes.
constexpr int kMaxTall = 8;
constexpr int kTallPasses = 1;
constexpr int kTallRows = 32 * kTallPasses;
struct TallItem {
    int32_t tensor;        // index in the plan's tensor table
    int32_t tiles_c;       // cols / 256
    int64_t rows, cols;
    int64_t tile_begin;    // first workgroup of this tensor
};
struct TallArgs {
    TallItem it[kMaxTall];
    int32_t n;
};

template <int DT, bool SUMS>
__global__ __launch_bounds__(kThreads) void q8_update_tcar_kernel(const PlanTensor *__restrict__ tensors, TallArgs ta,
                                                                 float beta, double *__restrict__ block_sums,
                                                                 CarrierOut co) {
    static_assert(kThreads == 256, "four waves of eight rows per pass");
    __shared__ float cmax[4][256];
    __shared__ float cinv[256];
    __shared__ uint32_t sbyte[256];
    __shared__ uint32_t tbytes[256][kTallRows / 4 + 1];   // column c's bytes as words (+1 against bank conflicts)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, cl = lane & 31;
    int k = 0;
    while (k + 1 < ta.n && ta.it[k + 1].tile_begin <= (int64_t)blockIdx.x) k++;
    const TallItem &it = ta.it[k];
    const int64_t t = (int64_t)blockIdx.x - it.tile_begin;
    const int64_t tr = t / it.tiles_c, tc = t % it.tiles_c;
    const int64_t r0 = kTallRows * tr, c0 = 256 * tc;
    const PlanTensor T = tensors[it.tensor];
    int8_t *codes = gmem<int8_t>(T.codes);
    float *absmax = gmem<float>(T.absmax);
    const float omb = 1.0f - beta;
    sbyte[threadIdx.x] = 0;

    for (int pass = 0; pass < kTallPasses; pass++) {
        float m[4][8];
        float cm[8];
#pragma unroll
        for (int j = 0; j < 8; j++) cm[j] = 0.0f;
        uint2 qv[4];
        float g[4][8];
        int64_t kb[4];
        float step[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {   // all loads of the pass first
            const int64_t r = r0 + 32 * pass + 8 * wave + 4 * h + i;
            const int64_t e = r * it.cols + c0 + 8 * cl;
            kb[i] = (r * it.cols + c0) / kBlock;   // the row segment's block
            step[i] = absmax[kb[i]] / 127.0f;
            const ntv2 qn = __builtin_nontemporal_load(reinterpret_cast<const ntv2 *>(codes + e));
            qv[i] = make_uint2(qn.x, qn.y);
            load_grad_vec<DT>(gmem<const void>(T.grad), gpos(T, e), g[i]);
            if constexpr (DT == QM_F32) load_grad_vec<DT>(gmem<const void>(T.grad), gpos(T, e) + 4, g[i] + 4);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t r = r0 + 32 * pass + 8 * wave + 4 * h + i;
            const int64_t e = r * it.cols + c0 + 8 * cl;
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t w = j < 4 ? qv[i].x : qv[i].y;
                const float old = (float)(int8_t)(w >> (8 * (j & 3))) * step[i];
                const float t1 = beta * old;
                const float t2 = omb * g[i][j];
                m[i][j] = t1 + t2;
                amax = fmaxf(amax, fabsf(m[i][j]));
                cm[j] = fmaxf(cm[j], fabsf(m[i][j]));
            }
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, xor_lanes(amax, off));
            float sc;
            const float inv = requant_inv(amax, sc);
            float mx[8];   // m, scaled by sc only when some lane of the wave has a tiny block
#pragma unroll
            for (int j = 0; j < 8; j++) mx[j] = m[i][j];
            if (__any(sc != 1.0f))
#pragma unroll
                for (int j = 0; j < 8; j++) mx[j] = m[i][j] * sc;
            // nearest rounding by the added 1.5 * 2^23, as in K1
            uint32_t q[8];
#pragma unroll
            for (int j = 0; j < 8; j++) q[j] = __float_as_uint(fminf(fmaxf(mx[j] * inv, -127.0f), 127.0f) + 0x1.8p23f);
            store_codes_vec<8>(codes, e, q);
            if constexpr (SUMS) {
                double sq = 0.0;
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const double d = (double)m[i][j];
                    sq += d * d;
                }
#pragma unroll
                for (int off = 1; off < 32; off <<= 1) sq += xor_lanes(sq, off);
                if (cl == 0) block_sums[T.block_offset + kb[i]] = sq;
            }
            if (cl == 0) absmax[kb[i]] = amax;
        }
        // column maxima over the wave's 8 rows (the two lane halves), then LDS
#pragma unroll
        for (int j = 0; j < 8; j++) cm[j] = fmaxf(cm[j], __shfl_xor(cm[j], 32));
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 8; j++) cmax[wave][8 * cl + j] = cm[j];
        }
        __syncthreads();
        {
            // column c = thread: its block maximum over the pass's 32 rows, the
            // E8M0 byte (biased exponent minus 8, 0 for zero or tiny blocks, as
            // in K1) and 2^(127 - byte) to scale by
            const int c = threadIdx.x;
            const float xm = fmaxf(fmaxf(cmax[0][c], cmax[1][c]), fmaxf(cmax[2][c], cmax[3][c]));
            const uint32_t xe = __float_as_uint(xm) >> 23;
            const uint32_t sb = xe > 8u ? xe - 8u : 0u;
            cinv[c] = __uint_as_float((254u - sb) << 23);
            sbyte[c] |= sb << (8 * pass);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int c = 8 * cl + j;
            const float sc = cinv[c];
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; i++) x[i] = m[i][j] * sc;   // exact: a power of two
            tbytes[c][8 * pass + 2 * wave + h] = e4m3x4_rne_sat(x);   // rows 8 w + 4 h .. + 3 of the pass
        }
        __syncthreads();   // cmax and cinv are rewritten by the next pass
    }
    {
        // the tile's carrier rows (columns c0 .. c0 + 255 of m) hold kTallRows
        // bytes each: CPR threads store one row as 16-byte pieces, so a wave
        // writes 64 / CPR whole row segments at a time
        constexpr int CPR = kTallRows / 16;
        uint8_t *dst0 = gmem(co.data) + T.block_offset * kBlock + c0 * it.rows + r0;
#pragma unroll
        for (int q = 0; q < CPR; q++) {
            const int c = (q * 256 + threadIdx.x) / CPR, k = threadIdx.x % CPR;
            *reinterpret_cast<uint4 *>(dst0 + (int64_t)c * it.rows + 16 * k) =
                make_uint4(tbytes[c][4 * k], tbytes[c][4 * k + 1], tbytes[c][4 * k + 2], tbytes[c][4 * k + 3]);
        }
        const int c = threadIdx.x;
        uint8_t *sdst = gmem(co.scale) + T.block_offset * (kBlock / 32) + (c0 + c) * (it.rows / 32) + r0 / 32;
        if constexpr (kTallPasses == 4) *reinterpret_cast<uint32_t *>(sdst) = sbyte[c];
        else
#pragma unroll
            for (int p = 0; p < kTallPasses; p++) sdst[p] = (uint8_t)(sbyte[c] >> (8 * p));
    }
}

// ------------------------------------------------- K2: group sums, inverse norms
// K2a: one workgroup per chunk (<= 256 runs of one group, each <= 16
// blocks).  Sixteen lanes take one run, one block each, so a wave reads four
// runs' block sums as four contiguous 128-byte pieces; a fixed butterfly
// over the sixteen lanes gives the run's sum.  The 16 run slots of the
// workgroup (4 waves x 4) each add their runs in pass order, and the slots
// are added in slot order.  K2b: one wave per group; lane l adds the
// group's chunk partials l, l + 64, ... in chunk order, then a butterfly over
// the 64 lanes adds the lane sums (every lane ends with the same bits: each
// level adds the same two values in either order).  Results depend only on
// the plan, never on scheduling, and no atomics are used.

__global__ __launch_bounds__(kThreads) void chunk_reduce_kernel(const int64_t *__restrict__ run_offsets,
                                                                const PlanRun *__restrict__ runs,
                                                                const int64_t *__restrict__ chunk_offsets,
                                                                const int32_t *__restrict__ chunk_group,
                                                                const double *__restrict__ block_sums,
                                                                double *__restrict__ partials) {
    static_assert(kRunMax == 16 && kChunkRuns % 16 == 0, "sixteen lanes per run");
    const int64_t c = blockIdx.x;
    const int g = chunk_group[c];
    const int64_t r0 = run_offsets[g] + (c - chunk_offsets[g]) * kChunkRuns;
    const int64_t r_end = run_offsets[g + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = wave * 4 + (lane >> 4), b = lane & 15;
    // All run descriptors of the chunk are loaded first, then all block
    // sums, so a workgroup waits for two memory latencies instead of two
    // per pass; the sums are then added in the same pass order as ever.
    constexpr int NP = kChunkRuns / 16;
    int64_t start[NP];
    int count[NP];
#pragma unroll
    for (int pass = 0; pass < NP; pass++) {
        const int64_t r = r0 + pass * 16 + slot;
        start[pass] = 0;
        count[pass] = 0;
        if (r < r_end) {
            const PlanRun R = runs[r];
            start[pass] = R.start_block;
            count[pass] = R.count;
        }
    }
    double v[NP];
#pragma unroll
    for (int pass = 0; pass < NP; pass++) v[pass] = b < count[pass] ? block_sums[start[pass] + b] : 0.0;
    double acc = 0.0;
#pragma unroll
    for (int pass = 0; pass < NP; pass++) {
        double x = v[pass];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) x += __shfl_xor(x, off);
        acc += x;
    }
    __shared__ double part[16];
    if (b == 0) part[slot] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double S = part[0];
        for (int k = 1; k < 16; k++) S += part[k];
        partials[c] = S;
    }
}

__global__ __launch_bounds__(64) void group_final_kernel(const int64_t *__restrict__ chunk_offsets,
                                                         const double *__restrict__ partials, float eps,
                                                         double *__restrict__ group_sums,
                                                         float *__restrict__ inv_norm) {
    const int g = blockIdx.x, lane = threadIdx.x;
    double S = 0.0;
    for (int64_t c = chunk_offsets[g] + lane; c < chunk_offsets[g + 1]; c += 64) S += partials[c];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) S += __shfl_xor(S, off);
    if (lane == 0) {
        if (group_sums) group_sums[g] = S;
        inv_norm[g] = (float)(1.0 / (sqrt(S) + (double)eps));
    }
}

// Workgroups per streaming launch: one task per wave (the kernels keep
// their grid-stride loop, which then runs once).  Measured on the 8B layer,
// this beat grids capped at 8, 16 or 32 workgroups per CU by 5-10 %: the
// hardware dispatcher keeps every CU's wave slots refilled as tasks finish.
int stream_grid(int64_t n_tasks) {
    const int64_t want = (n_tasks + kWavesPerWG - 1) / kWavesPerWG;
    const int64_t cap = (int64_t)1 << 30;
    return (int)(want < cap ? want : cap);
}

template <typename T> const T *section(const void *dev_plan, int64_t off) {
    return reinterpret_cast<const T *>(static_cast<const char *>(dev_plan) + off);
}

qm_status check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return QM_OK;
}

}  // namespace

qm_status validate_update(const void *host_plan, const void *dev_plan, float beta,
                          const PlanHeader **out) {
    qm_status st;
    const PlanHeader *h = plan_header(host_plan, &st);
    if (!h) return st;
    if (!dev_plan) return fail(QM_E_ARG, "device plan is null");
    if (!aligned(dev_plan, 8)) return fail(QM_E_ALIGN, "device plan must be 8-byte aligned");
    if (!(beta >= 0.0f && beta <= 1.0f)) return fail(QM_E_ARG, "beta must lie in [0, 1]");
    *out = h;
    return QM_OK;
}

template <int DT, bool SR, bool CAR, int OUT>
void launch_update_dt(const PlanHeader *h, const void *dev_plan, float beta, double *block_sums, const SrParams &sr,
                      const CarrierOut &co, const NormIn &nz, hipStream_t stream) {
    const int64_t lo = h->dt_task_lo[DT], hi = h->dt_task_hi[DT];
    if (hi <= lo) return;
    const PlanTensor *tens = section<PlanTensor>(dev_plan, h->off_tensors);
    const int64_t *toff = section<int64_t>(dev_plan, h->off_task_offsets);
    const int32_t *tt = section<int32_t>(dev_plan, h->off_task_tensor);
    auto go = [&](int64_t a, int64_t b) {
        const int grid = stream_grid(b - a);
        if constexpr (OUT == kOutNorm)
            launch(q8_update_kernel<DT, false, SR, false, OUT>, grid, kThreads, 0, stream, tens, toff, tt,
                   h->n_tensors, a, b, beta, nullptr, sr, co, nz);
        else if (block_sums)
            launch(q8_update_kernel<DT, true, SR, CAR, OUT>, grid, kThreads, 0, stream, tens, toff, tt, h->n_tensors,
                   a, b, beta, block_sums, sr, co, nz);
        else
            launch(q8_update_kernel<DT, false, SR, CAR, OUT>, grid, kThreads, 0, stream, tens, toff, tt, h->n_tensors,
                   a, b, beta, nullptr, sr, co, nz);
    };
    if (!(CAR && co.skip)) {
        go(lo, hi);
        return;
    }
    // Tensors whose carrier another kernel writes (K1T) get no waves at all:
    // one launch per run of consecutive other tensors in task order (the
    // host blob holds the same tables as the device copy).
    const int64_t *htoff = section<int64_t>(h, h->off_task_offsets);
    const int32_t *htt = section<int32_t>(h, h->off_task_tensor);
    int64_t run = -1;
    for (int k = 0; k < h->n_tensors; k++) {
        const int64_t a = htoff[k];
        if (htoff[k + 1] <= lo || a >= hi) continue;   // another dtype's range
        const int ti = htt[k];
        const bool skipped = ti < 64 && ((co.skip >> ti) & 1u);
        if (!skipped && run < 0) run = a;
        if (skipped && run >= 0) {
            go(run, a);
            run = -1;
        }
    }
    if (run >= 0) go(run, hi);
}

template <bool SR, bool CAR, int OUT = kOutM>
void launch_update_all(const PlanHeader *h, const void *dev_plan, float beta, double *block_sums,
                       const SrParams &sr, const CarrierOut &co, hipStream_t stream, const NormIn &nz = NormIn{}) {
    launch_update_dt<QM_F32, SR, CAR, OUT>(h, dev_plan, beta, block_sums, sr, co, nz, stream);
    launch_update_dt<QM_BF16, SR, CAR, OUT>(h, dev_plan, beta, block_sums, sr, co, nz, stream);
    launch_update_dt<QM_F16, SR, CAR, OUT>(h, dev_plan, beta, block_sums, sr, co, nz, stream);
}

// The tall tensors of one grad dtype, at most kMaxTall per launch.
template <int DT>
void launch_tall_dt(const PlanHeader *h, const void *host_plan, const void *dev_plan, float beta,
                    double *block_sums, const CarrierOut &co, const qm::TallCarrier *tall, int n_tall,
                    hipStream_t stream) {
    const PlanTensor *hp = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(host_plan) + h->off_tensors);
    TallArgs ta{};
    int64_t tiles = 0;
    auto flush = [&]() {
        if (ta.n == 0) return;
        const PlanTensor *tens = section<PlanTensor>(dev_plan, h->off_tensors);
        if (block_sums)
            launch(q8_update_tcar_kernel<DT, true>, (unsigned)tiles, kThreads, 0, stream, tens, ta, beta, block_sums, co);
        else
            launch(q8_update_tcar_kernel<DT, false>, (unsigned)tiles, kThreads, 0, stream, tens, ta, beta, nullptr, co);
        ta = TallArgs{};
        tiles = 0;
    };
    for (int k = 0; k < n_tall; k++) {
        if (hp[tall[k].tensor].dtype != DT) continue;
        TallItem &it = ta.it[ta.n++];
        it.tensor = tall[k].tensor;
        it.rows = tall[k].rows;
        it.cols = tall[k].cols;
        it.tiles_c = (int32_t)(it.cols / 256);
        it.tile_begin = tiles;
        tiles += (it.rows / kTallRows) * it.tiles_c;
        if (ta.n == kMaxTall) flush();
    }
    flush();
}

// co non-null: the carrier replaces the grad write (nearest rounding only);
// tall (with co): tensors whose carrier goes out transposed, by K1T.
qm_status launch_update(const PlanHeader *h, const void *dev_plan, float beta, double *block_sums,
                        const qm_round_opts *ro, const CarrierOut *co, hipStream_t stream,
                        const void *host_plan = nullptr, const qm::TallCarrier *tall = nullptr, int n_tall = 0) {
    Timed tm(stream, QM_K_Q8_UPDATE);
    if (co && n_tall > 0) {
        CarrierOut cs = *co;
        for (int k = 0; k < n_tall; k++) cs.skip |= (uint64_t)1 << tall[k].tensor;
        launch_update_all<false, true>(h, dev_plan, beta, block_sums, SrParams{0, 0}, cs, stream);
        launch_tall_dt<QM_F32>(h, host_plan, dev_plan, beta, block_sums, *co, tall, n_tall, stream);
        launch_tall_dt<QM_BF16>(h, host_plan, dev_plan, beta, block_sums, *co, tall, n_tall, stream);
        launch_tall_dt<QM_F16>(h, host_plan, dev_plan, beta, block_sums, *co, tall, n_tall, stream);
    } else if (co)
        launch_update_all<false, true>(h, dev_plan, beta, block_sums, SrParams{0, 0}, *co, stream);
    else if (ro && ro->rounding == QM_ROUND_STOCHASTIC)
        launch_update_all<true, false>(h, dev_plan, beta, block_sums, SrParams{ro->seed, ro->offset},
                                       CarrierOut{nullptr, nullptr, 0}, stream);
    else
        launch_update_all<false, false>(h, dev_plan, beta, block_sums, SrParams{0, 0},
                                        CarrierOut{nullptr, nullptr, 0}, stream);
    return check_launch("q8 update");
}

qm_status launch_group_reduce(const PlanHeader *h, const void *dev_plan, const double *block_sums,
                              double *partials, float eps, double *group_sums, float *inv, hipStream_t stream) {
    const int64_t *ro = section<int64_t>(dev_plan, h->off_run_offsets);
    const int64_t *co = section<int64_t>(dev_plan, h->off_chunk_offsets);
    Timed tm(stream, QM_K_GROUP_REDUCE);
    launch(chunk_reduce_kernel, (unsigned)h->n_chunks, kThreads, 0, stream,
        ro, section<PlanRun>(dev_plan, h->off_runs), co, section<int32_t>(dev_plan, h->off_chunk_group),
        block_sums, partials);
    qm_status st = check_launch("chunk reduce");
    if (st != QM_OK) return st;
    launch(group_final_kernel, (unsigned)h->n_groups, 64, 0, stream, co, partials, eps, group_sums, inv);
    return check_launch("group reduce");
}

template <int DT>
void launch_sums_dt(const PlanHeader *h, const void *dev_plan, float beta, double *block_sums, hipStream_t stream) {
    const int64_t lo = h->dt_task_lo[DT], hi = h->dt_task_hi[DT];
    if (hi <= lo) return;
    launch(q8_sums_kernel<DT>, std::min(stream_grid(hi - lo), kSumsGrid), kThreads, 0, stream,
        section<PlanTensor>(dev_plan, h->off_tensors), section<int64_t>(dev_plan, h->off_task_offsets),
        section<int32_t>(dev_plan, h->off_task_tensor), h->n_tensors, lo, hi, beta, block_sums);
}

// The normalising update in two streaming passes (the sums pass, then
// kOutNorm once the group reduction has the inverse norms).
qm_status launch_update_normalized(const PlanHeader *h, const void *dev_plan, float beta, const UpdateWorkspace &w,
                                   float eps, double *sums, float *inv, const qm_round_opts *ro, hipStream_t stream) {
    {
        Timed tm(stream, QM_K_Q8_SUMS);
        launch_sums_dt<QM_F32>(h, dev_plan, beta, w.block_sums, stream);
        launch_sums_dt<QM_BF16>(h, dev_plan, beta, w.block_sums, stream);
        launch_sums_dt<QM_F16>(h, dev_plan, beta, w.block_sums, stream);
        const qm_status st = check_launch("q8 sums pass");
        if (st != QM_OK) return st;
    }
    qm_status st = launch_group_reduce(h, dev_plan, w.block_sums, w.partials, eps, sums, inv, stream);
    if (st != QM_OK) return st;
    Timed tm(stream, QM_K_Q8_UPDATE);
    const NormIn nz{section<int32_t>(dev_plan, h->off_block_group), inv};
    if (ro && ro->rounding == QM_ROUND_STOCHASTIC)
        launch_update_all<true, false, kOutNorm>(h, dev_plan, beta, nullptr, SrParams{ro->seed, ro->offset},
                                                 CarrierOut{nullptr, nullptr, 0}, stream, nz);
    else
        launch_update_all<false, false, kOutNorm>(h, dev_plan, beta, nullptr, SrParams{0, 0},
                                                  CarrierOut{nullptr, nullptr, 0}, stream, nz);
    return check_launch("q8 normalising update");
}

UpdateWorkspace update_workspace(const PlanHeader *h, void *ws) {
    UpdateWorkspace w;
    char *p = static_cast<char *>(ws);
    w.block_sums = reinterpret_cast<double *>(p);
    p += align_up(h->n_blocks * 8, 256);
    w.partials = reinterpret_cast<double *>(p);
    p += align_up(h->n_chunks * 8, 256);
    w.group_sums = reinterpret_cast<double *>(p);
    p += align_up((int64_t)h->n_groups * 8, 256);
    w.inv = reinterpret_cast<float *>(p);
    p += align_up((int64_t)h->n_groups * 4, 256);
    w.bytes = (size_t)(p - static_cast<char *>(ws));
    return w;
}

qm_status run_update_normalize(const PlanHeader *h, const void *dev_plan, float beta, float eps,
                               bool write_normalized, float *inv_out, double *sums_out, void *ws,
                               const qm_round_opts *ro, hipStream_t stream, uint8_t *carrier_data,
                               uint8_t *carrier_scale, const void *host_plan, const TallCarrier *tall, int n_tall) {
    const UpdateWorkspace w = update_workspace(h, ws);
    float *inv = inv_out ? inv_out : w.inv;
    double *sums = sums_out ? sums_out : w.group_sums;
    if (write_normalized && !carrier_data)
        return launch_update_normalized(h, dev_plan, beta, w, eps, sums, inv, ro, stream);
    const CarrierOut co{carrier_data, carrier_scale, 0};
    qm_status st = launch_update(h, dev_plan, beta, w.block_sums, ro, carrier_data ? &co : nullptr, stream,
                                 host_plan, tall, n_tall);
    if (st != QM_OK) return st;
    return launch_group_reduce(h, dev_plan, w.block_sums, w.partials, eps, sums, inv, stream);
}

qm_status check_carrier(const PlanHeader *h, const void *host_plan, const void *data, const void *scale) {
    if (!data || !scale) return fail(QM_E_ARG, "carrier arrays must not be null");
    if (!aligned(data, 8)) return fail(QM_E_ALIGN, "carrier data must be 8-byte aligned");
    const PlanTensor *pt = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(host_plan) + h->off_tensors);
    for (int32_t i = 0; i < h->n_tensors; i++)
        if (pt[i].numel % 32)
            return fail(QM_E_SHAPE, "tensor %d: %lld elements, not a multiple of the 32-element carrier block", i,
                        (long long)pt[i].numel);
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(data), s0 = reinterpret_cast<uintptr_t>(scale);
    const uintptr_t dn = (uintptr_t)h->n_blocks * kBlock, sn = (uintptr_t)h->n_blocks * (kBlock / 32);
    auto meets = [](uintptr_t a, uintptr_t an, uintptr_t b, uintptr_t bn) { return a < b + bn && b < a + an; };
    if (meets(d0, dn, s0, sn)) return fail(QM_E_ARG, "carrier data and scales overlap");
    // neither array may overlap a tensor's codes, absmax or grad span
    for (int32_t i = 0; i < h->n_tensors; i++) {
        const PlanTensor &T = pt[i];
        const uintptr_t esz = T.dtype == QM_F32 ? 4 : 2;
        const uintptr_t nblk = (uintptr_t)((T.numel + kBlock - 1) / kBlock);
        const uintptr_t gspan = T.grad_cols ? (uintptr_t)((T.numel / T.grad_cols - 1) * T.grad_ld + T.grad_cols) * esz
                                            : (uintptr_t)T.numel * esz;
        const uintptr_t r[3][2] = {{T.codes, (uintptr_t)T.numel}, {T.absmax, nblk * 4}, {T.grad, gspan}};
        for (const auto &b : r)
            if (meets(d0, dn, b[0], b[1]) || meets(s0, sn, b[0], b[1]))
                return fail(QM_E_ARG, "carrier arrays overlap tensor %d's state or grad", i);
    }
    return QM_OK;
}

}  // namespace qm

using namespace qm;

namespace {

qm_status check_round(const qm_round_opts *ro) {
    if (ro && ro->rounding != QM_ROUND_NEAREST && ro->rounding != QM_ROUND_STOCHASTIC)
        return fail(QM_E_ARG, "unknown rounding mode %d", ro->rounding);
    return QM_OK;
}

qm_status update_multi(const void *host_plan, const void *dev_plan, float beta, const qm_round_opts *ro,
                       double *block_sumsq, qm_stream_t stream) {
    clear_error();
    const PlanHeader *h = nullptr;
    qm_status st = validate_update(host_plan, dev_plan, beta, &h);
    if (st != QM_OK) return st;
    if ((st = check_round(ro)) != QM_OK) return st;
    if (block_sumsq && !aligned(block_sumsq, 8)) return fail(QM_E_ALIGN, "block_sumsq must be 8-byte aligned");
    return launch_update(h, dev_plan, beta, block_sumsq, ro, nullptr, static_cast<hipStream_t>(stream));
}

qm_status update_normalize(const void *host_plan, const void *dev_plan, float beta, float eps,
                           int32_t write_normalized, const qm_round_opts *ro, float *group_inv_norm,
                           double *group_sumsq, void *ws, size_t ws_bytes, qm_stream_t stream) {
    clear_error();
    const PlanHeader *h = nullptr;
    qm_status st = validate_update(host_plan, dev_plan, beta, &h);
    if (st != QM_OK) return st;
    if ((st = check_round(ro)) != QM_OK) return st;
    if (!(eps >= 0.0f) || isinf(eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    if (write_normalized != 0 && write_normalized != 1) return fail(QM_E_ARG, "write_normalized must be 0 or 1");
    if (group_inv_norm && !aligned(group_inv_norm, 4)) return fail(QM_E_ALIGN, "group_inv_norm alignment");
    if (group_sumsq && !aligned(group_sumsq, 8)) return fail(QM_E_ALIGN, "group_sumsq alignment");
    const size_t need = qm_update_workspace_bytes(host_plan);
    if (!ws || ws_bytes < need)
        return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    return run_update_normalize(h, dev_plan, beta, eps, write_normalized != 0, group_inv_norm, group_sumsq, ws,
                                ro, static_cast<hipStream_t>(stream));
}

qm_status update_carrier(const void *host_plan, const void *dev_plan, float beta, float eps, uint8_t *data,
                         uint8_t *scale, float *inv_norm, double *group_sumsq, void *ws, size_t ws_bytes,
                         qm_stream_t stream) {
    clear_error();
    const PlanHeader *h = nullptr;
    qm_status st = validate_update(host_plan, dev_plan, beta, &h);
    if (st != QM_OK) return st;
    if ((st = check_carrier(h, host_plan, data, scale)) != QM_OK) return st;
    if (!(eps >= 0.0f) || isinf(eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    if (!inv_norm || !aligned(inv_norm, 4)) return fail(QM_E_ARG, "inv_norm must be a 4-byte aligned device pointer");
    if (group_sumsq && !aligned(group_sumsq, 8)) return fail(QM_E_ALIGN, "group_sumsq alignment");
    const size_t need = qm_update_workspace_bytes(host_plan);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    return run_update_normalize(h, dev_plan, beta, eps, false, inv_norm, group_sumsq, ws, nullptr,
                                static_cast<hipStream_t>(stream), data, scale);
}

}  // namespace

// ---------------------------------------------------- no-allocation variant
//
// qmuon_update_normalize_groups for callers that cannot allocate: its
// workspace (per-block fp64 sums, chunk partials, group sums, inverse norms;
// every byte written before it is read in a call, so nothing is cleared) is
// a fixed array in device memory, one per GPU, held until the process ends.
// In host code `scratch` only names the array; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static_assert(QM_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[QM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = QM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices] = {};

qm_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(QM_E_HIP, "no current device");
    if (dev >= kMaxScratchDevices) return fail(QM_E_UNSUPPORTED, "device %d beyond the scratch table", dev);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(QM_E_HIP, "scratch address: %s", hipGetErrorString(e));
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return QM_OK;
}

}  // namespace

extern "C" qm_status qmuon_update_normalize_groups_noalloc(const void *host_plan, const void *dev_plan, float beta,
                                                           float eps, int32_t write_normalized,
                                                           float *group_inv_norm, double *group_sumsq,
                                                           qm_stream_t stream) {
    clear_error();
    const PlanHeader *h = nullptr;
    qm_status st = validate_update(host_plan, dev_plan, beta, &h);
    if (st != QM_OK) return st;
    const size_t need = qm_update_workspace_bytes(host_plan);
    if (need > kScratchBytes)
        return fail(QM_E_WORKSPACE, "plan needs %zu bytes of workspace, above the %zu-byte static scratch", need,
                    kScratchBytes);
    if (!(eps >= 0.0f) || isinf(eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    if (write_normalized != 0 && write_normalized != 1) return fail(QM_E_ARG, "write_normalized must be 0 or 1");
    if (group_inv_norm && !aligned(group_inv_norm, 4)) return fail(QM_E_ALIGN, "group_inv_norm alignment");
    if (group_sumsq && !aligned(group_sumsq, 8)) return fail(QM_E_ALIGN, "group_sumsq alignment");
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != QM_OK) return st;
    return run_update_normalize(h, dev_plan, beta, eps, write_normalized != 0, group_inv_norm, group_sumsq, ws,
                                nullptr, static_cast<hipStream_t>(stream));
}

extern "C" qm_status qmuon_update_mxfp8_carrier(const void *host_plan, const void *dev_plan, float beta, float eps,
                                                uint8_t *rowwise_data, uint8_t *rowwise_scale_inv, float *inv_norm,
                                                double *group_sumsq, void *ws, size_t ws_bytes, qm_stream_t stream) {
    return update_carrier(host_plan, dev_plan, beta, eps, rowwise_data, rowwise_scale_inv, inv_norm, group_sumsq, ws,
                          ws_bytes, stream);
}

extern "C" qm_status qmuon_update_multi(const void *host_plan, const void *dev_plan, float beta,
                                        double *block_sumsq, qm_stream_t stream) {
    return update_multi(host_plan, dev_plan, beta, nullptr, block_sumsq, stream);
}

extern "C" qm_status qmuon_update_multi_ex(const void *host_plan, const void *dev_plan, float beta,
                                           const qm_round_opts *opts, double *block_sumsq, qm_stream_t stream) {
    return update_multi(host_plan, dev_plan, beta, opts, block_sumsq, stream);
}

extern "C" qm_status qmuon_update_normalize_groups(const void *host_plan, const void *dev_plan, float beta,
                                                   float eps, int32_t write_normalized, float *group_inv_norm,
                                                   double *group_sumsq, void *ws, size_t ws_bytes,
                                                   qm_stream_t stream) {
    return update_normalize(host_plan, dev_plan, beta, eps, write_normalized, nullptr, group_inv_norm, group_sumsq,
                            ws, ws_bytes, stream);
}

extern "C" qm_status qmuon_update_normalize_groups_ex(const void *host_plan, const void *dev_plan, float beta,
                                                      float eps, int32_t write_normalized, const qm_round_opts *opts,
                                                      float *group_inv_norm, double *group_sumsq, void *ws,
                                                      size_t ws_bytes, qm_stream_t stream) {
    return update_normalize(host_plan, dev_plan, beta, eps, write_normalized, opts, group_inv_norm, group_sumsq, ws,
                            ws_bytes, stream);
}
