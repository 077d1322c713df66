// Quintic Newton-Schulz orthogonalisation on gfx950 MFMA, plus the full
// optimizer step built on it.
//
// What is computed ("NVIDIA impulsa optimizadores ... con Megatron",
// "Newton-Schulz distribuido" and "SYRK y reducción fusionada"; "MuonBP:
// Faster Muon via Block-Periodic Orthogonalization", key designs 1-3):
//   X0 = orient(M) * inv_norm        (orient: transpose if rows > cols)
//   T times:  A = X X^T;  B = b A + c A A;  X = a X + B X
//   output = orient^-1(X_T) in the input's dtype; optionally
//   W <- W - lr (s O + wd W).
//
// MI355X design (not the pages' Triton/CUDA kernels):
//   * All three products are written C[i][j] = sum_k P[i][k] Q[j][k] with
//     both operands row-major and K-contiguous: A = X X^T takes P = Q = X;
//     A A = A A^T (A symmetric) takes P = Q = A; B X takes P = B and
//     Q = X^T, a transposed copy of X that the previous product's epilogue
//     writes alongside X.  One MFMA kernel template serves all of them.
//   * The two symmetric products run only on lower-triangle tiles and store
//     each off-diagonal tile twice (the SYRK shortcut).
//   * Tiles are loaded global -> registers -> LDS (double buffered, one
//     barrier per k-tile) with a 16-byte XOR swizzle against bank conflicts;
//     every lane feeds v_mfma_f32_32x32x16_bf16 (or 32x32x2 f32) from one
//     16-byte LDS read per operand per step.
//   * Workgroup ids are remapped so each XCD (own L2) gets a contiguous
//     range of tiles.
//   * Internal buffers are zero-padded to multiples of 256: zero rows and
//     columns stay zero through the iteration, so no kernel needs bounds
//     checks in its main loop.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "internal.h"
#include "plan_layout.h"
#include "q8_internal.h"
#include "qmuon.h"

namespace qm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kPad = 256;       // internal dims are multiples of this
constexpr int kMaxItems = 8;    // matrices per launch chain
constexpr int kNormChunks = 256;

int64_t pad_up(int64_t v) { return (v + kPad - 1) / kPad * kPad; }

// ------------------------------------------------------------ conversions

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

struct bf16_t {
    uint16_t bits;
};

template <typename T> __device__ __forceinline__ T from_float(float v);
template <> __device__ __forceinline__ float from_float<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_float<bf16_t>(float v) { return bf16_t{to_bf16_bits(v)}; }

__device__ __forceinline__ float to_float(float v) { return v; }
__device__ __forceinline__ float to_float(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

__device__ __forceinline__ float load_any(const void *p, int64_t i, int dtype) {
    if (dtype == QM_F32) return static_cast<const float *>(p)[i];
    const uint16_t h = static_cast<const uint16_t *>(p)[i];
    if (dtype == QM_BF16) return __uint_as_float((uint32_t)h << 16);
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ void store_any(void *p, int64_t i, int dtype, float v) {
    if (dtype == QM_F32) static_cast<float *>(p)[i] = v;
    else if (dtype == QM_BF16) static_cast<uint16_t *>(p)[i] = to_bf16_bits(v);
    else static_cast<uint16_t *>(p)[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// ------------------------------------------------------------ MFMA step
// One step consumes one 16-byte LDS read per operand per lane.  bf16: the
// 8 values are k = 8h..8h+7 of a 16-wide slice (h = lane / 32), one
// 32x32x16 MFMA.  f32: the 4 values feed four 32x32x2 MFMAs; value j of
// lane half h is k-slot h of MFMA j.  Any k assignment is valid as long as
// both operands use the same one.

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static __device__ __forceinline__ void step(const u32x4 &a, const u32x4 &b, f32x16 &c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static __device__ __forceinline__ void step(const u32x4 &a, const u32x4 &b, f32x16 &c) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

// ------------------------------------------------------------ GEMM kernel

enum Epi { EPI_GRAM = 0, EPI_POLY = 1, EPI_UPDATE = 2, EPI_FINAL = 3 };

// Where the last product writes: the caller's matrix (original orientation,
// its dtype) and optionally fp32 weights.
struct FinalOut {
    void *out;
    float *w;
    int64_t ld, ldw;
    int32_t dtype, tall;
    int32_t m, n;          // valid extent in iteration orientation
    float lr_s, lr_wd;     // lr * s and lr * weight_decay
};

template <typename T> struct GemmArgs {
    const T *P; int64_t ldp, sp;   // element strides: row, item
    const T *Q; int64_t ldq, sq;
    T *C; int64_t ldc, sc;         // primary output
    T *CT; int64_t ldct, sct;      // transposed output (EPI_UPDATE)
    const T *D; int64_t ldd, sd;   // epilogue input
    int32_t tiles_m, tiles_n;      // tile grid per item (tiles_m == tiles_n for SYM)
    int32_t tiles_per_item, n_items;
    int32_t k_tiles;               // K / (128 / sizeof(T))
    float alpha, beta;
    FinalOut fo[kMaxItems];
};

// Logical tile for workgroup w: workgroups are issued to the 8 XCDs round
// robin; give every XCD a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int w, int nwg) {
    const int per = nwg / 8, rem = nwg % 8;
    const int x = w % 8, l = w / 8;
    return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + l;
}

__device__ __forceinline__ void tri_coords(int t, int &bi, int &bj) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > t) i--;
    while ((i + 1) * (i + 2) / 2 <= t) i++;
    bi = i;
    bj = t - i * (i + 1) / 2;
}

template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int EPI, bool SYM>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void gemm_nt_kernel(GemmArgs<T> args) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int ROWB = 128;                     // LDS bytes per tile row (one k-tile)
    constexpr int P_LOADS = BM * 8 / NT, Q_LOADS = BN * 8 / NT;
    static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile / thread count");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *sP = smem;                       // [2][BM][128]
    char *sQ = smem + 2 * BM * ROWB;       // [2][BN][128]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int item = L / args.tiles_per_item;
    const int t = L % args.tiles_per_item;
    int bi, bj;
    if constexpr (SYM) {
        tri_coords(t, bi, bj);
    } else {
        bi = t / args.tiles_n;
        bj = t % args.tiles_n;
    }

    const char *Pg = reinterpret_cast<const char *>(args.P + item * args.sp + (int64_t)bi * BM * args.ldp);
    const char *Qg = reinterpret_cast<const char *>(args.Q + item * args.sq + (int64_t)bj * BN * args.ldq);
    const int64_t ldpb = args.ldp * (int64_t)sizeof(T), ldqb = args.ldq * (int64_t)sizeof(T);

    u32x4 rp[P_LOADS], rq[Q_LOADS];
#define QM_GLOAD(kt)                                                                              \
    do {                                                                                          \
        _Pragma("unroll") for (int i_ = 0; i_ < P_LOADS; i_++) {                                  \
            const int idx = tid + i_ * NT, row = idx >> 3, ch = idx & 7;                          \
            rp[i_] = *reinterpret_cast<const u32x4 *>(Pg + row * ldpb + (int64_t)(kt)*ROWB + ch * 16); \
        }                                                                                         \
        _Pragma("unroll") for (int i_ = 0; i_ < Q_LOADS; i_++) {                                  \
            const int idx = tid + i_ * NT, row = idx >> 3, ch = idx & 7;                          \
            rq[i_] = *reinterpret_cast<const u32x4 *>(Qg + row * ldqb + (int64_t)(kt)*ROWB + ch * 16); \
        }                                                                                         \
    } while (0)
#define QM_SWRITE(buf)                                                                            \
    do {                                                                                          \
        char *dp_ = sP + (buf)*BM * ROWB;                                                         \
        char *dq_ = sQ + (buf)*BN * ROWB;                                                         \
        _Pragma("unroll") for (int i_ = 0; i_ < P_LOADS; i_++) {                                  \
            const int idx = tid + i_ * NT, row = idx >> 3, ch = idx & 7;                          \
            *reinterpret_cast<u32x4 *>(dp_ + row * ROWB + ((ch ^ (row & 7)) << 4)) = rp[i_];      \
        }                                                                                         \
        _Pragma("unroll") for (int i_ = 0; i_ < Q_LOADS; i_++) {                                  \
            const int idx = tid + i_ * NT, row = idx >> 3, ch = idx & 7;                          \
            *reinterpret_cast<u32x4 *>(dq_ + row * ROWB + ((ch ^ (row & 7)) << 4)) = rq[i_];      \
        }                                                                                         \
    } while (0)

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int KT = args.k_tiles;
    QM_GLOAD(0);
    QM_SWRITE(0);
    __syncthreads();
    const int lrow = lane & 31, lhalf = lane >> 5;
    for (int kt = 0; kt < KT; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < KT) QM_GLOAD(kt + 1);
        const char *cp = sP + cur * BM * ROWB;
        const char *cq = sQ + cur * BN * ROWB;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int ch = 2 * s + lhalf;
            u32x4 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int row = wm * WM + i * 32 + lrow;
                a[i] = *reinterpret_cast<const u32x4 *>(cp + row * ROWB + ((ch ^ (row & 7)) << 4));
            }
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int row = wn * WN + j * 32 + lrow;
                b[j] = *reinterpret_cast<const u32x4 *>(cq + row * ROWB + ((ch ^ (row & 7)) << 4));
            }
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) Mfma<T>::step(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < KT) QM_SWRITE(cur ^ 1);
        __syncthreads();
    }

#undef QM_GLOAD
#undef QM_SWRITE

    // ---------------------------------------------------------- epilogue
    // acc[i][j][r] holds C[row][col] with row = 8(r/4) + 4 lhalf + r%4 and
    // col = lrow inside the 32x32 MFMA tile.
    const bool mirror = SYM && bi != bj;
    T *C = args.C + item * args.sc;
    T *CT = args.CT ? args.CT + item * args.sct : nullptr;
    const T *D = args.D ? args.D + item * args.sd : nullptr;
    const FinalOut &fo = args.fo[item < kMaxItems ? item : 0];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t gr = (int64_t)bi * BM + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
                const int64_t gc = (int64_t)bj * BN + wn * WN + j * 32 + lrow;
                float v = acc[i][j][r];
                if constexpr (EPI == EPI_GRAM) {
                    const T o = from_float<T>(v);
                    C[gr * args.ldc + gc] = o;
                    if (mirror) C[gc * args.ldc + gr] = o;
                } else if constexpr (EPI == EPI_POLY) {
                    v = args.alpha * to_float(D[gr * args.ldd + gc]) + args.beta * v;
                    const T o = from_float<T>(v);
                    C[gr * args.ldc + gc] = o;
                    if (mirror) C[gc * args.ldc + gr] = o;
                } else if constexpr (EPI == EPI_UPDATE) {
                    v = args.alpha * to_float(D[gr * args.ldd + gc]) + v;
                    const T o = from_float<T>(v);
                    C[gr * args.ldc + gc] = o;
                    CT[gc * args.ldct + gr] = o;
                } else {
                    v = args.alpha * to_float(D[gr * args.ldd + gc]) + v;
                    if (gr < fo.m && gc < fo.n) {
                        // original orientation: (gr, gc) or transposed
                        const int64_t idx = fo.tall ? gc * fo.ld + gr : gr * fo.ld + gc;
                        store_any(fo.out, idx, fo.dtype, v);
                        if (fo.w) {
                            const int64_t wi = fo.tall ? gc * fo.ldw + gr : gr * fo.ldw + gc;
                            const float w = fo.w[wi];
                            fo.w[wi] = w - (fo.lr_s * v + fo.lr_wd * w);
                        }
                    }
                }
            }
}

// ------------------------------------------------------- norm + prologue

struct NsItem {
    const void *src;
    int64_t ld;
    int32_t dtype;
    int32_t tall;
    const float *inv;   // device scale, or null: compute from the data
};

struct PrologueArgs {
    NsItem it[kMaxItems];
    int32_t m, n;                  // valid extent in iteration orientation
    int64_t mp, np;                // padded
    int32_t tiles_n, tiles_per_item;
    void *X; void *XT; int64_t item_stride;   // element stride between items
    const float *inv_ws;           // per-item computed scales (when it[i].inv is null)
};

// Partial sums of squares: grid (kNormChunks, items); each workgroup covers
// a fixed slice of the item's rows.
__global__ __launch_bounds__(256) void norm_partial_kernel(PrologueArgs a, double *partials) {
    const int item = blockIdx.y;
    const NsItem &it = a.it[item];
    const int64_t rows = it.tall ? a.n : a.m, cols = it.tall ? a.m : a.n;
    const int64_t per = (rows + kNormChunks - 1) / kNormChunks;
    const int64_t r0 = blockIdx.x * per, r1 = min(rows, r0 + per);
    double acc = 0.0;
    for (int64_t r = r0; r < r1; r++)
        for (int64_t c = threadIdx.x; c < cols; c += 256) {
            const double v = (double)load_any(it.src, r * it.ld + c, it.dtype);
            acc += v * v;
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    __shared__ double part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) partials[item * kNormChunks + blockIdx.x] = ((part[0] + part[1]) + part[2]) + part[3];
}

__global__ void norm_final_kernel(const double *partials, float eps, float *inv_out) {
    const int item = blockIdx.x;
    if (threadIdx.x != 0) return;
    double s = 0.0;
    for (int k = 0; k < kNormChunks; k++) s += partials[item * kNormChunks + k];
    inv_out[item] = (float)(1.0 / (sqrt(s) + (double)eps));
}

// X0 = orient(src) * inv, written as X (m_p x n_p) and X^T (n_p x m_p),
// zero outside the valid extent.  One 64x64 tile per workgroup, transposed
// through LDS so that source reads and both writes are row-contiguous.
template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
    __shared__ float tile[64][65];
    const int item = blockIdx.x / a.tiles_per_item;
    const int t = blockIdx.x % a.tiles_per_item;
    const int64_t i0 = (int64_t)(t / a.tiles_n) * 64, j0 = (int64_t)(t % a.tiles_n) * 64;
    const NsItem &it = a.it[item];
    const float s = it.inv ? it.inv[0] : a.inv_ws[item];
    for (int idx = threadIdx.x; idx < 4096; idx += 256) {
        // read along the source's contiguous dimension
        const int ii = it.tall ? (idx & 63) : (idx >> 6);
        const int jj = it.tall ? (idx >> 6) : (idx & 63);
        const int64_t i = i0 + ii, j = j0 + jj;
        float v = 0.0f;
        if (i < a.m && j < a.n) {
            const int64_t src = it.tall ? j * it.ld + i : i * it.ld + j;
            v = load_any(it.src, src, it.dtype) * s;
        }
        tile[ii][jj] = v;
    }
    __syncthreads();
    T *X = static_cast<T *>(a.X) + item * a.item_stride;
    T *XT = static_cast<T *>(a.XT) + item * a.item_stride;
    for (int idx = threadIdx.x; idx < 4096; idx += 256) {
        const int ii = idx >> 6, jj = idx & 63;
        X[(i0 + ii) * a.np + j0 + jj] = from_float<T>(tile[ii][jj]);
        XT[(j0 + ii) * a.mp + i0 + jj] = from_float<T>(tile[jj][ii]);
    }
}

// steps == 0: the output is X0 itself.
template <typename T>
__global__ __launch_bounds__(256) void writeback_kernel(const T *X, int64_t item_stride, int64_t np,
                                                        int32_t tiles_n, int32_t tiles_per_item,
                                                        GemmArgs<T> g) {
    const int item = blockIdx.x / tiles_per_item;
    const int t = blockIdx.x % tiles_per_item;
    const int64_t i0 = (int64_t)(t / tiles_n) * 64, j0 = (int64_t)(t % tiles_n) * 64;
    const FinalOut &fo = g.fo[item];
    const T *Xi = X + item * item_stride;
    for (int idx = threadIdx.x; idx < 4096; idx += 256) {
        const int64_t i = i0 + (idx >> 6), j = j0 + (idx & 63);
        if (i >= fo.m || j >= fo.n) continue;
        const float v = to_float(Xi[i * np + j]);
        const int64_t o = fo.tall ? j * fo.ld + i : i * fo.ld + j;
        store_any(fo.out, o, fo.dtype, v);
        if (fo.w) {
            const int64_t wi = fo.tall ? j * fo.ldw + i : i * fo.ldw + j;
            const float w = fo.w[wi];
            fo.w[wi] = w - (fo.lr_s * v + fo.lr_wd * w);
        }
    }
}

// ------------------------------------------------------------ host driver

struct NsRequest {
    const void *src;      // matrix start
    void *out;            // where the result goes (== src for in place)
    int64_t rows, cols, ld;
    int32_t dtype;
    const float *inv;     // nullable device scale
    float *w;             // nullable fp32 weights (rows x cols, ldw)
    int64_t ldw;
    float lr_s, lr_wd;
};

struct Geometry {
    int64_t m, n, mp, np;
    size_t esz;
    int64_t x_elems, a_elems;    // per item
    size_t item_bytes;           // X + XT0 + XT1 + A + B, each 256-aligned
};

Geometry geometry(int64_t rows, int64_t cols, int precision) {
    Geometry g;
    g.m = std::min(rows, cols);
    g.n = std::max(rows, cols);
    g.mp = pad_up(g.m);
    g.np = pad_up(g.n);
    g.esz = precision == QM_NS_F32 ? 4 : 2;
    g.x_elems = g.mp * g.np;
    g.a_elems = g.mp * g.mp;
    g.item_bytes = 3 * align_up(g.x_elems * (int64_t)g.esz, 256) + 2 * align_up(g.a_elems * (int64_t)g.esz, 256);
    return g;
}

size_t ns_ws_bytes_for(int64_t rows, int64_t cols, int64_t items, int precision) {
    const Geometry g = geometry(rows, cols, precision);
    const int64_t k = std::min<int64_t>(items, kMaxItems);
    return (size_t)k * g.item_bytes + align_up(kMaxItems * kNormChunks * 8, 256) + align_up(kMaxItems * 4, 256);
}

template <typename T, int BM, int BN, int WMW, int WNW, int EPI, bool SYM>
qm_status launch_gemm(const GemmArgs<T> &args, int grid, hipStream_t stream) {
    constexpr int NT = WMW * WNW * 64;
    constexpr size_t lds = 2 * (BM + BN) * 128;
    auto kern = gemm_nt_kernel<T, BM, BN, WMW, WNW, EPI, SYM>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return fail(QM_E_HIP, "cannot reserve %zu bytes of LDS", lds);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds, stream, args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    return QM_OK;
}

// Tile configuration of the NS products.
constexpr int kBM = 128, kBN = 128, kWM = 2, kWN = 2;

template <typename T>
qm_status run_ns_typed(const std::vector<NsRequest> &req, int steps, float a, float b, float c, float eps,
                       void *ws, hipStream_t stream) {
    const Geometry g = geometry(req[0].rows, req[0].cols, sizeof(T) == 4 ? QM_NS_F32 : QM_NS_BF16);
    // Layout (as sized by ns_ws_bytes_for): kcap items, then the norm
    // partials, then the computed inverse norms.
    char *base = static_cast<char *>(ws);
    const int64_t kcap = std::min<int64_t>((int64_t)req.size(), kMaxItems);
    double *partials = reinterpret_cast<double *>(base + kcap * g.item_bytes);
    float *inv_ws = reinterpret_cast<float *>(base + kcap * g.item_bytes + align_up(kMaxItems * kNormChunks * 8, 256));

    for (size_t first = 0; first < req.size(); first += kMaxItems) {
        const int nit = (int)std::min<size_t>(kMaxItems, req.size() - first);
        // Item-major layout of the workspace: all X, then all XT0, XT1, A, B,
        // so that every buffer kind has one uniform item stride.
        const int64_t xs = align_up(g.x_elems * (int64_t)sizeof(T), 256) / (int64_t)sizeof(T);
        const int64_t as = align_up(g.a_elems * (int64_t)sizeof(T), 256) / (int64_t)sizeof(T);
        T *X = reinterpret_cast<T *>(base);
        T *XT0 = X + nit * xs;
        T *XT1 = XT0 + nit * xs;
        T *A = XT1 + nit * xs;
        T *B = A + nit * as;

        PrologueArgs pa{};
        bool need_norm = false;
        for (int i = 0; i < nit; i++) {
            const NsRequest &r = req[first + i];
            pa.it[i] = NsItem{r.src, r.ld, r.dtype, r.rows > r.cols ? 1 : 0, r.inv};
            need_norm |= r.inv == nullptr;
        }
        pa.m = (int32_t)g.m;
        pa.n = (int32_t)g.n;
        pa.mp = g.mp;
        pa.np = g.np;
        pa.tiles_n = (int32_t)(g.np / 64);
        pa.tiles_per_item = (int32_t)((g.mp / 64) * (g.np / 64));
        pa.X = X;
        pa.XT = XT0;
        pa.item_stride = xs;
        pa.inv_ws = inv_ws;
        if (need_norm) {
            norm_partial_kernel<<<dim3(kNormChunks, nit), 256, 0, stream>>>(pa, partials);
            norm_final_kernel<<<nit, 64, 0, stream>>>(partials, eps, inv_ws);
        }
        prologue_kernel<T><<<pa.tiles_per_item * nit, 256, 0, stream>>>(pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(QM_E_HIP, "prologue: %s", hipGetErrorString(e));

        GemmArgs<T> ga{};
        for (int i = 0; i < nit; i++) {
            const NsRequest &r = req[first + i];
            ga.fo[i] = FinalOut{r.out, r.w, r.ld, r.ldw, r.dtype, r.rows > r.cols ? 1 : 0,
                                (int32_t)g.m, (int32_t)g.n, r.lr_s, r.lr_wd};
        }
        if (steps == 0) {
            writeback_kernel<T><<<pa.tiles_per_item * nit, 256, 0, stream>>>(X, xs, g.np, pa.tiles_n,
                                                                              pa.tiles_per_item, ga);
            e = hipGetLastError();
            if (e != hipSuccess) return fail(QM_E_HIP, "writeback: %s", hipGetErrorString(e));
            continue;
        }
        const int tm = (int)(g.mp / kBM), tn = (int)(g.np / kBN);
        const int tri = tm * (tm + 1) / 2;
        constexpr int kElemsPerKTile = 128 / (int)sizeof(T);
        T *XTc = XT0, *XTn = XT1;
        for (int s = 0; s < steps; s++) {
            // A = X X^T
            GemmArgs<T> g1 = ga;
            g1.P = X; g1.ldp = g.np; g1.sp = xs;
            g1.Q = X; g1.ldq = g.np; g1.sq = xs;
            g1.C = A; g1.ldc = g.mp; g1.sc = as;
            g1.tiles_m = tm; g1.tiles_n = tm; g1.tiles_per_item = tri; g1.n_items = nit;
            g1.k_tiles = (int32_t)(g.np / kElemsPerKTile);
            qm_status st = launch_gemm<T, kBM, kBN, kWM, kWN, EPI_GRAM, true>(g1, tri * nit, stream);
            if (st != QM_OK) return st;
            // B = b A + c A A
            GemmArgs<T> g2 = ga;
            g2.P = A; g2.ldp = g.mp; g2.sp = as;
            g2.Q = A; g2.ldq = g.mp; g2.sq = as;
            g2.C = B; g2.ldc = g.mp; g2.sc = as;
            g2.D = A; g2.ldd = g.mp; g2.sd = as;
            g2.tiles_m = tm; g2.tiles_n = tm; g2.tiles_per_item = tri; g2.n_items = nit;
            g2.k_tiles = (int32_t)(g.mp / kElemsPerKTile);
            g2.alpha = b; g2.beta = c;
            st = launch_gemm<T, kBM, kBN, kWM, kWN, EPI_POLY, true>(g2, tri * nit, stream);
            if (st != QM_OK) return st;
            // X = a X + B X   (Q operand = X^T)
            GemmArgs<T> g3 = ga;
            g3.P = B; g3.ldp = g.mp; g3.sp = as;
            g3.Q = XTc; g3.ldq = g.mp; g3.sq = xs;
            g3.C = X; g3.ldc = g.np; g3.sc = xs;
            g3.CT = XTn; g3.ldct = g.mp; g3.sct = xs;
            g3.D = X; g3.ldd = g.np; g3.sd = xs;
            g3.tiles_m = tm; g3.tiles_n = tn; g3.tiles_per_item = tm * tn; g3.n_items = nit;
            g3.k_tiles = (int32_t)(g.mp / kElemsPerKTile);
            g3.alpha = a;
            if (s + 1 < steps)
                st = launch_gemm<T, kBM, kBN, kWM, kWN, EPI_UPDATE, false>(g3, tm * tn * nit, stream);
            else
                st = launch_gemm<T, kBM, kBN, kWM, kWN, EPI_FINAL, false>(g3, tm * tn * nit, stream);
            if (st != QM_OK) return st;
            std::swap(XTc, XTn);
        }
    }
    return QM_OK;
}

qm_status run_ns(const std::vector<NsRequest> &req, int steps, float a, float b, float c, float eps,
                 int precision, void *ws, hipStream_t stream) {
    if (precision == QM_NS_F32) return run_ns_typed<float>(req, steps, a, b, c, eps, ws, stream);
    return run_ns_typed<bf16_t>(req, steps, a, b, c, eps, ws, stream);
}

qm_status check_ns_common(void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld, int32_t steps,
                          float a, float b, float c, float eps, int32_t precision) {
    if (!x) return fail(QM_E_ARG, "x is null");
    if (dtype != QM_F32 && dtype != QM_BF16 && dtype != QM_F16) return fail(QM_E_DTYPE, "unknown dtype %d", dtype);
    if (precision != QM_NS_BF16 && precision != QM_NS_F32) return fail(QM_E_ARG, "unknown precision %d", precision);
    if (rows <= 0 || cols <= 0) return fail(QM_E_SHAPE, "rows and cols must be positive");
    if (ld < cols) return fail(QM_E_SHAPE, "ld must be >= cols");
    if (std::min(rows, cols) > (1 << 20) || std::max(rows, cols) > (1 << 24))
        return fail(QM_E_UNSUPPORTED, "matrix too large");
    if (steps < 0 || steps > 100) return fail(QM_E_ARG, "steps must lie in [0, 100]");
    if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) return fail(QM_E_ARG, "coefficients must be finite");
    if (!(eps >= 0.0f) || std::isinf(eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    const uintptr_t esz = dtype == QM_F32 ? 4 : 2;
    if (!aligned(x, esz)) return fail(QM_E_ALIGN, "x misaligned for its dtype");
    return QM_OK;
}

}  // namespace
}  // namespace qm

using namespace qm;

extern "C" size_t ns_workspace_bytes(int64_t rows, int64_t cols, int32_t batch, int32_t precision) {
    if (rows <= 0 || cols <= 0 || batch <= 0) return 0;
    return ns_ws_bytes_for(rows, cols, batch, precision);
}

extern "C" qm_status ns_orthogonalize(void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                      int32_t batch, int64_t batch_stride, int32_t steps, float a, float b,
                                      float c, float eps, const float *inv_norm, int32_t precision, void *ws,
                                      size_t ws_bytes, qm_stream_t stream) {
    clear_error();
    qm_status st = check_ns_common(x, dtype, rows, cols, ld, steps, a, b, c, eps, precision);
    if (st != QM_OK) return st;
    if (batch <= 0) return fail(QM_E_ARG, "batch must be positive");
    if (batch > 1 && batch_stride < (rows - 1) * ld + cols)
        return fail(QM_E_SHAPE, "batch_stride makes matrices overlap");
    if (inv_norm && !aligned(inv_norm, 4)) return fail(QM_E_ALIGN, "inv_norm misaligned");
    const size_t need = ns_ws_bytes_for(rows, cols, batch, precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t esz = dtype == QM_F32 ? 4 : 2;
    std::vector<NsRequest> req;
    for (int32_t i = 0; i < batch; i++) {
        char *p = static_cast<char *>(x) + (size_t)i * (size_t)batch_stride * esz;
        req.push_back(NsRequest{p, p, rows, cols, ld, dtype, inv_norm ? inv_norm + i : nullptr, nullptr, 0,
                                0.0f, 0.0f});
    }
    return run_ns(req, steps, a, b, c, eps, precision, ws, static_cast<hipStream_t>(stream));
}

extern "C" size_t ns_blocked_workspace_bytes(int64_t rows, int64_t cols, int64_t block_rows, int64_t block_cols,
                                             int32_t precision) {
    if (rows <= 0 || cols <= 0 || block_rows <= 0 || block_cols <= 0) return 0;
    if (rows % block_rows || cols % block_cols) return 0;
    return ns_ws_bytes_for(block_rows, block_cols, (rows / block_rows) * (cols / block_cols), precision);
}

extern "C" qm_status ns_orthogonalize_blocked(void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                              int64_t block_rows, int64_t block_cols, int32_t steps, float a,
                                              float b, float c, float eps, const float *inv_norm,
                                              int32_t precision, void *ws, size_t ws_bytes, qm_stream_t stream) {
    clear_error();
    qm_status st = check_ns_common(x, dtype, rows, cols, ld, steps, a, b, c, eps, precision);
    if (st != QM_OK) return st;
    if (block_rows <= 0 || block_cols <= 0 || rows % block_rows || cols % block_cols)
        return fail(QM_E_SHAPE, "blocks must tile the matrix");
    if (inv_norm && !aligned(inv_norm, 4)) return fail(QM_E_ALIGN, "inv_norm misaligned");
    const int64_t nbr = rows / block_rows, nbc = cols / block_cols;
    const size_t need = ns_ws_bytes_for(block_rows, block_cols, nbr * nbc, precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t esz = dtype == QM_F32 ? 4 : 2;
    std::vector<NsRequest> req;
    for (int64_t bi = 0; bi < nbr; bi++)
        for (int64_t bj = 0; bj < nbc; bj++) {
            char *p = static_cast<char *>(x) + ((size_t)(bi * block_rows) * (size_t)ld + (size_t)(bj * block_cols)) * esz;
            const float *inv = inv_norm ? inv_norm + bi * nbc + bj : nullptr;
            req.push_back(NsRequest{p, p, block_rows, block_cols, ld, dtype, inv, nullptr, 0, 0.0f, 0.0f});
        }
    return run_ns(req, steps, a, b, c, eps, precision, ws, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- muon step

namespace qm {
namespace {

struct StepPlan {
    bool full;
    const PlanHeader *h;
    const void *dev;
};

// The NS work of one step, grouped by (m, n) so same-shaped matrices batch.
std::vector<std::vector<NsRequest>> step_requests(const PlanHeader *h, const void *host_plan,
                                                  const qm_muon_matrix *mats, int32_t n, bool full,
                                                  const float *inv, const qm_muon_hparams *hp) {
    const PlanTensor *pt = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(host_plan) + h->off_tensors);
    std::vector<std::vector<NsRequest>> groups;
    std::vector<std::pair<int64_t, int64_t>> keys;
    int64_t g0 = 0;
    for (int32_t i = 0; i < n; i++) {
        const qm_muon_matrix &M = mats[i];
        const int64_t br = full ? M.rows : M.block_rows, bc = full ? M.cols : M.block_cols;
        const int64_t nbr = M.rows / br, nbc = M.cols / bc;
        const float lr = full ? hp->lr_full : hp->lr_block;
        const float s = hp->rms_scale * sqrtf((float)std::max(br, bc));
        const int32_t dt = pt[i].dtype;
        const size_t esz = dt == QM_F32 ? 4 : 2;
        char *grad = reinterpret_cast<char *>(pt[i].grad);
        for (int64_t bi = 0; bi < nbr; bi++)
            for (int64_t bj = 0; bj < nbc; bj++) {
                const size_t off = (size_t)(bi * br) * (size_t)M.cols + (size_t)(bj * bc);
                const float *ip = inv ? inv + g0 + bi * nbc + bj : nullptr;
                NsRequest r{grad + off * esz, grad + off * esz, br, bc, M.cols, dt, ip,
                            M.weight ? M.weight + off : nullptr, M.cols, lr * s, lr * hp->weight_decay};
                const std::pair<int64_t, int64_t> key{std::min(br, bc), std::max(br, bc)};
                size_t k = 0;
                while (k < keys.size() && keys[k] != key) k++;
                if (k == keys.size()) {
                    keys.push_back(key);
                    groups.emplace_back();
                }
                groups[k].push_back(r);
            }
        g0 += nbr * nbc;
    }
    return groups;
}

qm_status check_step_plan(const void *host_plan, const qm_muon_matrix *mats, int32_t n, bool full,
                          const PlanHeader **out) {
    qm_status st;
    const PlanHeader *h = plan_header(host_plan, &st);
    if (!h) return st;
    if (h->n_tensors != n) return fail(QM_E_SHAPE, "plan has %d tensors, %d matrices given", h->n_tensors, n);
    const PlanTensor *pt = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(host_plan) + h->off_tensors);
    int64_t g0 = 0;
    for (int32_t i = 0; i < n; i++) {
        const qm_muon_matrix &M = mats[i];
        if (M.rows <= 0 || M.cols <= 0) return fail(QM_E_SHAPE, "matrix %d: empty", i);
        if (pt[i].numel != M.rows * M.cols) return fail(QM_E_SHAPE, "matrix %d: size differs from plan tensor", i);
        const int64_t br = full ? M.rows : M.block_rows, bc = full ? M.cols : M.block_cols;
        if (br <= 0 || bc <= 0 || M.rows % br || M.cols % bc)
            return fail(QM_E_SHAPE, "matrix %d: blocks do not tile it", i);
        const int64_t nb = (M.rows / br) * (M.cols / bc);
        if (pt[i].group_lo != g0 || pt[i].group_hi != g0 + nb - 1)
            return fail(QM_E_PLAN, "matrix %d: plan groups %d..%d, expected %lld..%lld", i, pt[i].group_lo,
                        pt[i].group_hi, (long long)g0, (long long)(g0 + nb - 1));
        if (M.weight && !aligned(M.weight, 4)) return fail(QM_E_ALIGN, "matrix %d: weight misaligned", i);
        g0 += nb;
    }
    if (h->n_groups != g0) return fail(QM_E_PLAN, "plan has %d groups, expected %lld", h->n_groups, (long long)g0);
    *out = h;
    return QM_OK;
}

size_t step_ws_bytes(const PlanHeader *h, const void *host_plan, const qm_muon_matrix *mats, int32_t n,
                     bool full, int precision) {
    qm_muon_hparams dummy{};
    const auto groups = step_requests(h, host_plan, mats, n, full, nullptr, &dummy);
    size_t ns = 0;
    for (const auto &g : groups) ns = std::max(ns, ns_ws_bytes_for(g[0].rows, g[0].cols, (int64_t)g.size(), precision));
    return align_up(qm_update_workspace_bytes(host_plan), 256) + ns;
}

}  // namespace
}  // namespace qm

extern "C" size_t muon_step_workspace_bytes(const void *host_plan_full, const void *host_plan_block,
                                            const qm_muon_matrix *mats, int32_t n_mats, int32_t precision) {
    if (!mats || n_mats <= 0) return 0;
    const PlanHeader *h = nullptr;
    size_t need = 0;
    if (check_step_plan(host_plan_full, mats, n_mats, true, &h) != QM_OK) return 0;
    need = step_ws_bytes(h, host_plan_full, mats, n_mats, true, precision);
    if (host_plan_block) {
        if (check_step_plan(host_plan_block, mats, n_mats, false, &h) != QM_OK) return 0;
        need = std::max(need, step_ws_bytes(h, host_plan_block, mats, n_mats, false, precision));
    }
    return need;
}

namespace qm {
namespace {

qm_status check_hparams(const qm_muon_hparams *hp) {
    if (!hp) return fail(QM_E_ARG, "hparams is null");
    if (hp->precision != QM_NS_BF16 && hp->precision != QM_NS_F32) return fail(QM_E_ARG, "unknown precision");
    if (hp->ns_steps < 0 || hp->ns_steps > 100) return fail(QM_E_ARG, "ns_steps must lie in [0, 100]");
    if (!std::isfinite(hp->lr_full) || !std::isfinite(hp->lr_block) || !std::isfinite(hp->weight_decay) ||
        !std::isfinite(hp->rms_scale) || !std::isfinite(hp->a) || !std::isfinite(hp->b) || !std::isfinite(hp->c))
        return fail(QM_E_ARG, "hyperparameters must be finite");
    if (!(hp->eps >= 0.0f) || std::isinf(hp->eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    return QM_OK;
}

// NS + weight apply of every matrix (full) or block, NS workspace at ns_ws.
qm_status apply_phase(const PlanHeader *h, const void *host_plan, const qm_muon_matrix *mats, int32_t n,
                      bool full, const float *inv, const qm_muon_hparams *hp, void *ns_ws, hipStream_t s) {
    const auto groups = step_requests(h, host_plan, mats, n, full, inv, hp);
    for (const auto &g : groups) {
        const qm_status st = run_ns(g, hp->ns_steps, hp->a, hp->b, hp->c, hp->eps, hp->precision, ns_ws, s);
        if (st != QM_OK) return st;
    }
    return QM_OK;
}

}  // namespace
}  // namespace qm

extern "C" qm_status muon_apply(const void *host_plan, const qm_muon_matrix *mats, int32_t n_mats, int32_t full,
                                const float *inv_norm, const qm_muon_hparams *hp, void *ws, size_t ws_bytes,
                                qm_stream_t stream) {
    clear_error();
    qm_status st = check_hparams(hp);
    if (st != QM_OK) return st;
    if (!mats || n_mats <= 0) return fail(QM_E_ARG, "no matrices");
    if (full != 0 && full != 1) return fail(QM_E_ARG, "full must be 0 or 1");
    if (!inv_norm || !aligned(inv_norm, 4)) return fail(QM_E_ARG, "inv_norm must be a 4-byte aligned device pointer");
    const PlanHeader *h = nullptr;
    st = check_step_plan(host_plan, mats, n_mats, full != 0, &h);
    if (st != QM_OK) return st;
    const size_t need = step_ws_bytes(h, host_plan, mats, n_mats, full != 0, hp->precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t upd = align_up(qm_update_workspace_bytes(host_plan), 256);
    return apply_phase(h, host_plan, mats, n_mats, full != 0, inv_norm, hp, static_cast<char *>(ws) + upd,
                       static_cast<hipStream_t>(stream));
}

extern "C" qm_status muon_step(const void *host_plan_full, const void *dev_plan_full, const void *host_plan_block,
                               const void *dev_plan_block, const qm_muon_matrix *mats, int32_t n_mats,
                               int64_t step, const qm_muon_hparams *hp, void *ws, size_t ws_bytes,
                               qm_stream_t stream) {
    clear_error();
    qm_status st = check_hparams(hp);
    if (st != QM_OK) return st;
    if (!mats || n_mats <= 0) return fail(QM_E_ARG, "no matrices");
    if (step < 1) return fail(QM_E_ARG, "step is 1-based");
    const bool full = hp->period <= 1 || host_plan_block == nullptr || (step % hp->period) == 0;
    const void *hplan = full ? host_plan_full : host_plan_block;
    const void *dplan = full ? dev_plan_full : dev_plan_block;
    const PlanHeader *h = nullptr;
    st = validate_update(hplan, dplan, hp->beta, &h);
    if (st != QM_OK) return st;
    st = check_step_plan(hplan, mats, n_mats, full, &h);
    if (st != QM_OK) return st;
    if (full && host_plan_block) {
        const PlanHeader *hb = nullptr;
        st = check_step_plan(host_plan_block, mats, n_mats, false, &hb);
        if (st != QM_OK) return st;
    }
    const size_t need = muon_step_workspace_bytes(host_plan_full, host_plan_block, mats, n_mats, hp->precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t upd = align_up(qm_update_workspace_bytes(hplan), 256);
    const UpdateWorkspace uw = update_workspace(h, ws);
    st = run_update_normalize(h, dplan, hp->beta, hp->eps, false, nullptr, nullptr, ws, s);
    if (st != QM_OK) return st;
    return apply_phase(h, hplan, mats, n_mats, full, uw.inv, hp, static_cast<char *>(ws) + upd, s);
}
