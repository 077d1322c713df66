// GRASP 4-bit momentum step for gfx950 ("4-bit-Muon-GRASP"): the momentum
// of an m x n matrix is held as a rank-k factor P R^T (8-bit) plus a residual
// (4-bit), both grid-quantised over 64 x 64 blocks (entry / min(row max,
// column max) inside its block).  One step:
//   reconstruct M_{t-1}, M_t = mu M_{t-1} + g            (grasp_momentum)
//   Q = ColNorm(R_{t-1}) (zero columns: seeded warm start) (grasp_colnorm)
//   P = MGS(M_t Q), R = M_t^T P                           (momentum, mgs, rt)
//   requantise M_t - P R^T (4-bit), P and R (8-bit)       (residual_q4, factor_q8)
//   O = NS(M_t) in f32 arithmetic, W <- W - lr (O + wd W) (the NS kernels)
//
// Compiled with -ffp-contract=off: fp32 products and sums stay separately
// rounded, so the codes equal a CPU run of the same operations given the same
// fp32 P and R.  Long reductions (M Q, M^T P, norms) accumulate in fp64 in a
// fixed order (no atomics).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <vector>

#include "grasp_internal.h"
#include "internal.h"
#include "plan_layout.h"
#include "qmuon.h"

namespace qm {
namespace {

constexpr int kGrid = 64;
constexpr int kThreads = 256;

struct Dims {
    int64_t rows, cols;
    int32_t rank;
    int64_t nbr, nbc;       // 64-blocks along rows / cols
    int64_t packed_cols;    // bytes per residual row
};

__device__ __forceinline__ float load_grad(const void *p, int64_t i, int dtype) {
    if (dtype == QM_F32) return static_cast<const float *>(p)[i];
    const uint16_t h = static_cast<const uint16_t *>(p)[i];
    if (dtype == QM_BF16) return __uint_as_float((uint32_t)h << 16);
    return (float)__builtin_bit_cast(_Float16, h);
}

// Deterministic workgroup sum of one fp64 value per thread (fixed order).
__device__ __forceinline__ double block_sum(double v, double *scratch) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    const double s = ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
    __syncthreads();
    return s;
}

// --------------------------------------------------- dequantised factors
// P (rows x k) and R (cols x k): one 64-row block of either per k columns;
// divisor min(row max, column max), value code * (d / 127).
__global__ __launch_bounds__(kThreads) void deq_factors_kernel(const int8_t *pc, const float *prm, const float *pcm,
                                                               const int8_t *rc, const float *rrm, const float *rcm,
                                                               Dims d, float *Pd, float *Rd) {
    const int64_t n_p = d.rows * d.rank, n_all = n_p + d.cols * d.rank;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n_all; e += (int64_t)gridDim.x * kThreads) {
        const bool isp = e < n_p;
        const int64_t f = isp ? e : e - n_p;
        const int64_t i = f / d.rank;
        const int c = (int)(f % d.rank);
        const float rmax = isp ? prm[i] : rrm[i];
        const float cmax = isp ? pcm[(i / kGrid) * d.rank + c] : rcm[(i / kGrid) * d.rank + c];
        const float dv = fminf(rmax, cmax);
        const float step = dv / 127.0f;
        const float v = (float)(isp ? pc[f] : rc[f]) * step;
        if (isp) Pd[f] = v;
        else Rd[f] = v;
    }
}

// ------------------------------------------------------------ ColNorm
__global__ __launch_bounds__(kThreads) void colnorm_kernel(const float *Rd, const float *warm, Dims d, double *Q) {
    // every column's sum of squares in one pass over Rd (per column: thread
    // t adds rows t, t + 256, ... in order, then the block sum's fixed order)
    __shared__ double part[4][16];
    __shared__ double nrm[16], wnrm[16];
    const int K = d.rank;
    double s[16];
#pragma unroll
    for (int c = 0; c < 16; c++) s[c] = 0.0;
    for (int64_t j = threadIdx.x; j < d.cols; j += kThreads)
#pragma unroll
        for (int c = 0; c < 16; c++)
            if (c < K) {
                const double v = (double)Rd[j * K + c];
                s[c] += v * v;
            }
#pragma unroll
    for (int c = 0; c < 16; c++) {
        double v = s[c];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][c] = v;
    }
    __syncthreads();
    if (threadIdx.x < K) nrm[threadIdx.x] = sqrt(((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                                                part[3][threadIdx.x]);
    __syncthreads();
    bool any_zero = false;
    for (int c = 0; c < K; c++) any_zero |= !(nrm[c] > 0.0);
    if (any_zero) {   // warm-start columns: their norms, same order
#pragma unroll
        for (int c = 0; c < 16; c++) s[c] = 0.0;
        for (int64_t j = threadIdx.x; j < d.cols; j += kThreads)
#pragma unroll
            for (int c = 0; c < 16; c++)
                if (c < K) {
                    const double v = (double)warm[j * K + c];
                    s[c] += v * v;
                }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; c++) {
            double v = s[c];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][c] = v;
        }
        __syncthreads();
        if (threadIdx.x < K)
            wnrm[threadIdx.x] = sqrt(((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                                     part[3][threadIdx.x]);
        __syncthreads();
    }
    for (int64_t j = threadIdx.x; j < d.cols; j += kThreads)
        for (int c = 0; c < K; c++)
            Q[j * K + c] = nrm[c] > 0.0 ? (double)Rd[j * K + c] / nrm[c] : (double)warm[j * K + c] / wnrm[c];
}

// ------------------------------------------------- momentum and Y = M Q
// kMomRows rows per workgroup, lane t walks columns t, t+256, ...:
//   M_prev = (float)(res + sum_c Pd[i][c] Rd[j][c])  (fp64, c in order)
//   M = fl(fl(mu * M_prev) + g);   Y[i][c] = sum_j M[i][j] Q[j][c] (fp64)
// Column j's factor rows Rd[j] and Q[j] are loaded once for the rows, and
// the rows' elements are computed as independent straight-line
// code, so their loads are in flight together (rows past the matrix's end
// recompute row i0 and are dropped).  Each row's sums still run over j in
// the same order.
constexpr int kMomRows = 2;

template <int K>
__global__ __launch_bounds__(kThreads) void momentum_kernel(const uint8_t *res_codes, const float *res_rmax,
                                                            const float *res_cmax, const float *Pd, const float *Rd,
                                                            const double *Q, const void *g, int gdt, float mu, Dims d,
                                                            float *M, double *Y) {
    __shared__ double part[4][kMomRows * K];
    const int64_t i0 = (int64_t)blockIdx.x * kMomRows;
    const int nr = (int)min((int64_t)kMomRows, d.rows - i0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double y[kMomRows][K];
#pragma unroll
    for (int r = 0; r < kMomRows; r++)
#pragma unroll
        for (int c = 0; c < K; c++) y[r][c] = 0.0;
    float p[kMomRows][K];
#pragma unroll
    for (int r = 0; r < kMomRows; r++)
#pragma unroll
        for (int c = 0; c < K; c++) p[r][c] = Pd[(i0 + (r < nr ? r : 0)) * K + c];
    for (int64_t j = threadIdx.x; j < d.cols; j += kThreads) {
        // 16-byte loads of the factor rows (lanes hold consecutive rows)
        float rd[K];
        double qj[K];
        if constexpr (K % 4 == 0) {
#pragma unroll
            for (int c = 0; c < K; c += 4) *reinterpret_cast<float4 *>(rd + c) = *reinterpret_cast<const float4 *>(Rd + j * K + c);
        } else {
#pragma unroll
            for (int c = 0; c < K; c++) rd[c] = Rd[j * K + c];
        }
        if constexpr (K % 2 == 0) {
#pragma unroll
            for (int c = 0; c < K; c += 2) *reinterpret_cast<double2 *>(qj + c) = *reinterpret_cast<const double2 *>(Q + j * K + c);
        } else {
#pragma unroll
            for (int c = 0; c < K; c++) qj[c] = Q[j * K + c];
        }
        float m[kMomRows];
#pragma unroll
        for (int r = 0; r < kMomRows; r++) {
            const int64_t i = i0 + (r < nr ? r : 0);
            const uint8_t byte = res_codes[i * d.packed_cols + (j >> 1)];
            const int nib = (j & 1) ? (byte >> 4) : (byte & 0xF);
            const int code = nib >= 8 ? nib - 16 : nib;
            const float dv = fminf(res_rmax[i * d.nbc + j / kGrid], res_cmax[(i / kGrid) * d.cols + j]);
            const float step = dv / 7.0f;
            const float resd = (float)code * step;
            double acc = (double)resd;
#pragma unroll
            for (int c = 0; c < K; c++) acc = acc + (double)p[r][c] * (double)rd[c];
            const float mprev = (float)acc;
            const float t1 = mu * mprev;
            m[r] = t1 + load_grad(g, i * d.cols + j, gdt);
        }
#pragma unroll
        for (int r = 0; r < kMomRows; r++) {
            if (r < nr) {
                M[(i0 + r) * d.cols + j] = m[r];
#pragma unroll
                for (int c = 0; c < K; c++) y[r][c] += (double)m[r] * qj[c];
            }
        }
    }
    // fixed-order reduction: butterfly inside each wave, then waves 0..3
#pragma unroll
    for (int r = 0; r < kMomRows; r++)
#pragma unroll
        for (int c = 0; c < K; c++) {
            double v = y[r][c];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if (lane == 0) part[wave][r * K + c] = v;
        }
    __syncthreads();
    if (threadIdx.x < kMomRows * K) {
        const int r = threadIdx.x / K, c = threadIdx.x % K;
        if (i0 + r < d.rows)
            Y[(i0 + r) * K + c] = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                                  part[3][threadIdx.x];
    }
}

// ------------------------------------------------------------ MGS
// One workgroup of 1024 threads: P = Y column by column, each earlier column
// projected out with the current remainder (modified Gram-Schmidt), then
// normalised.  The columns are worked on in a column-major copy Pc (rows x k
// as k rows of `rows`), so every pass reads consecutive addresses; thread t
// takes rows t, t + 1024, ... and the 16 waves' partial sums are added in
// wave order.
constexpr int kMgsThreads = 1024;

__device__ __forceinline__ double block_sum_1024(double v, double *scratch) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = scratch[0];
#pragma unroll
    for (int w = 1; w < kMgsThreads / 64; w++) s += scratch[w];
    __syncthreads();
    return s;
}

__global__ __launch_bounds__(kMgsThreads) void mgs_kernel(const double *Y, Dims d, double *Pc, double *P, float *P32) {
    __shared__ double scratch[kMgsThreads / 64];
    const int K = d.rank;
    const int64_t n = d.rows;
    for (int64_t e = threadIdx.x; e < n * K; e += kMgsThreads) Pc[(e % K) * n + e / K] = Y[e];
    __syncthreads();
    for (int c = 0; c < K; c++) {
        double *pc = Pc + c * n;
        for (int p = 0; p < c; p++) {
            const double *pp = Pc + p * n;
            double s = 0.0;
            for (int64_t i = threadIdx.x; i < n; i += kMgsThreads) s += pp[i] * pc[i];
            const double dot = block_sum_1024(s, scratch);
            for (int64_t i = threadIdx.x; i < n; i += kMgsThreads) {
                const double t = dot * pp[i];
                pc[i] = pc[i] - t;
            }
            __syncthreads();
        }
        double s = 0.0;
        for (int64_t i = threadIdx.x; i < n; i += kMgsThreads) s += pc[i] * pc[i];
        const double nrm = sqrt(block_sum_1024(s, scratch));
        for (int64_t i = threadIdx.x; i < n; i += kMgsThreads) pc[i] = nrm > 0.0 ? pc[i] / nrm : 0.0;
        __syncthreads();
    }
    for (int64_t e = threadIdx.x; e < n * K; e += kMgsThreads) {
        const double v = Pc[(e % K) * n + e / K];
        P[e] = v;
        P32[e] = (float)v;
    }
}

// The same computation with the columns in registers, for rows <= 4 * 1024
// and k <= 8: thread t holds rows t + 1024 r (r < 4) of every column, so a
// pass is thread-local arithmetic plus one workgroup sum (the operations
// and their order are those of mgs_kernel).
template <int K>
__global__ __launch_bounds__(kMgsThreads) void mgs_reg_kernel(const double *Y, Dims d, double *P, float *P32) {
    constexpr int R = 4;
    __shared__ double scratch[kMgsThreads / 64];
    const int64_t n = d.rows;
    double v[R][K];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int64_t i = threadIdx.x + (int64_t)r * kMgsThreads;
#pragma unroll
        for (int c = 0; c < K; c++) v[r][c] = i < n ? Y[i * K + c] : 0.0;
    }
#pragma unroll
    for (int c = 0; c < K; c++) {
#pragma unroll
        for (int p = 0; p < c; p++) {
            double s = 0.0;
#pragma unroll
            for (int r = 0; r < R; r++)
                if (threadIdx.x + (int64_t)r * kMgsThreads < n) s += v[r][p] * v[r][c];
            const double dot = block_sum_1024(s, scratch);
#pragma unroll
            for (int r = 0; r < R; r++) {
                const double t = dot * v[r][p];
                v[r][c] = v[r][c] - t;
            }
        }
        double s = 0.0;
#pragma unroll
        for (int r = 0; r < R; r++)
            if (threadIdx.x + (int64_t)r * kMgsThreads < n) s += v[r][c] * v[r][c];
        const double nrm = sqrt(block_sum_1024(s, scratch));
#pragma unroll
        for (int r = 0; r < R; r++) v[r][c] = nrm > 0.0 ? v[r][c] / nrm : 0.0;
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int64_t i = threadIdx.x + (int64_t)r * kMgsThreads;
        if (i < n)
#pragma unroll
            for (int c = 0; c < K; c++) {
                P[i * K + c] = v[r][c];
                P32[i * K + c] = (float)v[r][c];
            }
    }
}

// ------------------------------------------------------------ R = M^T P
// Workgroup (bx, by) covers columns 64 bx .. 64 bx + 63 and rows
// kRtRows by .. kRtRows (by + 1) - 1: lane (c, g) = (t % 64, t / 64) sums rows
// g, g+4, ... of the chunk (fp64), the four row groups are added in order,
// and the chunk's partial goes to Rpart[by].  rt_combine adds the chunks in
// order and rounds to fp32.
constexpr int kRtRows = 128;

template <int K>
__global__ __launch_bounds__(kThreads) void rt_partial_kernel(const float *M, const double *P, Dims d,
                                                              double *Rpart) {
    __shared__ double part[4][64 * K];
    const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + c;
    const int64_t i0 = (int64_t)blockIdx.y * kRtRows;
    const int64_t i1 = min(d.rows, i0 + kRtRows);
    double acc[K];
#pragma unroll
    for (int k = 0; k < K; k++) acc[k] = 0.0;
    if (j < d.cols)
        for (int64_t i = i0 + grp; i < i1; i += 4) {
            const double m = (double)M[i * d.cols + j];
#pragma unroll
            for (int k = 0; k < K; k++) acc[k] += m * P[i * K + k];
        }
#pragma unroll
    for (int k = 0; k < K; k++) part[grp][c * K + k] = acc[k];
    __syncthreads();
    double *out = Rpart + (int64_t)blockIdx.y * d.cols * K;
    for (int e = threadIdx.x; e < 64 * K; e += kThreads) {
        const int64_t jj = (int64_t)blockIdx.x * 64 + e / K;
        if (jj < d.cols) out[jj * K + e % K] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
    }
}

__global__ __launch_bounds__(kThreads) void rt_combine_kernel(const double *Rpart, int64_t chunks, Dims d,
                                                              float *R32) {
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t n = d.cols * d.rank;
    if (e >= n) return;
    double s = 0.0;
    for (int64_t ch = 0; ch < chunks; ch++) s += Rpart[ch * n + e];
    R32[e] = (float)s;
}

// ------------------------------------------------ residual, 4-bit codes
// One 64x64 block (clipped) per workgroup:
//   res = (float)(M - sum_c P32[i][c] R32[j][c])   (fp64, c in order)
//   row / column maxima of |res| inside the block; code = d == 0 ? 0 :
//   clamp(rint((res / d) * 7), -7, 7), two codes per byte (even column low).
template <int K>
__global__ __launch_bounds__(kThreads) void residual_q4_kernel(const float *M, const float *P32, const float *R32,
                                                               Dims d, uint8_t *codes, float *rmax_out,
                                                               float *cmax_out) {
    __shared__ float tile[64][65];
    __shared__ float rm[64], cm[64];
    __shared__ float ps[64][K], rs[64][K];   // the block's rows of P32 and of R32
    const int64_t bi = blockIdx.y, bj = blockIdx.x;
    const int64_t r0 = bi * 64, c0 = bj * 64;
    const int br = (int)min<int64_t>(64, d.rows - r0), bc = (int)min<int64_t>(64, d.cols - c0);
    for (int e = threadIdx.x; e < 64 * K; e += kThreads) {
        const int r = e / K, c = e % K;
        ps[r][c] = r < br ? P32[(r0 + r) * K + c] : 0.0f;
        rs[r][c] = r < bc ? R32[(c0 + r) * K + c] : 0.0f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 4096; idx += kThreads) {
        const int ii = idx >> 6, jj = idx & 63;
        float v = 0.0f;
        if (ii < br && jj < bc) {
            const int64_t i = r0 + ii, j = c0 + jj;
            double acc = (double)M[i * d.cols + j];
#pragma unroll
            for (int c = 0; c < K; c++) acc = acc - (double)ps[ii][c] * (double)rs[jj][c];
            v = (float)acc;
        }
        tile[ii][jj] = v;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        float m = 0.0f;
        for (int jj = 0; jj < bc; jj++) m = fmaxf(m, fabsf(tile[threadIdx.x][jj]));
        rm[threadIdx.x] = m;
        if (threadIdx.x < br) rmax_out[(r0 + threadIdx.x) * d.nbc + bj] = m;
    } else if (threadIdx.x < 128) {
        const int jj = threadIdx.x - 64;
        float m = 0.0f;
        for (int ii = 0; ii < br; ii++) m = fmaxf(m, fabsf(tile[ii][jj]));
        cm[jj] = m;
        if (jj < bc) cmax_out[bi * d.cols + c0 + jj] = m;
    }
    __syncthreads();
    for (int pidx = threadIdx.x; pidx < 64 * 32; pidx += kThreads) {
        const int ii = pidx >> 5, jp = pidx & 31;
        if (ii >= br || 2 * jp >= bc) continue;
        int q[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int jj = 2 * jp + h;
            if (jj >= bc) break;
            const float dv = fminf(rm[ii], cm[jj]);
            if (dv != 0.0f) {
                float r = rintf((tile[ii][jj] / dv) * 7.0f);
                r = fminf(fmaxf(r, -7.0f), 7.0f);
                q[h] = (int)r;
            }
        }
        codes[(r0 + ii) * d.packed_cols + bj * 32 + jp] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
    }
}

// ------------------------------------------------ factors, 8-bit codes
// P32 (rows x k) or R32 (cols x k): one 64-row block per workgroup; the k
// columns form one clipped grid block.
__global__ __launch_bounds__(kThreads) void factor_q8_kernel(const float *X, int64_t n, int K, int8_t *codes,
                                                             float *rmax_out, float *cmax_out) {
    __shared__ float rm[64], cm[64];
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int br = (int)min<int64_t>(64, n - r0);
    if (threadIdx.x < 64) {
        float m = 0.0f;
        if (threadIdx.x < br)
            for (int c = 0; c < K; c++) m = fmaxf(m, fabsf(X[(r0 + threadIdx.x) * K + c]));
        rm[threadIdx.x] = m;
        if (threadIdx.x < br) rmax_out[r0 + threadIdx.x] = m;
    } else if (threadIdx.x < 64 + K) {
        const int c = threadIdx.x - 64;
        float m = 0.0f;
        for (int ii = 0; ii < br; ii++) m = fmaxf(m, fabsf(X[(r0 + ii) * K + c]));
        cm[c] = m;
        cmax_out[blockIdx.x * K + c] = m;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < br * K; e += kThreads) {
        const int ii = e / K, c = e % K;
        const float dv = fminf(rm[ii], cm[c]);
        int q = 0;
        if (dv != 0.0f) {
            float r = rintf((X[(r0 + ii) * K + c] / dv) * 127.0f);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            q = (int)r;
        }
        codes[(r0 + ii) * K + c] = (int8_t)q;
    }
}

struct Ws {
    float *M, *Pd, *Rd, *P32, *R32;
    double *Q, *Y, *P, *Pc, *Rpart;
    int64_t rt_chunks;
    void *ns;
    size_t bytes;
};

Ws carve(const Dims &d, void *base) {
    Ws w{};
    char *p = static_cast<char *>(base);
    auto take = [&](int64_t bytes) {
        char *q = p;
        p += align_up(bytes, 256);
        return q;
    };
    const int64_t rk = d.rows * d.rank, ck = d.cols * d.rank;
    w.M = reinterpret_cast<float *>(take(d.rows * d.cols * 4));
    w.Pd = reinterpret_cast<float *>(take(rk * 4));
    w.Rd = reinterpret_cast<float *>(take(ck * 4));
    w.P32 = reinterpret_cast<float *>(take(rk * 4));
    w.R32 = reinterpret_cast<float *>(take(ck * 4));
    w.Q = reinterpret_cast<double *>(take(ck * 8));
    w.Y = reinterpret_cast<double *>(take(rk * 8));
    w.P = reinterpret_cast<double *>(take(rk * 8));
    w.Pc = reinterpret_cast<double *>(take(rk * 8));
    w.rt_chunks = (d.rows + kRtRows - 1) / kRtRows;
    w.Rpart = reinterpret_cast<double *>(take(w.rt_chunks * ck * 8));
    w.ns = p;
    w.bytes = (size_t)(p - static_cast<char *>(base));
    return w;
}

Dims dims(int64_t rows, int64_t cols, int32_t rank) {
    Dims d;
    d.rows = rows;
    d.cols = cols;
    d.rank = rank;
    d.nbr = (rows + kGrid - 1) / kGrid;
    d.nbc = (cols + kGrid - 1) / kGrid;
    d.packed_cols = (cols + 1) / 2;
    return d;
}

qm_status launched(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return QM_OK;
}

template <int K>
void launch_rank_kernels(const qm_grasp_state *s, const Dims &d, const Ws &w, const void *grad, int gdt, float mu,
                         hipStream_t st) {
    momentum_kernel<K><<<(unsigned)((d.rows + kMomRows - 1) / kMomRows), kThreads, 0, st>>>(
        s->res_codes, s->res_rmax, s->res_cmax, w.Pd, w.Rd, w.Q, grad, gdt, mu, d, w.M, w.Y);
}

template <int K>
void launch_rt_residual(const qm_grasp_state *s, const Dims &d, const Ws &w, hipStream_t st) {
    rt_partial_kernel<K><<<dim3((unsigned)((d.cols + 63) / 64), (unsigned)w.rt_chunks), kThreads, 0, st>>>(
        w.M, w.P, d, w.Rpart);
    rt_combine_kernel<<<(unsigned)((d.cols * K + kThreads - 1) / kThreads), kThreads, 0, st>>>(w.Rpart, w.rt_chunks,
                                                                                              d, w.R32);
    residual_q4_kernel<K><<<dim3((unsigned)d.nbc, (unsigned)d.nbr), kThreads, 0, st>>>(
        w.M, w.P32, w.R32, d, s->res_codes, s->res_rmax, s->res_cmax);
}

}  // namespace
}  // namespace qm

using namespace qm;

extern "C" size_t grasp_workspace_bytes(int64_t rows, int64_t cols, int32_t rank) {
    if (rows <= 0 || cols <= 0 || rank <= 0 || rank > 16) return 0;
    const Dims d = dims(rows, cols, rank);
    const Ws w = carve(d, nullptr);
    return w.bytes + ns_f32_workspace_bytes(rows, cols);
}

extern "C" qm_status grasp_step(const qm_grasp_state *state, int64_t rows, int64_t cols, int32_t rank,
                                int32_t grid, void *grad, int32_t grad_dtype, const float *warm, float mu,
                                int32_t ns_steps, float a, float b, float c, float eps, int32_t ns_precision,
                                float *weight, float lr, float weight_decay, void *ws, size_t ws_bytes,
                                qm_stream_t stream) {
    clear_error();
    if (!state || !grad || !warm) return fail(QM_E_ARG, "state, grad and warm are required");
    if (!state->res_codes || !state->res_rmax || !state->res_cmax || !state->p_codes || !state->p_rmax ||
        !state->p_cmax || !state->r_codes || !state->r_rmax || !state->r_cmax)
        return fail(QM_E_ARG, "state buffer missing");
    if (rows <= 0 || cols <= 0) return fail(QM_E_SHAPE, "rows and cols must be positive");
    if (rank < 1 || rank > 16 || (rank & (rank - 1)))
        return fail(QM_E_UNSUPPORTED, "rank must be 1, 2, 4, 8 or 16");
    if (grid != kGrid) return fail(QM_E_UNSUPPORTED, "grid blocks must be 64x64");
    if (grad_dtype != QM_F32 && grad_dtype != QM_BF16 && grad_dtype != QM_F16)
        return fail(QM_E_DTYPE, "unknown grad dtype %d", grad_dtype);
    if (!aligned(grad, grad_dtype == QM_F32 ? 4 : 2) || !aligned(warm, 4) || (weight && !aligned(weight, 4)))
        return fail(QM_E_ALIGN, "misaligned pointer");
    if (!std::isfinite(mu) || !std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(a) ||
        !std::isfinite(b) || !std::isfinite(c) || !(eps >= 0.0f) || std::isinf(eps))
        return fail(QM_E_ARG, "hyperparameters must be finite (eps >= 0)");
    if (ns_steps < 0 || ns_steps > 100) return fail(QM_E_ARG, "ns_steps must lie in [0, 100]");
    if (ns_precision != QM_NS_F32 && ns_precision != QM_NS_BF16X3)
        return fail(QM_E_ARG, "ns_precision must be QM_NS_F32 or QM_NS_BF16X3");
    if (std::min(rows, cols) > (1 << 16) || std::max(rows, cols) > (1 << 22))
        return fail(QM_E_UNSUPPORTED, "matrix too large");
    const size_t need = grasp_workspace_bytes(rows, cols, rank);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");

    hipStream_t st = static_cast<hipStream_t>(stream);
    const Dims d = dims(rows, cols, rank);
    const Ws w = carve(d, ws);
    const qm_grasp_state *s = state;
    deq_factors_kernel<<<256, kThreads, 0, st>>>(s->p_codes, s->p_rmax, s->p_cmax, s->r_codes, s->r_rmax, s->r_cmax, d,
                                                 w.Pd, w.Rd);
    colnorm_kernel<<<1, kThreads, 0, st>>>(w.Rd, warm, d, w.Q);
    switch (rank) {
        case 1: launch_rank_kernels<1>(s, d, w, grad, grad_dtype, mu, st); break;
        case 2: launch_rank_kernels<2>(s, d, w, grad, grad_dtype, mu, st); break;
        case 4: launch_rank_kernels<4>(s, d, w, grad, grad_dtype, mu, st); break;
        case 8: launch_rank_kernels<8>(s, d, w, grad, grad_dtype, mu, st); break;
        default: launch_rank_kernels<16>(s, d, w, grad, grad_dtype, mu, st); break;
    }
    if (rows <= 4 * kMgsThreads && rank <= 8) {
        switch (rank) {
            case 1: mgs_reg_kernel<1><<<1, kMgsThreads, 0, st>>>(w.Y, d, w.P, w.P32); break;
            case 2: mgs_reg_kernel<2><<<1, kMgsThreads, 0, st>>>(w.Y, d, w.P, w.P32); break;
            case 4: mgs_reg_kernel<4><<<1, kMgsThreads, 0, st>>>(w.Y, d, w.P, w.P32); break;
            default: mgs_reg_kernel<8><<<1, kMgsThreads, 0, st>>>(w.Y, d, w.P, w.P32); break;
        }
    } else {
        mgs_kernel<<<1, kMgsThreads, 0, st>>>(w.Y, d, w.Pc, w.P, w.P32);
    }
    switch (rank) {
        case 1: launch_rt_residual<1>(s, d, w, st); break;
        case 2: launch_rt_residual<2>(s, d, w, st); break;
        case 4: launch_rt_residual<4>(s, d, w, st); break;
        case 8: launch_rt_residual<8>(s, d, w, st); break;
        default: launch_rt_residual<16>(s, d, w, st); break;
    }
    factor_q8_kernel<<<(unsigned)d.nbr, kThreads, 0, st>>>(w.P32, rows, rank, s->p_codes, s->p_rmax, s->p_cmax);
    factor_q8_kernel<<<(unsigned)d.nbc, kThreads, 0, st>>>(w.R32, cols, rank, s->r_codes, s->r_rmax, s->r_cmax);
    qm_status stt = launched("grasp state kernels");
    if (stt != QM_OK) return stt;
    // O = NS(M_t) on fp32 operands, written over the grad; W <- W - lr (O + wd W)
    return run_ns_f32_into(w.M, rows, cols, grad, grad_dtype, weight, lr, lr * weight_decay, ns_steps, a, b, c, eps,
                           ns_precision, w.ns, st);
}
