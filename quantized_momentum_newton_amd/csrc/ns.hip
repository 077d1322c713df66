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
//   * One launch per product covers every matrix of the request (up to 8,
//     of any shapes): tiles of all matrices form one index space, the matrix
//     with the longest K first, so 256 CUs stay busy even when one matrix
//     alone has few tiles.
//   * 256x256 output tiles, eight waves of 128x64 (two per SIMD, fp32
//     accumulators in registers), K-tiles of 128 bytes per row in a ring of
//     five one-operand LDS slots filled by direct global-to-LDS loads (no
//     staging registers); a 16-byte XOR swizzle keeps the 16-byte fragment
//     reads free of bank conflicts (64 banks: 16 lanes per cycle).  fp32
//     runs on matrices too small for a full round of 256x256 tiles take
//     128x128 or 64x64 tiles.
//   * Tiles are ordered in bands of 4 tile rows walked column by column, and
//     each XCD's 32 concurrent workgroups cover a 4x8 block of tiles (12
//     operand panels shared in that XCD's L2).  A symmetric product of
//     several rounds over matrices that differ in K gives each XCD an equal
//     share of every matrix's tiles (xcd_tile); other launches deal rounds
//     of 256 tiles (wg_position).
//   * Internal buffers are zero-padded to multiples of 256: zero rows and
//     columns stay zero through the iteration, so no kernel needs bounds
//     checks in its main loop.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <numeric>
#include <vector>

#include "grasp_internal.h"
#include "internal.h"
#include "launch.h"
#include "plan_layout.h"
#include "q8_internal.h"
#include "qmuon.h"

namespace qm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

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

// bf16x3 ("fp32 operands, bf16 MFMA"): an fp32 value x is split into
// hi = bf16(x) and lo = bf16(x - hi), both rounded to nearest even (x - hi
// is exact in fp32).  A product x y is taken as hi hi' + hi lo' + lo hi':
// each term an exact bf16 x bf16 product, accumulated in fp32 by the MFMA;
// the dropped lo lo' is below 2^-16 |x y|.  One fragment holds the 8
// consecutive k of a lane (two 16-byte chunks of fp32).
struct F8 {
    u32x4 x, y;
};
__device__ __forceinline__ void split_bf16x3(const F8 &f, u32x4 &hi, u32x4 &lo) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    const uint32_t w[8] = {f.x.x, f.x.y, f.x.z, f.x.w, f.y.x, f.y.y, f.y.z, f.y.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const f2 v = {__uint_as_float(w[2 * k]), __uint_as_float(w[2 * k + 1])};
        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
        const f2 r = {v.x - __uint_as_float(h << 16), v.y - __uint_as_float(h & 0xffff0000u)};
        hi[k] = h;
        lo[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, b2));
    }
}
__device__ __forceinline__ void mfma_bf16x3(const F8 &a, const F8 &b, f32x16 &c) {
    u32x4 ah, al, bh, bl;
    split_bf16x3(a, ah, al);
    split_bf16x3(b, bh, bl);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al), __builtin_bit_cast(bf16x8, bh), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah), __builtin_bit_cast(bf16x8, bl), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah), __builtin_bit_cast(bf16x8, bh), c, 0, 0, 0);
}

// ------------------------------------------------------------ GEMM kernel

enum Epi { EPI_GRAM = 0, EPI_POLY = 1, EPI_UPDATE = 2 };

// Where the result goes: the caller's matrix (original orientation, its
// dtype) and optionally fp32 weights.
struct FinalOut {
    void *out;
    float *w;
    int64_t ld, ldw;
    int32_t dtype, tall;
    int32_t m, n;          // valid extent in iteration orientation
    float lr_s, lr_wd;     // lr * s and lr * weight_decay
    int32_t vec_out, vec_w;  // out / w rows start 16-byte aligned (8-element segments move as vectors)
};

// One matrix of a grouped product (element strides).
template <typename T> struct GItem {
    const T *P;
    const T *Q;
    T *C;
    T *CT;
    const T *D;
    int64_t ldp, ldq, ldc, ldct, ldd;
    int32_t tiles_m;       // tile rows
    int32_t tiles_n;       // tile columns (== tiles_m for the symmetric products)
    int32_t tile_begin;    // first logical tile of this matrix
    int32_t k_tiles;       // K / (128 / sizeof(T))
    int64_t unit_begin;    // stream-K: first k-tile unit of this matrix (tiles x k_tiles before it)
};

template <typename T> struct GemmArgs {
    GItem<T> it[kMaxItems];
    int32_t n_items;
    int32_t total_tiles;   // tiles of all items (set at launch)
    int32_t xcd;           // 1: tiles dealt by xcd_tile, else by wg_position (set at launch)
    float alpha, beta;     // epilogue: C = alpha D + beta acc (beta = 1 for X = aX + BX)
    // dloop != 0: the D term is gathered inside the k-loop instead (acc +=
    // dgain D, dgain = alpha / beta), then C = beta acc.  Valid because D's
    // tile is a block of the Q operand (see gemm_nt_kernel).
    int32_t dloop;
    float dgain;
    // stream-K launches: sk_units k-tile units (all tiles' k-tiles, items in
    // launch order), workgroup w takes [w sk_len, (w + 1) sk_len); parts of
    // split tiles go to sk_part, two 4 BM BN-byte slots per workgroup
    int64_t sk_units, sk_len;
    float *sk_part;
};

// Workgroup -> (item, tile position in the item's band order).  Workgroups
// go to the 8 XCDs round robin (w % 8).  XCD x takes the x-th contiguous
// eighth of every item's tiles, items in launch order (longest K first), so
// each XCD gets the same share of long-K and short-K tiles and none runs
// out of work while another still holds a second round of long ones.  An
// item's tiles beyond a multiple of 8 go one each to the XCDs after those
// that took the previous item's, so XCD totals differ by at most one.  Its
// 32 concurrent workgroups walk consecutive band positions: a 4 x 8 block
// of tiles whose 4 + 8 operand panels are shared through that XCD's L2.
// The grid holds 8 x the largest XCD total; a workgroup past its XCD's
// total has no tile.
template <typename Args>
__device__ __forceinline__ bool xcd_tile(int w, const Args &args, int &item, int &t) {
    const int x = w & 7, l = w >> 3;
    int seen = 0, s = 0;
    for (int i = 0; i < args.n_items; i++) {
        const int begin = args.it[i].tile_begin;
        const int cnt = (i + 1 < args.n_items ? args.it[i + 1].tile_begin : args.total_tiles) - begin;
        const int q = cnt >> 3, r = cnt & 7;
        const int v = (x - s) & 7;   // which eighth of this item XCD x takes
        const int share = q + (v < r ? 1 : 0);
        if (l < seen + share) {
            item = i;
            t = v * q + min(v, r) + (l - seen);
            return true;
        }
        seen += share;
        s = (s + r) & 7;             // the next item's extra tiles start where these end
    }
    return false;
}

// Workgroup -> position in the tile order (launches that do not take
// xcd_tile).  Workgroups go to the 8 XCDs
// round robin (w % 8) and each XCD runs 32 at a time (one per CU); in every
// round of 256, XCD x takes positions [32x, 32x + 32).  With the band order
// below, those 32 positions are a 4 x 8 block of tiles: 4 + 8 operand
// panels shared through that XCD's L2 instead of up to 64.
__device__ __forceinline__ int wg_position(int w, int nwg) {
    const int full = nwg / 256 * 256;
    if (w >= full) return w;
    const int x = w & 7, l = w >> 3;
    return (l >> 5) * 256 + x * 32 + (l & 31);
}

constexpr int kBand = 4;   // tile rows per band

// Rectangular tile grid (tm x tn), bands of kBand tile rows, each band walked
// column by column.
__device__ __forceinline__ void band_coords(int p, int tm, int tn, int &bi, int &bj) {
    const int b = p / (kBand * tn);
    const int r0 = b * kBand;
    const int h = min(kBand, tm - r0);
    const int q = p - r0 * tn;
    bi = r0 + q % h;
    bj = q / h;
}

// Lower-triangle tile grid (bi >= bj), same band order: in band b (rows
// r0 .. r0+h-1) columns 0..r0 hold h tiles each, then column r0+k holds the
// h-k rows r0+k .. r0+h-1.  Rows below r0 hold r0 (r0 + 1) / 2 tiles.
__device__ __forceinline__ void band_coords_tri(int p, int tm, int &bi, int &bj) {
    int b = 0;
    while ((b + 1) * kBand < tm) {
        const int r1 = (b + 1) * kBand;
        if (r1 * (r1 + 1) / 2 > p) break;
        b++;
    }
    const int r0 = b * kBand;
    const int h = min(kBand, tm - r0);
    int q = p - r0 * (r0 + 1) / 2;
    if (q < (r0 + 1) * h) {
        bi = r0 + q % h;
        bj = q / h;
        return;
    }
    q -= (r0 + 1) * h;
    for (int k = 1; k < h; k++) {
        if (q < h - k) {
            bi = r0 + k + q;
            bj = r0 + k;
            return;
        }
        q -= h - k;
    }
    bi = bj = r0 + h - 1;  // not reached for valid p
}

__device__ __forceinline__ void lds_dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

// Eight consecutive elements <-> fp32: one 16-byte access for bf16, two
// for fp32 (16-byte aligned addresses).
__device__ __forceinline__ void unpack8(const u32x4 w, float *v) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}
// 16-byte accesses; NT: with the non-temporal hint, for data read once (the
// prologue's source: measured 6 % off the prologue and 9 % off the later
// write-back into the same buffer; the hint on the write-back's own accesses
// made it slower).
template <bool NT> __device__ __forceinline__ u32x4 ld16(const void *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else return *reinterpret_cast<const u32x4 *>(p);
}
template <bool NT> __device__ __forceinline__ void st16(void *p, u32x4 w) {
    if constexpr (NT) __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
    else *reinterpret_cast<u32x4 *>(p) = w;
}
template <bool NT = false> __device__ __forceinline__ void load8(const bf16_t *p, float *v) { unpack8(ld16<NT>(p), v); }
template <bool NT = false> __device__ __forceinline__ void load8(const float *p, float *v) {
    const u32x4 a = ld16<NT>(p), b = ld16<NT>(p + 4);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        v[k] = __uint_as_float(a[k]);
        v[4 + k] = __uint_as_float(b[k]);
    }
}
template <bool NT = false> __device__ __forceinline__ void store8(bf16_t *p, const float *v) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; k++)
        w[k] = (uint32_t)to_bf16_bits(v[2 * k]) | ((uint32_t)to_bf16_bits(v[2 * k + 1]) << 16);
    st16<NT>(p, w);
}
template <bool NT = false> __device__ __forceinline__ void store8(float *p, const float *v) {
    u32x4 a, b;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        a[k] = __float_as_uint(v[k]);
        b[k] = __float_as_uint(v[4 + k]);
    }
    st16<NT>(p, a);
    st16<NT>(p + 4, b);
}

// Workgroup barrier for the k-loop.  __syncthreads() carries a release
// fence whose lowering waits for every outstanding vector-memory operation,
// LDS-DMA loads of later stages included, which would drain the prefetch
// pipeline at each k-tile.  Here only LDS reads are completed (so no stage is
// overwritten while a wave still reads it); the DMA of the stage about to be
// read is waited for explicitly with wait_vmcnt_tiles before the barrier.
__device__ __forceinline__ void kloop_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt lgkmcnt(0) with x as an in/out operand: code using x cannot be
// scheduled above the wait (for results of LDS reads issued as assembly).
template <typename V>
__device__ __forceinline__ void lds_wait(V &x) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x));
}

// s_waitcnt vmcnt(n) with n a multiple of D chosen at run time (0..3 D).
template <int D>
__device__ __forceinline__ void wait_vmcnt_tiles(int tiles) {
    if (tiles <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (tiles == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
    else if (tiles == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * D) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * D) : "memory");
}

// One output tile, or one k-range of it.  The k-tiles [ka, kb) of tile t of
// item `item` are multiplied; the tile whole (ka = 0, kb = k_tiles) leaves
// through the epilogue, a part of it (stream-K) stores its raw fp32
// accumulators to `part`.  fix_unit >= 0 (stream-K fix-up, ka = kb = 0):
// the accumulators are the sum of the tile's stored parts, in k order, and
// leave through the epilogue.
template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int ROWB, int NSTAGE, int SLOTS, int MINB, int EPI,
          bool SYM, bool QT, bool X3>
__device__ __forceinline__ void gemm_tile(const GemmArgs<T> &args, int item, int t, int ka, int kb, float *part,
                                          int64_t fix_unit) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int CPR = ROWB / 16;                  // 16-byte chunks per tile row (one k-tile)
    constexpr int RPI = 64 / CPR;                   // tile rows per DMA instruction
    constexpr int SWD = 16 / CPR;                   // rows sharing one 256-byte bank row
    // MFMA k-steps per k-tile (X3: fp32 data, 16 k per bf16x3 step)
    constexpr int STEPS = X3 ? CPR / 4 : CPR / 2;
    static_assert(!X3 || (sizeof(T) == 4 && !QT), "bf16x3: fp32 operands, K-contiguous");
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int PI = BM / RPI / NW, QI = BN / RPI / NW;  // DMA instructions per wave per operand
    constexpr int DPT = PI + QI;                    // per wave per k-tile
    static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile / wave count");
    // QT: the Q operand is stored K x N (row k holds Q[.][k] for all n, n
    // contiguous), as X is for X = aX + BX.  Its k-tile is KK rows of BN
    // elements in LDS; fragments are read with the transposing LDS load.
    constexpr int KK = ROWB / (int)sizeof(T);       // k per k-tile
    constexpr int QRB = BN * (int)sizeof(T);        // bytes of one LDS row of a QT tile
    constexpr int QCPR = QRB / 16, QRPI = 64 / QCPR;
    static_assert(!QT || (sizeof(T) == 2 && KK * QRB == BN * ROWB && KK % (QRPI * NW) == 0 && KK / QRPI / NW == QI),
                  "QT layout: bf16, same stage size and DMA count as the NT layout");
    static_assert(FM >= 1 && FN >= 1 && NSTAGE >= 2 && NSTAGE <= 5, "config");
    // SLOTS > 0: the LDS holds SLOTS buffers of one operand's k-tile each
    // (P of tile kt in slot 2 kt mod SLOTS, Q in 2 kt + 1), instead of
    // NSTAGE stages of both operands; see the pipeline below.
    constexpr bool RING = SLOTS > 0;
    constexpr int HS = BM * ROWB;                   // one operand's k-tile
    static_assert(!RING || (SLOTS == 5 && BM == BN), "ring: five slots of equal operand tiles");
    constexpr size_t LDS_BYTES = RING ? (size_t)SLOTS * HS : (size_t)NSTAGE * STAGE;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const GItem<T> &I = args.it[item];
    int bi, bj;
    if constexpr (SYM) band_coords_tri(t, I.tiles_n, bi, bj);
    else band_coords(t, I.tiles_m, I.tiles_n, bi, bj);

    const int64_t ldpb = I.ldp * (int64_t)sizeof(T), ldqb = I.ldq * (int64_t)sizeof(T);
    // operand panels from k-tile ka on
    const char *Pg = reinterpret_cast<const char *>(I.P + (int64_t)bi * BM * I.ldp) + (int64_t)ka * ROWB;
    const char *Qg = QT ? reinterpret_cast<const char *>(I.Q + (int64_t)bj * BN) + (int64_t)ka * (ROWB / (int)sizeof(T)) * ldqb
                        : reinterpret_cast<const char *>(I.Q + (int64_t)bj * BN * I.ldq) + (int64_t)ka * ROWB;
    const int lrw = lane / CPR, lch = lane % CPR;

    // One DMA instruction of the Q operand's k-tile kt (i < QI) into the Q
    // buffer qb.  QT: QRPI rows of QRB bytes; the 16-byte chunk c of LDS
    // row k sits at position c ^ 4 (k % 4), so the transposing fragment
    // reads (4 rows x 64 bytes per half-wave) cover all 64 banks.
    auto dma_q = [&](int kt, char *qb, int i) {
        if constexpr (QT) {
            const int r0 = (wave + i * NW) * QRPI;
            const int row = r0 + lane / QCPR, pos = lane % QCPR;
            lds_dma16(Qg + ((int64_t)kt * KK + row) * ldqb + ((pos ^ (4 * (row & 3))) << 4), qb + r0 * QRB);
        } else {
            const int r0 = (wave + i * NW) * RPI;
            const int row = r0 + lrw;
            lds_dma16(Qg + row * ldqb + (int64_t)kt * ROWB + ((lch ^ ((row / SWD) % CPR)) << 4), qb + r0 * ROWB);
        }
    };
    // One DMA instruction of the P operand's k-tile kt (i < PI) into pb.
    auto dma_p = [&](int kt, char *pb, int i) {
        const int r0 = (wave + i * NW) * RPI;
        const int row = r0 + lrw;
        lds_dma16(Pg + row * ldpb + (int64_t)kt * ROWB + ((lch ^ ((row / SWD) % CPR)) << 4), pb + r0 * ROWB);
    };
    // operand buffers of k-tile kt
    // (slot offsets are wave-uniform: kept in scalar registers)
    auto pbuf = [&](int kt) -> char * {
        if constexpr (RING) return smem + __builtin_amdgcn_readfirstlane((2 * kt) % SLOTS * HS);
        else return smem + (kt % NSTAGE) * STAGE;
    };
    auto qbuf = [&](int kt) -> char * {
        if constexpr (RING) return smem + __builtin_amdgcn_readfirstlane((2 * kt + 1) % SLOTS * HS);
        else return smem + (kt % NSTAGE) * STAGE + BM * ROWB;
    };
    // In the k-loop, ring slot j places after P of tile kt, slot
    // (2 kt + j) mod SLOTS, from a running base instead of a division per use
    // (the scalar division cost the Gram 1.5 %).
    int rbase = 0;
    auto ring = [&](int j) -> char * {
        const int r = rbase + j;
        return smem + __builtin_amdgcn_readfirstlane((r >= SLOTS ? r - SLOTS : r) * HS);
    };

    // Direct loads: one instruction moves RPI tile rows (1 KiB) into LDS;
    // lane l lands at row r0 + l / CPR, position l % CPR, so it fetches global
    // chunk (l % CPR) ^ sw(row) -- the swizzle is applied on the global side.
    // sw(row) = (row / SWD) % CPR gives 16 consecutive rows' copies of one
    // logical chunk 16 distinct 16-byte slots of a 256-byte bank row: the 16
    // lanes a fragment read serves together never collide (64 banks).
    auto issue_p = [&](int kt) {
#pragma unroll
        for (int i = 0; i < PI; i++) dma_p(kt, pbuf(kt), i);
    };
    auto issue_q = [&](int kt) {
#pragma unroll
        for (int i = 0; i < QI; i++) dma_q(kt, qbuf(kt), i);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int KT = kb - ka;   // k-tiles of this call, counted from ka
    const int lrow = lane & 31, lhalf = lane >> 5;
    // QT reads.  ds_read_b64_tr_b16 works on groups of 16 lanes: if lane s
    // of a group points at 4 consecutive elements, lane t receives element
    // t % 4 of lanes t / 4, t / 4 + 4, t / 4 + 8, t / 4 + 12.  With lane s
    // pointing at row k0 + s / 4, column n0 + 4 (s % 4), lane t gets column
    // n0 + t of rows k0 .. k0 + 3.  read_qt4 gives lane l column
    // nb + 16 ((l / 16) % 2) + l % 16 at rows k0 .. k0+3 (k0 uniform per
    // group); read_qt8 the 8 rows k0 .. k0+7 as one MFMA fragment.
    //
    // The read is issued as inline assembly.  Through the builtin, the
    // compiler cannot tell it from a read of the stage an LDS-DMA load is
    // filling and puts s_waitcnt vmcnt(0) in front of it, which drains every
    // prefetched tile.  The stage protocol of the k-loop (explicit vmcnt
    // waits and barriers) already orders DMA and reads; the compiler does
    // not see these reads in its lgkmcnt accounting, so their results are
    // waited for with lds_wait below before first use.
    auto read_qt4 = [&](const char *cq, int k0, int nb) -> u32x2 {
        const int s16 = lane & 15;
        const int row = k0 + (s16 >> 2);
        const int cb = (nb + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;
        const char *p = cq + row * QRB + ((((cb >> 4) ^ (4 * (row & 3)))) << 4) + (cb & 15);
        const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
        u32x2 r;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
        return r;
    };
    auto read_qt8 = [&](const char *cq, int k0, int nb) -> u32x4 {
        const u32x2 lo = read_qt4(cq, k0, nb), hi = read_qt4(cq, k0 + 4, nb);
        return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    using Frag = std::conditional_t<X3, F8, u32x4>;
    // X3: lane half h of step s takes k 16 s + 8 h .. + 7: chunks 4 s + 2 h and 4 s + 2 h + 1
    auto read_frag = [&](const char *base, int row, int s) -> Frag {
        const int sw = (row / SWD) % CPR;
        if constexpr (X3) {
            const int c0 = 4 * s + 2 * lhalf;
            return F8{*reinterpret_cast<const u32x4 *>(base + row * ROWB + ((c0 ^ sw) << 4)),
                      *reinterpret_cast<const u32x4 *>(base + row * ROWB + (((c0 + 1) ^ sw) << 4))};
        } else {
            return *reinterpret_cast<const u32x4 *>(base + row * ROWB + (((2 * s + lhalf) ^ sw) << 4));
        }
    };
    auto read_frags = [&](const char *cp, const char *cq, int s, Frag *a, Frag *b) {
        const int ch = 2 * s + lhalf;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            a[i] = read_frag(cp, wm * WM + i * 32 + lrow, s);
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
            if constexpr (QT) {
                b[j] = read_qt8(cq, 16 * s + 8 * (lane >> 5), wn * WN + j * 32);
            } else {
                b[j] = read_frag(cq, wn * WN + j * 32 + lrow, s);
            }
        }
    };
    // Software pipeline.  Fragments for k-step s+1 are read into a second
    // register set while the MFMAs of step s run; the next tile's first
    // fragments are read right after the barrier, while the last MFMAs of
    // this tile drain.  The DMA issued during a tile is spread over its
    // k-steps (one slice per step).
    //  * NSTAGE stages: tiles kt+1 .. kt+NSTAGE-1 are in flight while tile kt
    //    is multiplied, and each iteration waits only for tile kt+1.
    //  * ring (five one-operand slots): while tile kt is multiplied, P of
    //    tile kt+1 is already in flight (issued during tile kt-1), and Q of
    //    kt+1 and P of kt+2 are issued into the two slots tile kt-1 freed;
    //    the iteration waits for everything but P of kt+2.  P loads thus get
    //    two tiles of lead and Q loads one, where two full stages give each
    //    load between a quarter and all of one tile.
    Frag fa[2][FM], fb[2][FN];
    constexpr int DPS = (DPT + STEPS - 1) / STEPS;  // DMA instructions per k-step
    auto issue_part = [&](int kt, int part) {
#pragma unroll
        for (int d = part * DPS; d < (part + 1) * DPS && d < DPT; d++) {
            if constexpr (RING) {
                if (d < QI) {
                    if (kt + 1 < KT) dma_q(kt + 1, ring(3), d);
                } else {
                    if (kt + 2 < KT) dma_p(kt + 2, ring(4), d - QI);
                }
            } else {
                const int nk = kt + NSTAGE - 1;
                if (nk < KT) {
                    if (d < PI) dma_p(nk, pbuf(nk), d);
                    else dma_q(nk, qbuf(nk), d - PI);
                }
            }
        }
    };
    if (KT > 0) {
        if constexpr (RING) {
            issue_p(0);
            issue_q(0);
            if (KT > 1) issue_p(1);
            wait_vmcnt_tiles<PI>(KT > 1 ? 1 : 0);
        } else {
#pragma unroll
            for (int k = 0; k < NSTAGE - 1; k++)
                if (k < KT) {
                    issue_p(k);
                    issue_q(k);
                }
            wait_vmcnt_tiles<DPT>(min(NSTAGE - 2, KT - 1));
        }
        kloop_barrier();
        read_frags(pbuf(0), qbuf(0), 0, fa[0], fb[0]);
    }
    // The D term in the k-loop.  For X = aX + BX (Q = X, or X^T in fp32
    // runs) and for B = bA + cA^2 (Q = A, symmetric), D's tile (bi, bj)
    // equals the Q panel bj at k in [bi BM, bi BM + BM): element (row R,
    // column C) of the tile is Q at (n = bj BN + C, k = bi BM + R).  While
    // such a k-tile is in LDS, the waves owning rows R add dgain * D to their
    // accumulators, so the epilogue reads no D from memory.  fp32 runs gather
    // it with VALU adds (four consecutive rows of one column are four
    // consecutive k: one 16-byte LDS read); bf16 runs add it with MFMAs
    // (below).
    static_assert(32 % KK == 0 || KK % 32 == 0, "k-tile vs sub-tile rows");
    const bool dloop = EPI != EPI_GRAM && args.dloop;
    auto gather_d = [&](const char *cq, int kt) {
        if constexpr (sizeof(T) == 4 && !QT)
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int64_t rb = (int64_t)bi * BM + wm * WM + i * 32;  // first k of sub-tile i
            if (rb / KK != kt + ka) continue;
            const int kk0 = (int)(rb % KK) + 4 * lhalf;
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int row = wn * WN + j * 32 + lrow;
                const char *qr = cq + row * ROWB;
                const int sw = (row / SWD) % CPR;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int ob = (kk0 + 8 * g) * (int)sizeof(T);
                    float d[4];
                    *reinterpret_cast<float4 *>(d) =
                        *reinterpret_cast<const float4 *>(qr + (((ob >> 4) ^ sw) << 4) + (ob & 15));
#pragma unroll
                    for (int q = 0; q < 4; q++) acc[i][j][4 * g + q] += args.dgain * d[q];
                }
            }
        }
    };
    // bf16: the D term as MFMAs.  D's tile row R is the Q operand at
    // k = bi BM + R (above), so dgain D = (dgain I) Q over those k: in the
    // k-step whose 16 k are rows 16 h .. 16 h + 15 of sub-tile i, an A
    // fragment holding dgain at (row 16 h + e, k e) times the step's B
    // fragments adds the term to acc[i][.].  dgain is split into bf16
    // hi = bf16(dgain) and lo = bf16(dgain - hi): two MFMAs whose products are
    // exact in fp32, |dgain - hi - lo| <= 2^-17 |dgain|.
    constexpr bool DMF = sizeof(T) == 2;
    static_assert(!DMF || (WM % KK == 0 && KK % 32 == 0), "D by MFMA: wave rows span whole k-tiles");
    const uint16_t dhi = to_bf16_bits(args.dgain);
    const uint16_t dlo = to_bf16_bits(args.dgain - __uint_as_float((uint32_t)dhi << 16));
    // A-fragment lane l holds row l % 32 at k 8 (l / 32) .. +7
    auto eye_frag = [&](int h, uint16_t v) -> u32x4 {
        const int e = lrow - 16 * h - 8 * lhalf;
        const uint32_t w = (e >= 0 && e < 8) ? ((uint32_t)v << (16 * (e & 1))) : 0u;
        const int q = e >> 1;
        return u32x4{q == 0 ? w : 0u, q == 1 ? w : 0u, q == 2 ? w : 0u, q == 3 ? w : 0u};
    };
    const int dkt0 = (int)(((int64_t)bi * BM + wm * WM) / KK) - ka;   // first k-tile of this wave's D rows
    for (int kt = 0; kt < KT; kt++) {
        const char *cp = RING ? ring(0) : pbuf(kt), *cq = RING ? ring(1) : qbuf(kt);
        if constexpr (!DMF) {
            if (dloop) gather_d(cq, kt);
        }
#pragma unroll
        for (int s = 0; s < STEPS; s++) {
            // QT: fragments of this step came from assembly reads issued a
            // step earlier; complete them (tied to the registers, so the
            // MFMAs below cannot move above the wait)
            if constexpr (QT) {
#pragma unroll
                for (int j = 0; j < FN; j++) lds_wait(fb[s & 1][j]);
            }
            if (s + 1 < STEPS) read_frags(cp, cq, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            issue_part(kt, s);
            // raised wave priority while the step's MFMAs issue: with two
            // waves per SIMD, the one holding ready MFMAs goes first (about
            // 1 % on the NS products)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    if constexpr (X3) mfma_bf16x3(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                    else Mfma<T>::step(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                }
            if constexpr (DMF) {
                if (dloop) {
                    const int t = kt - dkt0;
#pragma unroll
                    for (int tt = 0; tt < WM / KK; tt++)
                        if (t == tt) {
                            const int i = tt * (KK / 32) + s / 2, h = s % 2;
                            const u32x4 eh = eye_frag(h, dhi), el = eye_frag(h, dlo);
#pragma unroll
                            for (int j = 0; j < FN; j++) {
                                Mfma<T>::step(eh, fb[s & 1][j], acc[i][j]);
                                Mfma<T>::step(el, fb[s & 1][j], acc[i][j]);
                            }
                        }
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        // loads still allowed in flight: those of later tiles than kt+1
        if constexpr (RING)
            wait_vmcnt_tiles<PI>(kt + 2 < KT ? 1 : 0);
        else
            wait_vmcnt_tiles<DPT>(min(KT - 1, kt + NSTAGE - 1) - (kt + 1));
        kloop_barrier();
        if (kt + 1 < KT) {
            if constexpr (RING) read_frags(ring(2), ring(3), 0, fa[STEPS & 1], fb[STEPS & 1]);
            else read_frags(pbuf(kt + 1), qbuf(kt + 1), 0, fa[STEPS & 1], fb[STEPS & 1]);
        }
        if constexpr (RING) {
            rbase += 2;
            if (rbase >= SLOTS) rbase -= SLOTS;
        }
    }

    // ------------------------------------------------ stream-K parts
    // A part's accumulators are stored and loaded in register order: per
    // (wave, i, j, four-row group) one 16-byte unit per lane, 1 KiB per wave
    // instruction.  The parts of a tile come from consecutive workgroups w
    // of the stream-K launch (each takes units [w len, (w + 1) len)); the
    // part that begins a workgroup's range sits in slot 2 w, a later one
    // (its last, begun at a tile start) in slot 2 w + 1.
    auto part_at = [&](float *base, int i, int j, int r4) -> float4 * {
        return reinterpret_cast<float4 *>(base) + (((wave * FM + i) * FN + j) * 4 + r4) * 64 + lane;
    };
    if (part) {
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int r4 = 0; r4 < 4; r4++)
                    *part_at(part, i, j, r4) =
                        float4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
        return;
    }
    if (fix_unit >= 0) {
        const int64_t len = args.sk_len, u1 = fix_unit + I.k_tiles;
        for (int64_t w = fix_unit / len; w * len < u1; w++) {   // k order
            float *src = args.sk_part + (size_t)(2 * w + (fix_unit > w * len ? 1 : 0)) * BM * BN;
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
#pragma unroll
                    for (int r4 = 0; r4 < 4; r4++) {
                        const float4 v = *part_at(src, i, j, r4);
                        acc[i][j][4 * r4] += v.x;
                        acc[i][j][4 * r4 + 1] += v.y;
                        acc[i][j][4 * r4 + 2] += v.z;
                        acc[i][j][4 * r4 + 3] += v.w;
                    }
        }
    }

    // ---------------------------------------------------------- epilogue
    // The output tile leaves through LDS, ER rows per pass, so that every
    // global access is a 16-byte segment of a row:
    //  1. the waves owning the pass's rows write their fp32 accumulators to
    //     a padded LDS tile (acc[i][j][r] is row 8(r/4) + 4 lhalf + r%4,
    //     column lrow of its 32x32 MFMA tile);
    //  2. row phase: each thread takes 8 consecutive columns of one row,
    //     forms the epilogue value (loading D there unless the k-loop has
    //     gathered it), rounds it to T, stores the segment of C and writes
    //     the rounded value back in place;
    //  3. column phase (the fp32 runs' X^T copy, or the mirror tile of a
    //     symmetric product): each thread takes 8 consecutive rows of one column and
    //     stores them as a segment of the transposed target; the lanes of a
    //     wave read consecutive columns of one LDS row per instruction.
    // The loop's last barrier has passed, so every stage buffer is free.
    constexpr int ER = WM < 64 ? WM : 64;   // tile rows per pass
    constexpr int EP = BN + 8;       // fp32 pitch; 4 EP = 32 mod 64 banks separates the two half-waves
    constexpr int NTH = NW * 64;
    constexpr int RIT = ER * (BN / 8) / NTH;   // row-phase items per thread
    constexpr int CIT = BN * (ER / 8) / NTH;   // column-phase items per thread
    static_assert(WM % ER == 0 && ER % 32 == 0 && BM % ER == 0, "epilogue pass rows");
    static_assert((size_t)ER * EP * 4 <= LDS_BYTES, "epilogue tile must fit the stage buffers");
    static_assert(RIT * NTH == ER * (BN / 8) && CIT * NTH == BN * (ER / 8), "epilogue work split");
    float *et = reinterpret_cast<float *>(smem);
    T *tgt = nullptr;                // transposed target
    int64_t ldt = 0;
    if constexpr (EPI == EPI_UPDATE) {
        tgt = I.CT;
        ldt = I.ldct;
    } else if (SYM && bi != bj) {
        tgt = I.C;
        ldt = I.ldc;
    }
    const int64_t R0 = (int64_t)bi * BM, C0 = (int64_t)bj * BN;
    const float sc = EPI == EPI_POLY ? args.beta : 1.0f;
    // bf16: the D segments of every pass are loaded up front (16 bytes per
    // item, BM / ER * RIT registers of 4 dwords), so their latency is paid
    // once per tile instead of once per pass.
    constexpr bool DPRE = EPI != EPI_GRAM && sizeof(T) == 2;
    u32x4 dpre[DPRE ? BM / ER : 1][DPRE ? RIT : 1];
    if (DPRE && !dloop) {
#pragma unroll
        for (int p = 0; p < BM / ER; p++)
#pragma unroll
            for (int it = 0; it < RIT; it++) {
                const int idx = tid + it * NTH;
                const int r = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
                dpre[p][it] = *reinterpret_cast<const u32x4 *>(I.D + (R0 + p * ER + r) * I.ldd + C0 + c);
            }
    }
#pragma unroll
    for (int p = 0; p < BM / ER; p++) {
        const int pw = p * ER / WM;            // owning wave row
        const int i0 = (p * ER % WM) / 32;     // its first sub-tile in this pass
        if (wm == pw) {
#pragma unroll
            for (int ii = 0; ii < ER / 32; ii++)
#pragma unroll
                for (int j = 0; j < FN; j++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int row = ii * 32 + 8 * (r / 4) + 4 * lhalf + (r % 4);
                        et[row * EP + wn * WN + j * 32 + lrow] = acc[i0 + ii][j][r];
                    }
        }
        kloop_barrier();
        const int64_t pr = R0 + p * ER;
#pragma unroll
        for (int it = 0; it < RIT; it++) {
            const int idx = tid + it * NTH;
            const int r = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
            float *e = et + r * EP + c;
            float v[8];
            *reinterpret_cast<float4 *>(v) = *reinterpret_cast<const float4 *>(e);
            *reinterpret_cast<float4 *>(v + 4) = *reinterpret_cast<const float4 *>(e + 4);
            if constexpr (EPI != EPI_GRAM) {
                if (dloop) {
#pragma unroll
                    for (int k = 0; k < 8; k++) v[k] = sc * v[k];
                } else {
                    float d[8];
                    if constexpr (DPRE)
                        unpack8(dpre[p][it], d);
                    else
                        load8(I.D + (pr + r) * I.ldd + C0 + c, d);
#pragma unroll
                    for (int k = 0; k < 8; k++) v[k] = args.alpha * d[k] + sc * v[k];
                }
            }
            store8(I.C + (pr + r) * I.ldc + C0 + c, v);
            if (tgt) {
#pragma unroll
                for (int k = 0; k < 8; k++) v[k] = to_float(from_float<T>(v[k]));
                *reinterpret_cast<float4 *>(e) = *reinterpret_cast<const float4 *>(v);
                *reinterpret_cast<float4 *>(e + 4) = *reinterpret_cast<const float4 *>(v + 4);
            }
        }
        if (tgt) {
            kloop_barrier();
#pragma unroll
            for (int it = 0; it < CIT; it++) {
                const int idx = tid + it * NTH;
                const int c = idx % BN, r = (idx / BN) * 8;
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; k++) v[k] = et[(r + k) * EP + c];
                store8(tgt + (C0 + c) * ldt + pr + r, v);
            }
        }
        kloop_barrier();
    }
}

template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int ROWB, int NSTAGE, int SLOTS, int MINB, int EPI,
          bool SYM, bool QT, bool X3>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, MINB) void gemm_nt_kernel(GemmArgs<T> args) {
    int item = 0, t = 0;
    if (SYM && args.xcd) {
        if (!xcd_tile(blockIdx.x, args, item, t)) return;   // uniform: the whole workgroup
    } else {
        const int L = wg_position(blockIdx.x, gridDim.x);
        while (item + 1 < args.n_items && args.it[item + 1].tile_begin <= L) item++;
        t = L - args.it[item].tile_begin;
    }
    gemm_tile<T, BM, BN, WAVES_M, WAVES_N, ROWB, NSTAGE, SLOTS, MINB, EPI, SYM, QT, X3>(args, item, t, 0, args.it[item].k_tiles, nullptr, -1);
}

// Stream-K: a launch whose tiles would leave the last round of workgroups
// partly filled splits their k-tiles evenly over the workgroups instead.
// Workgroup w multiplies units [w len, (w + 1) len) of the units of all
// tiles (item by item, tile by tile, k-tile by k-tile): whole tiles leave
// through the epilogue, the pieces of a tile cut by a range boundary store
// their raw accumulators; gemm_sk_fixup_kernel then adds each cut tile's
// pieces in k order and runs the epilogue.  The sum order is fixed, so
// outputs are the same from run to run.
template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int ROWB, int NSTAGE, int SLOTS, int MINB, int EPI,
          bool SYM, bool QT, bool X3>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, MINB) void gemm_sk_kernel(GemmArgs<T> args) {
    const int64_t len = args.sk_len, w = blockIdx.x;
    int64_t u = w * len;
    const int64_t u1 = u + len < args.sk_units ? u + len : args.sk_units;
    while (u < u1) {   // uniform
        int item = 0;
        while (item + 1 < args.n_items && args.it[item + 1].unit_begin <= u) item++;
        const GItem<T> &I = args.it[item];
        const int64_t rel = u - I.unit_begin;
        const int t = (int)(rel / I.k_tiles), ka = (int)(rel % I.k_tiles);
        const int kb = (int)(ka + (u1 - u) < I.k_tiles ? ka + (u1 - u) : I.k_tiles);
        float *part = ka == 0 && kb == I.k_tiles
                          ? nullptr
                          : args.sk_part + (size_t)(2 * w + (u > w * len ? 1 : 0)) * BM * BN;
        gemm_tile<T, BM, BN, WAVES_M, WAVES_N, ROWB, NSTAGE, SLOTS, MINB, EPI, SYM, QT, X3>(args, item, t, ka, kb, part, -1);
        u += kb - ka;
    }
}

// One workgroup per range boundary b = (w + 1) len: the tile that b cuts is
// finished by the workgroup of the first boundary inside it.
template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int ROWB, int NSTAGE, int SLOTS, int MINB, int EPI,
          bool SYM, bool QT, bool X3>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, MINB) void gemm_sk_fixup_kernel(GemmArgs<T> args) {
    const int64_t len = args.sk_len, b = (int64_t)(blockIdx.x + 1) * len;
    if (b >= args.sk_units) return;
    int item = 0;
    while (item + 1 < args.n_items && args.it[item + 1].unit_begin <= b) item++;
    const GItem<T> &I = args.it[item];
    const int64_t rel = b - I.unit_begin;
    const int64_t ut = b - rel % I.k_tiles;   // first unit of the cut tile
    if (ut == b || b - len > ut) return;      // b starts a tile, or an earlier boundary owns it
    gemm_tile<T, BM, BN, WAVES_M, WAVES_N, ROWB, NSTAGE, SLOTS, MINB, EPI, SYM, QT, X3>(args, item, (int)(rel / I.k_tiles), 0, 0, nullptr, ut);
}

// ------------------------------------------------------------ MX Gram
// The first Gram product of an iteration whose input is an MXFP8 carrier
// ("Quantized Muon Momentum", section "Wave18B MXFP8 Carrier Probe": the
// carrier feeds the Gram GEMM): A = alpha X X^T, X = the carrier's E4M3
// bytes (rows x K, K contiguous) with one E8M0 scale per 32 k of a row,
// alpha = inv_norm^2, on gfx950's block-scaled v_mfma_scale_f32_32x32x64
// (fp8 operands, fp32 accumulation), output bf16.
//
// Operand layout of that instruction (measured with an in-bounds probe:
// one nonzero byte per test, all-ones other operand, distinct scales per
// lane half): lane l holds row l % 32; its bytes 0..15 lie in the first
// 32-k block of the 64-k step and bytes 16..31 in the second; the scale of
// block 0 of row r comes from lane r, that of block 1 from lane r + 32.
// So lane (r, h) of k-step s loads the 16-byte chunks 4s + h and 4s + 2 + h
// of its row's 128-byte k-tile and supplies the scale of 32-k block
// 2s + h (the order of k inside a block does not change the sum).
//
// Tiles as the bf16 Gram: 256 x 256 lower-triangle tiles, 8 waves of
// 128 x 64, two LDS stages filled by LDS-DMA; a stage holds 512 rows x 128
// bytes of data and each row's 4 scale bytes of the k-tile (one 4-byte DMA
// per wave covers 64 rows).  Requires rows % 256 == 0, K % 128 == 0.
struct MxItem {
    const uint8_t *X;      // rows x K bytes, row pitch ldx bytes
    const uint8_t *S;      // scales, row pitch lds bytes (K / 32 used)
    bf16_t *C;             // A, row pitch ldc elements
    const float *inv;      // device inverse norm: alpha = inv^2
    int64_t ldx, lds, ldc;
    int32_t tiles_m, tile_begin, k_tiles, pad;
};

struct MxGramArgs {
    MxItem it[kMaxItems];
    int32_t n_items;
    int32_t total_tiles;   // tiles of all items (set at launch)
    int32_t xcd;           // as in GemmArgs
};

typedef __attribute__((ext_vector_type(8))) int i32x8;

__global__ __launch_bounds__(512, 1) void gram_mx_kernel(MxGramArgs args) {
    constexpr int BM = 256, BN = 256, WAVES_N = 4, NW = 8;
    constexpr int WM = 128, WN = 64, FM = WM / 32, FN = WN / 32;
    constexpr int ROWB = 128, CPR = 8, RPI = 8, SWD = 2, NSTAGE = 2, STEPS = 2;
    constexpr int SROWS = BM + BN;
    constexpr int DATA = SROWS * ROWB;
    constexpr int STAGE = DATA + SROWS * 4;
    constexpr int PI = BM / RPI / NW, QI = BN / RPI / NW;
    constexpr int DPT = PI + QI + 1;                // + the scale DMA
    constexpr int DPS = (DPT + STEPS - 1) / STEPS;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int item = 0, t = 0;
    if (args.xcd) {
        if (!xcd_tile(blockIdx.x, args, item, t)) return;   // uniform: the whole workgroup
    } else {
        const int L = wg_position(blockIdx.x, gridDim.x);
        while (item + 1 < args.n_items && args.it[item + 1].tile_begin <= L) item++;
        t = L - args.it[item].tile_begin;
    }
    const MxItem &I = args.it[item];
    int bi, bj;
    band_coords_tri(t, I.tiles_m, bi, bj);

    const uint8_t *Pg = I.X + (int64_t)bi * BM * I.ldx, *Qg = I.X + (int64_t)bj * BN * I.ldx;
    const uint8_t *Ps = I.S + (int64_t)bi * BM * I.lds, *Qs = I.S + (int64_t)bj * BN * I.lds;
    const int lrw = lane / CPR, lch = lane % CPR;
    // DMA instruction d of k-tile kt: d < PI + QI move 8 rows x 128 bytes
    // (swizzled as the bf16 kernel: chunk c of row r at c ^ ((r / 2) % 8)),
    // the last one the scale dwords of rows 64 wave .. 64 wave + 63.  The
    // per-lane part of each address is a 32-bit offset from a wave-uniform
    // panel base (a panel spans < 2^32 bytes: 256 rows of < 2^22 bytes).
    uint32_t off[PI + QI];
#pragma unroll
    for (int d = 0; d < PI + QI; d++) {
        const int row = (wave + (d >= PI ? d - PI : d) * NW) * RPI + lrw;
        off[d] = (uint32_t)(row * I.ldx) + ((lch ^ ((row / SWD) % CPR)) << 4);
    }
    const int srow = wave * 64 + lane;             // stage row of this lane's scale dword: P rows, then Q rows
    const uint8_t *sbase = srow < BM ? Ps : Qs;
    const uint32_t soff = (uint32_t)((srow % BM) * I.lds);
    // The k-tile's part of an address goes through a wave-uniform register
    // (readfirstlane), so each load is a scalar base plus the 32-bit lane
    // offset and the compiler keeps no 64-bit per-lane address per load.
    auto uni = [](const uint8_t *p) -> const uint8_t * {
        const uint64_t v = reinterpret_cast<uint64_t>(p);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
    };
    auto dma = [&](int kt, char *base, int d) {
        if (d < PI + QI) {
            const bool q = d >= PI;
            const int r0 = (wave + (q ? d - PI : d) * NW) * RPI;
            lds_dma16(uni((q ? Qg : Pg) + (int64_t)kt * ROWB) + off[d], base + ((q ? BM : 0) + r0) * ROWB);
        } else {
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(uni(sbase + kt * 4) + soff),
                                             (__attribute__((address_space(3))) void *)(base + DATA + wave * 256),
                                             4, 0, 0);
        }
    };
    auto issue_part = [&](int kt, int stage, int part) {
        char *base = smem + stage * STAGE;
#pragma unroll
        for (int d = part * DPS; d < (part + 1) * DPS && d < DPT; d++) dma(kt, base, d);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int KT = I.k_tiles;
    const int lrow = lane & 31, lhalf = lane >> 5;
    auto frag = [&](const char *cp, int row, int s) -> i32x8 {
        const int sw = (row / SWD) % CPR;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(cp + row * ROWB + (((4 * s + lhalf) ^ sw) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(cp + row * ROWB + (((4 * s + 2 + lhalf) ^ sw) << 4));
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_frags = [&](const char *cp, int s, i32x8 *a, i32x8 *b) {
#pragma unroll
        for (int i = 0; i < FM; i++) a[i] = frag(cp, wm * WM + i * 32 + lrow, s);
#pragma unroll
        for (int j = 0; j < FN; j++) b[j] = frag(cp, BM + wn * WN + j * 32 + lrow, s);
    };
    auto read_scales = [&](const char *cp, uint32_t *sa, uint32_t *sb) {
        const uint32_t *sc = reinterpret_cast<const uint32_t *>(cp + DATA);
#pragma unroll
        for (int i = 0; i < FM; i++) sa[i] = sc[wm * WM + i * 32 + lrow];
#pragma unroll
        for (int j = 0; j < FN; j++) sb[j] = sc[BM + wn * WN + j * 32 + lrow];
    };

    // One register set of fragments (the 256 registers a wave has at two
    // waves per SIMD hold the 128 accumulators, one set of fragments and the
    // addresses); the other wave on the SIMD covers the LDS latency.
    i32x8 fa[FM], fb[FN];
    uint32_t sa[FM], sb[FN];
    issue_part(0, 0, 0);
    issue_part(0, 0, 1);
    wait_vmcnt_tiles<DPT>(0);
    kloop_barrier();
    // k-tile kt from stage kt % 2 while tile kt + 1 streams into the other
    // (the last tile is peeled off, so the loop body is branch-free and the
    // scheduling barriers keep one step's fragments live at a time)
    auto tile = [&](int kt, bool next) {
        const char *cp = smem + (kt % NSTAGE) * STAGE;
        read_scales(cp, sa, sb);
#pragma unroll
        for (int s = 0; s < STEPS; s++) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cp, s, fa, fb);
            if (next) issue_part(kt + 1, (kt + 1) % NSTAGE, s);
            const int sh = 8 * (2 * s + lhalf);      // this lane's 32-k block of the step
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], acc[i][j], 0, 0, 0, (int)(sa[i] >> sh), 0, (int)(sb[j] >> sh));
        }
        wait_vmcnt_tiles<DPT>(0);
        kloop_barrier();
    };
    for (int kt = 0; kt + 1 < KT; kt++) tile(kt, true);
    tile(KT - 1, false);

    // epilogue: C = alpha acc (bf16) through LDS, 64 rows per pass; the
    // mirror tile (bi != bj) from the same rounded values
    constexpr int ER = 64, EP = BN + 8, NTH = NW * 64;
    constexpr int RIT = ER * (BN / 8) / NTH, CIT = BN * (ER / 8) / NTH;
    static_assert((size_t)ER * EP * 4 <= (size_t)NSTAGE * STAGE, "epilogue tile must fit the stage buffers");
    float *et = reinterpret_cast<float *>(smem);
    const float alpha = I.inv[0] * I.inv[0];
    const int64_t R0 = (int64_t)bi * BM, C0 = (int64_t)bj * BN;
#pragma unroll
    for (int p = 0; p < BM / ER; p++) {
        const int pw = p * ER / WM, i0 = (p * ER % WM) / 32;
        if (wm == pw) {
#pragma unroll
            for (int ii = 0; ii < ER / 32; ii++)
#pragma unroll
                for (int j = 0; j < FN; j++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int row = ii * 32 + 8 * (r / 4) + 4 * lhalf + (r % 4);
                        et[row * EP + wn * WN + j * 32 + lrow] = acc[i0 + ii][j][r];
                    }
        }
        kloop_barrier();
        const int64_t pr = R0 + p * ER;
#pragma unroll
        for (int it = 0; it < RIT; it++) {
            const int idx = tid + it * NTH;
            const int r = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
            float *e = et + r * EP + c;
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; k++) v[k] = alpha * e[k];
            store8(I.C + (pr + r) * I.ldc + C0 + c, v);
            if (bi != bj) {
#pragma unroll
                for (int k = 0; k < 8; k++) e[k] = to_float(from_float<bf16_t>(v[k]));
            }
        }
        if (bi != bj) {
            kloop_barrier();
#pragma unroll
            for (int it = 0; it < CIT; it++) {
                const int idx = tid + it * NTH;
                const int c = idx % BN, r = (idx / BN) * 8;
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; k++) v[k] = et[(r + k) * EP + c];
                store8(I.C + (C0 + c) * I.ldc + pr + r, v);
            }
        }
        kloop_barrier();
    }
}

constexpr size_t kMxGramLds = 2 * (512 * 128 + 512 * 4);

// ------------------------------------------------------- norm + prologue

// Source format code of an MXFP8 carrier (payload bytes + per-32 E8M0
// scales); the public qm_dtype codes are 0..2.
constexpr int32_t kSrcMx8 = 16;

struct NsItem {
    const void *src;
    int64_t ld;
    const uint8_t *sc;     // carrier scales (kSrcMx8): byte (r, c / 32) at sc[r * sld + c / 32]
    int64_t sld;
    int32_t dtype;
    int32_t tall;
    const float *inv;      // device scale, or null: computed from the data
    void *X, *XT;          // internal buffers (element type of the run)
    int32_t m, n;          // valid extent in iteration orientation
    int64_t mp, np;        // padded
    int64_t ldx, ldxt;     // leading dimensions of X (np + pad) and X^T (mp + pad)
    int32_t tiles_n;       // 64-wide tiles per padded row
    int32_t tile_begin;    // first 64x64 tile of this item
    int32_t vec;           // src rows start 16-byte aligned
};

struct PrologueArgs {
    NsItem it[kMaxItems];
    int32_t n_items;
    const float *inv_ws;   // per-item computed scales (when it[i].inv is null)
};

__device__ __forceinline__ int find_item(const PrologueArgs &a, int L) {
    int item = 0;
    while (item + 1 < a.n_items && a.it[item + 1].tile_begin <= L) item++;
    return item;
}

// Origin (i0, j0) of 64 x 64 tile t of an item.  When the caller-side
// matrix (the one read in the prologue, written in the write-back) is the
// transpose of X, consecutive tiles walk down X's rows (i fastest), which
// is along the caller's contiguous rows: neighbouring workgroups then touch
// neighbouring 256-byte pieces of one row instead of pieces one row pitch
// apart, all at the same offset within the row.
__device__ __forceinline__ void tile_origin(const NsItem &it, int t, bool caller_tall, int64_t &i0, int64_t &j0) {
    if (caller_tall) {
        const int tm = (int)(it.mp / 64);
        i0 = (int64_t)(t % tm) * 64;
        j0 = (int64_t)(t / tm) * 64;
    } else {
        i0 = (int64_t)(t / it.tiles_n) * 64;
        j0 = (int64_t)(t % it.tiles_n) * 64;
    }
}

// Eight consecutive elements of a caller matrix at element index e, as
// fp32: n of them valid (0..8), zero beyond.  vec: the segment starts
// 16-byte aligned, so a full one moves with 16-byte accesses.
template <bool NT = false>
__device__ __forceinline__ void load_seg(const void *p, int64_t e, int dtype, int n, bool vec, float *v) {
    if (vec && n == 8) {
        if (dtype == QM_F32) {
            load8<NT>(static_cast<const float *>(p) + e, v);
        } else {
            const u32x4 w = ld16<NT>(static_cast<const uint16_t *>(p) + e);
            if (dtype == QM_BF16) {
                unpack8(w, v);
            } else {
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xffffu));
                    v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
                }
            }
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = k < n ? load_any(p, e + k, dtype) : 0.0f;
}
template <bool NT = false>
__device__ __forceinline__ void store_seg(void *p, int64_t e, int dtype, int n, bool vec, const float *v) {
    if (vec && n == 8) {
        if (dtype == QM_F32) {
            store8<NT>(static_cast<float *>(p) + e, v);
        } else if (dtype == QM_BF16) {
            store8<NT>(static_cast<bf16_t *>(p) + e, v);
        } else {
            u32x4 w;
#pragma unroll
            for (int k = 0; k < 4; k++)
                w[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * k]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * k + 1]) << 16);
            st16<NT>(static_cast<uint16_t *>(p) + e, w);
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; k++)
        if (k < n) store_any(p, e + k, dtype, v[k]);
}

// Valid length (0..8) of the segment at (row, col) of a rows x cols matrix.
__device__ __forceinline__ int seg_len(int64_t row, int64_t col, int64_t rows, int64_t cols) {
    if (row >= rows || col >= cols) return 0;
    return cols - col < 8 ? (int)(cols - col) : 8;
}

// Partial sums of squares: grid (kNormChunks, items); each workgroup covers
// a fixed slice of the item's rows, seen as a row-major list of 8-element
// segments; thread t adds segments t, t + 256, ... in order (four loads in
// flight), then a fixed combine order.
__global__ __launch_bounds__(256) void norm_partial_kernel(PrologueArgs a, double *partials) {
    const int item = blockIdx.y;
    const NsItem &it = a.it[item];
    if (it.inv) return;   // scale given (always so for a carrier source): nothing to sum
    const int64_t rows = it.tall ? it.n : it.m, cols = it.tall ? it.m : it.n;
    const int64_t per = (rows + kNormChunks - 1) / kNormChunks;
    const int64_t r0 = blockIdx.x * per, r1 = min(rows, r0 + per);
    const int64_t spr = (cols + 7) / 8;   // segments per row
    const int64_t nseg = r1 > r0 ? (r1 - r0) * spr : 0;
    double acc = 0.0;
    for (int64_t s0 = threadIdx.x; s0 < nseg; s0 += 4 * 256) {
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int64_t sg = s0 + u * 256;
            const int64_t r = r0 + sg / spr, c = (sg % spr) * 8;
            const int n = sg < nseg ? (int)min((int64_t)8, cols - c) : 0;
            load_seg(it.src, r * it.ld + c, it.dtype, n, it.vec, v[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int k = 0; k < 8; k++) acc += (double)v[u][k] * (double)v[u][k];
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

// Eight carrier elements (r, c .. c+7) of one 32-element block, as fp32:
// E4M3 byte (sign, 4 exponent bits biased by 7, 3 mantissa bits,
// subnormals k 2^-9, S.1111.111 NaN) times 2^(scale byte - 127).  gfx950's
// v_cvt_scalef32_pk_f32_fp8 decodes two bytes and applies the scale, given
// as an fp32, in one instruction; for every byte and every scale byte
// 0..254 its result has the bits of the field-by-field decode scaled with
// ldexp (an exhaustive comparison on gfx950; the carrier parity tests check
// the decode through the NS output).
__device__ __forceinline__ void load_mx8(const uint8_t *data, const uint8_t *sc, int64_t r, int64_t c, int64_t ld,
                                         int64_t sld, int n, float *v) {
    if (n == 0) {
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = 0.0f;
        return;
    }
    const uint2 w = *reinterpret_cast<const uint2 *>(data + r * ld + c);
    const float scale = ldexpf(1.0f, (int)sc[r * sld + c / 32] - 127);
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, scale, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, scale, true);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, scale, false);
    const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, scale, true);
    v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
    v[4] = d[0]; v[5] = d[1]; v[6] = e[0]; v[7] = e[1];
}

// X0 = orient(src) * inv, written as X (m_p x n_p) and, for fp32 runs, X^T
// (n_p x m_p), zero outside the valid extent.  One 64x64 tile per workgroup:
// each thread moves 8-element row segments (16-byte accesses where aligned),
// reading along the source's contiguous dimension; a tall source is
// transposed through LDS.
template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
    __shared__ float tile[64][65];
    const int item = find_item(a, blockIdx.x);
    const NsItem &it = a.it[item];
    int64_t i0, j0;
    tile_origin(it, blockIdx.x - it.tile_begin, it.tall, i0, j0);
    const float s = it.inv ? it.inv[0] : a.inv_ws[item];
    const int r = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;   // 32 rows x 8 segments per pass
    // source rows are rows of X, or of X^T when the source is tall
    const int64_t srows = it.tall ? it.n : it.m, scols = it.tall ? it.m : it.n;
    const int64_t sr0 = it.tall ? j0 : i0, sc0 = it.tall ? i0 : j0;
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
        const int rr = r + 32 * pass;
        const int64_t sr = sr0 + rr, sc = sc0 + c8;
        float v[8];
        const int n = seg_len(sr, sc, srows, scols);
        if (it.dtype == kSrcMx8)   // row length a multiple of 32: n is 0 or 8
            load_mx8(static_cast<const uint8_t *>(it.src), it.sc, sr, sc, it.ld, it.sld, n, v);
        else
            load_seg<true>(it.src, sr * it.ld + sc, it.dtype, n, it.vec, v);   // read once: non-temporal
#pragma unroll
        for (int k = 0; k < 8; k++) {
            if (it.tall) tile[c8 + k][rr] = v[k] * s;
            else tile[rr][c8 + k] = v[k] * s;
        }
    }
    __syncthreads();
    T *X = static_cast<T *>(it.X);
    T *XT = static_cast<T *>(it.XT);
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
        const int rr = r + 32 * pass;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = tile[rr][c8 + k];
        store8(X + (i0 + rr) * it.ldx + j0 + c8, v);
        if (XT) {
#pragma unroll
            for (int k = 0; k < 8; k++) v[k] = tile[c8 + k][rr];
            store8(XT + (j0 + rr) * it.ldxt + i0 + c8, v);
        }
    }
}

// Output of the iteration (X after the last product, or X0 when steps == 0)
// to the caller's matrix in its orientation and dtype, with the weight
// update W <- W - (lr s) O - (lr wd) W.  64x64 tiles through LDS; X is read
// and O and W are written as 8-element row segments.
struct WritebackArgs {
    FinalOut fo[kMaxItems];
};

template <typename T>
__global__ __launch_bounds__(256) void writeback_kernel(PrologueArgs a, WritebackArgs wb) {
    __shared__ float tile[64][65];
    const int item = find_item(a, blockIdx.x);
    const NsItem &it = a.it[item];
    const FinalOut &fo = wb.fo[item];
    int64_t i0, j0;
    tile_origin(it, blockIdx.x - it.tile_begin, fo.tall, i0, j0);
    const T *X = static_cast<const T *>(it.X);
    const int r = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;
    // caller rows are rows of X, or of X^T when the caller's matrix is tall
    const int64_t orows = fo.tall ? fo.n : fo.m, ocols = fo.tall ? fo.m : fo.n;
    const int64_t or0 = fo.tall ? j0 : i0, oc0 = fo.tall ? i0 : j0;
    // The weight segments do not depend on X: their loads are issued first,
    // so their latency overlaps that of X and the LDS transpose.  (Plain
    // accesses: non-temporal loads and stores made this kernel 5-10 %
    // slower on the 8B layer.)
    int n[2];
    float w[2][8];
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
        const int64_t orow = or0 + r + 32 * pass, oc = oc0 + c8;
        n[pass] = seg_len(orow, oc, orows, ocols);
        if (fo.w) load_seg(fo.w, orow * fo.ldw + oc, QM_F32, n[pass], fo.vec_w, w[pass]);
    }
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
        const int rr = r + 32 * pass;
        float v[8];
        load8(X + (i0 + rr) * it.ldx + j0 + c8, v);
#pragma unroll
        for (int k = 0; k < 8; k++) tile[rr][c8 + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
        const int rr = r + 32 * pass;
        const int64_t orow = or0 + rr, oc = oc0 + c8;
        if (n[pass] == 0) continue;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = fo.tall ? tile[c8 + k][rr] : tile[rr][c8 + k];
        store_seg(fo.out, orow * fo.ld + oc, fo.dtype, n[pass], fo.vec_out, v);
        if (fo.w) {
            float *wp = w[pass];
#pragma unroll
            for (int k = 0; k < 8; k++) wp[k] = wp[k] - (fo.lr_s * v[k] + fo.lr_wd * wp[k]);
            store_seg(fo.w, orow * fo.ldw + oc, QM_F32, n[pass], fo.vec_w, wp);
        }
    }
}

// ------------------------------------------------------------ host driver

struct NsRequest {
    const void *src;      // matrix start
    void *out;            // where the result goes (== src for in place)
    int64_t rows, cols, ld;
    int32_t dtype;        // of src (kSrcMx8: an MXFP8 carrier, inv required)
    int32_t out_dtype;    // of out
    const float *inv;     // nullable device scale
    float *w;             // nullable fp32 weights (rows x cols, ldw)
    int64_t ldw;
    float lr_s, lr_wd;
    const uint8_t *sc = nullptr;   // carrier scales and their row pitch
    int64_t sld = 0;
    int64_t out_ld = 0;            // row pitch of out; 0: ld
    int32_t src_t = 0;             // the source holds the transpose (cols x rows, pitch ld) of a tall matrix
};

// Row pitch of the internal operands: the padded width plus one 128-byte
// line, so that the rows one load instruction fetches (pitches that are
// multiples of 4 KiB otherwise) spread over the L2 channels instead of
// queueing on one.  The extra columns are never read.
constexpr int64_t kRowPadBytes = 128;

struct Geometry {
    int64_t m, n, mp, np;
    int64_t ldn, ldm;            // pitch (elements) of rows of length np / mp
    int64_t x_bytes, xt_bytes, a_bytes;  // X (mp x ldn), X^T (np x ldm), A (mp x ldm)
    int64_t item_bytes;          // X + XT0 + XT1 + A + B
};

Geometry geometry(int64_t rows, int64_t cols, size_t esz) {
    Geometry g;
    g.m = std::min(rows, cols);
    g.n = std::max(rows, cols);
    g.mp = pad_up(g.m);
    g.np = pad_up(g.n);
    g.ldn = g.np + kRowPadBytes / (int64_t)esz;
    g.ldm = g.mp + kRowPadBytes / (int64_t)esz;
    g.x_bytes = align_up(g.mp * g.ldn * (int64_t)esz, 256);
    g.xt_bytes = align_up(g.np * g.ldm * (int64_t)esz, 256);
    g.a_bytes = align_up(g.mp * g.ldm * (int64_t)esz, 256);
    // bf16 runs keep two X buffers (the product X = aX + BX reads X in its
    // K x N layout and writes the other); fp32 runs keep X and two X^T.
    g.item_bytes = esz == 2 ? 2 * g.x_bytes + 2 * g.a_bytes : g.x_bytes + 2 * g.xt_bytes + 2 * g.a_bytes;
    return g;
}

size_t elem_size(int precision) { return precision == QM_NS_BF16 ? 2 : 4; }

// Requests are processed in chunks of up to kMaxItems, largest first; the
// workspace holds the largest chunk plus the norm scratch.
std::vector<std::vector<size_t>> make_chunks(const std::vector<NsRequest> &req) {
    std::vector<size_t> order(req.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) {
        return req[x].rows * req[x].cols > req[y].rows * req[y].cols;
    });
    std::vector<std::vector<size_t>> chunks;
    for (size_t k = 0; k < order.size(); k += kMaxItems)
        chunks.emplace_back(order.begin() + k, order.begin() + std::min(order.size(), k + kMaxItems));
    return chunks;
}

constexpr int64_t kNormBytes = align_up_const(kMaxItems * kNormChunks * 8, 256) + align_up_const(kMaxItems * 4, 256);

int64_t sk_part_bytes(const std::vector<NsRequest> &req, const std::vector<size_t> &chunk, int precision);

size_t ns_ws_bytes_req(const std::vector<NsRequest> &req, int precision) {
    int64_t best = 0;
    for (const auto &ch : make_chunks(req)) {
        int64_t s = 0;
        for (size_t i : ch) s += geometry(req[i].rows, req[i].cols, elem_size(precision)).item_bytes;
        best = std::max(best, s + sk_part_bytes(req, ch, precision));
    }
    return (size_t)(best + kNormBytes);
}

size_t ns_ws_bytes_uniform(int64_t rows, int64_t cols, int64_t items, int precision) {
    std::vector<NsRequest> req((size_t)items);
    for (auto &r : req) {
        r.rows = rows;
        r.cols = cols;
    }
    return ns_ws_bytes_req(req, precision);
}

// Tile configurations: <BM, BN, waves_m, waves_n, row bytes per k-tile,
// LDS stages, workgroups per CU>.  The symmetric products need square tiles.
struct CfgSym {
    static constexpr int BM = 256, BN = 256, WM = 2, WN = 4, ROWB = 128, NST = 2, SLOTS = 5, MINB = 1;
};
struct CfgRect {
    static constexpr int BM = 256, BN = 256, WM = 2, WN = 4, ROWB = 128, NST = 2, SLOTS = 5, MINB = 1;
};
// fp32 runs on matrices too small to give every CU a 256 x 256 tile: the
// fp32 MFMA needs 16x fewer operand bytes per second than bf16, so smaller
// tiles cost little and keep all CUs busy (128 x 128: 4 waves of 64 x 64,
// two workgroups per CU; 64 x 64: 4 waves of 32 x 32, four per CU).
struct CfgF32Mid {
    static constexpr int BM = 128, BN = 128, WM = 2, WN = 2, ROWB = 128, NST = 2, SLOTS = 0, MINB = 2;
};
struct CfgF32Small {
    static constexpr int BM = 64, BN = 64, WM = 2, WN = 2, ROWB = 128, NST = 2, SLOTS = 0, MINB = 4;
};

// Per-device caches below are indexed by device ordinal; they are atomics
// because entry points may run on several host threads at once (the values
// written are the same whichever thread writes first).
constexpr int kMaxDevices = 64;

// Compute units of the current device (cached per device).
int64_t cu_count() {
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (done[] indexed by device; devices beyond the table are set on
// every call).
qm_status reserve_lds(const void *kern, size_t bytes, std::atomic<bool> *done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(QM_E_HIP, "no current device");
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached && done[dev].load(std::memory_order_acquire)) return QM_OK;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
        return fail(QM_E_HIP, "cannot reserve %zu bytes of LDS", bytes);
    if (cached) done[dev].store(true, std::memory_order_release);
    return QM_OK;
}

// Whether a symmetric launch deals its tiles by xcd_tile: only when it has
// more tiles than the GPU runs at once and its matrices differ in K.
// Measured: the Gram of the Llama-8B layer (700 tiles, K 14336 and 4096)
// ran 7 % faster; launches of a single round (MuonBP's block and full
// steps) ran 3-5 % slower than with tiles spread round robin, and so did
// X = aX + BX (equal K) by 1-2 %.
template <typename Args> bool use_xcd(const Args &args, int tiles, int per_cu) {
    bool k_differs = false;
    for (int i = 1; i < args.n_items; i++) k_differs |= args.it[i].k_tiles != args.it[0].k_tiles;
    return k_differs && tiles > cu_count() * per_cu;
}

// Grid for xcd_tile: 8 x the largest XCD total, i.e. the whole eighths of
// every item plus the extra tiles spread one per XCD.
template <typename Args> int xcd_grid(const Args &args, int total) {
    int64_t whole = 0, extra = 0;
    for (int i = 0; i < args.n_items; i++) {
        const int cnt = (i + 1 < args.n_items ? args.it[i + 1].tile_begin : total) - args.it[i].tile_begin;
        whole += cnt / 8;
        extra += cnt % 8;
    }
    return (int)(8 * (whole + (extra + 7) / 8));
}

template <typename T, typename C, int EPI, bool SYM, bool QT = false, bool X3 = false>
qm_status launch_gemm(GemmArgs<T> args, int tiles, hipStream_t stream) {
    constexpr int NT = C::WM * C::WN * 64;
    constexpr size_t lds = C::SLOTS ? (size_t)C::SLOTS * C::BM * C::ROWB : (size_t)C::NST * (C::BM + C::BN) * C::ROWB;
    auto kern = gemm_nt_kernel<T, C::BM, C::BN, C::WM, C::WN, C::ROWB, C::NST, C::SLOTS, C::MINB, EPI, SYM, QT, X3>;
    static std::atomic<bool> attr_set[kMaxDevices] = {};
    const qm_status st = reserve_lds(reinterpret_cast<const void *>(kern), lds, attr_set);
    if (st != QM_OK) return st;
    args.total_tiles = tiles;
    args.xcd = SYM && use_xcd(args, tiles, C::MINB) ? 1 : 0;
    const int grid = args.xcd ? xcd_grid(args, tiles) : tiles;
    Timed tm(stream, EPI == EPI_GRAM ? QM_K_NS_GRAM : EPI == EPI_POLY ? QM_K_NS_POLY : QM_K_NS_XUPDATE);
    launch(kern, dim3(grid), dim3(NT), lds, stream, args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    return QM_OK;
}

// Whether a launch of `tiles` tiles at per_cu workgroups per CU runs
// stream-K: it fills more than one round and leaves more than a tenth of
// its last round idle.  Used for fp32 symmetric products only, whose fp32
// MFMA work per tile is large against the 4 BM BN bytes a part moves.
bool sk_wanted(int64_t tiles, int per_cu) {
    const double r = (double)tiles / (double)(cu_count() * per_cu);
    return r > 1.0 && std::ceil(r) - r > 0.1;
}

template <typename T, typename C, int EPI, bool SYM, bool QT = false, bool X3 = false>
qm_status launch_gemm_sk(GemmArgs<T> args, int tiles, float *part, hipStream_t stream) {
    constexpr int NT = C::WM * C::WN * 64;
    constexpr size_t lds = C::SLOTS ? (size_t)C::SLOTS * C::BM * C::ROWB : (size_t)C::NST * (C::BM + C::BN) * C::ROWB;
    auto kern = gemm_sk_kernel<T, C::BM, C::BN, C::WM, C::WN, C::ROWB, C::NST, C::SLOTS, C::MINB, EPI, SYM, QT, X3>;
    auto fix = gemm_sk_fixup_kernel<T, C::BM, C::BN, C::WM, C::WN, C::ROWB, C::NST, C::SLOTS, C::MINB, EPI, SYM, QT, X3>;
    static std::atomic<bool> attr_set[kMaxDevices] = {}, attr_fix[kMaxDevices] = {};
    qm_status st = reserve_lds(reinterpret_cast<const void *>(kern), lds, attr_set);
    if (st == QM_OK) st = reserve_lds(reinterpret_cast<const void *>(fix), lds, attr_fix);
    if (st != QM_OK) return st;
    int64_t units = 0;
    for (int i = 0; i < args.n_items; i++) {
        GItem<T> &I = args.it[i];
        const int cnt = (i + 1 < args.n_items ? args.it[i + 1].tile_begin : tiles) - I.tile_begin;
        I.unit_begin = units;
        units += (int64_t)cnt * I.k_tiles;
    }
    const int64_t slots = cu_count() * C::MINB;
    args.total_tiles = tiles;
    args.xcd = 0;
    args.sk_units = units;
    args.sk_len = (units + slots - 1) / slots;
    args.sk_part = part;
    const int grid = (int)((units + args.sk_len - 1) / args.sk_len);   // <= slots: two part slots each
    Timed tm(stream, EPI == EPI_GRAM ? QM_K_NS_GRAM : EPI == EPI_POLY ? QM_K_NS_POLY : QM_K_NS_XUPDATE);
    launch(kern, dim3(grid), dim3(NT), lds, stream, args);
    if (grid > 1) launch(fix, dim3(grid - 1), dim3(NT), lds, stream, args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "stream-K gemm launch: %s", hipGetErrorString(e));
    return QM_OK;
}

qm_status launch_gram_mx(MxGramArgs args, int tiles, hipStream_t stream) {
    static std::atomic<bool> attr_set[kMaxDevices] = {};
    const qm_status st = reserve_lds(reinterpret_cast<const void *>(gram_mx_kernel), kMxGramLds, attr_set);
    if (st != QM_OK) return st;
    args.total_tiles = tiles;
    args.xcd = use_xcd(args, tiles, 1) ? 1 : 0;
    const int grid = args.xcd ? xcd_grid(args, tiles) : tiles;
    Timed tm(stream, QM_K_NS_GRAM);
    launch(gram_mx_kernel, dim3(grid), dim3(512), kMxGramLds, stream, args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "mx gram launch: %s", hipGetErrorString(e));
    return QM_OK;
}

// The first Gram product of a request can run on the carrier directly
// (gram_mx_kernel) when the request is a carrier iterated as it is (not
// tall), its rows a multiple of the 256-row tile, its K a multiple of the
// 128-byte k-tile, and the carrier rows and scale rows aligned for the
// 16-byte and 4-byte loads.
bool mx_gram_ok(const NsRequest &r) {
    // rows and K of the iterated matrix (the source as stored when it holds a transpose)
    const int64_t xr = r.src_t ? r.cols : r.rows, xc = r.src_t ? r.rows : r.cols;
    return r.dtype == kSrcMx8 && r.inv && xr <= xc && xr % 256 == 0 && xc % 128 == 0 && aligned(r.src, 16) &&
           r.ld % 16 == 0 && aligned(r.sc, 4) && r.sld % 4 == 0;
}

// bf16: X[0], X[1] ping-pong (X = aX + BX reads X in its K x N layout);
// fp32: X[0] updated in place, X^T in XT[0], XT[1] ping-pong.
struct ItemBufs {
    Geometry g;
    char *X[2] = {nullptr, nullptr};
    char *XT[2] = {nullptr, nullptr};
    char *A = nullptr, *B = nullptr;
};

// The T iterations of one chunk: A = X X^T, B = b A + c A A, X = a X + B X,
// with the symmetric products on tile configuration CS and the last on CR.
template <typename T, typename CS, typename CR, bool X3>
qm_status run_products(const std::vector<NsRequest> &req, const std::vector<size_t> &chunk,
                       const std::vector<ItemBufs> &bufs, const std::vector<int> &by_n, const std::vector<int> &by_m,
                       std::vector<int> &cur, int steps, float a, float b, float c, hipStream_t stream,
                       float *sk_part = nullptr) {
    const int nit = (int)chunk.size();
    constexpr bool kQT = sizeof(T) == 2;   // bf16: transposing reads, no X^T copy
    constexpr int64_t kSymK = CS::ROWB / (int64_t)sizeof(T);    // K elements per k-tile
    constexpr int64_t kRectK = CR::ROWB / (int64_t)sizeof(T);
    // stream-K symmetric products: fp32-operand runs (f32 and bf16x3) on the
    // 128 x 128 and 64 x 64 tiles
    constexpr bool kSk = sizeof(T) == 4 && CS::BM < 256;
    for (int s = 0; s < steps; s++) {
        // A = X X^T.  On the first iteration of a bf16 run whose requests
        // are all carriers that qualify, the block-scaled fp8 product runs
        // instead.  A chunk that mixes in other requests keeps one bf16
        // launch: two smaller launches back to back fill the GPU worse than
        // the fp8 product saves (measured on the 8B layer, whose tall gate
        // and up matrices cannot take it).
        bool all_mx = kQT && s == 0;
        for (int k = 0; k < nit; k++) all_mx = all_mx && mx_gram_ok(req[chunk[k]]);
        GemmArgs<T> g1{};
        MxGramArgs gx{};
        int tl = 0, tx = 0;
        for (int k = 0; k < nit; k++) {
            const ItemBufs &B = bufs[by_n[k]];
            const int tm = (int)(B.g.mp / CS::BM);
            const NsRequest &r = req[chunk[by_n[k]]];
            if (all_mx) {
                MxItem &M = gx.it[gx.n_items++];
                M.X = static_cast<const uint8_t *>(r.src);
                M.S = r.sc;
                M.C = reinterpret_cast<bf16_t *>(B.A);
                M.inv = r.inv;
                M.ldx = r.ld;
                M.lds = r.sld;
                M.ldc = B.g.ldm;
                M.tiles_m = tm;
                M.tile_begin = tx;
                M.k_tiles = (int32_t)((r.src_t ? r.rows : r.cols) / 128);
                tx += tm * (tm + 1) / 2;
                continue;
            }
            GItem<T> &I = g1.it[g1.n_items++];
            const char *X = kQT ? B.X[cur[by_n[k]]] : B.X[0];
            I.P = reinterpret_cast<const T *>(X); I.ldp = B.g.ldn;
            I.Q = reinterpret_cast<const T *>(X); I.ldq = B.g.ldn;
            I.C = reinterpret_cast<T *>(B.A); I.ldc = B.g.ldm;
            I.tiles_m = tm;
            I.tiles_n = tm;
            I.tile_begin = tl;
            I.k_tiles = (int32_t)(B.g.np / kSymK);
            tl += tm * (tm + 1) / 2;
        }
        qm_status st = QM_OK;
        if (g1.n_items) {
            if constexpr (kSk) {
                if (sk_part && sk_wanted(tl, CS::MINB)) st = launch_gemm_sk<T, CS, EPI_GRAM, true, false, X3>(g1, tl, sk_part, stream);
                else st = launch_gemm<T, CS, EPI_GRAM, true, false, X3>(g1, tl, stream);
            } else {
                st = launch_gemm<T, CS, EPI_GRAM, true, false, X3>(g1, tl, stream);
            }
        }
        if (st != QM_OK) return st;
        if (gx.n_items) st = launch_gram_mx(gx, tx, stream);
        if (st != QM_OK) return st;
        // B = b A + c A A
        GemmArgs<T> g2{};
        g2.n_items = nit;
        g2.alpha = b;
        g2.beta = c;
        g2.dloop = c != 0.0f;
        g2.dgain = c != 0.0f ? b / c : 0.0f;
        tl = 0;
        for (int k = 0; k < nit; k++) {
            const ItemBufs &B = bufs[by_m[k]];
            const int tm = (int)(B.g.mp / CS::BM);
            GItem<T> &I = g2.it[k];
            I.P = reinterpret_cast<const T *>(B.A); I.ldp = B.g.ldm;
            I.Q = reinterpret_cast<const T *>(B.A); I.ldq = B.g.ldm;
            I.C = reinterpret_cast<T *>(B.B); I.ldc = B.g.ldm;
            I.D = reinterpret_cast<const T *>(B.A); I.ldd = B.g.ldm;
            I.tiles_m = tm;
            I.tiles_n = tm;
            I.tile_begin = tl;
            I.k_tiles = (int32_t)(B.g.mp / kSymK);
            tl += tm * (tm + 1) / 2;
        }
        if constexpr (kSk) {
            if (sk_part && sk_wanted(tl, CS::MINB)) st = launch_gemm_sk<T, CS, EPI_POLY, true, false, X3>(g2, tl, sk_part, stream);
            else st = launch_gemm<T, CS, EPI_POLY, true, false, X3>(g2, tl, stream);
        } else {
            st = launch_gemm<T, CS, EPI_POLY, true, false, X3>(g2, tl, stream);
        }
        if (st != QM_OK) return st;
        // X = a X + B X: bf16 reads Q = X (K x N) and writes the other X
        // buffer; fp32 reads Q = X^T and updates X in place, writing X^T.
        GemmArgs<T> g3{};
        g3.n_items = nit;
        g3.alpha = a;
        g3.dloop = 1;
        g3.dgain = a;
        tl = 0;
        for (int k = 0; k < nit; k++) {
            const int i = by_m[k];
            const ItemBufs &B = bufs[i];
            const int tm = (int)(B.g.mp / CR::BM), tn = (int)(B.g.np / CR::BN);
            GItem<T> &I = g3.it[k];
            I.P = reinterpret_cast<const T *>(B.B); I.ldp = B.g.ldm;
            if constexpr (kQT) {
                I.Q = reinterpret_cast<const T *>(B.X[cur[i]]); I.ldq = B.g.ldn;
                I.C = reinterpret_cast<T *>(B.X[cur[i] ^ 1]); I.ldc = B.g.ldn;
                I.D = reinterpret_cast<const T *>(B.X[cur[i]]); I.ldd = B.g.ldn;
            } else {
                I.Q = reinterpret_cast<const T *>(B.XT[cur[i]]); I.ldq = B.g.ldm;
                I.C = reinterpret_cast<T *>(B.X[0]); I.ldc = B.g.ldn;
                I.CT = reinterpret_cast<T *>(B.XT[cur[i] ^ 1]); I.ldct = B.g.ldm;
                I.D = reinterpret_cast<const T *>(B.X[0]); I.ldd = B.g.ldn;
            }
            I.tiles_m = tm;
            I.tiles_n = tn;
            I.tile_begin = tl;
            I.k_tiles = (int32_t)(B.g.mp / kRectK);
            tl += tm * tn;
            if (s + 1 == steps) I.CT = nullptr;   // no further product reads X^T
        }
        st = launch_gemm<T, CR, EPI_UPDATE, false, kQT, X3>(g3, tl, stream);
        if (st != QM_OK) return st;
        for (int i = 0; i < nit; i++) cur[i] ^= 1;
    }
    return QM_OK;
}

// fp32 runs: the tile size of the symmetric products (sym) or of X = aX + BX
// from a model of the launch time: the tiles the busiest CU runs,
// ceil(tiles / CUs), x tile area / the tile's relative throughput (measured
// on the 4096-square NS: 256 x 256 0.76, 128 x 128 1, 64 x 64 0.94).  The
// fp32 MFMA needs 16x fewer operand bytes per second than bf16, so small
// tiles lose little, and a launch whose tiles do not fill the CUs evenly
// loses most of a round.  0: 256 x 256, 1: 128 x 128, 2: 64 x 64.
// bf16x3 runs (x3) take 128 x 128 when that gives every CU a tile, else
// 64 x 64: their tiles compute 2x faster, so the small tiles' overheads weigh
// more (64 x 64 ran at 0.54 - 0.87 of the 128 x 128 rate), and with 256 x 256
// tiles their fragments of 8 fp32 do not fit the registers.
int64_t tile_count(const std::vector<ItemBufs> &bufs, bool sym, int64_t s) {
    int64_t tiles = 0;
    for (const ItemBufs &b : bufs) {
        const int64_t tm = b.g.mp / s, tn = b.g.np / s;
        tiles += sym ? tm * (tm + 1) / 2 : tm * tn;
    }
    return tiles;
}
// fp32 symmetric launches of the 128 x 128 and 64 x 64 configurations run
// stream-K where sk_wanted says so; the model then counts their tiles as
// spread evenly over the CUs, plus 5 % for the parts and the fix-up.
constexpr int kF32Tile[3] = {256, 128, 64};
constexpr int kF32PerCu[3] = {1, 2, 4};
bool f32_sym_sk(const std::vector<ItemBufs> &bufs, int k) {
    return k > 0 && sk_wanted(tile_count(bufs, true, kF32Tile[k]), kF32PerCu[k]);
}
int pick_f32_tile(const std::vector<ItemBufs> &bufs, bool sym, bool x3) {
    static constexpr double kEff[3] = {0.76, 1.0, 0.94};
    const auto &kS = kF32Tile;
    const int64_t n_cu = cu_count();
    if (x3) return tile_count(bufs, sym, 128) >= n_cu ? 1 : 2;
    int best = 0;
    double best_t = 0;
    for (int k = 0; k < 3; k++) {
        const int64_t tiles = tile_count(bufs, sym, kS[k]);
        const double rounds = sym && f32_sym_sk(bufs, k) ? 1.05 * (double)tiles / (double)n_cu
                                                         : (double)((tiles + n_cu - 1) / n_cu);
        const double t = rounds * kS[k] * kS[k] / kEff[k];
        if (k == 0 || t < best_t) {
            best = k;
            best_t = t;
        }
    }
    return best;
}

// Bytes of stream-K parts a chunk needs: fp32-operand runs (f32, bf16x3)
// whose symmetric products run stream-K, two slots of 4 BM BN bytes per
// workgroup slot of the GPU.
int64_t sk_part_bytes(const std::vector<NsRequest> &req, const std::vector<size_t> &chunk, int precision) {
    if (precision != QM_NS_F32 && precision != QM_NS_BF16X3) return 0;
    std::vector<ItemBufs> bufs(chunk.size());
    for (size_t i = 0; i < chunk.size(); i++) bufs[i].g = geometry(req[chunk[i]].rows, req[chunk[i]].cols, 4);
    const int k = pick_f32_tile(bufs, true, precision == QM_NS_BF16X3);
    if (!f32_sym_sk(bufs, k)) return 0;
    return align_up(2 * cu_count() * kF32PerCu[k] * (int64_t)kF32Tile[k] * kF32Tile[k] * 4, 256);
}

// X3: fp32 runs on bf16x3 products (precision QM_NS_BF16X3).
template <typename T, bool X3 = false>
qm_status run_chunk(const std::vector<NsRequest> &req, const std::vector<size_t> &chunk, int steps, float a,
                    float b, float c, float eps, void *ws, hipStream_t stream) {
    const int nit = (int)chunk.size();
    constexpr bool kQT = sizeof(T) == 2;   // bf16: transposing reads, no X^T copy
    std::vector<ItemBufs> bufs(nit);
    char *p = static_cast<char *>(ws);
    for (int i = 0; i < nit; i++) {
        const NsRequest &r = req[chunk[i]];
        ItemBufs &B = bufs[i];
        B.g = geometry(r.rows, r.cols, sizeof(T));
        B.X[0] = p; p += B.g.x_bytes;
        if constexpr (kQT) {
            B.X[1] = p; p += B.g.x_bytes;
        } else {
            B.XT[0] = p; p += B.g.xt_bytes;
            B.XT[1] = p; p += B.g.xt_bytes;
        }
        B.A = p;   p += B.g.a_bytes;
        B.B = p;   p += B.g.a_bytes;
    }
    double *partials = reinterpret_cast<double *>(p);
    float *inv_ws = reinterpret_cast<float *>(p + align_up(kMaxItems * kNormChunks * 8, 256));
    // stream-K parts (fp32 runs whose symmetric products run stream-K)
    float *sk_part = sizeof(T) == 4 && sk_part_bytes(req, chunk, X3 ? QM_NS_BF16X3 : QM_NS_F32) > 0
                         ? reinterpret_cast<float *>(p + kNormBytes)
                         : nullptr;

    // ---- prologue: norms (if needed), orientation, padding, X and X^T
    PrologueArgs pa{};
    pa.n_items = nit;
    pa.inv_ws = inv_ws;
    bool need_norm = false;
    int tiles = 0;
    for (int i = 0; i < nit; i++) {
        const NsRequest &r = req[chunk[i]];
        const Geometry &g = bufs[i].g;
        NsItem &it = pa.it[i];
        it.src = r.src;
        it.ld = r.ld;
        it.sc = r.sc;
        it.sld = r.sld;
        it.dtype = r.dtype;
        it.vec = r.dtype != kSrcMx8 && aligned(r.src, 16) && (r.ld * (r.dtype == QM_F32 ? 4 : 2)) % 16 == 0 ? 1 : 0;
        it.tall = !r.src_t && r.rows > r.cols ? 1 : 0;   // a stored transpose is read as it is
        it.inv = r.inv;
        it.X = bufs[i].X[0];
        it.XT = bufs[i].XT[0];   // null for bf16
        it.m = (int32_t)g.m;
        it.n = (int32_t)g.n;
        it.mp = g.mp;
        it.np = g.np;
        it.ldx = g.ldn;
        it.ldxt = g.ldm;
        it.tiles_n = (int32_t)(g.np / 64);
        it.tile_begin = tiles;
        tiles += (int32_t)((g.mp / 64) * (g.np / 64));
        need_norm |= r.inv == nullptr;
    }
    if (need_norm) {
        Timed tm(stream, QM_K_NS_NORM);
        launch(norm_partial_kernel, dim3(kNormChunks, nit), 256, 0, stream, pa, partials);
        launch(norm_final_kernel, nit, 64, 0, stream, partials, eps, inv_ws);
    }
    {
        Timed tm(stream, QM_K_NS_PROLOGUE);
        launch(prologue_kernel<T>, tiles, 256, 0, stream, pa);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "prologue: %s", hipGetErrorString(e));

    FinalOut fo[kMaxItems];
    for (int i = 0; i < nit; i++) {
        const NsRequest &r = req[chunk[i]];
        const int64_t oesz = r.out_dtype == QM_F32 ? 4 : 2;
        const int64_t old_ = r.out_ld ? r.out_ld : r.ld;
        fo[i] = FinalOut{r.out, r.w, old_, r.ldw, r.out_dtype, r.rows > r.cols ? 1 : 0,
                         (int32_t)bufs[i].g.m, (int32_t)bufs[i].g.n, r.lr_s, r.lr_wd,
                         aligned(r.out, 16) && (old_ * oesz) % 16 == 0 ? 1 : 0,
                         r.w && aligned(r.w, 16) && (r.ldw * 4) % 16 == 0 ? 1 : 0};
    }
    WritebackArgs wb{};
    for (int i = 0; i < nit; i++) wb.fo[i] = fo[i];

    // Per-product item order: longest K first (all tiles of a matrix share K).
    std::vector<int> by_n(nit), by_m(nit);
    std::iota(by_n.begin(), by_n.end(), 0);
    std::iota(by_m.begin(), by_m.end(), 0);
    std::stable_sort(by_n.begin(), by_n.end(), [&](int x, int y) { return bufs[x].g.np > bufs[y].g.np; });
    std::stable_sort(by_m.begin(), by_m.end(), [&](int x, int y) {
        return bufs[x].g.mp * bufs[x].g.np > bufs[y].g.mp * bufs[y].g.np;
    });
    std::vector<int> cur(nit, 0);  // bf16: which X buffer is current; fp32: which X^T buffer
    qm_status st;
    if constexpr (sizeof(T) == 4) {
        const int ts = pick_f32_tile(bufs, true, X3), tr = pick_f32_tile(bufs, false, X3);
        auto run = [&](auto cs) -> qm_status {
            using CS = decltype(cs);
            if constexpr (!X3) {
                if (tr == 0)
                    return run_products<T, CS, CfgRect, X3>(req, chunk, bufs, by_n, by_m, cur, steps, a, b, c, stream, sk_part);
            }
            if (tr <= 1)
                return run_products<T, CS, CfgF32Mid, X3>(req, chunk, bufs, by_n, by_m, cur, steps, a, b, c, stream, sk_part);
            return run_products<T, CS, CfgF32Small, X3>(req, chunk, bufs, by_n, by_m, cur, steps, a, b, c, stream, sk_part);
        };
        if constexpr (X3) st = ts <= 1 ? run(CfgF32Mid{}) : run(CfgF32Small{});
        else st = ts == 0 ? run(CfgSym{}) : ts == 1 ? run(CfgF32Mid{}) : run(CfgF32Small{});
    } else {
        st = run_products<T, CfgSym, CfgRect, false>(req, chunk, bufs, by_n, by_m, cur, steps, a, b, c, stream);
    }
    if (st != QM_OK) return st;
    if constexpr (kQT)
        for (int i = 0; i < nit; i++) pa.it[i].X = bufs[i].X[cur[i]];
    {
        Timed tm(stream, QM_K_NS_WRITEBACK);
        launch(writeback_kernel<T>, tiles, 256, 0, stream, pa, wb);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return fail(QM_E_HIP, "writeback: %s", hipGetErrorString(e));
    return QM_OK;
}

qm_status run_ns(const std::vector<NsRequest> &req, int steps, float a, float b, float c, float eps,
                 int precision, void *ws, hipStream_t stream) {
    for (const auto &chunk : make_chunks(req)) {
        const qm_status st = precision == QM_NS_F32      ? run_chunk<float>(req, chunk, steps, a, b, c, eps, ws, stream)
                             : precision == QM_NS_BF16X3 ? run_chunk<float, true>(req, chunk, steps, a, b, c, eps, ws, stream)
                                                         : run_chunk<bf16_t>(req, chunk, steps, a, b, c, eps, ws, stream);
        if (st != QM_OK) return st;
    }
    return QM_OK;
}

qm_status check_ns_common(void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld, int32_t steps,
                          float a, float b, float c, float eps, int32_t precision) {
    if (!x) return fail(QM_E_ARG, "x is null");
    if (dtype != QM_F32 && dtype != QM_BF16 && dtype != QM_F16) return fail(QM_E_DTYPE, "unknown dtype %d", dtype);
    if (precision != QM_NS_BF16 && precision != QM_NS_F32 && precision != QM_NS_BF16X3)
        return fail(QM_E_ARG, "unknown precision %d", precision);
    if (rows <= 0 || cols <= 0) return fail(QM_E_SHAPE, "rows and cols must be positive");
    if (ld < cols) return fail(QM_E_SHAPE, "ld must be >= cols");
    if (std::min(rows, cols) > (1 << 16) || std::max(rows, cols) > (1 << 22))
        return fail(QM_E_UNSUPPORTED, "matrix too large");
    if (steps < 0 || steps > 100) return fail(QM_E_ARG, "steps must lie in [0, 100]");
    if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) return fail(QM_E_ARG, "coefficients must be finite");
    if (!(eps >= 0.0f) || std::isinf(eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    const uintptr_t esz = dtype == QM_F32 ? 4 : 2;
    if (!aligned(x, esz)) return fail(QM_E_ALIGN, "x misaligned for its dtype");
    return QM_OK;
}

}  // namespace

// Either fp32-operand mode (f32 or bf16x3); they may differ in stream-K part slots.
size_t ns_f32_workspace_bytes(int64_t rows, int64_t cols) {
    return std::max(ns_ws_bytes_uniform(rows, cols, 1, QM_NS_F32), ns_ws_bytes_uniform(rows, cols, 1, QM_NS_BF16X3));
}

qm_status run_ns_f32_into(const float *M, int64_t rows, int64_t cols, void *out, int32_t out_dtype, float *w,
                          float lr_s, float lr_wd, int steps, float a, float b, float c, float eps, int32_t precision,
                          void *ws, hipStream_t stream) {
    std::vector<NsRequest> req{NsRequest{M, out, rows, cols, cols, QM_F32, out_dtype, nullptr, w, cols, lr_s, lr_wd}};
    return run_ns(req, steps, a, b, c, eps, precision, ws, stream);
}

}  // namespace qm

using namespace qm;

extern "C" size_t ns_workspace_bytes(int64_t rows, int64_t cols, int32_t batch, int32_t precision) {
    if (rows <= 0 || cols <= 0 || batch <= 0) return 0;
    return ns_ws_bytes_uniform(rows, cols, batch, precision);
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
    const size_t need = ns_ws_bytes_uniform(rows, cols, batch, precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t esz = dtype == QM_F32 ? 4 : 2;
    std::vector<NsRequest> req;
    for (int32_t i = 0; i < batch; i++) {
        char *p = static_cast<char *>(x) + (size_t)i * (size_t)batch_stride * esz;
        req.push_back(NsRequest{p, p, rows, cols, ld, dtype, dtype, inv_norm ? inv_norm + i : nullptr, nullptr, 0,
                                0.0f, 0.0f});
    }
    return run_ns(req, steps, a, b, c, eps, precision, ws, static_cast<hipStream_t>(stream));
}

extern "C" qm_status ns_orthogonalize_mxfp8(const uint8_t *rowwise_data, const uint8_t *rowwise_scale_inv,
                                            const float *inv_norm, int64_t rows, int64_t cols, void *out,
                                            int32_t out_dtype, int64_t out_ld, int32_t steps, float a, float b,
                                            float c, int32_t precision, void *ws, size_t ws_bytes,
                                            qm_stream_t stream) {
    clear_error();
    qm_status st = check_ns_common(out, out_dtype, rows, cols, out_ld, steps, a, b, c, 0.0f, precision);
    if (st != QM_OK) return st;
    if (!rowwise_data || !rowwise_scale_inv) return fail(QM_E_ARG, "carrier arrays must not be null");
    if (!aligned(rowwise_data, 8)) return fail(QM_E_ALIGN, "carrier data must be 8-byte aligned");
    if (cols % 32) return fail(QM_E_SHAPE, "cols must be a multiple of the 32-element carrier block");
    if (!inv_norm || !aligned(inv_norm, 4)) return fail(QM_E_ARG, "inv_norm must be a 4-byte aligned device pointer");
    const size_t need = ns_ws_bytes_uniform(rows, cols, 1, precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    NsRequest r{rowwise_data, out, rows, cols, cols, kSrcMx8, out_dtype, inv_norm, nullptr, 0, 0.0f, 0.0f};
    r.sc = rowwise_scale_inv;
    r.sld = cols / 32;
    r.out_ld = out_ld;
    return run_ns(std::vector<NsRequest>{r}, steps, a, b, c, 0.0f, precision, ws, static_cast<hipStream_t>(stream));
}

extern "C" size_t ns_blocked_workspace_bytes(int64_t rows, int64_t cols, int64_t block_rows, int64_t block_cols,
                                             int32_t precision) {
    if (rows <= 0 || cols <= 0 || block_rows <= 0 || block_cols <= 0) return 0;
    if (rows % block_rows || cols % block_cols) return 0;
    return ns_ws_bytes_uniform(block_rows, block_cols, (rows / block_rows) * (cols / block_cols), precision);
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
    const size_t need = ns_ws_bytes_uniform(block_rows, block_cols, nbr * nbc, precision);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t esz = dtype == QM_F32 ? 4 : 2;
    std::vector<NsRequest> req;
    for (int64_t bi = 0; bi < nbr; bi++)
        for (int64_t bj = 0; bj < nbc; bj++) {
            char *p = static_cast<char *>(x) + ((size_t)(bi * block_rows) * (size_t)ld + (size_t)(bj * block_cols)) * esz;
            const float *inv = inv_norm ? inv_norm + bi * nbc + bj : nullptr;
            req.push_back(NsRequest{p, p, block_rows, block_cols, ld, dtype, dtype, inv, nullptr, 0, 0.0f, 0.0f});
        }
    return run_ns(req, steps, a, b, c, eps, precision, ws, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- muon step

namespace qm {
namespace {

// The NS work of one step: every matrix (full step) or every block.
// carrier: the MXFP8 carrier arrays of the plan (data, scales) the NS
// inputs are read from; null: the grads hold m.
struct CarrierIn {
    const uint8_t *data, *scale;
};

// Whether matrix i travels as the transposed carrier on this step: a tall
// matrix orthogonalised whole (a full step, or blocks the size of the
// matrix) with rows a multiple of 128 and cols of 256, so that the carrier
// of m^T feeds the block-scaled Gram along the matrix's rows.
bool transposed_carrier(const qm_muon_matrix &M, int32_t i, bool full) {
    const bool whole = full || (M.block_rows == M.rows && M.block_cols == M.cols);
    return whole && i < 64 && M.rows > M.cols && M.rows % 128 == 0 && M.cols % 256 == 0;
}

std::vector<NsRequest> step_requests(const PlanHeader *h, const void *host_plan, const qm_muon_matrix *mats,
                                     int32_t n, bool full, const float *inv, const qm_muon_hparams *hp,
                                     const CarrierIn *carrier = nullptr) {
    const PlanTensor *pt = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(host_plan) + h->off_tensors);
    std::vector<NsRequest> req;
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
        const int64_t gld = pt[i].grad_cols ? pt[i].grad_ld : M.cols;   // row pitch of the grad
        for (int64_t bi = 0; bi < nbr; bi++)
            for (int64_t bj = 0; bj < nbc; bj++) {
                const size_t goff = (size_t)(bi * br) * (size_t)gld + (size_t)(bj * bc);
                const size_t woff = (size_t)(bi * br) * (size_t)M.cols + (size_t)(bj * bc);
                const float *ip = inv ? inv + g0 + bi * nbc + bj : nullptr;
                req.push_back(NsRequest{grad + goff * esz, grad + goff * esz, br, bc, gld, dt, dt, ip,
                                        M.weight ? M.weight + woff : nullptr, M.cols, lr * s,
                                        lr * hp->weight_decay});
                if (carrier && transposed_carrier(M, i, full)) {
                    // the carrier of m^T: dense (cols, rows) bytes and (cols, rows / 32) scales
                    NsRequest &r = req.back();
                    const int64_t e0 = pt[i].block_offset * kBlock;
                    r.src = carrier->data + e0;
                    r.ld = M.rows;
                    r.dtype = kSrcMx8;
                    r.sc = carrier->scale + e0 / 32;
                    r.sld = M.rows / 32;
                    r.out_ld = gld;
                    r.src_t = 1;
                } else if (carrier) {   // dense (rows, cols) bytes and (rows, cols / 32) scales of tensor i
                    NsRequest &r = req.back();
                    const int64_t e0 = pt[i].block_offset * kBlock, e = (bi * br) * M.cols + bj * bc;
                    r.src = carrier->data + e0 + e;
                    r.ld = M.cols;
                    r.dtype = kSrcMx8;
                    r.sc = carrier->scale + (e0 + e) / 32;
                    r.sld = M.cols / 32;
                    r.out_ld = gld;
                }
            }
        g0 += nbr * nbc;
    }
    return req;
}

qm_status check_step_plan(const void *host_plan, const qm_muon_matrix *mats, int32_t n, bool full,
                          const PlanHeader **out, bool carrier = false) {
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
        if (pt[i].grad_cols != 0 && pt[i].grad_cols != M.cols)
            return fail(QM_E_SHAPE, "matrix %d: strided grad rows are not the matrix rows", i);
        const int64_t br = full ? M.rows : M.block_rows, bc = full ? M.cols : M.block_cols;
        if (br <= 0 || bc <= 0 || M.rows % br || M.cols % bc)
            return fail(QM_E_SHAPE, "matrix %d: blocks do not tile it", i);
        if (std::min(br, bc) > (1 << 16) || std::max(br, bc) > (1 << 22))
            return fail(QM_E_UNSUPPORTED, "matrix %d: too large", i);
        const int64_t nbc = M.cols / bc, nb = (M.rows / br) * nbc;
        if (pt[i].group_lo != g0 || pt[i].group_hi != g0 + nb - 1)
            return fail(QM_E_PLAN, "matrix %d: plan groups %d..%d, expected %lld..%lld", i, pt[i].group_lo,
                        pt[i].group_hi, (long long)g0, (long long)(g0 + nb - 1));
        if (nb > 1) {
            // Every NS block must be a union of whole 256-element quantisation
            // blocks (its norm group is a set of blocks), and the plan must give
            // quantisation block k the group of the NS block holding it, in
            // row-major block order: g0 + (r / br) nbc + c / bc.
            const bool whole = nbc == 1 ? (br * M.cols) % kBlock == 0 : M.cols % kBlock == 0 && bc % kBlock == 0;
            if (!whole)
                return fail(QM_E_SHAPE, "matrix %d: a 256-element quantisation block straddles two %lld x %lld blocks",
                            i, (long long)br, (long long)bc);
            const int32_t *bg = reinterpret_cast<const int32_t *>(static_cast<const char *>(host_plan) +
                                                                  h->off_block_group) + pt[i].block_offset;
            const int64_t nqb = (pt[i].numel + kBlock - 1) / kBlock;
            for (int64_t k = 0; k < nqb; k++) {
                const int64_t e = k * kBlock, r = e / M.cols, c = e % M.cols;
                const int64_t want = g0 + (r / br) * nbc + c / bc;
                if (bg[k] != want)
                    return fail(QM_E_PLAN, "matrix %d: quantisation block %lld is in group %d, its %lld x %lld block is %lld",
                                i, (long long)k, bg[k], (long long)br, (long long)bc, (long long)want);
            }
        }
        if (M.weight && !aligned(M.weight, 4)) return fail(QM_E_ALIGN, "matrix %d: weight misaligned", i);
        if (carrier && (M.cols % 32 || bc % 32))
            return fail(QM_E_SHAPE, "matrix %d: the MXFP8 carrier needs cols and block_cols multiples of 32", i);
        g0 += nb;
    }
    if (h->n_groups != g0) return fail(QM_E_PLAN, "plan has %d groups, expected %lld", h->n_groups, (long long)g0);
    *out = h;
    return QM_OK;
}

// The full-step and block-step plans of muon_step must describe the same
// tensors: the state of one step is the input of the next whichever plan
// updates it.
qm_status check_same_tensors(const void *plan_a, const void *plan_b) {
    qm_status st;
    const PlanHeader *ha = plan_header(plan_a, &st);
    if (!ha) return st;
    const PlanHeader *hb = plan_header(plan_b, &st);
    if (!hb) return st;
    if (ha->n_tensors != hb->n_tensors) return fail(QM_E_PLAN, "full and block plans differ in tensor count");
    const PlanTensor *a = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(plan_a) + ha->off_tensors);
    const PlanTensor *b = reinterpret_cast<const PlanTensor *>(static_cast<const char *>(plan_b) + hb->off_tensors);
    for (int32_t i = 0; i < ha->n_tensors; i++)
        if (a[i].codes != b[i].codes || a[i].absmax != b[i].absmax || a[i].grad != b[i].grad ||
            a[i].numel != b[i].numel || a[i].dtype != b[i].dtype || a[i].grad_cols != b[i].grad_cols ||
            (a[i].grad_cols && a[i].grad_ld != b[i].grad_ld))
            return fail(QM_E_PLAN, "tensor %d: the full and block plans point at different buffers", i);
    return QM_OK;
}

// Workspace: [update sums, norms][carrier data, scales (carrier mode)][NS].
int64_t carrier_ws_bytes(const PlanHeader *h) {
    return align_up(h->n_blocks * kBlock, 256) + align_up(h->n_blocks * (kBlock / 32), 256);
}

size_t step_ws_bytes(const PlanHeader *h, const void *host_plan, const qm_muon_matrix *mats, int32_t n,
                     bool full, int precision, bool carrier = false) {
    qm_muon_hparams dummy{};
    const auto req = step_requests(h, host_plan, mats, n, full, nullptr, &dummy);
    return align_up(qm_update_workspace_bytes(host_plan), 256) + (carrier ? carrier_ws_bytes(h) : 0) +
           ns_ws_bytes_req(req, precision);
}

size_t step_ws_total(const void *host_plan_full, const void *host_plan_block, const qm_muon_matrix *mats,
                     int32_t n_mats, int32_t precision, bool carrier) {
    if (!mats || n_mats <= 0) return 0;
    const PlanHeader *h = nullptr;
    if (check_step_plan(host_plan_full, mats, n_mats, true, &h, carrier) != QM_OK) return 0;
    size_t need = step_ws_bytes(h, host_plan_full, mats, n_mats, true, precision, carrier);
    if (host_plan_block) {
        if (check_step_plan(host_plan_block, mats, n_mats, false, &h, carrier) != QM_OK) return 0;
        if (check_same_tensors(host_plan_full, host_plan_block) != QM_OK) return 0;
        need = std::max(need, step_ws_bytes(h, host_plan_block, mats, n_mats, false, precision, carrier));
    }
    return need;
}

qm_status check_hparams(const qm_muon_hparams *hp) {
    if (!hp) return fail(QM_E_ARG, "hparams is null");
    if (hp->precision != QM_NS_BF16 && hp->precision != QM_NS_F32 && hp->precision != QM_NS_BF16X3)
        return fail(QM_E_ARG, "unknown precision");
    if (hp->ns_steps < 0 || hp->ns_steps > 100) return fail(QM_E_ARG, "ns_steps must lie in [0, 100]");
    if (!std::isfinite(hp->lr_full) || !std::isfinite(hp->lr_block) || !std::isfinite(hp->weight_decay) ||
        !std::isfinite(hp->rms_scale) || !std::isfinite(hp->a) || !std::isfinite(hp->b) || !std::isfinite(hp->c))
        return fail(QM_E_ARG, "hyperparameters must be finite");
    if (!(hp->eps >= 0.0f) || std::isinf(hp->eps)) return fail(QM_E_ARG, "eps must be finite and >= 0");
    if (hp->rounding != QM_ROUND_NEAREST && hp->rounding != QM_ROUND_STOCHASTIC)
        return fail(QM_E_ARG, "unknown rounding mode %d", hp->rounding);
    if (hp->carrier != 0 && hp->carrier != 1) return fail(QM_E_ARG, "carrier must be 0 or 1");
    if (hp->carrier && hp->rounding != QM_ROUND_NEAREST)
        return fail(QM_E_UNSUPPORTED, "the MXFP8 carrier update rounds to nearest only");
    return QM_OK;
}

// NS + weight apply of every matrix (full) or block, NS workspace at ns_ws.
qm_status apply_phase(const PlanHeader *h, const void *host_plan, const qm_muon_matrix *mats, int32_t n,
                      bool full, const float *inv, const qm_muon_hparams *hp, void *ns_ws, hipStream_t s,
                      const CarrierIn *carrier = nullptr) {
    const auto req = step_requests(h, host_plan, mats, n, full, inv, hp, carrier);
    return run_ns(req, hp->ns_steps, hp->a, hp->b, hp->c, hp->eps, hp->precision, ns_ws, s);
}

}  // namespace
}  // namespace qm

extern "C" size_t muon_step_workspace_bytes(const void *host_plan_full, const void *host_plan_block,
                                            const qm_muon_matrix *mats, int32_t n_mats, int32_t precision) {
    return step_ws_total(host_plan_full, host_plan_block, mats, n_mats, precision, false);
}

extern "C" size_t muon_step_workspace_bytes_ex(const void *host_plan_full, const void *host_plan_block,
                                               const qm_muon_matrix *mats, int32_t n_mats,
                                               const qm_muon_hparams *hp) {
    if (!hp) return 0;
    return step_ws_total(host_plan_full, host_plan_block, mats, n_mats, hp->precision, hp->carrier == 1);
}

extern "C" qm_status muon_apply(const void *host_plan, const qm_muon_matrix *mats, int32_t n_mats, int32_t full,
                                const float *inv_norm, const qm_muon_hparams *hp, void *ws, size_t ws_bytes,
                                qm_stream_t stream) {
    clear_error();
    qm_status st = check_hparams(hp);
    if (st != QM_OK) return st;
    if (!mats || n_mats <= 0) return fail(QM_E_ARG, "no matrices");
    if (full != 0 && full != 1) return fail(QM_E_ARG, "full must be 0 or 1");
    if (!inv_norm || !aligned(inv_norm, 4)) return fail(QM_E_ARG, "inv_norm must be a 4-byte aligned device pointer");
    if (hp->carrier) return fail(QM_E_UNSUPPORTED, "muon_apply reads m from the grads: carrier must be 0");
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
    const bool car = hp->carrier == 1;
    const void *hplan = full ? host_plan_full : host_plan_block;
    const void *dplan = full ? dev_plan_full : dev_plan_block;
    const PlanHeader *h = nullptr;
    st = validate_update(hplan, dplan, hp->beta, &h);
    if (st != QM_OK) return st;
    st = check_step_plan(hplan, mats, n_mats, full, &h, car);
    if (st != QM_OK) return st;
    if (host_plan_block) {
        const PlanHeader *hb = nullptr;
        if (full) {
            st = check_step_plan(host_plan_block, mats, n_mats, false, &hb, car);
            if (st != QM_OK) return st;
        }
        if ((st = check_same_tensors(host_plan_full, host_plan_block)) != QM_OK) return st;
    }
    const size_t need = step_ws_total(host_plan_full, host_plan_block, mats, n_mats, hp->precision, car);
    if (!ws || ws_bytes < need) return fail(QM_E_WORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QM_E_ALIGN, "workspace must be 256-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    char *p = static_cast<char *>(ws);
    const size_t upd = align_up(qm_update_workspace_bytes(hplan), 256);
    const UpdateWorkspace uw = update_workspace(h, ws);
    const qm_round_opts ro{hp->rounding, (uint32_t)step, hp->seed};
    if (!car) {
        st = run_update_normalize(h, dplan, hp->beta, hp->eps, false, nullptr, nullptr, ws, &ro, s);
        if (st != QM_OK) return st;
        return apply_phase(h, hplan, mats, n_mats, full, uw.inv, hp, p + upd, s);
    }
    uint8_t *cdata = reinterpret_cast<uint8_t *>(p + upd);
    uint8_t *cscale = cdata + align_up(h->n_blocks * kBlock, 256);
    if ((st = check_carrier(h, hplan, cdata, cscale)) != QM_OK) return st;
    std::vector<TallCarrier> tall;
    for (int32_t i = 0; i < n_mats; i++)
        if (transposed_carrier(mats[i], i, full)) tall.push_back(TallCarrier{i, mats[i].rows, mats[i].cols});
    st = run_update_normalize(h, dplan, hp->beta, hp->eps, false, nullptr, nullptr, ws, &ro, s, cdata, cscale, hplan,
                              tall.data(), (int)tall.size());
    if (st != QM_OK) return st;
    const CarrierIn cin{cdata, cscale};
    return apply_phase(h, hplan, mats, n_mats, full, uw.inv, hp, p + upd + carrier_ws_bytes(h), s, &cin);
}
