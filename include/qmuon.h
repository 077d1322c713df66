/*
 * qmuon.h -- C ABI of libqmuon.so: one Muon optimizer step on an AMD MI355X
 * (gfx950), as a blockwise-int8 momentum update followed by quintic
 * Newton-Schulz orthogonalisation.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless a parameter says "host".
 *   - The caller owns every buffer (state, grads, weights, plan copies,
 *     workspace).  The library never allocates or frees device memory, never
 *     synchronises the stream and never prints.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  A call returns after enqueueing.
 *   - All arguments are validated on the host before anything is enqueued;
 *     on any validation error nothing is launched and no buffer is written.
 *     A launch failure returns QM_E_HIP; buffers may then be partly updated.
 *   - qm_last_error() gives a per-thread description of the last failure.
 *   - Calls that share buffers or workspace on one stream run in order; the
 *     same workspace must not be used by two streams at once.
 *   - Entry points may be called from several host threads at once, each
 *     with its own buffers, workspace and stream; results do not depend on
 *     what else runs (every reduction has one fixed order).
 */
#ifndef QMUON_H
#define QMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QM_ABI_VERSION 4
#define QM_BLOCK 256           /* quantisation block: elements per absmax */

typedef void *qm_stream_t;     /* hipStream_t */

#ifndef QM_API
#define QM_API __attribute__((visibility("default")))
#endif

typedef enum {
    QM_OK = 0,
    QM_E_ARG = 1,          /* null pointer, bad count, bad hyperparameter   */
    QM_E_ALIGN = 2,        /* pointer or segment alignment violated          */
    QM_E_DTYPE = 3,        /* unknown or unsupported dtype                   */
    QM_E_SHAPE = 4,        /* shapes inconsistent or not divisible           */
    QM_E_WORKSPACE = 5,    /* workspace missing or too small                 */
    QM_E_HIP = 6,          /* a HIP launch or runtime call failed            */
    QM_E_UNSUPPORTED = 7,  /* valid request outside what is implemented      */
    QM_E_PLAN = 8          /* plan blob malformed or of another version      */
} qm_status;

typedef enum { QM_F32 = 0, QM_BF16 = 1, QM_F16 = 2 } qm_dtype;

/* Newton-Schulz arithmetic: bf16 operands with fp32 accumulation (X, A, B
 * all held in bf16); fp32 operands with fp32 accumulation on fp32 MFMAs; or
 * fp32 operands held in fp32, each product formed on bf16 MFMAs from a
 * hi + lo split of both factors (hi = bf16(x), lo = bf16(x - hi); terms
 * hi hi' + hi lo' + lo hi', fp32 accumulation; the dropped lo lo' is below
 * 2^-16 of each product), "bf16x3". */
typedef enum { QM_NS_BF16 = 0, QM_NS_F32 = 1, QM_NS_BF16X3 = 2 } qm_ns_precision;

/* ------------------------------------------------------------------------
 * q8 momentum state and norm plans
 *
 * State of one tensor ("Quantized Muon Momentum", section "What Exists"):
 * `codes` of the tensor's size and one fp32 absmax per 256-element block
 * (the last block of a tensor covers the remainder).  Codes lie in
 * [-127, 127]; element i dequantises to codes[i] * (absmax[i/256] / 127).
 * The page allows int8 or uint8 storage for the codes; a uint8 buffer holds
 * the same two's-complement bytes (no offset), so both are passed here as
 * `codes`.  Blocks follow the tensor's logical (row-major) element order.
 *
 * The codes and absmax are contiguous.  The grad may be contiguous
 * (grad_cols = 0) or a 2-D view of numel / grad_cols rows of grad_cols
 * elements with row pitch grad_ld elements, e.g. one slice of a fused
 * buffer; the page lists "contiguous only" among the limitations of its
 * kernel ("Known Limitations").
 * ---------------------------------------------------------------------- */
typedef struct {
    int8_t *codes;      /* [numel] int8 (or uint8 bytes), 16-byte aligned,
                           in/out                                            */
    float *absmax;      /* [ceil(numel/256)], 4-byte aligned, in/out         */
    void *grad;         /* grad_dtype, 16-byte aligned; in: g, out: m
                           (optionally normalised)                           */
    int64_t numel;      /* > 0                                               */
    int32_t grad_dtype; /* qm_dtype                                          */
    int32_t reserved;   /* must be 0                                         */
    int64_t grad_cols;  /* 0: grad contiguous; else row length, a multiple
                           of 8 dividing numel                               */
    int64_t grad_ld;    /* grad_cols > 0: row pitch in elements, a multiple
                           of 8, >= grad_cols; ignored otherwise             */
} qm_q8_tensor;

/* One slice of a tensor assigned to a norm group ("Quantized Muon Momentum",
 * section "Grouped QKV And Sharding": fused Q, K and V use one group each).
 * `start` and `length` are element offsets into the flattened tensor.  A
 * segment starts on a 256-element boundary and ends on one unless it ends at
 * the tensor's last element.  Every block of every tensor must belong to
 * exactly one segment. */
typedef struct {
    int32_t tensor_index;
    int32_t group_id;   /* 0 .. n_groups-1                                   */
    int64_t start;
    int64_t length;
} qm_norm_segment;

/* Build a plan blob (host only; touches no GPU).  The blob records the
 * tensors' device pointers, one group id per block and the blocks of every
 * group; it is built once and reused for every step.  The caller copies the
 * bytes verbatim into device memory once (8-byte aligned) and passes both
 * copies to the update calls.
 *   host_blob == NULL: only *inout_blob_bytes is set to the size needed.
 *   Otherwise *inout_blob_bytes must be >= that size; it is set to the size
 *   written.
 * Errors: QM_E_ARG (null/counts/group ids), QM_E_ALIGN (pointer alignment or
 * segment boundaries), QM_E_SHAPE (overlap or an uncovered block), QM_E_DTYPE. */
QM_API qm_status qm_plan_encode(const qm_q8_tensor *tensors, int32_t n_tensors,
                         const qm_norm_segment *segments, int32_t n_segments,
                         int32_t n_groups, void *host_blob,
                         size_t *inout_blob_bytes);

/* Plan facts read back from a host blob (any out pointer may be NULL). */
QM_API qm_status qm_plan_info(const void *host_blob, int32_t *n_tensors,
                       int32_t *n_groups, int64_t *n_blocks,
                       int64_t *total_numel);

/* Workspace bytes qmuon_update_normalize_groups needs for this plan. */
QM_API size_t qm_update_workspace_bytes(const void *host_blob);

/* Requantisation rounding.  Nearest: round half to even.  Stochastic (the
 * page lists it under "Known Limitations" as not yet implemented; this is
 * the reading taken): x = m * (127 / absmax') as for nearest; the code is
 * floor(x) + 1 if u < x - floor(x), else floor(x), clamped to [-127, 127],
 * both operations in binary32; u = (r >> 8) * 2^-24 where r is word (e mod 4)
 * of Philox4x32-10 ("Parallel random numbers: as easy as 1, 2, 3", Salmon,
 * Moraes, Dror and Shaw, SC 2011) with counter (e / 4 low word, e / 4 high
 * word, offset, the tensor's index in the plan) and key (seed low word, seed
 * high word), e the element's index in its tensor.  The codes remain
 * bit-identical to a CPU run of the same definition. */
typedef enum { QM_ROUND_NEAREST = 0, QM_ROUND_STOCHASTIC = 1 } qm_rounding;

typedef struct {
    int32_t rounding;   /* qm_rounding                                        */
    uint32_t offset;    /* counter word 2 (e.g. the step number)              */
    uint64_t seed;      /* Philox key                                         */
} qm_round_opts;

/* In-place multi-tensor q8 update in one launch ("Quantized Muon Momentum",
 * sections "What Exists" and "Algorithm"): for every block of every tensor,
 * dequantise the old momentum in fp32, m = beta*old + (1-beta)*g (two
 * separately rounded products, one rounded sum), write m to the grad buffer
 * (round to nearest even into its dtype), absmax' = max|m| over the block,
 * codes' = clamp(rint(m * (127/absmax')), -127, 127), or codes 0 and absmax 0
 * for an all-zero block.  Codes and absmax are bit-identical to a CPU run of
 * the same IEEE binary32 operations.
 *   block_sumsq: nullable; if given, [n_blocks] fp64 receives each block's
 *   sum of m*m (fp32 m, fp64 accumulation), indexed by global block (tensors
 *   in plan order).
 * Errors: QM_E_ARG, QM_E_PLAN, QM_E_HIP. */
QM_API qm_status qmuon_update_multi(const void *host_plan, const void *dev_plan,
                             float beta, double *block_sumsq,
                             qm_stream_t stream);

/* qmuon_update_multi with the requantisation rounding chosen by `opts`
 * (nullable: nearest).  Errors: as qmuon_update_multi; QM_E_ARG for an
 * unknown rounding mode. */
QM_API qm_status qmuon_update_multi_ex(const void *host_plan, const void *dev_plan,
                                float beta, const qm_round_opts *opts,
                                double *block_sumsq, qm_stream_t stream);

/* The update plus grouped Frobenius normalisation ("Quantized Muon
 * Momentum", section "Grouped QKV And Sharding"): the update kernel
 * accumulates per-block sums of m*m; S_g sums them per group (fp64, fixed
 * order, no atomics); inv_g = (float)(1 / (sqrt(S_g) + eps)).
 *   write_normalized = 1: every grad element becomes
 *     round(float(m_stored) * inv_g) (the page's in-place semantics: the
 *     value an in-place scale of the stored m gives).  Run as two streaming
 *     passes: block sums of m first, then the update with the normalised
 *     value written in place of m (m recomputed bit for bit), so the grad
 *     buffer never holds the unnormalised m;
 *   write_normalized = 0: grads keep m and only inv_g is produced, for a
 *     Newton-Schulz call to fold in.
 *   group_inv_norm: nullable [n_groups] fp32 out.
 *   group_sumsq:    nullable [n_groups] fp64 out (S_g).
 *   ws: >= qm_update_workspace_bytes(host_plan) bytes, 256-byte aligned.
 * Errors: QM_E_ARG, QM_E_PLAN, QM_E_WORKSPACE, QM_E_HIP. */
QM_API qm_status qmuon_update_normalize_groups(const void *host_plan,
                                        const void *dev_plan, float beta,
                                        float eps, int32_t write_normalized,
                                        float *group_inv_norm,
                                        double *group_sumsq, void *ws,
                                        size_t ws_bytes, qm_stream_t stream);

/* qmuon_update_normalize_groups with the requantisation rounding chosen by
 * `opts` (nullable: nearest).  Errors: as qmuon_update_normalize_groups;
 * QM_E_ARG for an unknown rounding mode. */
QM_API qm_status qmuon_update_normalize_groups_ex(const void *host_plan,
                                           const void *dev_plan, float beta,
                                           float eps, int32_t write_normalized,
                                           const qm_round_opts *opts,
                                           float *group_inv_norm,
                                           double *group_sumsq, void *ws,
                                           size_t ws_bytes, qm_stream_t stream);

/* qmuon_update_normalize_groups without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The workspace is a fixed
 * QM_NOALLOC_SCRATCH_BYTES array in device memory, one per GPU, set up on
 * the first call on that GPU and held until the process ends; the call
 * itself allocates nothing.  Every call on one GPU uses the same array:
 * calls that overlap on one GPU (two streams, or two host threads) race and
 * must be ordered by the caller.  Nothing in the array needs to start at
 * zero; a call writes every byte it reads.  Semantics and outputs as
 * qmuon_update_normalize_groups with nearest rounding.
 * Errors: as qmuon_update_normalize_groups; QM_E_WORKSPACE when the plan
 * needs more than QM_NOALLOC_SCRATCH_BYTES (qm_update_workspace_bytes tells:
 * about 8 bytes per 256-element block, so up to about 2e9 elements). */
#define QM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
QM_API qm_status qmuon_update_normalize_groups_noalloc(const void *host_plan,
                                                       const void *dev_plan,
                                                       float beta, float eps,
                                                       int32_t write_normalized,
                                                       float *group_inv_norm,
                                                       double *group_sumsq,
                                                       qm_stream_t stream);

/* The update emitting a row-wise MXFP8 carrier of m instead of writing m
 * to the grads ("Quantized Muon Momentum", section "Wave18B MXFP8 Carrier
 * Probe": uint8 E4M3 data, uint8 E8M0 inverse scales per 32 elements of a
 * row, one fp32 inverse Frobenius norm).  State: as qmuon_update_multi
 * with nearest rounding; the grads are only read.  Per 32 consecutive
 * elements of a tensor: amax = max|m|, scale byte
 * sb = clamp(floor(log2 amax) - 8, -127, 127) + 127 (0 when amax == 0),
 * data bytes = E4M3 of m * 2^(127 - sb) rounded to nearest even and
 * saturated at +-448 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, no infinities); m ~ E4M3 * 2^(sb - 127).  inv_norm: as
 * group_inv_norm of qmuon_update_normalize_groups, the input scale of
 * Newton-Schulz being inv_norm[g] times the decoded carrier.
 *   Layout: both arrays cover every tensor of the plan; tensor t occupies
 *   data bytes [256 B_t, 256 B_t + numel_t) and scale bytes
 *   [8 B_t, 8 B_t + numel_t / 32), B_t = sum of ceil(numel_s / 256) over the
 *   tensors s before t.  A row-major rows x cols tensor with cols % 32 == 0
 *   therefore has data shaped (rows, cols) and scales (rows, cols / 32).
 *   rowwise_data:      [n_blocks * 256] bytes, 8-byte aligned.
 *   rowwise_scale_inv: [n_blocks * 8] bytes.
 *   inv_norm:          [n_groups] fp32 out, required.
 *   group_sumsq:       nullable [n_groups] fp64 out.
 *   ws: >= qm_update_workspace_bytes(host_plan) bytes, 256-byte aligned.
 * Every tensor's numel must be a multiple of 32 (else QM_E_SHAPE); the
 * carrier arrays must not overlap each other or any tensor's codes, absmax
 * or grad span (QM_E_ARG).  Errors: QM_E_ARG, QM_E_ALIGN, QM_E_SHAPE,
 * QM_E_PLAN, QM_E_WORKSPACE, QM_E_HIP. */
QM_API qm_status qmuon_update_mxfp8_carrier(const void *host_plan,
                                            const void *dev_plan, float beta,
                                            float eps, uint8_t *rowwise_data,
                                            uint8_t *rowwise_scale_inv,
                                            float *inv_norm,
                                            double *group_sumsq, void *ws,
                                            size_t ws_bytes, qm_stream_t stream);

/* ------------------------------------------------------------------------
 * Newton-Schulz orthogonalisation
 *
 * Per matrix X0 (rows x cols, row stride ld elements): if rows > cols the
 * iteration runs on X0^T so the Gram matrix is min(rows, cols) square
 * ("MuonBP ...", key design 1, FLOP model with m <= n).  X0 is the input
 * times inv_norm[i] when given, else the input / (||input||_F + eps).  Then
 * T times ("NVIDIA ... Megatron", "Newton-Schulz distribuido": three products
 * per iteration):   A = X X^T;  B = b A + c A A;  X = a X + B X.
 * The first two products are symmetric and computed on lower-triangle tiles
 * only ("SYRK y reducción fusionada").  The result overwrites x in its dtype.
 * ---------------------------------------------------------------------- */

/* Workspace bytes for ns_orthogonalize on `batch` matrices of this shape.
 * For the fp32-operand precisions (QM_NS_F32, QM_NS_BF16X3) the figure
 * includes, where the symmetric products take the stream-K path, two part
 * slots per workgroup slot of the GPU, so it depends on the compute-unit
 * count of the current device: query it with the device that will run the
 * call current (the same holds for the muon_step, muon_apply and GRASP
 * workspace queries). */
QM_API size_t ns_workspace_bytes(int64_t rows, int64_t cols, int32_t batch,
                          int32_t precision);

/*   x: batch matrices; matrix i starts at x + i*batch_stride elements;
 *      dtype QM_F32 / QM_BF16 / QM_F16; ld >= cols.
 *   inv_norm: nullable device fp32 [batch].
 *   precision: qm_ns_precision.  steps >= 0.
 *   ws: >= ns_workspace_bytes(rows, cols, batch, precision), 256-byte aligned.
 * Errors: QM_E_ARG, QM_E_SHAPE, QM_E_DTYPE, QM_E_WORKSPACE, QM_E_HIP. */
QM_API qm_status ns_orthogonalize(void *x, int32_t dtype, int64_t rows, int64_t cols,
                           int64_t ld, int32_t batch, int64_t batch_stride,
                           int32_t steps, float a, float b, float c, float eps,
                           const float *inv_norm, int32_t precision, void *ws,
                           size_t ws_bytes, qm_stream_t stream);

/* Blockwise NS ("MuonBP ...", key design 1; "NVIDIA ... Megatron", blockwise
 * mode): the rows x cols matrix is cut into (rows/block_rows) x
 * (cols/block_cols) blocks, each orthogonalised independently with its own
 * norm and orientation, all in one batched run.  inv_norm: nullable device
 * fp32 [number of blocks], row-major block order.
 * Errors: as ns_orthogonalize; QM_E_SHAPE if the blocks do not tile. */
QM_API size_t ns_blocked_workspace_bytes(int64_t rows, int64_t cols,
                                  int64_t block_rows, int64_t block_cols,
                                  int32_t precision);
QM_API qm_status ns_orthogonalize_blocked(void *x, int32_t dtype, int64_t rows,
                                   int64_t cols, int64_t ld,
                                   int64_t block_rows, int64_t block_cols,
                                   int32_t steps, float a, float b, float c,
                                   float eps, const float *inv_norm,
                                   int32_t precision, void *ws,
                                   size_t ws_bytes, qm_stream_t stream);

/* Newton-Schulz of one rows x cols matrix handed over as an MXFP8 carrier
 * ("Quantized Muon Momentum", section "Wave18B MXFP8 Carrier Probe"; the
 * carrier of qmuon_update_mxfp8_carrier): X0 = inv_norm[0] * decode(data,
 * scale), decode(r, c) = E4M3(rowwise_data[r * cols + c]) *
 * 2^(rowwise_scale_inv[r * (cols / 32) + c / 32] - 127), then the iteration
 * of ns_orthogonalize; O is written to out (rows x cols, row pitch out_ld
 * elements, out_dtype).
 *   rowwise_data: [rows * cols] bytes, 8-byte aligned; cols % 32 == 0.
 *   rowwise_scale_inv: [rows * cols / 32] bytes.  inv_norm: device fp32
 *   [1], required.  ws: >= ns_workspace_bytes(rows, cols, 1, precision).
 * Errors: as ns_orthogonalize. */
QM_API qm_status ns_orthogonalize_mxfp8(const uint8_t *rowwise_data,
                                        const uint8_t *rowwise_scale_inv,
                                        const float *inv_norm, int64_t rows,
                                        int64_t cols, void *out,
                                        int32_t out_dtype, int64_t out_ld,
                                        int32_t steps, float a, float b,
                                        float c, int32_t precision, void *ws,
                                        size_t ws_bytes, qm_stream_t stream);

/* ------------------------------------------------------------------------
 * One full optimizer step
 * ---------------------------------------------------------------------- */
typedef struct {
    float beta;          /* momentum EMA factor                              */
    float eps;           /* Frobenius-normalisation epsilon                  */
    float a, b, c;       /* quintic coefficients                             */
    float lr_full;       /* step size on full steps                          */
    float lr_block;      /* step size on block steps                         */
    float weight_decay;  /* lambda, decoupled                                */
    float rms_scale;     /* update scale = rms_scale * sqrt(max(p, q))       */
    int32_t ns_steps;    /* T                                                */
    int32_t period;      /* P: step t is full iff t % P == 0 (P <= 1: all)   */
    int32_t precision;   /* qm_ns_precision                                  */
    int32_t rounding;    /* qm_rounding of the requantisation; stochastic uses
                            the step number as the counter offset            */
    int32_t carrier;     /* 1: the update hands m to Newton-Schulz as the
                            MXFP8 carrier of qmuon_update_mxfp8_carrier (in
                            the workspace; grads only read until O is
                            written; nearest rounding; cols and block_cols
                            multiples of 32); a tall matrix orthogonalised
                            whole (rows > cols, rows % 128 == 0, cols % 256
                            == 0, among the first 64) travels instead as the
                            row-wise carrier of m^T (one scale per 32 rows of
                            a column), which the first Gram product reads
                            along its contraction; 0: m is written to the
                            grads */
    uint64_t seed;       /* Philox key for stochastic rounding               */
} qm_muon_hparams;

typedef struct {
    int64_t rows, cols;              /* tensor i of the plans, row-major       */
    int64_t block_rows, block_cols;  /* partition used on block steps        */
    float *weight;                   /* fp32 [rows*cols], nullable           */
} qm_muon_matrix;

/* Workspace for muon_step over these matrices (both step kinds), with
 * carrier = 0. */
QM_API size_t muon_step_workspace_bytes(const void *host_plan_full,
                                 const void *host_plan_block,
                                 const qm_muon_matrix *mats, int32_t n_mats,
                                 int32_t precision);

/* Workspace for muon_step with these hyperparameters: as above, plus
 * 264 bytes per 256-element block for the carrier when hp->carrier = 1.
 * 0 if the plans, matrices or hp are unusable. */
QM_API size_t muon_step_workspace_bytes_ex(const void *host_plan_full,
                                    const void *host_plan_block,
                                    const qm_muon_matrix *mats, int32_t n_mats,
                                    const qm_muon_hparams *hp);

/* One Muon step with block-periodic orthogonalisation ("MuonBP ...",
 * flowchart and key designs 2-3):
 *   full = (period <= 1) || (step % period == 0) || no block plan;
 *   the q8 update with plan_full (one norm group per matrix, group i =
 *   tensor i) or plan_block (one group per block, row-major block order,
 *   numbered consecutively across matrices);
 *   NS of every matrix (full) or of every block (block step), input
 *   m * inv_g, output written over the grad buffer in its dtype;
 *   W <- W - lr (s O + weight_decay W), lr = lr_full or lr_block,
 *   s = rms_scale * sqrt(max(p, q)) for the p x q matrix orthogonalised.
 * step is 1-based.  With more than one block per matrix, every block must
 * consist of whole 256-element quantisation blocks (cols and block_cols
 * multiples of 256, or one column block with block_rows * cols a multiple
 * of 256), else QM_E_SHAPE; the block plan must give each quantisation block
 * the group of the block holding it, and both plans must name the same
 * tensors (codes, absmax, grad, size, dtype), else QM_E_PLAN.
 * Errors: as the calls above. */
QM_API qm_status muon_step(const void *host_plan_full, const void *dev_plan_full,
                    const void *host_plan_block, const void *dev_plan_block,
                    const qm_muon_matrix *mats, int32_t n_mats, int64_t step,
                    const qm_muon_hparams *hp, void *ws, size_t ws_bytes,
                    qm_stream_t stream);

/* The orthogonalise-and-apply half of muon_step on its own: given the group
 * inverse norms inv_norm (device fp32 [n_groups of the plan], e.g. from
 * qmuon_update_normalize_groups with write_normalized = 0) and the grads
 * holding m, run NS on every matrix (full = 1) or every block (full = 0) of
 * the plan's tensors, write O over the grads and apply the weight update.
 * muon_step is qmuon_update_normalize_groups followed by this call.
 * ws: >= muon_step_workspace_bytes(...) bytes (the same workspace works).
 * Errors: as muon_step. */
QM_API qm_status muon_apply(const void *host_plan, const qm_muon_matrix *mats,
                            int32_t n_mats, int32_t full,
                            const float *inv_norm, const qm_muon_hparams *hp,
                            void *ws, size_t ws_bytes, qm_stream_t stream);

/* ------------------------------------------------------------------------
 * GRASP 4-bit momentum ("4-bit-Muon-GRASP")
 *
 * The momentum of one rows x cols matrix is a rank-k factor P R^T (P rows x
 * k, R cols x k, 8-bit) plus a residual (4-bit), all grid-quantised over
 * 64 x 64 blocks (clipped at the edges): an entry is divided by the smaller
 * of its row's and its column's absolute maximum inside its block, and coded
 * as clamp(rint((x / d) * L), -L, L), L = 7 (4-bit) or 127 (8-bit), d = 0
 * giving code 0; it dequantises to code * (d / L).  The state starts as all
 * zeros.  Layout (all caller-owned device buffers):
 * ---------------------------------------------------------------------- */
typedef struct {
    uint8_t *res_codes;  /* [rows][ceil(cols/2)]: two 4-bit two's-complement
                            codes per byte, even column in the low nibble   */
    float *res_rmax;     /* [rows][ceil(cols/64)] row maxima per block      */
    float *res_cmax;     /* [ceil(rows/64)][cols] column maxima per block   */
    int8_t *p_codes;     /* [rows][k]                                       */
    float *p_rmax;       /* [rows]                                          */
    float *p_cmax;       /* [ceil(rows/64)][k]                              */
    int8_t *r_codes;     /* [cols][k]                                       */
    float *r_rmax;       /* [cols]                                          */
    float *r_cmax;       /* [ceil(cols/64)][k]                              */
} qm_grasp_state;

QM_API size_t grasp_workspace_bytes(int64_t rows, int64_t cols, int32_t rank);

/* One GRASP step (the page's update equations):
 *   M_{t-1} = deq(res) + deq(P) deq(R)^T;   M_t = mu M_{t-1} + g (no (1-mu))
 *   Q = R_{t-1} with unit columns (a zero column is replaced by the same
 *   column of `warm`, cols x k fp32, normalised);  P = MGS(M_t Q) (modified
 *   Gram-Schmidt, positive diagonal);  R = M_t^T P;  residual M_t - P R^T;
 *   requantise residual, P, R;  O = NS_T(M_t) on fp32 operands (ns_precision
 *   QM_NS_F32 or QM_NS_BF16X3), written over grad in its dtype;
 *   W <- W - lr (O + weight_decay W) if weight.
 * Reductions accumulate in fp64 in a fixed order; P, R are rounded to fp32
 * before the residual.  rank in {1, 2, 4, 8, 16}; grid must be 64.
 *   grad: in g, out O (rows x cols contiguous, dtype grad_dtype).
 *   ws: >= grasp_workspace_bytes(rows, cols, rank), 256-byte aligned.
 * Errors: QM_E_ARG, QM_E_SHAPE, QM_E_DTYPE, QM_E_ALIGN, QM_E_UNSUPPORTED,
 * QM_E_WORKSPACE, QM_E_HIP. */
QM_API qm_status grasp_step(const qm_grasp_state *state, int64_t rows,
                            int64_t cols, int32_t rank, int32_t grid,
                            void *grad, int32_t grad_dtype, const float *warm,
                            float mu, int32_t ns_steps, float a, float b,
                            float c, float eps, int32_t ns_precision,
                            float *weight, float lr, float weight_decay,
                            void *ws, size_t ws_bytes, qm_stream_t stream);

/* ------------------------------------------------------------------------
 * Launch timing (measurement aid, off by default).
 *
 * While enabled, the launches of each class below carry two HIP events on
 * their dispatches (hipExtLaunchKernel: the start event on the first kernel
 * of the class's launch group, the stop event on its last), so a reader gets
 * the same per-launch device time a kernel-trace profiler reports.  The events
 * still cost the stream a few microseconds per launch group, so a caller
 * timing whole calls may record on some steps only (mode 2 below).  Enabling
 * clears earlier records unless resumed with mode 2; disabling keeps them for
 * qm_timing_read.  Not for use inside HIP graph capture.  The recorder is
 * process-wide and locked; launches from several threads are recorded but
 * interleave in one list.
 */
typedef enum {
    QM_K_Q8_UPDATE = 0,     /* blockwise q8 momentum update kernel */
    QM_K_GROUP_REDUCE = 1,  /* per-group sum of squares (both stages) */
    QM_K_Q8_SCALE = 2,      /* in-place normalisation pass: no longer launched (the
                             * normalising update writes normalised values itself) */
    QM_K_NS_NORM = 3,       /* Frobenius norm of NS inputs (both stages) */
    QM_K_NS_PROLOGUE = 4,   /* orientation, scaling, X and X^T */
    QM_K_NS_GRAM = 5,       /* A = X X^T (symmetric product) */
    QM_K_NS_POLY = 6,       /* B = b A + c A A (symmetric product) */
    QM_K_NS_XUPDATE = 7,    /* X = a X + B X */
    QM_K_NS_WRITEBACK = 8,  /* output and fused weight update */
    QM_K_Q8_SUMS = 9,       /* block sums of m only: first pass of the normalising update */
    QM_K_CLASSES = 10
} qm_kernel_class;

/* on == 1: clear records and start recording; on == 2: resume recording,
 * keeping the records so far; on == 0: stop.
 * Errors: QM_E_ARG (another value), QM_E_HIP (event creation failed). */
QM_API qm_status qm_timing_enable(int32_t on);

/* Sum of the recorded launch durations of one class (milliseconds) and the
 * number of launches.  Waits for the recorded events to complete.
 * Errors: QM_E_ARG (class out of range, null outputs), QM_E_HIP. */
QM_API qm_status qm_timing_read(int32_t kernel_class, double *total_ms,
                                int64_t *launches);

/* Measurement aid: copy `bytes` from src to dst (device pointers, 16-byte
 * aligned, bytes a multiple of 16, not overlapping) with the q8 update
 * kernel's access pattern (16-byte non-temporal loads and stores, each wave
 * instruction one contiguous 1 KiB span).  It gives the achievable HBM rate
 * for a 50/50 read/write stream, the ceiling the update kernels are measured
 * against, and a kernel of exactly known traffic to calibrate HBM byte
 * counters.  Errors: QM_E_ARG (null, overlap), QM_E_ALIGN, QM_E_HIP. */
QM_API qm_status qm_hbm_stream_copy(const void *src, void *dst, size_t bytes,
                                    qm_stream_t stream);

/* ------------------------------------------------------------------------ */
QM_API const char *qm_status_string(qm_status s);
QM_API const char *qm_last_error(void);
QM_API int qm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QMUON_H */
