"""Python binding of libqmuon.so: one quantized-momentum Muon step on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libqmuon.so.  PyTorch supplies device memory and the stream
(torch's current stream unless one is given).  There is no CPU or PyTorch
fallback; if the library is missing the import fails.

Entry points (same names as the C ABI in include/qmuon.h):
  Plan(...)                        qm_plan_encode + one host-to-device copy
  qmuon_update_multi               q8 momentum update, many tensors, one launch
  qmuon_update_normalize_groups    update + grouped Frobenius normalisation
  qmuon_update_normalize_groups_noalloc
                                   the same without a workspace (fixed per-GPU
                                   scratch; for callers that cannot allocate)
  MXCarrier, qmuon_update_mxfp8_carrier
                                   update emitting the MXFP8 carrier of m
  ns_orthogonalize_mxfp8           Newton-Schulz of a carrier-held matrix
  ns_orthogonalize                 quintic Newton-Schulz, batched
  ns_orthogonalize_blocked         blockwise Newton-Schulz
  muon_step                        update + NS + weight apply, block-periodic
  muon_apply                       the NS + weight-apply half of muon_step
  GraspState, grasp_step           the GRASP 4-bit momentum variant
  timing_enable, timing_read       per-kernel-class launch timing (HIP events)
"""
import ctypes

import torch

from . import _lib as L

_LIB = L.load()

QUINTIC = (3.4445, -4.7750, 2.0315)
BLOCK = 256      # elements per absmax block
PRECISION = {"bf16": L.QM_NS_BF16, "f32": L.QM_NS_F32, "bf16x3": L.QM_NS_BF16X3}
_DTYPES = {torch.float32: L.QM_F32, torch.bfloat16: L.QM_BF16, torch.float16: L.QM_F16}


class QmuonError(RuntimeError):
    def __init__(self, status):
        self.status = status
        name = L.STATUS_NAMES.get(status, str(status))
        msg = (_LIB.qm_last_error() or b"").decode()
        super().__init__(f"{name}: {msg}")


def _check(st):
    if st != L.QM_OK:
        raise QmuonError(st)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require(t, name, dtype, device, numel=None, shape=None):
    """Raise unless t is a contiguous `dtype` tensor on `device` with exactly
    `numel` elements / this shape (the C side reads that many elements at
    t.data_ptr())."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _dtype(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def abi_version():
    return _LIB.qm_abi_version()


# Kernel classes of qm_timing_read (qm_kernel_class in include/qmuon.h).
KERNEL_CLASSES = {"q8_update": 0, "group_reduce": 1, "q8_scale": 2, "ns_norm": 3, "ns_prologue": 4,
                  "ns_gram": 5, "ns_poly": 6, "ns_xupdate": 7, "ns_writeback": 8, "q8_sums": 9}


def timing_enable(on=True, resume=False):
    """Start (clearing earlier records), resume (keeping them) or stop
    recording launch times."""
    _check(_LIB.qm_timing_enable((2 if resume else 1) if on else 0))


def timing_read(kernel_class):
    """(total milliseconds, launches) recorded for one kernel class."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(_LIB.qm_timing_read(KERNEL_CLASSES[kernel_class], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class Plan:
    """A norm plan over q8 tensors, encoded once and copied to the device once.

    tensors : list of (codes, absmax fp32, grad) device tensors.  codes are int8,
              or uint8 holding the same bytes; codes and absmax contiguous.  grad
              is contiguous, or a 2-D view with unit column stride (rows of
              grad.shape[1] elements at pitch grad.stride(0)).
    segments: list of (tensor_index, start, length, group_id) element ranges
              (logical row-major element order)
    n_groups: number of norm groups
    """

    def __init__(self, tensors, segments, n_groups, device=None):
        n = len(tensors)
        arr = (L.Q8Tensor * n)()
        for i, (codes, absmax, grad) in enumerate(tensors):
            for t in (codes, absmax):
                if not t.is_contiguous():
                    raise ValueError("codes and absmax must be contiguous")
            if codes.dtype not in (torch.int8, torch.uint8):
                raise TypeError("codes must be int8 or uint8")
            cols, ld = 0, 0
            if not grad.is_contiguous():
                if grad.dim() != 2 or grad.stride(1) != 1:
                    raise ValueError("a non-contiguous grad must be 2-D with unit column stride")
                cols, ld = grad.shape[1], grad.stride(0)
            arr[i] = L.Q8Tensor(codes.data_ptr(), absmax.data_ptr(), grad.data_ptr(),
                                grad.numel(), _dtype(grad), 0, cols, ld)
        segs = (L.NormSegment * len(segments))()
        for k, (ti, start, length, gid) in enumerate(segments):
            segs[k] = L.NormSegment(ti, gid, start, length)
        size = ctypes.c_size_t(0)
        _check(_LIB.qm_plan_encode(arr, n, segs, len(segments), n_groups, None,
                                   ctypes.byref(size)))
        self.host = torch.empty(size.value, dtype=torch.uint8)
        _check(_LIB.qm_plan_encode(arr, n, segs, len(segments), n_groups,
                                   ctypes.c_void_p(self.host.data_ptr()), ctypes.byref(size)))
        dev = device if device is not None else tensors[0][0].device
        self.dev = self.host.to(dev)
        self._keep = [t for trip in tensors for t in trip]
        nt, ng = ctypes.c_int32(), ctypes.c_int32()
        nb, numel = ctypes.c_int64(), ctypes.c_int64()
        _check(_LIB.qm_plan_info(self.hptr, ctypes.byref(nt), ctypes.byref(ng),
                                 ctypes.byref(nb), ctypes.byref(numel)))
        self.n_tensors, self.n_groups = nt.value, ng.value
        self.n_blocks, self.total_numel = nb.value, numel.value
        self.device = dev
        # global index of each tensor's first 256-element block (plan order)
        self.numels = [int(t[2].numel()) for t in tensors]
        self.block_offsets = [0]
        for n_ in self.numels[:-1]:
            self.block_offsets.append(self.block_offsets[-1] + -(-n_ // BLOCK))

    @property
    def hptr(self):
        return ctypes.c_void_p(self.host.data_ptr())

    @property
    def dptr(self):
        return ctypes.c_void_p(self.dev.data_ptr())

    def workspace_bytes(self):
        return _LIB.qm_update_workspace_bytes(self.hptr)

    def workspace(self):
        return torch.empty(max(self.workspace_bytes(), 256), dtype=torch.uint8, device=self.device)


ROUNDING = {"nearest": L.QM_ROUND_NEAREST, "stochastic": L.QM_ROUND_STOCHASTIC}


def _round_opts(rounding, seed, offset):
    if rounding == "nearest":
        return None
    return ctypes.byref(L.RoundOpts(ROUNDING[rounding], offset, seed))


def qmuon_update_multi(plan, beta, block_sumsq=None, stream=None, rounding="nearest", seed=0, offset=0):
    """In-place q8 update of every tensor in the plan; block_sumsq (fp64
    [n_blocks]) optionally receives the per-block sums of m*m.  rounding:
    "nearest" or "stochastic" (random stream chosen by seed and offset)."""
    if rounding == "nearest":
        _check(_LIB.qmuon_update_multi(plan.hptr, plan.dptr, beta, _ptr(block_sumsq), _stream(stream)))
    else:
        _check(_LIB.qmuon_update_multi_ex(plan.hptr, plan.dptr, beta, _round_opts(rounding, seed, offset),
                                          _ptr(block_sumsq), _stream(stream)))


def qmuon_update_normalize_groups(plan, beta, eps, write_normalized=True, group_inv_norm=None,
                                  group_sumsq=None, ws=None, stream=None, rounding="nearest", seed=0,
                                  offset=0):
    if ws is None:
        ws = plan.workspace()
    if rounding == "nearest":
        _check(_LIB.qmuon_update_normalize_groups(
            plan.hptr, plan.dptr, beta, eps, int(write_normalized), _ptr(group_inv_norm),
            _ptr(group_sumsq), _ptr(ws), ws.numel(), _stream(stream)))
    else:
        _check(_LIB.qmuon_update_normalize_groups_ex(
            plan.hptr, plan.dptr, beta, eps, int(write_normalized), _round_opts(rounding, seed, offset),
            _ptr(group_inv_norm), _ptr(group_sumsq), _ptr(ws), ws.numel(), _stream(stream)))


def qmuon_update_normalize_groups_noalloc(plan, beta, eps, write_normalized=True, group_inv_norm=None,
                                          group_sumsq=None, stream=None):
    """qmuon_update_normalize_groups with the library's fixed per-GPU scratch
    instead of a workspace (the call allocates nothing).  Calls that overlap
    on one GPU race: order them.  Plans needing more than
    QM_NOALLOC_SCRATCH_BYTES of workspace are refused."""
    for t, dt, n in ((group_inv_norm, torch.float32, plan.n_groups), (group_sumsq, torch.float64, plan.n_groups)):
        if t is not None:
            _require(t, "group output", dt, plan.device, numel=n)
    _check(_LIB.qmuon_update_normalize_groups_noalloc(plan.hptr, plan.dptr, beta, eps, int(write_normalized),
                                                      _ptr(group_inv_norm), _ptr(group_sumsq), _stream(stream)))


class MXCarrier:
    """Row-wise MXFP8 carrier arrays covering every tensor of a plan (the
    layout qmuon_update_mxfp8_carrier writes): E4M3 bytes [n_blocks * 256],
    E8M0 scale bytes [n_blocks * 8], fp32 inverse norms [n_groups]."""

    def __init__(self, plan):
        self.plan = plan
        dev = plan.device
        self.rowwise_data = torch.empty(plan.n_blocks * BLOCK, dtype=torch.uint8, device=dev)
        self.rowwise_scale_inv = torch.empty(plan.n_blocks * (BLOCK // 32), dtype=torch.uint8, device=dev)
        self.inv_norm = torch.empty(plan.n_groups, dtype=torch.float32, device=dev)

    def data(self, i, shape=None):
        """Tensor i's E4M3 bytes (numel, or shaped (rows, cols))."""
        e0, n = self.plan.block_offsets[i] * BLOCK, self.plan.numels[i]
        v = self.rowwise_data[e0:e0 + n]
        return v.view(shape) if shape is not None else v

    def scale_inv(self, i, shape=None):
        """Tensor i's E8M0 bytes (numel / 32, or shaped (rows, cols / 32))."""
        e0, n = self.plan.block_offsets[i] * (BLOCK // 32), self.plan.numels[i] // 32
        v = self.rowwise_scale_inv[e0:e0 + n]
        return v.view(shape[0], shape[1] // 32) if shape is not None else v


def qmuon_update_mxfp8_carrier(plan, beta, eps, carrier=None, group_sumsq=None, ws=None, stream=None):
    """q8 update of every tensor in the plan emitting the MXFP8 carrier of m
    (and the group inverse norms into carrier.inv_norm); grads are only read.
    Returns the carrier."""
    if carrier is None:
        carrier = MXCarrier(plan)
    if ws is None:
        ws = plan.workspace()
    _check(_LIB.qmuon_update_mxfp8_carrier(plan.hptr, plan.dptr, beta, eps, _ptr(carrier.rowwise_data),
                                           _ptr(carrier.rowwise_scale_inv), _ptr(carrier.inv_norm),
                                           _ptr(group_sumsq), _ptr(ws), ws.numel(), _stream(stream)))
    return carrier


def ns_orthogonalize_mxfp8(data, scale_inv, inv_norm, out, steps=5, coeffs=QUINTIC, precision="bf16",
                           ws=None, stream=None):
    """NS of the rows x cols matrix carried as (data uint8 (rows, cols),
    scale_inv uint8 (rows, cols / 32), inv_norm fp32 [1]); O written to out
    (rows x cols, unit column stride, fp32/bf16/f16)."""
    rows, cols = out.shape
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    for t in (data, scale_inv):
        if not t.is_contiguous():
            raise ValueError("carrier arrays must be contiguous")
    if data.numel() != rows * cols or scale_inv.numel() * 32 != rows * cols:
        raise ValueError("carrier arrays do not match out's shape")
    prec = PRECISION[precision]
    if ws is None:
        ws = torch.empty(_LIB.ns_workspace_bytes(rows, cols, 1, prec), dtype=torch.uint8, device=out.device)
    a, b, c = coeffs
    _check(_LIB.ns_orthogonalize_mxfp8(_ptr(data), _ptr(scale_inv), _ptr(inv_norm), rows, cols, _ptr(out),
                                       _dtype(out), out.stride(0), steps, a, b, c, prec, _ptr(ws), ws.numel(),
                                       _stream(stream)))


def _matrix_args(x):
    if x.dim() == 2:
        rows, cols = x.shape
        if x.stride(1) != 1:
            raise ValueError("rows must be contiguous")
        return 1, rows, cols, x.stride(0), 0
    if x.dim() == 3:
        b, rows, cols = x.shape
        if x.stride(2) != 1:
            raise ValueError("rows must be contiguous")
        return b, rows, cols, x.stride(1), x.stride(0)
    raise ValueError("expected a 2-D matrix or a 3-D batch of matrices")


def ns_workspace_bytes(rows, cols, batch=1, precision="bf16"):
    return _LIB.ns_workspace_bytes(rows, cols, batch, PRECISION[precision])


def ns_orthogonalize(x, steps=5, coeffs=QUINTIC, eps=1e-7, inv_norm=None, precision="bf16",
                     ws=None, stream=None):
    """Overwrite x (rows x cols, or batch x rows x cols) with NS_T(x)."""
    batch, rows, cols, ld, bstride = _matrix_args(x)
    prec = PRECISION[precision]
    if ws is None:
        ws = torch.empty(_LIB.ns_workspace_bytes(rows, cols, batch, prec), dtype=torch.uint8,
                         device=x.device)
    a, b, c = coeffs
    _check(_LIB.ns_orthogonalize(_ptr(x), _dtype(x), rows, cols, ld, batch, bstride, steps, a, b, c,
                                 eps, _ptr(inv_norm), prec, _ptr(ws), ws.numel(), _stream(stream)))


def ns_orthogonalize_blocked(x, block_rows, block_cols, steps=5, coeffs=QUINTIC, eps=1e-7,
                             inv_norm=None, precision="bf16", ws=None, stream=None):
    """Overwrite every block_rows x block_cols block of x with its own NS."""
    _, rows, cols, ld, _ = _matrix_args(x)
    prec = PRECISION[precision]
    if ws is None:
        ws = torch.empty(_LIB.ns_blocked_workspace_bytes(rows, cols, block_rows, block_cols, prec),
                         dtype=torch.uint8, device=x.device)
    a, b, c = coeffs
    _check(_LIB.ns_orthogonalize_blocked(_ptr(x), _dtype(x), rows, cols, ld, block_rows, block_cols,
                                         steps, a, b, c, eps, _ptr(inv_norm), prec, _ptr(ws),
                                         ws.numel(), _stream(stream)))


def make_hparams(beta=0.95, eps=1e-7, coeffs=QUINTIC, lr_full=0.02, lr_block=0.01,
                 weight_decay=0.0, rms_scale=0.2, ns_steps=5, period=5, precision="bf16",
                 rounding="nearest", seed=0, carrier=False):
    a, b, c = coeffs
    return L.MuonHparams(beta, eps, a, b, c, lr_full, lr_block, weight_decay, rms_scale,
                         ns_steps, period, PRECISION[precision], ROUNDING[rounding], int(carrier), seed)


def _matrices(mats, device):
    """qm_muon_matrix array; each weight (optional) must be a contiguous fp32
    tensor of rows x cols elements on the plan's device."""
    arr = (L.MuonMatrix * len(mats))()
    for i, (rows, cols, br, bc, w) in enumerate(mats):
        if w is not None:
            _require(w, f"weight {i}", torch.float32, device, numel=rows * cols)
        arr[i] = L.MuonMatrix(rows, cols, br, bc, w.data_ptr() if w is not None else None)
    return arr


def muon_step_workspace_bytes(plan_full, plan_block, mats, precision="bf16", hparams=None):
    arr = _matrices(mats, plan_full.device)
    if hparams is not None:
        return _LIB.muon_step_workspace_bytes_ex(plan_full.hptr, plan_block.hptr if plan_block else None,
                                                 arr, len(mats), ctypes.byref(hparams))
    return _LIB.muon_step_workspace_bytes(plan_full.hptr, plan_block.hptr if plan_block else None,
                                          arr, len(mats), PRECISION[precision])


def muon_step(plan_full, plan_block, mats, step, hparams, ws=None, stream=None):
    """One block-periodic Muon step.  mats: list of (rows, cols, block_rows,
    block_cols, weight fp32 tensor or None), tensor i of both plans."""
    arr = _matrices(mats, plan_full.device)
    if ws is None:
        nbytes = _LIB.muon_step_workspace_bytes_ex(plan_full.hptr,
                                                   plan_block.hptr if plan_block else None,
                                                   arr, len(mats), ctypes.byref(hparams))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=plan_full.device)
    _check(_LIB.muon_step(plan_full.hptr, plan_full.dptr,
                          plan_block.hptr if plan_block else None,
                          plan_block.dptr if plan_block else None,
                          arr, len(mats), step, ctypes.byref(hparams), _ptr(ws), ws.numel(),
                          _stream(stream)))


def muon_apply(plan, mats, full, inv_norm, hparams, ws, stream=None):
    """NS + weight apply for the plan's matrices given group inverse norms
    (device fp32 [plan.n_groups]); muon_step = update + this."""
    _require(inv_norm, "inv_norm", torch.float32, plan.device, numel=plan.n_groups)
    arr = _matrices(mats, plan.device)
    _check(_LIB.muon_apply(plan.hptr, arr, len(mats), int(full), _ptr(inv_norm),
                           ctypes.byref(hparams), _ptr(ws), ws.numel(), _stream(stream)))


def hbm_stream_copy(src, dst, stream=None):
    """Measurement aid: copy src into dst (same byte size, contiguous, 16-byte
    aligned) with the update kernels' access pattern."""
    for t in (src, dst):
        if not t.is_contiguous():
            raise ValueError("stream copy operands must be contiguous")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("stream copy operands differ in size")
    _check(_LIB.qm_hbm_stream_copy(_ptr(src), _ptr(dst), n, _stream(stream)))


GRASP_GRID = 64


class GraspState:
    """Zero-initialised GRASP state buffers of one rows x cols matrix (the
    layout of qm_grasp_state)."""

    def __init__(self, rows, cols, rank, device="cuda"):
        nbr, nbc = -(-rows // GRASP_GRID), -(-cols // GRASP_GRID)
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.rows, self.cols, self.rank = rows, cols, rank
        self.res_codes = z((rows, (cols + 1) // 2), torch.uint8)
        self.res_rmax = z((rows, nbc), torch.float32)
        self.res_cmax = z((nbr, cols), torch.float32)
        self.p_codes = z((rows, rank), torch.int8)
        self.p_rmax = z((rows,), torch.float32)
        self.p_cmax = z((nbr, rank), torch.float32)
        self.r_codes = z((cols, rank), torch.int8)
        self.r_rmax = z((cols,), torch.float32)
        self.r_cmax = z((nbc, rank), torch.float32)

    def c_struct(self):
        return L.GraspStateC(*(t.data_ptr() for t in (
            self.res_codes, self.res_rmax, self.res_cmax, self.p_codes, self.p_rmax, self.p_cmax,
            self.r_codes, self.r_rmax, self.r_cmax)))


def grasp_workspace_bytes(rows, cols, rank):
    return _LIB.grasp_workspace_bytes(rows, cols, rank)


def grasp_step(state, grad, warm, mu=0.95, ns_steps=5, coeffs=QUINTIC, eps=1e-7, weight=None,
               lr=0.02, weight_decay=0.0, ws=None, stream=None, ns_precision="f32"):
    """One GRASP step: state updated in place, grad (in: g) overwritten with
    O = NS(M_t), weight (optional) updated.  ns_precision: "f32" (fp32
    MFMAs) or "bf16x3" (fp32 operands, products from a bf16 hi + lo split)."""
    if grad.dim() != 2:
        raise ValueError("grad must be a 2-D matrix")
    rows, cols = grad.shape
    _require(grad, "grad", grad.dtype, grad.device)
    _dtype(grad)
    if (state.rows, state.cols) != (rows, cols):
        raise ValueError(f"state is {state.rows} x {state.cols}, grad {rows} x {cols}")
    _require(warm, "warm", torch.float32, grad.device, shape=(cols, state.rank))
    if weight is not None:
        _require(weight, "weight", torch.float32, grad.device, numel=rows * cols)
    if ws is None:
        ws = torch.empty(_LIB.grasp_workspace_bytes(rows, cols, state.rank), dtype=torch.uint8,
                         device=grad.device)
    a, b, c = coeffs
    st = state.c_struct()
    _check(_LIB.grasp_step(ctypes.byref(st), rows, cols, state.rank, GRASP_GRID, _ptr(grad),
                           _dtype(grad), _ptr(warm), mu, ns_steps, a, b, c, eps, PRECISION[ns_precision],
                           _ptr(weight), lr,
                           weight_decay, _ptr(ws), ws.numel(), _stream(stream)))
