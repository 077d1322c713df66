"""ctypes declarations of libqmuon.so (the C ABI in include/qmuon.h).

The library is loaded from this package directory.  There is no fallback:
if it is missing, importing the package raises.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmuon.so")

QM_OK = 0
QM_ROUND_NEAREST, QM_ROUND_STOCHASTIC = 0, 1
STATUS_NAMES = {0: "QM_OK", 1: "QM_E_ARG", 2: "QM_E_ALIGN", 3: "QM_E_DTYPE",
                4: "QM_E_SHAPE", 5: "QM_E_WORKSPACE", 6: "QM_E_HIP",
                7: "QM_E_UNSUPPORTED", 8: "QM_E_PLAN"}
QM_F32, QM_BF16, QM_F16 = 0, 1, 2
QM_NS_BF16, QM_NS_F32, QM_NS_BF16X3 = 0, 1, 2
QM_NOALLOC_SCRATCH_BYTES = 64 << 20

c_void_p = ctypes.c_void_p
c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_f32 = ctypes.c_float
c_size = ctypes.c_size_t


class Q8Tensor(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("absmax", c_void_p), ("grad", c_void_p),
                ("numel", c_i64), ("grad_dtype", c_i32), ("reserved", c_i32),
                ("grad_cols", c_i64), ("grad_ld", c_i64)]


class NormSegment(ctypes.Structure):
    _fields_ = [("tensor_index", c_i32), ("group_id", c_i32),
                ("start", c_i64), ("length", c_i64)]


class MuonHparams(ctypes.Structure):
    _fields_ = [("beta", c_f32), ("eps", c_f32), ("a", c_f32), ("b", c_f32), ("c", c_f32),
                ("lr_full", c_f32), ("lr_block", c_f32), ("weight_decay", c_f32),
                ("rms_scale", c_f32), ("ns_steps", c_i32), ("period", c_i32),
                ("precision", c_i32), ("rounding", c_i32), ("carrier", c_i32),
                ("seed", ctypes.c_uint64)]


class RoundOpts(ctypes.Structure):
    _fields_ = [("rounding", c_i32), ("offset", ctypes.c_uint32), ("seed", ctypes.c_uint64)]


class MuonMatrix(ctypes.Structure):
    _fields_ = [("rows", c_i64), ("cols", c_i64), ("block_rows", c_i64),
                ("block_cols", c_i64), ("weight", c_void_p)]


class GraspStateC(ctypes.Structure):
    _fields_ = [("res_codes", c_void_p), ("res_rmax", c_void_p), ("res_cmax", c_void_p),
                ("p_codes", c_void_p), ("p_rmax", c_void_p), ("p_cmax", c_void_p),
                ("r_codes", c_void_p), ("r_rmax", c_void_p), ("r_cmax", c_void_p)]


# name -> (restype, argtypes); every symbol include/qmuon.h declares.
SIGNATURES = {
    "qm_plan_encode": (c_i32, [ctypes.POINTER(Q8Tensor), c_i32, ctypes.POINTER(NormSegment),
                               c_i32, c_i32, c_void_p, ctypes.POINTER(c_size)]),
    "qm_plan_info": (c_i32, [c_void_p, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32),
                             ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
    "qm_update_workspace_bytes": (c_size, [c_void_p]),
    "qmuon_update_multi": (c_i32, [c_void_p, c_void_p, c_f32, c_void_p, c_void_p]),
    "qmuon_update_normalize_groups": (c_i32, [c_void_p, c_void_p, c_f32, c_f32, c_i32,
                                              c_void_p, c_void_p, c_void_p, c_size, c_void_p]),
    "qmuon_update_multi_ex": (c_i32, [c_void_p, c_void_p, c_f32, ctypes.POINTER(RoundOpts), c_void_p,
                                      c_void_p]),
    "qmuon_update_normalize_groups_noalloc": (c_i32, [c_void_p, c_void_p, c_f32, c_f32, c_i32,
                                                       c_void_p, c_void_p, c_void_p]),
    "qmuon_update_normalize_groups_ex": (c_i32, [c_void_p, c_void_p, c_f32, c_f32, c_i32,
                                                 ctypes.POINTER(RoundOpts), c_void_p, c_void_p,
                                                 c_void_p, c_size, c_void_p]),
    "qmuon_update_mxfp8_carrier": (c_i32, [c_void_p, c_void_p, c_f32, c_f32, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_size, c_void_p]),
    "ns_orthogonalize_mxfp8": (c_i32, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_i32, c_i64,
                                       c_i32, c_f32, c_f32, c_f32, c_i32, c_void_p, c_size, c_void_p]),
    "muon_step_workspace_bytes_ex": (c_size, [c_void_p, c_void_p, ctypes.POINTER(MuonMatrix), c_i32,
                                              ctypes.POINTER(MuonHparams)]),
    "ns_workspace_bytes": (c_size, [c_i64, c_i64, c_i32, c_i32]),
    "ns_orthogonalize": (c_i32, [c_void_p, c_i32, c_i64, c_i64, c_i64, c_i32, c_i64, c_i32,
                                 c_f32, c_f32, c_f32, c_f32, c_void_p, c_i32, c_void_p,
                                 c_size, c_void_p]),
    "ns_blocked_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i64, c_i32]),
    "ns_orthogonalize_blocked": (c_i32, [c_void_p, c_i32, c_i64, c_i64, c_i64, c_i64, c_i64,
                                         c_i32, c_f32, c_f32, c_f32, c_f32, c_void_p, c_i32,
                                         c_void_p, c_size, c_void_p]),
    "muon_step_workspace_bytes": (c_size, [c_void_p, c_void_p, ctypes.POINTER(MuonMatrix),
                                           c_i32, c_i32]),
    "muon_step": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, ctypes.POINTER(MuonMatrix),
                          c_i32, c_i64, ctypes.POINTER(MuonHparams), c_void_p, c_size,
                          c_void_p]),
    "muon_apply": (c_i32, [c_void_p, ctypes.POINTER(MuonMatrix), c_i32, c_i32, c_void_p,
                           ctypes.POINTER(MuonHparams), c_void_p, c_size, c_void_p]),
    "grasp_workspace_bytes": (c_size, [c_i64, c_i64, c_i32]),
    "grasp_step": (c_i32, [ctypes.POINTER(GraspStateC), c_i64, c_i64, c_i32, c_i32, c_void_p, c_i32,
                           c_void_p, c_f32, c_i32, c_f32, c_f32, c_f32, c_f32, c_i32, c_void_p, c_f32, c_f32,
                           c_void_p, c_size, c_void_p]),
    "qm_timing_enable": (c_i32, [c_i32]),
    "qm_timing_read": (c_i32, [c_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]),
    "qm_hbm_stream_copy": (c_i32, [c_void_p, c_void_p, c_size, c_void_p]),
    "qm_status_string": (ctypes.c_char_p, [c_i32]),
    "qm_last_error": (ctypes.c_char_p, []),
    "qm_abi_version": (ctypes.c_int, []),
}


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
