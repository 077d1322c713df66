"""CPU oracle for the quantized-momentum Muon step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and the product path never calls it.

Parts:
  * q8 momentum update, group sums and the scale pass: plain C in q8.c
    (binary32 with the exact operation order, fp64 sums), wrapped here;
  * norm plans: expansion of norm segments into one group id per block;
  * Newton-Schulz, blocked Newton-Schulz and the block-periodic schedule:
    fp64 numpy in ns.py / muonbp.py;
  * the GRASP 4-bit momentum step: grasp.py.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BLOCK = 256
F32, BF16, F16 = 0, 1, 2

_lib = None


def lib():
    """Load liboracle.so, compiling it first if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.or_bf16_from_f32.argtypes = [ctypes.c_float]
        L.or_bf16_from_f32.restype = ctypes.c_uint16
        L.or_f16_from_f32.argtypes = [ctypes.c_float]
        L.or_f16_from_f32.restype = ctypes.c_uint16
        L.or_q8_update.argtypes = [p, p, p, ctypes.c_int, i64, ctypes.c_float, p]
        L.or_q8_update_ex.argtypes = [p, p, p, ctypes.c_int, i64, ctypes.c_float, p, ctypes.c_int,
                                      ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        L.or_philox4x32_10.argtypes = [p, p, p]
        L.or_e4m3_from_f32.argtypes = [ctypes.c_float]
        L.or_e4m3_from_f32.restype = ctypes.c_uint8
        L.or_f32_from_e4m3.argtypes = [ctypes.c_uint8]
        L.or_f32_from_e4m3.restype = ctypes.c_float
        L.or_mx_scale_byte.argtypes = [ctypes.c_float]
        L.or_mx_scale_byte.restype = ctypes.c_uint8
        L.or_q8_update_carrier.argtypes = [p, p, p, ctypes.c_int, i64, ctypes.c_float, p, p, p]
        L.or_q8_update_carrier_t.argtypes = [p, p, p, ctypes.c_int, i64, i64, ctypes.c_float, p, p, p]
        L.or_q8_update.restype = None
        L.or_group_sums.argtypes = [p, p, i64, ctypes.c_int32, p]
        L.or_group_inv_norm.argtypes = [p, ctypes.c_int32, ctypes.c_float, p]
        L.or_scale_by_group.argtypes = [p, ctypes.c_int, i64, p, p]
        L.or_round_array.argtypes = [p, i64, ctypes.c_int, p]
        L.or_widen_array.argtypes = [p, i64, ctypes.c_int, p]
        L.or_num_threads.argtypes = []
        L.or_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _grad_dtype(a):
    if a.dtype == np.float32:
        return F32
    raise TypeError("pass fp32 arrays directly; 16-bit grads as (uint16 bits, dtype)")


def num_threads():
    """OpenMP threads the C oracle runs with."""
    return lib().or_num_threads()


# ------------------------------------------------------------------ dtypes

def round_to(x, dtype):
    """fp32 array -> uint16 bit patterns of bf16 (dtype=BF16) or f16 (F16), RNE."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_round_array(_ptr(x), x.size, dtype, _ptr(out))
    return out


def widen(bits, dtype):
    """uint16 bit patterns of bf16/f16 -> fp32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().or_widen_array(_ptr(bits), bits.size, dtype, _ptr(out))
    return out


# --------------------------------------------------------------- q8 update

ROUND_NEAREST, ROUND_STOCHASTIC = 0, 1


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter and 2-word key (C implementation)."""
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def q8_update(codes, absmax, grad, beta, dtype=F32, rounding=ROUND_NEAREST, seed=0, offset=0, tensor=0):
    """One tensor's q8 momentum update ("Quantized Muon Momentum", "Algorithm").

    codes  : int8 [numel]      prior state codes
    absmax : float32 [nblk]    prior per-256-block absmax
    grad   : float32 [numel] (dtype F32) or uint16 bits (BF16/F16)
    rounding: ROUND_NEAREST, or ROUND_STOCHASTIC with the random stream chosen
    by (seed, offset, tensor) (q8.c header).
    Returns (codes', absmax', m_stored, block_sumsq): the new state, m rounded
    to the grad dtype (what lands in the grad buffer) and fp64 sum of m^2 per
    block.  Inputs are not modified.
    """
    codes = np.array(codes, dtype=np.int8, copy=True).ravel()
    absmax = np.array(absmax, dtype=np.float32, copy=True).ravel()
    if dtype == F32:
        g = np.array(grad, dtype=np.float32, copy=True).ravel()
    else:
        g = np.array(grad, dtype=np.uint16, copy=True).ravel()
    numel = codes.size
    nblk = (numel + BLOCK - 1) // BLOCK
    if absmax.size != nblk or g.size != numel:
        raise ValueError("shape mismatch between codes, absmax and grad")
    sums = np.empty(nblk, dtype=np.float64)
    lib().or_q8_update_ex(_ptr(codes), _ptr(absmax), _ptr(g), dtype, numel, ctypes.c_float(beta), _ptr(sums),
                          rounding, seed, offset, tensor)
    return codes, absmax, g, sums


# ----------------------------------------------------------- MXFP8 carrier

def e4m3_from_f32(v):
    """fp32 -> E4M3 byte: round to nearest even, saturating at +-448 (q8.c)."""
    return int(lib().or_e4m3_from_f32(float(np.float32(v))))


def f32_from_e4m3(c):
    return float(lib().or_f32_from_e4m3(int(c)))


def mx_scale_byte(amax):
    """E8M0 scale byte of a 32-element block with absolute maximum amax."""
    return int(lib().or_mx_scale_byte(float(np.float32(amax))))


def decode_carrier(payload, scales):
    """Payload bytes [n] and scale bytes [n / 32] -> fp64 values (m as carried)."""
    payload = np.asarray(payload, np.uint8).ravel()
    scales = np.asarray(scales, np.uint8).ravel()
    table = np.array([f32_from_e4m3(c) for c in range(256)], dtype=np.float64)
    x = table[payload].reshape(-1, 32)
    return (x * np.ldexp(1.0, scales.astype(np.int64) - 127)[:, None]).ravel()


def q8_update_carrier(codes, absmax, grad, beta, dtype=F32):
    """The q8 update emitting the MXFP8 carrier instead of writing m (q8.c,
    "Wave18B MXFP8 Carrier Probe").  numel a multiple of 32.  Returns (codes',
    absmax', payload uint8 [numel], scales uint8 [numel / 32], block_sumsq).
    codes and absmax are copied; the grad goes to the C routine as it is, which
    only reads it."""
    codes = np.array(codes, dtype=np.int8, copy=True).ravel()
    absmax = np.array(absmax, dtype=np.float32, copy=True).ravel()
    g = np.ascontiguousarray(grad, dtype=np.float32 if dtype == F32 else np.uint16).reshape(-1)  # read in place
    numel = codes.size
    if numel % 32:
        raise ValueError("numel must be a multiple of 32")
    if absmax.size != (numel + BLOCK - 1) // BLOCK or g.size != numel:
        raise ValueError("shape mismatch between codes, absmax and grad")
    payload = np.zeros(numel, np.uint8)
    scales = np.zeros(numel // 32, np.uint8)
    sums = np.empty((numel + BLOCK - 1) // BLOCK, dtype=np.float64)
    lib().or_q8_update_carrier(_ptr(codes), _ptr(absmax), _ptr(g), dtype, numel, ctypes.c_float(beta),
                               _ptr(payload), _ptr(scales), _ptr(sums))
    return codes, absmax, payload, scales, sums


def transposed_carrier_applies(rows, cols):
    """Reading R29: in carrier mode a tall matrix (rows > cols) whose rows are
    a multiple of 128 and columns a multiple of 256, orthogonalised whole, is
    handed over as the row-wise carrier of its transpose."""
    return rows > cols and rows % 128 == 0 and cols % 256 == 0


def q8_update_carrier_t(codes, absmax, grad, beta, rows, cols, dtype=F32):
    """The q8 update of a rows x cols tensor emitting the MXFP8 carrier of
    m^T (q8.c or_q8_update_carrier_t): state as q8_update; payload uint8
    (cols, rows) with byte [c][r] coding m[r][c]; scales uint8 (cols, rows / 32),
    one per 32 consecutive rows of a column.  rows a multiple of 32."""
    codes = np.array(codes, dtype=np.int8, copy=True).ravel()
    absmax = np.array(absmax, dtype=np.float32, copy=True).ravel()
    g = np.ascontiguousarray(grad, dtype=np.float32 if dtype == F32 else np.uint16).reshape(-1)  # read in place
    numel = rows * cols
    if rows % 32:
        raise ValueError("rows must be a multiple of 32")
    if codes.size != numel or g.size != numel or absmax.size != (numel + BLOCK - 1) // BLOCK:
        raise ValueError("shape mismatch between codes, absmax and grad")
    payload = np.zeros((cols, rows), np.uint8)
    scales = np.zeros((cols, rows // 32), np.uint8)
    sums = np.empty((numel + BLOCK - 1) // BLOCK, dtype=np.float64)
    lib().or_q8_update_carrier_t(_ptr(codes), _ptr(absmax), _ptr(g), dtype, rows, cols, ctypes.c_float(beta),
                                 _ptr(payload), _ptr(scales), _ptr(sums))
    return codes, absmax, payload, scales, sums


# -------------------------------------------------------------- norm plans

def expand_segments(numels, segments, ngroups):
    """Norm segments -> one int32 group id per 256-block, per tensor.

    segments: iterable of (tensor_index, start, length, group_id), element
    offsets into the flattened tensor ("Quantized Muon Momentum", "Grouped QKV
    And Sharding").  Every segment starts on a block boundary and ends on one
    unless it ends at the tensor's end; every block of every tensor belongs to
    exactly one segment (our reading: an uncovered block would silently skip
    normalisation).  Raises ValueError otherwise.
    """
    ids = [np.full((n + BLOCK - 1) // BLOCK, -1, dtype=np.int32) for n in numels]
    for (t, start, length, gid) in segments:
        n = numels[t]
        if not (0 <= gid < ngroups):
            raise ValueError("group id out of range")
        if length <= 0 or start < 0 or start + length > n:
            raise ValueError("segment outside its tensor")
        if start % BLOCK:
            raise ValueError("segment start not block aligned")
        end = start + length
        if end % BLOCK and end != n:
            raise ValueError("segment end not block aligned")
        b0, b1 = start // BLOCK, (end + BLOCK - 1) // BLOCK
        if np.any(ids[t][b0:b1] != -1):
            raise ValueError("overlapping segments")
        ids[t][b0:b1] = gid
    for a in ids:
        if np.any(a < 0):
            raise ValueError("block not covered by any segment")
    return ids


def group_sums(block_sums, block_groups, ngroups):
    """S_g = sum of block sums of group g, tensors in order, blocks ascending."""
    bs = np.ascontiguousarray(np.concatenate(block_sums), dtype=np.float64)
    bg = np.ascontiguousarray(np.concatenate(block_groups), dtype=np.int32)
    out = np.empty(ngroups, dtype=np.float64)
    lib().or_group_sums(_ptr(bs), _ptr(bg), bs.size, ngroups, _ptr(out))
    return out


def group_inv_norm(sums, eps):
    """inv_g = 1/(sqrt(S_g) + eps) in fp64, rounded to fp32."""
    sums = np.ascontiguousarray(sums, dtype=np.float64)
    out = np.empty(sums.size, dtype=np.float32)
    lib().or_group_inv_norm(_ptr(sums), sums.size, ctypes.c_float(eps), _ptr(out))
    return out


def scale_by_group(grad, dtype, block_group, inv):
    """Scale pass: grad <- round(float(grad) * inv[group]) (returns a copy)."""
    g = np.array(grad, dtype=np.float32 if dtype == F32 else np.uint16, copy=True).ravel()
    bg = np.ascontiguousarray(block_group, dtype=np.int32)
    inv = np.ascontiguousarray(inv, dtype=np.float32)
    lib().or_scale_by_group(_ptr(g), dtype, g.size, _ptr(bg), _ptr(inv))
    return g


def update_normalize_groups(states, grads, dtypes, segments, ngroups, beta,
                            eps, write_normalized=True, rounding=ROUND_NEAREST, seed=0, offset=0):
    """Multi-tensor q8 update + grouped Frobenius normalisation.

    states : list of (codes, absmax); grads: list of fp32 arrays or uint16
    bits; dtypes: list of F32/BF16/F16.  Returns (new_states, grads_out,
    group_sums, inv_norm, block_groups).  grads_out holds m (rounded to the
    grad dtype) and, with write_normalized, m scaled by its group's inverse
    norm ("Quantized Muon Momentum", "What Exists" and "Grouped QKV And
    Sharding").
    """
    numels = [np.asarray(c).size for (c, _) in states]
    bgs = expand_segments(numels, segments, ngroups)
    new_states, outs, bsums = [], [], []
    for ti, ((c, a), g, dt) in enumerate(zip(states, grads, dtypes)):
        c2, a2, m, s = q8_update(c, a, g, beta, dt, rounding, seed, offset, ti)
        new_states.append((c2, a2))
        outs.append(m)
        bsums.append(s)
    S = group_sums(bsums, bgs, ngroups)
    inv = group_inv_norm(S, eps)
    if write_normalized:
        outs = [scale_by_group(m, dt, bg, inv) for m, dt, bg in zip(outs, dtypes, bgs)]
    return new_states, outs, S, inv, bgs
