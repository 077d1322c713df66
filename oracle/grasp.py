"""GRASP 4-bit momentum step oracle (TEST INFRASTRUCTURE ONLY).

Source: "4-bit-Muon-GRASP" (the page's update equations and the definitions
under them).  The momentum is kept as a rank-k top factor P R^T (P m x k,
R n x k, 8-bit) plus a residual (4-bit), both grid-quantised: every entry of
an s x s block is divided by the smaller of its row's and its column's
absolute maximum inside that block.  One step:
    M_{t-1} = M_res + P R^T;   M_t = mu M_{t-1} + g_t
    Q = ColNorm(R_{t-1});  P = Orthogonalize(M_t Q);  R = M_t^T P
    M_res = M_t - P R^T;   store QUANT_4(M_res), QUANT_8(P), QUANT_8(R)
    O = NewtonSchulz(M_t, T);   W <- W - eta (O + lambda W)

Readings (the page leaves these open; each is listed in the design notes):
  * quantiser levels: symmetric uniform, L = 2^(b-1) - 1 (7 for 4 bits, 127
    for 8 bits); code = 0 if d == 0 else clamp(rint((x / d) * L), -L, L),
    d = min(row max, column max) in fp32; dequantised value code * (d / L);
  * blocks are s x s with s = 64, clipped at the matrix edge (so P and R,
    with k = 8 < 64 columns, use 64 x k blocks);
  * the stored scales are the per-block row maxima [rows][ceil(cols/s)] and
    column maxima [ceil(rows/s)][cols], fp32;
  * Orthogonalize is modified Gram-Schmidt in fp64 (unique thin QR with a
    positive diagonal); a column with zero norm stays zero;
  * ColNorm scales each column of the dequantised R to unit 2-norm; a zero
    column (the first step starts from P = R = 0) is replaced by the
    corresponding column of a seeded Gaussian `warm` (an input);
  * reductions (M Q, M^T P, norms) accumulate in fp64; P and R are rounded to
    fp32 before the residual; the reconstruction and the residual add the k
    rank-one terms in order k = 0..K-1 in fp64 and round once to fp32;
  * the EMA has no (1 - mu) factor, as on the page; fp32 products rounded
    separately: M = fl(fl(mu * M_prev) + g);
  * NS runs on the unquantised M_t (fp64 here; f32 arithmetic on the GPU),
    with the usual Frobenius normalisation and eps.
"""
import numpy as np

from . import ns

GRID = 64


def levels(bits):
    return (1 << (bits - 1)) - 1


def grid_scales(x, s=GRID):
    """Per-block row maxima [rows][nbc] and column maxima [nbr][cols]."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    nbr, nbc = -(-rows // s), -(-cols // s)
    rmax = np.zeros((rows, nbc), np.float32)
    cmax = np.zeros((nbr, cols), np.float32)
    if rows == 0 or cols == 0:
        return rmax, cmax
    a = np.abs(x)
    for bj in range(nbc):
        rmax[:, bj] = a[:, bj * s:(bj + 1) * s].max(axis=1)
    for bi in range(nbr):
        cmax[bi, :] = a[bi * s:(bi + 1) * s, :].max(axis=0)
    return rmax, cmax


def _divisor(rmax, cmax, s, shape):
    rows, cols = shape
    r = np.repeat(rmax, s, axis=1)[:, :cols]
    c = np.repeat(cmax, s, axis=0)[:rows, :]
    return np.minimum(r, c).astype(np.float32)


def grid_quantize(x, bits, s=GRID):
    """Returns (codes int8, rmax, cmax) for the b-bit grid quantiser."""
    x = np.asarray(x, dtype=np.float32)
    L = np.float32(levels(bits))
    rmax, cmax = grid_scales(x, s)
    d = _divisor(rmax, cmax, s, x.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x / d).astype(np.float32) * L
        q = np.clip(np.rint(t), -L, L)
    q = np.where(d == 0, 0, q).astype(np.int8)
    return q, rmax, cmax


def grid_dequantize(codes, rmax, cmax, bits, s=GRID):
    L = np.float32(levels(bits))
    d = _divisor(rmax, cmax, s, codes.shape)
    step = (d / L).astype(np.float32)
    return (codes.astype(np.float32) * step).astype(np.float32)


def pack_nibbles(codes):
    """int8 codes in [-8, 7] -> bytes, two per byte, even column in the low
    nibble (two's complement), rows padded to an even length with 0."""
    rows, cols = codes.shape
    c = np.zeros((rows, cols + (cols & 1)), np.int16)
    c[:, :cols] = codes
    lo = c[:, 0::2] & 0xF
    hi = c[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, cols):
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty((p.shape[0], p.shape[1] * 2), np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out[:, :cols].astype(np.int8)


def mgs(Y):
    """Modified Gram-Schmidt thin QR (fp64), positive diagonal; a column whose
    remainder has zero norm stays zero."""
    Y = np.array(Y, dtype=np.float64, copy=True)
    m, k = Y.shape
    P = np.zeros((m, k))
    for c in range(k):
        v = Y[:, c].copy()
        for p in range(c):
            v = v - np.dot(P[:, p], v) * P[:, p]
        nrm = np.sqrt(np.dot(v, v))
        if nrm > 0:
            P[:, c] = v / nrm
    return P


def col_norm(R, warm):
    """Unit-norm columns of R (fp64); zero columns replaced by warm's."""
    R = np.asarray(R, dtype=np.float64)
    W = np.asarray(warm, dtype=np.float64)
    Q = np.empty_like(R)
    for c in range(R.shape[1]):
        nrm = np.sqrt(np.dot(R[:, c], R[:, c]))
        if nrm > 0:
            Q[:, c] = R[:, c] / nrm
        else:
            Q[:, c] = W[:, c] / np.sqrt(np.dot(W[:, c], W[:, c]))
    return Q


def _rank_k_sum(base, P, R, sign):
    """(float32)(base + sign * sum_k P[:,k] R[:,k]^T) in fp64, k in order."""
    acc = np.asarray(base, dtype=np.float64).copy()
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    for k in range(P.shape[1]):
        term = P[:, k:k + 1] * R[:, k][None, :]
        acc = acc + term if sign > 0 else acc - term
    return acc.astype(np.float32)


class State:
    """Quantised GRASP state of one m x n matrix (codes unpacked here)."""

    def __init__(self, rows, cols, rank, s=GRID):
        self.rows, self.cols, self.rank, self.s = rows, cols, rank, s
        nbr, nbc = -(-rows // s), -(-cols // s)
        self.res = np.zeros((rows, cols), np.int8)
        self.res_rmax = np.zeros((rows, nbc), np.float32)
        self.res_cmax = np.zeros((nbr, cols), np.float32)
        self.p = np.zeros((rows, rank), np.int8)
        self.p_rmax = np.zeros((rows, -(-rank // s)), np.float32)
        self.p_cmax = np.zeros((nbr, rank), np.float32)
        self.r = np.zeros((cols, rank), np.int8)
        self.r_rmax = np.zeros((cols, -(-rank // s)), np.float32)
        self.r_cmax = np.zeros((nbc, rank), np.float32)

    def copy(self):
        o = State.__new__(State)
        o.__dict__ = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in self.__dict__.items()}
        return o

    def momentum(self):
        """M = deq4(res) + deq8(P) deq8(R)^T (fp32)."""
        s = self.s
        Pd = grid_dequantize(self.p, self.p_rmax, self.p_cmax, 8, s)
        Rd = grid_dequantize(self.r, self.r_rmax, self.r_cmax, 8, s)
        resd = grid_dequantize(self.res, self.res_rmax, self.res_cmax, 4, s)
        return _rank_k_sum(resd, Pd, Rd, +1), Rd


def grasp_step(state, g, mu, warm, ns_steps=5, coeffs=ns.QUINTIC, eps=ns.EPS, with_ns=True):
    """One GRASP step.  Returns (new_state, M_t fp32, P fp32, R fp32, O fp64);
    the input state is not modified.  with_ns=False skips O (returns None),
    for callers that check NS separately."""
    s = state.s
    Mprev, Rd = state.momentum()
    t = (np.float32(mu) * Mprev).astype(np.float32)
    M = (t + np.asarray(g, dtype=np.float32)).astype(np.float32)
    Q = col_norm(Rd, warm)
    M64 = M.astype(np.float64)
    Y = M64 @ Q
    P = mgs(Y)
    R = M64.T @ P
    P32, R32 = P.astype(np.float32), R.astype(np.float32)
    res = _rank_k_sum(M, P32, R32, -1)
    new = state.copy()
    new.res, new.res_rmax, new.res_cmax = grid_quantize(res, 4, s)
    new.p, new.p_rmax, new.p_cmax = grid_quantize(P32, 8, s)
    new.r, new.r_rmax, new.r_cmax = grid_quantize(R32, 8, s)
    O = ns.ns_orthogonalize(M64, ns_steps, coeffs, eps) if with_ns else None
    return new, M, P32, R32, O


def residual(M, P32, R32):
    """The fp32 residual M - P R^T the step quantises."""
    return _rank_k_sum(M, P32, R32, -1)


def apply_weights(W, O, lr, weight_decay=0.0):
    W = np.asarray(W, dtype=np.float64)
    return W - lr * (O + weight_decay * W)
