"""Newton-Schulz orthogonalisation oracle in fp64 (TEST INFRASTRUCTURE ONLY).

Sources:
  * "NVIDIA impulsa optimizadores avanzados ... con Megatron", section
    "Newton-Schulz distribuido": one NS iteration is three matrix products
    (Gram matrix X X^T, then the polynomial in it, then the product with X),
    and five iterations are the common choice;
  * the quintic polynomial p(s) = a s + b s^3 + c s^5 with
    (a, b, c) = (3.4445, -4.7750, 2.0315) and eps = 1e-7 are fixed by the
    workload definition, not by the pages;
  * "MuonBP: Faster Muon via Block-Periodic Orthogonalization", key design 1:
    the FLOP model 2(2nm^2 + m^3) assumes the Gram side is the smaller one
    (m <= n), so a tall matrix is iterated as its transpose.

The iteration is written in the order the pages give it; numpy's matmul is the
only library step.  `spectral_rows` is a second, independent route to the same
exact-arithmetic result (the iteration is a polynomial in X X^T applied to X),
used where the iteration is too slow to run on the CPU at full size.
"""
import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)
EPS = 1e-7


def _orient(M):
    X = np.array(M, dtype=np.float64, copy=True)
    tall = X.shape[0] > X.shape[1]
    return (X.T.copy() if tall else X), tall


def normalize(X, eps=EPS, inv_norm=None):
    """X0 = X / (||X||_F + eps), or X * inv_norm when the scale is given."""
    if inv_norm is None:
        return X / (np.sqrt(np.sum(X * X)) + eps)
    return X * float(inv_norm)


def ns_orthogonalize(M, steps=5, coeffs=QUINTIC, eps=EPS, inv_norm=None):
    """O = NS_T(M): quintic Newton-Schulz on the Frobenius-normalised M.

    Wide or square M (rows <= cols) is iterated as is; a tall M is iterated as
    M^T and the result transposed back, so the Gram matrix is min-dim square.
    Per iteration:  A = X X^T;  B = b A + c A A;  X = a X + B X.
    """
    a, b, c = (float(v) for v in coeffs)
    X, tall = _orient(M)
    X = normalize(X, eps, inv_norm)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def ns_blocked(M, block_rows, block_cols, steps=5, coeffs=QUINTIC, eps=EPS,
               inv_norms=None):
    """Blockwise NS: every (block_rows x block_cols) block is an independent NS
    input with its own Frobenius norm and orientation ("MuonBP", key design 1:
    a block step orthogonalises each local shard on its own, no communication;
    "NVIDIA ... Megatron", blockwise mode).  inv_norms, if given, is indexed
    by block in row-major block order."""
    M = np.asarray(M)
    R, C = M.shape
    if R % block_rows or C % block_cols:
        raise ValueError("matrix not divisible into blocks")
    out = np.empty((R, C), dtype=np.float64)
    k = 0
    for i in range(0, R, block_rows):
        for j in range(0, C, block_cols):
            inv = None if inv_norms is None else inv_norms[k]
            out[i:i + block_rows, j:j + block_cols] = ns_orthogonalize(
                M[i:i + block_rows, j:j + block_cols], steps, coeffs, eps, inv)
            k += 1
    return out


def spectral_rows(M, rows, steps=5, coeffs=QUINTIC, eps=EPS, inv_norm=None):
    """Selected rows of NS_T(M) (original orientation) through the spectrum.

    With X0 the normalised (and, if tall, transposed) input and
    G = X0 X0^T = U diag(lam) U^T, every iterate is h(G) X0 where, per
    eigenvalue, h_0 = 1, g_0 = lam, q = a + b g + c g^2, h <- h q,
    g <- g q^2.  Exact arithmetic gives the same matrix as ns_orthogonalize;
    this route costs one Gram product and one symmetric eigensolve, then
    O(m^2 + m n) per requested row.
    """
    a, b, c = (float(v) for v in coeffs)
    X, tall = _orient(M)
    X = normalize(X, eps, inv_norm)
    lam, U = np.linalg.eigh(X @ X.T)
    h = np.ones_like(lam)
    g = lam.copy()
    for _ in range(steps):
        q = a + b * g + c * g * g
        h = h * q
        g = g * q * q
    rows = np.asarray(rows)
    if tall:
        # O = (h(G) X0)^T, row r of O = X0[:, r]^T h(G)
        Xr = X[:, rows].T                   # (len(rows), m)
        return ((Xr @ U) * h) @ U.T
    W = (U[rows] * h) @ U.T                 # (len(rows), m)
    return W @ X


def ns_flops(m, n, steps):
    """Algorithmic FLOPs of T iterations with m <= n, counting the symmetric
    Gram products at their lower-triangle cost (n m(m+1) and m m(m+1)) and the
    last product at 2 m^2 n; the dense-equivalent count is 2(2 n m^2 + m^3)."""
    if m > n:
        m, n = n, m
    sym = n * m * (m + 1) + m * m * (m + 1) + 2 * m * m * n
    dense = 2 * (2 * n * m * m + m ** 3)
    return steps * sym, steps * dense
