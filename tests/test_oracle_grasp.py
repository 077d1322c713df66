"""Pins for the GRASP part of the CPU oracle (no GPU)."""
import os

import numpy as np
import pytest

from oracle import grasp, ns

RNG = np.random.default_rng(99)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        out[k] = np.array([float(t) for t in v])
    return out


def test_grid_quant_hand_worked_example():
    g = _golden("grid_quant_2x2.txt")
    x = g["x"].reshape(2, 2).astype(np.float32)
    q, rmax, cmax = grasp.grid_quantize(x, 4, s=2)
    assert np.array_equal(rmax.ravel(), g["rmax"].astype(np.float32))
    assert np.array_equal(cmax.ravel(), g["cmax"].astype(np.float32))
    assert np.array_equal(q.ravel(), g["codes"].astype(np.int8))
    deq = grasp.grid_dequantize(q, rmax, cmax, 4, s=2)
    assert np.allclose(deq.ravel(), g["deq"], rtol=1e-6)


@pytest.mark.parametrize("bits,shape", [(4, (130, 200)), (8, (300, 8)), (4, (64, 64))])
def test_grid_quant_invariants(bits, shape):
    """|code| <= L, each block's largest entry codes to +-L, and the error is
    at most half a level of its own divisor."""
    x = (RNG.standard_normal(shape) * np.exp(RNG.standard_normal(shape))).astype(np.float32)
    L = grasp.levels(bits)
    s = 64
    q, rmax, cmax = grasp.grid_quantize(x, bits, s)
    assert np.all(np.abs(q.astype(int)) <= L)
    d = np.minimum(np.repeat(rmax, s, axis=1)[:, :shape[1]], np.repeat(cmax, s, axis=0)[:shape[0], :])
    assert np.all(np.abs(x) <= d)
    for bi in range(0, shape[0], s):
        for bj in range(0, shape[1], s):
            blk = np.abs(x[bi:bi + s, bj:bj + s])
            i, j = np.unravel_index(np.argmax(blk), blk.shape)
            assert abs(int(q[bi + i, bj + j])) == L
    deq = grasp.grid_dequantize(q, rmax, cmax, bits, s)
    assert np.all(np.abs(deq - x) <= d / (2 * L) * (1 + 1e-5) + 1e-30)


def test_row_outlier_does_not_coarsen_other_rows():
    """A row of outliers dominates every column maximum of its block, so all
    other rows are divided by their own row maxima (not by the outliers, as a
    plain per-block absmax would) -- what the grid quantiser is for."""
    x = RNG.standard_normal((64, 64)).astype(np.float32)
    x[5] *= 1000
    rmax, cmax = grasp.grid_scales(x)
    d = np.minimum(rmax, cmax)                  # one 64x64 block: (64,1) vs (1,64)
    others = np.r_[0:5, 6:64]
    assert np.array_equal(d[others], np.broadcast_to(rmax[others], (63, 64)))
    assert np.all(d[others] < 10)


def test_nibble_pack_round_trip():
    for cols in (1, 2, 7, 64):
        c = RNG.integers(-8, 8, (5, cols)).astype(np.int8)
        p = grasp.pack_nibbles(c)
        assert p.shape == (5, (cols + 1) // 2)
        assert np.array_equal(grasp.unpack_nibbles(p, cols), c)
    p = grasp.pack_nibbles(np.array([[-1, 3]], np.int8))
    assert p[0, 0] == 0x3F            # even column in the low nibble, two's complement


def test_mgs_matches_numpy_qr():
    Y = RNG.standard_normal((500, 8))
    P = grasp.mgs(Y)
    Q, R = np.linalg.qr(Y)
    Q = Q * np.sign(np.diag(R))
    assert np.allclose(P, Q, atol=1e-12)
    assert np.allclose(P.T @ P, np.eye(8), atol=1e-13)


def test_col_norm_and_warm_replacement():
    R = RNG.standard_normal((50, 3))
    R[:, 1] = 0
    W = RNG.standard_normal((50, 3))
    Q = grasp.col_norm(R, W)
    assert np.allclose(np.linalg.norm(Q, axis=0), 1.0)
    assert np.allclose(Q[:, 1], W[:, 1] / np.linalg.norm(W[:, 1]))
    assert np.allclose(Q[:, 0], R[:, 0] / np.linalg.norm(R[:, 0]))


def test_exact_low_rank_momentum_is_captured_by_the_factor():
    """g of exact rank 8 with the warm start spanning its right factor: P
    spans the left factor, the residual is rounding-level, and the
    reconstructed momentum equals M up to the 8-bit factor quantisation."""
    m, n, k = 256, 192, 8
    U, _ = np.linalg.qr(RNG.standard_normal((m, k)))
    V, _ = np.linalg.qr(RNG.standard_normal((n, k)))
    g = ((U * np.linspace(3, 1, k)) @ V.T).astype(np.float32)
    st = grasp.State(m, n, k)
    new, M, P, R, O = grasp.grasp_step(st, g, 0.95, V)
    res = M.astype(np.float64) - P.astype(np.float64) @ R.astype(np.float64).T
    assert np.linalg.norm(res) / np.linalg.norm(M) < 1e-6
    s = np.linalg.svd(U.T @ P, compute_uv=False)
    assert np.all(s > 1 - 1e-6)                      # span(P) == span(U)
    Mrec, _ = new.momentum()
    assert np.linalg.norm(Mrec - M) / np.linalg.norm(M) < 2e-2


def test_rank_zero_reduces_to_grid_quantised_momentum():
    m, n = 128, 128
    g = (RNG.standard_normal((m, n)) * 1e-3).astype(np.float32)
    st = grasp.State(m, n, 0)
    new, M, P, R, O = grasp.grasp_step(st, g, 0.95, np.zeros((n, 0)))
    assert np.array_equal(M, g)                      # zero state: M = mu*0 + g
    q, rmax, cmax = grasp.grid_quantize(g, 4)
    assert np.array_equal(new.res, q) and np.array_equal(new.res_rmax, rmax)
    g2 = np.zeros_like(g)
    _, M2, _, _, _ = grasp.grasp_step(new, g2, 0.5, np.zeros((n, 0)))
    deq = grasp.grid_dequantize(q, rmax, cmax, 4)
    assert np.array_equal(M2, (np.float32(0.5) * deq).astype(np.float32))


def test_ema_has_no_one_minus_mu_factor():
    """Page's form M_t = mu M_{t-1} + g: a zero gradient scales the
    reconstructed momentum by exactly mu (fp32 product)."""
    m, n, k = 128, 64, 4
    g = (RNG.standard_normal((m, n))).astype(np.float32)
    st = grasp.State(m, n, k)
    warm = RNG.standard_normal((n, k))
    s1, M1, _, _, _ = grasp.grasp_step(st, g, 0.9, warm)
    Mprev, _ = s1.momentum()
    _, M2, _, _, _ = grasp.grasp_step(s1, np.zeros_like(g), 0.9, warm)
    assert np.array_equal(M2, (np.float32(0.9) * Mprev).astype(np.float32))


def test_ns_output_is_ns_of_unquantised_momentum():
    m, n, k = 96, 128, 4
    g = RNG.standard_normal((m, n)).astype(np.float32)
    st = grasp.State(m, n, k)
    _, M, _, _, O = grasp.grasp_step(st, g, 0.95, RNG.standard_normal((n, k)))
    assert np.allclose(O, ns.ns_orthogonalize(M.astype(np.float64)), atol=1e-14)


def test_apply_weights_hand_worked_2x2():
    """W' = W - lr (O + lambda W) on a 2 x 2 case worked by hand
    ("4-bit-Muon-GRASP", update equations; decoupled weight decay):
    lr = lambda = 0.5 gives W' = 0.75 W - 0.5 O."""
    W = np.array([[1.0, 2.0], [3.0, 4.0]])
    O = np.array([[0.5, 0.0], [0.0, -0.5]])
    got = grasp.apply_weights(W, O, 0.5, 0.5)
    assert np.array_equal(got, np.array([[0.5, 1.5], [2.25, 3.25]]))
    assert np.array_equal(grasp.apply_weights(W, O, 0.5), np.array([[0.75, 2.0], [3.0, 4.25]]))


def test_first_step_with_weight_decay_closed_form():
    """From the zero state M_1 = g exactly.  g = rows 0..15 of a 256-order
    Hadamard matrix / 16 has orthonormal rows, so with eps = 0 the NS output
    is p^5(1/4) g, and the weights move by -lr (p^5(1/4) g + lambda W)."""
    H = np.array([[1.0]])
    while H.shape[0] < 256:
        H = np.block([[H, H], [H, -H]])
    g = (H[:16] / 16.0).astype(np.float32)
    st = grasp.State(16, 256, 2)
    warm = RNG.standard_normal((256, 2)).astype(np.float32)
    _, M, _, _, O = grasp.grasp_step(st, g, 0.95, warm, eps=0.0)
    assert np.array_equal(M, g)
    s = 0.25
    for _ in range(5):
        s = ns.QUINTIC[0] * s + ns.QUINTIC[1] * s ** 3 + ns.QUINTIC[2] * s ** 5
    assert np.allclose(O, s * g.astype(np.float64), rtol=0, atol=1e-13)
    W = (RNG.standard_normal((16, 256)) * 0.02).astype(np.float32)
    W2 = grasp.apply_weights(W, O, 0.02, 0.1)
    exp = W.astype(np.float64) - 0.02 * (s * g.astype(np.float64) + 0.1 * W.astype(np.float64))
    assert np.allclose(W2, exp, rtol=0, atol=1e-15)
