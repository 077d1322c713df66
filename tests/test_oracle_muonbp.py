"""Pins for the block-periodic schedule oracle (no GPU)."""
import math

import numpy as np

import oracle
from oracle import muonbp, ns

RNG = np.random.default_rng(4242)


def test_schedule_special_cases():
    """P = 1 is plain Muon (every step full); P beyond the run is BlockMuon;
    P = 5 makes steps 5, 10, 15, 20 full."""
    assert all(muonbp.is_full_step(t, 1) for t in range(1, 21))
    assert not any(muonbp.is_full_step(t, 1000) for t in range(1, 21))
    assert [t for t in range(1, 21) if muonbp.is_full_step(t, 5)] == [5, 10, 15, 20]


def test_rms_factor_matches_orthogonal_rms():
    """For an orthogonal p x q matrix (RMS 1/sqrt(max(p,q))) the factor gives
    an update whose RMS is exactly rms_scale."""
    for p, q in ((64, 256), (256, 64), (100, 100)):
        Q, _ = np.linalg.qr(RNG.standard_normal((max(p, q), min(p, q))))
        O = Q if p > q else Q.T
        rms = np.sqrt(np.mean(O ** 2))
        assert math.isclose(muonbp.rms_factor(p, q, 0.2) * rms, 0.2, rel_tol=1e-12)


def test_block_group_ids_geometry():
    ids = muonbp.block_group_ids(4, 2048, 4, 512)
    # each row holds 8 quantisation blocks, two per 512-column block
    assert list(ids[:8]) == [0, 0, 1, 1, 2, 2, 3, 3]
    assert ids.size == 32 and set(ids) == {0, 1, 2, 3}
    ids2 = muonbp.block_group_ids(8, 512, 4, 512)
    assert list(ids2) == [0] * 8 + [1] * 8


def test_block_and_full_steps_follow_their_step_sizes():
    """With an orthogonal-direction check: the update on a block step equals
    -lr_block * s_block * blockwise NS, on a full step -lr_full * s_full *
    full NS, and the q8 state evolves independently of W."""
    rows, cols, br, bc = 8, 1024, 8, 256
    W = RNG.standard_normal((rows, cols)).astype(np.float32) * 0.02
    codes = RNG.integers(-127, 128, rows * cols).astype(np.int8)
    absmax = RNG.uniform(1e-4, 1e-2, rows * cols // 256).astype(np.float32)
    g = (RNG.standard_normal(rows * cols) * 1e-3).astype(np.float32)
    kw = dict(rows=rows, cols=cols, block_rows=br, block_cols=bc, period=2,
              beta=0.95, eps=1e-7, coeffs=ns.QUINTIC, ns_steps=5, lr_full=0.02,
              lr_block=0.01, rms_scale=0.2)
    W1, c1, a1, O1, full1 = muonbp.muon_step(W, codes, absmax, g, oracle.F32, t=1, **kw)
    W2, c2, a2, O2, full2 = muonbp.muon_step(W, codes, absmax, g, oracle.F32, t=2, **kw)
    assert not full1 and full2
    assert np.array_equal(c1, c2) and np.array_equal(a1, a2)
    _, _, m, _ = oracle.q8_update(codes, absmax, g, 0.95)
    m = m.reshape(rows, cols).astype(np.float64)
    exp_block = ns.ns_blocked(m, br, bc)
    exp_full = ns.ns_orthogonalize(m)
    assert np.allclose(O1, exp_block, atol=1e-6) and np.allclose(O2, exp_full, atol=1e-6)
    assert np.allclose(W1 - W, -0.01 * 0.2 * math.sqrt(256) * O1, atol=1e-12)
    assert np.allclose(W2 - W, -0.02 * 0.2 * math.sqrt(1024) * O2, atol=1e-12)


def _sylvester(n):
    """Sylvester-Hadamard matrix of order n (a power of two): entries +-1,
    rows pairwise orthogonal."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def _quintic_power(s, steps=5):
    a, b, c = ns.QUINTIC
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def test_weight_decay_on_block_and_full_steps_closed_form():
    """Decoupled weight decay, W <- W - eta (s O + lambda W) ("4-bit-Muon-GRASP",
    update equations), pinned through inputs whose NS output is known exactly.

    beta = 0 makes m equal to the grad bit for bit.  The grad is four 16 x 256
    blocks, block j holding rows 16j .. 16j+15 of a 256-order Hadamard matrix
    divided by 16 (entries +-1/16, orthonormal rows).  So every block has all
    singular values 1 and Frobenius norm 4: with eps = 0 its inverse norm
    1/4 is exact and O_block = p^5(1/4) * block.  The whole 16 x 1024 matrix
    has M M^T = 4 I: norm 8, X0 = M / 8 with singular values 1/4, and
    O_full = p^5(1/4) * M / 2.  A dropped or sign-flipped lambda W term, or a
    missing eta on it, moves W by about lambda |W| or more."""
    rows, cols, br, bc = 16, 1024, 16, 256
    H = _sylvester(256) / 16.0
    g = np.concatenate([H[16 * j:16 * j + 16] for j in range(4)], axis=1).astype(np.float32)
    W = (RNG.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    W64 = W.astype(np.float64)
    codes = RNG.integers(-127, 128, rows * cols).astype(np.int8)
    absmax = RNG.uniform(1e-4, 1e-2, rows * cols // 256).astype(np.float32)
    lr_full, lr_block, rms, lam = 0.02, 0.01, 0.2, 0.1
    kw = dict(rows=rows, cols=cols, block_rows=br, block_cols=bc, period=2, beta=0.0, eps=0.0,
              coeffs=ns.QUINTIC, ns_steps=5, lr_full=lr_full, lr_block=lr_block, rms_scale=rms,
              weight_decay=lam)
    p = _quintic_power(0.25)
    M = g.astype(np.float64)
    # t = 1: block step, s = rms * sqrt(256)
    W1, _, _, O1, full1 = muonbp.muon_step(W, codes, absmax, g.reshape(-1), oracle.F32, t=1, **kw)
    assert not full1
    assert np.allclose(O1, p * M, rtol=0, atol=1e-13)
    exp1 = W64 - lr_block * (rms * 16.0 * p * M + lam * W64)
    assert np.allclose(W1, exp1, rtol=0, atol=1e-13)
    # t = 2: full step, s = rms * sqrt(1024)
    W2, _, _, O2, full2 = muonbp.muon_step(W, codes, absmax, g.reshape(-1), oracle.F32, t=2, **kw)
    assert full2
    assert np.allclose(O2, p * M / 2.0, rtol=0, atol=1e-13)
    exp2 = W64 - lr_full * (rms * 32.0 * p * M / 2.0 + lam * W64)
    assert np.allclose(W2, exp2, rtol=0, atol=1e-13)
    # the decay term is really there: without it the result is off by eta lambda W
    assert np.max(np.abs(W2 - (exp2 + lr_full * lam * W64))) > 1e-5


def test_weight_decay_with_zero_momentum_is_pure_shrink():
    """Zero state and zero grad give m = 0, O = 0 (0 times the finite 1/eps is
    0), so the step only shrinks the weights: W' = (1 - eta lambda) W."""
    rows, cols = 8, 512
    W = (RNG.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    z8 = np.zeros(rows * cols, np.int8)
    za = np.zeros(rows * cols // 256, np.float32)
    g = np.zeros(rows * cols, np.float32)
    W2, c2, a2, O, full = muonbp.muon_step(W, z8, za, g, oracle.F32, 1, rows, cols, rows, cols, 1, 0.95, 1e-7,
                                           ns.QUINTIC, 5, 0.5, 0.5, 0.2, weight_decay=0.25)
    assert full and np.all(O == 0) and np.all(c2 == 0) and np.all(a2 == 0)
    assert np.array_equal(W2, W.astype(np.float64) * (1.0 - 0.5 * 0.25))
