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
