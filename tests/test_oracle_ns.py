"""Pins for the Newton-Schulz part of the CPU oracle (no GPU).

The iteration X <- a X + (b A + c A^2) X with A = X X^T maps every singular
value s of the normalised input to p(s) = a s + b s^3 + c s^5 and keeps the
singular vectors, so T iterations give U diag(p^T(s)) V^T exactly.  That
closed form comes from numpy's SVD, independent of the oracle's matmuls.
"""
import numpy as np
import pytest

from oracle import ns

COEF = ns.QUINTIC
RNG = np.random.default_rng(777)


def _svd_form(M, steps, coeffs=COEF, eps=ns.EPS):
    a, b, c = coeffs
    U, s, Vt = np.linalg.svd(np.asarray(M, np.float64), full_matrices=False)
    s = s / (np.linalg.norm(M) + eps)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


@pytest.mark.parametrize("shape", [(64, 96), (96, 64), (80, 80), (256, 512)])
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_iteration_matches_svd_closed_form(shape, steps):
    M = RNG.standard_normal(shape)
    O = ns.ns_orthogonalize(M, steps)
    ref = _svd_form(M, steps)
    assert O.shape == shape
    assert np.linalg.norm(O - ref) / np.linalg.norm(ref) < 1e-12


def test_orthogonal_input_gives_scalar_multiple():
    """Q with orthonormal rows: every singular value is 1, so after
    normalisation s = 1/sqrt(r) (r = min dim) and O = p^T(s) Q."""
    Q, _ = np.linalg.qr(RNG.standard_normal((200, 50)))
    M = 3.0 * Q.T                                 # 50 x 200, orthonormal rows (x3)
    s = 3.0 / (3.0 * np.sqrt(50) + ns.EPS)
    for _ in range(5):
        s = COEF[0] * s + COEF[1] * s ** 3 + COEF[2] * s ** 5
    O = ns.ns_orthogonalize(M, 5)
    assert np.allclose(O, s * Q.T, rtol=0, atol=1e-13)


def test_transpose_equivariance_and_scale_invariance():
    M = RNG.standard_normal((48, 130))
    O = ns.ns_orthogonalize(M)
    assert np.allclose(ns.ns_orthogonalize(M.T), O.T, atol=1e-13)
    # equal up to eps: eps/||M|| ~ 1e-9, amplified at most a^5 ~ 500 times
    assert np.allclose(ns.ns_orthogonalize(1e3 * M), O, atol=1e-6)


def test_coefficients_are_not_interchangeable():
    """A swapped or sign-flipped coefficient moves the result far away, so
    the SVD pin above really fixes them."""
    M = RNG.standard_normal((64, 128))
    base = ns.ns_orthogonalize(M)
    for coeffs in [(COEF[0], COEF[2], COEF[1]), (COEF[0], -COEF[1], COEF[2]),
                   (COEF[1], COEF[0], COEF[2])]:
        alt = ns.ns_orthogonalize(M, coeffs=coeffs)
        assert np.linalg.norm(alt - base) > 0.1 * np.linalg.norm(base)


def test_singular_values_land_in_the_quintic_band():
    """For normalised singular values in [0.01, 1], five steps of this quintic
    put every output singular value in [0.68, 1.135] (the polynomial's
    attracting two-cycle band)."""
    M = RNG.standard_normal((128, 512))
    O = ns.ns_orthogonalize(M)
    s_in = np.linalg.svd(M / np.linalg.norm(M), compute_uv=False)
    assert s_in.min() > 0.01
    s_out = np.linalg.svd(O, compute_uv=False)
    assert s_out.min() > 0.68 and s_out.max() < 1.135


def test_explicit_scale_equals_norm():
    M = RNG.standard_normal((32, 64))
    inv = 1.0 / (np.linalg.norm(M) + ns.EPS)
    assert np.allclose(ns.ns_orthogonalize(M, inv_norm=inv), ns.ns_orthogonalize(M), atol=1e-15)


def test_zero_steps_and_linear_coefficients():
    M = RNG.standard_normal((16, 40))
    X0 = M / (np.linalg.norm(M) + ns.EPS)
    assert np.allclose(ns.ns_orthogonalize(M, 0), X0, atol=1e-16)
    assert np.allclose(ns.ns_orthogonalize(M, 3, coeffs=(2.0, 0.0, 0.0)), 8 * X0, atol=1e-15)


@pytest.mark.parametrize("shape", [(60, 150), (150, 60), (70, 70)])
def test_spectral_rows_match_iteration(shape):
    M = RNG.standard_normal(shape)
    rows = np.array([0, 3, shape[0] - 1])
    ref = ns.ns_orthogonalize(M)[rows]
    got = ns.spectral_rows(M, rows)
    assert np.allclose(got, ref, atol=1e-12)


def test_rank_deficient_input_keeps_null_space():
    """A rank-3 input: the output has rank 3 and the same row/column spaces."""
    M = RNG.standard_normal((40, 3)) @ RNG.standard_normal((3, 90))
    O = ns.ns_orthogonalize(M)
    s = np.linalg.svd(O, compute_uv=False)
    assert np.all(s[3:] < 1e-10) and np.all(s[:3] > 0.1)
    assert np.allclose(O, _svd_form(M, 5), atol=1e-12)


def test_blocked_is_independent_per_block():
    M = RNG.standard_normal((64, 96))
    out = ns.ns_blocked(M, 64, 32)
    for j in range(3):
        blk = M[:, 32 * j:32 * (j + 1)]
        assert np.allclose(out[:, 32 * j:32 * (j + 1)], _svd_form(blk, 5), atol=1e-12)
    M2 = M.copy()
    M2[:, :32] *= -7.0
    out2 = ns.ns_blocked(M2, 64, 32)
    assert np.allclose(out2[:, 32:], out[:, 32:], atol=0)
    with pytest.raises(ValueError):
        ns.ns_blocked(M, 64, 40)


def test_flop_model_matches_dense_formula():
    """Dense-equivalent count is the MuonBP page's 2(2nm^2 + m^3) per step."""
    sym, dense = ns.ns_flops(4096, 14336, 5)
    assert dense == 5 * 2 * (2 * 14336 * 4096 ** 2 + 4096 ** 3)
    assert ns.ns_flops(14336, 4096, 5) == (sym, dense)
    assert sym < dense
