"""Pins for the q8 part of the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: exact
rational arithmetic, torch/numpy library routines, closed forms and the
invariants that the page's definition of the state fixes ("Quantized Muon
Momentum", sections "What Exists" and "Algorithm").
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F16, F32

RNG = np.random.default_rng(12345)


def _state(numel, rng=RNG, lo=1e-4, hi=1e-2):
    codes = rng.integers(-127, 128, numel).astype(np.int8)
    absmax = rng.uniform(lo, hi, (numel + 255) // 256).astype(np.float32)
    return codes, absmax


def _grad(numel, std=1e-3, rng=RNG):
    return (rng.standard_normal(numel) * std).astype(np.float32)


# ----------------------------------------------------------------- dtypes

def test_bf16_rounding_matches_torch():
    x = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * 10.0 ** RNG.integers(-40, 38, 20000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -1.00390625, 3.0e38,
                  3.4e38, np.inf, -np.inf, 1e-40, -1e-45], dtype=np.float32),
        # exact ties: low 16 bits == 0x8000
        (np.arange(0, 4000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32)[1:],
    ]).astype(np.float32)
    x = x[np.isfinite(x) | np.isinf(x)]
    ours = oracle.round_to(x, BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.widen(ours, BF16)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_f16_rounding_matches_numpy():
    x = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * 10.0 ** RNG.integers(-9, 6, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e5, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0001, 3 * 2.0 ** -26, 6.1e-5, np.inf], dtype=np.float32),
        (np.arange(1, 6000, dtype=np.uint32) << 13 | 0x1000 | (0x70 << 23)).view(np.float32),
    ]).astype(np.float32)
    ours = oracle.round_to(x, F16)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(oracle.widen(ours, F16), ref.view(np.float16).astype(np.float32))


# ----------------------------------------------------------- EMA and codes

def _exact(f):
    return Fraction(float(f))


def test_ema_matches_exact_arithmetic_within_rounding():
    """m = beta*old + (1-beta)*g with old = code*absmax/127, against exact
    rational arithmetic: the fp32 result may differ by the three roundings of
    the chosen op order (and the rounding of absmax/127), never more."""
    n = 1000
    codes, absmax = _state(n)
    g = _grad(n)
    beta = np.float32(0.95)
    _, _, m, _ = oracle.q8_update(codes, absmax, g, float(beta), F32)
    b = _exact(beta)
    for i in range(0, n, 7):
        old = Fraction(int(codes[i])) * _exact(absmax[i // 256]) / 127
        exact = b * old + (1 - b) * _exact(g[i])
        err = abs(_exact(m[i]) - exact)
        scale = abs(b * old) + abs((1 - b) * _exact(g[i]))
        # 4 roundings of relative size <= 2^-24 each (step, old, two products, sum)
        assert err <= scale * Fraction(5, 2 ** 24) + Fraction(1, 2 ** 149), i


def test_codes_are_nearest_symmetric_levels():
    """Every code is the nearest integer to m*127/amax in exact arithmetic,
    |code| <= 127, and a non-zero block reaches +-127 at its absmax."""
    n = 4096
    codes, absmax = _state(n)
    g = _grad(n)
    q, a, m, _ = oracle.q8_update(codes, absmax, g, 0.95, F32)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    for b in range(n // 256):
        blk = m[b * 256:(b + 1) * 256]
        amax = np.max(np.abs(blk))
        assert a[b] == amax
        qb = q[b * 256:(b + 1) * 256].astype(np.int32)
        assert np.max(np.abs(qb)) == 127
        A = _exact(amax)
        for i in range(0, 256, 5):
            t = _exact(blk[i]) * 127 / A
            d = abs(t - qb[i])
            if d > Fraction(1, 2):
                # only a value within fp32 noise of a tie may round the other way
                assert d - Fraction(1, 2) < Fraction(1, 2 ** 16), (b, i)


def test_roundtrip_bound():
    """|m - code*absmax/127| <= absmax/254 (1 + 2^-20): half a level."""
    n = 256 * 64
    codes, absmax = _state(n)
    g = _grad(n)
    q, a, m, _ = oracle.q8_update(codes, absmax, g, 0.9, F32)
    deq = q.astype(np.float64) * np.repeat(a.astype(np.float64), 256) / 127
    bound = np.repeat(a.astype(np.float64), 256) / 254 * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - m.astype(np.float64)) <= bound)


def test_beta_zero_reduces_to_absmax_quantiser_of_grad():
    n = 256 * 8
    codes, absmax = _state(n)
    g = _grad(n)
    q, a, m, _ = oracle.q8_update(codes, absmax, g, 0.0, F32)
    assert np.array_equal(m, g)
    assert np.array_equal(a, np.abs(g).reshape(-1, 256).max(axis=1))
    q0, a0, _, _ = oracle.q8_update(np.zeros(n, np.int8), np.zeros_like(absmax), g, 0.0, F32)
    assert np.array_equal(q, q0) and np.array_equal(a, a0)


def test_beta_one_is_idempotent():
    """beta = 1: m equals the dequantised state exactly, and re-quantising a
    state whose block holds a +-127 code reproduces the codes."""
    n = 256 * 8
    codes, absmax = _state(n)
    for b in range(8):
        codes[b * 256 + 17] = 127 if b % 2 else -127
    g = _grad(n)
    q, a, m, _ = oracle.q8_update(codes, absmax, g, 1.0, F32)
    step = (absmax / np.float32(127)).astype(np.float32)
    old = (codes.astype(np.float32) * np.repeat(step, 256)).astype(np.float32)
    assert np.array_equal(m, old)
    assert np.array_equal(q, codes)


@pytest.mark.parametrize("scale", [1e30, 1e-20, 1e-37, 2.0 ** -64, 2.0 ** -64 * (1 - 2.0 ** -24), 5e-39, 2e-41])
def test_beta_one_is_idempotent_at_every_block_scale(scale):
    """The idempotence above at block maxima from 1e30 down to subnormals:
    the codes stay the nearest levels even where 127 / amax overflows
    binary32 (block maxima below about 3.7e-37), and zero codes stay 0."""
    n = 256 * 4
    rng = np.random.default_rng(777)
    codes = rng.integers(-127, 128, n).astype(np.int8)
    codes[::7] = 0
    codes[5::256] = 127
    codes[6::256] = -127
    absmax = np.full(4, scale, np.float32)
    q, a, m, _ = oracle.q8_update(codes, absmax, np.zeros(n, np.float32), 1.0, F32)
    assert np.all(a > 0) and np.all(np.isfinite(a))
    assert np.array_equal(q, codes)


def test_non_finite_momentum_codes():
    """Reading for non-finite m (outside the method's contract, defined so
    both implementations agree): a NaN m codes as -127 (the clamp returns
    the number when its other operand is NaN) and is ignored by the block
    maximum; an infinite m makes its block's absmax infinite, so 127 / amax
    is 0: the block's finite elements code 0 and the infinite one
    (inf * 0 = NaN) -127."""
    n = 512
    codes = np.zeros(n, np.int8)
    absmax = np.zeros(2, np.float32)
    g = _grad(n)
    g[10] = np.nan
    g[300] = np.inf
    q, a, m, _ = oracle.q8_update(codes, absmax, g, 0.0, F32)
    assert np.isnan(m[10]) and q[10] == -127
    finite0 = np.delete(np.arange(256), 10)
    assert a[0] == np.max(np.abs(g[finite0]))
    assert np.max(np.abs(q[finite0].astype(np.int32))) == 127
    assert np.isinf(a[1]) and q[300] == -127
    assert np.all(q[256:300] == 0) and np.all(q[301:512] == 0)


def test_zero_block_and_partial_tail():
    """A block of zeros stores codes 0 / absmax 0; numel = 1000 has 4 blocks,
    the last one covering elements 768..999 only."""
    n = 1000
    codes = np.zeros(n, np.int8)
    absmax = np.zeros(4, np.float32)
    g = _grad(n)
    g[256:512] = 0.0
    q, a, m, s = oracle.q8_update(codes, absmax, g, 0.5, F32)
    assert a[1] == 0.0 and np.all(q[256:512] == 0) and s[1] == 0.0
    assert a.size == 4 and a[3] == np.max(np.abs(m[768:]))
    # the tail's absmax must not see anything outside its own elements
    g2 = g.copy()
    g2[767] = 1.0
    _, a2, _, _ = oracle.q8_update(codes, absmax, g2, 0.5, F32)
    assert a2[3] == a[3] and a2[2] != a[2]


def test_block_sumsq_matches_numpy():
    n = 256 * 16 + 77
    codes, absmax = _state(n)
    g = _grad(n)
    _, _, m, s = oracle.q8_update(codes, absmax, g, 0.95, F32)
    m64 = np.concatenate([m.astype(np.float64), np.zeros(256 - 77)]).reshape(-1, 256)
    assert np.allclose(s, np.sum(m64 * m64, axis=1), rtol=1e-14, atol=0)


def test_constant_grad_closed_form():
    """g constant per element: m_t = beta^t m_0 + (1 - beta^t) g before
    quantisation; with requantisation the dequantised state stays within
    sum_j beta^(t-1-j) absmax_j / 254 of it."""
    n = 256 * 4
    codes, absmax = _state(n)
    g = _grad(n) * 5
    beta = 0.95
    b32 = float(np.float32(beta))
    m0 = codes.astype(np.float64) * np.repeat(absmax.astype(np.float64), 256) / 127
    bound = np.zeros(n)
    c, a = codes, absmax
    for t in range(1, 41):
        c, a, m, _ = oracle.q8_update(c, a, g, beta, F32)
        bound = b32 * bound + np.repeat(a.astype(np.float64), 256) / 254 * (1 + 1e-5)
        deq = c.astype(np.float64) * np.repeat(a.astype(np.float64), 256) / 127
        ideal = b32 ** t * m0 + (1 - b32 ** t) * g.astype(np.float64)
        assert np.all(np.abs(deq - ideal) <= bound + 1e-9 * np.abs(ideal) + 1e-12), t
    assert np.max(np.abs(deq - g)) < 0.2 * np.max(np.abs(g))


def test_bf16_and_f16_grads_store_rounded_m():
    """The 16-bit paths compute in fp32 (same codes and absmax as the fp32
    path on the widened grad) and store m rounded by torch's/numpy's cast."""
    n = 256 * 8 + 100
    codes, absmax = _state(n)
    g32 = _grad(n)
    for dt in (BF16, F16):
        gbits = oracle.round_to(g32, dt)
        gw = oracle.widen(gbits, dt)
        qa, aa, ma, sa = oracle.q8_update(codes, absmax, gw, 0.95, F32)
        qb, ab, mb, sb = oracle.q8_update(codes, absmax, gbits, 0.95, dt)
        assert np.array_equal(qa, qb) and np.array_equal(aa, ab) and np.array_equal(sa, sb)
        if dt == BF16:
            ref = torch.from_numpy(ma).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            ref = ma.astype(np.float16).view(np.uint16)
        assert np.array_equal(mb, ref)


# ------------------------------------------------------------- norm groups

def test_segment_expansion_brute_force_and_errors():
    numels = [2560 * 64, 1000]
    segs = [(0, 0, 2048 * 64, 0), (0, 2048 * 64, 256 * 64, 1), (0, 2304 * 64, 256 * 64, 2),
            (1, 0, 512, 3), (1, 512, 488, 4)]
    ids = oracle.expand_segments(numels, segs, 5)
    for t, n in enumerate(numels):
        per_elem = np.full(n, -1)
        for (ti, s, ln, gid) in segs:
            if ti == t:
                per_elem[s:s + ln] = gid
        for b in range(ids[t].size):
            assert set(per_elem[b * 256:(b + 1) * 256]) == {ids[t][b]}
    with pytest.raises(ValueError):
        oracle.expand_segments([1024], [(0, 0, 300, 0), (0, 300, 724, 1)], 2)   # misaligned
    with pytest.raises(ValueError):
        oracle.expand_segments([1024], [(0, 0, 768, 0), (0, 512, 512, 1)], 2)   # overlap
    with pytest.raises(ValueError):
        oracle.expand_segments([1024], [(0, 0, 512, 0)], 1)                      # uncovered
    with pytest.raises(ValueError):
        oracle.expand_segments([1024], [(0, 0, 1024, 2)], 2)                     # bad group


def test_single_group_is_global_frobenius_norm():
    shapes = [(64, 128), (32, 100)]
    states = [_state(r * c) for r, c in shapes]
    grads = [_grad(r * c) for r, c in shapes]
    segs = [(i, 0, r * c, 0) for i, (r, c) in enumerate(shapes)]
    eps = 1e-7
    _, outs, S, inv, _ = oracle.update_normalize_groups(
        states, grads, [F32, F32], segs, 1, 0.95, eps, write_normalized=False)
    allm = np.concatenate([o.astype(np.float64) for o in outs])
    assert np.isclose(S[0], np.sum(allm ** 2), rtol=1e-13)
    assert inv[0] == np.float32(1.0 / (np.linalg.norm(allm) + eps))
    _, outs_n, _, _, _ = oracle.update_normalize_groups(
        states, grads, [F32, F32], segs, 1, 0.95, eps, write_normalized=True)
    normed = np.concatenate([o.astype(np.float64) for o in outs_n])
    assert abs(np.linalg.norm(normed) - 1.0) < 1e-6


def test_qkv_groups_normalise_independently():
    rows, cols = 2560, 64
    st = _state(rows * cols)
    g = oracle.round_to(_grad(rows * cols) * np.repeat([1.0, 30.0, 0.1], [2048 * 64, 256 * 64, 256 * 64]).astype(np.float32), BF16)
    segs = [(0, 0, 2048 * cols, 0), (0, 2048 * cols, 256 * cols, 1), (0, 2304 * cols, 256 * cols, 2)]
    _, outs, S, inv, _ = oracle.update_normalize_groups([st], [g], [BF16], segs, 3, 0.95, 1e-7)
    x = oracle.widen(outs[0], BF16).astype(np.float64).reshape(rows, cols)
    for r0, r1 in ((0, 2048), (2048, 2304), (2304, 2560)):
        assert abs(np.linalg.norm(x[r0:r1]) - 1.0) < 5e-3
