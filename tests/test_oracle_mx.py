"""Pins of the oracle's MXFP8 carrier pieces ("Quantized Muon Momentum",
section "Wave18B MXFP8 Carrier Probe"): E4M3 payload bytes, E8M0 per-32
scale bytes, and the carrier-emitting q8 update.

The E4M3 encoder is checked against facts of the format (1 sign, 4 exponent
bits biased by 7, 3 mantissa bits, subnormals, no infinities, largest finite
value 448, NaN = S.1111.111) and against a brute-force nearest search over
the finite codes; the scale rule against exact powers of two; the carrier
update against the plain q8 update, which its own tests pin."""
import numpy as np
import pytest

import oracle


def _pos_values():
    """All finite non-negative E4M3 values by enumeration from the format
    definition: subnormals k 2^-9, normals (1 + m/8) 2^(e-7)."""
    vals = [k * 2.0 ** -9 for k in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                           # NaN
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


POS = _pos_values()


def test_e4m3_known_codes():
    cases = {0.0: 0x00, 2.0 ** -9: 0x01, 7 * 2.0 ** -9: 0x07, 2.0 ** -6: 0x08, 1.0: 0x38, 1.125: 0x39,
             1.875: 0x3F, 2.0: 0x40, 256.0: 0x78, 448.0: 0x7E, -1.0: 0xB8, -448.0: 0xFE}
    for v, c in cases.items():
        assert oracle.e4m3_from_f32(v) == c, (v, hex(c))
    assert oracle.e4m3_from_f32(-0.0) == 0x80
    assert oracle.e4m3_from_f32(float("nan")) & 0x7F == 0x7F
    assert np.isnan(oracle.f32_from_e4m3(0x7F)) and np.isnan(oracle.f32_from_e4m3(0xFF))


def test_e4m3_decode_enumerates_the_format():
    dec = np.array([oracle.f32_from_e4m3(c) for c in range(0x7F)])
    assert np.array_equal(dec, POS)                # code order is value order, 127 finite values
    neg = np.array([oracle.f32_from_e4m3(0x80 | c) for c in range(0x7F)])
    assert np.array_equal(neg, -POS)
    assert POS.max() == 448.0


def test_e4m3_round_trip_of_every_finite_code():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        v = oracle.f32_from_e4m3(c)
        assert oracle.e4m3_from_f32(v) == c, hex(c)


def _nearest_code(v):
    """Brute force: the finite code nearest to v, ties to the even code,
    magnitudes beyond 448 clamped to 448."""
    a = min(abs(v), 448.0)
    d = np.abs(POS - a)
    best = np.flatnonzero(d == d.min())
    k = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return k | (0x80 if np.signbit(v) else 0)


def test_e4m3_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(11)
    mids = (POS[1:] + POS[:-1]) / 2                                   # every tie
    vals = np.concatenate([POS, mids, -mids,
                           rng.standard_normal(3000) * np.exp2(rng.integers(-12, 9, 3000)),
                           rng.uniform(440, 600, 200), [1e30, -1e30, 479.9, 480.0, 2.0 ** -10]])
    vals = vals.astype(np.float32)                                     # encoder input is fp32
    for v in vals:
        v = float(v)
        assert oracle.e4m3_from_f32(v) == _nearest_code(v), v


def test_e4m3_ties_round_to_even():
    assert oracle.e4m3_from_f32(1.0625) == 0x38      # between 0x38 and 0x39
    assert oracle.e4m3_from_f32(1.1875) == 0x3A      # between 0x39 and 0x3A
    assert oracle.e4m3_from_f32(2.0 ** -10) == 0x00  # half the smallest subnormal
    assert oracle.e4m3_from_f32(3 * 2.0 ** -10) == 0x02
    assert oracle.e4m3_from_f32(7.5 * 2.0 ** -9) == 0x08   # subnormal/normal boundary
    assert oracle.e4m3_from_f32(464.0) == 0x7E       # halfway to the next binade value: saturates


@pytest.mark.parametrize("amax,byte", [
    (1.0, 119), (1.999, 119), (2.0, 120), (448.0, 127), (255.99, 126), (256.0, 127),
    (2.0 ** -100, 19), (2.0 ** -119, 0), (2.0 ** -130, 0), (0.0, 0), (3.0e38, 246),
])
def test_mx_scale_byte(amax, byte):
    # scale 2^(floor(log2 amax) - 8), byte = exponent + 127, clamped at 0
    assert oracle.mx_scale_byte(amax) == byte


def test_scaled_block_max_lands_in_the_top_binade():
    rng = np.random.default_rng(3)
    for amax in np.abs(rng.standard_normal(500) * np.exp2(rng.integers(-40, 40, 500))).astype(np.float32):
        sb = oracle.mx_scale_byte(float(amax))
        r = float(amax) * 2.0 ** (127 - sb)
        assert 256.0 <= r < 512.0


def _q8_inputs(numel, seed, dtype=oracle.F32):
    rng = np.random.default_rng(seed)
    nb = (numel + 255) // 256
    codes = rng.integers(-127, 128, numel).astype(np.int8)
    absmax = (np.abs(rng.standard_normal(nb)) * 0.05).astype(np.float32)
    g = (rng.standard_normal(numel) * np.exp2(rng.integers(-8, 2, numel))).astype(np.float32)
    if dtype == oracle.F32:
        return codes, absmax, g
    return codes, absmax, (g.view(np.uint32) >> 16).astype(np.uint16) if dtype == oracle.BF16 else \
        g.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("numel", [32, 256, 1024 + 96, 4096])
def test_carrier_update_state_matches_plain_update(numel):
    codes, absmax, g = _q8_inputs(numel, numel)
    c1, a1, p, s, sums1 = oracle.q8_update_carrier(codes, absmax, g, 0.9)
    c2, a2, m, sums2 = oracle.q8_update(codes, absmax, g.copy(), 0.9)
    assert np.array_equal(c1, c2) and np.array_equal(a1.view(np.uint32), a2.view(np.uint32))
    assert np.array_equal(sums1, sums2)
    assert p.shape == (numel,) and s.shape == (numel // 32,)


def test_carrier_update_leaves_the_grad_alone():
    codes, absmax, g = _q8_inputs(512, 5, oracle.BF16)
    before = g.copy()
    oracle.q8_update_carrier(codes, absmax, g, 0.9, dtype=oracle.BF16)
    assert np.array_equal(g, before)


def test_carrier_decodes_to_m_within_e4m3_precision():
    numel = 4096
    codes, absmax, g = _q8_inputs(numel, 7)
    _, _, p, s, _ = oracle.q8_update_carrier(codes, absmax, g, 0.95)
    _, _, m, _ = oracle.q8_update(codes, absmax, g.copy(), 0.95)
    m = m.astype(np.float64)
    dec = oracle.decode_carrier(p, s)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32)
    # half an E4M3 step: 2^-4 relative for normals, 2^-10 scale for subnormals;
    # values above 448 scale saturate
    bound = np.maximum.reduce([np.abs(m) * 2.0 ** -4, scale * 2.0 ** -10, np.abs(m) - 448 * scale])
    assert np.all(np.abs(dec - m) <= bound * (1 + 1e-12))
    # the block scale follows the block maximum
    bm = np.abs(m).reshape(-1, 32).max(axis=1)
    assert np.array_equal(s, np.array([oracle.mx_scale_byte(float(np.float32(v))) for v in bm], np.uint8))


def test_carrier_zero_and_tiny_blocks():
    numel = 256
    codes = np.zeros(numel, np.int8)
    absmax = np.zeros(1, np.float32)
    g = np.zeros(numel, np.float32)
    g[64:96] = 2.0 ** -118                       # m ~ 2^-121.3: scale exponent -130 clamps to -127
    _, _, p, s, _ = oracle.q8_update_carrier(codes, absmax, g, 0.9)
    assert np.all(p[:64] == 0) and np.all(s[:2] == 0) and np.all(p[96:] == 0)
    assert s[2] == 0
    m = (np.float32(1) - np.float32(0.9)) * np.float32(2.0 ** -118)     # (1 - beta) g in fp32
    want = oracle.e4m3_from_f32(float(np.float32(m * np.float32(2.0 ** 127))))
    assert np.all(p[64:96] == want) and want != 0


def test_carrier_rejects_ragged_sizes():
    with pytest.raises(ValueError):
        oracle.q8_update_carrier(np.zeros(40, np.int8), np.zeros(1, np.float32), np.zeros(40, np.float32), 0.9)


# ------------------------------------------------------- transposed carrier
# A tall matrix orthogonalised whole travels as the row-wise carrier of m^T:
# one E8M0 scale per 32 consecutive rows of a column (reading R29).

@pytest.mark.parametrize("rows,cols,dtype", [(512, 256, oracle.F32), (256, 512, oracle.BF16),
                                              (96, 64, oracle.F16)])
def test_transposed_carrier_state_matches_plain_update(rows, cols, dtype):
    codes, absmax, g = _q8_inputs(rows * cols, rows + cols, dtype)
    c1, a1, p, s, sums1 = oracle.q8_update_carrier_t(codes, absmax, g, 0.9, rows, cols, dtype)
    c2, a2, _, sums2 = oracle.q8_update(codes, absmax, g.copy(), 0.9, dtype)
    assert np.array_equal(c1, c2) and np.array_equal(a1.view(np.uint32), a2.view(np.uint32))
    assert np.array_equal(sums1, sums2)
    assert p.shape == (cols, rows) and s.shape == (cols, rows // 32)


def test_transposed_carrier_is_the_rowwise_carrier_of_the_transpose():
    """beta = 0 makes m equal to the fp32 grad exactly, so the transposed
    carrier of g must equal, byte for byte, the row-wise carrier (pinned above
    against the format) of g^T."""
    rows, cols = 256, 96
    codes, absmax, g = _q8_inputs(rows * cols, 11)
    g = g.reshape(rows, cols)
    g[:, 5] = 0.0                                  # a zero column: zero bytes, scale byte 0
    _, _, p, s, _ = oracle.q8_update_carrier_t(codes, absmax, g.reshape(-1), 0.0, rows, cols)
    gt = np.ascontiguousarray(g.T).reshape(-1)
    _, _, p_rw, s_rw, _ = oracle.q8_update_carrier(np.zeros(rows * cols, np.int8),
                                                    np.zeros(rows * cols // 256, np.float32), gt, 0.0)
    assert np.array_equal(p.reshape(-1), p_rw) and np.array_equal(s.reshape(-1), s_rw)
    assert np.all(p[5] == 0) and np.all(s[5] == 0)


def test_transposed_carrier_decodes_to_m_within_e4m3_precision():
    rows, cols = 384, 256
    codes, absmax, g = _q8_inputs(rows * cols, 13)
    _, _, p, s, _ = oracle.q8_update_carrier_t(codes, absmax, g, 0.95, rows, cols)
    _, _, m, _ = oracle.q8_update(codes, absmax, g.copy(), 0.95)
    mt = m.astype(np.float64).reshape(rows, cols).T            # (cols, rows)
    dec = oracle.decode_carrier(p, s).reshape(cols, rows)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    bound = np.maximum.reduce([np.abs(mt) * 2.0 ** -4, scale * 2.0 ** -10, np.abs(mt) - 448 * scale])
    assert np.all(np.abs(dec - mt) <= bound * (1 + 1e-12))
    bm = np.abs(mt).reshape(cols, rows // 32, 32).max(axis=2)
    assert np.array_equal(s, np.vectorize(lambda v: oracle.mx_scale_byte(float(np.float32(v))))(bm).astype(np.uint8))


def test_transposed_carrier_rule_and_shape_checks():
    assert oracle.transposed_carrier_applies(14336, 4096)
    assert not oracle.transposed_carrier_applies(4096, 14336)      # wide: the row-wise carrier
    assert not oracle.transposed_carrier_applies(4096, 4096)       # square: the row-wise carrier
    assert not oracle.transposed_carrier_applies(14336 + 64, 4096)  # rows off the 128 grid
    assert not oracle.transposed_carrier_applies(14336, 4096 + 128)  # cols off the 256 grid
    with pytest.raises(ValueError):
        oracle.q8_update_carrier_t(np.zeros(40 * 8, np.int8), np.zeros(2, np.float32), np.zeros(40 * 8, np.float32),
                                   0.9, 40, 8)
