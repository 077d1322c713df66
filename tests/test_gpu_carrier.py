"""GPU parity of the MXFP8 carrier path ("Quantized Muon Momentum", section
"Wave18B MXFP8 Carrier Probe"): the update emitting the carrier, Newton-Schulz
reading it, and muon_step in carrier mode.

Codes, absmax, carrier bytes, scale bytes and group inverse norms are
compared bit for bit with the oracle on the same seeded inputs, and the
grads must come back untouched; the NS output within the bf16 bound, and
bit for bit when no iteration runs in fp32 (then it is the decoded carrier
times the inverse norm, one rounding).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_momentum_newton_amd as q
from gpu_util import (NS_BF16_COS, NS_BF16_REL, NS_F32_COS, NS_F32_REL, TORCH_TO_ORACLE, Q8Set, as_f64,
                      assert_bits_equal, host, host_grad, ns_parity, ns_whole, say)
from harness import inputs as H
from oracle import muonbp, ns

pytestmark = pytest.mark.gpu
DEV = "cuda"
COEF = tuple(float(np.float32(c)) for c in H.NS_COEFFS)


def _within(got, ref, what):
    rel, cos = ns_parity(got, ref)
    say(f"   {what}: relF {rel:.3e} min cos {cos:.6f}")
    assert rel <= NS_BF16_REL and cos >= NS_BF16_COS, (what, rel, cos)


def check_carrier(qs, segments, ngroups, beta, eps, idx=None):
    """Carrier update on the GPU over every tensor of qs; tensors idx (all if
    None) and the groups they fully contain are compared with the oracle."""
    idx = list(range(len(qs.shapes))) if idx is None else list(idx)
    plan = q.Plan(qs.triples(), segments, ngroups)
    sums = torch.empty(ngroups, dtype=torch.float64, device=DEV)
    car = q.qmuon_update_mxfp8_carrier(plan, beta, eps, group_sumsq=sums)
    torch.cuda.synchronize()
    bsums = {}
    for i in idx:
        c, a, p, s, bs = oracle.q8_update_carrier(qs.h_codes[i], qs.h_absmax[i], qs.h_grads[i], beta, qs.odt(i))
        assert_bits_equal(host(qs.codes[i]), c, f"codes[{i}]")
        assert_bits_equal(host(qs.absmax[i]), a, f"absmax[{i}]")
        assert_bits_equal(host(car.data(i)), p, f"carrier data[{i}]")
        assert_bits_equal(host(car.scale_inv(i)), s, f"carrier scales[{i}]")
        assert_bits_equal(host_grad(qs.grads[i]).reshape(-1), qs.h_grads[i].reshape(-1), f"grad[{i}] untouched")
        bsums[i] = bs
    # groups lying entirely in the checked tensors
    local = {t: k for k, t in enumerate(idx)}
    outside = {g for (t, _, _, g) in segments if t not in local}
    inside = {g for (t, _, _, g) in segments if t in local} - outside
    gids = oracle.expand_segments([int(np.prod(qs.shapes[i])) for i in idx],
                                  [(local[t], s, ln, g) for (t, s, ln, g) in segments if t in local], ngroups)
    S = oracle.group_sums([bsums[i] for i in idx], gids, ngroups)
    inv = oracle.group_inv_norm(S, eps)
    inv_g, sums_g = host(car.inv_norm), host(sums)
    assert inside
    for g in sorted(inside):
        assert np.isclose(sums_g[g], S[g], rtol=1e-12, atol=0), g
        assert inv_g[g] == inv[g], (g, inv_g[g], inv[g])
    return plan, car


def test_carrier_update_ragged_mixed_dtypes():
    numels = [32, 96, 256, 288, 1024, 1056, 4128, 70016, 3200]
    dts = [torch.float32, torch.bfloat16, torch.float16] * 3
    qs = Q8Set([(n,) for n in numels], dts[:len(numels)], seed=41)
    say("carrier update, ragged mixed dtypes", numels)
    check_carrier(qs, [(i, 0, n, i) for i, n in enumerate(numels)], len(numels), 0.9, 1e-7)


def test_carrier_update_qkv_groups():
    # two layers of hidden 256: fused qkv rows (256 | 32 | 32) in three groups
    shapes, segs, gid = [], [], 0
    for layer in range(2):
        base = len(shapes)
        shapes += [(320, 256), (256, 256), (768, 256), (768, 256), (256, 768)]
        for r0, r1 in ((0, 256), (256, 288), (288, 320)):
            segs.append((base, r0 * 256, (r1 - r0) * 256, gid))
            gid += 1
        for t in range(1, 5):
            r, c = shapes[base + t]
            segs.append((base + t, 0, r * c, gid))
            gid += 1
    qs = Q8Set(shapes, [torch.bfloat16] * len(shapes), seed=42, outlier_frac=0.01)
    say("carrier update, qkv groups", gid)
    check_carrier(qs, segs, gid, H.BETA, H.NS_EPS)


def test_carrier_update_zero_and_beta_edges():
    for beta in (0.0, 1.0):
        qs = Q8Set([(2048,), (800,)], [torch.bfloat16, torch.float32], seed=43)
        qs.grads[0][256:512].zero_()
        qs.codes[0][256:512].zero_()
        torch.cuda.synchronize()
        qs.snapshot()
        say("carrier update, beta", beta)
        check_carrier(qs, [(0, 0, 2048, 0), (1, 0, 800, 1)], 2, beta, 1e-7)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_carrier_update_strided_grad_views(dtype):
    rows, widths, pad = 96, [512, 320, 160], 32
    W = sum(widths) + pad
    buf = H.grad((rows, W), dtype, DEV, 44, 0)
    views, c0 = [], 0
    for w in widths:
        views.append(buf[:, c0:c0 + w])
        c0 += w
    states = [H.prior_state(v.numel(), DEV, 44, i + 1) for i, v in enumerate(views)]
    torch.cuda.synchronize()
    h_buf = host_grad(buf)
    plan = q.Plan([(c, a, v) for (c, a), v in zip(states, views)], [(i, 0, v.numel(), i) for i, v in
                                                                     enumerate(views)], len(views))
    h_states = [(host(c), host(a)) for c, a in states]
    say("carrier update, strided views", dtype)
    car = q.qmuon_update_mxfp8_carrier(plan, H.BETA, H.NS_EPS)
    torch.cuda.synchronize()
    odt = TORCH_TO_ORACLE[dtype]
    c0 = 0
    for i, v in enumerate(views):
        g = np.ascontiguousarray(h_buf[:, c0:c0 + widths[i]]).reshape(-1)
        c0 += widths[i]
        c, a, p, s, _ = oracle.q8_update_carrier(h_states[i][0], h_states[i][1], g, H.BETA, odt)
        assert_bits_equal(host(states[i][0]), c, f"codes[{i}]")
        assert_bits_equal(host(states[i][1]), a, f"absmax[{i}]")
        assert_bits_equal(host(car.data(i)), p, f"data[{i}]")
        assert_bits_equal(host(car.scale_inv(i)), s, f"scales[{i}]")
    assert_bits_equal(host_grad(buf).reshape(-1), h_buf.reshape(-1), "fused grad buffer untouched")


def test_carrier_update_llama8b_layer_full():
    """The Llama-8B layer (7 bf16 tensors, 218M elements): every byte checked."""
    tensors, segments, ng = H.llama8b_layer_layout()
    shapes = [(r, c) for (_, r, c) in tensors]
    qs = Q8Set(shapes, [torch.bfloat16] * len(shapes), seed=45)
    say("carrier update, llama-8B layer")
    check_carrier(qs, segments, ng, H.BETA, H.NS_EPS)


def test_carrier_e4m3_encoding_sweep():
    """Every fp32 pattern of magnitude 2^-12 .. 512 on a 2^12-ulp grid (all
    E4M3 codes, every tie, the values just around ties, saturation), both
    signs.  beta = 0 and a zero state make m the fp32 grad exactly; each
    32-element block leads with 256, so its scale is 2^0 and the payload is
    the E4M3 byte of the value itself."""
    pats = np.arange(0x39800000, 0x44000000, 1 << 12, dtype=np.uint32)
    vals = np.concatenate([pats.view(np.float32), -pats.view(np.float32)])
    nblk32 = -(-vals.size // 31)
    body = np.zeros(nblk32 * 31, np.float32)
    body[:vals.size] = vals
    g = np.concatenate([np.full((nblk32, 1), 256.0, np.float32), body.reshape(nblk32, 31)], axis=1).reshape(-1)
    pad = (-g.size) % 256
    g = np.concatenate([g, np.zeros(pad, np.float32)])
    n = g.size
    codes = torch.zeros(n, dtype=torch.int8, device=DEV)
    absmax = torch.zeros(n // 256, dtype=torch.float32, device=DEV)
    grad = torch.from_numpy(g).to(DEV)
    plan = q.Plan([(codes, absmax, grad)], [(0, 0, n, 0)], 1)
    say("e4m3 sweep", vals.size, "values")
    car = q.qmuon_update_mxfp8_carrier(plan, 0.0, 1e-7)
    torch.cuda.synchronize()
    c, a, p, sc, _ = oracle.q8_update_carrier(np.zeros(n, np.int8), np.zeros(n // 256, np.float32), g, 0.0)
    assert_bits_equal(host(car.data(0)), p, "payload")
    assert_bits_equal(host(car.scale_inv(0)), sc, "scales")
    assert_bits_equal(host(codes), c, "codes")
    assert np.all(sc[:nblk32] == 127)
    # the oracle's bytes for this sweep are the format's nearest codes (its own pins cover the encoder)
    assert p.reshape(-1, 32)[0, 0] == 0x78


def test_carrier_rejects_sizes_off_the_32_grid():
    qs = Q8Set([(1000,)], [torch.bfloat16], seed=46)
    plan = q.Plan(qs.triples(), [(0, 0, 1000, 0)], 1)
    with pytest.raises(q.QmuonError, match="32"):
        q.qmuon_update_mxfp8_carrier(plan, 0.9, 1e-7)
    torch.cuda.synchronize()
    assert_bits_equal(host(qs.codes[0]), qs.h_codes[0], "codes untouched after the rejected call")


def _carrier_input(rows, cols, seed, zero_rows=(), gaussian=False):
    """Carrier arrays on the device, the decoded matrix and its inverse norm.
    Random bytes (every code, scale bytes 110..126), or (gaussian) the
    oracle's carrier of a Gaussian m."""
    if gaussian:
        g = host(H.gaussian((rows, cols), DEV, seed)).reshape(-1) * np.float32(1e-3)
        nb = (rows * cols + 255) // 256
        _, _, p, s, _ = oracle.q8_update_carrier(np.zeros(rows * cols, np.int8), np.zeros(nb, np.float32),
                                                 g, 0.0)
        data = torch.from_numpy(p.reshape(rows, cols)).to(DEV)
        scale = torch.from_numpy(s.reshape(rows, cols // 32)).to(DEV)
    else:
        data, scale = H.carrier_bytes(rows, cols, DEV, seed)
    for r in zero_rows:
        data[r].zero_()
        scale[r].zero_()
    torch.cuda.synchronize()
    m = oracle.decode_carrier(host(data).reshape(-1), host(scale).reshape(-1)).reshape(rows, cols)
    inv = np.float32(1.0 / (np.sqrt(np.sum(m * m)) + 1e-7))
    return data, scale, m, torch.tensor([inv], device=DEV)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ns_mxfp8_no_iteration_is_decode_times_inv(out_dtype):
    """steps = 0 in fp32: O = fl32(decode * inv) exactly; every code of the
    format and zero blocks are present."""
    rows, cols = 200, 352
    data, scale, m, inv = _carrier_input(rows, cols, 47, zero_rows=(3,))
    out = torch.empty(rows, cols, dtype=out_dtype, device=DEV)
    q.ns_orthogonalize_mxfp8(data, scale, inv, out, steps=0, precision="f32")
    torch.cuda.synchronize()
    exp = (m * np.float64(host(inv)[0])).astype(np.float32)
    if out_dtype == torch.float32:
        assert_bits_equal(host(out).reshape(-1), exp.reshape(-1), "O")
    else:
        assert_bits_equal(host_grad(out).reshape(-1), oracle.round_to(exp.reshape(-1), oracle.BF16), "O")


# (256, 512), (1024, 1024), (512, 1536): the first Gram runs on block-scaled fp8
# MFMA (rows a multiple of 256, cols of 128, not tall); the others on bf16
@pytest.mark.parametrize("rows,cols", [(96, 320), (320, 96), (256, 512), (640, 224), (1024, 1024), (512, 1536),
                                       (768, 640)])
def test_ns_mxfp8_matches_oracle(rows, cols):
    data, scale, m, inv = _carrier_input(rows, cols, 48 + rows, gaussian=True)
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=DEV)
    say("ns from carrier", rows, cols)
    q.ns_orthogonalize_mxfp8(data, scale, inv, out, steps=5, coeffs=COEF)
    torch.cuda.synchronize()
    ref = ns.ns_orthogonalize(m, 5, COEF, inv_norm=float(host(inv)[0]))
    _within(as_f64(out), ref, f"O {rows}x{cols}")


def test_ns_mxfp8_into_strided_output():
    rows, cols = 192, 256
    data, scale, m, inv = _carrier_input(rows, cols, 49, gaussian=True)
    big = torch.full((rows, cols + 64), 7.0, dtype=torch.float32, device=DEV)
    out = big[:, 32:32 + cols]
    q.ns_orthogonalize_mxfp8(data, scale, inv, out, steps=5, coeffs=COEF)
    torch.cuda.synchronize()
    ref = ns.ns_orthogonalize(m, 5, COEF, inv_norm=float(host(inv)[0]))
    _within(as_f64(out), ref, "O strided")
    hb = host(big)
    assert np.all(hb[:, :32] == 7.0) and np.all(hb[:, 32 + cols:] == 7.0)


def _plans(trip, mats):
    full = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c, _, _, _) in enumerate(mats)], len(mats))
    segs, g0 = [], 0
    for i, (r, c, br, bc, _) in enumerate(mats):
        s, ng = H.blocked_segments(r, c, br, bc, i, g0)
        segs += s
        g0 += ng
    return full, q.Plan(trip, segs, g0)


def test_muon_step_carrier_mode_muonbp():
    """Two matrices, P = 3, 6 steps (two full) with the carrier hand-off: the
    state bit-exact every step, O and dW from the decoded carrier."""
    shapes = [(64, 2048, 64, 256), (512, 256, 256, 256)]
    trip, mats, W_host, states = [], [], [], []
    for i, (r, c, br, bc) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3101, i)
        g = torch.empty(r * c, dtype=torch.bfloat16, device=DEV)
        w = H.weights((r, c), DEV, 3101, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, br, bc, w))
        W_host.append(as_f64(w))
        states.append((host(codes), host(absmax)))
    full, block = _plans(trip, mats)
    params = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, lr_block=0.01,
                            weight_decay=0.01, rms_scale=0.2, ns_steps=5, period=3, carrier=True)
    assert q.muon_step_workspace_bytes(full, block, mats, hparams=params) > \
        q.muon_step_workspace_bytes(full, block, mats)
    for t in range(1, 7):
        for i, (r, c, _, _) in enumerate(shapes):
            trip[i][2].copy_(H.grad((r, c), torch.bfloat16, DEV, 3101, i, t).reshape(-1))
        torch.cuda.synchronize()
        gh = [host_grad(trip[i][2]) for i in range(2)]
        say("carrier step", t)
        q.muon_step(full, block, mats, t, params)
        torch.cuda.synchronize()
        for i, (r, c, br, bc) in enumerate(shapes):
            W2, c2, a2, O, is_full = muonbp.muon_step(
                W_host[i], states[i][0], states[i][1], gh[i], oracle.BF16, t, r, c, br, bc, 3, 0.95, 1e-7,
                COEF, 5, 0.02, 0.01, 0.2, 0.01, carrier=True)
            assert is_full == (t % 3 == 0)
            assert_bits_equal(host(trip[i][0]), c2, f"t{t} codes[{i}]")
            assert_bits_equal(host(trip[i][1]), a2, f"t{t} absmax[{i}]")
            states[i] = (c2, a2)
            _within(as_f64(trip[i][2]).reshape(r, c), O, f"t{t} O[{i}]")
            _within(as_f64(mats[i][4]) - W_host[i], W2 - W_host[i], f"t{t} dW[{i}]")
            W_host[i] = as_f64(mats[i][4])


def test_muon_step_carrier_mode_llama8b_layer():
    """One full carrier-mode step on the Llama-8B layer: state bit-exact, O
    and dW of every matrix, whole, against NS of the decoded carrier (gate
    and up travel as the carrier of m^T, so every first Gram runs on fp8)."""
    tensors, segments, ng = H.llama8b_layer_layout()
    trip, mats, hin = [], [], []
    for i, (name, r, c) in enumerate(tensors):
        codes, absmax = H.prior_state(r * c, DEV, 1103, i)
        g = H.grad((r, c), torch.bfloat16, DEV, 1103, i).reshape(-1)
        w = H.weights((r, c), DEV, 1103, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, w))
    torch.cuda.synchronize()
    for i in range(len(tensors)):
        hin.append((host(trip[i][0]), host(trip[i][1]), host_grad(trip[i][2])))
    W0 = [host(m[4]) for m in mats]
    full = q.Plan(trip, segments, ng)
    params = q.make_hparams(lr_full=0.02, rms_scale=0.2, period=1, carrier=True)
    say("llama-8B layer muon_step, carrier mode")
    q.muon_step(full, None, mats, 1, params)
    torch.cuda.synchronize()
    for i, (name, r, c) in enumerate(tensors):
        if oracle.transposed_carrier_applies(r, c):    # gate, up: the carrier of m^T (R29)
            c2, a2, p, s, bs = oracle.q8_update_carrier_t(hin[i][0], hin[i][1], hin[i][2], H.BETA, r, c, oracle.BF16)
            m = oracle.decode_carrier(p, s).reshape(c, r).T
        else:
            c2, a2, p, s, bs = oracle.q8_update_carrier(hin[i][0], hin[i][1], hin[i][2], H.BETA, oracle.BF16)
            m = oracle.decode_carrier(p, s).reshape(r, c)
        assert_bits_equal(host(trip[i][0]), c2, f"codes[{name}]")
        assert_bits_equal(host(trip[i][1]), a2, f"absmax[{name}]")
        inv = oracle.group_inv_norm(oracle.group_sums([bs], [np.zeros(bs.size, np.int32)], 1), H.NS_EPS)[0]
        ref = ns_whole(m, 5, COEF, H.NS_EPS, inv_norm=float(np.float32(inv)))
        _within(as_f64(trip[i][2]).reshape(r, c), ref, f"O[{name}]")
        sc = 0.2 * math.sqrt(max(r, c))
        dW = host(mats[i][4]).astype(np.float64) - W0[i]
        _within(dW, -0.02 * sc * ref, f"dW[{name}]")


@pytest.mark.parametrize("steps", [1, 2])
def test_ns_mxfp8_first_gram_few_steps(steps):
    """T = 1, 2 on a shape whose first Gram runs on fp8 MFMA: the output is
    dominated by that product, so an error in it (scale association, lane
    layout, the alpha = inv^2 factor) shows directly."""
    rows, cols = 512, 1024
    data, scale, m, inv = _carrier_input(rows, cols, 50, gaussian=True)
    out = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
    q.ns_orthogonalize_mxfp8(data, scale, inv, out, steps=steps, coeffs=COEF)
    torch.cuda.synchronize()
    ref = ns.ns_orthogonalize(m, steps, COEF, inv_norm=float(host(inv)[0]))
    _within(host(out).astype(np.float64), ref, f"O T={steps}")


def test_ns_mxfp8_scales_vary_per_block():
    """Random bytes with scale bytes spread over 100..140 (per-32 scales that
    differ by up to 2^40 within a row): each lane's fp8 values must meet their
    own block's scale."""
    rows, cols = 256, 1024
    data, scale = H.carrier_bytes(rows, cols, DEV, 51, scale_lo=100, scale_hi=140)
    torch.cuda.synchronize()
    m = oracle.decode_carrier(host(data).reshape(-1), host(scale).reshape(-1)).reshape(rows, cols)
    inv = torch.tensor([np.float32(1.0 / (np.sqrt(np.sum(m * m)) + 1e-7))], device=DEV)
    out = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
    q.ns_orthogonalize_mxfp8(data, scale, inv, out, steps=1, coeffs=COEF)
    torch.cuda.synchronize()
    ref = ns.ns_orthogonalize(m, 1, COEF, inv_norm=float(host(inv)[0]))
    _within(host(out).astype(np.float64), ref, "O T=1, wide scale spread")


def test_muon_step_carrier_mode_fp8_gram():
    """Carrier-mode steps where every matrix is wide with rows a multiple of
    256 and cols of 128, so the first Gram of each step runs on fp8 MFMA:
    state bit-exact, O and dW from the decoded carrier."""
    shapes = [(256, 1024), (512, 2048), (768, 768)]
    trip, mats, W_host, states = [], [], [], []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3201, i)
        g = torch.empty(r * c, dtype=torch.bfloat16, device=DEV)
        w = H.weights((r, c), DEV, 3201, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, w))
        W_host.append(as_f64(w))
        states.append((host(codes), host(absmax)))
    plan = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)], len(shapes))
    params = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, weight_decay=0.01, rms_scale=0.2,
                            ns_steps=5, period=1, carrier=True)
    for t in (1, 2):
        for i, (r, c) in enumerate(shapes):
            trip[i][2].copy_(H.grad((r, c), torch.bfloat16, DEV, 3201, i, t).reshape(-1))
        torch.cuda.synchronize()
        gh = [host_grad(trip[i][2]) for i in range(len(shapes))]
        say("fp8-gram carrier step", t)
        q.muon_step(plan, None, mats, t, params)
        torch.cuda.synchronize()
        for i, (r, c) in enumerate(shapes):
            W2, c2, a2, O, _ = muonbp.muon_step(
                W_host[i], states[i][0], states[i][1], gh[i], oracle.BF16, t, r, c, r, c, 1, 0.95, 1e-7,
                COEF, 5, 0.02, 0.02, 0.2, 0.01, carrier=True)
            assert_bits_equal(host(trip[i][0]), c2, f"t{t} codes[{i}]")
            assert_bits_equal(host(trip[i][1]), a2, f"t{t} absmax[{i}]")
            states[i] = (c2, a2)
            _within(as_f64(trip[i][2]).reshape(r, c), O, f"t{t} O[{i}]")
            _within(as_f64(mats[i][4]) - W_host[i], W2 - W_host[i], f"t{t} dW[{i}]")
            W_host[i] = as_f64(mats[i][4])


def test_muon_step_carrier_mode_strided_views():
    """Carrier mode with grads as column slices of one fused buffer, P = 2
    over 4 steps: the carrier is dense whatever the grad's pitch, O lands in
    the views, the buffer's other columns stay untouched."""
    rows, widths, pad = 512, [256, 512], 64
    blocks = [(256, 256), (512, 256)]
    buf = torch.zeros((rows, sum(widths) + pad), dtype=torch.bfloat16, device=DEV)
    views = [buf[:, 0:256], buf[:, 256:768]]
    buf[:, 768:] = 7.0
    trip, mats, W_host, states = [], [], [], []
    for i, (v, (br, bc)) in enumerate(zip(views, blocks)):
        r, c = v.shape
        codes, absmax = H.prior_state(r * c, DEV, 3301, i)
        w = H.weights((r, c), DEV, 3301, i)
        trip.append((codes, absmax, v))
        mats.append((r, c, br, bc, w))
        W_host.append(as_f64(w))
        states.append((host(codes), host(absmax)))
    full, block = _plans(trip, mats)
    params = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, lr_block=0.01, rms_scale=0.2,
                            ns_steps=5, period=2, carrier=True)
    for t in range(1, 5):
        for i, v in enumerate(views):
            v.copy_(H.grad(tuple(v.shape), torch.bfloat16, DEV, 3301, i, t))
        torch.cuda.synchronize()
        gh = [host_grad(v) for v in views]
        say("carrier strided step", t)
        q.muon_step(full, block, mats, t, params)
        torch.cuda.synchronize()
        for i, v in enumerate(views):
            r, c = v.shape
            br, bc = blocks[i]
            W2, c2, a2, O, _ = muonbp.muon_step(W_host[i], states[i][0], states[i][1], gh[i], oracle.BF16, t, r, c,
                                                br, bc, 2, 0.95, 1e-7, COEF, 5, 0.02, 0.01, 0.2, 0.0, carrier=True)
            assert_bits_equal(host(trip[i][0]), c2, f"t{t} codes[{i}]")
            assert_bits_equal(host(trip[i][1]), a2, f"t{t} absmax[{i}]")
            states[i] = (c2, a2)
            _within(as_f64(v), O, f"t{t} O[{i}]")
            _within(as_f64(mats[i][4]) - W_host[i], W2 - W_host[i], f"t{t} dW[{i}]")
            W_host[i] = as_f64(mats[i][4])
        assert bool((buf[:, 768:] == 7.0).all())


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_muon_step_carrier_mode_other_grad_dtypes(dtype):
    """Carrier mode with fp32 and f16 grads: the update reads them, the carrier
    is the same format, O is written back in the grad's dtype."""
    shapes = [(256, 512), (512, 256)]
    trip, mats, states = [], [], []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3401, i)
        g = H.grad((r, c), dtype, DEV, 3401, i).reshape(-1)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, None))
        states.append((host(codes), host(absmax)))
    torch.cuda.synchronize()
    gh = [host_grad(t[2]) for t in trip]
    plan = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)], len(shapes))
    params = q.make_hparams(coeffs=COEF, period=1, carrier=True)
    say("carrier step, grads", dtype)
    q.muon_step(plan, None, mats, 1, params)
    torch.cuda.synchronize()
    odt = TORCH_TO_ORACLE[dtype]
    for i, (r, c) in enumerate(shapes):
        _, c2, a2, O, _ = muonbp.muon_step(np.zeros((r, c), np.float32), states[i][0], states[i][1], gh[i], odt, 1,
                                           r, c, r, c, 1, H.BETA, H.NS_EPS, COEF, 5, 0.0, 0.0, 0.2, carrier=True)
        assert_bits_equal(host(trip[i][0]), c2, f"codes[{i}]")
        assert_bits_equal(host(trip[i][1]), a2, f"absmax[{i}]")
        _within(as_f64(trip[i][2]).reshape(r, c), O, f"O[{i}] ({dtype})")


@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
def test_muon_step_carrier_mode_fp32_operand_ns(precision):
    """Carrier mode with an NS on fp32 operands: the prologue decodes the
    carrier times the group inverse norm into fp32 X (exact decode, one fp32
    rounding), the products run in f32 or bf16x3; O within the f32 bound."""
    shapes = [(256, 512), (512, 256)]
    trip, mats, states = [], [], []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3501, i)
        g = H.grad((r, c), torch.float32, DEV, 3501, i).reshape(-1)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, None))
        states.append((host(codes), host(absmax)))
    torch.cuda.synchronize()
    gh = [host_grad(t[2]) for t in trip]
    plan = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)], len(shapes))
    params = q.make_hparams(coeffs=COEF, period=1, carrier=True, precision=precision)
    say("carrier step, fp32-operand NS", precision)
    q.muon_step(plan, None, mats, 1, params)
    torch.cuda.synchronize()
    for i, (r, c) in enumerate(shapes):
        _, c2, a2, O, _ = muonbp.muon_step(np.zeros((r, c), np.float32), states[i][0], states[i][1], gh[i],
                                           oracle.F32, 1, r, c, r, c, 1, H.BETA, H.NS_EPS, COEF, 5, 0.0, 0.0, 0.2,
                                           carrier=True)
        assert_bits_equal(host(trip[i][0]), c2, f"codes[{i}]")
        assert_bits_equal(host(trip[i][1]), a2, f"absmax[{i}]")
        rel, cos = ns_parity(as_f64(trip[i][2]).reshape(r, c), O)
        say(f"   O[{i}]: relF {rel:.3e} min cos {cos:.7f}")
        assert rel <= NS_F32_REL and cos >= NS_F32_COS, (i, rel, cos)


def test_muon_step_transposed_carrier_bytes():
    """Tall matrices orthogonalised whole travel as the carrier of m^T (one
    E8M0 byte per 32 rows of a column): the bytes and scales the update writes
    into the step's workspace equal the oracle's, bit for bit, as do the state
    and the group norms; a wide matrix beside them keeps the row-wise carrier;
    O and dW within the bf16 bound."""
    shapes = [(512, 256), (384, 256), (256, 512), (1024, 512)]
    trip, mats, W_host, states = [], [], [], []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3601, i)
        g = H.grad((r, c), torch.bfloat16, DEV, 3601, i).reshape(-1)
        w = H.weights((r, c), DEV, 3601, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, w))
        W_host.append(as_f64(w))
        states.append((host(codes), host(absmax)))
    torch.cuda.synchronize()
    gh = [host_grad(t[2]) for t in trip]
    plan = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)], len(shapes))
    params = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, weight_decay=0.01, rms_scale=0.2,
                            ns_steps=5, period=1, carrier=True)
    ws = torch.empty(q.muon_step_workspace_bytes(plan, None, mats, hparams=params), dtype=torch.uint8, device=DEV)
    say("transposed-carrier step", shapes)
    q.muon_step(plan, None, mats, 1, params, ws=ws)
    torch.cuda.synchronize()
    upd = -(-plan.workspace_bytes() // 256) * 256
    nb = plan.n_blocks
    cdata = host(ws[upd:upd + nb * 256])
    s0 = upd + -(-nb * 256 // 256) * 256
    cscale = host(ws[s0:s0 + nb * 8])
    for i, (r, c) in enumerate(shapes):
        b0 = plan.block_offsets[i]
        if oracle.transposed_carrier_applies(r, c):
            c2, a2, p, s, _ = oracle.q8_update_carrier_t(states[i][0], states[i][1], gh[i], 0.95, r, c, oracle.BF16)
        else:
            c2, a2, p, s, _ = oracle.q8_update_carrier(states[i][0], states[i][1], gh[i], 0.95, oracle.BF16)
        assert_bits_equal(host(trip[i][0]), c2, f"codes[{i}]")
        assert_bits_equal(host(trip[i][1]), a2, f"absmax[{i}]")
        assert_bits_equal(cdata[b0 * 256:b0 * 256 + r * c], p.reshape(-1), f"carrier data[{i}]")
        assert_bits_equal(cscale[b0 * 8:b0 * 8 + r * c // 32], s.reshape(-1), f"carrier scales[{i}]")
        W2, _, _, O, _ = muonbp.muon_step(W_host[i], states[i][0], states[i][1], gh[i], oracle.BF16, 1, r, c, r, c,
                                          1, 0.95, 1e-7, COEF, 5, 0.02, 0.02, 0.2, 0.01, carrier=True)
        _within(as_f64(trip[i][2]).reshape(r, c), O, f"O[{i}]")
        _within(as_f64(mats[i][4]) - W_host[i], W2 - W_host[i], f"dW[{i}]")
