"""GPU parity of the full block-periodic Muon step (update + NS + weights).

Int8 state bit-identical to the oracle on every step; the NS output and the
weight change within the bf16 Newton-Schulz bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_momentum_newton_amd as q
from gpu_util import (NS_BF16_COS, NS_BF16_REL, NS_F32_BF16OUT_REL, NS_F32_COS, NS_F32_REL, as_f64,
                      assert_bits_equal, host, host_grad, ns_parity, ns_whole, say)
from harness import inputs as H
from oracle import muonbp

pytestmark = pytest.mark.gpu
DEV = "cuda"
COEF = tuple(float(np.float32(c)) for c in H.NS_COEFFS)


def _within(got, ref, what):
    rel, cos = ns_parity(got, ref)
    say(f"   {what}: relF {rel:.3e} min cos {cos:.6f}")
    assert rel <= NS_BF16_REL and cos >= NS_BF16_COS, (what, rel, cos)


def _plans(trip, mats):
    full = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c, _, _, _) in enumerate(mats)], len(mats))
    segs, g0 = [], 0
    for i, (r, c, br, bc, _) in enumerate(mats):
        s, ng = H.blocked_segments(r, c, br, bc, i, g0)
        segs += s
        g0 += ng
    block = q.Plan(trip, segs, g0)
    return full, block


def test_reduced_muonbp_run_20_steps():
    """Two matrices (64x2048 in 8 column blocks, 512x256 in 2 row blocks),
    P = 5, 20 steps: state bit-exact each step, O and W checked each step."""
    shapes = [(64, 2048, 64, 256), (512, 256, 256, 256)]
    hp = dict(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, lr_block=0.01,
              weight_decay=0.01, rms_scale=0.2, ns_steps=5, period=5)
    trip, mats, W_host, states = [], [], [], []
    for i, (r, c, br, bc) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3001, i)
        g = torch.empty(r * c, dtype=torch.bfloat16, device=DEV)
        w = H.weights((r, c), DEV, 3001, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, br, bc, w))
        W_host.append(as_f64(w))
        states.append((host(codes), host(absmax)))
    full, block = _plans(trip, mats)
    params = q.make_hparams(beta=hp["beta"], eps=hp["eps"], coeffs=COEF, lr_full=hp["lr_full"],
                            lr_block=hp["lr_block"], weight_decay=hp["weight_decay"],
                            rms_scale=hp["rms_scale"], ns_steps=5, period=5)
    for t in range(1, 21):
        for i, (r, c, _, _) in enumerate(shapes):
            trip[i][2].copy_(H.grad((r, c), torch.bfloat16, DEV, 3001, i, t).reshape(-1))
        torch.cuda.synchronize()
        gh = [host_grad(trip[i][2]) for i in range(2)]
        say("step", t)
        q.muon_step(full, block, mats, t, params)
        torch.cuda.synchronize()
        for i, (r, c, br, bc) in enumerate(shapes):
            W2, c2, a2, O, is_full = muonbp.muon_step(
                W_host[i], states[i][0], states[i][1], gh[i], oracle.BF16, t, r, c, br, bc,
                hp["period"], hp["beta"], hp["eps"], COEF, 5, hp["lr_full"], hp["lr_block"],
                hp["rms_scale"], hp["weight_decay"])
            assert is_full == (t % 5 == 0)
            assert_bits_equal(host(trip[i][0]), c2, f"t{t} codes[{i}]")
            assert_bits_equal(host(trip[i][1]), a2, f"t{t} absmax[{i}]")
            states[i] = (c2, a2)
            _within(as_f64(trip[i][2]).reshape(r, c), O, f"t{t} O[{i}]")
            dW_gpu = as_f64(mats[i][4]) - W_host[i]
            _within(dW_gpu, W2 - W_host[i], f"t{t} dW[{i}]")
            W_host[i] = as_f64(mats[i][4])


def test_llama8b_layer_full_step():
    """One full Muon step on the Llama-8B layer: state bit-exact; O and the
    weight change of every matrix, whole, against the fp64 oracle."""
    tensors, segments, ng = H.llama8b_layer_layout()
    trip, mats, hin = [], [], []
    for i, (name, r, c) in enumerate(tensors):
        codes, absmax = H.prior_state(r * c, DEV, 1003, i)
        g = H.grad((r, c), torch.bfloat16, DEV, 1003, i).reshape(-1)
        w = H.weights((r, c), DEV, 1003, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, w))
    torch.cuda.synchronize()
    for i in range(len(tensors)):
        hin.append((host(trip[i][0]), host(trip[i][1]), host_grad(trip[i][2])))
    W0 = [host(m[4]) for m in mats]
    full = q.Plan(trip, segments, ng)
    params = q.make_hparams(lr_full=0.02, rms_scale=0.2, period=1)
    say("llama-8B layer muon_step")
    q.muon_step(full, None, mats, 1, params)
    torch.cuda.synchronize()
    states, outs, S, inv, _ = oracle.update_normalize_groups(
        [(a, b) for a, b, _ in hin], [g for _, _, g in hin], [oracle.BF16] * 7, segments, ng,
        H.BETA, H.NS_EPS, write_normalized=False)
    for i, (name, r, c) in enumerate(tensors):
        assert_bits_equal(host(trip[i][0]), states[i][0], f"codes[{name}]")
        assert_bits_equal(host(trip[i][1]), states[i][1], f"absmax[{name}]")
        m = oracle.widen(outs[i], oracle.BF16).astype(np.float64).reshape(r, c)
        ref = ns_whole(m, 5, COEF, H.NS_EPS, inv_norm=float(inv[i]))
        _within(as_f64(trip[i][2]).reshape(r, c), ref, f"O[{name}]")
        s = 0.2 * math.sqrt(max(r, c))
        dW = host(mats[i][4]).astype(np.float64) - W0[i]
        _within(dW, -0.02 * s * ref, f"dW[{name}]")


def test_f32_grouped_step_stream_k_mixed_k():
    """One full step over 2048 x 4096, 3072 x 3072 and 4096 x 2048 in fp32
    operands: the grouped symmetric products run stream-K over items of
    different K (4096, 3072, 4096), with tiles cut between workgroups and
    between matrices.  State bit-exact; O and the weight change (weight
    decay on) of every matrix, whole, within the fp32-operand bound."""
    shapes = [(2048, 4096), (3072, 3072), (4096, 2048)]
    trip, mats, hin = [], [], []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 1011, i)
        g = H.grad((r, c), torch.bfloat16, DEV, 1011, i).reshape(-1)
        w = H.weights((r, c), DEV, 1011, i)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, w))
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        hin.append((host(trip[i][0]), host(trip[i][1]), host_grad(trip[i][2])))
    W0 = [host(m[4]).astype(np.float64) for m in mats]
    segments = [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)]
    plan = q.Plan(trip, segments, len(shapes))
    params = q.make_hparams(lr_full=0.02, rms_scale=0.2, weight_decay=0.01, period=1, precision="f32")
    say("fp32 grouped muon_step, stream-K symmetric products", shapes)
    q.muon_step(plan, None, mats, 1, params)
    torch.cuda.synchronize()
    states, outs, S, inv, _ = oracle.update_normalize_groups(
        [(a, b) for a, b, _ in hin], [g for _, _, g in hin], [oracle.BF16] * len(shapes), segments, len(shapes),
        H.BETA, H.NS_EPS, write_normalized=False)
    for i, (r, c) in enumerate(shapes):
        assert_bits_equal(host(trip[i][0]), states[i][0], f"codes[{i}]")
        assert_bits_equal(host(trip[i][1]), states[i][1], f"absmax[{i}]")
        m = oracle.widen(outs[i], oracle.BF16).astype(np.float64).reshape(r, c)
        ref = ns_whole(m, 5, COEF, H.NS_EPS, inv_norm=float(inv[i]))
        rel, cos = ns_parity(as_f64(trip[i][2]).reshape(r, c), ref)
        say(f"   O[{i}] {r}x{c}: relF {rel:.3e} min cos {cos:.7f}")
        assert rel <= NS_F32_BF16OUT_REL and cos >= NS_F32_COS, (i, rel, cos)
        s = 0.2 * math.sqrt(max(r, c))
        dW = host(mats[i][4]).astype(np.float64) - W0[i]
        rel, cos = ns_parity(dW, -0.02 * (s * ref + 0.01 * W0[i]))
        say(f"   dW[{i}]: relF {rel:.3e} min cos {cos:.7f}")
        assert rel <= NS_F32_BF16OUT_REL and cos >= NS_F32_COS, (i, rel, cos)


def test_muonbp_full_size_state_and_ns():
    """4096x14336, 8 column blocks, P = 5, 20 steps: the q8 state is
    bit-exact on all 20 steps (it does not depend on NS or W); O and the
    weight change are compared whole at a block step (t = 4: all 8 blocks)
    and at a full step (t = 5)."""
    cfg = H.muonbp_4096x14336_shape()
    r, c, br, bc = cfg["rows"], cfg["cols"], cfg["block_rows"], cfg["block_cols"]
    codes, absmax = H.prior_state(r * c, DEV, 1004, 0)
    g = torch.empty(r * c, dtype=torch.bfloat16, device=DEV)
    w = H.weights((r, c), DEV, 1004, 0)
    trip = [(codes, absmax, g)]
    mats = [(r, c, br, bc, w)]
    full, block = _plans(trip, mats)
    params = q.make_hparams(lr_full=cfg["lr_full"], lr_block=cfg["lr_block"],
                            rms_scale=cfg["rms_scale"], period=cfg["period"], weight_decay=cfg["weight_decay"])
    hc, ha = host(codes), host(absmax)
    bid = muonbp.block_group_ids(r, c, br, bc)
    fid = np.zeros(bid.size, np.int32)
    for t in range(1, cfg["steps"] + 1):
        g.copy_(H.grad((r, c), torch.bfloat16, DEV, 1004, 0, t).reshape(-1))
        torch.cuda.synchronize()
        gh = host_grad(g)
        check_ns = t in (4, 5)
        if check_ns:
            W0 = as_f64(w)
        say("muonbp step", t)
        q.muon_step(full, block, mats, t, params)
        torch.cuda.synchronize()
        hc, ha, m, bs = oracle.q8_update(hc, ha, gh, H.BETA, oracle.BF16)
        assert_bits_equal(host(codes), hc, f"t{t} codes")
        assert_bits_equal(host(absmax), ha, f"t{t} absmax")
        if check_ns:
            is_full = t % 5 == 0
            gid = fid if is_full else bid
            ngr = 1 if is_full else 8
            inv = oracle.group_inv_norm(oracle.group_sums([bs], [gid], ngr), H.NS_EPS)
            mf = oracle.widen(m, oracle.BF16).astype(np.float64).reshape(r, c)
            O = as_f64(g).reshape(r, c)
            dW = as_f64(w) - W0
            if is_full:
                ref = ns_whole(mf, 5, COEF, H.NS_EPS, float(inv[0]))
                s, lr = muonbp.rms_factor(r, c, cfg["rms_scale"]), cfg["lr_full"]
                _within(O, ref, "full O")
                _within(dW, -lr * (s * ref + cfg["weight_decay"] * W0), "full dW")
            else:
                s, lr = muonbp.rms_factor(br, bc, cfg["rms_scale"]), cfg["lr_block"]
                for j in range(8):
                    sl = slice(bc * j, bc * (j + 1))
                    ref = ns_whole(mf[:, sl], 5, COEF, H.NS_EPS, float(inv[j]))
                    _within(O[:, sl], ref, f"block {j} O")
                    _within(dW[:, sl], -lr * (s * ref + cfg["weight_decay"] * W0[:, sl]), f"block {j} dW")


def test_muon_step_on_strided_grad_views():
    """Grads as column slices of one fused buffer (row pitch > row length), P = 2
    over 4 steps (block and full steps): state bit-exact and O, W within the
    bf16 bound against the oracle on contiguous copies; the fused buffer's
    remaining columns are untouched."""
    rows, widths, pad = 512, [256, 512], 64     # block rows must start on 256-element blocks
    blocks = [(256, 256), (512, 256)]
    W = sum(widths) + pad
    buf = torch.zeros((rows, W), dtype=torch.bfloat16, device=DEV)
    views = [buf[:, 0:256], buf[:, 256:768]]
    buf[:, 768:] = 7.0
    trip, mats, W_host, states = [], [], [], []
    for i, (v, (br, bc)) in enumerate(zip(views, blocks)):
        r, c = v.shape
        codes, absmax = H.prior_state(r * c, DEV, 3003, i)
        w = H.weights((r, c), DEV, 3003, i)
        trip.append((codes, absmax, v))
        mats.append((r, c, br, bc, w))
        W_host.append(as_f64(w))
        states.append((host(codes), host(absmax)))
    full, block = _plans(trip, mats)
    params = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, lr_block=0.01,
                            weight_decay=0.0, rms_scale=0.2, ns_steps=5, period=2)
    for t in range(1, 5):
        for i, v in enumerate(views):
            v.copy_(H.grad(tuple(v.shape), torch.bfloat16, DEV, 3003, i, t))
        torch.cuda.synchronize()
        gh = [host_grad(v) for v in views]
        say("strided step", t)
        q.muon_step(full, block, mats, t, params)
        torch.cuda.synchronize()
        for i, v in enumerate(views):
            r, c = v.shape
            br, bc = blocks[i]
            W2, c2, a2, O, is_full = muonbp.muon_step(
                W_host[i], states[i][0], states[i][1], gh[i], oracle.BF16, t, r, c, br, bc,
                2, 0.95, 1e-7, COEF, 5, 0.02, 0.01, 0.2, 0.0)
            assert is_full == (t % 2 == 0)
            assert_bits_equal(host(trip[i][0]), c2, f"t{t} codes[{i}]")
            assert_bits_equal(host(trip[i][1]), a2, f"t{t} absmax[{i}]")
            states[i] = (c2, a2)
            _within(as_f64(v), O, f"t{t} O[{i}]")
            _within(as_f64(mats[i][4]) - W_host[i], W2 - W_host[i], f"t{t} dW[{i}]")
            W_host[i] = as_f64(mats[i][4])
        assert bool((buf[:, 768:] == 7.0).all())


def test_muon_step_stochastic_rounding_state():
    """muon_step with stochastic requantisation: the state after steps 1..3 is
    bit-identical to the oracle's update with the step number as the counter
    offset (the NS half is the one checked by the other tests)."""
    shapes = [(256, 512), (128, 256)]
    seed = 99
    trip, mats, states = [], [], []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 3005, i)
        g = torch.empty(r * c, dtype=torch.bfloat16, device=DEV)
        trip.append((codes, absmax, g))
        mats.append((r, c, r, c, None))
        states.append((host(codes), host(absmax)))
    full, _ = _plans(trip, mats)
    params = q.make_hparams(period=1, rounding="stochastic", seed=seed)
    for t in range(1, 4):
        for i, (r, c) in enumerate(shapes):
            trip[i][2].copy_(H.grad((r, c), torch.bfloat16, DEV, 3005, i, t).reshape(-1))
        torch.cuda.synchronize()
        gh = [host_grad(trip[i][2]) for i in range(2)]
        say("stochastic muon step", t)
        q.muon_step(full, None, mats, t, params)
        torch.cuda.synchronize()
        segs = [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)]
        st, _, _, _, _ = oracle.update_normalize_groups(states, gh, [oracle.BF16] * 2, segs, 2, 0.95, 1e-7, False,
                                                        oracle.ROUND_STOCHASTIC, seed, t)
        for i in range(2):
            assert_bits_equal(host(trip[i][0]), st[i][0], f"t{t} codes[{i}]")
            assert_bits_equal(host(trip[i][1]), st[i][1], f"t{t} absmax[{i}]")
        states = [(c, a) for c, a in st]


@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
def test_fp32_256x512_step_fp32_operands(precision):
    """The single 256x512 fp32 matrix: update, normalise, NS on fp32 operands
    (fp32 MFMAs, or bf16 MFMAs on a hi + lo split) and the weight apply,
    three full steps: state bit-exact, O and dW within the f32 bound."""
    (_, r, c), = H.fp32_256x512_shapes()
    codes, absmax = H.prior_state(r * c, DEV, 3101, 0)
    g = torch.empty(r * c, dtype=torch.float32, device=DEV)
    w = H.weights((r, c), DEV, 3101, 0)
    trip, mats = [(codes, absmax, g)], [(r, c, r, c, w)]
    plan = q.Plan(trip, [(0, 0, r * c, 0)], 1)
    params = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, weight_decay=0.01, ns_steps=5, period=1,
                            precision=precision)
    W_host, state = as_f64(w), (host(codes), host(absmax))
    for t in range(1, 4):
        g.copy_(H.grad((r, c), torch.float32, DEV, 3101, 0, t).reshape(-1))
        torch.cuda.synchronize()
        gh = host_grad(g)
        say("fp32 step", precision, t)
        q.muon_step(plan, None, mats, t, params)
        torch.cuda.synchronize()
        W2, c2, a2, O, is_full = muonbp.muon_step(W_host, state[0], state[1], gh, oracle.F32, t, r, c, r, c, 1, 0.95,
                                                  1e-7, COEF, 5, 0.02, 0.01, 0.2, 0.01)
        assert is_full
        assert_bits_equal(host(codes), c2, f"t{t} codes")
        assert_bits_equal(host(absmax), a2, f"t{t} absmax")
        state = (c2, a2)
        for got, ref, what in ((as_f64(g).reshape(r, c), O, "O"), (as_f64(w) - W_host, W2 - W_host, "dW")):
            rel, cos = ns_parity(got, ref)
            say(f"   t{t} {what}: relF {rel:.3e} min cos {cos:.7f}")
            assert rel <= NS_F32_REL and cos >= NS_F32_COS, (what, rel, cos)
        W_host = as_f64(w)


def test_grouped_products_equal_single_matrix_products():
    """Four matrices of different K in one chunk: 136 + 78 + 36 + 10 = 260
    lower-triangle tiles, more than one round of 256, so the Gram and A^2
    launches deal their tiles evenly over the XCDs.  Each tile's arithmetic
    does not depend on which workgroup computes it, so every output must equal,
    bit for bit, the same matrix orthogonalised alone (one matrix per launch,
    tiles dealt round robin); a tile dealt twice or never would show here."""
    shapes = [(4096, 4096), (3072, 3072), (2048, 8192), (1024, 6144)]
    trip = []
    for i, (r, c) in enumerate(shapes):
        codes, absmax = H.prior_state(r * c, DEV, 4401, i)
        trip.append((codes, absmax, H.grad((r, c), torch.bfloat16, DEV, 4401, i).reshape(-1)))
    mats = [(r, c, r, c, None) for r, c in shapes]
    plan = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c) in enumerate(shapes)], len(shapes))
    inv = torch.empty(len(shapes), dtype=torch.float32, device=DEV)
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, False, group_inv_norm=inv)
    m = [t[2].clone() for t in trip]
    hp = q.make_hparams(period=1)
    ws = torch.empty(q.muon_step_workspace_bytes(plan, None, mats, hparams=hp), dtype=torch.uint8, device=DEV)
    say("grouped:", shapes)
    q.muon_apply(plan, mats, True, inv, hp, ws)
    torch.cuda.synchronize()
    grouped = [t[2].clone() for t in trip]
    for i, (r, c) in enumerate(shapes):
        trip[i][2].copy_(m[i])
        one = q.Plan([trip[i]], [(0, 0, r * c, 0)], 1)
        ws1 = torch.empty(q.muon_step_workspace_bytes(one, None, [mats[i]], hparams=hp), dtype=torch.uint8,
                          device=DEV)
        q.muon_apply(one, [mats[i]], True, inv[i:i + 1].clone(), hp, ws1)
        torch.cuda.synchronize()
        say("  alone:", (r, c))
        assert torch.equal(trip[i][2].view(torch.int16), grouped[i].view(torch.int16)), (r, c)
