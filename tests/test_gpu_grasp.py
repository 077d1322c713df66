"""GPU parity of the GRASP 4-bit momentum step.

Each GPU step is compared with the oracle stepped from the GPU's own previous
state, so every step is judged on its own.  Codes and block scales are
expected bit-identical (both sides do the same fp32 operations on the same
fp32 inputs; the fp64 reductions differ only in order).  A code may differ
only by one level and only where the oracle's pre-rounding value lies within
1e-4 of a rounding boundary (a last-bit difference in P or R from the
reduction order); a scale only by 1e-6 relative.  O and the weight change
within the Newton-Schulz bound.
"""
import numpy as np
import pytest
import torch

import quantized_momentum_newton_amd as q
from gpu_util import NS_BF16_COS, NS_BF16_REL, NS_F32_BF16OUT_REL, NS_F32_COS, as_f64, host, ns_parity, ns_whole, say
from harness import inputs as H
from oracle import grasp as OG

pytestmark = pytest.mark.gpu
DEV = "cuda"
COEF = tuple(float(np.float32(c)) for c in H.NS_COEFFS)


def to_oracle(st):
    o = OG.State(st.rows, st.cols, st.rank)
    o.res = OG.unpack_nibbles(host(st.res_codes), st.cols)
    o.res_rmax, o.res_cmax = host(st.res_rmax), host(st.res_cmax)
    o.p, o.p_rmax, o.p_cmax = host(st.p_codes), host(st.p_rmax).reshape(-1, 1), host(st.p_cmax)
    o.r, o.r_rmax, o.r_cmax = host(st.r_codes), host(st.r_rmax).reshape(-1, 1), host(st.r_cmax)
    return o


def _pre(x, rmax, cmax, L, s=64):
    d = np.minimum(np.repeat(rmax, s, axis=1)[:, :x.shape[1]], np.repeat(cmax, s, axis=0)[:x.shape[0], :])
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(d > 0, (x / d).astype(np.float32) * np.float32(L), 0.0)


def check_scales(got, exp, what):
    bad = got != exp
    if bad.any():
        rel = np.abs(got[bad] - exp[bad]) / np.maximum(np.abs(exp[bad]), 1e-30)
        assert rel.max() <= 1e-6 and bad.mean() < 1e-3, (what, int(bad.sum()), rel.max())


def check_codes(got, exp, pre, what):
    bad = got != exp
    if not bad.any():
        return 0
    assert np.all(np.abs(got[bad].astype(int) - exp[bad].astype(int)) == 1), what
    t = pre[bad]
    assert np.all(np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4), (what, t[:5])
    assert bad.mean() < 1e-4, (what, int(bad.sum()))
    return int(bad.sum())


def compare_step(st_gpu, ref, M, P32, R32):
    res = OG.residual(M, P32, R32)
    g = to_oracle(st_gpu)
    n = check_codes(g.res, ref.res, _pre(res, ref.res_rmax, ref.res_cmax, 7), "res codes")
    check_scales(g.res_rmax, ref.res_rmax, "res rmax")
    check_scales(g.res_cmax, ref.res_cmax, "res cmax")
    n += check_codes(g.p, ref.p, _pre(P32, ref.p_rmax, ref.p_cmax, 127), "P codes")
    n += check_codes(g.r, ref.r, _pre(R32, ref.r_rmax, ref.r_cmax, 127), "R codes")
    for a, b, w in ((g.p_rmax, ref.p_rmax, "P rmax"), (g.p_cmax, ref.p_cmax, "P cmax"),
                    (g.r_rmax, ref.r_rmax, "R rmax"), (g.r_cmax, ref.r_cmax, "R cmax")):
        check_scales(a, b, w)
    return n


def _within(got, ref, what):
    rel, cos = ns_parity(got, ref)
    say(f"   {what}: relF {rel:.3e} min cos {cos:.6f}")
    assert rel <= NS_BF16_REL and cos >= NS_BF16_COS, (what, rel, cos)


def _grad(rows, cols, spike, seed, t):
    noise = H.grad((rows, cols), torch.float32, DEV, seed, t)
    return (noise + spike).to(torch.bfloat16)


def test_grasp_small_chain_20_steps():
    rows, cols, k, mu, lr, wd = 256, 192, 8, 0.95, 0.02, 0.01
    spike = H.spike(rows, cols, k, DEV, 5001)
    warm = H.gaussian((cols, k), DEV, 5001)
    st = q.GraspState(rows, cols, k)
    W = H.weights((rows, cols), DEV, 5001)
    hw = host(warm)
    mism = 0
    for t in range(1, 21):
        g = _grad(rows, cols, spike, 5001, t)
        gh = g.float().cpu().numpy()
        prev = to_oracle(st)
        W0 = as_f64(W)
        say("grasp step", t)
        q.grasp_step(st, g, warm, mu=mu, ns_steps=5, coeffs=COEF, eps=H.NS_EPS, weight=W, lr=lr,
                     weight_decay=wd)
        torch.cuda.synchronize()
        ref, M, P32, R32, O = OG.grasp_step(prev, gh, mu, hw, 5, COEF, H.NS_EPS)
        mism += compare_step(st, ref, M, P32, R32)
        _within(as_f64(g), O, f"t{t} O")
        _within(as_f64(W) - W0, OG.apply_weights(W0, O, lr, wd) - W0, f"t{t} dW")
    say("code mismatches over 20 steps:", mism)


@pytest.mark.parametrize("ns_precision", ["f32", "bf16x3"])
def test_grasp_ragged_shape_and_rank4(ns_precision):
    """Edge blocks clipped on both sides (rows 100, cols 77 -> odd packing);
    the NS on fp32 operands, fp32 MFMAs or bf16 MFMAs on a hi + lo split."""
    rows, cols, k = 100, 77, 4
    st = q.GraspState(rows, cols, k)
    warm = H.gaussian((cols, k), DEV, 5002)
    for t in range(1, 4):
        g = H.grad((rows, cols), torch.float32, DEV, 5002, t)
        gh = host(g)
        prev = to_oracle(st)
        q.grasp_step(st, g, warm, ns_steps=5, coeffs=COEF, ns_precision=ns_precision)
        torch.cuda.synchronize()
        ref, M, P32, R32, O = OG.grasp_step(prev, gh, 0.95, host(warm), 5, COEF, H.NS_EPS)
        compare_step(st, ref, M, P32, R32)
        rel, cos = ns_parity(as_f64(g), O)
        assert rel < 1e-4 and cos > 0.99999, (rel, cos)     # fp32 output, f32 NS


@pytest.mark.parametrize("rows,cols,k", [(4160, 256, 8), (320, 192, 16)])
def test_grasp_generic_mgs_path(rows, cols, k):
    """More than 4096 rows, or rank 16: the MGS that keeps its columns in
    global memory rather than in registers; state and NS as elsewhere."""
    spike = H.spike(rows, cols, min(k, 8), DEV, 5003)
    warm = H.gaussian((cols, k), DEV, 5003)
    st = q.GraspState(rows, cols, k)
    hw = host(warm)
    for t in range(1, 4):
        g = _grad(rows, cols, spike, 5003, t)
        gh = g.float().cpu().numpy()
        prev = to_oracle(st)
        say("grasp generic-mgs step", rows, cols, k, t)
        q.grasp_step(st, g, warm, ns_steps=5, coeffs=COEF, eps=H.NS_EPS)
        torch.cuda.synchronize()
        ref, M, P32, R32, O = OG.grasp_step(prev, gh, 0.95, hw, 5, COEF, H.NS_EPS)
        compare_step(st, ref, M, P32, R32)
        _within(as_f64(g), O, f"t{t} O")


@pytest.mark.parametrize("ns_precision", ["f32", "bf16x3"])
def test_grasp_4096_full_size(ns_precision):
    """4096x4096, rank-8 spike of norm 10x the noise, mu = 0.95, 20 steps:
    state checked on every step; NS of the last step, whole, within the
    fp32-operand bound plus the rounding of O into the bf16 grad."""
    cfg = H.grasp_4096_shape()
    rows, cols, k, mu = cfg["rows"], cfg["cols"], cfg["rank"], cfg["mu"]
    spike = H.spike(rows, cols, k, DEV, 1005)
    warm = H.gaussian((cols, k), DEV, 1005)
    hw = host(warm)
    st = q.GraspState(rows, cols, k)
    ws = torch.empty(q.grasp_workspace_bytes(rows, cols, k), dtype=torch.uint8, device=DEV)
    mism = 0
    for t in range(1, cfg["steps"] + 1):
        g = _grad(rows, cols, spike, 1005, t)
        gh = g.float().cpu().numpy()
        prev = to_oracle(st)
        say("grasp 4096x4096 step", t)
        q.grasp_step(st, g, warm, mu=mu, ns_steps=5, coeffs=COEF, eps=H.NS_EPS, ws=ws, ns_precision=ns_precision)
        torch.cuda.synchronize()
        ref, M, P32, R32, _ = OG.grasp_step(prev, gh, mu, hw, 5, COEF, H.NS_EPS, with_ns=False)
        mism += compare_step(st, ref, M, P32, R32)
    rel, cos = ns_parity(as_f64(g), ns_whole(M, 5, COEF, H.NS_EPS))
    say(f"   t20 O (whole, {ns_precision}): relF {rel:.3e} min cos {cos:.7f}")
    assert rel <= NS_F32_BF16OUT_REL and cos >= NS_F32_COS, (rel, cos)
    say("code mismatches over 20 steps:", mism)
