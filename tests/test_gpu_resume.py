"""Checkpoint and resume ("Quantized Muon Momentum", section "Known
Limitations": checkpoint integration is named there as missing).  The
optimizer state lives in caller-owned buffers, so a checkpoint is a copy of
them (and of the step number, which drives the block-periodic schedule and
the stochastic-rounding stream).  Twenty steps in one run must equal, bit for
bit, ten steps, a copy of the state to the host, fresh device buffers (new
addresses, so new plans) filled from that copy, and ten more steps."""
import numpy as np
import pytest
import torch

import quantized_momentum_newton_amd as q
from gpu_util import host, say
from harness import inputs as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
COEF = tuple(float(np.float32(c)) for c in H.NS_COEFFS)
SHAPES = [(256, 1024, 256, 256), (512, 256, 256, 256)]


def _plans(trip):
    full = q.Plan(trip, [(i, 0, r * c, i) for i, (r, c, _, _) in enumerate(SHAPES)], len(SHAPES))
    segs, g0 = [], 0
    for i, (r, c, br, bc) in enumerate(SHAPES):
        s, ng = H.blocked_segments(r, c, br, bc, i, g0)
        segs += s
        g0 += ng
    return full, q.Plan(trip, segs, g0)


def _fresh(state):
    """Device buffers filled from a host checkpoint [(codes, absmax, W)]."""
    trip, mats = [], []
    for (r, c, br, bc), (codes, absmax, w) in zip(SHAPES, state):
        trip.append((torch.from_numpy(codes).to(DEV), torch.from_numpy(absmax).to(DEV),
                     torch.empty(r * c, dtype=torch.bfloat16, device=DEV)))
        mats.append((r, c, br, bc, torch.from_numpy(w).to(DEV)))
    return trip, mats


def _run(trip, mats, steps, hp):
    full, block = _plans(trip)
    outs = []
    for t in steps:
        for i, (r, c, _, _) in enumerate(SHAPES):
            trip[i][2].copy_(H.grad((r, c), torch.bfloat16, DEV, 6001, i, t).reshape(-1))
        q.muon_step(full, block, mats, t, hp)
        outs.append([tr[2].clone() for tr in trip])
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_muonbp_q8_resume_is_bitwise(rounding):
    hp = q.make_hparams(beta=0.95, eps=1e-7, coeffs=COEF, lr_full=0.02, lr_block=0.01, weight_decay=0.01,
                        rms_scale=0.2, ns_steps=5, period=3, rounding=rounding, seed=77)
    init = []
    for i, (r, c, _, _) in enumerate(SHAPES):
        codes, absmax = H.prior_state(r * c, DEV, 6001, i)
        init.append((host(codes), host(absmax), host(H.weights((r, c), DEV, 6001, i))))
    say("straight 20 steps", rounding)
    trip, mats = _fresh(init)
    straight = _run(trip, mats, range(1, 21), hp)
    end_a = [(host(a), host(b), host(m[4])) for (a, b, _), m in zip(trip, mats)]
    say("10 steps, checkpoint, 10 steps")
    trip, mats = _fresh(init)
    first = _run(trip, mats, range(1, 11), hp)
    ckpt = [(host(a), host(b), host(m[4])) for (a, b, _), m in zip(trip, mats)]
    del trip, mats
    torch.cuda.empty_cache()
    trip, mats = _fresh(ckpt)
    second = _run(trip, mats, range(11, 21), hp)
    end_b = [(host(a), host(b), host(m[4])) for (a, b, _), m in zip(trip, mats)]
    for k, (x, y) in enumerate(zip(straight, first + second)):
        for i in range(len(SHAPES)):
            assert torch.equal(x[i].view(torch.int16), y[i].view(torch.int16)), (k + 1, i)
    for i in range(len(SHAPES)):
        for a, b, what in zip(end_a[i], end_b[i], ("codes", "absmax", "W")):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (i, what)


GRASP_FIELDS = ("res_codes", "res_rmax", "res_cmax", "p_codes", "p_rmax", "p_cmax", "r_codes", "r_rmax", "r_cmax")


def test_grasp_resume_is_bitwise():
    rows, cols, k = 256, 192, 8
    spike = H.spike(rows, cols, k, DEV, 6101)
    warm = H.gaussian((cols, k), DEV, 6101)
    W0 = host(H.weights((rows, cols), DEV, 6101))

    def run(st, W, steps):
        outs = []
        for t in steps:
            g = (H.grad((rows, cols), torch.float32, DEV, 6101, t) + spike).to(torch.bfloat16)
            q.grasp_step(st, g, warm, mu=0.95, ns_steps=5, coeffs=COEF, eps=H.NS_EPS, weight=W, lr=0.02,
                         weight_decay=0.01)
            outs.append(g)
        torch.cuda.synchronize()
        return outs

    say("grasp straight 20 steps")
    st = q.GraspState(rows, cols, k)
    W = torch.from_numpy(W0.copy()).to(DEV)
    straight = run(st, W, range(1, 21))
    end_a = [host(getattr(st, f)) for f in GRASP_FIELDS] + [host(W)]
    say("grasp 10 steps, checkpoint, 10 steps")
    st = q.GraspState(rows, cols, k)
    W = torch.from_numpy(W0.copy()).to(DEV)
    first = run(st, W, range(1, 11))
    ckpt = [host(getattr(st, f)) for f in GRASP_FIELDS] + [host(W)]
    del st, W
    st = q.GraspState(rows, cols, k)
    for f, v in zip(GRASP_FIELDS, ckpt):
        getattr(st, f).copy_(torch.from_numpy(v))
    W = torch.from_numpy(ckpt[-1]).to(DEV)
    second = run(st, W, range(11, 21))
    end_b = [host(getattr(st, f)) for f in GRASP_FIELDS] + [host(W)]
    for t, (x, y) in enumerate(zip(straight, first + second)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), t + 1
    for f, a, b in zip(GRASP_FIELDS + ("W",), end_a, end_b):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f
