"""Entry points called from several host threads at once.

Each thread works on its own stream, data and workspace.  The kernels are
deterministic (every output tile and every norm partial has one fixed
summation order), so each concurrent result must equal, bit for bit, the
same call made alone afterwards.  A thread whose call fails gets its own
error text back while the others run on.
"""
import threading

import pytest
import torch

import quantized_momentum_newton_amd as q
from gpu_util import say
from harness import inputs as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
COEF = H.NS_COEFFS

CASES = [((512, 1024), torch.bfloat16, "bf16"), ((1024, 512), torch.float32, "f32"),
         ((300, 700), torch.float32, "bf16x3"), ((256, 256), torch.float16, "bf16"),
         ((640, 384), torch.bfloat16, "bf16"), ((200, 200), torch.float32, "f32")]


def _ws(shape, precision):
    return torch.empty(q.ns_workspace_bytes(shape[0], shape[1], 1, precision), dtype=torch.uint8, device=DEV)


def test_concurrent_ns_calls_match_serial():
    inputs = [H.grad(shape, dt, DEV, 3101, i) for i, (shape, dt, _) in enumerate(CASES)]
    outs = [x.clone() for x in inputs]
    wss = [_ws(shape, p) for shape, _, p in CASES]
    streams = [torch.cuda.Stream() for _ in CASES]
    torch.cuda.synchronize()
    start = threading.Barrier(len(CASES) + 1)
    errors = []

    def work(i):
        try:
            start.wait()
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    outs[i].copy_(inputs[i])
                    q.ns_orthogonalize(outs[i], 5, COEF, H.NS_EPS, precision=CASES[i][2], ws=wss[i],
                                       stream=streams[i])
        except Exception as e:  # reported below, with the case
            errors.append((i, repr(e)))

    def bad_call():
        # an argument error on a thread of its own: its message must be its own
        try:
            start.wait()
            y = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
            q.ns_orthogonalize(y, 101, COEF, H.NS_EPS)
        except Exception as e:
            errors.append(("bad", str(e)))

    say("threads:", len(CASES), "ns calls + 1 failing call")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(CASES))]
    threads.append(threading.Thread(target=bad_call))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    bad = [e for e in errors if e[0] == "bad"]
    assert [e for e in errors if e[0] != "bad"] == []
    assert len(bad) == 1 and "steps must lie in [0, 100]" in bad[0][1], bad

    for i, (shape, dt, p) in enumerate(CASES):
        y = inputs[i].clone()
        q.ns_orthogonalize(y, 5, COEF, H.NS_EPS, precision=p, ws=wss[i])
        torch.cuda.synchronize()
        say("  case", shape, dt, p)
        bits = torch.int32 if dt == torch.float32 else torch.int16
        assert torch.equal(y.view(bits), outs[i].view(bits))


def _update_set(i):
    """Two tensors (a bf16 matrix and a ragged fp32 vector) in two groups."""
    shapes = [(256 + 64 * i, 512), (1000 + 37 * i,)]
    dts = [torch.bfloat16, torch.float32]
    trip = []
    for j, (shape, dt) in enumerate(zip(shapes, dts)):
        numel = 1
        for d in shape:
            numel *= d
        c, a = H.prior_state(numel, DEV, 3201 + i, j)
        trip.append((c, a, H.grad(shape, dt, DEV, 3201 + i, j).reshape(-1)))
    segs = [(0, 0, trip[0][2].numel(), 0), (1, 0, trip[1][2].numel(), 1)]
    return trip, segs


def test_concurrent_updates_match_serial():
    n = 4
    live = [_update_set(i) for i in range(n)]
    alone = [([tuple(t.clone() for t in tr) for tr in trip], segs) for trip, segs in live]
    plans = [q.Plan(trip, segs, 2) for trip, segs in live]
    invs = [torch.empty(2, dtype=torch.float32, device=DEV) for _ in range(n)]
    wss = [p.workspace() for p in plans]
    streams = [torch.cuda.Stream() for _ in range(n)]
    torch.cuda.synchronize()
    start = threading.Barrier(n)
    errors = []

    def work(i):
        try:
            start.wait()
            q.qmuon_update_normalize_groups(plans[i], 0.95, H.NS_EPS, True, group_inv_norm=invs[i],
                                            ws=wss[i], stream=streams[i])
        except Exception as e:
            errors.append((i, repr(e)))

    say("threads:", n, "grouped updates")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert errors == []

    for i, (trip, segs) in enumerate(alone):
        inv = torch.empty(2, dtype=torch.float32, device=DEV)
        q.qmuon_update_normalize_groups(q.Plan(trip, segs, 2), 0.95, H.NS_EPS, True, group_inv_norm=inv)
        torch.cuda.synchronize()
        assert torch.equal(inv.view(torch.int32), invs[i].view(torch.int32)), i
        for j, ((c1, a1, g1), (c2, a2, g2)) in enumerate(zip(trip, live[i][0])):
            bits = torch.int32 if g1.dtype == torch.float32 else torch.int16
            assert torch.equal(c1, c2) and torch.equal(a1.view(torch.int32), a2.view(torch.int32)), (i, j)
            assert torch.equal(g1.view(bits), g2.view(bits)), (i, j)
