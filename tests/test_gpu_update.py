"""GPU parity of the q8 momentum update and grouped normalisation.

Int8 codes, absmax and the stored m are compared bit for bit with the CPU
oracle on the same seeded inputs; per-block sums of squares to fp64 rounding
(the reduction orders differ); group inverse norms and normalised grads bit
for bit (both sides reduce in fp64 before the one fp32 rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_momentum_newton_amd as q
from gpu_util import TORCH_TO_ORACLE, Q8Set, assert_bits_equal, host, host_grad, say
from harness import inputs as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_and_compare(qs, segments, ngroups, beta, eps, check_idx=None, write_normalized=True):
    """Run update+normalize on the GPU over every tensor of qs; compare the
    tensors in check_idx (all if None) and the groups they fully contain."""
    idx = list(range(len(qs.shapes))) if check_idx is None else list(check_idx)
    plan = q.Plan(qs.triples(), segments, ngroups)
    inv = torch.empty(ngroups, dtype=torch.float32, device=DEV)
    sums = torch.empty(ngroups, dtype=torch.float64, device=DEV)
    q.qmuon_update_normalize_groups(plan, beta, eps, write_normalized, group_inv_norm=inv,
                                    group_sumsq=sums)
    torch.cuda.synchronize()
    # oracle on the checked tensors only: groups fully inside them
    local = {t: k for k, t in enumerate(idx)}
    segs_local = [(local[t], s, ln, g) for (t, s, ln, g) in segments if t in local]
    groups = sorted({g for (_, _, _, g) in segs_local})
    gmap = {g: k for k, g in enumerate(groups)}
    groups_outside = {g for (t, _, _, g) in segments if t not in local}
    segs_local = [(t, s, ln, gmap[g]) for (t, s, ln, g) in segs_local]
    states, outs, S, inv_o, _ = oracle.update_normalize_groups(
        qs.host_states(idx), [qs.h_grads[i] for i in idx], [qs.odt(i) for i in idx],
        segs_local, len(groups), beta, eps, write_normalized)
    for k, i in enumerate(idx):
        assert_bits_equal(host(qs.codes[i]), states[k][0], f"codes[{i}]")
        assert_bits_equal(host(qs.absmax[i]), states[k][1], f"absmax[{i}]")
    inv_g, sums_g = host(inv), host(sums)
    complete = [g for g in groups if g not in groups_outside]
    for g in complete:
        assert np.isclose(sums_g[g], S[gmap[g]], rtol=1e-12, atol=0), g
        assert inv_g[g] == inv_o[gmap[g]], (g, inv_g[g], inv_o[gmap[g]])
    for k, i in enumerate(idx):
        tensor_groups = {g for (t, _, _, g) in segments if t == i}
        if write_normalized and not tensor_groups <= set(complete):
            continue
        assert_bits_equal(host_grad(qs.grads[i]), outs[k], f"grad[{i}]")
    return plan


def test_update_multi_ragged_mixed_dtypes():
    numels = [1, 255, 256, 257, 1000, 1023, 1024, 1025, 4097, 70001]
    dts = [torch.float32, torch.bfloat16, torch.float16] * 4
    qs = Q8Set([(n,) for n in numels], dts[:len(numels)], seed=11)
    say("ragged multi-tensor update", numels)
    plan = q.Plan(qs.triples(), [(i, 0, n, 0) for i, n in enumerate(numels)], 1)
    bs = torch.empty(plan.n_blocks, dtype=torch.float64, device=DEV)
    q.qmuon_update_multi(plan, 0.9, block_sumsq=bs)
    torch.cuda.synchronize()
    bs = host(bs)
    off = 0
    for i, n in enumerate(numels):
        c, a, m, s = oracle.q8_update(qs.h_codes[i], qs.h_absmax[i], qs.h_grads[i], 0.9, qs.odt(i))
        assert_bits_equal(host(qs.codes[i]), c, f"codes[{i}]")
        assert_bits_equal(host(qs.absmax[i]), a, f"absmax[{i}]")
        assert_bits_equal(host_grad(qs.grads[i]), m, f"m[{i}]")
        assert np.allclose(bs[off:off + a.size], s, rtol=1e-12, atol=1e-300)
        off += a.size


def test_update_without_sums_matches():
    qs = Q8Set([(3000,), (512,)], [torch.bfloat16, torch.float32], seed=12)
    plan = q.Plan(qs.triples(), [(0, 0, 3000, 0), (1, 0, 512, 0)], 1)
    q.qmuon_update_multi(plan, 0.95)
    torch.cuda.synchronize()
    for i in range(2):
        c, a, m, _ = oracle.q8_update(qs.h_codes[i], qs.h_absmax[i], qs.h_grads[i], 0.95, qs.odt(i))
        assert_bits_equal(host(qs.codes[i]), c, "codes")
        assert_bits_equal(host(qs.absmax[i]), a, "absmax")
        assert_bits_equal(host_grad(qs.grads[i]), m, "m")


def test_single_256x512_fp32():
    qs = Q8Set([(256, 512)], [torch.float32], seed=1001)
    say("256x512 fp32 update+normalize")
    run_and_compare(qs, [(0, 0, 256 * 512, 0)], 1, H.BETA, H.NS_EPS)


@pytest.mark.parametrize("write_normalized", [True, False])
def test_qkv_groups_reduced_layer_set(write_normalized):
    # the 28-layer layout shrunk to 2 layers of hidden 256 (q 256, k 32, v 32 rows)
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
    qs = Q8Set(shapes, [torch.bfloat16] * len(shapes), seed=1002, outlier_frac=0.01)
    say("reduced layer set, groups", gid, "normalized", write_normalized)
    run_and_compare(qs, segs, gid, H.BETA, H.NS_EPS, write_normalized=write_normalized)


def test_interleaved_qkv_segments():
    """The page's interleaved QKV shape (4096, 3584) with split (2, 1, 1):
    a repeating q, q, k, v row pattern, 3072 segments, 57344 blocks."""
    rows, cols = 4096, 3584
    segs = []
    for r in range(0, rows, 4):
        segs.append((0, r * cols, 2 * cols, 0))
        segs.append((0, (r + 2) * cols, cols, 1))
        segs.append((0, (r + 3) * cols, cols, 2))
    qs = Q8Set([(rows, cols)], [torch.bfloat16], seed=1006)
    say("interleaved qkv", len(segs), "segments")
    plan = run_and_compare(qs, segs, 3, H.BETA, H.NS_EPS)
    assert plan.n_blocks == 57344 and len(segs) == 3072


def test_layerset28_full_size():
    """All 140 tensors of the 28-layer set in the benchmark's launch: every
    tensor's codes, absmax and normalised grad bit for bit, every one of the
    196 group sums (rtol 1e-12) and inverse norms (bit for bit) against the
    oracle."""
    tensors, segments, ng = H.layerset28_layout()
    shapes = [(r, c) for (_, r, c) in tensors]
    qs = Q8Set.__new__(Q8Set)
    qs.shapes, qs.dtypes = shapes, [torch.bfloat16] * len(shapes)
    qs.codes, qs.absmax, qs.grads = [], [], []
    for i, shape in enumerate(shapes):
        c, a = H.prior_state(shape[0] * shape[1], DEV, 1002, i)
        g = H.grad(shape, torch.bfloat16, DEV, 1002, i, outlier_frac=0.01).reshape(-1)
        qs.codes.append(c)
        qs.absmax.append(a)
        qs.grads.append(g)
    torch.cuda.synchronize()
    qs.snapshot()
    say("28-layer set, 140 tensors,", ng, "groups")
    assert len(shapes) == 140 and ng == 196
    run_and_compare(qs, segments, ng, H.BETA, H.NS_EPS)


def test_llama8b_layer_update_full():
    tensors, segments, ng = H.llama8b_layer_layout()
    shapes = [(r, c) for (_, r, c) in tensors]
    qs = Q8Set(shapes, [torch.bfloat16] * len(shapes), seed=1003)
    say("llama-8B layer update+normalize")
    run_and_compare(qs, segments, ng, H.BETA, H.NS_EPS)


def test_beta_edges_and_zero_block():
    for beta in (0.0, 1.0):
        qs = Q8Set([(2048,), (777,)], [torch.bfloat16, torch.float32], seed=1007)
        run_and_compare(qs, [(0, 0, 2048, 0), (1, 0, 777, 1)], 2, beta, 1e-7)
    # zero state and zero grad in one block, zero group
    qs = Q8Set([(1024,), (512,)], [torch.bfloat16, torch.bfloat16], seed=1008)
    qs.codes[0][256:512] = 0
    qs.grads[0][256:512] = 0
    qs.codes[1].zero_()
    qs.grads[1].zero_()
    torch.cuda.synchronize()
    qs.snapshot()
    run_and_compare(qs, [(0, 0, 1024, 0), (1, 0, 512, 1)], 2, 0.95, 1e-7)
    assert host(qs.absmax[0])[1] == 0 and np.all(host(qs.absmax[1]) == 0)


def test_repeated_steps_state_chain():
    """Twenty steps with fresh grads: the GPU state stays bit-identical to
    the oracle's state chain (the page's repeated-update drift test, here
    against the exact CPU definition)."""
    shapes = [(96, 300), (1000,)]
    dts = [torch.bfloat16, torch.float16]
    qs = Q8Set(shapes, dts, seed=1009)
    hc = [qs.h_codes[i] for i in range(2)]
    ha = [qs.h_absmax[i] for i in range(2)]
    plan = q.Plan(qs.triples(), [(0, 0, 96 * 300, 0), (1, 0, 1000, 1)], 2)
    for step in range(20):
        for i, shape in enumerate(shapes):
            qs.grads[i].copy_(H.grad(shape, dts[i], DEV, 1009, i, step).reshape(-1))
        torch.cuda.synchronize()
        hg = [host_grad(qs.grads[i]) for i in range(2)]
        q.qmuon_update_multi(plan, 0.95)
        torch.cuda.synchronize()
        for i in range(2):
            hc[i], ha[i], m, _ = oracle.q8_update(hc[i], ha[i], hg[i], 0.95, qs.odt(i))
            assert_bits_equal(host(qs.codes[i]), hc[i], f"step {step} codes[{i}]")
            assert_bits_equal(host(qs.absmax[i]), ha[i], f"step {step} absmax[{i}]")
            assert_bits_equal(host_grad(qs.grads[i]), m, f"step {step} m[{i}]")


def test_determinism_and_canaries():
    """Two runs from identical inputs give identical bits, and nothing is
    written outside the tensors (guard regions around every buffer)."""
    n = 5000
    pad = 4096
    results = []
    for rep in range(2):
        big_c = torch.full((n + 2 * pad,), 99, dtype=torch.int8, device=DEV)
        big_a = torch.full(((n + 255) // 256 + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
        big_g = torch.full((n + 2 * pad,), 3.0, dtype=torch.bfloat16, device=DEV)
        c, a = H.prior_state(n, DEV, 1010)
        g = H.grad((n,), torch.bfloat16, DEV, 1010)
        big_c[pad:pad + n] = c
        big_a[pad:pad + a.numel()] = a
        big_g[pad:pad + n] = g
        views = (big_c[pad:pad + n], big_a[pad:pad + a.numel()], big_g[pad:pad + n])
        plan = q.Plan([views], [(0, 0, n, 0)], 1)
        inv = torch.empty(1, dtype=torch.float32, device=DEV)
        q.qmuon_update_normalize_groups(plan, 0.95, 1e-7, True, group_inv_norm=inv)
        torch.cuda.synchronize()
        hc, ha, hg = host(big_c), host(big_a), host_grad(big_g)
        assert np.all(hc[:pad] == 99) and np.all(hc[pad + n:] == 99)
        assert np.all(ha[:pad] == 7.0) and np.all(ha[pad + a.numel():] == 7.0)
        gg = hg.view(np.uint16)
        three = np.float32(3.0).view(np.uint32) >> 16
        assert np.all(gg[:pad] == three) and np.all(gg[pad + n:] == three)
        results.append((hc, ha, hg, host(inv)))
    for x, y in zip(results[0], results[1]):
        assert np.array_equal(x, y)


def test_launch_timing_records_each_kernel_class():
    """The event timer sees one launch group per kernel class per call, with
    a positive duration, nothing while it is off, and keeps its records
    across a resume.  The q8 update here is two launches (a bf16 and an fp32
    tensor): the class's one record spans both."""
    qs = Q8Set([(4096, 512), (1000,)], [torch.bfloat16, torch.float32], seed=1011)
    plan = q.Plan(qs.triples(), [(0, 0, 4096 * 512, 0), (1, 0, 1000, 1)], 2)
    inv = torch.empty(2, dtype=torch.float32, device=DEV)
    say("launch timing: update+normalize timed, untimed, resumed")
    q.timing_enable(True)
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv)
    q.timing_enable(False)
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv)
    q.timing_enable(True, resume=True)
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv)
    q.timing_enable(False)
    torch.cuda.synchronize()
    # the normalising update: a sums pass, the group reduction, the update
    # writing normalised values (no separate scale pass)
    for k in ("q8_sums", "group_reduce", "q8_update"):
        ms, n = q.timing_read(k)
        assert n == 2 and ms > 0.0, (k, ms, n)
    assert q.timing_read("q8_scale") == (0.0, 0)
    assert q.timing_read("ns_gram") == (0.0, 0)
    say("launch timing: NS of one 512 x 768 matrix, T = 5")
    x = H.grad((512, 768), torch.bfloat16, DEV, 1012, 0)
    q.timing_enable(True)
    q.ns_orthogonalize(x, steps=5)
    q.timing_enable(False)
    torch.cuda.synchronize()
    for k, want in (("ns_norm", 1), ("ns_prologue", 1), ("ns_gram", 5), ("ns_poly", 5), ("ns_xupdate", 5),
                    ("ns_writeback", 1)):
        ms, n = q.timing_read(k)
        assert n == want and ms > 0.0, (k, ms, n)
    assert q.timing_read("q8_update") == (0.0, 0)


def _fused_views(rows, widths, pad, dtype, seed):
    """A fused (rows x sum(widths)+pad) grad buffer and 2-D views of its column
    slices (unit column stride, row pitch the full width); the last `pad`
    columns are canaries no view covers."""
    W = sum(widths) + pad
    buf = H.grad((rows, W), dtype, DEV, seed, 0)
    views, c0 = [], 0
    for w in widths:
        views.append(buf[:, c0:c0 + w])
        c0 += w
    return buf, views


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_strided_grad_views_of_a_fused_buffer(dtype):
    """Grads given as column slices of one fused buffer (row pitch > row length):
    blocks of 256 follow each view's row-major order and cross rows; codes,
    absmax, the views' m and the normalised values match the oracle on the
    contiguous copies bit for bit; the buffer's other columns are untouched."""
    rows, widths, pad = 300, [512, 320, 184], 40
    buf, views = _fused_views(rows, widths, pad, dtype, 1021)
    states = [H.prior_state(v.numel(), DEV, 1021, i + 1) for i, v in enumerate(views)]
    torch.cuda.synchronize()
    h_states = [(host(c), host(a)) for c, a in states]
    h_grads = [host_grad(v).reshape(-1) for v in views]
    h_canary = host_grad(buf[:, sum(widths):]).reshape(-1)
    segs = [(i, 0, v.numel(), i) for i, v in enumerate(views)]
    plan = q.Plan([(c, a, v) for (c, a), v in zip(states, views)], segs, len(views))
    inv = torch.empty(len(views), dtype=torch.float32, device=DEV)
    say("strided views", dtype, widths)
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv)
    torch.cuda.synchronize()
    odt = TORCH_TO_ORACLE[dtype]
    o_states, outs, S, inv_o, _ = oracle.update_normalize_groups(
        h_states, h_grads, [odt] * len(views), segs, len(views), H.BETA, H.NS_EPS, True)
    for i, v in enumerate(views):
        assert_bits_equal(host(states[i][0]), o_states[i][0], f"codes[{i}]")
        assert_bits_equal(host(states[i][1]), o_states[i][1], f"absmax[{i}]")
        assert_bits_equal(host_grad(v).reshape(-1), outs[i], f"grad view[{i}]")
    assert np.array_equal(host(inv), np.asarray(inv_o, dtype=np.float32))
    assert_bits_equal(host_grad(buf[:, sum(widths):]).reshape(-1), h_canary, "canary columns")


def test_uint8_codes_same_bytes_as_int8():
    """uint8 storage of the codes: the kernel reads and writes the same bytes as
    for int8, so codes, absmax and m agree bit for bit with the int8 run."""
    shapes = [(4096, 128), (999,)]
    a = Q8Set(shapes, [torch.bfloat16, torch.float32], seed=1023)
    b = Q8Set(shapes, [torch.bfloat16, torch.float32], seed=1023)
    segs = [(0, 0, 4096 * 128, 0), (1, 0, 999, 1)]
    pa = q.Plan(a.triples(), segs, 2)
    pb = q.Plan([(c.view(torch.uint8), am, g) for c, am, g in b.triples()], segs, 2)
    say("uint8 codes")
    for _ in range(2):
        q.qmuon_update_multi(pa, H.BETA)
        q.qmuon_update_multi(pb, H.BETA)
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(a.codes[i], b.codes[i])
        assert torch.equal(a.absmax[i], b.absmax[i])
        assert torch.equal(a.grads[i].view(torch.int16) if a.grads[i].dtype != torch.float32 else a.grads[i],
                           b.grads[i].view(torch.int16) if b.grads[i].dtype != torch.float32 else b.grads[i])


def test_f16_negative_zero_survives_normalisation():
    """Momentum that rounds to f16 -0 stays -0 through the normalisation pass.
    With absmax 127 * 2^-16 (exact), code 1 and grads 0x8cc0..0x8cc2, the fp32
    EMA gives a value in (-2^-25, 0), stored as 0x8000; float(-0) * inv is -0.
    (A fused mixed-precision multiply-add with a +0 addend would give +0.)"""
    n = 2048
    rng = np.random.default_rng(1031)
    codes = rng.integers(-127, 128, n).astype(np.int8)
    codes[1::2] = 1
    absmax = np.full(n // 256, 127.0 * 2.0 ** -16, dtype=np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
    g[1::2] = np.array([0x8cc0, 0x8cc1, 0x8cc2], dtype=np.uint16)[np.arange(n // 2) % 3]
    c_d = torch.from_numpy(codes.copy()).to(DEV)
    a_d = torch.from_numpy(absmax.copy()).to(DEV)
    g_d = torch.from_numpy(g.view(np.int16).copy()).to(DEV).view(torch.float16)
    plan = q.Plan([(c_d, a_d, g_d)], [(0, 0, n, 0)], 1)
    inv = torch.empty(1, dtype=torch.float32, device=DEV)
    say("f16 negative zero")
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv)
    torch.cuda.synchronize()
    st, outs, _, _, _ = oracle.update_normalize_groups([(codes, absmax)], [g], [oracle.F16], [(0, 0, n, 0)], 1,
                                                        H.BETA, H.NS_EPS, True)
    exp = np.asarray(outs[0])
    assert (exp[1::2] == 0x8000).all()          # the case is exercised
    assert_bits_equal(host(c_d), st[0][0], "codes")
    assert_bits_equal(host(a_d), st[0][1], "absmax")
    assert_bits_equal(host_grad(g_d), exp, "normalised grad")


def test_stochastic_rounding_matches_oracle():
    """Stochastic requantisation: codes, absmax, m and the normalised grads bit
    for bit against the oracle's definition (Philox4x32-10 stream per element,
    tensor index and offset) over mixed dtypes and ragged tails; another offset
    gives other codes; the same offset the same ones."""
    shapes = [(2048, 96), (1000,), (257, 33)]
    dts = [torch.bfloat16, torch.float32, torch.float16]
    segs = [(0, 0, 2048 * 96, 0), (1, 0, 1000, 1), (2, 0, 257 * 33, 2)]
    seed, offset = 0x1234_5678_9abc_def0, 17
    qs = Q8Set(shapes, dts, seed=1041)
    plan = q.Plan(qs.triples(), segs, 3)
    inv = torch.empty(3, dtype=torch.float32, device=DEV)
    say("stochastic rounding: seed", hex(seed), "offset", offset)
    q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv, rounding="stochastic",
                                    seed=seed, offset=offset)
    torch.cuda.synchronize()
    idx = [0, 1, 2]
    st, outs, S, inv_o, _ = oracle.update_normalize_groups(
        qs.host_states(idx), [qs.h_grads[i] for i in idx], [qs.odt(i) for i in idx], segs, 3, H.BETA, H.NS_EPS,
        True, oracle.ROUND_STOCHASTIC, seed, offset)
    for i in idx:
        assert_bits_equal(host(qs.codes[i]), st[i][0], f"codes[{i}]")
        assert_bits_equal(host(qs.absmax[i]), st[i][1], f"absmax[{i}]")
        assert_bits_equal(host_grad(qs.grads[i]), outs[i], f"grad[{i}]")
    near = oracle.update_normalize_groups(qs.host_states(idx), [qs.h_grads[i] for i in idx],
                                          [qs.odt(i) for i in idx], segs, 3, H.BETA, H.NS_EPS, True)[0]
    assert not np.array_equal(st[0][0], near[0][0])           # the stochastic path is exercised
    # same stream twice, another offset
    runs = []
    for off in (5, 5, 6):
        q2 = Q8Set(shapes, dts, seed=1041)
        p2 = q.Plan(q2.triples(), segs, 3)
        q.qmuon_update_multi(p2, H.BETA, rounding="stochastic", seed=seed, offset=off)
        torch.cuda.synchronize()
        runs.append(host(q2.codes[0]))
    assert np.array_equal(runs[0], runs[1]) and not np.array_equal(runs[0], runs[2])


def test_nonfinite_grad_stays_in_its_block():
    """Non-finite momentum is outside the method's contract, but it must
    neither fault nor spread: with a NaN in block 3 and an Inf in block 5 of
    one tensor, its other blocks (codes, absmax) and the other tensors and
    their groups stay bit-exact with the oracle; the two blocks keep codes
    inside [-127, 127]."""
    qs = Q8Set([(4096,), (2048,), (777,)], [torch.bfloat16, torch.bfloat16, torch.float32], seed=1011)
    qs.grads[0][3 * 256 + 17] = float("nan")
    qs.grads[0][5 * 256 + 200] = float("inf")
    torch.cuda.synchronize()
    qs.snapshot()
    run_and_compare(qs, [(0, 0, 4096, 0), (1, 0, 2048, 1), (2, 0, 777, 2)], 3, 0.95, 1e-7, check_idx=[1, 2])
    c_ref, a_ref, _, _ = oracle.q8_update(qs.h_codes[0], qs.h_absmax[0], qs.h_grads[0].copy(), 0.95,
                                          dtype=qs.odt(0))
    codes, absmax = host(qs.codes[0]), host(qs.absmax[0])
    keep = np.ones(16, bool)
    keep[[3, 5]] = False
    assert_bits_equal(codes.reshape(16, 256)[keep].ravel(), c_ref.reshape(16, 256)[keep].ravel(), "codes, finite blocks")
    assert_bits_equal(absmax[keep], a_ref[keep], "absmax, finite blocks")
    assert codes.min() >= -127 and codes.max() <= 127
    # the oracle's reading for non-finite m (NaN codes -127, an infinite
    # block maximum makes 127 / amax zero) holds on the GPU as well
    assert_bits_equal(codes, c_ref, "codes, all blocks")
    assert_bits_equal(absmax, a_ref, "absmax, all blocks")


def _absmax_giving(target_bits, qv):
    """A block absmax a with fl(qv * fl(a / 127)) equal to the fp32 value of
    target_bits (searched among a's neighbours in fp32), or None."""
    t = np.array([target_bits], dtype=np.uint32).view(np.float32)[0]
    g64 = np.float64(t) * 127.0 / qv
    if not (0 < g64 < np.finfo(np.float32).max):
        return None
    guess = np.float32(g64)
    gi = np.array([guess], dtype=np.float32).view(np.int32)[0]
    for d in sorted(range(-400, 401), key=abs):
        a = np.array([gi + d], dtype=np.int32).view(np.float32)[0]
        if not np.isfinite(a) or a <= 0:
            continue
        step = np.float32(a) / np.float32(127.0)
        with np.errstate(over="ignore"):
            m = np.float32(qv) * step
        if m.view(np.uint32) == np.uint32(target_bits):
            return a
    return None


def _edge_state():
    """Codes and block maxima whose dequantised values (beta = 1) are the
    narrowing's edge cases: bf16 and f16 rounding ties with an even and an
    odd kept bit, one ulp either side of a tie, fp32 subnormals (ties among
    them), values that round to the largest finite value or to infinity, the
    smallest normals; block maxima from 1e38 down to 1e-43, so 127 / amax
    overflows binary32 in the smallest blocks."""
    targets = [0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x40C38000, 0x41818000,
               0x00808000, 0x00818000, 0x00008000, 0x00018000, 0x00000001, 0x007FFFFF, 0x00400000,
               0x7F7F8000, 0x7F7F7FFF, 0x7F7FFFFF, 0x7E808000, 0x00800000,
               # f16: ties at 13 dropped bits, the f16 subnormal range, the largest finite f16
               0x3F801000, 0x3F803000, 0x3F800FFF, 0x33801000, 0x33803000, 0x477FE000, 0x477FF000, 0x38801000]
    absmax, codes = [], []
    rng = np.random.default_rng(2025)
    for tb in targets:
        for qv in (1, 127, 3):
            a = _absmax_giving(tb, qv)
            if a is None:
                continue
            c = rng.integers(-127, 128, size=256).astype(np.int8)
            c[:64] = qv
            c[64:128] = -qv
            c[200:208] = 0
            absmax.append(a)
            codes.append(c)
    return np.concatenate(codes), np.array(absmax, dtype=np.float32)


@pytest.mark.parametrize("dtype,mode", [(torch.bfloat16, "nearest"), (torch.float16, "nearest"),
                                        (torch.bfloat16, "stochastic"), (torch.bfloat16, "carrier")])
def test_grad_rounding_edge_values_match_oracle(dtype, mode):
    """With beta = 1, m is the dequantised state q * (absmax / 127) exactly,
    so the edge state above puts m on the narrowing's edge cases and the
    requantisation on the smallest block scales.  The grad's bits (or the
    carrier's bytes and scales), codes and absmax must match the oracle,
    whose rounding is integer arithmetic on the bit patterns."""
    h_codes, h_absmax = _edge_state()
    n = h_codes.size
    say("edge values:", n // 256, "blocks", dtype, mode)
    assert n // 256 >= 40
    g = torch.zeros(n, dtype=dtype, device=DEV)             # (1 - beta) g = 0
    codes_d = torch.from_numpy(h_codes.copy()).to(DEV)
    absmax_d = torch.from_numpy(h_absmax.copy()).to(DEV)
    plan = q.Plan([(codes_d, absmax_d, g)], [(0, 0, n, 0)], 1)
    odt = TORCH_TO_ORACLE[dtype]
    zeros = np.zeros(n, dtype=np.uint16)
    if mode == "carrier":
        car = q.qmuon_update_mxfp8_carrier(plan, 1.0, 1e-7)
        torch.cuda.synchronize()
        c2, a2, pay, sc, _ = oracle.q8_update_carrier(h_codes, h_absmax, zeros, 1.0, odt)
        assert_bits_equal(host(car.data(0)), pay, "carrier bytes")
        assert_bits_equal(host(car.scale_inv(0)), sc, "carrier scales")
    else:
        sr = mode == "stochastic"
        q.qmuon_update_multi(plan, 1.0, rounding=mode, seed=99, offset=5)
        torch.cuda.synchronize()
        c2, a2, m2, _ = oracle.q8_update(h_codes, h_absmax, zeros, 1.0, odt,
                                         oracle.ROUND_STOCHASTIC if sr else oracle.ROUND_NEAREST, 99, 5)
        assert_bits_equal(host_grad(g), m2, "stored m")
    assert_bits_equal(host(codes_d), c2, "codes")
    assert_bits_equal(host(absmax_d), a2, "absmax")
