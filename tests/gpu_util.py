"""Helpers for the GPU parity tests: host copies and q8 input sets."""
import sys

import numpy as np
import torch

import oracle
from harness import inputs as H
from oracle import ns

TORCH_TO_ORACLE = {torch.float32: oracle.F32, torch.bfloat16: oracle.BF16, torch.float16: oracle.F16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_grad(t):
    """Device grad -> numpy (fp32 array, or uint16 bit patterns for 16-bit)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host(t):
    return t.detach().contiguous().cpu().numpy().copy()


class Q8Set:
    """Device q8 tensors plus host copies of their inputs taken before any kernel."""

    def __init__(self, shapes, dtypes, seed, device="cuda", outlier_frac=0.0, std=1e-3):
        self.shapes = shapes
        self.dtypes = dtypes
        self.codes, self.absmax, self.grads = [], [], []
        for i, (shape, dt) in enumerate(zip(shapes, dtypes)):
            numel = int(np.prod(shape))
            c, a = H.prior_state(numel, device, seed, i)
            g = H.grad(shape, dt, device, seed, i, std=std, outlier_frac=outlier_frac).reshape(-1)
            self.codes.append(c)
            self.absmax.append(a)
            self.grads.append(g)
        torch.cuda.synchronize()
        self.snapshot()

    def snapshot(self, which=None):
        idx = range(len(self.shapes)) if which is None else which
        self.h_codes = {i: host(self.codes[i]) for i in idx}
        self.h_absmax = {i: host(self.absmax[i]) for i in idx}
        self.h_grads = {i: host_grad(self.grads[i]) for i in idx}

    def triples(self):
        return list(zip(self.codes, self.absmax, self.grads))

    def odt(self, i):
        return TORCH_TO_ORACLE[self.dtypes[i]]

    def host_states(self, idx):
        return [(self.h_codes[i], self.h_absmax[i]) for i in idx]


def assert_bits_equal(got, exp, what):
    got = np.asarray(got)
    exp = np.asarray(exp)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    if got.dtype.kind == "f":
        got = got.view(np.uint32 if got.dtype == np.float32 else np.uint64)
        exp = exp.view(got.dtype)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: {got[bad[:5]]} vs {exp[bad[:5]]}"


def ns_parity(got, ref):
    """(relative Frobenius error, minimum per-row cosine) of got vs ref; rows
    of ref with zero norm are skipped for the cosine."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    num = np.sum(got * ref, axis=1)
    den = np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1)
    ok = np.linalg.norm(ref, axis=1) > 0
    cos = num[ok] / np.maximum(den[ok], 1e-300)
    return rel, (cos.min() if cos.size else 1.0)


def as_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# Tolerances.  bf16 Newton-Schulz: the workload's stated bound.  f32: fp32
# products with fp32 accumulation over at most a few thousand terms, five
# iterations; the quintic amplifies input perturbations by at most
# a^5 ~ 500 for the smallest singular values, so relative errors stay well
# below 1e-4 on these inputs.
NS_BF16_REL, NS_BF16_COS = 2e-2, 0.999
NS_F32_REL, NS_F32_COS = 1e-4, 0.99999
# fp32-operand NS whose output is stored in bf16 (the GRASP grads): rounding to
# nearest bf16 moves every element by at most 2^-9 of its magnitude, so
# ||bf16(O) - O||_F <= 2^-9 ||O||_F on top of the fp32 arithmetic's bound.
NS_F32_BF16OUT_REL = NS_F32_REL + 2.0 ** -9


def ns_whole(M, steps, coeffs, eps, inv_norm=None):
    """fp64 NS_T(M) for every row: the oracle's spectral route (one Gram
    product and one symmetric eigensolve; in exact arithmetic the same matrix
    as the iteration, and pinned to it on the CPU).  Affordable at the full
    sizes where running the iteration itself on the host would take minutes."""
    M = np.asarray(M, dtype=np.float64)
    return ns.spectral_rows(M, np.arange(M.shape[0]), steps, coeffs, eps, inv_norm)
