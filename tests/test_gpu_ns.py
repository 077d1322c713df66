"""GPU parity of Newton-Schulz orthogonalisation against the fp64 oracle.

bf16 mode: relative Frobenius error <= 2e-2 and every row's cosine >= 0.999
(the workload's stated bound); f32 and bf16x3 modes (fp32 operands; fp32
MFMAs, or bf16 MFMAs on a hi + lo split): <= 1e-4 and >= 0.99999.  At full
size the oracle runs through its spectral route, over every row.
"""
import numpy as np
import pytest
import torch

import quantized_momentum_newton_amd as q
from gpu_util import (NS_BF16_COS, NS_BF16_REL, NS_F32_COS, NS_F32_REL, as_f64, ns_parity, ns_whole, say)
from harness import inputs as H
from oracle import ns

pytestmark = pytest.mark.gpu
DEV = "cuda"
COEF = tuple(float(np.float32(c)) for c in H.NS_COEFFS)


def _check(got, ref, precision):
    rel, cos = ns_parity(got, ref)
    lim_rel, lim_cos = (NS_BF16_REL, NS_BF16_COS) if precision == "bf16" else (NS_F32_REL, NS_F32_COS)
    say(f"   relF {rel:.3e}  min row cos {cos:.7f}")
    assert rel <= lim_rel and cos >= lim_cos, (rel, cos)


@pytest.mark.parametrize("shape", [(256, 512), (512, 256), (100, 300), (300, 100), (128, 128),
                                   (1, 7), (7, 1), (257, 513)])
@pytest.mark.parametrize("precision,dtype", [("bf16", torch.bfloat16), ("f32", torch.float32),
                                             ("bf16", torch.float16), ("bf16x3", torch.float32)])
def test_ns_small_shapes(shape, precision, dtype):
    say("ns", shape, precision, dtype)
    x = H.grad(shape, dtype, DEV, 2001, *shape)
    x0 = as_f64(x)
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS, precision=precision)
    torch.cuda.synchronize()
    ref = ns.ns_orthogonalize(x0, 5, COEF, H.NS_EPS)
    _check(as_f64(x), ref, precision if dtype == torch.float32 else "bf16")


@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
def test_256x512_f32_mode(precision):
    """256x512 fp32, fp32-operand arithmetic, 5 quintic steps."""
    x = H.grad((256, 512), torch.float32, DEV, 1001, 7)
    x0 = as_f64(x)
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS, precision=precision)
    torch.cuda.synchronize()
    _check(as_f64(x), ns.ns_orthogonalize(x0, 5, COEF, H.NS_EPS), precision)


@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
def test_rank8_spike_needs_fp32_operands(precision):
    """The GRASP gradient's shape, a rank-8 spike of 10x the noise norm on
    Gaussian noise: both fp32-operand modes within the f32 bound."""
    rows, cols = 1024, 768
    x = (H.grad((rows, cols), torch.float32, DEV, 2301) + H.spike(rows, cols, 8, DEV, 2301)).contiguous()
    x0 = as_f64(x)
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS, precision=precision)
    torch.cuda.synchronize()
    _check(as_f64(x), ns.ns_orthogonalize(x0, 5, COEF, H.NS_EPS), precision)


def test_given_inverse_norm_and_zero_steps():
    x = H.grad((200, 300), torch.float32, DEV, 2002)
    x0 = as_f64(x)
    inv = torch.tensor([1.0 / (np.linalg.norm(x0) + 1e-7)], dtype=torch.float32, device=DEV)
    y = x.clone()
    q.ns_orthogonalize(y, 5, COEF, 1e-7, inv_norm=inv, precision="f32")
    z = x.clone()
    q.ns_orthogonalize(z, 0, COEF, 1e-7, inv_norm=inv, precision="f32")
    torch.cuda.synchronize()
    invf = float(inv.item())
    _check(as_f64(y), ns.ns_orthogonalize(x0, 5, COEF, 1e-7, inv_norm=invf), "f32")
    assert np.allclose(as_f64(z), x0 * invf, rtol=1e-6, atol=0)


def test_batched_strided_with_canaries():
    """Three 96x200 matrices inside a padded buffer (ld 256, gap rows):
    each gets its own NS, the padding is untouched."""
    b, rows, cols, ld, gap = 3, 96, 200, 256, 5
    buf = torch.full((b * (rows + gap), ld), 7.0, dtype=torch.bfloat16, device=DEV)
    view = torch.as_strided(buf, (b, rows, cols), ((rows + gap) * ld, ld, 1))
    for i in range(b):
        view[i].copy_(H.grad((rows, cols), torch.bfloat16, DEV, 2003, i))
    ins = [as_f64(view[i]) for i in range(b)]
    q.ns_orthogonalize(view, 5, COEF, H.NS_EPS)
    torch.cuda.synchronize()
    for i in range(b):
        _check(as_f64(view[i]), ns.ns_orthogonalize(ins[i], 5, COEF, H.NS_EPS), "bf16")
    mask = torch.ones_like(buf, dtype=torch.bool)
    for i in range(b):
        mask[i * (rows + gap):i * (rows + gap) + rows, :cols] = False
    assert torch.all(buf[mask] == 7.0)


def test_blocked_small():
    x = H.grad((256, 1024), torch.bfloat16, DEV, 2004)
    x0 = as_f64(x)
    q.ns_orthogonalize_blocked(x, 256, 128, 5, COEF, H.NS_EPS)
    torch.cuda.synchronize()
    _check(as_f64(x), ns.ns_blocked(x0, 256, 128, 5, COEF, H.NS_EPS), "bf16")


@pytest.mark.parametrize("name,shape", [("q", (4096, 4096)), ("k", (1024, 4096)),
                                        ("gate", (14336, 4096)), ("down", (4096, 14336))])
def test_llama8b_shapes_full_size(name, shape):
    """The Llama-8B layer's shapes, whole output against the fp64 oracle."""
    say("full-size NS", name, shape)
    x = H.grad(shape, torch.bfloat16, DEV, 1003, name == "gate", shape[0])
    x0 = as_f64(x)
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS)
    torch.cuda.synchronize()
    _check(as_f64(x), ns_whole(x0, 5, COEF, H.NS_EPS), "bf16")


@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
@pytest.mark.parametrize("shape", [(3000, 3300), (3300, 3000), (2048, 2048), (4096, 4096)])
def test_f32_mid_and_small_tile_runs(shape, precision):
    """fp32-operand runs on the sizes whose products take 128 x 128 or 64 x 64
    tiles (3000 x 3300 is padded to 3072 x 3328; the 4096-square Gram and A^2
    take 128 x 128 by stream-K, 528 tiles over 512 workgroup slots, its
    X = aX + BX 128 x 128 tiles whole); whole output against the exact
    iterate."""
    say("fp32-operand NS", shape, precision)
    x = H.grad(shape, torch.float32, DEV, 2101, *shape)
    x0 = as_f64(x)
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS, precision=precision)
    torch.cuda.synchronize()
    _check(as_f64(x), ns_whole(x0, 5, COEF, H.NS_EPS), precision)


def test_stream_k_batch_whole_and_repeatable():
    """Three 2048-square fp32 matrices in one grouped launch: the symmetric
    products run stream-K on 64 x 64 tiles (1584 tiles over 1024 workgroup
    slots, items at different unit offsets, tiles cut between workgroups).
    Every matrix whole within the f32 bound; a second run gives the same
    bits (the pieces of a cut tile are added in a fixed order)."""
    x = H.grad((3, 2048, 2048), torch.float32, DEV, 2103, 2048, 2048)
    x0 = as_f64(x)
    y = x.clone()
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS, precision="f32")
    q.ns_orthogonalize(y, 5, COEF, H.NS_EPS, precision="f32")
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    for b in range(3):
        say("  stream-K batch item", b)
        _check(as_f64(x[b]), ns_whole(x0[b], 5, COEF, H.NS_EPS), "f32")


def test_blocked_muonbp_shape():
    """4096x14336 cut into 8 column blocks of 4096x1792, one batched NS; every
    block whole against its own fp64 NS."""
    x = H.grad((4096, 14336), torch.bfloat16, DEV, 1004)
    x0 = as_f64(x)
    q.ns_orthogonalize_blocked(x, 4096, 1792, 5, COEF, H.NS_EPS)
    torch.cuda.synchronize()
    out = as_f64(x)
    for j in range(8):
        say("  block", j)
        ref = ns_whole(x0[:, 1792 * j:1792 * (j + 1)], 5, COEF, H.NS_EPS)
        _check(out[:, 1792 * j:1792 * (j + 1)], ref, "bf16")


@pytest.mark.parametrize("precision,dtype", [("bf16", torch.bfloat16), ("f32", torch.float32),
                                             ("bf16x3", torch.float32)])
def test_degenerate_inputs(precision, dtype):
    """Degenerate inputs the iteration keeps exact in any arithmetic:
      * a zero matrix stays exactly zero (eps keeps the inverse norm finite,
        0 * 1/eps = 0, and every product of zeros is zero);
      * zero rows of the input are exactly zero rows of every iterate, and
        the other rows match the oracle.
    Other rank-deficient inputs (duplicate rows, low rank) are not parity
    cases: rounding gives their zero singular values tiny nonzero parts,
    which the iteration multiplies by about a = 3.44 per step towards one,
    as it does any small singular value."""
    say("ns degenerate", precision)
    z = torch.zeros((300, 200), dtype=dtype, device=DEV)
    q.ns_orthogonalize(z, 5, COEF, H.NS_EPS, precision=precision)
    torch.cuda.synchronize()
    assert torch.all(z == 0) and not torch.any(torch.isnan(z))

    x = H.grad((256, 384), dtype, DEV, 2203)
    x[::3] = 0
    x0 = as_f64(x)
    q.ns_orthogonalize(x, 5, COEF, H.NS_EPS, precision=precision)
    torch.cuda.synchronize()
    out = as_f64(x)
    assert np.all(out[::3] == 0)
    _check(out, ns.ns_orthogonalize(x0, 5, COEF, H.NS_EPS), precision)


def test_validation_errors():
    x = torch.zeros((16, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QmuonError):
        q.ns_orthogonalize(x, -1)
    with pytest.raises(q.QmuonError):
        q.ns_orthogonalize_blocked(x, 16, 5)
    with pytest.raises(q.QmuonError):
        q.ns_orthogonalize(x, 5, ws=torch.empty(16, dtype=torch.uint8, device=DEV))
