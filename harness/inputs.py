"""Seeded synthetic inputs for the five workloads.

This module holds no arithmetic of the method: it only draws random numbers
(torch's seeded generators, on the requested device) and lays out shapes.  Both
the oracle side and the HIP side take their inputs from here; tests copy the
generated tensors to the host before any kernel runs, so CPU and GPU draws
never need to agree bit for bit.

Recipes (our readings of the workload definitions):
  * "~N(0, 1e-3)" means standard deviation 1e-3, drawn in fp32, then rounded
    to the grad dtype by torch's cast;
  * prior int8 codes: the 255 integers -127..127 equiprobable; prior absmax per
    256-block: uniform in [1e-4, 1e-2], drawn in fp32;
  * "1% outlier rows x20": ceil(0.01 * rows) distinct rows, chosen by seeded
    permutation, multiplied by 20 before the cast;
  * the GRASP gradient adds a fixed rank-8 spike U diag(s) V^T with
    orthonormal seeded U, V (torch QR of Gaussians) and equal s chosen so that
    ||S||_F = 10 * std * sqrt(rows * cols), the expected noise norm;
  * weights ~ N(0, 0.02^2) in fp32.
"""
import math

import torch

BLOCK = 256


def _seed(*keys):
    """Fold integer keys into one 63-bit seed (a fixed polynomial hash)."""
    h = 1469598103934665603
    for k in keys:
        h = ((h ^ (int(k) & 0xFFFFFFFFFFFF)) * 1099511628211) % (1 << 63)
    return h


def gen(device, *keys):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*keys))
    return g


def nblocks(numel):
    return (numel + BLOCK - 1) // BLOCK


def prior_state(numel, device, *keys):
    """int8 codes U{-127..127} and fp32 absmax U(1e-4, 1e-2) per 256-block."""
    g = gen(device, 1, *keys)
    codes = torch.randint(-127, 128, (numel,), generator=g, device=device,
                          dtype=torch.int16).to(torch.int8)
    absmax = torch.rand(nblocks(numel), generator=g, device=device,
                        dtype=torch.float32) * (1e-2 - 1e-4) + 1e-4
    return codes, absmax


def grad(shape, dtype, device, *keys, std=1e-3, outlier_frac=0.0, outlier_mult=20.0):
    """Gaussian grad of the given shape, optional outlier rows, cast to dtype."""
    g = gen(device, 2, *keys)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    if outlier_frac > 0:
        rows = shape[0]
        k = math.ceil(outlier_frac * rows)
        idx = torch.randperm(rows, generator=g, device=device)[:k]
        x[idx] *= outlier_mult
    return x.to(dtype)


def weights(shape, device, *keys, std=0.02):
    g = gen(device, 3, *keys)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def gaussian(shape, device, *keys, dtype=torch.float32):
    g = gen(device, 4, *keys)
    return torch.randn(shape, generator=g, device=device, dtype=dtype)


def spike(rows, cols, rank, device, *keys, std=1e-3, ratio=10.0):
    """Fixed rank-`rank` matrix with orthonormal factors and equal singular
    values, Frobenius norm ratio * std * sqrt(rows*cols)."""
    g = gen(device, 5, *keys)
    u = torch.randn(rows, rank, generator=g, device=device, dtype=torch.float64)
    v = torch.randn(cols, rank, generator=g, device=device, dtype=torch.float64)
    u, _ = torch.linalg.qr(u)
    v, _ = torch.linalg.qr(v)
    s = ratio * std * math.sqrt(rows * cols) / math.sqrt(rank)
    return ((u * s) @ v.T).to(torch.float32)


# ------------------------------------------------------------ workloads

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7
NS_STEPS = 5
BETA = 0.95


def fp32_256x512_shapes():
    """Single 256x512 fp32 grad."""
    return [("w", 256, 512)]


def layerset28_layout(layers=28, hidden=2048):
    """One 2048-hidden layer set x28: fused QKV 2560x2048 (q 2048 rows, k 256,
    v 256), o 2048x2048, gate/up 6144x2048, down 2048x6144.  Returns
    (tensors, segments, ngroups): tensors = [(name, rows, cols)], segments =
    [(tensor_index, start, length, group_id)] with q/k/v as three groups."""
    ffn = 6144
    tensors, segments = [], []
    gid = 0
    for layer in range(layers):
        base = len(tensors)
        tensors += [(f"l{layer}.qkv", 2560, hidden), (f"l{layer}.o", hidden, hidden),
                    (f"l{layer}.gate", ffn, hidden), (f"l{layer}.up", ffn, hidden),
                    (f"l{layer}.down", hidden, ffn)]
        for r0, r1 in ((0, 2048), (2048, 2304), (2304, 2560)):
            segments.append((base, r0 * hidden, (r1 - r0) * hidden, gid))
            gid += 1
        for t in range(1, 5):
            _, r, c = tensors[base + t]
            segments.append((base + t, 0, r * c, gid))
            gid += 1
    return tensors, segments, gid


def llama8b_layer_layout():
    """Llama-8B-shaped layer: q/o 4096x4096, k/v 1024x4096, gate/up
    14336x4096, down 4096x14336; one norm group per tensor."""
    tensors = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
               ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
               ("down", 4096, 14336)]
    segments = [(i, 0, r * c, i) for i, (_, r, c) in enumerate(tensors)]
    return tensors, segments, len(tensors)


def blocked_segments(rows, cols, block_rows, block_cols, tensor_index=0, group0=0):
    """Norm segments that make every (block_rows x block_cols) block of a
    row-major rows x cols tensor its own group (row-major block order)."""
    if cols % block_cols or rows % block_rows:
        raise ValueError("blocks must tile the matrix")
    nbc = cols // block_cols
    segs = []
    for r in range(rows):
        bi = r // block_rows
        for bj in range(nbc):
            segs.append((tensor_index, r * cols + bj * block_cols, block_cols,
                         group0 + bi * nbc + bj))
    return segs, (rows // block_rows) * nbc


def muonbp_4096x14336_shape():
    """MuonBP-shaped momentum 4096x14336, 8 column blocks of 4096x1792, P=5."""
    return dict(rows=4096, cols=14336, block_rows=4096, block_cols=1792,
                period=5, steps=20, lr_full=0.02, lr_block=0.01,
                rms_scale=0.2, weight_decay=0.0)


def grasp_4096_shape():
    """GRASP-shaped 4096x4096, rank 8, 64x64 grid blocks, mu=0.95, 20 steps."""
    return dict(rows=4096, cols=4096, rank=8, grid=64, mu=0.95, steps=20,
                lr=0.02, weight_decay=0.0)


def carrier_bytes(rows, cols, device, *keys, scale_lo=110, scale_hi=126):
    """Random MXFP8 carrier arrays of a rows x cols matrix: payload bytes
    uniform over every code except the two NaN patterns (0x7F, 0xFF, which
    become 0x7E, 0xFE), one scale byte per 32 elements of a row, uniform in
    [scale_lo, scale_hi]."""
    g = gen(device, 5, *keys)
    data = torch.randint(0, 256, (rows, cols), generator=g, device=device, dtype=torch.int32)
    data = torch.where((data & 0x7F) == 0x7F, data - 1, data).to(torch.uint8)
    scale = torch.randint(scale_lo, scale_hi + 1, (rows, cols // 32), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    return data, scale
