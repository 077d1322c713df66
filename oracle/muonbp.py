"""Block-periodic Muon step oracle (TEST INFRASTRUCTURE ONLY).

Source: "MuonBP: Faster Muon via Block-Periodic Orthogonalization"
(papernotes summary), section "方法详解" (method): the flowchart and key
designs 1-3.
  * On P-1 of every P steps each block (a shard in the model-parallel layout)
    is orthogonalised on its own and the weights move by eta_block; on the
    P-th step the full momentum is orthogonalised and the weights move by
    eta_full.  P = 1 is plain Muon, P -> infinity is BlockMuon.
  * Block steps and full steps use different step sizes (Theorem 2).
  * Updates are RMS-matched: block steps scale by the block's dimensions,
    full steps by the full matrix's.
Readings (the page gives no formula for these):
  * steps count from t = 1 and step t is full iff t mod P == 0;
  * the RMS factor is rms_scale * sqrt(max(p, q)) for the p x q matrix that
    was orthogonalised (an orthogonal p x q matrix has RMS 1/sqrt(max(p, q)));
  * W <- W - eta (s O + lambda W), decoupled weight decay as on the GRASP page;
  * the momentum is the q8 update of "Quantized Muon Momentum" (the (1-beta)
    form); its Frobenius normalisation uses one group per block on block
    steps and one group for the whole matrix on full steps.
"""
import math

import numpy as np

import oracle
from . import ns


def is_full_step(t, period):
    return period <= 1 or t % period == 0


def rms_factor(p, q, rms_scale):
    return rms_scale * math.sqrt(max(p, q))


def block_group_ids(rows, cols, block_rows, block_cols):
    """Group id of every 256-element quantisation block when each
    (block_rows x block_cols) block of a row-major matrix is its own group
    (row-major block order).  Requires block_cols % 256 == 0 or a single
    column block with cols % 256 == 0, so no quantisation block straddles two
    groups."""
    nbc = cols // block_cols
    numel = rows * cols
    starts = np.arange(0, numel, oracle.BLOCK)
    r, c = starts // cols, starts % cols
    ids = (r // block_rows) * nbc + c // block_cols
    ends = np.minimum(starts + oracle.BLOCK, numel) - 1
    r2, c2 = ends // cols, ends % cols
    if np.any((r2 // block_rows) * nbc + c2 // block_cols != ids):
        raise ValueError("a quantisation block straddles two norm blocks")
    return ids.astype(np.int32)


def muon_step(W, codes, absmax, grad, dtype, t, rows, cols, block_rows,
              block_cols, period, beta, eps, coeffs, ns_steps, lr_full,
              lr_block, rms_scale, weight_decay=0.0, carrier=False):
    """One step for one matrix.  Returns (W', codes', absmax', O, full).

    carrier: m reaches Newton-Schulz as the MXFP8 carrier ("Quantized Muon
    Momentum", section "Wave18B MXFP8 Carrier Probe"): the NS input is the
    decoded carrier times the group inverse norm, which still comes from the
    fp32 m of the update; otherwise it is m as stored in the grad dtype.  A
    tall matrix orthogonalised whole (rows > cols, rows % 128 == 0,
    cols % 256 == 0) travels as the carrier of m^T, one scale per 32 rows of
    a column (reading R29)."""
    full = is_full_step(t, period)
    br, bc = (rows, cols) if full else (block_rows, block_cols)
    gid = block_group_ids(rows, cols, br, bc)
    ngroups = (rows // br) * (cols // bc)
    if carrier and br == rows and bc == cols and oracle.transposed_carrier_applies(rows, cols):
        # a tall matrix orthogonalised whole: the carrier of m^T (reading R29)
        c2, a2, payload, scales, bsum = oracle.q8_update_carrier_t(codes, absmax, grad, beta, rows, cols, dtype)
        mf = oracle.decode_carrier(payload, scales).reshape(cols, rows).T.ravel()
    elif carrier:
        c2, a2, payload, scales, bsum = oracle.q8_update_carrier(codes, absmax, grad, beta, dtype)
        mf = oracle.decode_carrier(payload, scales)
    else:
        c2, a2, m, bsum = oracle.q8_update(codes, absmax, grad, beta, dtype)
        mf = (m if dtype == oracle.F32 else oracle.widen(m, dtype)).astype(np.float64)
    S = oracle.group_sums([bsum], [gid], ngroups)
    inv = oracle.group_inv_norm(S, eps)
    mf = mf.reshape(rows, cols)
    O = ns.ns_blocked(mf, br, bc, ns_steps, coeffs, eps, inv_norms=inv)
    lr = lr_full if full else lr_block
    s = rms_factor(br, bc, rms_scale)
    W2 = W.astype(np.float64) - lr * (s * O + weight_decay * W.astype(np.float64))
    return W2, c2, a2, O, full
