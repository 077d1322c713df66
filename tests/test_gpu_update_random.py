"""GPU parity of the grouped update on seeded random plans.

Each case draws 1-6 tensors of random length (block-aligned or ragged),
random grad dtypes, norm segments cut at random 256-element boundaries and
assigned to random groups (a group may span tensors, a tensor may hold
several groups), beta, write_normalized and the rounding mode.  Codes,
absmax, the grads (m or the normalised m) and the group inverse norms are
compared with the oracle bit for bit, the group sums to rtol 1e-12.  This
drives the sums pass and the normalising update over group layouts the
workload tests do not have (groups crossing tensors, single-block groups,
tails inside a multi-group tensor).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_momentum_newton_amd as q
from gpu_util import TORCH_TO_ORACLE, Q8Set, assert_bits_equal, host, host_grad, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTYPES = [torch.float32, torch.bfloat16, torch.float16]


def random_case(rng):
    n_t = int(rng.integers(1, 7))
    numels, dts = [], []
    for _ in range(n_t):
        blocks = int(rng.integers(1, 40))
        ragged = bool(rng.integers(0, 2))
        numels.append(blocks * 256 - (int(rng.integers(1, 256)) if ragged else 0))
        dts.append(DTYPES[int(rng.integers(0, 3))])
    # segments: cut each tensor at random block boundaries
    pieces = []
    for t, n in enumerate(numels):
        nb = (n + 255) // 256
        cuts = sorted(set(int(x) for x in rng.integers(1, nb, size=int(rng.integers(0, 4)))) if nb > 1 else [])
        bounds = [0] + cuts + [nb]
        for b0, b1 in zip(bounds[:-1], bounds[1:]):
            start, end = b0 * 256, min(b1 * 256, n)
            pieces.append((t, start, end - start))
    n_groups = int(rng.integers(1, len(pieces) + 1))
    # every group gets at least one piece
    gid = list(range(n_groups)) + [int(x) for x in rng.integers(0, n_groups, size=len(pieces) - n_groups)]
    rng.shuffle(gid)
    segments = [(t, s, ln, g) for (t, s, ln), g in zip(pieces, gid)]
    beta = float(rng.choice([0.0, 0.5, 0.9, 0.95, 1.0]))
    write_normalized = bool(rng.integers(0, 2))
    stochastic = bool(rng.integers(0, 4) == 0)
    return numels, dts, segments, n_groups, beta, write_normalized, stochastic


@pytest.mark.parametrize("case", range(96))
def test_random_plans_match_oracle(case):
    rng = np.random.default_rng(9000 + case)
    numels, dts, segments, ng, beta, wn, sr = random_case(rng)
    say("random plan", case, "numels", numels, "groups", ng, "beta", beta, "normalized", wn, "stochastic", sr)
    qs = Q8Set([(n,) for n in numels], dts, seed=9100 + case)
    plan = q.Plan(qs.triples(), segments, ng)
    inv = torch.empty(ng, dtype=torch.float32, device=DEV)
    sums = torch.empty(ng, dtype=torch.float64, device=DEV)
    seed, offset = 0x5eed_0000 + case, case
    q.qmuon_update_normalize_groups(plan, beta, 1e-7, wn, group_inv_norm=inv, group_sumsq=sums,
                                    rounding="stochastic" if sr else "nearest", seed=seed, offset=offset)
    torch.cuda.synchronize()
    idx = list(range(len(numels)))
    states, outs, S, inv_o, _ = oracle.update_normalize_groups(
        qs.host_states(idx), [qs.h_grads[i] for i in idx], [TORCH_TO_ORACLE[d] for d in dts], segments, ng,
        beta, 1e-7, wn, oracle.ROUND_STOCHASTIC if sr else oracle.ROUND_NEAREST, seed, offset)
    for i in idx:
        assert_bits_equal(host(qs.codes[i]), states[i][0], f"codes[{i}]")
        assert_bits_equal(host(qs.absmax[i]), states[i][1], f"absmax[{i}]")
        assert_bits_equal(host_grad(qs.grads[i]), outs[i], f"grad[{i}]")
    assert np.allclose(host(sums), S, rtol=1e-12, atol=0)
    assert_bits_equal(host(inv), inv_o, "inv_norm")
