"""The no-allocation update entry point (fixed per-GPU scratch instead of a
workspace argument) against qmuon_update_normalize_groups on the same
inputs: codes, absmax, grads, group sums and inverse norms bit for bit, on
two calls in a row, the second with a smaller plan (the scratch then holds
the first call's bytes)."""
import pytest
import torch

import quantized_momentum_newton_amd as q
from gpu_util import Q8Set, say
from harness import inputs as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32) if t.element_size() == 4 else t


def _compare(shapes, dtypes, segments, ngroups, seed, write_normalized):
    ref = Q8Set(shapes, dtypes, seed, outlier_frac=0.01)
    got = [(c.clone(), a.clone(), g.clone()) for c, a, g in ref.triples()]
    p_ref = q.Plan(ref.triples(), segments, ngroups)
    p_got = q.Plan(got, segments, ngroups)
    inv_r = torch.empty(ngroups, dtype=torch.float32, device=DEV)
    inv_g = torch.empty(ngroups, dtype=torch.float32, device=DEV)
    sum_r = torch.empty(ngroups, dtype=torch.float64, device=DEV)
    sum_g = torch.empty(ngroups, dtype=torch.float64, device=DEV)
    q.qmuon_update_normalize_groups(p_ref, H.BETA, H.NS_EPS, write_normalized, group_inv_norm=inv_r,
                                    group_sumsq=sum_r)
    q.qmuon_update_normalize_groups_noalloc(p_got, H.BETA, H.NS_EPS, write_normalized, group_inv_norm=inv_g,
                                            group_sumsq=sum_g)
    torch.cuda.synchronize()
    for i, ((c0, a0, g0), (c1, a1, g1)) in enumerate(zip(ref.triples(), got)):
        assert torch.equal(c0, c1), f"codes[{i}]"
        assert torch.equal(_bits(a0), _bits(a1)), f"absmax[{i}]"
        assert torch.equal(_bits(g0), _bits(g1)), f"grad[{i}]"
    assert torch.equal(_bits(inv_r), _bits(inv_g)), "inv_norm"
    assert torch.equal(sum_r.view(torch.int64), sum_g.view(torch.int64)), "group sums"


def test_noalloc_matches_workspace_entry_twice():
    tensors, segments, ng = H.llama8b_layer_layout()
    shapes = [(r, c) for (_, r, c) in tensors]
    say("no-alloc update: Llama-8B layer,", len(shapes), "tensors")
    _compare(shapes, [torch.bfloat16] * len(shapes), segments, ng, 7101, False)
    small = [(1000,), (4097,), (256, 384)]
    say("no-alloc update: small ragged plan")
    _compare(small, [torch.float32, torch.bfloat16, torch.float16],
             [(0, 0, 1000, 0), (1, 0, 4097, 1), (2, 0, 256 * 256, 2), (2, 256 * 256, 256 * 128, 1)], 3, 7102, True)


def test_noalloc_refuses_plans_beyond_the_scratch():
    """A plan whose workspace exceeds the scratch is refused before launch."""
    n = (q._lib.QM_NOALLOC_SCRATCH_BYTES // 8) * 256 + 256 * 4096
    codes = torch.empty(n, dtype=torch.int8, device=DEV)
    absmax = torch.empty(-(-n // 256), dtype=torch.float32, device=DEV)
    grad = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    plan = q.Plan([(codes, absmax, grad)], [(0, 0, n, 0)], 1)
    assert plan.workspace_bytes() > q._lib.QM_NOALLOC_SCRATCH_BYTES
    with pytest.raises(q.QmuonError) as e:
        q.qmuon_update_normalize_groups_noalloc(plan, 0.9, 1e-7)
    assert e.value.status == 5
