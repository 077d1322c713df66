"""The last build's kernels (no GPU): no kernel spills registers to scratch
memory, and the streamed update kernels keep the occupancy their launch
bounds ask for.  The figures are the compiler's resource-usage remarks,
which quantized_momentum_newton_amd/build.py records in
_build/kernel_resources.tsv; the test is skipped when no build left it."""
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TSV = os.path.join(ROOT, "_build", "kernel_resources.tsv")


def _rows():
    if not os.path.exists(TSV):
        pytest.skip("no build record (run __graft_entry__.build() first)")
    lines = open(TSV).read().splitlines()
    head = lines[0].split("\t")
    return [dict(zip(head, l.split("\t"))) for l in lines[1:] if l.strip()]


def test_every_kernel_was_recorded():
    names = " ".join(r["kernel"] for r in _rows())
    for k in ("q8_update_kernel", "q8_update_tcar_kernel", "q8_scale_kernel", "chunk_reduce_kernel",
              "gemm_nt_kernel", "gram_mx_kernel", "prologue_kernel", "writeback_kernel", "hbm_stream_kernel"):
        assert k in names, k


def test_no_kernel_spills():
    bad = [(r["kernel"], r["vgpr_spill"], r["sgpr_spill"], r["scratch_per_lane"]) for r in _rows()
           if int(r["vgpr_spill"] or 0) or int(r["sgpr_spill"] or 0) or int(r["scratch_per_lane"] or 0)]
    assert not bad, bad


def test_update_kernels_keep_their_occupancy():
    """The 16-bit-grad update kernels (nearest rounding) stream at 8 waves
    per SIMD in 64 VGPRs; one more register halves the waves in flight."""
    rows = [r for r in _rows() if "q8_update_kernelILi1E" in r["kernel"] or "q8_update_kernelILi2E" in r["kernel"]]
    rows = [r for r in rows if "ELb0ELb0EE" in r["kernel"] or "ELb0ELb1EE" in r["kernel"]]   # no stochastic rounding
    assert rows
    for r in rows:
        assert int(r["vgprs"]) <= 64 and int(r["occupancy"]) >= 8, (r["kernel"], r["vgprs"], r["occupancy"])
