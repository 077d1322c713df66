"""The last build's kernels (no GPU): no kernel spills registers to scratch
memory, and the streamed update kernels keep the occupancy their launch
bounds ask for.  The figures are the compiler's resource-usage remarks,
which quantized_momentum_newton_amd/build.py records in
_build/kernel_resources.tsv; the test is skipped when no build left it."""
import os
import re

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
    for k in ("q8_update_kernel", "q8_update_tcar_kernel", "q8_sums_kernel", "chunk_reduce_kernel",
              "gemm_nt_kernel", "gram_mx_kernel", "prologue_kernel", "writeback_kernel", "hbm_stream_kernel"):
        assert k in names, k


def test_no_kernel_spills():
    bad = [(r["kernel"], r["vgpr_spill"], r["sgpr_spill"], r["scratch_per_lane"]) for r in _rows()
           if int(r["vgpr_spill"] or 0) or int(r["sgpr_spill"] or 0) or int(r["scratch_per_lane"] or 0)]
    assert not bad, bad


def test_update_kernels_keep_their_occupancy():
    """The 16-bit-grad update kernels (nearest rounding) stream at 8 waves
    per SIMD in 64 VGPRs; one more register halves the waves in flight."""
    # template <dtype, sums, stochastic rounding, carrier, output mode>: bf16 / f16, nearest
    # and the read-only sums pass of the normalising update, per dtype
    pat = re.compile(r"q8_update_kernelILi[12]ELb[01]ELb0ELb[01]ELi[01]EE|q8_sums_kernelILi[12]EE")
    rows = [r for r in _rows() if pat.search(r["kernel"])]
    assert len(rows) == 2 * (4 + 1 + 1), [r["kernel"] for r in rows]   # per dtype: plain / carrier x sums, normalising, sums pass
    for r in rows:
        assert int(r["vgprs"]) <= 64 and int(r["occupancy"]) >= 8, (r["kernel"], r["vgprs"], r["occupancy"])
