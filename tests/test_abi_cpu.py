"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and its host-side validation rejects bad requests before
anything would be launched (no call here reaches a kernel)."""
import ctypes
import glob
import os
import re

import pytest

import quantized_momentum_newton_amd as q
from quantized_momentum_newton_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = q._LIB

# Fake device addresses: only alignment is ever looked at on the host.
BASE = 0x7f0000000000


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names |= set(re.findall(r"^QM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M))
    return names


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_symbols()
    assert len(names) >= 14
    for n in names:
        assert hasattr(LIB, n), n
    assert names == set(L.SIGNATURES), names ^ set(L.SIGNATURES)
    assert LIB.qm_abi_version() == 4
    assert LIB.qm_status_string(0) == b"ok"


def _tensors(specs):
    """specs: list of (numel, dtype) -> array of Q8Tensor at disjoint fake addresses."""
    arr = (L.Q8Tensor * len(specs))()
    addr = BASE
    for i, (n, dt) in enumerate(specs):
        esz = 4 if dt == L.QM_F32 else 2
        codes = addr
        addr += (n + 4095) // 4096 * 4096
        absmax = addr
        addr += ((n + 255) // 256 * 4 + 4095) // 4096 * 4096
        grad = addr
        addr += (n * esz + 4095) // 4096 * 4096
        arr[i] = L.Q8Tensor(codes, absmax, grad, n, dt, 0)
    return arr


def _segs(lst):
    arr = (L.NormSegment * len(lst))()
    for k, (t, s, ln, g) in enumerate(lst):
        arr[k] = L.NormSegment(t, g, s, ln)
    return arr


def _encode(tens, segs, ngroups):
    size = ctypes.c_size_t(0)
    st = LIB.qm_plan_encode(tens, len(tens), segs, len(segs), ngroups, None, ctypes.byref(size))
    if st != 0:
        return st, None
    buf = (ctypes.c_uint64 * ((size.value + 7) // 8))()
    st = LIB.qm_plan_encode(tens, len(tens), segs, len(segs), ngroups, ctypes.cast(buf, ctypes.c_void_p),
                            ctypes.byref(size))
    return st, buf


def test_plan_encode_and_info():
    tens = _tensors([(2560 * 64, L.QM_BF16), (1000, L.QM_F32)])
    segs = _segs([(0, 0, 2048 * 64, 0), (0, 2048 * 64, 256 * 64, 1), (0, 2304 * 64, 256 * 64, 2),
                  (1, 0, 1000, 3)])
    st, buf = _encode(tens, segs, 4)
    assert st == 0
    nt, ng, nb, numel = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    assert LIB.qm_plan_info(ctypes.cast(buf, ctypes.c_void_p), ctypes.byref(nt), ctypes.byref(ng),
                            ctypes.byref(nb), ctypes.byref(numel)) == 0
    assert (nt.value, ng.value, nb.value, numel.value) == (2, 4, 640 + 4, 2560 * 64 + 1000)
    ws = LIB.qm_update_workspace_bytes(ctypes.cast(buf, ctypes.c_void_p))
    assert ws >= 644 * 8 + 4 * 8 + 4 * 4


@pytest.mark.parametrize("segs,ngroups,status", [
    ([(0, 0, 300, 0), (0, 300, 724, 1)], 2, 2),       # misaligned boundary -> QM_E_ALIGN
    ([(0, 0, 768, 0), (0, 512, 512, 1)], 2, 4),       # overlap -> QM_E_SHAPE
    ([(0, 0, 512, 0)], 1, 4),                         # uncovered block -> QM_E_SHAPE
    ([(0, 0, 1024, 2)], 2, 1),                        # group id out of range -> QM_E_ARG
    ([(1, 0, 1024, 0)], 1, 1),                        # tensor index out of range
    ([(0, 0, 2048, 0)], 1, 1),                        # outside the tensor
    ([(0, 0, 1024, 0)], 2, 4),                        # group 1 empty -> QM_E_SHAPE
])
def test_plan_encode_rejects(segs, ngroups, status):
    st, _ = _encode(_tensors([(1024, L.QM_BF16)]), _segs(segs), ngroups)
    assert st == status, LIB.qm_last_error()
    assert LIB.qm_last_error()


def test_plan_encode_rejects_bad_tensors():
    tens = _tensors([(1024, L.QM_BF16)])
    tens[0].codes += 8                                  # codes not 16-byte aligned
    assert _encode(tens, _segs([(0, 0, 1024, 0)]), 1)[0] == 2
    tens = _tensors([(1024, 7)])
    assert _encode(tens, _segs([(0, 0, 1024, 0)]), 1)[0] == 3
    tens = _tensors([(1024, L.QM_BF16), (1024, L.QM_BF16)])
    tens[1].grad = tens[0].grad + 1024                  # grads overlap
    assert _encode(tens, _segs([(0, 0, 1024, 0), (1, 0, 1024, 0)]), 1)[0] == 1


@pytest.mark.parametrize("cols,ld,status", [
    (64, 64, 0),        # strided view with pitch == row length
    (64, 96, 0),        # rows of 64 at pitch 96
    (48, 48, 4),        # 48 does not divide 1024 -> QM_E_SHAPE
    (64, 32, 4),        # pitch below the row length -> QM_E_SHAPE
    (4, 8, 2),          # row length not a multiple of 8 -> QM_E_ALIGN
    (64, 100, 2),       # pitch not a multiple of 8 -> QM_E_ALIGN
    (-8, 8, 4),         # negative row length
])
def test_plan_strided_grad_rules(cols, ld, status):
    tens = _tensors([(1024, L.QM_BF16)])
    tens[0].grad_cols, tens[0].grad_ld = cols, ld
    st, _ = _encode(tens, _segs([(0, 0, 1024, 0)]), 1)
    assert st == status, LIB.qm_last_error()


def test_plan_strided_grad_span_counts_in_overlap_check():
    # 1024 elements as 16 rows of 64 at pitch 4096 span 61 KiB of bf16: a second
    # tensor's grad placed 32 KiB after the first must be reported as an overlap
    tens = _tensors([(1024, L.QM_BF16), (1024, L.QM_BF16)])
    tens[0].grad_cols, tens[0].grad_ld = 64, 4096
    tens[1].grad = tens[0].grad + 32768
    assert _encode(tens, _segs([(0, 0, 1024, 0), (1, 0, 1024, 0)]), 1)[0] == 1
    tens[1].grad = tens[0].grad + 16 * 4096 * 2
    tens[1].codes = tens[1].codes + 16 * 4096 * 2      # keep codes clear of the moved grad
    tens[1].absmax = tens[1].absmax + 16 * 4096 * 2
    assert _encode(tens, _segs([(0, 0, 1024, 0), (1, 0, 1024, 0)]), 1)[0] == 0, LIB.qm_last_error()


def test_final_partial_block_segment_is_allowed():
    st, _ = _encode(_tensors([(1000, L.QM_F16)]), _segs([(0, 0, 768, 0), (0, 768, 232, 1)]), 2)
    assert st == 0


def test_update_calls_validate_before_launch():
    tens = _tensors([(1024, L.QM_BF16)])
    st, buf = _encode(tens, _segs([(0, 0, 1024, 0)]), 1)
    hp = ctypes.cast(buf, ctypes.c_void_p)
    fake_dev = ctypes.c_void_p(BASE)
    assert LIB.qmuon_update_multi(None, fake_dev, 0.9, None, None) == 1
    assert LIB.qmuon_update_multi(hp, None, 0.9, None, None) == 1
    assert LIB.qmuon_update_multi(hp, fake_dev, 1.5, None, None) == 1
    bad = (ctypes.c_uint64 * 16)()
    assert LIB.qmuon_update_multi(ctypes.cast(bad, ctypes.c_void_p), fake_dev, 0.9, None, None) == 8
    need = LIB.qm_update_workspace_bytes(hp)
    assert LIB.qmuon_update_normalize_groups(hp, fake_dev, 0.9, 1e-7, 1, None, None,
                                             ctypes.c_void_p(BASE), need - 1, None) == 5
    assert LIB.qmuon_update_normalize_groups(hp, fake_dev, 0.9, -1.0, 1, None, None,
                                             ctypes.c_void_p(BASE), need, None) == 1
    assert LIB.qmuon_update_normalize_groups(hp, fake_dev, 0.9, 1e-7, 1, None, None,
                                             ctypes.c_void_p(BASE + 8), need, None) == 2


def test_timing_recorder_host_checks():
    """The launch-timing recorder: bad class or null outputs are rejected;
    with nothing launched every class reads zero launches."""
    ms, n = ctypes.c_double(-1.0), ctypes.c_int64(-1)
    assert LIB.qm_timing_read(99, ctypes.byref(ms), ctypes.byref(n)) == 1  # QM_E_ARG
    assert LIB.qm_timing_read(-1, ctypes.byref(ms), ctypes.byref(n)) == 1  # QM_E_ARG
    assert LIB.qm_timing_read(0, None, ctypes.byref(n)) == 1  # QM_E_ARG
    assert LIB.qm_timing_enable(3) == 1 and LIB.qm_timing_enable(-1) == 1   # QM_E_ARG: modes 0, 1, 2 only
    q.timing_enable(True)
    q.timing_enable(False)
    q.timing_enable(True, resume=True)
    q.timing_enable(False)
    for k in q.KERNEL_CLASSES:
        assert q.timing_read(k) == (0.0, 0)
    assert sorted(q.KERNEL_CLASSES.values()) == list(range(10))


@pytest.mark.parametrize("c1,ld1,off1,c2,ld2,off2,status", [
    (64, 256, 0, 128, 256, 64, 0),      # disjoint column slices of one fused buffer
    (64, 256, 0, 128, 256, 32, 1),      # second slice starts inside the first -> overlap
    (128, 256, 128, 128, 256, 0, 0),    # slices in the other order
    (64, 256, 0, 64, 264, 64, 1),       # different pitches with intersecting spans: reported
    (64, 256, 192, 64, 256, 0, 0),      # first slice ends at the row end, second starts at 0
])
def test_plan_strided_views_of_one_buffer(c1, ld1, off1, c2, ld2, off2, status):
    tens = _tensors([(64 * c1, L.QM_BF16), (64 * c2, L.QM_BF16)])
    base = BASE + (1 << 30)              # fused buffer far from the state arrays
    for t, (c, ld, off) in zip(tens, ((c1, ld1, off1), (c2, ld2, off2))):
        t.grad, t.grad_cols, t.grad_ld = base + off * 2, c, ld
    segs = _segs([(0, 0, 64 * c1, 0), (1, 0, 64 * c2, 1)])
    assert _encode(tens, segs, 2)[0] == status, LIB.qm_last_error()


def test_rounding_options_are_validated():
    tens = _tensors([(1024, L.QM_BF16)])
    st, buf = _encode(tens, _segs([(0, 0, 1024, 0)]), 1)
    hp = ctypes.cast(buf, ctypes.c_void_p)
    fake_dev = ctypes.c_void_p(BASE)
    bad = L.RoundOpts(7, 0, 0)
    assert LIB.qmuon_update_multi_ex(hp, fake_dev, 0.9, ctypes.byref(bad), None, None) == 1
    need = LIB.qm_update_workspace_bytes(hp)
    assert LIB.qmuon_update_normalize_groups_ex(hp, fake_dev, 0.9, 1e-7, 1, ctypes.byref(bad), None, None,
                                                ctypes.c_void_p(BASE), need, None) == 1
    assert "rounding" in LIB.qm_last_error().decode()
    assert ctypes.sizeof(L.MuonHparams) == 64 and ctypes.sizeof(L.RoundOpts) == 16


def _carrier_call(hp, ws_need, data=BASE + (1 << 32), scale=BASE + (1 << 33), inv=BASE + (1 << 34), eps=1e-7,
                  ws=BASE + (1 << 35), ws_bytes=None):
    v = lambda a: ctypes.c_void_p(a) if a is not None else None
    return LIB.qmuon_update_mxfp8_carrier(hp, ctypes.c_void_p(BASE), 0.9, eps, v(data), v(scale), v(inv), None,
                                          v(ws), ws_need if ws_bytes is None else ws_bytes, None)


def test_carrier_update_validates_before_launch():
    tens = _tensors([(1024, L.QM_BF16), (1000, L.QM_F32)])
    st, buf = _encode(tens, _segs([(0, 0, 1024, 0), (1, 0, 1000, 1)]), 2)
    hp = ctypes.cast(buf, ctypes.c_void_p)
    need = LIB.qm_update_workspace_bytes(hp)
    assert _carrier_call(hp, need) == 4                        # 1000 elements: off the 32 grid
    assert "32" in LIB.qm_last_error().decode()
    tens = _tensors([(1024, L.QM_BF16), (992, L.QM_F32)])
    st, buf = _encode(tens, _segs([(0, 0, 1024, 0), (1, 0, 992, 1)]), 2)
    hp = ctypes.cast(buf, ctypes.c_void_p)
    need = LIB.qm_update_workspace_bytes(hp)
    assert _carrier_call(hp, need, data=None) == 1
    assert _carrier_call(hp, need, data=BASE + (1 << 32) + 4) == 2     # data 8-byte alignment
    assert _carrier_call(hp, need, scale=BASE + (1 << 32) + 512) == 1  # scales inside the data array
    assert _carrier_call(hp, need, inv=None) == 1
    assert _carrier_call(hp, need, eps=-1.0) == 1
    assert _carrier_call(hp, need, ws_bytes=need - 1) == 5
    assert _carrier_call(hp, need, data=tens[1].grad) == 1                  # data over a grad
    assert _carrier_call(hp, need, scale=tens[0].codes + 64) == 1           # scales inside codes


def test_ns_mxfp8_validates_before_launch():
    def call(data=BASE, scale=BASE + (1 << 30), inv=BASE + (1 << 31), rows=64, cols=256, out=BASE + (1 << 32),
             ws_bytes=1 << 30):
        v = lambda a: ctypes.c_void_p(a) if a is not None else None
        return LIB.ns_orthogonalize_mxfp8(v(data), v(scale), v(inv), rows, cols, v(out), L.QM_BF16, cols, 5, 3.4445,
                                          -4.775, 2.0315, 0, ctypes.c_void_p(BASE + (1 << 33)), ws_bytes, None)
    assert call(cols=48) == 4                                  # cols off the 32 grid
    assert call(inv=None) == 1
    assert call(data=BASE + 4) == 2
    assert call(data=None) == 1
    assert call(out=None) == 1
    assert call(ws_bytes=16) == 5
    need = LIB.ns_workspace_bytes(64, 256, 1, 0)
    assert call(ws_bytes=need - 1) == 5


def test_carrier_hparams_and_workspace():
    tens = _tensors([(64 * 256, L.QM_BF16)])
    st, buf = _encode(tens, _segs([(0, 0, 64 * 256, 0)]), 1)
    hp = ctypes.cast(buf, ctypes.c_void_p)
    mats = (L.MuonMatrix * 1)()
    mats[0] = L.MuonMatrix(64, 256, 64, 256, None)
    h = q.make_hparams(period=1)
    plain = LIB.muon_step_workspace_bytes(hp, None, mats, 1, 0)
    assert LIB.muon_step_workspace_bytes_ex(hp, None, mats, 1, ctypes.byref(h)) == plain
    h.carrier = 1
    nb = 64
    assert LIB.muon_step_workspace_bytes_ex(hp, None, mats, 1, ctypes.byref(h)) == plain + nb * 256 + 512
    fake = ctypes.c_void_p(BASE)
    ws = ctypes.c_void_p(BASE + (1 << 34))
    h.carrier = 2
    assert LIB.muon_step(hp, fake, None, None, mats, 1, 1, ctypes.byref(h), ws, 1 << 40, None) == 1
    h.carrier, h.rounding = 1, L.QM_ROUND_STOCHASTIC
    assert LIB.muon_step(hp, fake, None, None, mats, 1, 1, ctypes.byref(h), ws, 1 << 40, None) == 7
    h.rounding = L.QM_ROUND_NEAREST
    assert LIB.muon_apply(hp, mats, 1, 1, fake, ctypes.byref(h), ws, 1 << 40, None) == 7
    # cols off the 32 grid: no carrier-mode workspace
    tens = _tensors([(64 * 48, L.QM_BF16)])
    st, buf = _encode(tens, _segs([(0, 0, 64 * 48, 0)]), 1)
    mats[0] = L.MuonMatrix(64, 48, 64, 48, None)
    assert LIB.muon_step_workspace_bytes_ex(ctypes.cast(buf, ctypes.c_void_p), None, mats, 1, ctypes.byref(h)) == 0


def test_ns_precisions_workspace_and_validation():
    """bf16x3 holds X, A, B in fp32 like the f32 mode (same workspace, the
    stream-K part slots included where the symmetric products take that
    path: two 4 x 128 x 128-byte slots per workgroup slot for 4096^2, 256 CUs
    assumed without a GPU); an unknown precision is refused before any
    launch."""
    for rows, cols in ((64, 256), (300, 200), (4096, 14336), (4096, 4096)):
        f32 = LIB.ns_workspace_bytes(rows, cols, 2, L.QM_NS_F32)
        assert LIB.ns_workspace_bytes(rows, cols, 2, L.QM_NS_BF16X3) == f32
        assert f32 > LIB.ns_workspace_bytes(rows, cols, 2, L.QM_NS_BF16)
    # X, two X^T, A, B in fp32 (rows padded), plus the part slots
    assert LIB.ns_workspace_bytes(4096, 4096, 1, L.QM_NS_F32) >= 5 * 4096 * 4096 * 4 + 2 * 256 * 2 * 128 * 128 * 4
    assert LIB.ns_workspace_bytes(256, 512, 1, L.QM_NS_F32) < 2 * 256 * 2 * 128 * 128 * 4
    x = ctypes.c_void_p(BASE)
    ws = ctypes.c_void_p(BASE + (1 << 34))
    for prec in (3, -1):
        assert LIB.ns_orthogonalize(x, L.QM_F32, 64, 256, 256, 1, 0, 5, 3.4445, -4.775, 2.0315, 1e-7, None, prec,
                                    ws, 1 << 40, None) == 1


def _cpu_plan(rows, cols):
    import torch
    codes = torch.zeros(rows * cols, dtype=torch.int8)
    absmax = torch.zeros((rows * cols + 255) // 256, dtype=torch.float32)
    grad = torch.zeros(rows * cols, dtype=torch.bfloat16)
    return q.Plan([(codes, absmax, grad)], [(0, 0, rows * cols, 0)], 1)


@pytest.mark.parametrize("bad,exc", [
    ("bf16", TypeError),          # a bf16 master weight: the C side writes rows x cols fp32
    ("strided", ValueError),      # not contiguous
    ("short", ValueError),        # fewer than rows x cols elements
    ("device", ValueError),       # another device than the plan's
])
def test_muon_wrappers_reject_bad_weights(bad, exc):
    """muon_step / muon_apply / the workspace query check every weight before
    its address reaches the library (no call here gets that far)."""
    import torch
    rows, cols = 64, 256
    plan = _cpu_plan(rows, cols)
    w = {"bf16": torch.zeros((rows, cols), dtype=torch.bfloat16),
         "strided": torch.zeros((rows, 2 * cols), dtype=torch.float32)[:, ::2],
         "short": torch.zeros((rows, cols - 8), dtype=torch.float32),
         "device": torch.zeros((rows, cols), dtype=torch.float32, device="meta")}[bad]
    mats = [(rows, cols, rows, cols, w)]
    hp = q.make_hparams(period=1)
    with pytest.raises(exc):
        q.muon_step(plan, None, mats, 1, hp, ws=torch.empty(256, dtype=torch.uint8))
    with pytest.raises(exc):
        q.muon_step_workspace_bytes(plan, None, mats, hparams=hp)
    with pytest.raises(exc):
        q.muon_apply(plan, mats, True, torch.zeros(1, dtype=torch.float32), hp, torch.empty(256, dtype=torch.uint8))


def test_muon_apply_rejects_bad_inverse_norms():
    import torch
    plan = _cpu_plan(64, 256)
    mats = [(64, 256, 64, 256, None)]
    hp = q.make_hparams(period=1)
    ws = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(ValueError):
        q.muon_apply(plan, mats, True, torch.zeros(2, dtype=torch.float32), hp, ws)
    with pytest.raises(TypeError):
        q.muon_apply(plan, mats, True, torch.zeros(1, dtype=torch.float64), hp, ws)


@pytest.mark.parametrize("bad", ["grad_strided", "grad_shape", "warm_shape", "warm_dtype", "weight_dtype",
                                 "weight_numel"])
def test_grasp_step_rejects_bad_arguments(bad):
    import torch
    rows, cols, rank = 128, 192, 8
    st = q.GraspState(rows, cols, rank, device="cpu")
    grad = torch.zeros((rows, cols), dtype=torch.float32)
    warm = torch.zeros((cols, rank), dtype=torch.float32)
    weight = None
    if bad == "grad_strided":
        grad = torch.zeros((rows, 2 * cols), dtype=torch.float32)[:, :cols]
    elif bad == "grad_shape":
        grad = torch.zeros((rows, cols + 64), dtype=torch.float32)
    elif bad == "warm_shape":
        warm = torch.zeros((rows, rank), dtype=torch.float32)
    elif bad == "warm_dtype":
        warm = torch.zeros((cols, rank), dtype=torch.bfloat16)
    elif bad == "weight_dtype":
        weight = torch.zeros((rows, cols), dtype=torch.bfloat16)
    else:
        weight = torch.zeros((rows, cols // 2), dtype=torch.float32)
    with pytest.raises((TypeError, ValueError)):
        q.grasp_step(st, grad, warm, weight=weight, ws=torch.empty(256, dtype=torch.uint8))


def _step_call(hplan_full, hplan_block, mats_spec, step=1, call=True):
    """(workspace bytes, muon_step status); call=False skips muon_step (a valid
    request would go on to launch kernels)."""
    mats = (L.MuonMatrix * len(mats_spec))()
    for i, (r, c, br, bc) in enumerate(mats_spec):
        mats[i] = L.MuonMatrix(r, c, br, bc, None)
    h = q.make_hparams(period=2)
    fake = ctypes.c_void_p(BASE)
    ws = ctypes.c_void_p(BASE + (1 << 34))
    vp = lambda b: ctypes.cast(b, ctypes.c_void_p) if b is not None else None
    need = LIB.muon_step_workspace_bytes_ex(vp(hplan_full), vp(hplan_block), mats, len(mats_spec), ctypes.byref(h))
    if not call:
        return need, None
    st = LIB.muon_step(vp(hplan_full), fake, vp(hplan_block), fake if hplan_block is not None else None, mats,
                       len(mats_spec), step, ctypes.byref(h), ws, 1 << 40, None)
    return need, st


def test_block_plan_numbering_must_be_row_major():
    """A 64 x 1024 matrix in four 64 x 256 blocks: the block plan must give
    quantisation block k the group of its NS block in row-major block order.
    The same groups numbered right to left are refused (each block would get
    another block's norm)."""
    rows, cols, bc = 64, 1024, 256
    tens = _tensors([(rows * cols, L.QM_BF16)])
    _, full = _encode(tens, _segs([(0, 0, rows * cols, 0)]), 1)
    ok = [(0, r * cols + j * bc, bc, j) for r in range(rows) for j in range(4)]
    rev = [(0, r * cols + j * bc, bc, 3 - j) for r in range(rows) for j in range(4)]
    _, good = _encode(tens, _segs(ok), 4)
    _, bad = _encode(tens, _segs(rev), 4)
    need, _ = _step_call(full, good, [(rows, cols, rows, bc)], call=False)
    assert need > 0, LIB.qm_last_error()
    need, st = _step_call(full, bad, [(rows, cols, rows, bc)])
    assert need == 0 and st == 8, LIB.qm_last_error()
    assert "group" in LIB.qm_last_error().decode()


@pytest.mark.parametrize("rows,cols,br,bc,groups", [
    (4, 384, 4, 128, [0, 1, 2, 0, 1, 2]),     # 128-column blocks: quantisation blocks cross them
    (8, 96, 4, 96, [0, 1, 1]),                # 4 x 96 = 384 elements per block: not whole blocks
])
def test_block_plan_straddling_quantisation_blocks_refused(rows, cols, br, bc, groups):
    tens = _tensors([(rows * cols, L.QM_BF16)])
    _, full = _encode(tens, _segs([(0, 0, rows * cols, 0)]), 1)
    n = rows * cols
    segs = [(0, 256 * k, min(256, n - 256 * k), g) for k, g in enumerate(groups)]
    st0, blk = _encode(tens, _segs(segs), max(groups) + 1)
    assert st0 == 0, LIB.qm_last_error()
    need, st = _step_call(full, blk, [(rows, cols, br, bc)])
    assert need == 0 and st == 4, LIB.qm_last_error()
    assert "straddles" in LIB.qm_last_error().decode()


def test_full_and_block_plans_must_share_tensors():
    rows, cols, bc = 64, 1024, 256
    tens = _tensors([(rows * cols, L.QM_BF16)])
    _, full = _encode(tens, _segs([(0, 0, rows * cols, 0)]), 1)
    other = _tensors([(rows * cols, L.QM_BF16)])
    other[0].grad = other[0].grad + (1 << 28)       # the block plan points at another grad buffer
    segs = [(0, r * cols + j * bc, bc, j) for r in range(rows) for j in range(4)]
    _, blk = _encode(other, _segs(segs), 4)
    for step in (1, 2):                             # a block step and a full step
        need, st = _step_call(full, blk, [(rows, cols, rows, bc)], step)
        assert need == 0 and st == 8, LIB.qm_last_error()


def test_hbm_stream_copy_validates_before_launch():
    v = ctypes.c_void_p
    assert LIB.qm_hbm_stream_copy(None, v(BASE), 1024, None) == 1
    assert LIB.qm_hbm_stream_copy(v(BASE), v(BASE + 4096), 1000, None) == 2       # size not a multiple of 16
    assert LIB.qm_hbm_stream_copy(v(BASE + 8), v(BASE + 8192), 1024, None) == 2   # misaligned source
    assert LIB.qm_hbm_stream_copy(v(BASE), v(BASE + 512), 1024, None) == 1        # overlap
    assert LIB.qm_hbm_stream_copy(v(BASE), v(BASE + 4096), 0, None) == 0          # nothing to copy
