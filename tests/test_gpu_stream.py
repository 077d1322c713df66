"""The HBM stream-copy measurement aid copies exactly (ragged last workgroup
included) and leaves the bytes around the destination alone."""
import pytest
import torch

import quantized_momentum_newton_amd as q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("units", [1, 255, 1024, 4097, 1 << 20])
def test_stream_copy_exact(units):
    g = torch.Generator(device="cuda")
    g.manual_seed(units)
    src = torch.randint(0, 1 << 30, (units * 4,), generator=g, device="cuda", dtype=torch.int32)
    buf = torch.full((units * 4 + 8,), -1, dtype=torch.int32, device="cuda")
    dst = buf[4:4 + units * 4]
    q.hbm_stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.all(buf[:4] == -1) and torch.all(buf[-4:] == -1)
