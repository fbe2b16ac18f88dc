"""The device fills of the seeded generator reproduce the host fills bit for bit."""
import numpy as np
import pytest

import qsagen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,e0", [(1, 0), (1000, 7), (65536 + 3, 123456789), (4096, 2**40)])
def test_device_normal_equals_host(n, e0):
    import torch
    tid = qsagen.tensor_id(qsagen.KIND_RAW, layer=3, seq=1)
    h32 = qsagen.host_normal((n,), 11, tid, e0=e0)
    d32 = qsagen.dev_normal_(torch.empty(n, dtype=torch.float32, device="cuda"), 11, tid, e0)
    d16 = qsagen.dev_normal_(torch.empty(n, dtype=torch.float16, device="cuda"), 11, tid, e0)
    torch.cuda.synchronize()
    assert np.array_equal(d32.cpu().numpy().view(np.uint32), h32.view(np.uint32))
    assert np.array_equal(d16.cpu().numpy().view(np.uint16), h32.astype(np.float16).view(np.uint16))


def test_device_unit_equals_host():
    import torch
    tid = qsagen.tensor_id(qsagen.KIND_GAMMA, layer=2)
    for off in (0.0, 0.5):
        h = qsagen.host_unit((5000,), 3, tid, e0=9, offset=off)
        d = qsagen.dev_unit_(torch.empty(5000, dtype=torch.float32, device="cuda"), 3, tid, 9, off)
        assert np.array_equal(d.cpu().numpy().view(np.uint32), h.view(np.uint32))
