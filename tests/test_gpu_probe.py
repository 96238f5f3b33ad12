"""The streaming probe (a measurement helper, not part of the method) moves exactly the bytes its
contract names: unit u's write chunks hold the lane-wise XOR of its read chunks; nothing else is written."""
import numpy as np
import pytest
import torch

import combine_ep_layout_02_amd as ep
from test_gpu_parity import DEV, log, setup_module  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("policy", [0, 1, 2, 3, 4, 7])
@pytest.mark.parametrize("units,r,w", [(1, 1, 1), (5, 4, 3), (37, 16, 2), (9, 2, 8), (3, 8, 64)])
def test_probe_stream_contract(units, r, w, policy):
    log(f"[probe] units={units} r={r} w={w} policy={policy}")
    rng = np.random.default_rng(units * 100 + r * 10 + w)
    src = rng.integers(0, 256, size=units * r * 1024, dtype=np.uint8)
    d_src = torch.from_numpy(src).to(DEV)
    d_dst = torch.full((units * w * 1024 + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    ep.ep_probe_stream(d_src, d_dst, units, r, w, policy)
    torch.cuda.synchronize()
    got = d_dst.cpu().numpy()
    want = np.bitwise_xor.reduce(src.reshape(units, r, 1024), axis=1)          # [units, 1024]
    assert np.array_equal(got[: units * w * 1024].reshape(units, w, 1024), np.repeat(want[:, None], w, axis=1))
    assert (got[units * w * 1024:] == 0xA5).all()
