"""moe_stream_read (the HBM read-ceiling helper) through the C ABI: every
byte of the buffer is read, checked by the XOR of the per-slice words
against the XOR of the buffer computed on the host, for sizes that split
evenly, unevenly, and into fewer 16-byte words than slices."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from moe_expert_layer_fp32_amd import load_library
    load_library()


@pytest.mark.parametrize("nbytes", [16, 16 * 300, 16 * 512 * 4096, 16 * 1_000_003])
def test_stream_read_reads_every_byte(nbytes):
    import gpu_util as U
    from moe_expert_layer_fp32_amd import lib as L
    U.say(f"[gpu] stream_read bytes={nbytes}")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((L.STREAM_READ_WGS,), -1, dtype=torch.int32, device="cuda")
    L.moe_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
