"""The measurement kernels behind bench.py's measured peaks (include/moe_probe.h).

The read stream must read every 16-byte vector of the buffer exactly once:
the XOR of the per-workgroup folds equals the XOR of all 32-bit words of the
buffer.  The MFMA loop must run and give the same sums on every call.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
from gpu_cases import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 64 << 20])
def test_read_stream_reads_every_word_once(nbytes):
    say(f"probe_read {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(moe.lib.moe_probe_read_blocks(), dtype=torch.int32, device="cuda")
    moe.probe_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_mfma_loop_runs_and_repeats(dtype):
    say(f"probe_mfma {dtype}")
    sink = torch.empty(moe.lib.moe_probe_mfma_blocks() * 256, dtype=torch.float32, device="cuda")
    f = moe.probe_mfma(dtype, 10, sink)
    torch.cuda.synchronize()
    a = sink.clone()
    moe.probe_mfma(dtype, 10, sink)
    torch.cuda.synchronize()
    assert f > 0 and torch.isfinite(a).all() and torch.equal(a, sink)
