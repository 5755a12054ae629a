"""The measurement helpers behind the practical ceilings that bench.py
reports: the streaming read reads every byte once (the XOR of its digest
words is the XOR of the buffer's 32-bit words), and the register-resident
MFMA loop computes what it claims (deterministic, and its accumulator sums
grow linearly with the iteration count)."""
import numpy as np
import pytest
import torch

from block_diffusion_amd import api

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 96 << 20])
def test_stream_read_digest(nbytes):
    g = np.random.default_rng(nbytes % 1000)
    host = g.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    data = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.zeros(api.lib().dbd_stream_read_sink_words(), dtype=torch.int32, device="cuda")
    api.dbd_stream_read(data, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_mfma_peak_consistent():
    L = api.lib()
    g = np.random.default_rng(3)
    nb = L.dbd_mfma_peak_operand_bytes()
    ops = torch.from_numpy(g.standard_normal(nb // 2).astype(np.float32)).to("cuda").to(torch.bfloat16)
    n = L.dbd_mfma_peak_sink_floats()
    s1 = torch.full((n,), float("nan"), device="cuda")
    s1b = torch.full((n,), float("nan"), device="cuda")
    s3 = torch.full((n,), float("nan"), device="cuda")
    f1 = api.dbd_mfma_peak(ops, 1, s1)
    api.dbd_mfma_peak(ops, 1, s1b)
    api.dbd_mfma_peak(ops, 3, s3)
    torch.cuda.synchronize()
    a, b, c = s1.cpu().numpy(), s1b.cpu().numpy(), s3.cpu().numpy()
    assert f1 == L.dbd_mfma_peak_flops(1)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)
    # three iterations accumulate the same products three times
    err = np.abs(c - 3 * a).max()
    assert err <= 1e-3 * max(1.0, np.abs(3 * a).max()), err
