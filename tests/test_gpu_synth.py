"""The device implementation of the input generator produces the host
implementation's bits (so the oracle and the HIP path see identical inputs),
including past the 32-bit counter word; the copy probe copies."""
import numpy as np
import pytest
import torch

from synth import gen
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,std", [(gen.MODE_F32, 0.02), (gen.MODE_ABS, 1e-6),
                                      (gen.MODE_BF16, 1e-3)])
@pytest.mark.parametrize("start", [0, 123457, (1 << 32) - 1000, 68_000_000_000])
def test_device_generator_matches_host(mode, std, start):
    n = 1 << 18
    dt = torch.uint16 if mode == gen.MODE_BF16 else torch.float32
    d = torch.empty(n, dtype=dt, device="cuda")
    gen.dev_fill(d, 3, 1 + mode, 5, start, std, mode)
    torch.cuda.synchronize()
    assert_bits(host(d), gen.host_fill(3, 1 + mode, 5, start, n, std, mode), f"mode {mode}")


def test_copy_probe():
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    gen.dev_copy(src, dst, src.numel() * 4)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
