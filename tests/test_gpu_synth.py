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


def test_read_and_write_probes():
    n = 1 << 22
    a = torch.arange(n, dtype=torch.int32, device="cuda")
    sink = torch.zeros(gen.probe_out_words(n * 4), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):                       # a short sink is refused on the host
        gen.dev_read(a, sink[:-1], n * 4)
    gen.dev_read(a, sink, n * 4)
    b = torch.zeros(n, dtype=torch.int32, device="cuda")
    gen.dev_write(b, n * 4)
    torch.cuda.synchronize()
    w = b.view(-1, 4).cpu()
    assert torch.equal(w[:, 0], torch.arange(n // 4, dtype=torch.int32))
    assert (w[:, 1] == 1).all() and (w[:, 3] == 3).all()
    # every loaded word is folded into some lane's xor: the lanes' xor is the xor of all words
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy())) == \
        int(np.bitwise_xor.reduce(np.arange(n, dtype=np.int32)))


def test_read_streams_probe():
    g = torch.Generator().manual_seed(5)
    host_bufs = [torch.randint(-2**31, 2**31 - 1, (1 << 16,), generator=g, dtype=torch.int32)
                 for _ in range(9)]
    bufs = [b.cuda() for b in host_bufs]
    sink = torch.zeros(gen.probe_out_words(4 * (1 << 16)), dtype=torch.int32, device="cuda")
    gen.dev_read_streams(bufs, 4 * (1 << 16), sink)
    torch.cuda.synchronize()
    want = 0
    for b in host_bufs:
        want ^= int(np.bitwise_xor.reduce(b.numpy()))
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy())) == want


@pytest.mark.parametrize("mode,std", [(gen.MODE_F32, 0.02), (gen.MODE_BF16, 1e-3)])
def test_pieces_fill_equals_per_piece_fills(mode, std):
    dt = torch.uint16 if mode == gen.MODE_BF16 else torch.float32
    n = 50000
    pieces = [(0, 1000, 300), (300, 7, 0), (300, 2 ** 32 - 50, 100), (1000, 0, 4096),
              (9000, 123456, 40000), (49990, 5, 10)]
    a = torch.full((n,), 7, dtype=dt, device="cuda")
    gen.dev_fill_pieces(a, pieces, 3, 2, 9, std, mode)
    b = torch.full((n,), 7, dtype=dt, device="cuda")
    for dst, param, k in pieces:
        if k:
            gen.dev_fill(b[dst:dst + k], 3, 2, 9, param, std, mode)
    torch.cuda.synchronize()
    assert_bits(host(a), host(b), "pieces fill")                  # covered and uncovered alike
    with pytest.raises(ValueError):                               # out of range: refused on the host
        gen.dev_fill_pieces(a, [(n - 5, 0, 6)], 3, 2, 9, std, mode)
