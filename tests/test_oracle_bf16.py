"""Pins for the oracle's bf16 codec: a library routine (torch's bfloat16
conversion, round to nearest even) and hand-worked ties."""
import numpy as np
import torch

from oracle.bf16 import narrow, widen


def test_narrow_matches_torch_on_a_million_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 1e-3, 1 << 20), rng.normal(0, 1e3, 1 << 16),
                        rng.uniform(-1, 1, 1 << 16) * 1e-38]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(narrow(x), want)


def test_ties_round_to_even():
    # 1 + 2^-8 sits halfway between bf16 1.0 (0x3F80) and 1 + 2^-7 (0x3F81): even wins.
    # 1 + 3*2^-8 sits halfway between 0x3F81 and 0x3F82: even (0x3F82) wins.
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], dtype=np.float32)
    assert narrow(x).tolist() == [0x3F80, 0x3F82, 0xBF80]
    # just above the tie rounds up
    assert narrow(np.array([np.nextafter(np.float32(1 + 2.0 ** -8), np.float32(2))]))[0] == 0x3F81


def test_specials_and_exact_widening():
    x = np.array([np.inf, -np.inf, 0.0, -0.0, np.nan], dtype=np.float32)
    b = narrow(x)
    assert b[:4].tolist() == [0x7F80, 0xFF80, 0x0000, 0x8000]
    assert np.isnan(widen(b[4:]))[0]
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allbits[(allbits & 0x7F80) != 0x7F80]
    assert np.array_equal(narrow(widen(finite)), finite)
    assert np.array_equal(widen(finite),
                          torch.from_numpy(finite.view(np.int16)).view(torch.bfloat16).float().numpy())
