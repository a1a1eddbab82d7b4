"""Pins for the oracle's number formats (CPU only).

Each codec is checked against something other than itself: the OCP E4M3 spec
points stored under tests/golden/, torch's own float8_e4m3fn and bfloat16
casts, and exhaustive round trips.
"""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e4m3_spec_points():
    for code, val in _rows("e4m3_spec_points.txt"):
        got = codecs.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_vs_torch_in_range():
    rng = np.random.default_rng(7)
    pos = codecs.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)          # exact ties
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rnd = rng.standard_normal(200000).astype(np.float32) * np.float32(40)
    tiny = rng.uniform(0, 2.0 ** -5, 20000).astype(np.float32)
    x = np.concatenate([mids, near, rnd, tiny, pos.astype(np.float32)])
    x = x[np.abs(x) < 464.0]
    x = np.concatenate([x, -x])
    assert np.array_equal(codecs.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_saturates():
    x = np.array([448.0, 463.9, 464.0, 480.0, 1e6, np.float32(3e38), -500.0, -1e9], np.float32)
    got = codecs.e4m3_encode(x)
    assert list(got) == [0x7E] * 6 + [0xFE] * 2
    assert codecs.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_encode_ties_to_even():
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): -> 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even): -> 0x3A
    got = codecs.e4m3_encode(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10], np.float32))
    assert list(got) == [0x38, 0x3A, 0x00, 0x02]


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        rng.standard_normal(1000).astype(np.float32) * 1e-30,
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.4e38], np.float32)])
    # exact ties: low 16 bits = 0x8000
    u = rng.integers(0, 2 ** 31, 1000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & 0x7F7F0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codecs.bf16_round(x), ref)


def test_bf16_decode():
    x = np.array([1.5, -2.25, 0.0, 3.0e10], np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_decode(bits),
                          torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_int4_nibbles_golden():
    for b, lo, hi in _rows("int4_nibbles.txt"):
        got = codecs.int4_unpack(np.array([int(b, 16)], np.uint8))
        assert list(got) == [int(lo), int(hi)]


def test_int4_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    got = codecs.int4_unpack(b).reshape(256, 2).astype(np.int64)
    # an independent formula: v = nibble - 16 * (nibble >> 3)
    lo, hi = b & 15, b >> 4
    assert np.array_equal(got[:, 0], lo.astype(np.int64) - 16 * (lo >> 3))
    assert np.array_equal(got[:, 1], hi.astype(np.int64) - 16 * (hi >> 3))
    assert got.min() == -8 and got.max() == 7


@pytest.mark.parametrize("shape", [(3, 8), (2, 4, 6)])
def test_int4_shape(shape):
    p = np.zeros(shape, np.uint8)
    assert codecs.int4_unpack(p).shape == shape[:-1] + (shape[-1] * 2,)
