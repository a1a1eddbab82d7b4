"""Pins for the oracle's MX formats (CPU only): E8M0 scales, E2M1 elements,
MXFP8 quantisation of activations and intermediates, MX weight dequantisation,
and a one-expert layer written with torch's fp8 casts.

The quantisation follows the OCP MX specification v1.0 (shared exponent
floor(log2 amax) minus the element type's emax, elements rounded to nearest
even and clamped to the largest normal); the tests recompute it with other
tools: math.frexp per block, torch's float8_e4m3fn and float8_e8m0fnu dtypes.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import codecs
from oracle import moe as om

R = np.random.default_rng
GOLD = os.path.join(os.path.dirname(__file__), "golden", "e2m1_e8m0_spec_points.txt")


def _gold():
    rows = []
    for ln in open(GOLD):
        if ln.startswith("#") or not ln.strip():
            continue
        kind, code, val = ln.split()
        rows.append((kind, int(code), float(val)))
    return rows


def test_spec_points():
    for kind, code, val in _gold():
        if kind == "e2m1":
            got = codecs.e2m1_unpack_decode(np.array([code], np.uint8))[0]  # low nibble
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got)
        else:
            assert codecs.e8m0_decode(np.array([code], np.uint8))[0] == val


def test_e8m0_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e8m0fnu).double().numpy()
    got = codecs.e8m0_decode(c)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_e2m1_nibble_order_and_all_codes():
    # byte b = hi << 4 | lo: the even element is lo, the odd one hi
    b = np.array([[0x21, 0xF7]], np.uint8)
    np.testing.assert_array_equal(codecs.e2m1_unpack_decode(b), [[0.5, 1.0, 6.0, -6.0]])
    vals = codecs.e2m1_unpack_decode(np.arange(16, dtype=np.uint8)[None, :] | 0)[0, 0::2]
    mags = sorted(set(np.abs(vals)))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mx8_by_loops(v):
    """Shared exponent with math.frexp, elements with torch's e4m3 cast."""
    v = np.asarray(v, np.float32)
    R_, C = v.shape
    codes = np.zeros((R_, C), np.uint8)
    sc = np.zeros((R_, C // 32), np.uint8)
    for r in range(R_):
        for b in range(C // 32):
            blk = v[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = float(np.max(np.abs(blk)))
            if amax == 0:
                X = -127
            else:
                m, ex = math.frexp(amax)       # amax = m 2^ex, 0.5 <= m < 1
                X = min(max(ex - 1 - 8, -127), 127)
            sc[r, b] = X + 127
            scaled = np.clip(blk / 2.0 ** X, -448, 448).astype(np.float32)
            codes[r, 32 * b:32 * b + 32] = torch.from_numpy(scaled).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, sc


@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.0, 1e-30])
def test_quant_mx8_matches_loops_and_torch(scale):
    rng = R(3)
    v = (rng.standard_normal((5, 96)) * scale).astype(np.float32)
    v[1, 32:64] = 0.0                         # an all-zero block
    v[2, :32] *= rng.uniform(0, 1e4, 32).astype(np.float32)   # a wide-range block
    q, s = om.quant_mx8(v)
    rq, rs = _mx8_by_loops(v)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)
    assert s[1, 1] == 0 and np.all(q[1, 32:64] & 0x7F == 0)


def test_quant_mx8_worked_values():
    # amax 1.0: X = -8 (scale code 119), 1.0 -> 256 = e4m3 0x78
    v = np.zeros((1, 32), np.float32)
    v[0, 0], v[0, 1], v[0, 2] = 1.0, -0.5, 2.0 ** -17
    q, s = om.quant_mx8(v)
    assert s[0, 0] == 119 and q[0, 0] == 0x78 and q[0, 1] == 0xF0
    assert q[0, 2] == 0x01                    # 2^-17 * 2^8 = 2^-9, the least subnormal
    # amax 1.99: X = -8, 1.99 * 256 = 509.4 is clamped to 448 (0x7E)
    v[0, 0] = 1.99
    q, s = om.quant_mx8(v)
    assert s[0, 0] == 119 and q[0, 0] == 0x7E


def test_mx_weight_dequant_by_loops():
    rng = R(5)
    n, k = 48, 96
    c8 = rng.integers(0, 256, (1, n, k)).astype(np.uint8)
    c8[(c8 & 0x7F) == 0x7F] = 0x30
    c4 = rng.integers(0, 256, (1, n, k // 2)).astype(np.uint8)
    sc = rng.integers(110, 140, (1, n, k // 32)).astype(np.uint8)
    w8 = om.dequant_w2(c8, sc, "mxfp8", 0)
    w4 = om.dequant_w2(c4, sc, "mxfp4", 0)
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(0, n, 7):
        for kk in range(0, k, 5):
            s = 2.0 ** (int(sc[0, r, kk // 32]) - 127)
            ref8 = float(torch.tensor([int(c8[0, r, kk])], dtype=torch.uint8)
                         .view(torch.float8_e4m3fn).double()) * s
            assert w8[r, kk] == ref8
            nib = (int(c4[0, r, kk // 2]) >> (4 * (kk % 2))) & 0xF
            ref4 = (-1 if nib & 8 else 1) * e2m1[nib & 7] * s
            assert w4[r, kk] == ref4


@pytest.mark.parametrize("quant", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("act", ["silu", "relu2"])
def test_mx_single_expert_with_torch(quant, act):
    """E = 1: the layer is the MLP on MXFP8-quantised x with the MXFP8
    intermediate, both quantised here by the loop/torch route."""
    rng = R(21)
    H, I, T = 128, 128, 6
    N1 = 2 * I if act == "silu" else I
    sc13 = rng.integers(118, 124, (1, N1, H // 32)).astype(np.uint8)
    sc2 = rng.integers(118, 124, (1, H, I // 32)).astype(np.uint8)
    if quant == "mxfp8":
        c13 = rng.integers(0, 0x70, (1, N1, H)).astype(np.uint8) | (rng.integers(0, 2, (1, N1, H)) << 7).astype(np.uint8)
        c2 = rng.integers(0, 0x70, (1, H, I)).astype(np.uint8) | (rng.integers(0, 2, (1, H, I)) << 7).astype(np.uint8)
        dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    else:
        c13 = rng.integers(0, 256, (1, N1, H // 2)).astype(np.uint8)
        c2 = rng.integers(0, 256, (1, H, I // 2)).astype(np.uint8)
        tab = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
        dec = lambda c: np.stack([tab[c & 0xF], tab[c >> 4]], axis=-1).reshape(c.shape[0], -1)
    W13 = dec(c13[0]) * np.repeat(2.0 ** (sc13[0].astype(np.float64) - 127), 32, axis=1)
    W2 = dec(c2[0]) * np.repeat(2.0 ** (sc2[0].astype(np.float64) - 127), 32, axis=1)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).bfloat16().double().numpy()

    def mx(a):
        q, s = _mx8_by_loops(np.asarray(a, np.float32))
        return torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * \
            np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)

    xt = torch.from_numpy(mx(x))
    h = xt @ torch.from_numpy(W13).T
    a = F.silu(h[:, :I]) * h[:, I:] if act == "silu" else F.relu(h) ** 2
    ref = torch.from_numpy(mx(a.numpy())) @ torch.from_numpy(W2).T
    got = oracle.moe_forward(x, c13, c2, quant=quant, act=act, E_routed=1, top_k=1,
                             renormalize=True, logits=np.zeros((T, 1), np.float32),
                             w13_scale=sc13, w2_scale=sc2)["out"]
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("quant", ["mxfp8", "mxfp4"])
def test_mx_interleaved_equals_split(quant):
    """Interleaved W13 codes find their per-row E8M0 scales through the row's
    split-layout origin."""
    import dataclasses
    import synth
    cfg = dataclasses.replace(synth.CONFIGS[1], quant=quant, E_routed=3, top_k=2, H=128, I=64)
    W = synth.make_weights(cfg, seed=31)
    T = 7
    x = torch.from_numpy(R(9).standard_normal((T, 128)).astype(np.float32)).bfloat16().double().numpy()
    lg = R(10).standard_normal((T, 3)).astype(np.float32)
    kw = dict(quant=quant, act="silu", E_routed=3, top_k=2, renormalize=True, logits=lg,
              w13_scale=W["w13_scale"], w2_scale=W["w2_scale"])
    a = oracle.moe_forward(x, W["w13"], W["w2"], **kw)["out"]
    b = oracle.moe_forward(x, oracle.interleave_rows(W["w13"], 16), W["w2"], layout_g=16, **kw)["out"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
