"""Seeded generators for weights, hidden states, router logits and static scales.

Recipe (one generator stream per (seed, tensor, expert), numpy PCG64 through
``default_rng([seed, tensor, expert])``, so any single expert can be
regenerated on its own):
 * hidden states x ~ N(0, 1), stored as bf16;
 * router logits ~ N(0, 1), fp32;
 * weights ~ N(0, 1/sqrt(fan_in)) (standard deviation), fan_in = H for the
   up-projection and I for the down-projection, stored as
   - bf16,
   - fp8 e4m3 with one fp32 scale per expert (scale = amax / 448),
   - fp8 e4m3 with one fp32 scale per 128x128 block, scale ~ U(0.5, 2) / 64,
   - signed int4 with one bf16 scale per 128 consecutive K (scale = amax/7),
     packed two per byte, even k in the low nibble,
   - MXFP8: e4m3 codes with one E8M0 scale per row per 32 K, the scale
     2^(floor(log2 amax) - 8) of the 32 values (torch's e4m3 cast, clamped),
   - MXFP4: E2M1 codes (nearest of the 16 values) with one E8M0 scale per
     row per 32 K, 2^(floor(log2 amax) - 2), packed two per byte, even k in
     the low nibble.
 * static activation scales for the per-tensor modes: a1 = amax(x) / 448 and
   a fixed a2 per configuration.

Weights are laid out as the checkpoints on the pages store them: the
up-projection is ``[E, N1, H]`` with the gate rows first and the up rows second
(N1 = 2I) for gated activations, or ``[E, I, H]`` for relu^2; the
down-projection is ``[E, H, I]``.  K (the reduction dim) is contiguous.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

from .configs import MoEConfig

_T_W13, _T_W2, _T_S13, _T_S2, _T_X, _T_LOGITS = 1, 2, 3, 4, 5, 6


def weight_seed(cid: int) -> int:
    return 1000 * cid


def token_seed(cid: int, M: int) -> int:
    return 1000 * cid + M


def _rng(seed: int, tensor: int, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tensor, idx])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even cast), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes with torch's cast, after clamping to +-448."""
    c = np.clip(np.asarray(a, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(c)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _pack_int4(q: np.ndarray) -> np.ndarray:
    """[.., K] int8 in [-8, 7] -> [.., K/2] uint8, even k in the low nibble."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _mx_exponent(w: np.ndarray, emax: int) -> np.ndarray:
    """Per row and 32 K: floor(log2 amax) - emax (-127 for an all-zero block)."""
    n, k = w.shape
    amax = np.abs(w.reshape(n, k // 32, 32)).max(axis=-1).astype(np.float64)
    _, ex = np.frexp(amax)
    return np.clip(np.where(amax > 0, ex - 1 - emax, -127), -127, 127).astype(np.int64)


def _to_e2m1_codes(v: np.ndarray) -> np.ndarray:
    """float -> 4-bit E2M1 codes: the nearest magnitude of the table, sign bit 3."""
    mag = np.abs(v)[..., None]
    idx = np.argmin(np.abs(mag - _E2M1_MAG), axis=-1).astype(np.uint8)
    return idx | ((np.signbit(v) & (idx > 0)).astype(np.uint8) << 3)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gen_expert(cfg: MoEConfig, seed: int, which: int, e: int):
    """One expert's matrix in the configuration's storage format."""
    if which == _T_W13:
        n, k = cfg.N1, cfg.H
    else:
        n, k = cfg.H, cfg.I
    std = 1.0 / np.sqrt(k)
    w = _rng(seed, which, e).standard_normal((n, k), dtype=np.float32) * np.float32(std)
    q = cfg.quant
    if q == "bf16":
        return to_bf16_bits(w), None
    if q == "fp8_tensor":
        s = np.float32(np.abs(w).max()) / np.float32(448.0)
        return to_e4m3_codes(w / s), np.float32(s)
    if q == "fp8_block":
        rs = _rng(seed, _T_S13 if which == _T_W13 else _T_S2, e)
        s = (rs.uniform(0.5, 2.0, size=(n // 128, k // 128)) / 64.0).astype(np.float32)
        full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
        return to_e4m3_codes(w / full), s
    if q == "w4a8":
        g = w.reshape(n, k // 128, 128)
        amax = np.abs(g).max(axis=-1)
        s_bits = to_bf16_bits(np.maximum(amax / np.float32(7.0), np.float32(1e-30)))
        s = bf16_bits_to_f32(s_bits)
        qv = np.clip(np.rint(g / s[..., None]), -8, 7).astype(np.int8).reshape(n, k)
        return _pack_int4(qv), s_bits
    if q in ("mxfp8", "mxfp4"):
        emax = 8 if q == "mxfp8" else 2
        X = _mx_exponent(w, emax)
        full = np.repeat(np.exp2(-X.astype(np.float64)), 32, axis=1)
        scaled = (w.astype(np.float64) * full).astype(np.float32)
        sc = (X + 127).astype(np.uint8)
        if q == "mxfp8":
            return to_e4m3_codes(scaled), sc
        c = _to_e2m1_codes(scaled)
        return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8), sc
    raise ValueError(q)


def make_weights(cfg: MoEConfig, seed: int = None) -> dict:
    """All experts' weights (and weight scales) in the canonical split layout.

    Returns a dict with
      ``w13``: bf16 bits uint16 [E,N1,H] | e4m3 uint8 [E,N1,H] | int4 uint8 [E,N1,H/2]
      ``w2``:  same formats, [E,H,I] (int4: [E,H,I/2])
      ``w13_scale``/``w2_scale``: None (bf16) | fp32 [E] | fp32 [E,N/128,K/128]
                                  | bf16 bits uint16 [E,N,K/128]
    """
    if seed is None:
        seed = weight_seed(cfg.cid)
    out = {}
    for which, name in ((_T_W13, "w13"), (_T_W2, "w2")):
        with ThreadPoolExecutor(_workers()) as ex:
            parts = list(ex.map(lambda e: _gen_expert(cfg, seed, which, e), range(cfg.E)))
        out[name] = np.stack([p[0] for p in parts])
        out[name + "_scale"] = None if parts[0][1] is None else np.stack(
            [np.asarray(p[1]) for p in parts])
    return out


def make_tokens(cfg: MoEConfig, M: int, seed: int = None) -> dict:
    """Hidden states (bf16 bits and the fp32 draw) and fp32 router logits."""
    if seed is None:
        seed = token_seed(cfg.cid, M)
    x32 = _rng(seed, _T_X).standard_normal((M, cfg.H), dtype=np.float32)
    logits = _rng(seed, _T_LOGITS).standard_normal((M, cfg.E_routed), dtype=np.float32)
    return {"x_bits": to_bf16_bits(x32), "x_f32": x32, "logits": logits}


def make_act_scales(cfg: MoEConfig, x_bits: np.ndarray) -> dict:
    """Static per-tensor activation scales (a1 for x, a2 for the intermediate).

    Only the per-tensor modes (fp8_tensor, w4a8) use them; the block mode
    quantises activations dynamically per 128 columns.
    """
    if cfg.quant not in ("fp8_tensor", "w4a8"):
        return {"a1": None, "a2": None}
    amax = np.float32(np.abs(bf16_bits_to_f32(x_bits)).max()) if x_bits.size else np.float32(1.0)
    a1 = np.float32(max(amax, np.float32(1e-30)) / np.float32(448.0))
    return {"a1": a1, "a2": np.float32(cfg.a2_const)}
