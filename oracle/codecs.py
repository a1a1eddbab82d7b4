"""Number formats used by the layer, written from their definitions.

TEST INFRASTRUCTURE (see the package docstring).

* bf16: the upper 16 bits of an IEEE binary32 pattern; fp32 -> bf16 rounds to
  nearest, ties to even.
* OCP 8-bit floating point, E4M3FN variant (the "FP8" / ``fp8_w8a8`` format of
  the Qwen3-Next FP8 page and the TRTLLM-Gen page): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m/8 * 2^-6; S.1111.111 is NaN; there are no infinities; the largest finite
  magnitude is 448.  Encoding rounds to the nearest representable value with
  ties to the even code and, in the saturating mode used here, clamps
  magnitudes above 448 to 448.
* signed int4: two's complement in [-8, 7], two per byte, even k in the low
  nibble (the W4A8 page stores int4 weights with group scales; it does not
  print the nibble order, this is the reading taken).
* OCP Microscaling (MX) formats, as the OCP MX specification v1.0 defines
  them (the TRTLLM-Gen page names MXFP8 weights with one scale per 32 K
  elements; the 4-bit weights of the pages are taken as MXFP4):
  - E8M0 scale: 8 exponent bits, bias 127, no sign or mantissa; code c is
    2^(c - 127); 0xFF is NaN;
  - E2M1 element (FP4): 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
    bit; exponent field 0 is subnormal (m/2); magnitudes 0, 0.5, 1, 1.5, 2,
    3, 4, 6; no NaN or infinity.  Two per byte, even k in the low nibble.
"""
import numpy as np

E4M3_MAX = 448.0


def bf16_decode(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x):
    """Round to the nearest bf16, ties to even, via fp32; returns float64.

    The value is first taken to fp32 (the kernels' working precision), then the
    low 16 bits of the fp32 pattern are rounded away.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    out = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def _e4m3_value(codes):
    """The e4m3fn value of each code, from the field definitions."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(exp == 0,
                   man / 8.0 * 2.0 ** -6,
                   (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0))
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


_E4M3_TABLE = _e4m3_value(np.arange(256, dtype=np.uint8))


def e4m3_decode(codes):
    """OCP e4m3fn codes (uint8) -> float64 values (a lookup in the table of all
    256 codes evaluated from the field definitions)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# The non-negative finite values in code order: code c (0..126) has value
# _POS[c], and the values increase with the code.
_POS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(x):
    """fp32 values -> OCP e4m3fn codes, round-to-nearest-even, saturating.

    Written as "pick the nearest of the 127 non-negative representable values"
    rather than with bit arithmetic: ties go to the even code (the even
    mantissa), magnitudes >= 448 give 448, the sign bit is copied from the
    input (so -0.0 -> 0x80), NaN -> 0x7F.
    """
    f = np.asarray(x, dtype=np.float32)
    a = np.abs(f.astype(np.float64))
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 1, 126)
    lo = hi - 1
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)
    code = np.where(a == 0.0, 0, code)
    code = code | (np.signbit(f).astype(np.int64) << 7)
    code = np.where(np.isnan(f), 0x7F, code)
    return code.astype(np.uint8)


def int4_unpack(packed):
    """[..., K/2] uint8 -> [..., K] int8: low nibble is the even k, two's complement."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def e8m0_decode(codes):
    """E8M0 scale codes (uint8) -> float64 2^(c - 127); 0xFF -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2((c - 127).astype(np.float64)))


def _e2m1_value(codes):
    """The E2M1 value of each 4-bit code, from the field definitions."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = (c >> 3) & 1
    exp = (c >> 1) & 0x3
    man = c & 0x1
    mag = np.where(exp == 0, man / 2.0, (1.0 + man / 2.0) * np.exp2(exp - 1.0))
    return np.where(sign == 1, -mag, mag)


_E2M1_TABLE = _e2m1_value(np.arange(16))


def e2m1_unpack_decode(packed):
    """[..., K/2] uint8 of two E2M1 codes (even k in the low nibble) ->
    [..., K] float64 values."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = _E2M1_TABLE[p & 0xF]
    out[..., 1::2] = _E2M1_TABLE[p >> 4]
    return out
