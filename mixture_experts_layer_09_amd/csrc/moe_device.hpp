// Device helpers for the gfx950 kernels: vector types, MFMA wrappers, number
// format conversions and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Weights are read once per pass: keep them from displacing reused lines.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- MFMA
// D[16x16] += A[16x128] * B[128x16] with one E8M0 scale per row / column and
// 32 k (the OCP MX block): the scale of row (A) or column (B) r over k-block
// kb comes from lane 16 kb + r (sa: byte SA of the lane's register, sb: its
// low byte).  FA, FB: element formats, 0 = e4m3, 4 = e2m1.  An e4m3 operand
// lane l (g = l / 16) holds k 16g..16g+15 in bytes 0..15 and
// 64+16g..64+16g+15 in bytes 16..31; an e2m1 operand holds k 32g..32g+31 as
// 32 nibbles (low nibble first) in its first 16 bytes.
template <int FA, int FB, int SA = 0>
__device__ __forceinline__ f32x4 mfma_mx(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, SA, sa, 0, sb);
}

// The same with the A scale taken from byte `sel` (0..3, known once the
// caller's loop is unrolled) of `sa`: four weight tiles' scales in one register.
template <int FA, int FB>
__device__ __forceinline__ f32x4 mfma_mx_sel(const i32x8& a, const i32x8& b, f32x4 c, int sa,
                                             int sel, int sb) {
  switch (sel) {
    case 0: return mfma_mx<FA, FB, 0>(a, b, c, sa, sb);
    case 1: return mfma_mx<FA, FB, 1>(a, b, c, sa, sb);
    case 2: return mfma_mx<FA, FB, 2>(a, b, c, sa, sb);
    default: return mfma_mx<FA, FB, 3>(a, b, c, sa, sb);
  }
}

// D[16x16] += A[16x32] * B[32x16] in bf16.  Lane l holds row (A) / column
// (B) l % 16 and the 8 consecutive k at 8 * (l / 16); the result is
// D[4 * (l / 16) + i][l % 16] in element i.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D[16x16] += A[16x128] * B[128x16] in OCP e4m3 (unit block scales).  Lane l
// holds row / column l % 16 and the 32 consecutive k at 32 * (l / 16).
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------- formats
// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Four fp32 values -> four e4m3 codes (byte i from v[i]).  The hardware
// conversion rounds to nearest even but turns magnitudes past the largest
// finite value into NaN, so values are clamped to +-448 first.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return uint32_t(w);
}

// MXFP8 shared exponent of a block with maximum magnitude `amax` (OCP MX
// v1.0): floor(log2 amax) - 8 (8 = the e4m3 emax), at least -127; an
// all-zero or subnormal amax gives -127.  The E8M0 code is the result + 127.
__device__ __forceinline__ int mx8_exponent(float amax) {
  const int ef = int((__float_as_uint(amax) >> 23) & 0xFFu);
  return max(ef - 127 - 8, -127);
}

// e4m3 codes of v / 2^X (exact scaling), saturating at 448.
__device__ __forceinline__ uint32_t mx8x4(float a, float b, float c, float d, int X) {
  return e4m3x4(__builtin_amdgcn_ldexpf(a, -X), __builtin_amdgcn_ldexpf(b, -X),
                __builtin_amdgcn_ldexpf(c, -X), __builtin_amdgcn_ldexpf(d, -X));
}

// Signed int4 -> e4m3 codes, exact.  Bits 0-3 of each byte of `v` hold one
// nibble value (two's complement; bits 4-7 are ignored); the result holds
// the e4m3 code of each.  Two byte-permute table lookups on bits 0-2 (values
// 0..7 and -8..-1), and a per-byte select on the sign (bit 3) through a
// third permute: selector byte 5 reads a zero byte of the zero sources,
// selector 13 yields 0xFF.
__device__ __forceinline__ uint32_t int4x4_to_e4m3(uint32_t v) {
  const uint32_t sel = v & 0x07070707u;
  // codes of 0,1,2,3 | 4,5,6,7
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, sel);
  // codes of -8,-7,-6,-5 | -4,-3,-2,-1
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, sel);
  // 0xFF in the bytes whose sign bit is set
  const uint32_t m = __builtin_amdgcn_perm(0u, 0u, (v & 0x08080808u) | 0x05050505u);
  return (neg & m) | (pos & ~m);
}

// 16 bytes of packed int4 (32 values) -> 32 e4m3 codes.  Byte b of input
// dword q holds value 8q + b in its low nibble and 8q + 4 + b in its high
// nibble, so output dword 2q takes the low nibbles and 2q + 1 the high ones
// (shifted down by 4: each byte's bits 0-3 are then its high nibble).
__device__ __forceinline__ i32x8 int4x32_to_e4m3(const u32x4& v) {
  i32x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[2 * q] = int32_t(int4x4_to_e4m3(v[q]));
    r[2 * q + 1] = int32_t(int4x4_to_e4m3(v[q] >> 4));
  }
  return r;
}

// ---------------------------------------------------------------- math
// SiLU from its definition, g * sigmoid(g), in fp32 with the hardware base-2
// exponential and reciprocal (each within about one ulp): e^-g = 2^(-g log2 e).
// Large negative g gives 2^+inf = inf, reciprocal 0, result -0; large positive
// g gives 2^-inf = 0 and g itself.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// GELU, tanh form: 0.5 g (1 + tanh(u)), u = sqrt(2/pi) (g + 0.044715 g^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), this is g / (1 + 2^z) with
// z = -2 log2(e) u = g (c1 + c3 g^2): one exp2, one reciprocal, as SiLU.
__device__ __forceinline__ float gelu_tanh(float g) {
  constexpr float c1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float c3 = c1 * 0.044715f;
  const float z = g * __builtin_fmaf(c3, g * g, c1);
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- DPP
// Wave64 reductions and scans through DPP lane permutes (register to
// register, no LDS round trip): within each row of 16 lanes quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and row_mirror bring every
// lane the row's result; row_bcast:15 and row_bcast:31 then carry rows 0-2
// into row 3, whose last lane (63) ends with the whole wave's result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), CTRL, ROW_MASK, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t k) {
  const uint32_t lo = uint32_t(k), hi = uint32_t(k >> 32);
  const uint64_t o = (uint64_t(dpp<CTRL, ROW_MASK>(hi, hi)) << 32) | dpp<CTRL, ROW_MASK>(lo, lo);
  return o > k ? o : k;
}

// Maximum of a 64-bit key over the wave, returned to every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = dpp_max_step<kDppXor1, 0xF>(k);
  k = dpp_max_step<kDppXor2, 0xF>(k);
  k = dpp_max_step<kDppHalfMirror, 0xF>(k);
  k = dpp_max_step<kDppMirror, 0xF>(k);
  k = dpp_max_step<kDppBcast15, 0xA>(k);
  k = dpp_max_step<kDppBcast31, 0xC>(k);
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(k), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(k >> 32), 63);
  return (uint64_t(hi) << 32) | lo;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_step(float v) {
  return v + __uint_as_float(dpp<CTRL, ROW_MASK>(0u, __float_as_uint(v)));
}

// Sum of a float over the wave, returned to every lane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __uint_as_float(dpp<kDppXor1, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppXor2, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppHalfMirror, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppMirror, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppBcast15, 0xA>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppBcast31, 0xC>(0u, __float_as_uint(v)));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Inclusive prefix sum of an int over the wave (lane i gets lanes 0..i).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += int(dpp<kDppShr1, 0xF>(0u, uint32_t(v)));
  v += int(dpp<kDppShr2, 0xF>(0u, uint32_t(v)));
  v += int(dpp<kDppShr4, 0xF>(0u, uint32_t(v)));
  v += int(dpp<kDppShr8, 0xF>(0u, uint32_t(v)));
  v += int(dpp<kDppBcast15, 0xA>(0u, uint32_t(v)));
  v += int(dpp<kDppBcast31, 0xC>(0u, uint32_t(v)));
  return v;
}

}  // namespace moe
