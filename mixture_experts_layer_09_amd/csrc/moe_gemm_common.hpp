// Pieces shared by the grouped GEMM kernels.
#pragma once

#include "moe_device.hpp"
#include "moe_plan.hpp"

namespace moe {

struct GemmArgs {
  const uint8_t* b;          // B rows: GEMM1 x [T][K], GEMM2 a2 [rows][K]
  const float* b_scale;      // FP8_BLOCK: per B row per 128 K
  const uint8_t* w;          // packed weights
  const float* w_scale;      // packed scales
  const float* a1;           // static x scale (FP8_TENSOR, W4A8)
  const float* a2;           // static intermediate scale (FP8_TENSOR, W4A8)
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  const float* topk_w;       // GEMM2
  uint8_t* out;              // GEMM1: a2 [rows][I]; GEMM2: y fp32 [A][H]
  float* out_scale;          // GEMM1 FP8_BLOCK: [rows][I/128]
  const uint8_t* b_sc8;      // MX: E8M0 per B row per 32 K
  const uint8_t* w_sc8;      // MX: packed E8M0 weight scales [E][tiles/4][steps][64][4]
  uint8_t* out_sc8;          // GEMM1 MX: E8M0 [rows][I/32]
  int K, N, I, H, Kp, A, steps, tiles;
  int slices;                // tiled kernel: workgroups along the weight rows
  int nwg;                   // tiled kernel: real workgroups (grid is padded to 8)
  int E;                     // expert slots
  // one-token decode (Plan::slot_rows): the expert of each assignment; GEMM1
  // block b holds assignment b alone and the intermediate of slot f sits at
  // row 16 f (null: blocks and rows from the alignment)
  const int32_t* slot_ids;
};

// Per-format constants: u32x4 loads per A / B fragment, bytes per A
// fragment, K elements per MFMA k-step, B element bytes.
template <int Q> struct QT;
template <> struct QT<MOE_QUANT_BF16> {
  static constexpr int AV = 1, BV = 1, FRAG = 1024, KSTEP = 32, EB = 2;
};
template <> struct QT<MOE_QUANT_FP8_TENSOR> {
  static constexpr int AV = 2, BV = 2, FRAG = 2048, KSTEP = 128, EB = 1;
};
template <> struct QT<MOE_QUANT_FP8_BLOCK> {
  static constexpr int AV = 2, BV = 2, FRAG = 2048, KSTEP = 128, EB = 1;
};
template <> struct QT<MOE_QUANT_W4A8> {
  static constexpr int AV = 1, BV = 2, FRAG = 1024, KSTEP = 128, EB = 1;
};
template <> struct QT<MOE_QUANT_MXFP8> {
  static constexpr int AV = 2, BV = 2, FRAG = 2048, KSTEP = 128, EB = 1;
};
template <> struct QT<MOE_QUANT_MXFP4> {
  static constexpr int AV = 1, BV = 2, FRAG = 1024, KSTEP = 128, EB = 1;
};

template <int Q> constexpr bool kMx = Q == MOE_QUANT_MXFP8 || Q == MOE_QUANT_MXFP4;
// Element format of the weights in the scaled MFMA: 0 e4m3, 4 e2m1.
template <int Q> constexpr int kMxWFmt = Q == MOE_QUANT_MXFP4 ? 4 : 0;

// An MX token (B) fragment's two 16-byte halves: k 16g.. and 64+16g.. of the
// k-step for lane group g (the scaled MFMA's e4m3 operand order).
constexpr int kMxHalfStride = 64;

// The weight operand of the scaled MFMA from a fragment's lane bytes.
template <int Q>
__device__ __forceinline__ i32x8 mx_weight_operand(const u32x4& lo, const u32x4& hi) {
  if constexpr (Q == MOE_QUANT_MXFP4) {
    i32x8 r;
    r[0] = int(lo[0]); r[1] = int(lo[1]); r[2] = int(lo[2]); r[3] = int(lo[3]);
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
  } else {
    i32x8 r;
    r[0] = int(lo[0]); r[1] = int(lo[1]); r[2] = int(lo[2]); r[3] = int(lo[3]);
    r[4] = int(hi[0]); r[5] = int(hi[1]); r[6] = int(hi[2]); r[7] = int(hi[3]);
    return r;
  }
}

__device__ __forceinline__ i32x8 fp8_pair(const u32x4& lo, const u32x4& hi) {
  i32x8 r;
  r[0] = int(lo[0]); r[1] = int(lo[1]); r[2] = int(lo[2]); r[3] = int(lo[3]);
  r[4] = int(hi[0]); r[5] = int(hi[1]); r[6] = int(hi[2]); r[7] = int(hi[3]);
  return r;
}

// GEMM2's per-assignment rows, summed by the combine.  bf16 for int4
// weights (W4A8), whose outputs the method holds to a relative L2 error of
// 3e-2 only -- rounding the ~8 weighted rows of a token to bf16 adds ~1e-3.
// Otherwise fp32 rounded to nearest even at its upper 24 bits (sign, the full
// exponent, 15 mantissa bits: relative error <= 2^-16 per row, ~1e-4 of an
// output at most against the 2e-2 bound) and stored in 3 bytes, so that the
// rows' round trip through HBM moves three quarters of fp32's bytes.
template <int Q> constexpr bool kRowsBf16 = rows_bf16(Q);

// The 24-bit row code of v: round to nearest even at bit 8 (a carry into
// the exponent is the correct rounding, up to infinity); a NaN keeps its
// upper bits with the quiet bit set, so that no payload is rounded away.
__device__ __forceinline__ uint32_t f24_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t c = (u + 0x7Fu + ((u >> 8) & 1u)) >> 8;
  return v != v ? (u >> 8) | 0x4000u : c;
}
__device__ __forceinline__ float f24_to_f32(uint32_t code) { return __uint_as_float(code << 8); }

// The value GEMM2 stores for v.
template <int Q>
__device__ __forceinline__ float row_round(float v) {
  if constexpr (kRowsBf16<Q>) return bf16_to_f32(bf16_bits(v));
  else return f24_to_f32(f24_bits(v));
}

// Four consecutive values of row f (element n, a multiple of 4) of the
// per-assignment rows y: 8 bytes (bf16) or 12 (24-bit codes, value i in bytes
// 3i .. 3i + 2, little-endian; three 4-byte stores, the address being a
// multiple of 4 only).
template <int Q>
__device__ __forceinline__ void store_row4(uint8_t* y, size_t f, int H, int n, const f32x4& v) {
  if constexpr (kRowsBf16<Q>) {
    u32x2 o;
    o[0] = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
    o[1] = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
    *reinterpret_cast<u32x2*>(y + (f * H + n) * 2) = o;
  } else {
    const uint32_t c0 = f24_bits(v[0]), c1 = f24_bits(v[1]), c2 = f24_bits(v[2]),
                   c3 = f24_bits(v[3]);
    uint32_t* d = reinterpret_cast<uint32_t*>(y + (f * H + n) * 3);
    d[0] = c0 | (c1 << 24);
    d[1] = (c1 >> 8) | (c2 << 16);
    d[2] = (c2 >> 16) | (c3 << 8);
  }
}

// Gated activations pair a gate and an up channel; relu2 is the one that is not.
constexpr bool act_gated(int act) { return act != MOE_ACT_RELU2; }

// The gate half's nonlinearity of a gated activation.
template <int ACT>
__device__ __forceinline__ float gate_act(float g) {
  if constexpr (ACT == MOE_ACT_GELU_TANH_GATED) return gelu_tanh(g);
  else return silu(g);
}

// Weight row block (128 rows, checkpoint order) of a packed W13 row tile.
__device__ __forceinline__ int w13_row_block(int tile, int I, bool gated) {
  if (!gated) return tile / 8;
  const int pair = tile >> 1, half = tile & 1;
  return (half * I + pair * 16) / 128;
}

// The tiled (prefill) kernels; `a.slices` and `a.nwg` must be set.
hipError_t launch_gemm_tiled(int phase, const moe_problem& p, const GemmCfg& c,
                             const GemmArgs& a, hipStream_t st);

}  // namespace moe
