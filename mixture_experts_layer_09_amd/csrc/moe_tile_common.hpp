// Pieces shared by the tiled prefill GEMM kernels: the epilogue (activation,
// quantisation, routing weight), the workgroup -> tile mapping over the XCDs,
// the counted wait for direct-to-LDS loads and the load wrappers.
#pragma once

#include "moe_device.hpp"
#include "moe_gemm_common.hpp"

namespace moe {

// Epilogue of the tiled kernels, called by every thread of the workgroup:
// GEMM1 dequantises, applies the activation and stores the half-width rows
// (fp8-block: per token and 128 channels s = amax / 448 across the waves,
// through `lds_amax` [4][BM]); GEMM2 dequantises, applies the routing weight
// and writes the assignments' rows (24-bit codes, or bf16 for int4 weights).
template <int PHASE, int Q, int ACT, int WT, int NT>
__device__ __forceinline__ void tiled_epilogue(const GemmArgs& g, f32x4 (&acc)[WT][NT], int e,
                                               int row0, int ct, int tile0, bool active,
                                               float* lds_amax) {
  constexpr int BM = NT * 16;
  constexpr bool GATED = PHASE == 1 && act_gated(ACT);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4;
  const int mylane_row = lane & 15;
  if (PHASE == 1) {
    // ---- GEMM1 epilogue: dequantise, activate, store the half-width rows
    float alpha = 1.f;
    if (Q == MOE_QUANT_FP8_TENSOR) alpha = g.w_scale[e] * *g.a1;
    if (Q == MOE_QUANT_W4A8) alpha = *g.a1;
    constexpr int NV = GATED ? WT / 2 : WT;
    int cbase[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) cbase[v] = (GATED ? (tile0 / 2 + v) : (tile0 + v)) * 16 + grp * 4;
    auto act = [&](int c, float (&a)[NV][4]) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (GATED) {
            a[v][i] = gate_act<ACT>(alpha * acc[2 * v][c][i]) * (alpha * acc[2 * v + 1][c][i]);
          } else {
            const float h = fmaxf(alpha * acc[v][c][i], 0.f);
            a[v][i] = h * h;
          }
        }
    };
    if constexpr (kMx<Q>) {
      // MXFP8 per token and 32 channels: vectors 2b and 2b + 1 are block b
      static_assert(NV % 2 == 0, "whole 32-channel blocks per wave");
      if (active) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c < ct) {
            float a[NV][4];
            act(c, a);
            const int m = row0 + c * 16 + mylane_row;
#pragma unroll
            for (int b = 0; b < NV / 2; ++b) {
              float am = 0.f;
#pragma unroll
              for (int v = 2 * b; v < 2 * b + 2; ++v)
#pragma unroll
                for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(a[v][i]));
              am = fmaxf(am, __shfl_xor(am, 16, 64));
              am = fmaxf(am, __shfl_xor(am, 32, 64));
              const int X = mx8_exponent(am);
#pragma unroll
              for (int v = 2 * b; v < 2 * b + 2; ++v)
                *reinterpret_cast<uint32_t*>(g.out + size_t(m) * g.I + cbase[v]) =
                    mx8x4(a[v][0], a[v][1], a[v][2], a[v][3], X);
              if (grp == 0)
                g.out_sc8[size_t(m) * (g.I / 32) + cbase[2 * b] / 32] = uint8_t(X + 127);
            }
          }
        }
      }
    } else if (Q == MOE_QUANT_FP8_BLOCK) {
      // per token and 128 channels: s = amax / 448, q = e4m3(a / s)
      constexpr int CH = NV * 16;    // channels per wave
      constexpr int WPG = 128 / CH;  // waves per 128-channel group
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        float am = 0.f;
        if (active && c < ct) {
          float a[NV][4];
          act(c, a);
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(a[v][i]));
        }
        am = fmaxf(am, __shfl_xor(am, 16, 64));
        am = fmaxf(am, __shfl_xor(am, 32, 64));
        if (grp == 0) lds_amax[wave * BM + c * 16 + mylane_row] = am;
      }
      __syncthreads();
      if (active) {
        const int w0 = wave - wave % WPG;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c < ct) {
            float gm = 0.f;
#pragma unroll
            for (int w = 0; w < WPG; ++w) gm = fmaxf(gm, lds_amax[(w0 + w) * BM + c * 16 + mylane_row]);
            const float s = gm > 0.f ? gm / 448.f : 1.f;
            const float rs = 1.f / s;
            float a[NV][4];
            act(c, a);
            const int m = row0 + c * 16 + mylane_row;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const uint32_t q = e4m3x4(a[v][0] * rs, a[v][1] * rs, a[v][2] * rs, a[v][3] * rs);
              *reinterpret_cast<uint32_t*>(g.out + size_t(m) * g.I + cbase[v]) = q;
            }
            if (grp == 0 && wave == w0)
              g.out_scale[size_t(m) * (g.I / 128) + cbase[0] / 128] = s;
          }
        }
      }
    } else if (active) {
      // quotients by the intermediate scale as products with its reciprocal
      const float rs2 = (Q == MOE_QUANT_BF16) ? 1.f : 1.f / *g.a2;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        if (c < ct) {
          float a[NV][4];
          act(c, a);
          const int m = row0 + c * 16 + mylane_row;
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            if (Q == MOE_QUANT_BF16) {
              u32x2 o;
              o[0] = bf16_bits(a[v][0]) | (bf16_bits(a[v][1]) << 16);
              o[1] = bf16_bits(a[v][2]) | (bf16_bits(a[v][3]) << 16);
              *reinterpret_cast<u32x2*>(g.out + (size_t(m) * g.I + cbase[v]) * 2) = o;
            } else {
              const uint32_t q = e4m3x4(a[v][0] * rs2, a[v][1] * rs2, a[v][2] * rs2, a[v][3] * rs2);
              *reinterpret_cast<uint32_t*>(g.out + size_t(m) * g.I + cbase[v]) = q;
            }
          }
        }
      }
    }
  } else {
    // ---- GEMM2 epilogue: dequantise, weight, write the assignments' rows
    if (!active) return;
    float alpha = 1.f;
    if (Q == MOE_QUANT_FP8_TENSOR) alpha = g.w_scale[e] * *g.a2;
    if (Q == MOE_QUANT_W4A8) alpha = *g.a2;
    // the rows' assignment indices and routing weights first, all loads in
    // flight together (every row of the block exists; padding reads weight 0)
    int fs[NT];
    float ws[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) fs[c] = g.sorted_ids[row0 + c * 16 + mylane_row];
#pragma unroll
    for (int c = 0; c < NT; ++c) ws[c] = g.topk_w[fs[c] < g.A ? fs[c] : 0];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int f = fs[c];
      if (c < ct && f < g.A) {
        const float wgt = alpha * ws[c];
#pragma unroll
        for (int r = 0; r < WT; ++r) {
          const int n = (tile0 + r) * 16 + grp * 4;
          store_row4<Q>(g.out, size_t(f), g.H, n, acc[r][c] * wgt);
        }
      }
    }
  }
}

// Workgroup -> tile.  Workgroups are dealt to the 8 XCDs round robin; the
// tiles of the real blocks (known on the device only) are cut into 8
// contiguous ranges, one per XCD, so that workgroups sharing a block's token
// rows or an expert's weights run on one L2.  Workgroups past the real tiles
// return at once, spread over all XCDs rather than piled on the last one.
__device__ __forceinline__ bool xcd_tile(const GemmArgs& g, int BM, int& L) {
  const int nact = min(g.nwg, (*g.num_padded / BM) * g.slices);
  const int per = (nact + 7) / 8;
  const int j = blockIdx.x / 8;
  L = (blockIdx.x % 8) * per + j;
  return j < per && L < nact;
}

// Waits until at most N vector-memory operations of this wave are in flight
// and all its LDS operations are done, then joins the workgroup barrier.  The
// barrier carries no memory fence: the loads that matter (LDS-DMA of the
// stage about to be read) are covered by the counted wait, and the loads
// still in flight for later stages must stay in flight.
template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (no wait), lgkmcnt 11:8 = 0
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS access moves across the barrier
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

__device__ __forceinline__ void ld_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void ld_lds4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_base, 4, 0, 0);
}

}  // namespace moe
