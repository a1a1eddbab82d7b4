// Grouped expert GEMMs: GEMM1 with the activation in its epilogue, GEMM2 with
// the routing weight, and the combine back into token order.
//
// GEMM1 (sglang PR 32944 page, sections 1-2; flashinfer PR 4329 page,
// section 2): for each block of 16 aligned rows of expert e, h = W13[e] . x
// over the gathered tokens; the packed W13 holds each group of 16 gate rows
// next to its 16 up rows, so a wave computing a (gate, up) tile pair holds
// gate channel c and up channel c in the same lane and register and applies
// SiLU(gate) * up or GELU_tanh(gate) * up (flashinfer PR 4329 page, sections
// 1 and 3) -- or relu(h)^2 for the non-gated layer (sglang PR 21321 page) --
// before anything leaves registers; only the I activated columns are stored,
// in the compute format.
// GEMM2 (flashinfer PR 4329 page, sections 3-4): y = W2[e] . a, scaled by the
// routing weight, written per assignment (fp32 rounded to 24 bits, bf16 for
// int4 weights); the combine then sums each token's K' rows in fp32 in slot
// order and rounds once to bf16.
//
// MFMA operands: the weights are the A operand (16 weight rows per tile) and
// the tokens the B operand (16 tokens per tile), so a block with a handful of
// tokens still streams whole weight rows through the matrix cores.  Weights
// come straight from HBM into registers in 16-byte lane loads of pre-tiled
// fragments (1 or 2 KiB per wave load); several k-steps of fragments are in
// flight per wave.  The MX modes feed each lane's E8M0 weight and token
// scales to the scaled MFMA, which applies them per 32 k.
#include "moe_device.hpp"
#include "moe_gemm_common.hpp"
#include "moe_launch.hpp"

namespace moe {

namespace {
template <int Q, int WT>
struct Stage {
  u32x4 a[WT][QT<Q>::AV];
  u32x4 b[QT<Q>::BV];
  float bs;        // FP8_BLOCK: B row scale of this k-block
  float ws[WT];    // FP8_BLOCK: weight block scale per tile
  f32x4 ws4[WT];   // W4A8: group scales of the lane's 4 rows per tile
  int bsc;         // MX: the lane's E8M0 B scale (its column, k-block l / 16)
  int wsc4;        // MX: the lane's E8M0 weight scales of the 4 tiles, a byte each
};
}  // namespace

template <int PHASE, int Q, int ACT, int WT, int KS>
__global__ __launch_bounds__(256) void gemm_stream(GemmArgs g) {
  using T = QT<Q>;
  constexpr int RG = 4 / KS;       // waves along the weight rows
  constexpr int TPW = RG * WT;     // row tiles per workgroup
  constexpr int D = Q == MOE_QUANT_BF16 ? 4 : 2;  // k-steps loaded ahead
  constexpr bool GATED = PHASE == 1 && act_gated(ACT);
  constexpr bool MX = kMx<Q>;
  // B bytes of a lane: one 32-byte k-run, or (MX) two 16-byte halves 64 apart
  constexpr int BRUN = MX ? 16 : T::KSTEP / 4, BHALF = MX ? kMxHalfStride : 16;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = wave % RG, kp = wave / RG;
  const int blk = blockIdx.y;
  int e;
  if (g.slot_ids) {  // block blk: assignment blk alone (a masked slot has no block)
    e = g.slot_ids[blk];
    if (e < 0 || e >= g.E) return;  // uniform
  } else {
    if (blk * 16 >= *g.num_padded) return;  // uniform: past the last real block
    e = g.block_expert[blk];
  }
  const int tile0 = blockIdx.x * TPW + rg * WT;
  const bool active = tile0 < g.tiles;
  const int grp = lane >> 4;            // k-run of the lane
  const int m = blk * 16 + (lane & 15); // padded row = B column of the lane
  const int f = g.slot_ids ? ((lane & 15) == 0 ? blk : g.A) : g.sorted_ids[m];

  // B row of the lane: GEMM1 gathers the token, GEMM2 reads the padded row.
  int brow;
  if (PHASE == 1) brow = f < g.A ? f / g.Kp : 0;
  else brow = m;
  const uint8_t* bp = g.b + (size_t(brow) * g.K + grp * BRUN) * T::EB;
  const size_t ebytes = size_t(g.tiles) * g.steps * T::FRAG;
  const uint8_t* wp = g.w + size_t(e) * ebytes + size_t(tile0) * g.steps * T::FRAG + lane * 16;
  const int kblocks = g.K / 128;

  const int per = (g.steps + KS - 1) / KS;
  const int s0 = min(g.steps, kp * per), s1 = min(g.steps, s0 + per);

  f32x4 acc[WT];
#pragma unroll
  for (int j = 0; j < WT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](Stage<Q, WT>& S, int s) {
#pragma unroll
    for (int j = 0; j < WT; ++j) {
      const uint8_t* p = wp + (size_t(j) * g.steps + s) * T::FRAG;
#pragma unroll
      for (int v = 0; v < T::AV; ++v) S.a[j][v] = ld16_stream(p + v * 1024);
    }
    const uint8_t* q = bp + size_t(s) * T::KSTEP * T::EB;
#pragma unroll
    for (int v = 0; v < T::BV; ++v) S.b[v] = ld16(q + v * BHALF);
    if (Q == MOE_QUANT_FP8_BLOCK) {
      S.bs = g.b_scale[size_t(brow) * kblocks + s];
#pragma unroll
      for (int j = 0; j < WT; ++j) {
        const int rb = PHASE == 1 ? w13_row_block(tile0 + j, g.I, GATED) : (tile0 + j) / 8;
        S.ws[j] = g.w_scale[(size_t(e) * (g.N / 128) + rb) * kblocks + s];
      }
    }
    if (Q == MOE_QUANT_W4A8) {
#pragma unroll
      for (int j = 0; j < WT; ++j)
        S.ws4[j] = *reinterpret_cast<const f32x4*>(
            g.w_scale + ((size_t(e) * g.tiles + tile0 + j) * g.steps + s) * 16 + grp * 4);
    }
    if (MX) {
      S.bsc = g.b_sc8[size_t(brow) * (g.K / 32) + s * 4 + grp];
      S.wsc4 = *reinterpret_cast<const int*>(
          g.w_sc8 + (((size_t(e) * (g.tiles / 4) + tile0 / 4) * g.steps + s) * 64 + lane) * 4);
    }
  };

  auto compute = [&](const Stage<Q, WT>& S) {
    if (Q == MOE_QUANT_BF16) {
#pragma unroll
      for (int j = 0; j < WT; ++j) acc[j] = mfma_bf16(S.a[j][0], S.b[0], acc[j]);
    } else if (MX) {
      static_assert(!MX || WT == 4, "MX: a wave's tiles are one 4-tile scale group");
      const i32x8 bb = fp8_pair(S.b[0], S.b[1]);
#pragma unroll
      for (int j = 0; j < WT; ++j)
        acc[j] = mfma_mx_sel<kMxWFmt<Q>, 0>(mx_weight_operand<Q>(S.a[j][0], S.a[j][T::AV - 1]),
                                            bb, acc[j], S.wsc4, j, S.bsc);
    } else {
      const i32x8 bb = fp8_pair(S.b[0], S.b[1]);
#pragma unroll
      for (int j = 0; j < WT; ++j) {
        if (Q == MOE_QUANT_FP8_TENSOR) {
          acc[j] = mfma_fp8(fp8_pair(S.a[j][0], S.a[j][1]), bb, acc[j]);
        } else if (Q == MOE_QUANT_FP8_BLOCK) {
          const f32x4 p = mfma_fp8(fp8_pair(S.a[j][0], S.a[j][1]), bb, f32x4{0.f, 0.f, 0.f, 0.f});
          const float sc = S.bs * S.ws[j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(p[i], sc, acc[j][i]);
        } else {
          const f32x4 p = mfma_fp8(int4x32_to_e4m3(S.a[j][0]), bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(p[i], S.ws4[j][i], acc[j][i]);
        }
      }
    }
  };

  if (active) {
    // D stages in a ring; the r steps past the last whole group of D are
    // loaded as the last group's stages free up (not one at a time, each
    // waiting for its own load); steps are computed in k order throughout
    Stage<Q, WT> st[D];
    const int n = s1 - s0;
    const int G = n / D, r = n - G * D;
    if (G > 0) {
#pragma unroll
      for (int d = 0; d < D; ++d) load(st[d], s0 + d);
      for (int gi = 0; gi < G - 1; ++gi) {
        const int sn = s0 + (gi + 1) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          compute(st[d]);
          load(st[d], sn + d);
        }
      }
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute(st[d]);
        if (d < r) load(st[d], s0 + G * D + d);
      }
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d)
        if (d < r) load(st[d], s0 + d);
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < r) compute(st[d]);
  }

  // ---- K-split: the partial sums of waves kp > 0 join wave kp == 0
  if (KS > 1) {
    __shared__ f32x4 red[(KS > 1 ? KS - 1 : 1) * RG * WT * 64];
    if (kp > 0) {
#pragma unroll
      for (int j = 0; j < WT; ++j) red[(((kp - 1) * RG + rg) * WT + j) * 64 + lane] = acc[j];
    }
    __syncthreads();
    if (kp == 0) {
      for (int k = 1; k < KS; ++k) {
#pragma unroll
        for (int j = 0; j < WT; ++j) {
          const f32x4 o = red[(((k - 1) * RG + rg) * WT + j) * 64 + lane];
          acc[j] += o;
        }
      }
    }
    if (kp > 0) return;
  }

  if (PHASE == 1) {
    // ---- GEMM1 epilogue: dequantise, activate, store the half-width row
    float alpha = 1.f;
    if (Q == MOE_QUANT_FP8_TENSOR) alpha = g.w_scale[e] * *g.a1;
    if (Q == MOE_QUANT_W4A8) alpha = *g.a1;
    constexpr int NV = GATED ? WT / 2 : WT;  // 4-channel vectors per lane
    float a[NV][4];
    int cbase[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (GATED) {
          const float gt = alpha * acc[2 * v][i], up = alpha * acc[2 * v + 1][i];
          a[v][i] = gate_act<ACT>(gt) * up;
        } else {
          const float h = fmaxf(alpha * acc[v][i], 0.f);
          a[v][i] = h * h;
        }
      }
      cbase[v] = (GATED ? (tile0 / 2 + v) : (tile0 + v)) * 16 + grp * 4;
    }
    if (Q == MOE_QUANT_BF16) {
      if (active) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          u32x2 o;
          o[0] = bf16_bits(a[v][0]) | (bf16_bits(a[v][1]) << 16);
          o[1] = bf16_bits(a[v][2]) | (bf16_bits(a[v][3]) << 16);
          *reinterpret_cast<u32x2*>(g.out + (size_t(m) * g.I + cbase[v]) * 2) = o;
        }
      }
    } else if (MX) {
      // MXFP8 per token and 32 channels: vectors 2b and 2b + 1 are block b
      static_assert(!MX || NV % 2 == 0, "whole 32-channel blocks per wave");
      if (active) {
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
          if (grp == 0) g.out_sc8[size_t(m) * (g.I / 32) + cbase[2 * b] / 32] = uint8_t(X + 127);
        }
      }
    } else if (Q == MOE_QUANT_FP8_BLOCK) {
      // per token and 128 channels: s = amax / 448, q = e4m3(a / s)
      __shared__ float amax_s[4][16];
      constexpr int CH = NV * 16;  // channels per wave
      constexpr int WPG = 128 / CH;  // waves per 128-channel group
      float am = 0.f;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(a[v][i]));
      am = fmaxf(am, __shfl_xor(am, 16, 64));
      am = fmaxf(am, __shfl_xor(am, 32, 64));
      if (grp == 0) amax_s[wave][lane & 15] = active ? am : 0.f;
      __syncthreads();
      const int w0 = wave - wave % WPG;
      float gm = 0.f;
#pragma unroll
      for (int w = 0; w < WPG; ++w) gm = fmaxf(gm, amax_s[w0 + w][lane & 15]);
      const float s = gm > 0.f ? gm / 448.f : 1.f;
      if (active) {
        const float rs = 1.f / s;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const uint32_t q = e4m3x4(a[v][0] * rs, a[v][1] * rs, a[v][2] * rs, a[v][3] * rs);
          *reinterpret_cast<uint32_t*>(g.out + size_t(m) * g.I + cbase[v]) = q;
        }
        if (grp == 0 && wave == w0) g.out_scale[size_t(m) * (g.I / 128) + cbase[0] / 128] = s;
      }
    } else {
      if (active) {
        const float rs2 = 1.f / *g.a2;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const uint32_t q = e4m3x4(a[v][0] * rs2, a[v][1] * rs2, a[v][2] * rs2, a[v][3] * rs2);
          *reinterpret_cast<uint32_t*>(g.out + size_t(m) * g.I + cbase[v]) = q;
        }
      }
    }
  } else {
    // ---- GEMM2 epilogue: dequantise, weight, write the assignment's row
    if (!active || f >= g.A) return;
    float alpha = 1.f;
    if (Q == MOE_QUANT_FP8_TENSOR) alpha = g.w_scale[e] * *g.a2;
    if (Q == MOE_QUANT_W4A8) alpha = *g.a2;
    const float wgt = alpha * g.topk_w[f];
#pragma unroll
    for (int j = 0; j < WT; ++j) {
      const int n = (tile0 + j) * 16 + grp * 4;
      store_row4<Q>(g.out, size_t(f), g.H, n, acc[j] * wgt);
    }
  }
}

// out[t][:] = bf16(sum over valid slots j of y[t*K' + j][:]) with y in 24-bit
// codes (RB = 3) or bf16 (RB = 2, the rows of int4 weights), summed in fp32,
// one thread per 8 hidden values.  The rows of up to 8 slots are loaded
// before any is added, so each thread has 16 loads in flight; the sum still
// runs in slot order.  Every slot's row lies inside y, so the rows are
// loaded together with the ids rather than after them; a slot whose id is
// outside [0, E) (never written by GEMM2) is loaded and left out of the sum.
// (4 or 16 values per thread, or plain instead of non-temporal loads, were
// measured slower.)
template <int RB>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ ids,
                                                     const void* __restrict__ yv,
                                                     uint16_t* __restrict__ out, int T, int H,
                                                     int Kp, int E) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int h8 = H / 8;
  if (i >= int64_t(T) * h8) return;
  const int t = int(i / h8), c = int(i % h8) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < Kp; j0 += 8) {
    f32x4 v[8][2];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const int e = j < Kp ? ids[size_t(t) * Kp + j] : -1;
      ok[u] = e >= 0 && e < E;
      if (j < Kp) {
        const size_t at = (size_t(t) * Kp + j) * H + c;
        if constexpr (RB == 2) {
          const u32x4 b = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(yv) + at));
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            v[u][0][2 * k] = bf16_to_f32(b[k] & 0xFFFFu);
            v[u][0][2 * k + 1] = bf16_to_f32(b[k] >> 16);
            v[u][1][2 * k] = bf16_to_f32(b[2 + k] & 0xFFFFu);
            v[u][1][2 * k + 1] = bf16_to_f32(b[2 + k] >> 16);
          }
        } else {
          // 24 bytes, 8-byte aligned (H is a multiple of 8): value i of a
          // group of four in bytes 3i .. 3i + 2
          const u32x2* row = reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(yv) + at * 3);
          const u32x2 p0 = __builtin_nontemporal_load(row), p1 = __builtin_nontemporal_load(row + 1),
                      p2 = __builtin_nontemporal_load(row + 2);
          const uint32_t d[6] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1]};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t a = d[3 * h], b = d[3 * h + 1], c2 = d[3 * h + 2];
            v[u][h][0] = f24_to_f32(a);
            v[u][h][1] = f24_to_f32((a >> 24) | (b << 8));
            v[u][h][2] = f24_to_f32((b >> 16) | (c2 << 16));
            v[u][h][3] = f24_to_f32(c2 >> 8);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (ok[u]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          s[k] += v[u][0][k];
          s[4 + k] += v[u][1][k];
        }
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = bf16_bits(s[2 * k]) | (bf16_bits(s[2 * k + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + size_t(t) * H + c) = o;
}

// GEMM2 and the combine in one kernel, token by token, for small batches: a
// workgroup owns one token and 16 output channels and runs GEMM2 for each of
// the token's slots -- the same fragments, k ranges and four-way K split as
// gemm_stream<2, Q, 0, WT, 4>, so every slot's row is the one that kernel
// writes (rounded as it stores it) -- then sums the routing-weighted rows in
// slot order and rounds once to bf16, as combine_kernel does: the output is
// bit-identical to gemm_stream<2> followed by combine_kernel, without the
// per-assignment rows leaving the chip.  16 waves: wave w takes K quarter w % 4 of the slots
// (w / 4), (w / 4) + 4, ..., so that a wave has all its k-steps in flight at
// once.  The padded row of each slot's intermediate is found by a scan of
// sorted_ids.  Each weight tile a token routes to is streamed for that token
// alone, which is what a batch of a handful of tokens does anyway.
template <int Q>
__global__ __launch_bounds__(1024) void gemm2_combine_tok(GemmArgs g, const int32_t* __restrict__ ids,
                                                         uint16_t* __restrict__ out, int E) {
  using T = QT<Q>;
  constexpr int KS = 4, SG = 4;                       // K quarters x slot groups = 16 waves
  constexpr int D = Q == MOE_QUANT_BF16 ? 8 : 4;      // (slot, k-step) items in flight per wave
  constexpr bool MX = kMx<Q>;
  constexpr int BRUN = MX ? 16 : T::KSTEP / 4, BHALF = MX ? kMxHalfStride : 16;
  constexpr int KMAX = kMaxSlots;
  __shared__ int slot_row[KS * SG * KMAX];  // per wave: padded row of each slot
  __shared__ float slot_wgt[KMAX];
  __shared__ f32x4 red[KS][KMAX][4];  // the 4 lanes holding column 0, per K quarter and slot
  __shared__ f32x4 rowv[KMAX][4];     // each valid slot's row (16 channels), in slot order

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4;
  const int kq = wave % KS, sg = wave / KS;
  const int tile = blockIdx.x, t = blockIdx.y, Kp = g.Kp, f0 = t * Kp;
  // ---- the token's slots, in every wave: lane j holds slot j's expert; the
  // valid slots (ids in [0, E)) in slot order are the set bits of `vmask`
  const int my_e = lane < Kp ? ids[f0 + lane] : -1;
  const uint64_t vmask = __ballot(my_e >= 0 && my_e < E);
  const int nv = __popcll(vmask);
  // the j-th valid slot: the position of the j-th set bit
  auto nth_slot = [&](int q) {
    uint64_t m = vmask;
    for (int c = 0; c < q; ++c) m &= m - 1;
    return int(__builtin_ctzll(m));
  };
  // the padded row of each slot's intermediate, from a scan of sorted_ids by
  // this wave (into this wave's part of slot_row: no barrier needed), or,
  // with one block per assignment, row 16 f
  int* rows = slot_row + wave * KMAX;
  if (g.slot_ids) {
    if (lane < Kp) rows[lane] = (f0 + lane) * 16;
  } else {
    const int npad = *g.num_padded;
    for (int r0 = 0; r0 < npad; r0 += 64) {
      const int r = r0 + lane;
      const int f = r < npad ? g.sorted_ids[r] : g.A;
      if (f >= f0 && f < f0 + Kp) rows[f - f0] = r;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes done (lgkmcnt 0)
  __builtin_amdgcn_wave_barrier();
  if (wave == 0 && lane < Kp) slot_wgt[lane] = g.topk_w[f0 + lane];

  const int per = (g.steps + KS - 1) / KS;
  const int s0 = min(g.steps, kq * per), s1 = min(g.steps, s0 + per);
  const int nsw = s1 - s0;                          // k-steps of this wave per slot
  const int nmine = nv > sg ? (nv - sg + SG - 1) / SG : 0;  // slots of this wave
  const int n = nmine * nsw;                        // (slot, k-step) items, slot-major
  const size_t ebytes = size_t(g.tiles) * g.steps * T::FRAG;
  const int kblocks = g.K / 128;
  // this wave's slots in registers, lane q holding its q-th: slot, expert,
  // padded row (read back per item with a scalar readlane)
  const int q_slot = lane < nmine ? nth_slot(sg + SG * lane) : 0;
  const int q_exp = __shfl(my_e, q_slot, 64);
  const int q_row = lane < nmine ? rows[q_slot] : 0;

  struct Item {
    u32x4 a[T::AV];
    u32x4 b[T::BV];
    float bs, ws;
    f32x4 ws4;
    int bsc, wsc4;
  };
  auto load = [&](Item& it, int i) {
    const int qi = i / nsw, s = s0 + i % nsw;
    const int e = __builtin_amdgcn_readlane(q_exp, qi), m = __builtin_amdgcn_readlane(q_row, qi);
    const uint8_t* wp = g.w + size_t(e) * ebytes + (size_t(tile) * g.steps + s) * T::FRAG +
                        lane * 16;
#pragma unroll
    for (int v = 0; v < T::AV; ++v) it.a[v] = ld16_stream(wp + v * 1024);
    const uint8_t* bp = g.b + (size_t(m) * g.K + grp * BRUN) * T::EB + size_t(s) * T::KSTEP * T::EB;
#pragma unroll
    for (int v = 0; v < T::BV; ++v) it.b[v] = ld16(bp + v * BHALF);
    if (Q == MOE_QUANT_FP8_BLOCK) {
      it.bs = g.b_scale[size_t(m) * kblocks + s];
      it.ws = g.w_scale[(size_t(e) * (g.N / 128) + tile / 8) * kblocks + s];
    }
    if (Q == MOE_QUANT_W4A8)
      it.ws4 = *reinterpret_cast<const f32x4*>(
          g.w_scale + ((size_t(e) * g.tiles + tile) * g.steps + s) * 16 + grp * 4);
    if (MX) {
      it.bsc = g.b_sc8[size_t(m) * (g.K / 32) + s * 4 + grp];
      it.wsc4 = *reinterpret_cast<const int*>(
          g.w_sc8 + (((size_t(e) * (g.tiles / 4) + tile / 4) * g.steps + s) * 64 + lane) * 4);
    }
  };
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Item& it) {
    if (Q == MOE_QUANT_BF16) {
      acc = mfma_bf16(it.a[0], it.b[0], acc);
    } else if (MX) {
      const i32x8 bb = fp8_pair(it.b[0], it.b[1]);
      acc = mfma_mx_sel<kMxWFmt<Q>, 0>(mx_weight_operand<Q>(it.a[0], it.a[T::AV - 1]), bb, acc,
                                       it.wsc4, tile % 4, it.bsc);
    } else {
      const i32x8 bb = fp8_pair(it.b[0], it.b[1]);
      if (Q == MOE_QUANT_FP8_TENSOR) {
        acc = mfma_fp8(fp8_pair(it.a[0], it.a[1]), bb, acc);
      } else if (Q == MOE_QUANT_FP8_BLOCK) {
        const f32x4 p = mfma_fp8(fp8_pair(it.a[0], it.a[1]), bb, f32x4{0.f, 0.f, 0.f, 0.f});
        const float sc = it.bs * it.ws;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(p[i], sc, acc[i]);
      } else {
        const f32x4 p = mfma_fp8(int4x32_to_e4m3(it.a[0]), bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(p[i], it.ws4[i], acc[i]);
      }
    }
  };
  // the item ring: D items in flight; a slot's partial sum goes to the LDS
  // after its last k-step
  Item st[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < n) load(st[d], d);
  for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      if (i < n) {
        compute(st[d]);
        if (i + D < n) load(st[d], i + D);
        if ((i + 1) % nsw == 0) {
          if ((lane & 15) == 0) red[kq][__builtin_amdgcn_readlane(q_slot, i / nsw)][grp] = acc;
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  if (nsw == 0)
    for (int q = 0; q < nmine; ++q) {
      const int j = __builtin_amdgcn_readlane(q_slot, q);
      if ((lane & 15) == 0) red[kq][j][grp] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  __syncthreads();
  // ---- each valid slot's row, one wave per slot (the lanes holding column
  // 0): K-split partial sums in quarter order, routing weight, rounded as
  // GEMM2 stores it (bf16 for int4 weights, 24 bits otherwise) -- the
  // product kept apart from any sum so that no fused multiply-add changes
  // the rounding
  const bool col0 = (lane & 15) == 0;
  for (int q = wave; q < nv; q += KS * SG) {  // uniform per wave
    const int j = nth_slot(q);
    const int e = __shfl(my_e, j, 64);
    float alpha = 1.f;
    if (Q == MOE_QUANT_FP8_TENSOR) alpha = g.w_scale[e] * *g.a2;
    if (Q == MOE_QUANT_W4A8) alpha = *g.a2;
    const float wgt = alpha * slot_wgt[j];
    if (col0) {
      f32x4 a = red[0][j][grp];
#pragma unroll
      for (int k = 1; k < KS; ++k) a += red[k][j][grp];
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = row_round<Q>(__fmul_rn(a[i], wgt));
      rowv[q][grp] = r;
    }
  }
  __syncthreads();
  // ---- the slot-order sum (wave 0), rounded once to bf16
  if (wave == 0) {
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    if (col0)
      for (int q = 0; q < nv; ++q) {
        const f32x4 r = rowv[q][grp];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] = __fadd_rn(sum[i], r[i]);
      }
    if (col0) {
      u32x2 o;
      o[0] = bf16_bits(sum[0]) | (bf16_bits(sum[1]) << 16);
      o[1] = bf16_bits(sum[2]) | (bf16_bits(sum[3]) << 16);
      *reinterpret_cast<u32x2*>(out + size_t(t) * g.H + tile * 16 + grp * 4) = o;
    }
  }
}

namespace {

template <int PHASE, int Q, int ACT>
hipError_t dispatch_stream(const GemmCfg& c, dim3 grid, const GemmArgs& a, hipStream_t st) {
  const dim3 block(256);
  if constexpr (PHASE == 1 && Q == MOE_QUANT_FP8_BLOCK) {
    // the per-128-channel amax needs the whole workgroup on one row range
    if (c.wt == 4 && c.ksplit == 1) gemm_stream<PHASE, Q, ACT, 4, 1><<<grid, block, 0, st>>>(a);
    else return hipErrorInvalidValue;
  } else if constexpr (kMx<Q>) {
    // a wave's 4 tiles hold whole 32-channel scale blocks of GEMM1's output
    if (c.wt == 4 && c.ksplit == 4) gemm_stream<PHASE, Q, ACT, 4, 4><<<grid, block, 0, st>>>(a);
    else if (c.wt == 4 && c.ksplit == 2) gemm_stream<PHASE, Q, ACT, 4, 2><<<grid, block, 0, st>>>(a);
    else if (c.wt == 4 && c.ksplit == 1) gemm_stream<PHASE, Q, ACT, 4, 1><<<grid, block, 0, st>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (c.wt == 4 && c.ksplit == 1) gemm_stream<PHASE, Q, ACT, 4, 1><<<grid, block, 0, st>>>(a);
    else if (c.wt == 4 && c.ksplit == 2) gemm_stream<PHASE, Q, ACT, 4, 2><<<grid, block, 0, st>>>(a);
    else if (c.wt == 4 && c.ksplit == 4) gemm_stream<PHASE, Q, ACT, 4, 4><<<grid, block, 0, st>>>(a);
    else if (c.wt == 2 && c.ksplit == 4) gemm_stream<PHASE, Q, ACT, 2, 4><<<grid, block, 0, st>>>(a);
    else if (c.wt == 2 && c.ksplit == 2) gemm_stream<PHASE, Q, ACT, 2, 2><<<grid, block, 0, st>>>(a);
    else if (c.wt == 2 && c.ksplit == 1) gemm_stream<PHASE, Q, ACT, 2, 1><<<grid, block, 0, st>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int PHASE, int ACT>
hipError_t dispatch_quant(int quant, const GemmCfg& c, dim3 grid, const GemmArgs& a,
                          hipStream_t st) {
  switch (quant) {
    case MOE_QUANT_BF16: return dispatch_stream<PHASE, MOE_QUANT_BF16, ACT>(c, grid, a, st);
    case MOE_QUANT_FP8_TENSOR: return dispatch_stream<PHASE, MOE_QUANT_FP8_TENSOR, ACT>(c, grid, a, st);
    case MOE_QUANT_FP8_BLOCK: return dispatch_stream<PHASE, MOE_QUANT_FP8_BLOCK, ACT>(c, grid, a, st);
    case MOE_QUANT_W4A8: return dispatch_stream<PHASE, MOE_QUANT_W4A8, ACT>(c, grid, a, st);
    case MOE_QUANT_MXFP8: return dispatch_stream<PHASE, MOE_QUANT_MXFP8, ACT>(c, grid, a, st);
    case MOE_QUANT_MXFP4: return dispatch_stream<PHASE, MOE_QUANT_MXFP4, ACT>(c, grid, a, st);
  }
  return hipErrorInvalidValue;
}

dim3 stream_grid(const GemmCfg& c, int tiles, int64_t blocks) {
  const int tpw = (4 / c.ksplit) * c.wt;
  return dim3(unsigned((tiles + tpw - 1) / tpw), unsigned(blocks));
}

}  // namespace

hipError_t launch_gemm1(const moe_problem& p, const Plan& q, const void* x, const void* xs,
                        const moe_weights& w, const int32_t* sorted_ids,
                        const int32_t* block_expert, const int32_t* num_padded, void* a2,
                        void* a2s, hipStream_t stream, const int32_t* slot_ids) {
  if (q.max_blocks == 0) return hipSuccess;
  GemmArgs a{};
  a.E = p.E;
  a.slot_ids = slot_ids;
  a.b = static_cast<const uint8_t*>(x);
  a.b_scale = static_cast<const float*>(xs);
  a.b_sc8 = static_cast<const uint8_t*>(xs);
  a.w = static_cast<const uint8_t*>(w.w13);
  a.w_scale = static_cast<const float*>(w.w13_scale);
  a.w_sc8 = static_cast<const uint8_t*>(w.w13_scale);
  a.a1 = w.a1_scale;
  a.a2 = w.a2_scale;
  a.sorted_ids = sorted_ids;
  a.block_expert = block_expert;
  a.num_padded = num_padded;
  a.out = static_cast<uint8_t*>(a2);
  a.out_scale = static_cast<float*>(a2s);
  a.out_sc8 = static_cast<uint8_t*>(a2s);
  a.K = p.H;
  a.N = q.N1;
  a.I = p.I;
  a.H = p.H;
  a.Kp = q.Kp;
  a.A = int(q.A);
  a.steps = q.ksteps_h;
  a.tiles = q.N1 / 16;
  if (q.g1.kind >= 1) {
    a.slices = (a.tiles + 4 * q.g1.wt - 1) / (4 * q.g1.wt);
    a.nwg = int(q.max_blocks) * a.slices;
    return launch_gemm_tiled(1, p, q.g1, a, stream);
  }
  const dim3 grid = stream_grid(q.g1, a.tiles, q.max_blocks);
  if (p.act == MOE_ACT_GELU_TANH_GATED)
    return dispatch_quant<1, MOE_ACT_GELU_TANH_GATED>(p.quant, q.g1, grid, a, stream);
  if (q.gated) return dispatch_quant<1, MOE_ACT_SILU_GATED>(p.quant, q.g1, grid, a, stream);
  return dispatch_quant<1, MOE_ACT_RELU2>(p.quant, q.g1, grid, a, stream);
}

hipError_t launch_gemm2(const moe_problem& p, const Plan& q, const void* a2, const void* a2s,
                        const moe_weights& w, const int32_t* sorted_ids,
                        const int32_t* block_expert, const int32_t* num_padded,
                        const float* topk_w, float* y, hipStream_t stream) {
  if (q.max_blocks == 0) return hipSuccess;
  GemmArgs a{};
  a.b = static_cast<const uint8_t*>(a2);
  a.b_scale = static_cast<const float*>(a2s);
  a.b_sc8 = static_cast<const uint8_t*>(a2s);
  a.w = static_cast<const uint8_t*>(w.w2);
  a.w_scale = static_cast<const float*>(w.w2_scale);
  a.w_sc8 = static_cast<const uint8_t*>(w.w2_scale);
  a.a1 = w.a1_scale;
  a.a2 = w.a2_scale;
  a.sorted_ids = sorted_ids;
  a.block_expert = block_expert;
  a.num_padded = num_padded;
  a.topk_w = topk_w;
  a.out = reinterpret_cast<uint8_t*>(y);
  a.K = p.I;
  a.N = p.H;
  a.I = p.I;
  a.H = p.H;
  a.Kp = q.Kp;
  a.A = int(q.A);
  a.steps = q.ksteps_i;
  a.tiles = p.H / 16;
  if (q.g2.kind >= 1) {
    a.slices = (a.tiles + 4 * q.g2.wt - 1) / (4 * q.g2.wt);
    a.nwg = int(q.max_blocks) * a.slices;
    return launch_gemm_tiled(2, p, q.g2, a, stream);
  }
  const dim3 grid = stream_grid(q.g2, a.tiles, q.max_blocks);
  return dispatch_quant<2, 0>(p.quant, q.g2, grid, a, stream);
}

hipError_t launch_gemm2_combine_tok(const moe_problem& p, const Plan& q, const void* a2,
                                   const void* a2s, const moe_weights& w,
                                   const int32_t* sorted_ids, const int32_t* num_padded,
                                   const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                                   hipStream_t stream, bool slot_rows) {
  if (p.T == 0) return hipSuccess;
  GemmArgs a{};
  a.E = p.E;
  a.slot_ids = slot_rows ? topk_ids : nullptr;
  a.b = static_cast<const uint8_t*>(a2);
  a.b_scale = static_cast<const float*>(a2s);
  a.b_sc8 = static_cast<const uint8_t*>(a2s);
  a.w = static_cast<const uint8_t*>(w.w2);
  a.w_scale = static_cast<const float*>(w.w2_scale);
  a.w_sc8 = static_cast<const uint8_t*>(w.w2_scale);
  a.a1 = w.a1_scale;
  a.a2 = w.a2_scale;
  a.sorted_ids = sorted_ids;
  a.num_padded = num_padded;
  a.topk_w = topk_w;
  a.K = p.I;
  a.N = p.H;
  a.I = p.I;
  a.H = p.H;
  a.Kp = q.Kp;
  a.A = int(q.A);
  a.steps = q.ksteps_i;
  a.tiles = p.H / 16;
  const dim3 grid(unsigned(a.tiles), unsigned(p.T)), block(1024);
  switch (p.quant) {
    case MOE_QUANT_BF16:
      gemm2_combine_tok<MOE_QUANT_BF16><<<grid, block, 0, stream>>>(a, topk_ids, out, p.E);
      break;
    case MOE_QUANT_FP8_TENSOR:
      gemm2_combine_tok<MOE_QUANT_FP8_TENSOR><<<grid, block, 0, stream>>>(a, topk_ids, out, p.E);
      break;
    case MOE_QUANT_FP8_BLOCK:
      gemm2_combine_tok<MOE_QUANT_FP8_BLOCK><<<grid, block, 0, stream>>>(a, topk_ids, out, p.E);
      break;
    case MOE_QUANT_W4A8:
      gemm2_combine_tok<MOE_QUANT_W4A8><<<grid, block, 0, stream>>>(a, topk_ids, out, p.E);
      break;
    case MOE_QUANT_MXFP8:
      gemm2_combine_tok<MOE_QUANT_MXFP8><<<grid, block, 0, stream>>>(a, topk_ids, out, p.E);
      break;
    case MOE_QUANT_MXFP4:
      gemm2_combine_tok<MOE_QUANT_MXFP4><<<grid, block, 0, stream>>>(a, topk_ids, out, p.E);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const moe_problem& p, const Plan& q, const int32_t* topk_ids,
                          const float* y, uint16_t* out, hipStream_t stream) {
  const int64_t n = int64_t(p.T) * (p.H / 8);
  if (n == 0) return hipSuccess;
  if (rows_bf16(p.quant))
    combine_kernel<2><<<unsigned((n + 255) / 256), 256, 0, stream>>>(topk_ids, y, out, p.T, p.H,
                                                                   q.Kp, p.E);
  else
    combine_kernel<3><<<unsigned((n + 255) / 256), 256, 0, stream>>>(topk_ids, y, out, p.T, p.H,
                                                                   q.Kp, p.E);
  return hipGetLastError();
}

}  // namespace moe
