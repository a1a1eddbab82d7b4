// Grouped expert GEMMs for prefill-sized batches (many tokens per expert).
//
// Same operation as the weight-streaming kernels in moe_gemm.hip -- GEMM1
// with the gated (SiLU or GELU_tanh of the gate, times up) or relu^2 epilogue
// on the 16-row gate/up interleave (sglang PR 32944 page, sections 1-3;
// flashinfer PR 4329 page, sections 1-3), GEMM2 with the routing weight --
// tiled for reuse:
//  * a workgroup of 4 waves takes one aligned block of BM = 16*NT token rows
//    of one expert and a slice of 4*WT*16 weight rows; each wave owns WT
//    16-row weight tiles (gate/up pairs for gated GEMM1) against all NT
//    token tiles, so every weight fragment feeds NT MFMAs and every token
//    fragment 4*WT;
//  * token rows are staged through LDS in stages of 128 K, double buffered,
//    rows padded by 16 bytes so the 16 lanes reading one fragment column hit
//    distinct banks; the weight fragments of the next stage are loaded into
//    registers while the current stage computes;
//  * token tiles holding only padding rows are skipped, so the padding of an
//    expert's last block costs at most 15 rows of MFMA work;
//  * workgroup h runs on XCD h % 8; each XCD walks a contiguous range of
//    (block, slice) pairs, slices innermost, so the blocks of one expert --
//    which share weights -- and the slices of one block -- which share token
//    rows -- meet in the same L2.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "moe_device.hpp"
#include "moe_gemm_common.hpp"
#include "moe_launch.hpp"
#include "moe_tile_common.hpp"

namespace moe {

template <int PHASE, int Q, int ACT, int WT, int NT>
__global__ __launch_bounds__(256, 1) void gemm_tiled(GemmArgs g) {
  using T = QT<Q>;
  constexpr int BM = NT * 16;
  constexpr int KST = 128;                  // K elements per stage
  constexpr int SUB = KST / T::KSTEP;       // MFMA k-steps per stage
  constexpr int ROWB = KST * T::EB;         // B bytes per row per stage
  constexpr int LROW = ROWB + 16;           // LDS row stride
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  constexpr int PIECES = BM * CPR / 256;    // chunks per thread per stage
  constexpr bool GATED = PHASE == 1 && act_gated(ACT);
  constexpr int TPW = 4 * WT;               // row tiles per workgroup
  static_assert(PIECES >= 1 && BM * CPR % 256 == 0, "stage does not split over the threads");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * LROW];
  __shared__ float lds_bs[2][Q == MOE_QUANT_FP8_BLOCK ? BM : 1];
  __shared__ float lds_amax[4][PHASE == 1 && Q == MOE_QUANT_FP8_BLOCK ? BM : 1];

  int L;
  if (!xcd_tile(g, BM, L)) return;  // uniform: no real block for this workgroup
  const int blk = L / g.slices, slice = L % g.slices;
  const int row0 = blk * BM;
  const int e = g.block_expert[blk];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4;
  const int mylane_row = lane & 15;

  // the real rows of a block come first; count them
  const int f_mine = tid < BM ? g.sorted_ids[row0 + tid] : g.A;
  const int nvalid = __syncthreads_count(tid < BM && f_mine < g.A);
  const int ct = (nvalid + 15) >> 4;        // token tiles with real rows
  const int tile0 = slice * TPW + wave * WT;
  const bool active = tile0 < g.tiles;      // tiles is a multiple of WT

  // B rows staged by this thread (offsets in bytes from g.b)
  uint32_t bofs[PIECES];
  uint32_t lofs[PIECES];
  bool bon[PIECES];
#pragma unroll
  for (int j = 0; j < PIECES; ++j) {
    const int p = tid + 256 * j;
    const int r = p / CPR, c16 = p % CPR;
    int brow;
    if (PHASE == 1) {
      const int f = g.sorted_ids[row0 + r];
      brow = f < g.A ? f / g.Kp : 0;
    } else {
      brow = r < nvalid ? row0 + r : row0;
    }
    bofs[j] = uint32_t(brow) * uint32_t(g.K * T::EB) + c16 * 16;
    lofs[j] = r * LROW + c16 * 16;
    bon[j] = r < ct * 16;
  }
  // FP8_BLOCK: the B row scale of row `tid` per stage
  int bs_row = 0;
  if (Q == MOE_QUANT_FP8_BLOCK && tid < BM)
    bs_row = PHASE == 1 ? (f_mine < g.A ? f_mine / g.Kp : 0) : (tid < nvalid ? row0 + tid : row0);
  const int kblocks = g.K / 128;

  const size_t ebytes = size_t(g.tiles) * g.steps * T::FRAG;
  const uint8_t* wp = g.w + size_t(e) * ebytes + size_t(tile0) * g.steps * T::FRAG + lane * 16;
  const int nst = g.K / KST;

  u32x4 areg[2][WT][SUB][T::AV];
  u32x4 breg[PIECES];
  float bsreg = 0.f;
  float wsreg[2][WT];
  f32x4 ws4reg[2][WT];
  f32x4 acc[WT][NT];
#pragma unroll
  for (int r = 0; r < WT; ++r)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](auto bufc, int st) {
    constexpr int B = decltype(bufc)::value;
#pragma unroll
    for (int r = 0; r < WT; ++r) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const uint8_t* p = wp + (size_t(r) * g.steps + st * SUB + u) * T::FRAG;
#pragma unroll
        for (int v = 0; v < T::AV; ++v) areg[B][r][u][v] = ld16_stream(p + v * 1024);
      }
      if (Q == MOE_QUANT_FP8_BLOCK) {
        const int rb = PHASE == 1 ? w13_row_block(tile0 + r, g.I, GATED) : (tile0 + r) / 8;
        wsreg[B][r] = g.w_scale[(size_t(e) * (g.N / 128) + rb) * kblocks + st];
      }
      if (Q == MOE_QUANT_W4A8)
        ws4reg[B][r] = *reinterpret_cast<const f32x4*>(
            g.w_scale + ((size_t(e) * g.tiles + tile0 + r) * g.steps + st) * 16 + grp * 4);
    }
  };
  auto load_b = [&](int st) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
      if (bon[j]) breg[j] = ld16(g.b + bofs[j] + size_t(st) * ROWB);
    if (Q == MOE_QUANT_FP8_BLOCK && tid < BM) bsreg = g.b_scale[size_t(bs_row) * kblocks + st];
  };
  auto store_b = [&](auto bufc) {
    constexpr int B = decltype(bufc)::value;
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
      if (bon[j]) *reinterpret_cast<u32x4*>(&lds[B][lofs[j]]) = breg[j];
    if (Q == MOE_QUANT_FP8_BLOCK && tid < BM) lds_bs[B][tid] = bsreg;
  };
  auto compute = [&](auto bufc) {
    constexpr int B = decltype(bufc)::value;
    i32x8 a8[WT];
    if (Q == MOE_QUANT_W4A8) {
#pragma unroll
      for (int r = 0; r < WT; ++r) a8[r] = int4x32_to_e4m3(areg[B][r][0][0]);
    }
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        if (c < ct) {
          const uint8_t* lp = &lds[B][(c * 16 + mylane_row) * LROW + u * T::KSTEP * T::EB +
                                      grp * (T::KSTEP / 4) * T::EB];
          u32x4 bf[T::BV];
#pragma unroll
          for (int v = 0; v < T::BV; ++v) bf[v] = *reinterpret_cast<const u32x4*>(lp + v * 16);
          if (Q == MOE_QUANT_BF16) {
#pragma unroll
            for (int r = 0; r < WT; ++r) acc[r][c] = mfma_bf16(areg[B][r][u][0], bf[0], acc[r][c]);
          } else {
            const i32x8 bb = fp8_pair(bf[0], bf[1]);
            if (Q == MOE_QUANT_FP8_TENSOR) {
#pragma unroll
              for (int r = 0; r < WT; ++r)
                acc[r][c] = mfma_fp8(fp8_pair(areg[B][r][u][0], areg[B][r][u][1]), bb, acc[r][c]);
            } else if (Q == MOE_QUANT_FP8_BLOCK) {
              const float bs = lds_bs[B][c * 16 + mylane_row];
#pragma unroll
              for (int r = 0; r < WT; ++r) {
                const f32x4 t = mfma_fp8(fp8_pair(areg[B][r][u][0], areg[B][r][u][1]), bb,
                                         f32x4{0.f, 0.f, 0.f, 0.f});
                const float sc = bs * wsreg[B][r];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[r][c][i] = fmaf(t[i], sc, acc[r][c][i]);
              }
            } else {
#pragma unroll
              for (int r = 0; r < WT; ++r) {
                const f32x4 t = mfma_fp8(a8[r], bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[r][c][i] = fmaf(t[i], ws4reg[B][r][i], acc[r][c][i]);
              }
            }
          }
        }
      }
    }
  };
  auto stage = [&](auto bufc, int st) {
    constexpr int B = decltype(bufc)::value;
    using Next = std::integral_constant<int, B ^ 1>;
    const bool more = st + 1 < nst;
    if (more) {
      load_b(st + 1);
      if (active) load_a(Next{}, st + 1);
    }
    if (active) compute(bufc);
    if (more) store_b(Next{});
    __syncthreads();
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (active) load_a(B0{}, 0);
  load_b(0);
  store_b(B0{});
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    stage(B0{}, st);
    if (st + 1 < nst) stage(B1{}, st + 1);
  }

  tiled_epilogue<PHASE, Q, ACT, WT, NT>(g, acc, e, row0, ct, tile0, active, lds_amax[0]);
}

// ---------------------------------------------------------------------------
// LDS-pipelined variant for blocks of 128 or more token rows (fp8, W4A8, MX,
// and bf16 where the intermediate size is a multiple of 64).  Weight
// fragments and token rows go from global memory straight into LDS
// (global_load_lds with 16 bytes per lane: lane l's bytes land at
// base + 16 l, which is exactly the lane order of a pre-tiled weight fragment
// and of an MFMA B fragment), so S stages can be in flight without holding
// registers.  A stage covers 128 bytes of K per row: one 128-k step of the
// fp8/fp4 MFMA, or, in bf16, 64 k as two 32-k MFMA steps whose A and B
// halves each lane reads at its own LDS offset.  Per stage a
// workgroup (4 waves, 16 weight row tiles x 8 token tiles) loads 16 weight
// fragments, 8 token fragments and the stage's scales; every wave issues the
// same number of loads, waits for its loads of the oldest stage, then a
// barrier makes all of them visible.  Weight and token fragments are read
// back with lane-contiguous ds_read_b128 (no bank conflicts).

// Workgroup tile of the LDS-staged kernel.  Each of the NWV waves computes
// WT weight tiles x 8 token tiles; the waves stand WR along the weight rows
// and WC along the tokens.  4 waves of 4 tiles, WC = 1: 256 weight rows x
// 128 tokens, three (fp8) or four (int4) stages.  8 waves of 2 tiles,
// WC = 1: the same 256 x 128 with two waves per SIMD (int4, fp8 block
// scales: one wave's conversions and scale FMAs run under the other's
// MFMAs).  8 waves of 4 tiles, WC = 2: 256 x 256, two stages; one wave's
// LDS reads run under the other's MFMAs, and each weight byte serves twice
// the tokens.
template <int Q, int WC, int NWV, int WT = 4, int NW = 8> struct LdsCfg {
  static constexpr int WR = NWV / WC;
  static constexpr int TILES = WT * WR, NT = NW * WC;  // weight / token tiles per workgroup
  // A stage holds 128 bytes of K per row: one fp8 / int4 / MX k-step, two
  // bf16 k-steps (two 1 KiB fragments of each weight tile, contiguous in the
  // packed weights).  SF: a weight tile's bytes per stage, SAV: its 16-byte
  // lane loads.
  static constexpr int SF = Q == MOE_QUANT_BF16 ? 2048 : QT<Q>::FRAG;
  static constexpr int SAV = SF / 1024;
  static constexpr int A_BYTES = TILES * SF;
  static constexpr int B_BYTES = NT * 2048;
  // scales of a stage: fp8 block / int4 group scales in 1 KiB; MX: E8M0
  // weight scales (64 bytes per tile; every wave loads 256 bytes per load
  // round, the rounds' tail past the last tile is not read), then the token
  // rows' (4 bytes per row, 64 rows per wave; the waves past the rows load
  // copies that are not read)
  static constexpr int MXW = kMx<Q> ? (TILES * 64 + NWV * 256 - 1) / (NWV * 256) : 0;
  static constexpr int SC_W8 = MXW * NWV * 256;
  static constexpr int SC_BYTES = (Q == MOE_QUANT_FP8_BLOCK || Q == MOE_QUANT_W4A8) ? 1024
                                  : kMx<Q> ? SC_W8 + NWV * 256 : 0;
  static constexpr int SC_LOADS = kMx<Q> ? MXW + 1 : (SC_BYTES ? 1 : 0);
  static constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  // stages: as many as fit, at most 4
  static constexpr int SMAX = 4;
  static constexpr int S = (160 * 1024 - 4096) / STAGE < SMAX ? (160 * 1024 - 4096) / STAGE : SMAX;
  // loads per wave per stage: weight fragments, token fragments, scales
  static constexpr int LOADS = TILES * SAV / NWV + NT * 2 / NWV + SC_LOADS;
  static_assert(S * STAGE <= 160 * 1024 - 4096, "stage buffers exceed the LDS");
  static_assert(Q != MOE_QUANT_FP8_BLOCK || WC == 1,
                "block scales: one workgroup spans the 128 output channels of a group");
  static_assert(TILES % NWV == 0 && NT % NWV == 0, "whole fragments per wave");
  static_assert(!kMx<Q> || (TILES % 4 == 0 && NT * 16 % 64 == 0 && NT * 16 <= 64 * NWV),
                "MX: whole 4-tile weight-scale loads, the token rows in 64-row loads");
};

// GEMM1 epilogue of the 8-wave fp8 per-tensor tile through the LDS: each
// wave writes its e4m3 outputs (4 channels of one token per lane and MFMA
// tile) into a row-major [token][channel] copy of the workgroup's output
// tile -- rows 0-127 in s0, 128-255 in s1, rows padded by 16 bytes so the 16
// tokens of one store fall in distinct banks -- and the workgroup then
// writes whole rows (256 or 128 bytes) with 16 bytes per lane, instead of
// 16 rows x 16 bytes per store.
template <int ACT, int WT, int NW>
__device__ __forceinline__ void lds_epilogue1(const GemmArgs& g, const f32x4 (&acc)[WT][NW],
                                              int e, int row0, int wr, int wc, int ct,
                                              int ct_all, int wg_tile0, bool active,
                                              uint8_t* s0, uint8_t* s1) {
  constexpr bool GATED = act_gated(ACT);
  constexpr int NV = GATED ? WT / 2 : WT;  // 4-channel vectors per lane and token tile
  constexpr int OC = GATED ? 128 : 256;    // output channels (bytes) of the workgroup tile
  constexpr int OCP = OC + 16;
  const int lane = threadIdx.x & 63, grp = lane >> 4, lrow = lane & 15;
  if (active) {
    const float alpha = g.w_scale[e] * *g.a1;
    const float rs2 = 1.f / *g.a2;
    uint8_t* ob = wc == 0 ? s0 : s1;
#pragma unroll
    for (int c = 0; c < NW; ++c) {
      if (c < ct) {
        uint8_t* orow = ob + (c * 16 + lrow) * OCP + grp * 4;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (GATED) {
              a[i] = gate_act<ACT>(alpha * acc[2 * v][c][i]) * (alpha * acc[2 * v + 1][c][i]);
            } else {
              const float h = fmaxf(alpha * acc[v][c][i], 0.f);
              a[i] = h * h;
            }
          }
          *reinterpret_cast<uint32_t*>(orow + (wr * NV + v) * 16) =
              e4m3x4(a[0] * rs2, a[1] * rs2, a[2] * rs2, a[3] * rs2);
        }
      }
    }
  }
  __syncthreads();
  // whole rows out: the rows of the token tiles holding real rows, the
  // channels of the real weight tiles
  const int col0 = (GATED ? wg_tile0 / 2 : wg_tile0) * 16;
  const int ncols = min(OC, g.I - col0);
  const int nrows = ct_all * 16;
  constexpr int LPR = OC / 16, RPP = 512 / LPR;  // lanes per row, rows per pass
  const int ch = (threadIdx.x % LPR) * 16;
  if (ch < ncols) {
    for (int r = threadIdx.x / LPR; r < nrows; r += RPP) {
      const uint8_t* src = (r < 128 ? s0 : s1) + (r & 127) * OCP + ch;
      *reinterpret_cast<u32x4*>(g.out + size_t(row0 + r) * g.I + col0 + ch) =
          *reinterpret_cast<const u32x4*>(src);
    }
  }
}

template <int PHASE, int Q, int ACT, int WC, int NWV, bool PERSIST, int WT = 4, int NW = 8>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_lds(GemmArgs g) {
  using T = QT<Q>;
  using C = LdsCfg<Q, WC, NWV, WT, NW>;
  // WT x NW: one wave's weight tiles x token tiles; BM: token rows of the workgroup
  constexpr int NT = C::NT, BM = NT * 16, S = C::S, WR = C::WR;
  static_assert(S >= 2, "two stages at least");
  constexpr bool GATED = PHASE == 1 && act_gated(ACT);
  // one array per stage: the compiler then sees that a stage's LDS reads do
  // not alias the LDS-DMA writes into the other stages and does not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s2[S > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s3[S > 3 ? C::STAGE : 16];
  __shared__ float lds_amax[PHASE == 1 && Q == MOE_QUANT_FP8_BLOCK ? NWV * BM : 1];
  auto stage_buf = [&](auto bufc) -> uint8_t* {
    constexpr int B = decltype(bufc)::value;
    if constexpr (B == 0) return lds_s0;
    else if constexpr (B == 1) return lds_s1;
    else if constexpr (B == 2) return lds_s2;
    else return lds_s3;
  };

  // one tile: the BM token rows of block L / slices against 16 * TILES weight rows
  auto tile = [&](const int L) {
    const int blk = L / g.slices, slice = L % g.slices;
    const int row0 = blk * BM;
    const int e = g.block_expert[blk];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4;
    const int lrow = lane & 15;

    // this wave's weight / token group (constants when the waves stand in a row)
    const int wr = WC == 1 ? wave : wave % WR, wc = WC == 1 ? 0 : wave / WR;
    const int f_mine = tid < BM ? g.sorted_ids[row0 + tid] : g.A;
    const int nvalid = __syncthreads_count(tid < BM && f_mine < g.A);
    // token tiles holding rows, counted within this wave's group
    const int ct = min(max(((nvalid + 15) >> 4) - wc * NW, 0), NW);
    const int wg_tile0 = slice * C::TILES;
    const int tile0 = wg_tile0 + wr * WT;
    const bool active = tile0 < g.tiles && ct > 0;
    const int kblocks = g.K / 128;
    const int nst = g.K * T::EB / 128;  // stages of 128 bytes of K per row
    constexpr bool MX = kMx<Q>;
    constexpr int BRUN = MX ? 16 : 32, BHALF = MX ? kMxHalfStride : 16;

    // ---- per-lane source addresses, fixed over the stages
    const size_t ebytes = size_t(g.tiles) * g.steps * T::FRAG;
    const uint8_t* wexp = g.w + size_t(e) * ebytes;
    // weight fragments loaded into LDS by this wave: tiles wave*LA ..
    // wave*LA+LA-1 of the workgroup (clamped to a real tile past the last
    // one, never computed); token tiles wave*LB .. wave*LB+LB-1
    constexpr int LA = C::TILES / NWV, LB = NT / NWV;
    const uint8_t* asrc[LA];
  #pragma unroll
    for (int r = 0; r < LA; ++r) {
      const int t = min(wg_tile0 + wave * LA + r, g.tiles - 1);
      asrc[r] = wexp + size_t(t) * g.steps * T::FRAG + lane * 16;
    }
    // Padding rows (past the block's real rows) read a real row instead of
    // their own: GEMM1 reads token row 0, GEMM2 the block's first row, so
    // their loads hit lines the L1 already holds and bring nothing into L2.
    // Their products are never stored.
    uint32_t bsrc[LB];
  #pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int r = (LB * wave + q) * 16 + lrow;
      int brow;
      if (PHASE == 1) {
        const int f = g.sorted_ids[row0 + r];
        brow = f < g.A ? f / g.Kp : 0;
      } else {
        brow = r < nvalid ? row0 + r : row0;
      }
      bsrc[q] = uint32_t(brow) * uint32_t(g.K * T::EB) + grp * BRUN;
    }
    // scales of a stage: fp8-block token-row scales (waves 1, 2) and weight
    // scales (every other wave, the same values); W4A8 group scales (every
    // wave loads the same)
    const float* ssrc = nullptr;
    int sdst = 0;
    if (Q == MOE_QUANT_FP8_BLOCK) {
      if (wave != 1 && wave != 2) {
        const int t = min(wg_tile0 + (lane & 15), g.tiles - 1);
        const int rb = PHASE == 1 ? w13_row_block(t, g.I, GATED) : t / 8;
        ssrc = g.w_scale + (size_t(e) * (g.N / 128) + rb) * kblocks;
        sdst = 0;
      } else {
        const int r = (wave - 1) * 64 + lane;
        int brow;
        if (PHASE == 1) {
          const int f = g.sorted_ids[row0 + r];
          brow = f < g.A ? f / g.Kp : 0;
        } else {
          brow = r < nvalid ? row0 + r : row0;
        }
        ssrc = g.b_scale + size_t(brow) * kblocks;
        sdst = 256 + (wave - 1) * 256;
      }
    }
    if (Q == MOE_QUANT_W4A8) {
      const int t = min(wg_tile0 + lane / 4, g.tiles - 1);
      ssrc = g.w_scale + (size_t(e) * g.tiles + t) * g.steps * 16 + (lane % 4) * 4;
    }
    // MX: the weight scales of 4-tile group j NWV + wave of the workgroup
    // (lane l: the dword of MFMA lane l, one byte per tile); the token row
    // scales (4 k-blocks, 4 bytes) of row 64 (wave % (BM / 64)) + lane
    constexpr int MXW = C::MXW;           // weight-scale loads per wave
    const uint8_t* mx_wsrc[MXW > 0 ? MXW : 1];
    const uint8_t* mx_tsrc = nullptr;
    if constexpr (MX) {
#pragma unroll
      for (int j = 0; j < MXW; ++j) {
        const int gq = min(wg_tile0 / 4 + j * NWV + wave, g.tiles / 4 - 1);
        mx_wsrc[j] = g.w_sc8 + (size_t(e) * (g.tiles / 4) + gq) * g.steps * 256 + lane * 4;
      }
      const int r = 64 * (wave % (BM / 64)) + lane;
      int brow;
      if (PHASE == 1) {
        const int f = r < BM ? g.sorted_ids[row0 + r] : g.A;
        brow = f < g.A ? f / g.Kp : 0;
      } else {
        brow = r < nvalid ? row0 + r : row0;
      }
      mx_tsrc = g.b_sc8 + size_t(brow) * (g.K / 32);
    }

    auto issue = [&](auto bufc, int st) {
      uint8_t* base = stage_buf(bufc);
  #pragma unroll
      for (int r = 0; r < LA; ++r)
  #pragma unroll
        for (int v = 0; v < C::SAV; ++v)
          ld_lds16(asrc[r] + size_t(st) * C::SF + v * 1024,
                     base + (wave * LA + r) * C::SF + v * 1024);
  #pragma unroll
      for (int q = 0; q < LB; ++q)
  #pragma unroll
        for (int h = 0; h < 2; ++h)
          ld_lds16(g.b + bsrc[q] + size_t(st) * 128 + h * BHALF,
                     base + C::A_BYTES + (LB * wave + q) * 2048 + h * 1024);
      if (Q == MOE_QUANT_FP8_BLOCK) ld_lds4(ssrc + st, base + C::A_BYTES + C::B_BYTES + sdst);
      if (Q == MOE_QUANT_W4A8) ld_lds16(ssrc + size_t(st) * 16, base + C::A_BYTES + C::B_BYTES);
      if constexpr (MX) {
  #pragma unroll
        for (int j = 0; j < MXW; ++j)
          ld_lds4(mx_wsrc[j] + size_t(st) * 256,
                  base + C::A_BYTES + C::B_BYTES + (j * NWV + wave) * 256);
        ld_lds4(mx_tsrc + st * 4, base + C::A_BYTES + C::B_BYTES + C::SC_W8 + wave * 256);
      }
    };

    f32x4 acc[WT][NW];
  #pragma unroll
    for (int r = 0; r < WT; ++r)
  #pragma unroll
      for (int c = 0; c < NW; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // byte offsets of this lane's fragments in a stage.  Every LDS read below
    // indexes the stage array once with a whole offset: a longer chain of
    // pointer steps hides from the compiler which array a read touches, and
    // it then waits for every direct-to-LDS load in flight before the read.
    const int a_off = wr * WT * C::SF + lane * 16;
    const int b_off = C::A_BYTES + wc * NW * 2048 + lane * 16;
    // bf16: a token tile's stage holds, at h * 1024 + 16 L, bytes 32 (L / 16)
    // + 16 h of row L % 16 (the fp8 fragment order); the 16 x 16 x 32 MFMA's
    // lane (g, r) needs, for the stage's k-step j, bytes 64 j + 16 g of row r:
    // L = 16 (2 j + g / 2) + r, h = g % 2
    const int bf_off = C::A_BYTES + wc * NW * 2048 + (grp & 1) * 1024 + (grp >> 1) * 256 + lrow * 16;
    auto rd16 = [](const uint8_t* base, int off) {
      return *reinterpret_cast<const u32x4*>(base + off);
    };
    auto compute = [&](auto bufc) {
      const uint8_t* base = stage_buf(bufc);
      if constexpr (Q == MOE_QUANT_BF16) {
        // two k-steps of 32 per stage, in k order
        u32x4 a2[WT][2];
  #pragma unroll
        for (int r = 0; r < WT; ++r)
  #pragma unroll
          for (int j = 0; j < 2; ++j) a2[r][j] = rd16(base, a_off + r * C::SF + j * 1024);
  #pragma unroll
        for (int c = 0; c < NW; ++c) {
          if (c < ct) {
  #pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u32x4 bb = rd16(base, bf_off + c * 2048 + j * 512);
  #pragma unroll
              for (int r = 0; r < WT; ++r) acc[r][c] = mfma_bf16(a2[r][j], bb, acc[r][c]);
            }
          }
          if constexpr (NW > 8) __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      const float* sc = reinterpret_cast<const float*>(base + C::A_BYTES + C::B_BYTES);
      i32x8 a8[WT];
  #pragma unroll
      for (int r = 0; r < WT; ++r) {
        if constexpr (MX) {
          a8[r] = mx_weight_operand<Q>(rd16(base, a_off + r * C::SF),
                                       rd16(base, a_off + r * C::SF + (T::AV - 1) * 1024));
        } else if (Q == MOE_QUANT_W4A8) {
          a8[r] = int4x32_to_e4m3(rd16(base, a_off + r * C::SF));
        } else {
          a8[r] = fp8_pair(rd16(base, a_off + r * C::SF), rd16(base, a_off + r * C::SF + 1024));
        }
      }
      float ws[WT];
      f32x4 ws4[WT];
      int wsc4 = 0;  // MX: this wave's 4 tiles' weight scales, a byte each
      if constexpr (MX) {
        static_assert(!MX || WT == 4, "MX: a wave's tiles are one 4-tile scale group");
        wsc4 = *reinterpret_cast<const int*>(base + C::A_BYTES + C::B_BYTES + wr * 256 + lane * 4);
      }
      if (Q == MOE_QUANT_FP8_BLOCK) {
  #pragma unroll
        for (int r = 0; r < WT; ++r) ws[r] = sc[wr * WT + r];
      }
      if (Q == MOE_QUANT_W4A8) {
  #pragma unroll
        for (int r = 0; r < WT; ++r)
          ws4[r] = *reinterpret_cast<const f32x4*>(sc + (wr * WT + r) * 16 + grp * 4);
      }
      if constexpr (Q == MOE_QUANT_W4A8 && NW > 8) {
        // 16 token tiles with group scales, software-pipelined: tile c's
        // fragments are read while tile c-1 computes, and tile c's MFMAs are
        // issued before tile c-1's scale FMAs, whose products are ready by
        // then -- neither the LDS read nor the MFMA result is waited for in
        // line.  Products alternate between two register sets.  Every
        // accumulator takes the same FMAs in the same order as in the loop
        // below; tiles past ct are neither multiplied nor folded.  (The same
        // schedule on the fp8 block-scaled 8 x 8 tile measured slower.)
        auto frag = [&](int c) {
          return fp8_pair(rd16(base, b_off + c * 2048), rd16(base, b_off + c * 2048 + 1024));
        };
        i32x8 bb = frag(0);
        f32x4 t2[2][WT];
  #pragma unroll
        for (int c = 0; c <= NW; ++c) {
          // the next tile's fragments (in the stage buffer: read even past ct)
          const i32x8 bn = c + 1 < NW ? frag(c + 1) : bb;
          if (c < NW && c < ct) {
  #pragma unroll
            for (int r = 0; r < WT; ++r)
              t2[c & 1][r] = mfma_fp8(a8[r], bb, f32x4{0.f, 0.f, 0.f, 0.f});
          }
          if (c > 0 && c <= ct) {
  #pragma unroll
            for (int r = 0; r < WT; ++r)
  #pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[r][c - 1][i] = fmaf(t2[(c - 1) & 1][r][i], ws4[r][i], acc[r][c - 1][i]);
          }
          bb = bn;
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
  #pragma unroll
      for (int c = 0; c < NW; ++c) {
        if (c < ct) {
          const i32x8 bb = fp8_pair(rd16(base, b_off + c * 2048), rd16(base, b_off + c * 2048 + 1024));
          if constexpr (MX) {
            // token row c*16 + lrow of this wave's group, k-block grp of the step
            const int bsc = base[C::A_BYTES + C::B_BYTES + C::SC_W8 +
                                 ((wc * NW + c) * 16 + lrow) * 4 + grp];
  #pragma unroll
            for (int r = 0; r < WT; ++r)
              acc[r][c] = mfma_mx_sel<kMxWFmt<Q>, 0>(a8[r], bb, acc[r][c], wsc4, r, bsc);
          } else if (Q == MOE_QUANT_FP8_TENSOR) {
  #pragma unroll
            for (int r = 0; r < WT; ++r) acc[r][c] = mfma_fp8(a8[r], bb, acc[r][c]);
          } else {
            float bs = 1.f;
            if (Q == MOE_QUANT_FP8_BLOCK) bs = sc[64 + c * 16 + lrow];
  #pragma unroll
            for (int r = 0; r < WT; ++r) {
              const f32x4 t = mfma_fp8(a8[r], bb, f32x4{0.f, 0.f, 0.f, 0.f});
              if (Q == MOE_QUANT_FP8_BLOCK) {
                const float s = bs * ws[r];
  #pragma unroll
                for (int i = 0; i < 4; ++i) acc[r][c][i] = fmaf(t[i], s, acc[r][c][i]);
              } else {
  #pragma unroll
                for (int i = 0; i < 4; ++i) acc[r][c][i] = fmaf(t[i], ws4[r][i], acc[r][c][i]);
              }
            }
          }
        }
        // 16 token tiles, or MX on 8 waves: keep the LDS reads of each tile
        // (MX: of each pair of tiles) next to their MFMAs (read all ahead,
        // they and the accumulators do not fit; MX pairs measured 1-2% faster
        // than single tiles, groups of 4 spill)
        if constexpr (NW > 8 || (MX && NWV == 8)) {
          if (NW > 8 || c % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // One pipeline step on buffer B: wait until this wave's loads of stage st
    // have landed (the S-2 newer stages stay in flight), barrier, refill the
    // buffer the previous step freed, compute stage st.  Every step issues
    // exactly one stage of loads -- past the last stage the last one is loaded
    // again and never read -- so the number of loads in flight is the same on
    // every path and the counted wait is exact.
    auto step = [&](auto bufc, int st) {
      constexpr int B = decltype(bufc)::value;
      using Refill = std::integral_constant<int, (B + S - 1) % S>;
      wait_vm_then_barrier<C::LOADS * (S - 2)>();
      issue(Refill{}, min(st + S - 1, nst - 1));
      if (active) compute(bufc);
    };

    // the first S - 1 stages
    issue(std::integral_constant<int, 0>{}, 0);
    if constexpr (S > 2) issue(std::integral_constant<int, 1>{}, min(1, nst - 1));
    if constexpr (S > 3) issue(std::integral_constant<int, 2>{}, min(2, nst - 1));
    // whole rounds of S steps without conditions (a conditional step inside the
    // loop makes the compiler assume any buffer may hold the newest loads and
    // wait for all of them), then the remaining steps
    int st = 0;
    for (; st + S <= nst; st += S) {
      step(std::integral_constant<int, 0>{}, st);
      step(std::integral_constant<int, 1>{}, st + 1);
      if constexpr (S > 2) step(std::integral_constant<int, 2>{}, st + 2);
      if constexpr (S > 3) step(std::integral_constant<int, 3 % S>{}, st + 3);
    }
    if (st < nst) step(std::integral_constant<int, 0>{}, st);
    if (S > 2 && st + 1 < nst) step(std::integral_constant<int, 1 % S>{}, st + 1);
    if (S > 3 && st + 2 < nst) step(std::integral_constant<int, 2 % S>{}, st + 2);
    // drain the surplus loads before the LDS is handed back
    wait_vm_then_barrier<0>();
    if constexpr (NWV == 8 && WC == 2 && PHASE == 1 && Q == MOE_QUANT_FP8_TENSOR) {
      static_assert(Q == MOE_QUANT_FP8_TENSOR && C::STAGE >= 128 * (256 + 16), "8-wave GEMM1 tile");
      lds_epilogue1<ACT, WT, NW>(g, acc, e, row0, wr, wc, ct, (nvalid + 15) >> 4, wg_tile0,
                                 active, lds_s0, lds_s1);
    } else {
      tiled_epilogue<PHASE, Q, ACT, WT, NW>(g, acc, e, row0 + wc * NW * 16, ct, tile0, active,
                                            lds_amax);
    }
  };

  if constexpr (!PERSIST) {
    int L;
    if (!xcd_tile(g, BM, L)) return;  // uniform: no real block for this workgroup
    tile(L);
  } else {
    // Persistent: one workgroup per CU, tiles taken in rounds; in round r
    // the workgroups of XCD x (x = id % 8) take the contiguous tiles
    // (8r + x)·P + j, so the ones sharing an expert's weights and a block's
    // token rows start each round together.  Before each tile the previous
    // tile's stores drain, so the counted waits of the next pipeline see
    // loads only.
    const int nact = min(g.nwg, (*g.num_padded / BM) * g.slices);
    const int P = gridDim.x / 8, x = blockIdx.x % 8, j = blockIdx.x / 8;
    for (int r = 0;; ++r) {
      const int L = (r * 8 + x) * P + j;
      if (L >= nact) break;  // uniform; L grows with r
      if (r > 0) wait_vm_then_barrier<0>();
      tile(L);
    }
  }
}

namespace {

// Workgroups that fit at once when each takes a whole CU, rounded down to a
// multiple of the 8 XCDs (per device, queried once).
int persistent_slots() {
  static std::atomic<int> slots[64];  // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = slots[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    v = cus / 8 * 8;
    slots[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int PHASE, int Q, int ACT>
hipError_t dispatch_tiled(const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  const dim3 grid(unsigned((a.nwg + 7) / 8 * 8)), block(256);
  {
    if (c.kind == 2 || c.kind == 3) {
      // kind 3: one workgroup per CU (the stage buffers take most of the LDS)
      const dim3 pgrid(c.kind == 3 ? std::min<unsigned>(grid.x, unsigned(persistent_slots()))
                                   : grid.x);
      if (c.nt == 8) {
        // int4 and block-scaled weights: 8 waves of 2 weight tiles each, two
        // waves per SIMD, so that one wave's conversions and scale FMAs run
        // under the other's MFMAs
        if constexpr (Q == MOE_QUANT_W4A8 || Q == MOE_QUANT_FP8_BLOCK) {
          if (c.kind == 3) gemm_lds<PHASE, Q, ACT, 1, 8, true, 2><<<pgrid, dim3(512), 0, st>>>(a);
          else gemm_lds<PHASE, Q, ACT, 1, 8, false, 2><<<pgrid, dim3(512), 0, st>>>(a);
          return hipGetLastError();
        }
        if (c.kind == 3) gemm_lds<PHASE, Q, ACT, 1, 4, true><<<pgrid, block, 0, st>>>(a);
        else gemm_lds<PHASE, Q, ACT, 1, 4, false><<<pgrid, block, 0, st>>>(a);
        return hipGetLastError();
      }
      if constexpr (Q == MOE_QUANT_W4A8) {
        // 8 waves of 2 weight tiles x 16 token tiles: 256 x 256, each
        // converted weight fragment feeds 16 MFMAs; one workgroup per tile
        // (the persistent loop's state does not fit beside the pipelined
        // token-tile loop's registers)
        if (c.nt == 16 && c.kind == 2) {
          gemm_lds<PHASE, Q, ACT, 1, 8, false, 2, 16><<<grid, dim3(512), 0, st>>>(a);
          return hipGetLastError();
        }
      }
      if constexpr (Q == MOE_QUANT_FP8_TENSOR || kMx<Q> || Q == MOE_QUANT_BF16) {
        // 8 waves, 256 x 256: one workgroup per tile (the persistent loop's
        // state does not fit the registers of 8 waves of 4 x 8 tiles)
        if (c.nt == 16 && c.kind == 2) {
          gemm_lds<PHASE, Q, ACT, 2, 8, false><<<grid, dim3(512), 0, st>>>(a);
          return hipGetLastError();
        }
      }
      return hipErrorInvalidValue;
    }
  }
  if constexpr (kMx<Q>) {
    return hipErrorInvalidValue;  // MX prefill runs the LDS pipeline only
  } else {
    if (c.nt == 8) gemm_tiled<PHASE, Q, ACT, 4, 8><<<grid, block, 0, st>>>(a);
    else if (c.nt == 4) gemm_tiled<PHASE, Q, ACT, 4, 4><<<grid, block, 0, st>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_gemm_tiled(int phase, const moe_problem& p, const GemmCfg& c,
                             const GemmArgs& a, hipStream_t st) {
#define MOE_TQ(PH, ACT)                                                                      \
  switch (p.quant) {                                                                         \
    case MOE_QUANT_BF16: return dispatch_tiled<PH, MOE_QUANT_BF16, ACT>(c, a, st);           \
    case MOE_QUANT_FP8_TENSOR: return dispatch_tiled<PH, MOE_QUANT_FP8_TENSOR, ACT>(c, a, st); \
    case MOE_QUANT_FP8_BLOCK: return dispatch_tiled<PH, MOE_QUANT_FP8_BLOCK, ACT>(c, a, st); \
    case MOE_QUANT_W4A8: return dispatch_tiled<PH, MOE_QUANT_W4A8, ACT>(c, a, st);           \
    case MOE_QUANT_MXFP8: return dispatch_tiled<PH, MOE_QUANT_MXFP8, ACT>(c, a, st);         \
    case MOE_QUANT_MXFP4: return dispatch_tiled<PH, MOE_QUANT_MXFP4, ACT>(c, a, st);         \
  }
  if (phase == 1) {
    switch (p.act) {
      case MOE_ACT_SILU_GATED: MOE_TQ(1, MOE_ACT_SILU_GATED) break;
      case MOE_ACT_GELU_TANH_GATED: MOE_TQ(1, MOE_ACT_GELU_TANH_GATED) break;
      default: MOE_TQ(1, MOE_ACT_RELU2)
    }
  } else {
    MOE_TQ(2, 0)
  }
#undef MOE_TQ
  return hipErrorInvalidValue;
}

}  // namespace moe
