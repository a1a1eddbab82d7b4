// Grouped expert GEMMs for prefill-sized batches (many tokens per expert).
//
// Same operation as the weight-streaming kernels in moe_gemm.hip -- GEMM1
// with the SiLU*up / relu^2 epilogue on the 16-row gate/up interleave (sglang
// PR 32944 page, sections 1-3; flashinfer PR 4329 page, section 2), GEMM2
// with the routing weight -- tiled for reuse:
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
#include <type_traits>

#include "moe_device.hpp"
#include "moe_gemm_common.hpp"
#include "moe_launch.hpp"

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
  constexpr bool GATED = PHASE == 1 && ACT == MOE_ACT_SILU_GATED;
  constexpr int TPW = 4 * WT;               // row tiles per workgroup
  static_assert(PIECES >= 1 && BM * CPR % 256 == 0, "stage does not split over the threads");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * LROW];
  __shared__ float lds_bs[2][Q == MOE_QUANT_FP8_BLOCK ? BM : 1];
  __shared__ float lds_amax[4][PHASE == 1 && Q == MOE_QUANT_FP8_BLOCK ? BM : 1];

  const int per = gridDim.x / 8;
  const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= g.nwg) return;
  const int blk = L / g.slices, slice = L % g.slices;
  const int row0 = blk * BM;
  if (row0 >= *g.num_padded) return;  // uniform: past the last real block
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
      brow = row0 + r;
    }
    bofs[j] = uint32_t(brow) * uint32_t(g.K * T::EB) + c16 * 16;
    lofs[j] = r * LROW + c16 * 16;
    bon[j] = r < ct * 16;
  }
  // FP8_BLOCK: the B row scale of row `tid` per stage
  int bs_row = 0;
  if (Q == MOE_QUANT_FP8_BLOCK && tid < BM)
    bs_row = PHASE == 1 ? (f_mine < g.A ? f_mine / g.Kp : 0) : row0 + tid;
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
            a[v][i] = silu(alpha * acc[2 * v][c][i]) * (alpha * acc[2 * v + 1][c][i]);
          } else {
            const float h = fmaxf(alpha * acc[v][c][i], 0.f);
            a[v][i] = h * h;
          }
        }
    };
    if (Q == MOE_QUANT_FP8_BLOCK) {
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
        if (grp == 0) lds_amax[wave][c * 16 + mylane_row] = am;
      }
      __syncthreads();
      if (active) {
        const int w0 = wave - wave % WPG;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c < ct) {
            float gm = 0.f;
#pragma unroll
            for (int w = 0; w < WPG; ++w) gm = fmaxf(gm, lds_amax[w0 + w][c * 16 + mylane_row]);
            const float s = gm > 0.f ? gm / 448.f : 1.f;
            float a[NV][4];
            act(c, a);
            const int m = row0 + c * 16 + mylane_row;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const uint32_t q = e4m3x4(a[v][0] / s, a[v][1] / s, a[v][2] / s, a[v][3] / s);
              *reinterpret_cast<uint32_t*>(g.out + size_t(m) * g.I + cbase[v]) = q;
            }
            if (grp == 0 && wave == w0)
              g.out_scale[size_t(m) * (g.I / 128) + cbase[0] / 128] = s;
          }
        }
      }
    } else if (active) {
      const float s2 = (Q == MOE_QUANT_BF16) ? 1.f : *g.a2;
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
              const uint32_t q = e4m3x4(a[v][0] / s2, a[v][1] / s2, a[v][2] / s2, a[v][3] / s2);
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
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if (c < ct) {
        const int m = row0 + c * 16 + mylane_row;
        const int f = g.sorted_ids[m];
        if (f < g.A) {
          const float wgt = alpha * g.topk_w[f];
#pragma unroll
          for (int r = 0; r < WT; ++r) {
            const int n = (tile0 + r) * 16 + grp * 4;
            *reinterpret_cast<f32x4*>(g.out + (size_t(f) * g.H + n) * 4) = acc[r][c] * wgt;
          }
        }
      }
    }
  }
}

namespace {

template <int PHASE, int Q, int ACT>
hipError_t dispatch_tiled(const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  const dim3 grid(unsigned((a.nwg + 7) / 8 * 8)), block(256);
  if constexpr (Q == MOE_QUANT_FP8_TENSOR) {
    if (c.nt == 16) {
      gemm_tiled<PHASE, Q, ACT, 4, 16><<<grid, block, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  if (c.nt == 8) gemm_tiled<PHASE, Q, ACT, 4, 8><<<grid, block, 0, st>>>(a);
  else if (c.nt == 4) gemm_tiled<PHASE, Q, ACT, 4, 4><<<grid, block, 0, st>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tiled(int phase, const moe_problem& p, const GemmCfg& c,
                             const GemmArgs& a, hipStream_t st) {
  const bool gated = p.act == MOE_ACT_SILU_GATED;
#define MOE_TQ(PH, ACT)                                                                      \
  switch (p.quant) {                                                                         \
    case MOE_QUANT_BF16: return dispatch_tiled<PH, MOE_QUANT_BF16, ACT>(c, a, st);           \
    case MOE_QUANT_FP8_TENSOR: return dispatch_tiled<PH, MOE_QUANT_FP8_TENSOR, ACT>(c, a, st); \
    case MOE_QUANT_FP8_BLOCK: return dispatch_tiled<PH, MOE_QUANT_FP8_BLOCK, ACT>(c, a, st); \
    case MOE_QUANT_W4A8: return dispatch_tiled<PH, MOE_QUANT_W4A8, ACT>(c, a, st);           \
  }
  if (phase == 1) {
    if (gated) {
      MOE_TQ(1, MOE_ACT_SILU_GATED)
    } else {
      MOE_TQ(1, MOE_ACT_RELU2)
    }
  } else {
    MOE_TQ(2, 0)
  }
#undef MOE_TQ
  return hipErrorInvalidValue;
}

}  // namespace moe
