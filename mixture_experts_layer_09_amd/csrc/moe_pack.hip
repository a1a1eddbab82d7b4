// Load-time weight packing.
//
// The checkpoint layouts (row-major [E][rows][K], K contiguous) become the
// layout the GEMM kernels stream:
//  * gated W13: the optional [Up, Gate] -> [Gate, Up] swap and the zero
//    padding of the intermediate size (sglang PR 21321 page, section 2), then
//    gate and up rows interleaved in groups of 16 -- packed row tile 2p holds
//    gate channels 16p..16p+15 and tile 2p+1 the matching up channels -- so a
//    gate value and its up value land in the same lane and register of two
//    MFMA accumulators (the load-time interleave of the sglang PR 32944 page,
//    section 3, at the granularity of the MFMA tile instead of 1);
//  * every matrix is cut into 16-row x k-step fragments stored in MFMA
//    operand order, so that one wave loads a fragment with contiguous 16-byte
//    lane accesses: fragment (tile t, step s) at ((e*tiles + t)*steps + s),
//    lane l owning row t*16 + l%16 and the k-run at 8 (bf16), 32 (fp8, int4)
//    times l/16;
//      bf16 : 1 KiB fragments, 16 B per lane;
//      fp8  : 2 KiB fragments, lane bytes 0..15 at l*16, 16..31 at 1024 + l*16;
//      int4 : 1 KiB fragments, 16 B per lane; byte b of lane dword q holds
//             k-run element 8q+b in its low nibble and 8q+4+b in its high one;
//      MXFP8: 2 KiB fragments in the scaled MFMA's e4m3 order: lane l
//             (g = l/16) holds k 16g..16g+15 at l*16 and 64+16g..64+16g+15 at
//             1024 + l*16;
//      MXFP4: 1 KiB fragments, lane l holds k 32g..32g+31 as 32 nibbles, the
//             even k in the low nibble (the checkpoint's own nibble order);
//  * block scales (fp8 128x128) keep the checkpoint's row order (the halves
//    swapped when asked); int4 group scales become fp32 in packed row order,
//    [E][tiles][steps][16]; MX E8M0 scales four tiles to a lane dword,
//    [E][tiles/4][steps][64][4]: byte r of lane l's dword in group g is the
//    scale of row (4g + r)*16 + l%16 over k-block 4s + l/16 (lane l feeds it
//    to the scaled MFMA, which picks byte r with its operand select).
#include "moe_device.hpp"
#include "moe_launch.hpp"

namespace moe {

namespace {

struct PackArgs {
  const uint8_t* src;
  uint8_t* dst;
  int E, rows, K;       // packed rows / K of one expert
  int src_rows, src_K;  // checkpoint rows / K of one expert
  int src_I, I;         // unpadded / padded intermediate
  int which;            // 13 or 2
  int gated, swap;
  int steps;            // k-steps per row tile
};

// Checkpoint row of packed row r (W13), or -1 for a zero (padding) row.
__device__ __forceinline__ int w13_src_row(const PackArgs& a, int r) {
  if (!a.gated) return r < a.src_I ? r : -1;
  const int pair = r / 32, within = r % 32;
  const int half = within / 16, c = pair * 16 + within % 16;
  if (c >= a.src_I) return -1;
  const int sh = a.swap ? 1 - half : half;
  return sh * a.src_I + c;
}

// Element `k` of checkpoint row `sr` of expert e as raw bits (bf16: 16 bits,
// fp8: 8 bits, int4 / fp4: the 4-bit nibble), or 0 outside the checkpoint.
template <int FMT>
__device__ __forceinline__ uint32_t src_elem(const PackArgs& a, int e, int sr, int k) {
  if (sr < 0 || k >= a.src_K) return 0;  // zero padding rows / columns
  const size_t idx = (size_t(e) * a.src_rows + sr) * a.src_K + k;
  if (FMT == 0) return reinterpret_cast<const uint16_t*>(a.src)[idx];
  if (FMT == 1 || FMT == 3) return a.src[idx];
  const uint8_t b = a.src[idx / 2];
  return (idx & 1) ? (b >> 4) : (b & 0xF);
}

}  // namespace

// One thread per 16 bytes of packed output.  FMT: 0 bf16, 1 fp8, 2 int4,
// 3 MXFP8, 4 MXFP4.
template <int FMT>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a, int64_t n16) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (c >= n16) return;
  constexpr int frag_chunks = (FMT == 1 || FMT == 3) ? 128 : 64;  // 16-B chunks per fragment
  const int64_t frag = c / frag_chunks;
  const int cf = int(c % frag_chunks);
  const int lane = cf % 64, half = cf / 64;
  const int tiles = a.rows / 16;
  const int e = int(frag / (int64_t(tiles) * a.steps));
  const int rem = int(frag % (int64_t(tiles) * a.steps));
  const int t = rem / a.steps, s = rem % a.steps;
  const int r = t * 16 + lane % 16, g = lane / 16;
  const int sr = a.which == 13 ? w13_src_row(a, r) : r;
  u32x4 out = {0, 0, 0, 0};
  if (FMT == 0) {
    const int k0 = s * 32 + g * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      out[j / 2] |= src_elem<0>(a, e, sr, k0 + j) << (16 * (j & 1));
    }
  } else if (FMT == 1 || FMT == 3) {
    const int k0 = FMT == 1 ? s * 128 + g * 32 + half * 16 : s * 128 + half * 64 + g * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      out[j / 4] |= src_elem<FMT>(a, e, sr, k0 + j) << (8 * (j & 3));
    }
  } else if (FMT == 4) {
    const int k0 = s * 128 + g * 32;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      out[j / 8] |= src_elem<4>(a, e, sr, k0 + j) << (4 * (j & 7));
    }
  } else {
    const int k0 = s * 128 + g * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int klo = k0 + 8 * q + b, khi = klo + 4;
        const uint32_t lo = src_elem<2>(a, e, sr, klo);
        const uint32_t hi = src_elem<2>(a, e, sr, khi);
        out[q] |= (lo | (hi << 4)) << (8 * b);
      }
    }
  }
  *reinterpret_cast<u32x4*>(a.dst + c * 16) = out;
}

// fp8 block scales: W13 rows keep the checkpoint order with the halves
// swapped when asked; W2 is copied.  dst [E][rb][kb].
__global__ void pack_block_scales(const float* __restrict__ src, float* __restrict__ dst, int E,
                                  int rb, int kb, int gated_swap) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = int64_t(E) * rb * kb;
  if (i >= n) return;
  const int k = int(i % kb);
  const int r = int((i / kb) % rb);
  const int e = int(i / (int64_t(kb) * rb));
  int sr = r;
  if (gated_swap) {
    const int hb = rb / 2;
    sr = r < hb ? r + hb : r - hb;
  }
  dst[i] = src[(int64_t(e) * rb + sr) * kb + k];
}

// int4 group scales (bf16 [E][src_rows][K/128]) -> fp32 [E][tiles][steps][16]
// in packed row order.
__global__ void pack_group_scales(PackArgs a, const uint16_t* __restrict__ src,
                                  float* __restrict__ dst, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int rr = int(i % 16);
  const int s = int((i / 16) % a.steps);
  const int64_t et = i / (16 * int64_t(a.steps));
  const int tiles = a.rows / 16;
  const int t = int(et % tiles), e = int(et / tiles);
  const int r = t * 16 + rr;
  const int sr = a.which == 13 ? w13_src_row(a, r) : r;
  float v = 0.f;
  if (sr >= 0) v = bf16_to_f32(src[(size_t(e) * a.src_rows + sr) * (a.src_K / 128) + s]);
  dst[i] = v;
}

// MX E8M0 scales (bytes [E][src_rows][src_K/32]) -> [E][tiles/4][steps][64][4]:
// byte 4l + j of (group g, step s) is the scale of packed row (4g + j)*16 +
// l%16 over k-block 4s + l/16.  Padding rows and columns take 127 (2^0;
// their weights are zero).
__global__ void pack_mx_scales(PackArgs a, const uint8_t* __restrict__ src,
                               uint8_t* __restrict__ dst, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int j = int(i % 4);
  const int l = int((i / 4) % 64);
  const int s = int((i / 256) % a.steps);
  const int64_t eg = i / (256 * int64_t(a.steps));
  const int groups = a.rows / 64;
  const int t = int(eg % groups) * 4 + j, e = int(eg / groups);
  const int r = t * 16 + l % 16, kb = 4 * s + l / 16;
  const int sr = a.which == 13 ? w13_src_row(a, r) : r;
  uint8_t v = 127;
  if (sr >= 0 && kb * 32 < a.src_K) v = src[(size_t(e) * a.src_rows + sr) * (a.src_K / 32) + kb];
  dst[i] = v;
}

hipError_t launch_pack_w(const moe_problem& p, const Plan& q, int which, const void* src,
                         int32_t src_I, int32_t swap, const void* src_scale, void* dst,
                         void* dst_scale, hipStream_t stream) {
  PackArgs a;
  a.src = static_cast<const uint8_t*>(src);
  a.dst = static_cast<uint8_t*>(dst);
  a.E = p.E;
  a.which = which;
  a.gated = q.gated ? 1 : 0;
  a.swap = swap;
  a.src_I = src_I;
  a.I = p.I;
  if (which == 13) {
    a.rows = q.N1;
    a.K = p.H;
    a.src_rows = q.gated ? 2 * src_I : src_I;
    a.src_K = p.H;
  } else {
    a.rows = p.H;
    a.K = p.I;
    a.src_rows = p.H;
    a.src_K = src_I;
  }
  a.steps = a.K / q.kstep;
  const int64_t bytes = int64_t(packed_weight_bytes(p, which));
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const dim3 grid(unsigned((n16 + 255) / 256)), block(256);
  if (p.quant == MOE_QUANT_BF16) pack_kernel<0><<<grid, block, 0, stream>>>(a, n16);
  else if (p.quant == MOE_QUANT_W4A8) pack_kernel<2><<<grid, block, 0, stream>>>(a, n16);
  else if (p.quant == MOE_QUANT_MXFP8) pack_kernel<3><<<grid, block, 0, stream>>>(a, n16);
  else if (p.quant == MOE_QUANT_MXFP4) pack_kernel<4><<<grid, block, 0, stream>>>(a, n16);
  else pack_kernel<1><<<grid, block, 0, stream>>>(a, n16);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (p.quant == MOE_QUANT_FP8_TENSOR) {
    return hipMemcpyAsync(dst_scale, src_scale, size_t(p.E) * 4, hipMemcpyDeviceToDevice, stream);
  }
  if (p.quant == MOE_QUANT_FP8_BLOCK) {
    const int rb = a.rows / 128, kb = a.K / 128;
    const int64_t n = int64_t(p.E) * rb * kb;
    pack_block_scales<<<unsigned((n + 255) / 256), 256, 0, stream>>>(
        static_cast<const float*>(src_scale), static_cast<float*>(dst_scale), p.E, rb, kb,
        which == 13 && q.gated && swap ? 1 : 0);
    return hipGetLastError();
  }
  if (quant_is_mx(p.quant)) {
    const int64_t n = int64_t(p.E) * (a.rows / 16) * a.steps * 64;
    pack_mx_scales<<<unsigned((n + 255) / 256), 256, 0, stream>>>(
        a, static_cast<const uint8_t*>(src_scale), static_cast<uint8_t*>(dst_scale), n);
    return hipGetLastError();
  }
  if (p.quant == MOE_QUANT_W4A8) {
    const int64_t n = int64_t(p.E) * (a.rows / 16) * a.steps * 16;
    pack_group_scales<<<unsigned((n + 255) / 256), 256, 0, stream>>>(
        a, static_cast<const uint16_t*>(src_scale), static_cast<float*>(dst_scale), n);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace moe
