// fp8 (OCP e4m3) quantisation of the hidden states before GEMM1.
//
// Static per-tensor scale (sglang PR 21321 page: the fp8 op's `input_scale`,
// i.e. a1): q = e4m3(sat(x / a1)).  Dynamic per token and 128 columns (the
// 128x128-block fp8 w8a8 mode of the sglang PR 26204 page): s = amax / 448
// (1 for an all-zero group), q = e4m3(x / s).  IEEE fp32 division; e4m3
// rounds to nearest even and saturates at 448.  MXFP8 per token and 32
// columns (the MX modes; OCP MX v1.0): shared exponent X = floor(log2 amax) -
// 8, at least -127, q = e4m3(x / 2^X) (exact scaling), E8M0 byte X + 127.
#include "moe_device.hpp"
#include "moe_launch.hpp"

namespace moe {

// One thread per 8 consecutive elements.
__global__ __launch_bounds__(256) void quant_tensor_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ a1,
                                                           uint8_t* __restrict__ xq, int64_t n8) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const float s = *a1;
  const u32x4 v = ld16(x + i * 8);
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_to_f32(v[k] & 0xFFFFu) / s;
    f[2 * k + 1] = bf16_to_f32(v[k] >> 16) / s;
  }
  u32x2 o;
  o[0] = e4m3x4(f[0], f[1], f[2], f[3]);
  o[1] = e4m3x4(f[4], f[5], f[6], f[7]);
  *reinterpret_cast<u32x2*>(xq + i * 8) = o;
}

// 16 threads per (token, 128-column group), 8 elements each.
__global__ __launch_bounds__(256) void quant_group_kernel(const uint16_t* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          float* __restrict__ xs, int64_t n8) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool in = i < n8;  // n8 is a multiple of 16: whole groups are in or out
  const u32x4 v = in ? ld16(x + i * 8) : u32x4{0, 0, 0, 0};
  float f[8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_to_f32(v[k] & 0xFFFFu);
    f[2 * k + 1] = bf16_to_f32(v[k] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * k]), fabsf(f[2 * k + 1])));
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  if (!in) return;
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = f[k] / s;
  u32x2 o;
  o[0] = e4m3x4(f[0], f[1], f[2], f[3]);
  o[1] = e4m3x4(f[4], f[5], f[6], f[7]);
  *reinterpret_cast<u32x2*>(xq + i * 8) = o;
  if ((threadIdx.x & 15) == 0) xs[i / 16] = s;
}

// 4 threads per (token, 32-column block), 8 elements each.
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ xq,
                                                       uint8_t* __restrict__ xs, int64_t n8) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool in = i < n8;  // n8 is a multiple of 4: whole blocks are in or out
  const u32x4 v = in ? ld16(x + i * 8) : u32x4{0, 0, 0, 0};
  float f[8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_to_f32(v[k] & 0xFFFFu);
    f[2 * k + 1] = bf16_to_f32(v[k] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * k]), fabsf(f[2 * k + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  if (!in) return;
  const int X = mx8_exponent(amax);
  u32x2 o;
  o[0] = mx8x4(f[0], f[1], f[2], f[3], X);
  o[1] = mx8x4(f[4], f[5], f[6], f[7], X);
  *reinterpret_cast<u32x2*>(xq + i * 8) = o;
  if ((threadIdx.x & 3) == 0) xs[i / 4] = uint8_t(X + 127);
}

hipError_t launch_quant_act(const moe_problem& p, const uint16_t* x, const float* a1,
                            uint8_t* xq, void* xs, hipStream_t stream) {
  const int64_t n8 = int64_t(p.T) * p.H / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 grid(unsigned((n8 + 255) / 256)), block(256);
  if (quant_is_mx(p.quant))
    quant_mx_kernel<<<grid, block, 0, stream>>>(x, xq, static_cast<uint8_t*>(xs), n8);
  else if (p.quant == MOE_QUANT_FP8_BLOCK)
    quant_group_kernel<<<grid, block, 0, stream>>>(x, xq, static_cast<float*>(xs), n8);
  else
    quant_tensor_kernel<<<grid, block, 0, stream>>>(x, a1, xq, n8);
  return hipGetLastError();
}

}  // namespace moe
