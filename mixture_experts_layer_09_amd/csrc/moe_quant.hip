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
#include "moe_route.hpp"

namespace moe {

// Each body quantises the 8 consecutive elements of thread i (i in units
// of 8 elements); a kernel's thread i is blockIdx.x * 256 + threadIdx.x, or
// the same counted from the first quantising workgroup of the fused
// routing + quantisation launch below.

// Per tensor: q = e4m3(sat(x / a1)).
__device__ __forceinline__ void quant_tensor_body(int64_t i, const uint16_t* __restrict__ x,
                                                  const float* __restrict__ a1,
                                                  uint8_t* __restrict__ xq, int64_t n8) {
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

// Per token and 128 columns: 16 consecutive threads, 8 elements each.
__device__ __forceinline__ void quant_group_body(int64_t i, const uint16_t* __restrict__ x,
                                                 uint8_t* __restrict__ xq,
                                                 float* __restrict__ xs, int64_t n8) {
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

// MXFP8 per token and 32 columns: 4 consecutive threads, 8 elements each.
__device__ __forceinline__ void quant_mx_body(int64_t i, const uint16_t* __restrict__ x,
                                              uint8_t* __restrict__ xq,
                                              uint8_t* __restrict__ xs, int64_t n8) {
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

__global__ __launch_bounds__(256) void quant_tensor_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ a1,
                                                           uint8_t* __restrict__ xq, int64_t n8) {
  quant_tensor_body(int64_t(blockIdx.x) * 256 + threadIdx.x, x, a1, xq, n8);
}
__global__ __launch_bounds__(256) void quant_group_kernel(const uint16_t* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          float* __restrict__ xs, int64_t n8) {
  quant_group_body(int64_t(blockIdx.x) * 256 + threadIdx.x, x, xq, xs, n8);
}
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ xq,
                                                       uint8_t* __restrict__ xs, int64_t n8) {
  quant_mx_body(int64_t(blockIdx.x) * 256 + threadIdx.x, x, xq, xs, n8);
}

// Routing and quantisation of a prefill-sized batch in one launch: the
// first `route_wgs` workgroups route (as route_kernel: 4 waves, 64 / L
// tokens per wave), the others quantise x (as the kernels above).  The two
// parts share no data; in one launch the routing's vector arithmetic and the
// quantisation's HBM traffic overlap instead of following each other.
struct RouteQuantArgs {
  const float* logits;
  int T, Er, top_k, n_shared, renorm;
  float shared_gate;
  int32_t* ids;
  float* wts;
  const uint16_t* x;
  const float* a1;
  uint8_t* xq;
  void* xs;
  int64_t n8;
  int route_wgs;
};

template <int L, int NPL, int QM>
__global__ __launch_bounds__(256) void route_quant_kernel(RouteQuantArgs a) {
  if (int(blockIdx.x) < a.route_wgs) {
    constexpr int TPW = 64 / L;  // tokens per wave
    const int first = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
    if (first >= a.T) return;  // whole waves leave together
    const int t = first + (threadIdx.x & 63) / L;
    const bool valid = t < a.T;
    const int tt = valid ? t : 0;
    const int Kp = a.top_k + a.n_shared;
    route_token<L, NPL>(a.logits + size_t(tt) * a.Er, valid, a.Er, a.top_k, a.n_shared,
                        a.shared_gate, a.renorm, a.ids + size_t(tt) * Kp, a.wts + size_t(tt) * Kp,
                        nullptr);
    return;
  }
  const int64_t i = int64_t(blockIdx.x - a.route_wgs) * 256 + threadIdx.x;
  if (QM == 1) quant_tensor_body(i, a.x, a.a1, a.xq, a.n8);
  else if (QM == 2) quant_group_body(i, a.x, a.xq, static_cast<float*>(a.xs), a.n8);
  else quant_mx_body(i, a.x, a.xq, static_cast<uint8_t*>(a.xs), a.n8);
}

namespace {
template <int L, int QM>
hipError_t route_quant_lq(const RouteQuantArgs& a0, hipStream_t stream) {
  RouteQuantArgs a = a0;
  constexpr int TPB = 4 * (64 / L);  // tokens per routing workgroup
  a.route_wgs = (a.T + TPB - 1) / TPB;
  const dim3 grid(unsigned(a.route_wgs + (a.n8 + 255) / 256)), block(256);
  const int npl = (a.Er + L - 1) / L;
  if (npl <= 1) route_quant_kernel<L, 1, QM><<<grid, block, 0, stream>>>(a);
  else if (npl <= 2) route_quant_kernel<L, 2, QM><<<grid, block, 0, stream>>>(a);
  else if (npl <= 4) route_quant_kernel<L, 4, QM><<<grid, block, 0, stream>>>(a);
  else if (npl <= 8) route_quant_kernel<L, 8, QM><<<grid, block, 0, stream>>>(a);
  else route_quant_kernel<L, 16, QM><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}
template <int L>
hipError_t route_quant_l(const moe_problem& p, const RouteQuantArgs& a, hipStream_t stream) {
  if (quant_is_mx(p.quant)) return route_quant_lq<L, 3>(a, stream);
  if (p.quant == MOE_QUANT_FP8_BLOCK) return route_quant_lq<L, 2>(a, stream);
  return route_quant_lq<L, 1>(a, stream);
}
}  // namespace

hipError_t launch_route_quant(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                              const uint16_t* x, const float* a1, uint8_t* xq, void* xs,
                              hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  RouteQuantArgs a{};
  a.logits = logits;
  a.T = p.T;
  a.Er = p.E_routed;
  a.top_k = p.top_k;
  a.n_shared = p.n_shared;
  a.renorm = p.renormalize;
  a.shared_gate = p.shared_gate;
  a.ids = ids;
  a.wts = w;
  a.x = x;
  a.a1 = a1;
  a.xq = xq;
  a.xs = xs;
  a.n8 = int64_t(p.T) * p.H / 8;
  return route_in_rows(p) ? route_quant_l<16>(p, a, stream) : route_quant_l<64>(p, a, stream);
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
