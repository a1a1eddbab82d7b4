// Top-k softmax routing, one wave64 per token.
//
// Per token the k largest router logits are taken in k rounds of a wave-wide
// (value, index) argmax -- larger value first, lower index on equal values --
// and weighted by a softmax: over the k selected logits with renormalisation,
// over all routed logits otherwise (sglang PR 21321 page, section 1: the op's
// `topk` and `renormalize` arguments).  Shared-expert slots follow the routed
// ones with weight `shared_gate` (sglang PR 26204 page: the shared expert
// fused as an extra expert slot).  Selection compares logits, which orders
// experts exactly as their softmax probabilities do.
#include <float.h>
#include <limits.h>

#include "moe_device.hpp"
#include "moe_launch.hpp"

namespace moe {

template <int NPL>  // logits per lane: E_routed <= 64 * NPL
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int Er, int top_k, int n_shared,
                                                    float shared_gate, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave leaves together
  const float* row = logits + size_t(t) * Er;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < Er ? row[j] : -FLT_MAX;
  }
  uint32_t taken = 0;
  float my_val = 0.f;  // lane r keeps the r-th selected logit
  int my_idx = 0;
  for (int r = 0; r < top_k; ++r) {
    float bv = -FLT_MAX;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int j = lane + 64 * i;
      if (j < Er && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && j < bi))) {
        bv = v[i];
        bi = j;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      my_val = bv;
      my_idx = bi;
    }
  }
  const float vmax = __shfl(my_val, 0, 64);  // the first pick is the largest logit
  float denom;
  if (renorm) {
    denom = wave_sum(lane < top_k ? expf(my_val - vmax) : 0.f);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i < Er) s += expf(v[i] - vmax);
    denom = wave_sum(s);
  }
  const int Kp = top_k + n_shared;
  if (lane < top_k) {
    ids[size_t(t) * Kp + lane] = my_idx;
    wts[size_t(t) * Kp + lane] = expf(my_val - vmax) / denom;
  } else if (lane < Kp) {
    ids[size_t(t) * Kp + lane] = Er + (lane - top_k);
    wts[size_t(t) * Kp + lane] = shared_gate;
  }
}

hipError_t launch_route(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                        hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const dim3 grid((p.T + 3) / 4), block(256);
  const int npl = (p.E_routed + 63) / 64;
#define MOE_ROUTE(N)                                                                     \
  route_kernel<N><<<grid, block, 0, stream>>>(logits, p.T, p.E_routed, p.top_k,         \
                                              p.n_shared, p.shared_gate, p.renormalize, \
                                              ids, w)
  if (npl <= 1) MOE_ROUTE(1);
  else if (npl <= 2) MOE_ROUTE(2);
  else if (npl <= 4) MOE_ROUTE(4);
  else if (npl <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
