// Top-k softmax routing.
//
// Per token the k largest router logits are taken in k rounds of a maximum
// over the token's lane group -- larger value first, lower index on equal
// values -- and weighted by a softmax: over the k selected logits with
// renormalisation, over all routed logits otherwise (sglang PR 21321 page,
// section 1: the op's `topk` and `renormalize` arguments).  Shared-expert
// slots follow the routed ones with weight `shared_gate` (sglang PR 26204
// page: the shared expert fused as an extra expert slot).  Selection compares
// logits, which orders experts exactly as their softmax probabilities do.
//
// Each (logit, index) pair becomes one 64-bit key whose unsigned order is the
// selection order: the logit's bits mapped to an order-preserving unsigned
// integer (+0.0 and -0.0 made equal) in the high word, the complemented index
// in the low word.  A round is one 64-bit maximum through DPP lane permutes:
// within a 16-lane row when the token's logits fit 16 lanes (four tokens per
// wave), across the wave otherwise.
#include "moe_device.hpp"
#include "moe_launch.hpp"
#include "moe_route.hpp"

namespace moe {

template <int L, int NPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int Er, int top_k, int n_shared,
                                                    float shared_gate, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts) {
  constexpr int TPW = 64 / L;  // tokens per wave
  const int first = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  if (first >= T) return;  // whole waves leave together
  const int t = first + (threadIdx.x & 63) / L;
  const bool valid = t < T;
  const int tt = valid ? t : 0;
  const int Kp = top_k + n_shared;
  route_token<L, NPL>(logits + size_t(tt) * Er, valid, Er, top_k, n_shared, shared_gate, renorm,
                      ids + size_t(tt) * Kp, wts + size_t(tt) * Kp, nullptr);
}

namespace {
template <int L>
hipError_t route_l(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                   hipStream_t stream) {
  constexpr int TPB = 4 * (64 / L);  // tokens per workgroup
  const dim3 grid((p.T + TPB - 1) / TPB), block(256);
  const int npl = (p.E_routed + L - 1) / L;
#define MOE_ROUTE(N)                                                                          \
  route_kernel<L, N><<<grid, block, 0, stream>>>(logits, p.T, p.E_routed, p.top_k,           \
                                                 p.n_shared, p.shared_gate, p.renormalize,   \
                                                 ids, w)
  if (npl <= 1) MOE_ROUTE(1);
  else if (npl <= 2) MOE_ROUTE(2);
  else if (npl <= 4) MOE_ROUTE(4);
  else if (npl <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}
}  // namespace

bool route_in_rows(const moe_problem& p) {
  return p.E_routed <= 16 * 16 && p.top_k + p.n_shared <= 16;
}

hipError_t launch_route(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                        hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  return route_in_rows(p) ? route_l<16>(p, logits, ids, w, stream)
                          : route_l<64>(p, logits, ids, w, stream);
}

}  // namespace moe
