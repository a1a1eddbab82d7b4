// One token's routing by a group of L lanes (L = 16: a DPP row, four tokens
// per wave; L = 64: the whole wave).  Shared by the routing kernel and the
// fused decode prologue kernel.
#pragma once

#include "moe_device.hpp"

namespace moe {

// Unsigned integer with the same order as the float (+0.0 and -0.0 equal).
__device__ __forceinline__ uint32_t float_order_bits(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0.0 + 0.0 = +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Maximum of a 64-bit key over the lane group; every lane of the group gets it.
template <int L>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t k) {
  k = dpp_max_step<kDppXor1, 0xF>(k);
  k = dpp_max_step<kDppXor2, 0xF>(k);
  k = dpp_max_step<kDppHalfMirror, 0xF>(k);
  k = dpp_max_step<kDppMirror, 0xF>(k);
  if (L == 16) return k;
  k = dpp_max_step<kDppBcast15, 0xA>(k);
  k = dpp_max_step<kDppBcast31, 0xC>(k);
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(k), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(k >> 32), 63);
  return (uint64_t(hi) << 32) | lo;
}

// Maximum of a 32-bit value over the lane group; every lane of the group gets
// it.  Lanes a DPP step does not reach read 0 (bound_ctrl), the identity of an
// unsigned maximum, so each step folds into one v_max_u32 with a DPP operand.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xF, true));
  return v > o ? v : o;
}
template <int L>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
  v = dpp_umax<kDppXor1, 0xF>(v);
  v = dpp_umax<kDppXor2, 0xF>(v);
  v = dpp_umax<kDppHalfMirror, 0xF>(v);
  v = dpp_umax<kDppMirror, 0xF>(v);
  if (L == 16) return v;
  v = dpp_umax<kDppBcast15, 0xA>(v);
  v = dpp_umax<kDppBcast31, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Sorts a lane's keys in descending order (bitonic network, N a power of 2).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&k)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size *= 2)
#pragma unroll
    for (int stride = size / 2; stride > 0; stride /= 2)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;  // this half of the sequence descending
          const uint64_t a = k[i], b = k[j];
          const bool swap = desc ? (a < b) : (a > b);
          k[i] = swap ? b : a;
          k[j] = swap ? a : b;
        }
      }
}

// Sum over the lane group; every lane of the group gets it.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if (L == 64) return wave_sum_dpp(v);
  v += __uint_as_float(dpp<kDppXor1, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppXor2, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppHalfMirror, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kDppMirror, 0xF>(0u, __float_as_uint(v)));
  return v;
}

// Routes the token whose Er logits start at `row` (Er <= L * NPL, K' <= L):
// writes K' = top_k + n_shared ids and weights to ids_out / w_out (and the
// ids to lds_ids when it is not null).  Called by all lanes of the group, with
// every lane of the wave active.  `valid` false makes the group compute
// without writing (for the groups past the last token); `row` must still
// point at a real row of Er logits.
template <int L, int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, bool valid, int Er,
                                            int top_k, int n_shared, float shared_gate,
                                            int renorm, int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out, int* lds_ids) {
  const int gl = threadIdx.x & (L - 1);  // lane within the group
  uint64_t key[NPL];
  float v[NPL];
  // All NPL loads are issued before any is used: the index is clamped into
  // the row (every lane, valid or not, reads inside a real row) rather than
  // the load being predicated, which made the compiler wait for each load
  // before issuing the next.
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = gl + L * i;
    v[i] = row[j < Er ? j : Er - 1];
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = gl + L * i;
    const bool in = valid && j < Er;
    if (!in) v[i] = 0.f;
    key[i] = in ? (uint64_t(float_order_bits(v[i])) << 32) | uint32_t(~uint32_t(j)) : 0;
  }
  // Each lane sorts its keys (value's order bits, then the complemented
  // index: larger value first, lower index first on ties); round r takes the
  // largest head over the group -- the value's maximum, then among the lanes
  // holding that value the lowest index -- and the lane holding it drops its
  // head.  The picks come out in the order of the full keys.
  sort_desc<NPL>(key);
  float my_val = 0.f;  // lane r of the group keeps the r-th selected logit
  int my_idx = 0;
  float vmax = 0.f;
  for (int r = 0; r < top_k; ++r) {
    const uint32_t hv = uint32_t(key[0] >> 32), hj = ~uint32_t(key[0]);
    const uint32_t gv = group_umax<L>(hv);
    // lowest index at that value: with the whole wave as the group and one
    // lane holding the value (no tie), that lane's index, read directly
    uint32_t gj;
    if constexpr (L == 64) {
      const uint64_t at = __ballot(hv == gv);
      gj = __popcll(at) == 1 ? uint32_t(__builtin_amdgcn_readlane(int(hj), __builtin_ctzll(at)))
                             : ~group_umax<L>(hv == gv ? ~hj : 0u);
    } else {
      gj = ~group_umax<L>(hv == gv ? ~hj : 0u);
    }
    const int j = int(gj);
    const float val = float_from_order_bits(gv);
    if (hv == gv && hj == gj) {  // this lane held the pick: drop it
#pragma unroll
      for (int i = 0; i + 1 < NPL; ++i) key[i] = key[i + 1];
      key[NPL - 1] = 0;
    }
    if (r == 0) vmax = val;  // the first pick is the largest logit
    if (gl == r) {
      my_val = val;
      my_idx = j;
    }
  }
  float denom;
  if (renorm) {
    denom = group_sum<L>(gl < top_k ? expf(my_val - vmax) : 0.f);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (valid && gl + L * i < Er) s += expf(v[i] - vmax);
    denom = group_sum<L>(s);
  }
  const int Kp = top_k + n_shared;
  if (valid && gl < Kp) {
    int id;
    float wt;
    if (gl < top_k) {
      id = my_idx;
      wt = expf(my_val - vmax) / denom;
    } else {
      id = Er + (gl - top_k);
      wt = shared_gate;
    }
    ids_out[gl] = id;
    w_out[gl] = wt;
    if (lds_ids) lds_ids[gl] = id;
  }
}

}  // namespace moe
