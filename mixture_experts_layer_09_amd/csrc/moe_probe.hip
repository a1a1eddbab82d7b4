// Measurement helpers (not part of the layer): the achievable peaks the
// layer's kernels are compared with, measured on the same device and run.
//  * read stream: every byte of a buffer read once with 16-byte non-temporal
//    lane loads, as the decode GEMMs read their weights;
//  * MFMA loop: back-to-back v_mfma_f32_32x32x16_bf16 (measured on gfx950 at
//    about twice the throughput of the 16x16x32 shape) or
//    v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) on register operands,
//    eight independent accumulators per wave, all SIMDs busy.
#include <atomic>

#include <string>

#include "../../include/moe_probe.h"
#include "moe_device.hpp"
#include "moe_gemm_common.hpp"
#include "moe_plan.hpp"

namespace moe {
namespace {

// Grid-stride read of n16 16-byte vectors; each workgroup folds what it read
// into one word so that the loads cannot be dropped.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = int64_t(gridDim.x) * 256 * 4;
  for (int64_t i = int64_t(blockIdx.x) * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * 256;
      v[u] = j < n16 ? __builtin_nontemporal_load(src + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int FP8>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  u32x4 a4 = {uint32_t(lane) * 0x01010101u, 0x3c3c3c3cu, 0x38383838u, uint32_t(lane)};
  float s = 0.f;
  if constexpr (FP8) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x8 a;
    a[0] = int(a4[0]); a[1] = int(a4[1]); a[2] = int(a4[2]); a[3] = int(a4[3]);
    a[4] = int(a4[0]); a[5] = int(a4[1]); a[6] = int(a4[2]); a[7] = int(a4[3]);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = mfma_fp8(a, a, acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
    const bf16x8 a = __builtin_bit_cast(bf16x8, a4);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][15];
  }
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// One matrix-core instruction on one wave: D = A.B + C on a 16 x 16 tile
// with the lane layouts of include/moe_probe.h (fmt 0 bf16, fmt 1 e4m3 with
// the E8M0 scale codes of each lane).
template <int FMT>
__global__ __launch_bounds__(64) void probe_mfma_tile_kernel(const uint8_t* __restrict__ a,
                                                             const uint8_t* __restrict__ b,
                                                             const uint8_t* __restrict__ sa,
                                                             const uint8_t* __restrict__ sb,
                                                             const float* __restrict__ c,
                                                             float* __restrict__ d) {
  const int l = threadIdx.x;
  const f32x4 cc = *reinterpret_cast<const f32x4*>(c + l * 4);
  f32x4 r;
  if constexpr (FMT == 0) {
    const u32x4 av = *reinterpret_cast<const u32x4*>(a + l * 16);
    const u32x4 bv = *reinterpret_cast<const u32x4*>(b + l * 16);
    r = mfma_bf16(av, bv, cc);
  } else {
    const u32x4* ap = reinterpret_cast<const u32x4*>(a + l * 32);
    const u32x4* bp = reinterpret_cast<const u32x4*>(b + l * 32);
    const int sav = sa ? int(sa[l]) : 127, sbv = sb ? int(sb[l]) : 127;
    r = mfma_mx<0, 0>(fp8_pair(ap[0], ap[1]), fp8_pair(bp[0], bp[1]), cc, sav, sbv);
  }
  *reinterpret_cast<f32x4*>(d + l * 4) = r;
}

int cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v < 1)
      v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace
}  // namespace moe

extern "C" {

int32_t moe_probe_read_blocks(void) { return moe::cu_count() * 8; }

int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, moe_stream_t stream) {
  moe::clear_error();
  if (!buf || !sink || bytes % 16 != 0)
    return moe::fail(MOE_ERR_INVALID_ARG, "moe_probe_read: null pointer or bytes not a multiple of 16");
  (void)hipGetLastError();
  moe::probe_read_kernel<<<moe::cu_count() * 8, 256, 0, (hipStream_t)stream>>>(
      static_cast<const moe::u32x4*>(buf), int64_t(bytes / 16), sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe::fail(MOE_ERR_HIP, std::string("moe_probe_read: ") + hipGetErrorString(e));
  return MOE_OK;
}

int32_t moe_probe_mfma_blocks(void) { return moe::cu_count() * 4; }

int64_t moe_probe_mfma_flops(int32_t dtype, int32_t iters) {
  const int64_t per = dtype == 1 ? 16 * 16 * 128 * 2 : 32 * 32 * 16 * 2;
  return int64_t(moe::cu_count()) * 4 * 4 * 8 * int64_t(iters) * per;
}

int moe_probe_mfma(int32_t dtype, int32_t iters, float* sink, moe_stream_t stream) {
  moe::clear_error();
  if ((dtype != 0 && dtype != 1) || iters < 1 || !sink)
    return moe::fail(MOE_ERR_INVALID_ARG, "moe_probe_mfma: dtype 0 or 1, iters >= 1, sink");
  (void)hipGetLastError();
  const dim3 grid(unsigned(moe::cu_count() * 4)), block(256);
  if (dtype == 1) moe::probe_mfma_kernel<1><<<grid, block, 0, (hipStream_t)stream>>>(iters, sink);
  else moe::probe_mfma_kernel<0><<<grid, block, 0, (hipStream_t)stream>>>(iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe::fail(MOE_ERR_HIP, std::string("moe_probe_mfma: ") + hipGetErrorString(e));
  return MOE_OK;
}

int moe_probe_mfma_tile(int32_t fmt, const void* a, const void* b, const uint8_t* sa,
                        const uint8_t* sb, const float* c, float* d, moe_stream_t stream) {
  moe::clear_error();
  if ((fmt != 0 && fmt != 1) || !a || !b || !c || !d)
    return moe::fail(MOE_ERR_INVALID_ARG, "moe_probe_mfma_tile: fmt 0 or 1, a, b, c, d");
  (void)hipGetLastError();
  const auto* ab = static_cast<const uint8_t*>(a);
  const auto* bb = static_cast<const uint8_t*>(b);
  if (fmt == 0)
    moe::probe_mfma_tile_kernel<0><<<1, 64, 0, (hipStream_t)stream>>>(ab, bb, sa, sb, c, d);
  else
    moe::probe_mfma_tile_kernel<1><<<1, 64, 0, (hipStream_t)stream>>>(ab, bb, sa, sb, c, d);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return moe::fail(MOE_ERR_HIP, std::string("moe_probe_mfma_tile: ") + hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"
