// moe_forward for callers that cannot allocate device memory: the workspace
// (routing ids and weights, the aligned row order, the quantised tokens, the
// intermediate and GEMM2's per-assignment rows) lives in one fixed array of
// this library on each GPU instead of a caller-provided buffer.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is ever handed to the
// kernels.
#include <mutex>
#include <string>

#include "moe_launch.hpp"

// MOE_NOALLOC_WORKSPACE_BYTES of device memory per GPU the library runs on,
// held until the process ends.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device

// The device address of `scratch` on `dev`, looked up on the first call for
// that device (which must be the current device).
int scratch_on(int dev, void** ptr) {
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return moe::fail(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                        hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_problem* p, const moe_weights* w,
                                   const uint16_t* x, const float* logits, int32_t* topk_ids,
                                   float* topk_w, uint16_t* out, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (q.ws_total > size_t(MOE_NOALLOC_WORKSPACE_BYTES))
    return moe::fail(MOE_ERR_WORKSPACE,
                     "the problem needs " + std::to_string(q.ws_total) +
                         " bytes of workspace; moe_forward_noalloc holds " +
                         std::to_string(size_t(MOE_NOALLOC_WORKSPACE_BYTES)) +
                         " (use moe_forward with a caller workspace)");
  if (p->T == 0) return MOE_OK;
  // the device the work runs on: the stream's, or the current one for the
  // null stream; the lookup needs it current, which it is for the null
  // stream and is checked otherwise
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return moe::fail(MOE_ERR_HIP, "hipGetDevice failed");
  int dev = cur;
  if (stream && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
    return moe::fail(MOE_ERR_HIP, "hipStreamGetDevice failed");
  if (dev != cur)
    return moe::fail(MOE_ERR_INVALID_ARG, "stream belongs to another device than the current one");
  if (dev < 0 || dev >= kMaxDevices)
    return moe::fail(MOE_ERR_UNSUPPORTED, "device index beyond 63");
  void* ws = nullptr;
  if ((st = scratch_on(dev, &ws)) != MOE_OK) return st;
  return moe_forward(p, w, x, logits, topk_ids, topk_w, out, ws,
                     size_t(MOE_NOALLOC_WORKSPACE_BYTES), stream);
}
