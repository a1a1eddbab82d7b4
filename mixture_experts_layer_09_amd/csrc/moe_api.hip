// C ABI entry points: validate on the host, then enqueue the kernels.
// The operation each entry point performs is specified in include/moe.h.
#include <algorithm>
#include <string>

#include "moe_launch.hpp"

namespace {

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return moe::fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The runtime's last-error slot is per thread and shared with every other
// HIP user in the process; a launch status read after our launches must not
// pick up an error left there by earlier, unrelated calls.
void clear_stale_launch_error() { (void)hipGetLastError(); }

int null_arg(const char* name) {
  return moe::fail(MOE_ERR_INVALID_ARG, std::string("null pointer: ") + name);
}

bool fp8_static(int quant) {
  return quant == MOE_QUANT_FP8_TENSOR || quant == MOE_QUANT_W4A8;
}

// Modes whose activations carry scales computed on the fly (x_scale, a2_scale).
bool dynamic_scales(int quant) {
  return quant == MOE_QUANT_FP8_BLOCK || moe::quant_is_mx(quant);
}

// Source intermediate sizes the packers take for the mode.
int check_src_I(const moe_problem& p, int32_t src_I) {
  if (src_I < 1 || src_I > p.I) return moe::fail(MOE_ERR_INVALID_ARG, "need 1 <= src_I <= I");
  if ((p.quant == MOE_QUANT_FP8_BLOCK || p.quant == MOE_QUANT_W4A8) && src_I != p.I)
    return moe::fail(MOE_ERR_ALIGNMENT, "block / group scaled weights need src_I == I");
  if (moe::quant_is_mx(p.quant) && src_I % 32 != 0)
    return moe::fail(MOE_ERR_ALIGNMENT, "MX weights need src_I to be a multiple of 32");
  return MOE_OK;
}

// Pointer checks shared by the GEMM entry points.
int check_weights(const moe_problem& p, const moe_weights* w, int which) {
  if (!w) return null_arg("weights");
  if (which == 13 && !w->w13) return null_arg("weights->w13");
  if (which == 2 && !w->w2) return null_arg("weights->w2");
  if (p.quant != MOE_QUANT_BF16) {
    if (which == 13 && !w->w13_scale) return null_arg("weights->w13_scale");
    if (which == 2 && !w->w2_scale) return null_arg("weights->w2_scale");
  }
  if (fp8_static(p.quant)) {
    if (!w->a1_scale && which == 13) return null_arg("weights->a1_scale");
    if (!w->a2_scale) return null_arg("weights->a2_scale");
  }
  return MOE_OK;
}

// One layer pass over p.T tokens with plan q (its workspace layout in ws).
int forward_pass(const moe_problem& p, const moe::Plan& q, const moe_weights& w,
                 const uint16_t* x, const float* logits, int32_t* topk_ids, float* topk_w,
                 uint16_t* out, void* ws, hipStream_t s) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(base + q.off_ids);
  float* wts = topk_w ? topk_w : reinterpret_cast<float*>(base + q.off_w);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + q.off_sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(base + q.off_bexp);
  int32_t* offs = reinterpret_cast<int32_t*>(base + q.off_offsets);
  int32_t* npad = reinterpret_cast<int32_t*>(base + q.off_npad);
  int32_t* scratch = reinterpret_cast<int32_t*>(base + q.off_align);
  uint8_t* xq = base + q.off_xq;
  void* xs = base + q.off_xs;
  void* a2 = base + q.off_a2;
  void* a2s = base + q.off_a2s;
  float* y = reinterpret_cast<float*>(base + q.off_y);
  int st;
  const bool quantise = p.quant != MOE_QUANT_BF16;
  // one token (q.slot_rows): no alignment; GEMM1 takes a block per assignment
  if ((st = hip_status(moe::launch_prologue(p, q, logits, ids, wts, x, w.a1_scale, xq, xs,
                                            quantise, sorted, bexp, offs, npad, scratch, s,
                                            !q.slot_rows),
                       "route/align/quantise")) != MOE_OK)
    return st;
  const void* xin = quantise ? static_cast<const void*>(xq) : static_cast<const void*>(x);
  if ((st = hip_status(moe::launch_gemm1(p, q, xin, xs, w, sorted, bexp, npad, a2, a2s, s,
                                         q.slot_rows ? ids : nullptr),
                       "gemm1")) != MOE_OK)
    return st;
  if (q.g2_tok)
    return hip_status(moe::launch_gemm2_combine_tok(p, q, a2, a2s, w, sorted, npad, ids, wts,
                                                    out, s, q.slot_rows),
                      "gemm2+combine");
  if ((st = hip_status(moe::launch_gemm2(p, q, a2, a2s, w, sorted, bexp, npad, wts, y, s),
                       "gemm2")) != MOE_OK)
    return st;
  return hip_status(moe::launch_combine(p, q, ids, y, out, s), "combine");
}

}  // namespace

extern "C" {

int moe_pack_w13(const moe_problem* p, const void* src, int32_t src_I, int32_t swap_halves,
                 const void* src_scale, void* dst, void* dst_scale, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if ((st = check_src_I(*p, src_I)) != MOE_OK) return st;
  if (swap_halves != 0 && swap_halves != 1)
    return moe::fail(MOE_ERR_INVALID_ARG, "swap_halves must be 0 or 1");
  if (!src) return null_arg("src");
  if (!dst) return null_arg("dst");
  if (p->quant != MOE_QUANT_BF16 && (!src_scale || !dst_scale)) return null_arg("scale");
  clear_stale_launch_error();
  return hip_status(moe::launch_pack_w(*p, q, 13, src, src_I, q.gated ? swap_halves : 0,
                                       src_scale, dst, dst_scale, (hipStream_t)stream),
                    "moe_pack_w13");
}

int moe_pack_w2(const moe_problem* p, const void* src, int32_t src_I, const void* src_scale,
                void* dst, void* dst_scale, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if ((st = check_src_I(*p, src_I)) != MOE_OK) return st;
  if (!src) return null_arg("src");
  if (!dst) return null_arg("dst");
  if (p->quant != MOE_QUANT_BF16 && (!src_scale || !dst_scale)) return null_arg("scale");
  clear_stale_launch_error();
  return hip_status(moe::launch_pack_w(*p, q, 2, src, src_I, 0, src_scale, dst, dst_scale,
                                       (hipStream_t)stream),
                    "moe_pack_w2");
}

int moe_route(const moe_problem* p, const float* logits, int32_t* topk_ids, float* topk_w,
              moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (p->E_routed > moe::kMaxRouted)
    return moe::fail(MOE_ERR_UNSUPPORTED, "moe_route handles at most 1024 routed experts");
  if (p->T == 0) return MOE_OK;
  if (!logits) return null_arg("logits");
  if (!topk_ids) return null_arg("topk_ids");
  if (!topk_w) return null_arg("topk_w");
  clear_stale_launch_error();
  return hip_status(moe::launch_route(*p, logits, topk_ids, topk_w, (hipStream_t)stream),
                    "moe_route");
}

int moe_align(const moe_problem* p, const int32_t* topk_ids, int32_t* sorted_ids,
              int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded, void* ws,
              size_t ws_bytes, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (!expert_offsets) return null_arg("expert_offsets");
  if (!num_padded) return null_arg("num_padded");
  if (q.A > 0) {
    if (!topk_ids) return null_arg("topk_ids");
    if (!sorted_ids) return null_arg("sorted_ids");
    if (!block_expert) return null_arg("block_expert");
  }
  if (q.chunks > 1) {
    if (!ws) return null_arg("ws");
    if (ws_bytes < q.align_ws) return moe::fail(MOE_ERR_WORKSPACE, "align workspace too small");
  }
  clear_stale_launch_error();
  return hip_status(moe::launch_align(*p, q, topk_ids, sorted_ids, block_expert, expert_offsets,
                                      num_padded, static_cast<int32_t*>(ws),
                                      (hipStream_t)stream),
                    "moe_align");
}

int moe_prepare(const moe_problem* p, const float* logits, int32_t* topk_ids, float* topk_w,
                const uint16_t* x, const float* a1_scale, uint8_t* xq, void* x_scale,
                int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                int32_t* num_padded, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (logits && p->E_routed > moe::kMaxRouted)
    return moe::fail(MOE_ERR_UNSUPPORTED, "routing handles at most 1024 routed experts");
  if (!expert_offsets) return null_arg("expert_offsets");
  if (!num_padded) return null_arg("num_padded");
  const bool quantise = x && p->quant != MOE_QUANT_BF16;
  if (q.A > 0) {
    if (!topk_ids) return null_arg("topk_ids");
    if (logits && !topk_w) return null_arg("topk_w");
    if (!sorted_ids) return null_arg("sorted_ids");
    if (!block_expert) return null_arg("block_expert");
    if (quantise) {
      if (!xq) return null_arg("xq");
      if (dynamic_scales(p->quant) && !x_scale) return null_arg("x_scale");
      if (fp8_static(p->quant) && !a1_scale) return null_arg("a1_scale");
    }
  }
  if (q.chunks > 1) {
    if (!ws) return null_arg("ws");
    if (ws_bytes < q.align_ws) return moe::fail(MOE_ERR_WORKSPACE, "align workspace too small");
  }
  clear_stale_launch_error();
  if (q.A == 0)
    return hip_status(moe::launch_align(*p, q, topk_ids, sorted_ids, block_expert,
                                        expert_offsets, num_padded, static_cast<int32_t*>(ws),
                                        (hipStream_t)stream),
                      "moe_prepare");
  return hip_status(moe::launch_prologue(*p, q, logits, topk_ids, topk_w, x, a1_scale, xq,
                                         x_scale, quantise, sorted_ids, block_expert,
                                         expert_offsets, num_padded, static_cast<int32_t*>(ws),
                                         (hipStream_t)stream),
                    "moe_prepare");
}

int moe_quant_act(const moe_problem* p, const uint16_t* x, const float* a1_scale, uint8_t* xq,
                  void* x_scale, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (p->quant == MOE_QUANT_BF16)
    return moe::fail(MOE_ERR_INVALID_ARG, "moe_quant_act applies to the fp8, W4A8 and MX modes");
  if (p->T == 0) return MOE_OK;
  if (!x) return null_arg("x");
  if (!xq) return null_arg("xq");
  if (dynamic_scales(p->quant) && !x_scale) return null_arg("x_scale");
  if (fp8_static(p->quant) && !a1_scale) return null_arg("a1_scale");
  clear_stale_launch_error();
  return hip_status(moe::launch_quant_act(*p, x, a1_scale, xq, x_scale, (hipStream_t)stream),
                    "moe_quant_act");
}

int moe_gemm1_act(const moe_problem* p, const void* x, const void* x_scale,
                  const moe_weights* w, const int32_t* sorted_ids, const int32_t* block_expert,
                  const int32_t* num_padded, void* a2, void* a2_scale, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (q.A == 0) return MOE_OK;
  if ((st = check_weights(*p, w, 13)) != MOE_OK) return st;
  if (!x) return null_arg("x");
  if (!sorted_ids) return null_arg("sorted_ids");
  if (!block_expert) return null_arg("block_expert");
  if (!num_padded) return null_arg("num_padded");
  if (!a2) return null_arg("a2");
  if (dynamic_scales(p->quant)) {
    if (!x_scale) return null_arg("x_scale");
    if (!a2_scale) return null_arg("a2_scale");
  }
  clear_stale_launch_error();
  return hip_status(moe::launch_gemm1(*p, q, x, x_scale, *w, sorted_ids, block_expert,
                                      num_padded, a2, a2_scale, (hipStream_t)stream),
                    "moe_gemm1_act");
}

int moe_gemm2_combine(const moe_problem* p, const void* a2, const void* a2_scale,
                      const moe_weights* w, const int32_t* sorted_ids,
                      const int32_t* block_expert, const int32_t* num_padded,
                      const int32_t* topk_ids, const float* topk_w, void* y_ws,
                      size_t y_ws_bytes, uint16_t* out, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!out) return null_arg("out");
  if (!topk_ids) return null_arg("topk_ids");
  if ((st = check_weights(*p, w, 2)) != MOE_OK) return st;
  if (!a2) return null_arg("a2");
  if (!sorted_ids) return null_arg("sorted_ids");
  if (!block_expert) return null_arg("block_expert");
  if (!num_padded) return null_arg("num_padded");
  if (!topk_w) return null_arg("topk_w");
  if (dynamic_scales(p->quant) && !a2_scale) return null_arg("a2_scale");
  if (!y_ws) return null_arg("y_ws");
  if (y_ws_bytes < q.combine_ws) return moe::fail(MOE_ERR_WORKSPACE, "y workspace too small");
  float* y = static_cast<float*>(y_ws);
  hipStream_t s = (hipStream_t)stream;
  clear_stale_launch_error();
  if (q.g2_tok)
    return hip_status(moe::launch_gemm2_combine_tok(*p, q, a2, a2_scale, *w, sorted_ids,
                                                    num_padded, topk_ids, topk_w, out, s),
                      "moe_gemm2_combine");
  st = hip_status(moe::launch_gemm2(*p, q, a2, a2_scale, *w, sorted_ids, block_expert,
                                    num_padded, topk_w, y, s),
                  "moe_gemm2_combine (gemm)");
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_combine(*p, q, topk_ids, y, out, s), "moe_gemm2_combine (combine)");
}

int moe_forward(const moe_problem* p, const moe_weights* w, const uint16_t* x,
                const float* logits, int32_t* topk_ids, float* topk_w, uint16_t* out, void* ws,
                size_t ws_bytes, moe_stream_t stream) {
  moe::clear_error();
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!x) return null_arg("x");
  if (!out) return null_arg("out");
  if (!ws) return null_arg("ws");
  if (ws_bytes < q.ws_total) return moe::fail(MOE_ERR_WORKSPACE, "workspace too small");
  if ((st = check_weights(*p, w, 13)) != MOE_OK) return st;
  if ((st = check_weights(*p, w, 2)) != MOE_OK) return st;
  if (logits) {
    if (p->E_routed > moe::kMaxRouted)
      return moe::fail(MOE_ERR_UNSUPPORTED, "routing handles at most 1024 routed experts");
  } else if (!topk_ids || !topk_w) {
    return moe::fail(MOE_ERR_INVALID_ARG, "without logits, topk_ids and topk_w are required");
  }
  hipStream_t s = (hipStream_t)stream;
  clear_stale_launch_error();
  if (q.chunk_T >= p->T)
    return forward_pass(*p, q, *w, x, logits, topk_ids, topk_w, out, ws, s);
  // passes over chunk_T tokens each (the stream orders them, so every pass
  // reuses the one workspace); each pass is a layer call of its own
  for (int32_t t0 = 0; t0 < p->T; t0 += q.chunk_T) {
    moe_problem c = *p;
    c.T = std::min(q.chunk_T, p->T - t0);
    moe::Plan qc;
    if ((st = moe::make_plan(&c, &qc)) != MOE_OK) return st;
    if (qc.ws_total > ws_bytes) return moe::fail(MOE_ERR_WORKSPACE, "workspace too small");
    const size_t k0 = size_t(t0) * q.Kp;
    st = forward_pass(c, qc, *w, x + size_t(t0) * p->H,
                      logits ? logits + size_t(t0) * p->E_routed : nullptr,
                      topk_ids ? topk_ids + k0 : nullptr, topk_w ? topk_w + k0 : nullptr,
                      out + size_t(t0) * p->H, ws, s);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // extern "C"
