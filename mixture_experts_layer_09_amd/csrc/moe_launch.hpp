// Internal launchers shared by the C-ABI entry points.  Each one enqueues its
// kernels on `stream` and returns the launch status; arguments were validated
// by the caller.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_plan.hpp"

namespace moe {

hipError_t launch_route(const moe_problem& p, const float* logits, int32_t* ids,
                        float* w, hipStream_t stream);

hipError_t launch_align(const moe_problem& p, const Plan& q, const int32_t* ids,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                        int32_t* num_padded, int32_t* scratch, hipStream_t stream);

// Whether the routing runs one token per 16-lane row (else per wave).
bool route_in_rows(const moe_problem& p);

// Whether the decode-size prologue (one workgroup) takes the whole batch.
bool prologue_fits(const moe_problem& p, const Plan& q);

// Routing (when logits is not null; else ids are the caller's), alignment,
// and with `quantise` the fp8 quantisation of x -- one kernel for
// decode-sized batches, the separate kernels otherwise.
// align = false (Plan::slot_rows): routing and quantisation only.
hipError_t launch_prologue(const moe_problem& p, const Plan& q, const float* logits,
                           int32_t* ids, float* w, const uint16_t* x, const float* a1,
                           uint8_t* xq, void* xs, bool quantise, int32_t* sorted_ids,
                           int32_t* block_expert, int32_t* offsets, int32_t* num_padded,
                           int32_t* scratch, hipStream_t stream, bool align = true);

hipError_t launch_quant_act(const moe_problem& p, const uint16_t* x, const float* a1,
                            uint8_t* xq, void* xs, hipStream_t stream);

// launch_route and launch_quant_act as one launch (their workgroups side by
// side), for batches the decode-size prologue does not take.
hipError_t launch_route_quant(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                              const uint16_t* x, const float* a1, uint8_t* xq, void* xs,
                              hipStream_t stream);

hipError_t launch_pack_w(const moe_problem& p, const Plan& q, int which, const void* src,
                         int32_t src_I, int32_t swap, const void* src_scale, void* dst,
                         void* dst_scale, hipStream_t stream);

// slot_ids (Plan::slot_rows): the expert of each assignment, one block per
// assignment instead of sorted_ids / block_expert / num_padded.
hipError_t launch_gemm1(const moe_problem& p, const Plan& q, const void* x, const void* xs,
                        const moe_weights& w, const int32_t* sorted_ids,
                        const int32_t* block_expert, const int32_t* num_padded, void* a2,
                        void* a2s, hipStream_t stream, const int32_t* slot_ids = nullptr);

hipError_t launch_gemm2(const moe_problem& p, const Plan& q, const void* a2, const void* a2s,
                        const moe_weights& w, const int32_t* sorted_ids,
                        const int32_t* block_expert, const int32_t* num_padded,
                        const float* topk_w, float* y, hipStream_t stream);

// GEMM2 and the combine in one launch, token by token (Plan::g2_tok):
// bit-identical to launch_gemm2 followed by launch_combine.
// slot_rows: the intermediate of slot f at row 16 f (GEMM1 run with slot_ids).
hipError_t launch_gemm2_combine_tok(const moe_problem& p, const Plan& q, const void* a2,
                                   const void* a2s, const moe_weights& w,
                                   const int32_t* sorted_ids, const int32_t* num_padded,
                                   const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                                   hipStream_t stream, bool slot_rows = false);

hipError_t launch_combine(const moe_problem& p, const Plan& q, const int32_t* topk_ids,
                          const float* y, uint16_t* out, hipStream_t stream);

}  // namespace moe
