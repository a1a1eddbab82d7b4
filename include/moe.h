/*
 * moe.h -- C ABI of the fused Mixture-of-Experts forward layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer computes, for T tokens x[t] (bf16, hidden size H):
 *   1. routing   : top-k of the router logits, softmax weights, optional
 *                  renormalisation over the k, shared-expert slots appended
 *                  (moe_route);
 *   2. alignment : the T*K' (token, slot) assignments grouped by expert and
 *                  padded per expert to the GEMM row block (moe_align);
 *   3. GEMM1     : h = W13[e] . x[t] with the activation applied in the
 *                  epilogue -- SiLU(gate) * up or GELU_tanh(gate) * up for
 *                  gated layers, relu(h)^2 for non-gated ones -- storing only
 *                  the I activated columns (moe_gemm1_act);
 *   4. GEMM2     : y = W2[e] . a, multiplied by the routing weight and summed
 *                  back into the token's row (moe_gemm2_combine);
 * and moe_forward runs all of it in one call.
 *
 * Sources of the operation (the method's pages, by page and section):
 *   [TRTLLM]  sglang PR 21321 page, "FlashInfer TRTLLM-Gen MoE kernel
 *             optimisation: NemotronH support": the fused op's arguments
 *             (hidden_states, w13/w2 and their scales, expert_weights, topk,
 *             renormalize, activation_type) and its bf16 output of the input's
 *             shape (section 1); _is_gated, _align_fp8_moe_weights, the
 *             [Up, Gate] -> [Gate, Up] swap, the fp8 scale scalars,
 *             _align_mxfp8_moe_weights (MXFP8 weights with [.., K/32] scales,
 *             padded with them) (section 2).
 *   [GATED]   flashinfer PR 4329 page, "Gated MoE kernels for Blackwell":
 *             gated vs generic kernels chosen by activation, the gated
 *             activations silu and gelu_tanh (sections 1 and 3), gate and up
 *             projections paired in FC1 (section 2), FC2 non-gated, routing
 *             and scatter unchanged (sections 3-4).
 *   [SHARED]  sglang PR 26204 page, "Qwen3-Next FP8 MoE: Shared-Expert
 *             Fusion": fp8 w8a8 with [128, 128] block scales, E = 513 slots
 *             (512 routed + the shared expert), BLOCK_SIZE_M per batch size
 *             (section 1 and "why this is good").
 *   [SWIGLU]  sglang PR 32944 page, "SwiGLU fusion into the MoE up-GEMM
 *             epilogue": the load-time gate/up interleave (section 3), the
 *             epilogue SiLU*up with a half-width store and no full-width
 *             intermediate (sections 1-2).
 *   [W4A8]    sglang PR 38220 page, "W4A8 MoE GEMM for GLM-5.2": int4 weights
 *             with group scales, fp8 activations, per-expert problems from
 *             expert offsets (section 1).
 *
 * Conventions for every entry point:
 *   - Pointers named in a signature are DEVICE pointers unless the comment says
 *     "host".  All buffers are owned by the caller; the library allocates and
 *     frees nothing and keeps no pointer after it returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  The library never synchronises and never changes the
 *     current device.
 *   - Arguments are validated on the host before anything is enqueued: an
 *     invalid call returns a negative moe_status and enqueues nothing.  A launch
 *     failure returns MOE_ERR_HIP.  moe_last_error() gives a detail string for
 *     the last failing call on the calling thread.  Device-side faults surface
 *     at the caller's next synchronisation, as for any HIP kernel.
 *   - Sizes are int32; H and I are at most 2^20 and T*K'*max(H, I) must stay
 *     below 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 *   - Matrices are row-major.  bf16 values travel as uint16_t bit patterns and
 *     fp8 values as uint8_t OCP e4m3fn codes (bias 7, max 448, no infinities);
 *     the MX modes' scales as uint8_t E8M0 codes (2^(c - 127), OCP MX v1.0).
 *   - Calls are reentrant; concurrent calls on different streams must not share
 *     output or workspace buffers.
 *   - The device entry points enqueue kernels only (no allocation, memset,
 *     copy or synchronisation; moe_pack_* with FP8_TENSOR scales aside, which
 *     copies them), so a call can be captured into a HIP graph and replayed.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */

/* Status codes returned by every int-returning entry point. */
enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, enum or pointer is out of its domain  */
  MOE_ERR_UNSUPPORTED = -2, /* a valid combination the library does not run */
  MOE_ERR_ALIGNMENT = -3,   /* H or I breaks the alignment the formats need  */
  MOE_ERR_WORKSPACE = -4,   /* workspace / scratch smaller than required     */
  MOE_ERR_HIP = -5          /* a HIP launch or runtime call failed           */
};

/* Activation of GEMM1 ([TRTLLM] section 1 ActivationType; [GATED] sections 1
   and 3: silu and gelu_tanh among the gated activations). */
enum moe_act {
  MOE_ACT_SILU_GATED = 0,      /* a = SiLU(gate) * up, W13 holds 2I rows     */
  MOE_ACT_RELU2 = 1,           /* a = relu(h)^2, non-gated, W13 holds I rows */
  MOE_ACT_GELU_TANH_GATED = 2  /* a = GELU_tanh(gate) * up, 2I rows, where
                                  GELU_tanh(g) = 0.5 g (1 + tanh(sqrt(2/pi)
                                  (g + 0.044715 g^3)))                       */
};

/* Weight / activation formats. */
enum moe_quant {
  MOE_QUANT_BF16 = 0,       /* bf16 weights and activations                     */
  MOE_QUANT_FP8_TENSOR = 1, /* e4m3 weights, one fp32 scale per expert and
                               matrix; e4m3 activations with static per-tensor
                               scales a1 (x) and a2 (intermediate) [TRTLLM]     */
  MOE_QUANT_FP8_BLOCK = 2,  /* e4m3 weights with one fp32 scale per 128x128
                               block; e4m3 activations with one fp32 scale per
                               token per 128 columns, computed on the fly
                               [SHARED]                                         */
  MOE_QUANT_W4A8 = 3,       /* signed int4 weights with one bf16 scale per row
                               per 128 K; e4m3 activations with static a1, a2
                               [W4A8]                                           */
  MOE_QUANT_MXFP8 = 4,      /* OCP MX: e4m3 weights with one E8M0 scale per row
                               per 32 K ([TRTLLM] section 2,
                               _align_mxfp8_moe_weights: scales [E, N, K/32]);
                               x and the intermediate quantised to MXFP8 on
                               the fly (E8M0 per token per 32 columns)          */
  MOE_QUANT_MXFP4 = 5       /* OCP MX: E2M1 (fp4) weights, two per byte with the
                               even k in the low nibble, one E8M0 scale per row
                               per 32 K; activations MXFP8 as for MOE_QUANT_MXFP8
                               (the 4-bit weights of [TRTLLM] section 3 and
                               [GATED], taken as MXFP4)                         */
};

/* Shape and mode of one layer call. */
typedef struct moe_problem {
  int32_t T;            /* tokens (0 is a valid no-op)                          */
  int32_t H;            /* hidden size; multiple of 128                          */
  int32_t I;            /* intermediate size per expert, already padded to
                           moe_padded_intermediate(I, act, quant)                */
  int32_t E;            /* expert slots = E_routed + n_shared                    */
  int32_t E_routed;     /* routed experts = columns of the router logits        */
  int32_t top_k;        /* routed slots per token, 1 <= top_k <= E_routed        */
  int32_t n_shared;     /* shared-expert slots appended after the routed ones   */
  float shared_gate;    /* routing weight of every shared slot                  */
  int32_t renormalize;  /* 1: weights = softmax over the k selected logits;
                           0: softmax over all routed logits, taken at the k    */
  int32_t act;          /* enum moe_act                                          */
  int32_t quant;        /* enum moe_quant                                        */
  int32_t block_m;      /* alignment block (rows per GEMM tile): 0 = library
                           choice, else 16, 64, 128 or 256 (256: fp8
                           per-tensor, W4A8 and MX modes only; the MX modes
                           run 16, 128 and 256).  Every call of one
                           layer pass must see the same resolved value
                           (moe_block_m).                                        */
} moe_problem;

/* Packed weights (outputs of moe_pack_w13 / moe_pack_w2) and scales. */
typedef struct moe_weights {
  const void* w13;        /* packed up-projection                              */
  const void* w2;         /* packed down-projection                            */
  const void* w13_scale;  /* packed scales (moe_packed_bytes); NULL for bf16   */
  const void* w2_scale;   /* packed scales; NULL for bf16                       */
  const float* a1_scale;  /* [1] static x scale: FP8_TENSOR, W4A8; else NULL   */
  const float* a2_scale;  /* [1] static intermediate scale: FP8_TENSOR, W4A8    */
} moe_weights;

/* ---------------------------------------------------------------- host-only */

/* Human-readable name of a status code (host; static storage). */
const char* moe_status_string(int status);

/* Detail of the last failing call on this thread (host; thread-local storage,
 * valid until the next call on the thread). */
const char* moe_last_error(void);

/* Check a problem without launching anything.  Returns MOE_OK or the error the
 * entry points would return (host). */
int moe_validate(const moe_problem* p);

/* Intermediate size after padding: the TRTLLM-Gen rule ([TRTLLM] section 2,
 * _align_fp8_moe_weights: multiple of 16 gated, 128 non-gated) combined with
 * what the kernels need (bf16 gated: 32; fp8 and int4: 128).  Returns I when
 * already aligned, a negative status for an invalid act/quant (host). */
int32_t moe_padded_intermediate(int32_t I, int32_t act, int32_t quant);

/* Resolved alignment block (rows per GEMM tile) for the problem (host). */
int32_t moe_block_m(const moe_problem* p);

/* Capacity the caller must provide for block-indexed outputs: the largest
 * possible number of blocks and padded rows for the problem (host). */
int64_t moe_max_blocks(const moe_problem* p);
int64_t moe_max_padded_rows(const moe_problem* p);

/* Scratch bytes moe_align needs for the problem (host). */
size_t moe_align_workspace_bytes(const moe_problem* p);

/* Scratch bytes moe_gemm2_combine needs for its per-assignment rows (host). */
size_t moe_combine_workspace_bytes(const moe_problem* p);

/* Workspace bytes moe_forward needs for the problem (host): for more than
 * 65536 assignments, those of one pass of floor(65536 / K') tokens. */
size_t moe_workspace_bytes(const moe_problem* p);

/* Bytes of a packed weight (which = 13 for W13, 2 for W2) and of its packed
 * scales.  Returns a status (host). */
int moe_packed_bytes(const moe_problem* p, int32_t which, size_t* w_bytes,
                     size_t* s_bytes);

/* ---------------------------------------------------------- device launches */

/* Load-time packing of the up-projection ([TRTLLM] section 2 swap/pad/
 * reorder; [SWIGLU] section 3 interleave).
 *   src       : checkpoint layout [E][N1s][H] with N1s = 2*src_I (gated; gate
 *               rows first, or up rows first when swap_halves = 1) or src_I
 *               (non-gated).  Elements: bf16 bits (BF16), e4m3 codes (FP8_*),
 *               or int4 packed two per byte with the even k in the low nibble
 *               ([E][N1s][H/2], W4A8), e4m3 codes (MXFP8), E2M1 codes two per
 *               byte, even k in the low nibble ([E][N1s][H/2], MXFP4).
 *   src_I     : unpadded intermediate size, src_I <= p->I; rows src_I..I-1 of
 *               each half are zero-filled (FP8_BLOCK and W4A8 need src_I == I,
 *               the MX modes a multiple of 32).
 *   src_scale : FP8_TENSOR fp32 [E]; FP8_BLOCK fp32 [E][N1s/128][H/128];
 *               W4A8 bf16 bits [E][N1s][H/128]; MXFP8 / MXFP4 E8M0 bytes
 *               [E][N1s][H/32]; NULL for BF16.
 *   dst       : moe_packed_bytes(p, 13) bytes; gate/up rows interleaved in
 *               groups of 16 and pre-tiled in the MFMA operand order.
 *   dst_scale : the packed scales (moe_packed_bytes(p, 13) scale bytes).
 * dst must not overlap src. */
int moe_pack_w13(const moe_problem* p, const void* src, int32_t src_I,
                 int32_t swap_halves, const void* src_scale, void* dst,
                 void* dst_scale, moe_stream_t stream);

/* Load-time packing of the down-projection: src [E][H][src_I] (int4, fp4:
 * [E][H][src_I/2]), scales FP8_TENSOR [E], FP8_BLOCK [E][H/128][src_I/128],
 * W4A8 bf16 [E][H][src_I/128], MX E8M0 bytes [E][H][src_I/32]; columns
 * src_I..I-1 are zero-filled (the scale padding of [TRTLLM] section 2,
 * _align_mxfp8_moe_weights). */
int moe_pack_w2(const moe_problem* p, const void* src, int32_t src_I,
                const void* src_scale, void* dst, void* dst_scale,
                moe_stream_t stream);

/* Top-k softmax routing ([TRTLLM] section 1: topk, renormalize; [SHARED]:
 * the shared expert as an extra slot).
 *   logits   : fp32 [T][E_routed], finite values.
 *   topk_ids : int32 [T][K'] with K' = top_k + n_shared: the k routed experts
 *              by descending logit (lower index first on equal logits), then
 *              E_routed + s for shared slot s.
 *   topk_w   : fp32 [T][K']: softmax weights (see moe_problem.renormalize),
 *              then shared_gate for the shared slots.
 * Limits: E_routed <= 1024, K' <= 64. */
int moe_route(const moe_problem* p, const float* logits, int32_t* topk_ids,
              float* topk_w, moe_stream_t stream);

/* Sort and align the assignments into per-expert blocks ([SHARED]
 * BLOCK_SIZE_M; [W4A8] expert_offsets / problem sizes).  With A = T*K' and
 * BM = moe_block_m(p):
 *   topk_ids       : int32 [T][K']; ids outside [0, E) are skipped.
 *   sorted_ids     : int32 [moe_max_padded_rows]: per expert, in expert order,
 *                    the flat indices f = t*K'+j with topk_ids[f] == e in
 *                    ascending order, then the sentinel A up to the next
 *                    multiple of BM.  Entries past num_padded are untouched.
 *   block_expert   : int32 [moe_max_blocks]: expert of each block of BM rows.
 *   expert_offsets : int32 [E+1]: exclusive prefix of the padded counts.
 *   num_padded     : int32 [1]: expert_offsets[E].
 *   ws             : moe_align_workspace_bytes(p) bytes of scratch.
 * The result is deterministic and bit-identical to the stable definition. */
int moe_align(const moe_problem* p, const int32_t* topk_ids, int32_t* sorted_ids,
              int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
              void* ws, size_t ws_bytes, moe_stream_t stream);

/* Everything before GEMM1 in one call: moe_route (when logits is not NULL;
 * otherwise topk_ids is the caller's routing, an input), moe_quant_act (when
 * x is not NULL and the mode is fp8 / W4A8 / MX; a1_scale, xq, x_scale as there)
 * and moe_align, with the arguments of those entry points.  Decode-sized
 * batches (T <= 128, T*K' <= 1024) route, align and quantise in one kernel
 * launch (the quantisation in workgroups of their own); larger ones run the
 * separate kernels.  Outputs are bit-identical to the separate calls. */
int moe_prepare(const moe_problem* p, const float* logits, int32_t* topk_ids, float* topk_w,
                const uint16_t* x, const float* a1_scale, uint8_t* xq, void* x_scale,
                int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                int32_t* num_padded, void* ws, size_t ws_bytes, moe_stream_t stream);

/* fp8 activation quantisation of x (bf16 [T][H]) for the fp8, W4A8 and MX modes:
 *   FP8_TENSOR, W4A8 : xq = e4m3(sat(x / a1)), x_scale unused (may be NULL);
 *   FP8_BLOCK        : per token and 128 columns s = amax/448 (1 if amax = 0),
 *                      xq = e4m3(x / s), x_scale fp32 [T][H/128] = s;
 *   MXFP8, MXFP4     : MXFP8 per token and 32 columns (OCP MX v1.0): shared
 *                      exponent X = floor(log2 amax) - 8 in [-127, 127]
 *                      (-127 if amax = 0), xq = e4m3(sat(x / 2^X)), x_scale
 *                      E8M0 bytes [T][H/32] = X + 127.
 * Division is IEEE fp32; e4m3 rounds to nearest even and saturates at 448.
 * a1_scale is a device pointer to one float (FP8_TENSOR, W4A8). */
int moe_quant_act(const moe_problem* p, const uint16_t* x, const float* a1_scale,
                  uint8_t* xq, void* x_scale, moe_stream_t stream);

/* Grouped GEMM1 with the activation in the epilogue ([SWIGLU] sections 1-2;
 * [GATED] section 2).  For every padded row r < *num_padded of block
 * b = r / BM with expert e = block_expert[b] and f = sorted_ids[r]:
 *   h = W13[e] . xin[f / K']  (rows f == A are padding and produce
 *                              unspecified but finite values)
 *   a = SiLU(h_gate) * h_up  or  relu(h)^2, after dequantisation
 *   a2[r][:] = a in the compute format: bf16 (BF16), e4m3(sat(a / a2))
 *   (FP8_TENSOR, W4A8), per 128 columns e4m3(a / s) with s = amax/448
 *   written to a2_scale fp32 [rows][I/128] (FP8_BLOCK), or MXFP8 per 32
 *   columns as in moe_quant_act with the E8M0 bytes in a2_scale [rows][I/32]
 *   (MXFP8, MXFP4).
 *   x       : bf16 [T][H] (BF16) or e4m3 codes [T][H] (moe_quant_act).
 *   x_scale : fp32 [T][H/128] for FP8_BLOCK, E8M0 [T][H/32] for the MX modes,
 *             else ignored.
 *   a2      : [moe_max_padded_rows][I] bf16 or e4m3.
 * The full-width h is never written to memory. */
int moe_gemm1_act(const moe_problem* p, const void* x, const void* x_scale,
                  const moe_weights* w, const int32_t* sorted_ids,
                  const int32_t* block_expert, const int32_t* num_padded,
                  void* a2, void* a2_scale, moe_stream_t stream);

/* Grouped GEMM2 and the routing-weighted combine ([GATED] sections 3-4:
 * FC2 non-gated, scatter unchanged; [TRTLLM]: bf16 output of x's shape).
 *   y_f     = topk_w[f] * dequant(W2[e] . a2[r]) for each real row r, kept
 *             in y_ws ([T*K'][H]) as fp32 rounded to nearest even at its
 *             upper 24 bits (3 bytes a value: sign, exponent, 15 mantissa
 *             bits), or rounded to bf16 for W4A8 (whose outputs the method
 *             holds to relative L2 3e-2)
 *   out[t]  = bf16( sum over j with 0 <= topk_ids[t][j] < E of y_{t*K'+j} ),
 *             summed in slot order j = 0..K'-1, rounded once
 * out is written completely (rows with no valid slot become 0).
 *   y_ws   : moe_combine_workspace_bytes(p) bytes of scratch (not touched when
 *            the block is 16 rows, T <= 2 and T*K' <= 64: GEMM2 and the sum
 *            then run token by token in one kernel, with the same arithmetic
 *            and bit-identical output). */
int moe_gemm2_combine(const moe_problem* p, const void* a2, const void* a2_scale,
                      const moe_weights* w, const int32_t* sorted_ids,
                      const int32_t* block_expert, const int32_t* num_padded,
                      const int32_t* topk_ids, const float* topk_w, void* y_ws,
                      size_t y_ws_bytes, uint16_t* out, moe_stream_t stream);

/* The whole layer: [quant] -> route -> align -> GEMM1+act -> GEMM2+combine.
 *   x        : bf16 [T][H].
 *   logits   : fp32 [T][E_routed], or NULL for the pre-routed entry ([TRTLLM]
 *              section 1, the routed variant), in which case topk_ids and
 *              topk_w are the caller's routing (inputs).  With logits given,
 *              topk_ids / topk_w are optional outputs (NULL: kept in ws).
 *   out      : bf16 [T][H].
 *   ws       : moe_workspace_bytes(p) bytes.
 * A batch of more than 65536 assignments (T*K') runs as consecutive passes
 * over floor(65536 / K') tokens each, in stream order, every pass a layer
 * call of its own on the same workspace: the workspace is that of one pass,
 * so it stops growing with T (each token's output is computed as in a
 * single pass; only the blocking of the assignments differs). */
int moe_forward(const moe_problem* p, const moe_weights* w, const uint16_t* x,
                const float* logits, int32_t* topk_ids, float* topk_w,
                uint16_t* out, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Bytes of the library's fixed per-GPU workspace used by moe_forward_noalloc. */
#define MOE_NOALLOC_WORKSPACE_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory -- code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc: the same kernels and results as moe_forward (bit-identical
 * output), with the workspace taken from a fixed array of
 * MOE_NOALLOC_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * until the process ends.  It allocates nothing, calls no allocating routine
 * and leaves no state that a later call depends on (every value the kernels
 * read back is written earlier in the same call, so nothing must start at
 * zero).
 *   Arguments as moe_forward, without ws / ws_bytes.  `stream` must belong
 *   to the current device (NULL: the null stream of the current device).
 *   The first call on a device looks up the array's device address
 *   (hipGetSymbolAddress); make that call outside stream capture.
 * Returns MOE_ERR_WORKSPACE, before anything is enqueued, when
 * moe_workspace_bytes(p) exceeds MOE_NOALLOC_WORKSPACE_BYTES (decode-sized
 * batches fit: e.g. hidden 2048, 128 experts, top-8, intermediate 768 up to
 * several hundred tokens).  Every call on a GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams or threads) race
 * and must be serialised by the caller. */
int moe_forward_noalloc(const moe_problem* p, const moe_weights* w, const uint16_t* x,
                        const float* logits, int32_t* topk_ids, float* topk_w,
                        uint16_t* out, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
