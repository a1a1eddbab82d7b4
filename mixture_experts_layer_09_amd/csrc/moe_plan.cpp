// Host-side planning: validation, tile table, capacities, workspace layout.
// Pure C++ so that it builds with g++ and runs without a GPU.
#include "moe_plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace moe {

namespace {
thread_local std::string g_last_error;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool quant_is_fp8_act(int q) { return q != MOE_QUANT_BF16; }

// Decode-sized (16-row block) GEMM shapes, measured on MI355X over the bf16,
// fp8 and int4 decode workloads: GEMM1 streams fastest as 32 weight rows per
// workgroup with K split over its four waves, GEMM2 (shorter K) as 64 rows
// with K split four ways.  The fp8 block-scaled GEMM1 keeps 128 output
// channels (256 interleaved rows) in one workgroup, since the group maximum
// of its quantised output spans them.  {kind, nt, wt, ksplit, waves}.
constexpr GemmCfg kStreamG1{0, 1, 2, 4, 4};
constexpr GemmCfg kStreamG2{0, 1, 4, 4, 4};
constexpr GemmCfg kStreamG1Fp8Block{0, 1, 4, 1, 4};
// MX GEMM1: a wave's 4 tiles are whole 32-channel scale blocks of the output;
// K split 4 ways for e4m3 weights, 2 ways for the half-size e2m1 fragments
// (measured: MXFP4 at M = 64 39.7 vs 46.6 us, MXFP8 70.7 vs 76.7)
constexpr GemmCfg kStreamG1Mxfp8{0, 1, 4, 4, 4};
constexpr GemmCfg kStreamG1Mxfp4{0, 1, 4, 2, 4};
// Rows per expert from which fp8 per-tensor, int4 and MX weights take
// 256-row blocks.
constexpr int64_t kWideMinRows = 256;
}  // namespace

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

namespace {
bool valid_act(int32_t act) {
  return act == MOE_ACT_SILU_GATED || act == MOE_ACT_RELU2 || act == MOE_ACT_GELU_TANH_GATED;
}
bool is_gated(int32_t act) { return act != MOE_ACT_RELU2; }
}  // namespace

int32_t padded_intermediate(int32_t I, int32_t act, int32_t quant) {
  if (!valid_act(act)) return MOE_ERR_INVALID_ARG;
  if (quant < MOE_QUANT_BF16 || quant > MOE_QUANT_MXFP4) return MOE_ERR_INVALID_ARG;
  if (I <= 0) return MOE_ERR_INVALID_ARG;
  // the TRTLLM-Gen rule: 16 for gated, 128 for the non-gated relu2 path
  int32_t a = is_gated(act) ? 16 : 128;
  // what the kernels need: a bf16 MFMA k-step is 32 elements, an fp8 / int4
  // k-step, block scale and group scale cover 128
  int32_t k = quant == MOE_QUANT_BF16 ? 32 : 128;
  int32_t m = std::max(a, k);  // both are powers of two
  if (I > kMaxDim) return MOE_ERR_UNSUPPORTED;
  return (I + m - 1) / m * m;
}

size_t packed_weight_bytes(const moe_problem& p, int which) {
  const bool gated = is_gated(p.act);
  const int64_t n = which == 13 ? (gated ? 2 * int64_t(p.I) : p.I) : p.H;
  const int64_t k = which == 13 ? p.H : p.I;
  const int64_t elems = int64_t(p.E) * n * k;
  switch (p.quant) {
    case MOE_QUANT_BF16: return size_t(elems) * 2;
    case MOE_QUANT_FP8_TENSOR:
    case MOE_QUANT_FP8_BLOCK: return size_t(elems);
    case MOE_QUANT_W4A8:
    case MOE_QUANT_MXFP4: return size_t(elems / 2);
    case MOE_QUANT_MXFP8: return size_t(elems);
  }
  return 0;
}

size_t packed_scale_bytes(const moe_problem& p, int which) {
  const bool gated = is_gated(p.act);
  const int64_t n = which == 13 ? (gated ? 2 * int64_t(p.I) : p.I) : p.H;
  const int64_t k = which == 13 ? p.H : p.I;
  switch (p.quant) {
    case MOE_QUANT_BF16: return 0;
    case MOE_QUANT_FP8_TENSOR: return size_t(p.E) * 4;
    case MOE_QUANT_FP8_BLOCK: return size_t(p.E) * (n / kGroup) * (k / kGroup) * 4;
    case MOE_QUANT_W4A8: return size_t(p.E) * n * (k / kGroup) * 4;
    case MOE_QUANT_MXFP8:
    case MOE_QUANT_MXFP4: return size_t(p.E) * n * (k / kMxBlock);  // one E8M0 byte each
  }
  return 0;
}

int make_plan(const moe_problem* p, Plan* plan) {
  char buf[256];
  if (!p || !plan) return fail(MOE_ERR_INVALID_ARG, "null problem");
  if (!valid_act(p->act))
    return fail(MOE_ERR_INVALID_ARG,
                "act must be MOE_ACT_SILU_GATED, MOE_ACT_RELU2 or MOE_ACT_GELU_TANH_GATED");
  if (p->quant < MOE_QUANT_BF16 || p->quant > MOE_QUANT_MXFP4)
    return fail(MOE_ERR_INVALID_ARG, "unknown quant mode");
  if (p->T < 0 || p->H <= 0 || p->I <= 0)
    return fail(MOE_ERR_INVALID_ARG, "T must be >= 0, H and I > 0");
  if (p->H > kMaxDim || p->I > kMaxDim)
    return fail(MOE_ERR_UNSUPPORTED, "H and I must be at most 2^20");
  if (p->E_routed < 1 || p->n_shared < 0 || p->E != p->E_routed + p->n_shared)
    return fail(MOE_ERR_INVALID_ARG, "need E_routed >= 1, n_shared >= 0, E == E_routed + n_shared");
  if (p->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "at most 1024 expert slots");
  if (p->top_k < 1 || p->top_k > p->E_routed)
    return fail(MOE_ERR_INVALID_ARG, "need 1 <= top_k <= E_routed");
  if (p->top_k + p->n_shared > kMaxSlots) {
    std::snprintf(buf, sizeof buf, "top_k + n_shared must be <= %d", kMaxSlots);
    return fail(MOE_ERR_UNSUPPORTED, buf);
  }
  if (p->renormalize != 0 && p->renormalize != 1)
    return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
  if (!std::isfinite(p->shared_gate))
    return fail(MOE_ERR_INVALID_ARG, "shared_gate must be finite");
  if (p->H % kGroup != 0) return fail(MOE_ERR_ALIGNMENT, "H must be a multiple of 128");
  const int32_t ip = padded_intermediate(p->I, p->act, p->quant);
  if (ip != p->I) {
    std::snprintf(buf, sizeof buf, "I = %d is not aligned; pad it to %d (moe_padded_intermediate)",
                  p->I, ip);
    return fail(MOE_ERR_ALIGNMENT, buf);
  }
  if (p->block_m != 0 && p->block_m != 16 && p->block_m != 64 && p->block_m != 128 &&
      p->block_m != 256)
    return fail(MOE_ERR_INVALID_ARG, "block_m must be 0, 16, 64, 128 or 256");

  Plan q;
  q.Kp = p->top_k + p->n_shared;
  q.A = int64_t(p->T) * q.Kp;
  q.gated = is_gated(p->act);
  q.N1 = q.gated ? 2 * p->I : p->I;
  const int64_t big = std::max<int64_t>(p->H, q.N1);
  if (q.A * big >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T * K' * max(H, N1) must stay below 2^31");
  if (int64_t(p->E) * q.N1 * p->H >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "weights too large");

  // ---- tile table: the alignment block follows the expected rows per
  // expert.  Decode-sized problems stream weights 16 token rows at a time;
  // with many rows per expert the tiled kernels stage 128 token rows in LDS
  // and reuse every weight fragment across them; bf16, fp8 per-tensor, int4
  // and MX weights with 256 or more rows per expert take 256 token rows per
  // block, so that each weight byte brought into the LDS (and each int4
  // fragment converted to e4m3) serves twice the tokens.
  const int64_t rows_per_expert = q.A / std::max(1, p->E);
  // the LDS pipeline stages 128 bytes of K per row: bf16 needs I % 64 == 0
  // for GEMM2 (the other formats pad I to 128)
  const bool lds_ok = p->quant != MOE_QUANT_BF16 || p->I % 64 == 0;
  const bool wide_ok = (p->quant == MOE_QUANT_BF16 && lds_ok) || p->quant == MOE_QUANT_FP8_TENSOR ||
                       p->quant == MOE_QUANT_W4A8 || quant_is_mx(p->quant);
  if (p->block_m != 0) {
    q.BM = p->block_m;
  } else if (rows_per_expert >= kWideMinRows && wide_ok) {
    q.BM = 256;
  } else if (rows_per_expert >= kTiledMinRows) {
    q.BM = 128;
  } else {
    q.BM = 16;
  }
  if (q.BM == 256 && !wide_ok)
    return fail(MOE_ERR_UNSUPPORTED,
                "block_m = 256 runs for the bf16 (I a multiple of 64), fp8 per-tensor, int4 (W4A8) "
                "and MX modes only");
  if (quant_is_mx(p->quant) && q.BM == 64)
    return fail(MOE_ERR_UNSUPPORTED, "the MX modes run block_m = 16, 128 and 256");
  const int64_t nz = std::min<int64_t>(p->E, q.A);
  q.max_blocks = std::min<int64_t>(q.A, (q.A + nz * (q.BM - 1)) / q.BM);
  q.max_rows = q.max_blocks * q.BM;
  if (q.max_rows * big >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "padded rows * max(H, N1) must stay below 2^31");
  if (q.max_blocks > 65535)
    return fail(MOE_ERR_UNSUPPORTED, "more than 65535 row blocks in one call");
  q.chunks = int32_t((q.A + kAlignChunk - 1) / kAlignChunk);

  q.kstep = p->quant == MOE_QUANT_BF16 ? 32 : 128;
  q.ksteps_h = p->H / q.kstep;
  q.ksteps_i = p->I / q.kstep;
  q.a2_elem = p->quant == MOE_QUANT_BF16 ? 2 : 1;
  if (q.BM == 16) {
    q.g1 = p->quant == MOE_QUANT_FP8_BLOCK ? kStreamG1Fp8Block
           : p->quant == MOE_QUANT_MXFP8   ? kStreamG1Mxfp8
           : p->quant == MOE_QUANT_MXFP4   ? kStreamG1Mxfp4
                                           : kStreamG1;
    q.g2 = kStreamG2;
    // a handful of tokens: GEMM2 and the combine token by token in one
    // launch (every weight tile a token routes to is streamed for it alone,
    // which at this size is what the expert-major kernel does too)
    q.g2_tok = q.A <= kTokMaxAssign && p->T <= kTokMaxTokens;
    // one token: a block per assignment, each row with the arithmetic it
    // has in the aligned blocks (the routed experts of a token are distinct;
    // an expert repeated in caller-given ids streams its weights per slot)
    q.slot_rows = q.g2_tok && p->T == 1 && p->block_m == 0;
  } else {
    // 128-row blocks: weights and tokens staged in LDS by direct-to-LDS loads,
    // several stages in flight, one persistent workgroup per CU taking the
    // tiles in rounds (kind 3).  256-row blocks: 8 waves, one workgroup per
    // tile (kind 2).  64-row blocks: the register-staged tile (kind 1).
    const bool lds = q.BM >= 128 && lds_ok;
    q.g1 = GemmCfg{lds ? (q.BM == 256 ? 2 : 3) : 1, q.BM / 16, 4, 1, 4};
    q.g2 = q.g1;
  }

  // ---- scratch sizes and the moe_forward workspace layout
  q.align_ws = q.chunks > 1 ? align256(size_t(q.chunks) * p->E * 4) : 256;
  q.combine_ws = align256(size_t(q.A) * p->H * row_bytes(p->quant));
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align256(std::max<size_t>(bytes, 1)); return at; };
  q.off_ids = take(size_t(q.A) * 4);
  q.off_w = take(size_t(q.A) * 4);
  q.off_sorted = take(size_t(q.max_rows) * 4);
  q.off_bexp = take(size_t(q.max_blocks) * 4);
  q.off_offsets = take(size_t(p->E + 1) * 4);
  q.off_npad = take(4);
  q.off_align = take(q.align_ws);
  const bool fp8_act = quant_is_fp8_act(p->quant);
  q.off_xq = take(fp8_act ? size_t(p->T) * p->H : 0);
  const bool mx = quant_is_mx(p->quant);
  q.off_xs = take(p->quant == MOE_QUANT_FP8_BLOCK ? size_t(p->T) * (p->H / kGroup) * 4
                  : mx                            ? size_t(p->T) * (p->H / kMxBlock)
                                                  : 0);
  q.off_a2 = take(size_t(q.max_rows) * p->I * q.a2_elem);
  q.off_a2s = take(p->quant == MOE_QUANT_FP8_BLOCK ? size_t(q.max_rows) * (p->I / kGroup) * 4
                   : mx                            ? size_t(q.max_rows) * (p->I / kMxBlock)
                                                   : 0);
  q.off_y = take(q.combine_ws);
  q.ws_total = o;
  // moe_forward runs a large batch in passes of at most kChunkAssign
  // assignments, each with the workspace of its own (smaller) problem, so
  // that the workspace stops growing with T * K' * H
  q.chunk_T = p->T;
  if (q.A > kChunkAssign) {
    moe_problem c = *p;
    c.T = int32_t(kChunkAssign / q.Kp);
    Plan qc;
    const int st = make_plan(&c, &qc);  // no deeper: qc.A <= kChunkAssign
    if (st != MOE_OK) return st;
    q.chunk_T = c.T;
    q.off_ids = qc.off_ids;
    q.off_w = qc.off_w;
    q.off_sorted = qc.off_sorted;
    q.off_bexp = qc.off_bexp;
    q.off_offsets = qc.off_offsets;
    q.off_npad = qc.off_npad;
    q.off_align = qc.off_align;
    q.off_xq = qc.off_xq;
    q.off_xs = qc.off_xs;
    q.off_a2 = qc.off_a2;
    q.off_a2s = qc.off_a2s;
    q.off_y = qc.off_y;
    q.ws_total = qc.ws_total;
  }
  *plan = q;
  return MOE_OK;
}

}  // namespace moe

// ---------------------------------------------------------------- C ABI
extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_ALIGNMENT: return "MOE_ERR_ALIGNMENT";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return moe::last_error(); }

int moe_validate(const moe_problem* p) {
  moe::Plan q;
  return moe::make_plan(p, &q);
}

int32_t moe_padded_intermediate(int32_t I, int32_t act, int32_t quant) {
  return moe::padded_intermediate(I, act, quant);
}

int32_t moe_block_m(const moe_problem* p) {
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  return st == MOE_OK ? q.BM : st;
}

int64_t moe_max_blocks(const moe_problem* p) {
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  return st == MOE_OK ? q.max_blocks : st;
}

int64_t moe_max_padded_rows(const moe_problem* p) {
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  return st == MOE_OK ? q.max_rows : st;
}

size_t moe_align_workspace_bytes(const moe_problem* p) {
  moe::Plan q;
  return moe::make_plan(p, &q) == MOE_OK ? q.align_ws : 0;
}

size_t moe_combine_workspace_bytes(const moe_problem* p) {
  moe::Plan q;
  return moe::make_plan(p, &q) == MOE_OK ? q.combine_ws : 0;
}

size_t moe_workspace_bytes(const moe_problem* p) {
  moe::Plan q;
  return moe::make_plan(p, &q) == MOE_OK ? q.ws_total : 0;
}

int moe_packed_bytes(const moe_problem* p, int32_t which, size_t* w_bytes, size_t* s_bytes) {
  moe::Plan q;
  int st = moe::make_plan(p, &q);
  if (st != MOE_OK) return st;
  if (which != 13 && which != 2) return moe::fail(MOE_ERR_INVALID_ARG, "which must be 13 or 2");
  if (!w_bytes || !s_bytes) return moe::fail(MOE_ERR_INVALID_ARG, "null output pointer");
  *w_bytes = moe::packed_weight_bytes(*p, which);
  *s_bytes = moe::packed_scale_bytes(*p, which);
  return MOE_OK;
}

}  // extern "C"
