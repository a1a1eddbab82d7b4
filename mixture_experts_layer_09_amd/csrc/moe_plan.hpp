// Host-side planning for one layer call: validation, the tile table, buffer
// capacities and the workspace layout.  Pure C++ (no HIP), so it builds and is
// tested without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/moe.h"

namespace moe {

constexpr int kGroup = 128;        // block / group width of the quantised formats
constexpr int kAlignChunk = 1024;  // assignments per workgroup in the align kernels
constexpr int kMaxRouted = 1024;   // logits per token the routing kernel holds
constexpr int kMaxSlots = 64;      // K' = top_k + n_shared limit (one lane each)
constexpr int kTiledMinRows = 48;  // rows per expert from which the tiled GEMMs run
constexpr int kMxBlock = 32;       // elements per E8M0 scale in the MX modes
constexpr int kMaxDim = 1 << 20;   // largest H and I (keeps 2I and padding in int32)
constexpr int kTokMaxAssign = 64;  // GEMM2 runs token by token up to this many assignments
constexpr int kTokMaxTokens = 2;   // and tokens (measured: 8 tokens ran slower that way)
constexpr int64_t kChunkAssign = 65536;  // moe_forward passes over at most this many assignments

// GEMM2's per-assignment rows are bf16 for int4 weights (W4A8), otherwise
// fp32 rounded to its upper 24 bits (sign, exponent, 15 mantissa bits).
constexpr bool rows_bf16(int quant) { return quant == MOE_QUANT_W4A8; }
constexpr int row_bytes(int quant) { return rows_bf16(quant) ? 2 : 3; }

// The OCP MX modes (E8M0 scales per 32 K on weights and activations).
inline bool quant_is_mx(int q) { return q == MOE_QUANT_MXFP8 || q == MOE_QUANT_MXFP4; }

// Which GEMM kernel runs and how it is tiled.
//  kind 0: weight-streaming kernel, one 16-row block of tokens per workgroup,
//          A (weights) and B (tokens) fragments loaded straight into registers;
//  kind 1: tiled kernel, BM tokens staged through LDS and shared by the waves.
struct GemmCfg {
  int kind;    // 0 stream, 1 tiled (register-staged weights), 2 tiled LDS-DMA pipeline,
               // 3 the same, persistent (one workgroup per CU, tiles in rounds)
  int nt;      // 16-token MFMA tiles per block (BM = 16 * nt)
  int wt;      // 16-row weight tiles per wave
  int ksplit;  // waves of a workgroup that split K (stream kernel)
  int waves;   // waves per workgroup
};

struct Plan {
  int32_t Kp = 0;          // slots per token
  int64_t A = 0;           // assignments T * Kp
  int32_t BM = 0;          // resolved block_m
  int64_t max_blocks = 0;
  int64_t max_rows = 0;
  int32_t chunks = 0;      // align chunks of kAlignChunk assignments
  bool gated = false;
  int32_t N1 = 0;          // rows of W13 (2I or I)
  int32_t ksteps_h = 0;    // MFMA k-steps along H
  int32_t ksteps_i = 0;    // MFMA k-steps along I
  int32_t kstep = 0;       // K elements per MFMA k-step (32 bf16, 128 fp8/int4)
  int32_t a2_elem = 0;     // bytes per intermediate element
  GemmCfg g1{}, g2{};
  bool g2_tok = false;     // GEMM2 and the combine token by token, in one launch
  bool slot_rows = false;  // moe_forward on one token: GEMM1 block b holds assignment b
                           // alone, no alignment (the rows of slot f start at 16 f)
  int32_t chunk_T = 0;     // tokens per moe_forward pass (the workspace below is one pass's)
  // moe_forward workspace layout (byte offsets, 256-B aligned), for a pass of
  // chunk_T tokens
  size_t off_ids = 0, off_w = 0, off_sorted = 0, off_bexp = 0, off_offsets = 0,
         off_npad = 0, off_align = 0, off_xq = 0, off_xs = 0, off_a2 = 0,
         off_a2s = 0, off_y = 0, ws_total = 0;
  size_t align_ws = 0, combine_ws = 0;
};

// Records a failure detail for moe_last_error() and returns `status`.
int fail(int status, const std::string& msg);
void clear_error();
const char* last_error();

// Validates `p` and fills `plan`.  Returns MOE_OK or an error status.
int make_plan(const moe_problem* p, Plan* plan);

int32_t padded_intermediate(int32_t I, int32_t act, int32_t quant);
size_t packed_weight_bytes(const moe_problem& p, int which);
size_t packed_scale_bytes(const moe_problem& p, int which);

}  // namespace moe
