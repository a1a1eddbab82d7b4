// Host-side planner and validator under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ by tests/test_plan_sanitize.py).
//
// Walks a grid of problems -- valid ones, every argument error the validator
// guards against, and sizes at the edges of the int32 / int64 limits -- and
// calls every host-only entry point of include/moe.h on each, checking the
// invariants of the results: a valid plan has 256-byte aligned, increasing,
// non-overlapping workspace segments inside moe_workspace_bytes, its row
// capacity is blocks x block_m, and an invalid one returns the same negative
// status from every entry point and records a detail string.  Any undefined
// behaviour (signed overflow, out-of-range shift, bad access) aborts the run
// with the sanitizer's report.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "../mixture_experts_layer_09_amd/csrc/moe_plan.hpp"

namespace {

int g_fail = 0;

#define CHECK(cond)                                                                \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
      ++g_fail;                                                                    \
    }                                                                              \
  } while (0)

moe_problem make(int T, int H, int I, int Er, int k, int ns, int act, int quant, int bm) {
  moe_problem p{};
  p.T = T;
  p.H = H;
  p.I = I;
  p.E_routed = Er;
  p.n_shared = ns;
  p.E = Er + ns;
  p.top_k = k;
  p.shared_gate = 1.0f;
  p.renormalize = 1;
  p.act = act;
  p.quant = quant;
  p.block_m = bm;
  return p;
}

void check_problem(const moe_problem& p) {
  moe::Plan q;
  const int st = moe::make_plan(&p, &q);
  CHECK(moe_validate(&p) == st);
  if (st != MOE_OK) {
    CHECK(st < 0);
    CHECK(std::strlen(moe_last_error()) > 0);
    CHECK(moe_block_m(&p) == st);
    CHECK(moe_max_blocks(&p) == st);
    CHECK(moe_max_padded_rows(&p) == st);
    CHECK(moe_workspace_bytes(&p) == 0);
    CHECK(moe_align_workspace_bytes(&p) == 0);
    CHECK(moe_combine_workspace_bytes(&p) == 0);
    size_t w = 1, s = 1;
    CHECK(moe_packed_bytes(&p, 13, &w, &s) == st);
    return;
  }
  CHECK(moe_block_m(&p) == q.BM);
  CHECK(q.BM == 16 || q.BM == 64 || q.BM == 128 || q.BM == 256);
  CHECK(moe_max_blocks(&p) == q.max_blocks);
  CHECK(moe_max_padded_rows(&p) == q.max_blocks * q.BM);
  CHECK(q.A == int64_t(p.T) * (p.top_k + p.n_shared));
  CHECK(q.max_blocks <= q.A);
  CHECK(q.max_rows >= q.A);
  CHECK(moe_workspace_bytes(&p) == q.ws_total);
  // moe_forward's workspace is that of one pass of chunk_T tokens
  const int64_t Kp = p.top_k + p.n_shared;
  moe::Plan w = q;  // the plan of a pass
  if (q.A <= moe::kChunkAssign) {
    CHECK(q.chunk_T == p.T);
  } else {
    CHECK(q.chunk_T == int32_t(moe::kChunkAssign / Kp));
    moe_problem c = p;
    c.T = q.chunk_T;
    CHECK(moe::make_plan(&c, &w) == MOE_OK);
    CHECK(w.A <= moe::kChunkAssign);
    CHECK(w.ws_total == q.ws_total);
    CHECK(w.off_y == q.off_y && w.off_a2 == q.off_a2 && w.off_sorted == q.off_sorted);
    // the short last pass fits the same workspace
    c.T = p.T % q.chunk_T;
    if (c.T > 0) {
      moe::Plan t;
      CHECK(moe::make_plan(&c, &t) == MOE_OK);
      CHECK(t.ws_total <= q.ws_total);
    }
  }
  const size_t offs[] = {w.off_ids, w.off_w,  w.off_sorted, w.off_bexp, w.off_offsets, w.off_npad,
                         w.off_align, w.off_xq, w.off_xs,   w.off_a2,   w.off_a2s,     w.off_y,
                         w.ws_total};
  for (size_t i = 0; i + 1 < sizeof(offs) / sizeof(offs[0]); ++i) {
    CHECK(offs[i] % 256 == 0);
    CHECK(offs[i] < offs[i + 1]);
  }
  // the segments hold what the kernels write into them
  CHECK(w.off_sorted - w.off_w >= size_t(w.A) * 4);
  CHECK(w.off_bexp - w.off_sorted >= size_t(w.max_rows) * 4);
  CHECK(w.off_offsets - w.off_bexp >= size_t(w.max_blocks) * 4);
  CHECK(w.off_npad - w.off_offsets >= size_t(p.E + 1) * 4);
  CHECK(w.off_xq - w.off_align >= w.align_ws);
  CHECK(w.off_a2s - w.off_a2 >= size_t(w.max_rows) * p.I * w.a2_elem);
  CHECK(w.ws_total - w.off_y >= w.combine_ws);
  CHECK(moe_align_workspace_bytes(&p) == q.align_ws);
  CHECK(moe_combine_workspace_bytes(&p) == q.combine_ws);
  size_t w13 = 0, s13 = 0, w2 = 0, s2 = 0;
  CHECK(moe_packed_bytes(&p, 13, &w13, &s13) == MOE_OK);
  CHECK(moe_packed_bytes(&p, 2, &w2, &s2) == MOE_OK);
  CHECK(w13 > 0 && w2 > 0);
  CHECK((s13 == 0) == (p.quant == MOE_QUANT_BF16));
  size_t dummy = 0;
  CHECK(moe_packed_bytes(&p, 5, &dummy, &dummy) == MOE_ERR_INVALID_ARG);
  CHECK(moe_packed_bytes(&p, 13, nullptr, &dummy) == MOE_ERR_INVALID_ARG);
}

}  // namespace

int main() {
  long n = 0;
  const int Ts[] = {0, 1, 7, 64, 4096, 65536, 1 << 20, std::numeric_limits<int>::max(), -1};
  const int Hs[] = {128, 200, 2048, 6144, 0, 1 << 30};
  const int Is[] = {32, 100, 128, 512, 768, 2688, 0, -5, 1 << 30};
  const int Es[][3] = {{1, 1, 0}, {8, 2, 0}, {128, 8, 0}, {512, 10, 1}, {20, 8, 0},
                       {1024, 64, 0}, {1100, 2, 0}, {100, 65, 0}, {8, 0, 0}, {8, 9, 0},
                       {1020, 60, 4}, {8, 2, -1}};
  const int bms[] = {0, 16, 64, 128, 256, 17};
  for (int quant = -1; quant <= 6; ++quant)
    for (int act = -1; act <= 3; ++act)
      for (int T : Ts)
        for (int H : Hs)
          for (int I : Is)
            for (const auto& e : Es)
              for (int bm : bms) {
                check_problem(make(T, H, I, e[0], e[1], e[2], act, quant, bm));
                ++n;
              }
  // fields a caller can leave inconsistent
  moe_problem p = make(8, 256, 512, 8, 2, 0, 0, 0, 0);
  p.E = 9;
  CHECK(moe_validate(&p) == MOE_ERR_INVALID_ARG);
  p = make(8, 256, 512, 8, 2, 0, 0, 0, 0);
  p.renormalize = 2;
  CHECK(moe_validate(&p) == MOE_ERR_INVALID_ARG);
  p.renormalize = 1;
  p.shared_gate = std::numeric_limits<float>::quiet_NaN();
  CHECK(moe_validate(&p) == MOE_ERR_INVALID_ARG);
  p.shared_gate = std::numeric_limits<float>::infinity();
  CHECK(moe_validate(&p) == MOE_ERR_INVALID_ARG);
  CHECK(moe_validate(nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_block_m(nullptr) < 0 && moe_max_blocks(nullptr) < 0);
  CHECK(moe_workspace_bytes(nullptr) == 0);
  for (int I = -3; I <= 4100; ++I)
    for (int act = -1; act <= 3; ++act)
      for (int quant = -1; quant <= 6; ++quant) {
        const int32_t r = moe_padded_intermediate(I, act, quant);
        if (r > 0) CHECK(r >= I && r % 32 == 0);
      }
  for (int st = -7; st <= 1; ++st) CHECK(moe_status_string(st) != nullptr);
  std::printf("plan_sanitize: %ld problems, %d failed checks\n", n, g_fail);
  return g_fail == 0 ? 0 : 1;
}
