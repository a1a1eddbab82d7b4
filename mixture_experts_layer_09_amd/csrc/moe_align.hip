// Alignment of the (token, slot) assignments into per-expert blocks.
//
// The flat assignments f = t*K' + j are grouped by expert, in ascending f
// within an expert, each group padded with the sentinel A = T*K' to a
// multiple of the GEMM row block BM; `expert_offsets` is the exclusive prefix
// of the padded counts and `block_expert` names the expert of every block
// (sglang PR 26204 page, BLOCK_SIZE_M of the fused-MoE config; sglang PR 38220
// page, the grouped GEMM's expert_offsets / problem sizes).
//
// Stable ranks come from wave ballots: within a wave, the lanes holding the
// same expert are found with one ballot per distinct expert (the expert read
// from the leader lane with v_readlane), and a lane's rank is the number of
// such lanes below it.  Ranks across the 16 waves of a workgroup add the
// earlier waves' counts; across workgroups (chunks of 1024 assignments) a
// per-chunk histogram is scanned per expert.
//   A <= 1024 : one workgroup, one launch -- and, for decode-sized batches,
//               together with the routing and the fp8 quantisation of x in the
//               same kernel;
//   A <= 4096 : one workgroup ranking the chunks one after another;
//   A >  4096 : histogram -> scan -> scatter, three launches.
#include "moe_device.hpp"
#include "moe_launch.hpp"
#include "moe_route.hpp"

namespace moe {

namespace {

constexpr int kThreads = kAlignChunk;  // 1024 threads, 16 waves
constexpr int kWaves = kThreads / 64;

// Rank of this lane among the active lanes with the same expert below it, and
// the number of active lanes with that expert.  The lanes sharing this lane's
// expert are found with one ballot per bit of the expert id: a lane matches
// when it agrees with this lane on every bit.
__device__ __forceinline__ void match_rank(int e, bool valid, int nbits, int& rank, int& cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    same &= bit ? ones : ~ones;
  }
  rank = valid ? __popcll(same & below) : 0;
  cnt = valid ? __popcll(same) : 0;
}

__device__ __forceinline__ int id_bits(int E) { return 32 - __clz(E > 1 ? E - 1 : 1); }

// Exclusive prefix sum over the 1024 threads of the block; returns this
// thread's prefix and writes the block total to *total.  `tmp` holds
// kWaves + 1 ints of shared memory.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kWaves ? tmp[lane] : 0;
    const int wi = wave_inclusive_scan(w);
    if (lane < kWaves) tmp[lane] = wi - w;
    if (lane == kWaves - 1) tmp[kWaves] = wi;
  }
  __syncthreads();
  const int res = tmp[wave] + incl - v;
  *total = tmp[kWaves];
  __syncthreads();
  return res;
}

// Padded offsets from per-expert counts held in shared memory `cnt[E]`;
// writes off[E+1] (shared) and the global expert_offsets / num_padded.
__device__ void padded_offsets(const int* cnt, int* off, int E, int BM, int* tmp,
                               int32_t* g_offsets, int32_t* g_npad) {
  const int per = (E + kThreads - 1) / kThreads;
  const int lo = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E) local += (cnt[e] + BM - 1) / BM * BM;
  }
  int total;
  int run = block_exclusive_scan(local, tmp, &total);
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E) {
      off[e] = run;
      g_offsets[e] = run;
      run += (cnt[e] + BM - 1) / BM * BM;
    }
  }
  if (threadIdx.x == 0) {
    off[E] = total;
    g_offsets[E] = total;
    *g_npad = total;
  }
  __syncthreads();
}

// Sentinels after each expert's real rows, and the expert of every block.
// Sixteen lanes per expert, so that a long tail (up to BM - 1 sentinels)
// is written by sixteen contiguous stores at a time rather than by one lane.
__device__ void fill_tail(const int* cnt, const int* off, int E, int BM, int A,
                          int32_t* sorted_ids, int32_t* block_expert) {
  const int sub = threadIdx.x & 15;
  for (int e = threadIdx.x >> 4; e < E; e += kThreads / 16) {
    const int end = off[e + 1];
    for (int r = off[e] + cnt[e] + sub; r < end; r += 16) sorted_ids[r] = A;
    for (int b = off[e] / BM + sub; b < end / BM; b += 16) block_expert[b] = e;
  }
}

// Whole alignment of A <= 1024 assignments held in shared memory `sids` by
// one workgroup.  `tab` provides cnt[E], off[E+1], wcnt[kWaves][E], tmp.
__device__ void align_in_block(const int* sids, int A, int E, int BM, int* tab,
                               int32_t* __restrict__ sorted_ids,
                               int32_t* __restrict__ block_expert,
                               int32_t* __restrict__ g_offsets, int32_t* __restrict__ g_npad) {
  int* cnt = tab;
  int* off = cnt + E;
  int* wcnt = off + E + 1;
  int* tmp = wcnt + kWaves * E;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  const int f = threadIdx.x;
  const int e = f < A ? sids[f] : -1;
  const bool valid = f < A && e >= 0 && e < E;
  int rank, c;
  match_rank(e, valid, id_bits(E), rank, c);
  if (valid && rank == 0) wcnt[wave * E + e] = c;
  __syncthreads();
  // per expert: total count, and the earlier waves' counts in place
  for (int x = threadIdx.x; x < E; x += kThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int v = wcnt[w * E + x];
      wcnt[w * E + x] = run;
      run += v;
    }
    cnt[x] = run;
  }
  __syncthreads();
  padded_offsets(cnt, off, E, BM, tmp, g_offsets, g_npad);
  if (valid) sorted_ids[off[e] + wcnt[wave * E + e] + rank] = f;
  fill_tail(cnt, off, E, BM, A, sorted_ids, block_expert);
}

size_t small_tables_bytes(int E) {
  return (size_t(E) + (E + 1) + size_t(kWaves) * E + kWaves + 1) * 4;
}

// Dynamic shared memory above the 64 KiB default needs the kernel's opt-in.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

}  // namespace

// One workgroup for A <= 1024: ids to shared memory, then the alignment.
__global__ __launch_bounds__(kThreads) void align_small(const int32_t* __restrict__ ids,
                                                        int A, int E, int BM,
                                                        int32_t* __restrict__ sorted_ids,
                                                        int32_t* __restrict__ block_expert,
                                                        int32_t* __restrict__ g_offsets,
                                                        int32_t* __restrict__ g_npad) {
  extern __shared__ int smem[];
  int* sids = smem;
  if (threadIdx.x < A) sids[threadIdx.x] = ids[threadIdx.x];
  __syncthreads();
  align_in_block(sids, A, E, BM, smem + kThreads, sorted_ids, block_expert, g_offsets, g_npad);
}

// The decode-size prologue in one launch (T <= 128, T*K' <= 1024): routing
// (groups of L lanes per token) or the caller's ids, then the alignment of
// the ids held in shared memory, in one workgroup; the fp8 / MXFP8
// quantisation of x in the launch's other workgroups.
struct PrologueArgs {
  const float* logits;     // null: pre-routed, ids_in given
  const int32_t* ids_in;
  int T, Er, top_k, n_shared;
  float shared_gate;
  int renorm, E, BM, H;
  int32_t* ids;
  float* wts;
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* offsets;
  int32_t* npad;
  int align;               // 0: routing (and quantisation) only
  const uint16_t* x;       // quantisation (QM != 0)
  const float* a1;
  uint8_t* xq;
  void* xs;                // fp32 (QM 2) or E8M0 bytes (QM 3)
};

// One 8-element group of x per thread: i indexes the groups of x [T][H].
// QM: 1 static per-tensor a1, 2 per token and 128 columns (a DPP row of 16
// lanes is one group), 3 MXFP8 per token and 32 columns (a DPP quad).  Every
// lane of the wave takes part in the reductions; lanes past the end hold 0.
template <int QM>
__device__ __forceinline__ void quant_group8(const PrologueArgs& a, int i) {
  const bool in = int64_t(i) < int64_t(a.T) * a.H / 8;
  const u32x4 v = in ? ld16(a.x + size_t(i) * 8) : u32x4{0, 0, 0, 0};
  float f[8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_to_f32(v[k] & 0xFFFFu);
    f[2 * k + 1] = bf16_to_f32(v[k] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * k]), fabsf(f[2 * k + 1])));
  }
  float s = QM == 1 ? *a.a1 : 1.f;
  if (QM >= 2) {
    amax = fmaxf(amax, __uint_as_float(dpp<kDppXor1, 0xF>(0u, __float_as_uint(amax))));
    amax = fmaxf(amax, __uint_as_float(dpp<kDppXor2, 0xF>(0u, __float_as_uint(amax))));
  }
  if (QM == 3) {
    const int X = mx8_exponent(amax);
    if (in) {
      u32x2 o;
      o[0] = mx8x4(f[0], f[1], f[2], f[3], X);
      o[1] = mx8x4(f[4], f[5], f[6], f[7], X);
      *reinterpret_cast<u32x2*>(a.xq + size_t(i) * 8) = o;
      if ((threadIdx.x & 3) == 0) static_cast<uint8_t*>(a.xs)[i / 4] = uint8_t(X + 127);
    }
    return;
  }
  if (QM == 2) {
    amax = fmaxf(amax, __uint_as_float(dpp<kDppHalfMirror, 0xF>(0u, __float_as_uint(amax))));
    amax = fmaxf(amax, __uint_as_float(dpp<kDppMirror, 0xF>(0u, __float_as_uint(amax))));
    s = amax > 0.f ? amax / 448.f : 1.f;
  }
  if (in) {
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] = f[k] / s;
    u32x2 o;
    o[0] = e4m3x4(f[0], f[1], f[2], f[3]);
    o[1] = e4m3x4(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<u32x2*>(a.xq + size_t(i) * 8) = o;
    if (QM == 2 && (threadIdx.x & 15) == 0) static_cast<float*>(a.xs)[i / 16] = s;
  }
}

// Workgroup 0 routes (groups of L lanes per token) or takes the caller's ids,
// then aligns them in shared memory; with QM != 0, workgroups 1.. quantise x
// at the same time, one 8-element group per thread (neither part reads what
// the other writes).
template <int L, int NPL, int QM>
__global__ __launch_bounds__(kThreads) void prologue_small(PrologueArgs a) {
  extern __shared__ int smem[];
  if constexpr (QM != 0) {
    if (blockIdx.x > 0) {  // uniform per workgroup: no barrier below is reached
      quant_group8<QM>(a, int(blockIdx.x - 1) * kThreads + int(threadIdx.x));
      return;
    }
  }
  int* sids = smem;
  const int Kp = a.top_k + a.n_shared;
  const int wave = threadIdx.x >> 6;
  if (a.logits) {
    constexpr int TPW = 64 / L;
    for (int base = 0; base < a.T; base += kWaves * TPW) {
      const int first = base + wave * TPW;
      if (first < a.T) {  // uniform per wave
        const int t = first + (threadIdx.x & 63) / L;
        const bool valid = t < a.T;
        const int tt = valid ? t : 0;
        route_token<L, NPL>(a.logits + size_t(tt) * a.Er, valid, a.Er, a.top_k, a.n_shared,
                            a.shared_gate, a.renorm, a.ids + size_t(tt) * Kp,
                            a.wts + size_t(tt) * Kp, sids + tt * Kp);
      }
    }
  } else if (a.align) {
    for (int f = threadIdx.x; f < a.T * Kp; f += kThreads) sids[f] = a.ids_in[f];
  }
  if (!a.align) return;  // uniform
  __syncthreads();
  align_in_block(sids, a.T * Kp, a.E, a.BM, smem + kThreads, a.sorted_ids, a.block_expert,
                 a.offsets, a.npad);
}

// One workgroup for 1024 < A <= kMidChunks * 1024: the chunks of 1024
// assignments are ranked one after another -- per expert, the count of the
// earlier chunks, plus the earlier waves of this chunk, plus the lane's rank
// in its wave -- then the padded offsets and the scatter.  Shared memory:
// run[E], wcnt[kWaves][E], off[E+1], tmp.
constexpr int kMidChunks = 4;
__global__ __launch_bounds__(kThreads) void align_mid(const int32_t* __restrict__ ids, int A,
                                                      int E, int BM,
                                                      int32_t* __restrict__ sorted_ids,
                                                      int32_t* __restrict__ block_expert,
                                                      int32_t* __restrict__ g_offsets,
                                                      int32_t* __restrict__ g_npad) {
  extern __shared__ int smem[];
  int* run = smem;
  int* wcnt = run + E;
  int* off = wcnt + kWaves * E;
  int* tmp = off + E + 1;
  const int wave = threadIdx.x >> 6;
  int ev[kMidChunks];
#pragma unroll
  for (int c = 0; c < kMidChunks; ++c) {
    const int f = c * kThreads + threadIdx.x;
    ev[c] = f < A ? ids[f] : -1;
  }
  for (int i = threadIdx.x; i < E; i += kThreads) run[i] = 0;
  const int nbits = id_bits(E);
  int rank[kMidChunks];
#pragma unroll
  for (int c = 0; c < kMidChunks; ++c) {
    for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
    __syncthreads();
    const int e = ev[c];
    const bool valid = c * kThreads + int(threadIdx.x) < A && e >= 0 && e < E;
    int r, cnt;
    match_rank(e, valid, nbits, r, cnt);
    if (valid && r == 0) wcnt[wave * E + e] = cnt;
    __syncthreads();
    // per expert: the waves' bases in place, the running count advanced
    for (int x = threadIdx.x; x < E; x += kThreads) {
      int acc = run[x];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int v = wcnt[w * E + x];
        wcnt[w * E + x] = acc;
        acc += v;
      }
      run[x] = acc;
    }
    __syncthreads();
    rank[c] = valid ? wcnt[wave * E + e] + r : -1;
    __syncthreads();  // wcnt is cleared for the next chunk
  }
  padded_offsets(run, off, E, BM, tmp, g_offsets, g_npad);
#pragma unroll
  for (int c = 0; c < kMidChunks; ++c)
    if (rank[c] >= 0) sorted_ids[off[ev[c]] + rank[c]] = c * kThreads + threadIdx.x;
  fill_tail(run, off, E, BM, A, sorted_ids, block_expert);
}

// Chunk histogram: hist[c][e] = assignments of chunk c with expert e.
__global__ __launch_bounds__(kThreads) void align_count(const int32_t* __restrict__ ids, int A,
                                                        int E, int32_t* __restrict__ hist) {
  extern __shared__ int h[];
  for (int i = threadIdx.x; i < E; i += kThreads) h[i] = 0;
  __syncthreads();
  const int f = blockIdx.x * kThreads + threadIdx.x;
  if (f < A) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kThreads) hist[size_t(blockIdx.x) * E + i] = h[i];
}

// One workgroup: totals, padded offsets, each chunk's base row per expert
// (in place in hist), tails.  When the histograms fit (chunks * E <=
// kScanStageInts) they are first copied into shared memory with all loads
// in flight at once and scanned there, then written back row by row;
// otherwise each thread walks its experts' columns in global memory.
// Shared memory: cnt[E], off[E+1], tmp[kWaves+1] (+ the staged hist).
constexpr int kScanStageInts = 32 * kThreads;

size_t scan_lds_bytes(int chunks, int E) {
  const size_t base = size_t(E) + (E + 1) + kWaves + 1;
  return (base + (size_t(chunks) * E <= size_t(kScanStageInts) ? size_t(chunks) * E : 0)) * 4;
}

__global__ __launch_bounds__(kThreads) void align_scan(int32_t* __restrict__ hist, int chunks,
                                                       int A, int E, int BM,
                                                       int32_t* __restrict__ sorted_ids,
                                                       int32_t* __restrict__ block_expert,
                                                       int32_t* __restrict__ g_offsets,
                                                       int32_t* __restrict__ g_npad) {
  extern __shared__ int smem[];
  int* cnt = smem;
  int* off = cnt + E;
  int* tmp = off + E + 1;
  int* h = tmp + kWaves + 1;
  if (int64_t(chunks) * E <= kScanStageInts) {
    const int n = chunks * E;
    {
      int v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int i = threadIdx.x + u * kThreads;
        v[u] = i < n ? hist[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int i = threadIdx.x + u * kThreads;
        if (i < n) h[i] = v[u];
      }
    }
    __syncthreads();
    // P consecutive lanes per expert (E <= 1024 = kThreads experts in one
    // pass), each over a contiguous range of the chunks: the range's count,
    // then a prefix over the expert's P lanes gives each range's start
    const int P = E > kThreads / 2 ? 1 : E > kThreads / 4 ? 2 : E > kThreads / 8 ? 4
                : E > kThreads / 16 ? 8 : 16;
    const int lane = threadIdx.x & 63, x = threadIdx.x / P, part = threadIdx.x % P;
    const bool own = x < E;
    const int per = (chunks + P - 1) / P;
    const int c0 = min(chunks, part * per), c1 = min(chunks, c0 + per);
    int sum = 0;
    if (own)
      for (int c = c0; c < c1; ++c) sum += h[c * E + x];
    int incl = sum;  // inclusive prefix over the expert's lanes (P divides 64)
    for (int d = 1; d < P; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (part >= d) incl += o;
    }
    const int total = __shfl(incl, lane - part + P - 1, 64);
    if (own && part == 0) cnt[x] = total;
    __syncthreads();
    padded_offsets(cnt, off, E, BM, tmp, g_offsets, g_npad);
    if (own) {
      int run = off[x] + incl - sum;
      for (int c = c0; c < c1; ++c) {
        const int v = h[c * E + x];
        h[c * E + x] = run;
        run += v;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) hist[i] = h[i];
  } else {
    // per expert, its chunks' counts: 8 independent loads in flight per pass
    for (int x = threadIdx.x; x < E; x += kThreads) {
      int run = 0;
      for (int c0 = 0; c0 < chunks; c0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = c0 + u < chunks ? hist[size_t(c0 + u) * E + x] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) run += v[u];
      }
      cnt[x] = run;
    }
    __syncthreads();
    padded_offsets(cnt, off, E, BM, tmp, g_offsets, g_npad);
    for (int x = threadIdx.x; x < E; x += kThreads) {
      int run = off[x];
      for (int c0 = 0; c0 < chunks; c0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = c0 + u < chunks ? hist[size_t(c0 + u) * E + x] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (c0 + u < chunks) hist[size_t(c0 + u) * E + x] = run;
          run += v[u];
        }
      }
    }
  }
  fill_tail(cnt, off, E, BM, A, sorted_ids, block_expert);
}

// Stable scatter of chunk c, starting each expert at base[c][e].
// Shared memory: wcnt[kWaves][E].
__global__ __launch_bounds__(kThreads) void align_scatter(const int32_t* __restrict__ ids, int A,
                                                          int E, const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ sorted_ids) {
  extern __shared__ int wcnt[];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  const int f = blockIdx.x * kThreads + threadIdx.x;
  const int e = f < A ? ids[f] : -1;
  const bool valid = f < A && e >= 0 && e < E;
  int rank, c;
  match_rank(e, valid, id_bits(E), rank, c);
  if (valid && rank == 0) wcnt[wave * E + e] = c;
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w * E + e];
    sorted_ids[base[size_t(blockIdx.x) * E + e] + before + rank] = f;
  }
}

hipError_t launch_align(const moe_problem& p, const Plan& q, const int32_t* ids,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                        int32_t* num_padded, int32_t* scratch, hipStream_t stream) {
  const int A = int(q.A), E = p.E, BM = q.BM;
  if (q.chunks <= 1) {
    const size_t sm = size_t(kThreads) * 4 + small_tables_bytes(E);
    hipError_t err = allow_lds(align_small, sm);
    if (err != hipSuccess) return err;
    align_small<<<1, kThreads, sm, stream>>>(ids, A, E, BM, sorted_ids, block_expert, offsets,
                                             num_padded);
    return hipGetLastError();
  }
  if (q.chunks <= kMidChunks) {
    const size_t sm = (size_t(E) + size_t(kWaves) * E + (E + 1) + kWaves + 1) * 4;
    hipError_t err = allow_lds(align_mid, sm);
    if (err != hipSuccess) return err;
    align_mid<<<1, kThreads, sm, stream>>>(ids, A, E, BM, sorted_ids, block_expert, offsets,
                                           num_padded);
    return hipGetLastError();
  }
  align_count<<<q.chunks, kThreads, size_t(E) * 4, stream>>>(ids, A, E, scratch);
  const size_t sm_scan = scan_lds_bytes(q.chunks, E);
  hipError_t err = allow_lds(align_scan, sm_scan);
  if (err != hipSuccess) return err;
  align_scan<<<1, kThreads, sm_scan, stream>>>(scratch, q.chunks, A, E, BM, sorted_ids,
                                               block_expert, offsets, num_padded);
  err = allow_lds(align_scatter, size_t(kWaves) * E * 4);
  if (err != hipSuccess) return err;
  align_scatter<<<q.chunks, kThreads, size_t(kWaves) * E * 4, stream>>>(ids, A, E, scratch,
                                                                          sorted_ids);
  return hipGetLastError();
}

namespace {
template <int L, int QM>
hipError_t prologue_l(const PrologueArgs& a, size_t sm, hipStream_t stream) {
  const int npl = (a.Er + L - 1) / L;
  const int64_t groups = QM != 0 ? int64_t(a.T) * a.H / 8 : 0;
  const unsigned grid = 1u + unsigned((groups + kThreads - 1) / kThreads);
#define MOE_PRO(N)                                                                 \
  do {                                                                             \
    hipError_t err = allow_lds(prologue_small<L, N, QM>, sm);                      \
    if (err != hipSuccess) return err;                                             \
    prologue_small<L, N, QM><<<grid, kThreads, sm, stream>>>(a);                   \
  } while (0)
  if (npl <= 1) MOE_PRO(1);
  else if (npl <= 2) MOE_PRO(2);
  else if (npl <= 4) MOE_PRO(4);
  else if (npl <= 8) MOE_PRO(8);
  else MOE_PRO(16);
#undef MOE_PRO
  return hipGetLastError();
}

template <int QM>
hipError_t prologue_q(const moe_problem& p, const PrologueArgs& a, size_t sm,
                      hipStream_t stream) {
  return route_in_rows(p) ? prologue_l<16, QM>(a, sm, stream) : prologue_l<64, QM>(a, sm, stream);
}
}  // namespace


bool prologue_fits(const moe_problem& p, const Plan& q) {
  return q.chunks <= 1 && p.T <= 128 && p.E_routed <= kMaxRouted;
}

hipError_t launch_prologue(const moe_problem& p, const Plan& q, const float* logits,
                           int32_t* ids, float* w, const uint16_t* x, const float* a1,
                           uint8_t* xq, void* xs, bool quantise, int32_t* sorted_ids,
                           int32_t* block_expert, int32_t* offsets, int32_t* num_padded,
                           int32_t* scratch, hipStream_t stream, bool align) {
  if (!align && !logits && !quantise) return hipSuccess;  // nothing to do
  if (!prologue_fits(p, q)) {
    // routing and quantisation in one launch when both run, then the alignment
    hipError_t err = hipSuccess;
    const bool fused = logits && quantise;
    if (fused) err = launch_route_quant(p, logits, ids, w, x, a1, xq, xs, stream);
    else if (logits) err = launch_route(p, logits, ids, w, stream);
    if (err != hipSuccess) return err;
    if (align)
      err = launch_align(p, q, ids, sorted_ids, block_expert, offsets, num_padded, scratch,
                         stream);
    if (err != hipSuccess || !quantise || fused) return err;
    return launch_quant_act(p, x, a1, xq, xs, stream);
  }
  PrologueArgs a{};
  a.logits = logits;
  a.ids_in = ids;
  a.T = p.T;
  a.Er = p.E_routed;
  a.top_k = p.top_k;
  a.n_shared = p.n_shared;
  a.shared_gate = p.shared_gate;
  a.renorm = p.renormalize;
  a.E = p.E;
  a.BM = q.BM;
  a.H = p.H;
  a.ids = ids;
  a.wts = w;
  a.sorted_ids = sorted_ids;
  a.block_expert = block_expert;
  a.offsets = offsets;
  a.npad = num_padded;
  a.align = align ? 1 : 0;
  a.x = x;
  a.a1 = a1;
  a.xq = xq;
  a.xs = xs;
  const size_t sm = size_t(kThreads) * 4 + small_tables_bytes(p.E);
  if (!quantise) return prologue_q<0>(p, a, sm, stream);
  if (p.quant == MOE_QUANT_FP8_BLOCK) return prologue_q<2>(p, a, sm, stream);
  if (quant_is_mx(p.quant)) return prologue_q<3>(p, a, sm, stream);
  return prologue_q<1>(p, a, sm, stream);
}

}  // namespace moe
