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
// same expert are found with one ballot per distinct expert, and a lane's rank
// is the number of such lanes below it.  Ranks across the 16 waves of a
// workgroup add the earlier waves' counts; across workgroups (chunks of 1024
// assignments) a per-chunk histogram is scanned per expert.
//   A <= 1024 : one kernel, one workgroup (decode sizes, one launch);
//   A >  1024 : histogram -> scan -> scatter, three launches.
#include "moe_device.hpp"
#include "moe_launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = kAlignChunk;  // 1024 threads, 16 waves
constexpr int kWaves = kThreads / 64;

// Rank of this lane among the active lanes with the same expert below it, and
// the number of active lanes with that expert.
__device__ __forceinline__ void match_rank(int e, bool valid, int& rank, int& cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  uint64_t todo = __ballot(valid);
  rank = 0;
  cnt = 0;
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int ev = __shfl(e, leader, 64);
    const uint64_t same = __ballot(valid && e == ev);
    if (valid && e == ev) {
      rank = __popcll(same & below);
      cnt = __popcll(same);
    }
    todo &= ~same;
  }
}

// Exclusive prefix sum over the 1024 threads of the block; returns this
// thread's prefix and writes the block total to *total.  `tmp` holds kWaves+1
// ints of shared memory.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = tmp[w];
      tmp[w] = run;
      run += c;
    }
    tmp[kWaves] = run;
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
__device__ void fill_tail(const int* cnt, const int* off, int E, int BM, int A,
                          int32_t* sorted_ids, int32_t* block_expert) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    for (int r = off[e] + cnt[e]; r < off[e + 1]; ++r) sorted_ids[r] = A;
    for (int b = off[e] / BM; b < off[e + 1] / BM; ++b) block_expert[b] = e;
  }
}

}  // namespace

// One workgroup for A <= 1024: count, offsets, stable scatter, tails.
// Shared memory: cnt[E], off[E+1], wcnt[kWaves][E], tmp[kWaves+1].
__global__ __launch_bounds__(kThreads) void align_small(const int32_t* __restrict__ ids,
                                                        int A, int E, int BM,
                                                        int32_t* __restrict__ sorted_ids,
                                                        int32_t* __restrict__ block_expert,
                                                        int32_t* __restrict__ g_offsets,
                                                        int32_t* __restrict__ g_npad) {
  extern __shared__ int smem[];
  int* cnt = smem;
  int* off = cnt + E;
  int* wcnt = off + E + 1;
  int* tmp = wcnt + kWaves * E;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  const int f = threadIdx.x;
  const int e = f < A ? ids[f] : -1;
  const bool valid = f < A && e >= 0 && e < E;
  int rank, c;
  match_rank(e, valid, rank, c);
  if (valid && rank == 0) wcnt[wave * E + e] = c;
  __syncthreads();
  // per expert: total count, and the earlier waves' counts in place
  for (int x = threadIdx.x; x < E; x += kThreads) {
    int run = 0;
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
// (in place in hist), tails.  Shared memory: cnt[E], off[E+1], tmp.
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
  for (int x = threadIdx.x; x < E; x += kThreads) {
    int run = 0;
    for (int c = 0; c < chunks; ++c) run += hist[size_t(c) * E + x];
    cnt[x] = run;
  }
  __syncthreads();
  padded_offsets(cnt, off, E, BM, tmp, g_offsets, g_npad);
  for (int x = threadIdx.x; x < E; x += kThreads) {
    int run = off[x];
    for (int c = 0; c < chunks; ++c) {
      const int v = hist[size_t(c) * E + x];
      hist[size_t(c) * E + x] = run;
      run += v;
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
  match_rank(e, valid, rank, c);
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
    const size_t sm = (size_t(E) + (E + 1) + size_t(kWaves) * E + kWaves + 1) * 4;
    align_small<<<1, kThreads, sm, stream>>>(ids, A, E, BM, sorted_ids, block_expert, offsets,
                                             num_padded);
    return hipGetLastError();
  }
  align_count<<<q.chunks, kThreads, size_t(E) * 4, stream>>>(ids, A, E, scratch);
  const size_t sm_scan = (size_t(E) + (E + 1) + kWaves + 1) * 4;
  align_scan<<<1, kThreads, sm_scan, stream>>>(scratch, q.chunks, A, E, BM, sorted_ids,
                                               block_expert, offsets, num_padded);
  align_scatter<<<q.chunks, kThreads, size_t(kWaves) * E * 4, stream>>>(ids, A, E, scratch,
                                                                          sorted_ids);
  return hipGetLastError();
}

}  // namespace moe
