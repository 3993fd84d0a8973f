// Token dispatch ("Mixture of Experts: Router, Token Dispatch, Grouped GEMM",
// section Token Dispatch; "MoE 的算量与通信" 二.3): the T*k (token, slot) pairs are
// reordered expert-major with tokens ascending inside each expert, i.e. a stable
// sort of the pairs by expert id.  Three kernels, no host synchronisation:
//   1. per-chunk expert histogram in LDS (chunk = kPermuteChunk pairs)
//   2. one block: per-expert totals, exclusive scan -> offsets, and each chunk's
//      starting row per expert
//   3. per chunk, one wavefront walks its pairs in order 64 at a time; lanes with
//      the same expert are ranked by ballot + popcount, which keeps the order
// Up to kPermuteSmall pairs (decode-sized batches) the three steps run as one
// single-block kernel with the same results.  A fourth small kernel turns the
// offsets into the grouped GEMMs' row ranges and row-tile prefixes (routed
// experts, then the shared expert as one more group).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kHistThreads = 256;
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kHistThreads) void hist_kernel(const int32_t* ids, int R, int E,
                                                            int32_t* blockcnt) {
  __shared__ int cnt[1024];
  for (int e = threadIdx.x; e < E; e += kHistThreads) cnt[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, R - base);
  for (int i = threadIdx.x; i < n; i += kHistThreads) {
    const int e = ids[base + i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kHistThreads)
    blockcnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// exclusive prefix sum over the kScanThreads threads of one block
__device__ int block_exclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kScanThreads / 64 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < kScanThreads / 64) wave_tot[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const int before = wave > 0 ? wave_tot[wave - 1] : 0;
  __syncthreads();
  return before + x - v;
}

// exclusive prefix sums of N values per thread over the kScanThreads threads of
// one block, all N in the same pass (wave_tot holds kScanThreads/64 * N ints)
template <int N>
__device__ void block_exclusive_scan_n(const int (&v)[N], int (&ex)[N], int* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = kScanThreads / 64;
  int x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = v[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int y = __shfl_up(x[i], off);
      if (lane >= off) x[i] += y;
    }
  }
  if (lane == 63)
#pragma unroll
    for (int i = 0; i < N; ++i) wave_tot[i * NW + wave] = x[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int w = lane < NW ? wave_tot[i * NW + lane] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(w, off);
        if (lane >= off) w += y;
      }
      if (lane < NW) wave_tot[i * NW + lane] = w;  // inclusive wave totals
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) ex[i] = (wave > 0 ? wave_tot[i * NW + wave - 1] : 0) + x[i] - v[i];
  __syncthreads();
}

// counts, offsets, and blockcnt rewritten in place as each chunk's first row per
// expert.  Each expert's column of chunk counts is cut into P = kScanThreads / E
// contiguous parts, one thread each (V4-Pro's 384 x 384 counts: 47 -> 27 us with
// two parts; DeepSeek-V3's 256 experts take four): part sums, the expert totals
// and their exclusive scan, then every part rewrites its range from its own
// starting row.  Integer sums in a fixed order: the result is the one-thread-per-
// expert walk's, bit for bit.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* blockcnt, int nblk, int E,
                                                            int32_t* counts, int32_t* offsets) {
  __shared__ int wave_tot[kScanThreads / 64];
  __shared__ int part_sum[kScanThreads];  // [P][E]
  __shared__ int expert_off[kScanThreads];
  const int P = max(1, kScanThreads / E);
  const int t = threadIdx.x, e = t % E, part = t / E;
  const bool act = part < P;
  const int per = (nblk + P - 1) / P;
  const int b0 = min(nblk, part * per), b1 = min(nblk, b0 + per);
  int sum = 0;
  if (act) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += blockcnt[static_cast<int64_t>(b) * E + e];
    part_sum[part * E + e] = sum;
  }
  __syncthreads();
  int total = 0;
  if (t < E)
    for (int q = 0; q < P; ++q) total += part_sum[q * E + t];
  const int off = block_exclusive_scan(t < E ? total : 0, wave_tot);
  if (t < E) {
    counts[t] = total;
    offsets[t] = off;
    if (t == E - 1) offsets[E] = off + total;
    expert_off[t] = off;
  }
  __syncthreads();
  if (act) {
    int run = expert_off[e];
    for (int q = 0; q < part; ++q) run += part_sum[q * E + e];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      int32_t* c = blockcnt + static_cast<int64_t>(b) * E + e;
      const int n = *c;
      *c = run;
      run += n;
    }
  }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* ids, const float* w, int R,
                                                     int k, int E, const int32_t* blockbase,
                                                     int32_t* sorted_tok, float* sorted_w,
                                                     int32_t* dispatch) {
  __shared__ int base[1024];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64)
    base[e] = blockbase[static_cast<int64_t>(blockIdx.x) * E + e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t below = (1ull << lane) - 1ull;
  const int start = blockIdx.x * kPermuteChunk;
  const int end = min(start + kPermuteChunk, R);
  for (int s = start; s < end; s += 64) {
    const int pidx = s + lane;
    const bool in = pidx < end;
    const int e = in ? ids[pidx] : -1;
    const bool valid = in && e >= 0 && e < E;
    // lanes holding the same expert id
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int row = -1;
    if (valid) {
      row = base[e] + __popcll(m & below);
      sorted_tok[row] = pidx / k;
      sorted_w[row] = w[pidx];
    }
    if (in) dispatch[pidx] = row;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid && (m >> lane) == 1ull) base[e] += __popcll(m);  // last lane of its expert
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// All three steps for R <= kPermuteSmall pairs in one block: LDS histogram,
// scan, then wavefront 0 walks the pairs in order exactly as scatter_kernel
__global__ __launch_bounds__(kScanThreads) void permute_small_kernel(
    const int32_t* ids, const float* w, int R, int k, int E, int32_t* counts, int32_t* offsets,
    int32_t* sorted_tok, float* sorted_w, int32_t* dispatch) {
  __shared__ int cnt[1024];
  __shared__ int base[1024];
  __shared__ int wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  for (int i = tid; i < R; i += kScanThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int total = tid < E ? cnt[tid] : 0;
  const int off = block_exclusive_scan(total, wave_tot);
  if (tid < E) {
    counts[tid] = total;
    offsets[tid] = off;
    if (tid == E - 1) offsets[E] = off + total;
    base[tid] = off;
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int s = 0; s < R; s += 64) {
    const int pidx = s + lane;
    const bool in = pidx < R;
    const int e = in ? ids[pidx] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int row = -1;
    if (valid) {
      row = base[e] + __popcll(m & below);
      sorted_tok[row] = pidx / k;
      sorted_w[row] = w[pidx];
    }
    if (in) dispatch[pidx] = row;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid && (m >> lane) == 1ull) base[e] += __popcll(m);  // last lane of its expert
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Routed rows are clamped to [0, routed_limit] so that caller-given offsets can
// never send the GEMMs past the dispatch arrays.
__global__ __launch_bounds__(kScanThreads) void build_tiles_kernel(const int32_t* offsets, int E,
                                                                   int routed_limit,
                                                                   int shared_begin,
                                                                   int shared_rows, int32_t* groups,
                                                                   int32_t* tile_prefix,
                                                                   int32_t* sorted_tok) {
  constexpr int H = kNumTileLists;
  __shared__ int wave_tot[kScanThreads / 64 * H];
  __shared__ int pass_total[H];
  const int G = E + (shared_rows > 0 ? 1 : 0);
  int32_t* g_begin = groups;
  int32_t* g_end = groups + G;
  // G <= 1025: thread i handles groups i and (for i == 0) the shared group E;
  // the prefixes of all tile heights come from one scan per pass
  int carry[H];
#pragma unroll
  for (int h = 0; h < H; ++h) carry[h] = 0;
  for (int g0 = 0; g0 < G; g0 += kScanThreads) {
    const int g = g0 + threadIdx.x;
    int b = 0, en = 0;
    if (g < E) {
      b = min(max(offsets[g], 0), routed_limit);
      en = min(max(offsets[g + 1], b), routed_limit);
    } else if (g < G) {
      b = shared_begin;
      en = shared_begin + shared_rows;
    }
    const int rows = en - b;
    if (g < G) {
      g_begin[g] = b;
      g_end[g] = en;
    }
    int tiles[H], ex[H];
#pragma unroll
    for (int h = 0; h < H; ++h) tiles[h] = g < G ? list_tiles(h, rows) : 0;
    block_exclusive_scan_n<H>(tiles, ex, wave_tot);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (g < G) tile_prefix[h * (G + 1) + g] = carry[h] + ex[h];
      // total of this pass: last thread's exclusive prefix + its own count
      if (threadIdx.x == kScanThreads - 1) pass_total[h] = ex[h] + tiles[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < H; ++h) carry[h] += pass_total[h];
    __syncthreads();
  }
  if (threadIdx.x == 0)
#pragma unroll
    for (int h = 0; h < H; ++h) tile_prefix[h * (G + 1) + G] = carry[h];
  for (int t = threadIdx.x; t < shared_rows; t += kScanThreads) sorted_tok[shared_begin + t] = t;
}

}  // namespace

hipError_t launch_permute(const moe_config& c, const int32_t* ids, const float* weights,
                          int32_t* blockcnt, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_tok, float* sorted_w, int32_t* dispatch,
                          hipStream_t s) {
  const int R = c.T * c.k;
  const int nblk = ceil_div(R, kPermuteChunk);
  if (R <= kPermuteSmall) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kScanThreads), 0, s, ids, weights, R,
                       c.k, c.E, counts, offsets, sorted_tok, sorted_w, dispatch);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(kHistThreads), 0, s, ids, R, c.E, blockcnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blockcnt, nblk, c.E, counts,
                     offsets);
  hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(64), 0, s, ids, weights, R, c.k, c.E,
                     blockcnt, sorted_tok, sorted_w, dispatch);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int routed_limit, int shared_begin,
                              int shared_rows, int32_t* groups, int32_t* tile_prefix,
                              int32_t* sorted_tok, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kScanThreads), 0, s, offsets, E,
                     routed_limit, shared_begin, shared_rows, groups, tile_prefix, sorted_tok);
  return hipGetLastError();
}

}  // namespace moe
