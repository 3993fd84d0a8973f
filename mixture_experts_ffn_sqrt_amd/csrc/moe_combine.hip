// Weighted combine ("Mixture of Experts: Router, Token Dispatch, Grouped GEMM",
// section Token Combine; "MoE 的算量与通信" 二.2 weighted sum plus shared experts;
// "DeepSeek-V4 MoE" 四, y_A = 0.7 E1(x_A) + 0.3 E5(x_A)):
//   out[t] = sum_j w[t,j] * Y[dispatch[t,j]]  (+ shared[t])
// Each token gathers its k dispatch rows in slot order and sums in float32, so
// the result does not depend on scheduling (no atomics).  A block covers one
// token and a chunk of kThreads * 16 bytes of its row (so that a small batch
// still spreads over the chip); each thread issues all of its row loads before
// it sums them.
//
// The expert rows are read once.  When they are more than the 256 MB Infinity
// Cache holds, the loads carry the non-temporal hint: V4-Pro's combine (1.6 GB
// of rows) 0.338 -> 0.293 ms, DeepSeek-V3's 0.220 -> 0.193 ms; batches whose
// rows the Infinity Cache still holds from GEMM 2 read them faster without it
// (Mixtral 18.4 vs 20.8 us).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 128;
constexpr int kMaxK = 16;

// 16 bytes of TE: raw load, and its float lanes
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;

// 16 bytes at p, non-temporal when NT
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* p) {
  if constexpr (NT) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

template <typename TE>
struct Vec;
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  template <bool NT>
  __device__ static uint4 load(const void* p) { return load16<NT>(p); }
  __device__ static void unpack(const uint4& v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(void* p, const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  template <bool NT>
  __device__ static uint4 load(const void* p) { return load16<NT>(p); }
  __device__ static void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ static void store(void* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

template <typename TE, bool NT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const TE* Y, const int32_t* dispatch,
                                                           const float* w, const TE* shared,
                                                           TE* out, int k, int d) {
  constexpr int V = Vec<TE>::N;
  const int t = blockIdx.x;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * V;
  if (c >= d) return;
  int rows[kMaxK];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = j < k ? dispatch[static_cast<int64_t>(t) * k + j] : -1;
    wt[j] = j < k ? w[static_cast<int64_t>(t) * k + j] : 0.0f;
  }
  uint4 raw[kMaxK + 1];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (rows[j] >= 0) raw[j] = Vec<TE>::template load<NT>(Y + static_cast<int64_t>(rows[j]) * d + c);
  if (shared) raw[kMaxK] = Vec<TE>::template load<NT>(shared + static_cast<int64_t>(t) * d + c);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (rows[j] < 0) continue;
    float x[V];
    Vec<TE>::unpack(raw[j], x);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += wt[j] * x[i];
  }
  if (shared) {
    float x[V];
    Vec<TE>::unpack(raw[kMaxK], x);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += x[i];
  }
  Vec<TE>::store(out + static_cast<int64_t>(t) * d + c, acc);
}

}  // namespace

hipError_t launch_combine(const moe_config& c, const void* expert_out, const int32_t* dispatch,
                          const float* weights, const void* shared_out, void* out,
                          hipStream_t s) {
  const int es = c.dtype == MOE_F32 ? 4 : 2;
  const int64_t row_bytes =
      (int64_t)c.T * (c.k + (shared_out ? 1 : 0)) * c.d * es;  // expert rows read
  const bool nt = row_bytes > kInfinityCacheBytes;
  if (c.dtype == MOE_F32) {
    auto kern = nt ? combine_kernel<float, true> : combine_kernel<float, false>;
    hipLaunchKernelGGL(kern, dim3(c.T, ceil_div(c.d, kThreads * 4)), dim3(kThreads), 0, s,
                       static_cast<const float*>(expert_out), dispatch, weights,
                       static_cast<const float*>(shared_out), static_cast<float*>(out), c.k, c.d);
  } else {
    auto kern = nt ? combine_kernel<uint16_t, true> : combine_kernel<uint16_t, false>;
    hipLaunchKernelGGL(kern, dim3(c.T, ceil_div(c.d, kThreads * 8)), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(expert_out), dispatch, weights,
                       static_cast<const uint16_t*>(shared_out), static_cast<uint16_t*>(out),
                       c.k, c.d);
  }
  return hipGetLastError();
}

}  // namespace moe
