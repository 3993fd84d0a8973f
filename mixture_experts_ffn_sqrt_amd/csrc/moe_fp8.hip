// FP8 (E4M3) experts: the 1x128 and 128x128 quantizers and the launchers of
// the FP8 grouped GEMMs ("MoE 架构与路由策略", FP4 QAT section and table
// dsv4-moe-fp4-vs-fp8: E4M3, one scale per 128x128 weight tile; table
// dsv4-moe-stages: the FP8 cast after the activation; "MoE 的算量与通信" 五.2:
// FP8 dispatch of the hidden rows).
//
// A group of values x gets the power-of-two scale s = 2^e, the smallest with
// max |x| <= 448 s (e >= -126; s = 1 for an all-zero group), and the codes
// E4M3(x / s), nearest-even (the division by s is exact).
#include "moe_gemm_fp8.h"

namespace moe {
namespace {
using namespace gemm;

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wavefront per (row, 128-column group): two elements per lane.
template <typename TIn>
__global__ __launch_bounds__(256) void quantize_rows_kernel(int n, int K, const TIn* x,
                                                            uint8_t* q, float* scales) {
  const int G = K / 128;
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= (int64_t)n * G) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = job / G;
  const int g = (int)(job - row * G);
  const int64_t base = row * K + g * 128 + 2 * lane;
  const float v0 = load_in(x, base), v1 = load_in(x, base + 1);
  const int e = fp8_scale_exp(wave_max64(fmaxf(fabsf(v0), fabsf(v1))));
  const float inv = ldexpf(1.0f, -e);
  const uint32_t c0 = e4m3_code(v0 * inv), c1 = e4m3_code(v1 * inv);
  *reinterpret_cast<uint16_t*>(q + base) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) scales[row * G + g] = ldexpf(1.0f, e);
}

// One block of 256 threads per 128x128 tile: thread t covers 64 consecutive
// elements of tile row t / 2.
template <typename TIn>
__global__ __launch_bounds__(256) void quantize_blocks_kernel(int R, int C, const TIn* w,
                                                              uint8_t* q, float* scales) {
  __shared__ float wmax[4];
  const int GC = C / 128;
  const int br = blockIdx.x / GC, bc = blockIdx.x % GC;
  const int t = threadIdx.x;
  const int64_t base = (int64_t)(br * 128 + (t >> 1)) * C + bc * 128 + (t & 1) * 64;
  float m = 0.0f;
  for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(load_in(w, base + i)));
  m = wave_max64(m);
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  const int e = fp8_scale_exp(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
  const float inv = ldexpf(1.0f, -e);
  for (int i = 0; i < 64; i += 4) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) word |= e4m3_code(load_in(w, base + i + j) * inv) << (8 * j);
    *reinterpret_cast<uint32_t*>(q + base + i) = word;
  }
  if (t == 0) scales[(int64_t)br * GC + bc] = ldexpf(1.0f, e);
}

template <int BM, int BN, int WM, int WN, int EPI, int ST>
hipError_t launch_fp8(const Fp8Args& q, int m_tiles_bound, hipStream_t s) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDS = ST * ((BM + BN) * 128 + (BM > 64 ? BM : 64) * 4 + 256);
  const int grid = m_tiles_bound * q.g.n_tiles;
  if (grid <= 0) return hipSuccess;
  auto kern = grouped_gemm_fp8<BM, BN, WM, WN, EPI, ST>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), LDS, s, q);
  return hipGetLastError();
}

int tile_bound8(int64_t rows, int groups, int bm) {
  const int64_t ne = rows < groups ? rows : groups;
  return (int)((rows + ne * (bm - 1)) / bm);
}

// 32-row streaming tiles when experts have a few rows each (decode), else
// 256x256 tiles (the same rule as the bf16 experts)
bool small_rows(const Fp8FfnArgs& a) {
  return a.rows_bound / (a.n_groups > 0 ? a.n_groups : 1) < 48;
}

}  // namespace

hipError_t launch_quantize_rows(int n, int K, int in_dtype, const void* x, uint8_t* q,
                                float* scales, hipStream_t s) {
  const int64_t jobs = (int64_t)n * (K / 128);
  if (jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)((jobs + 3) / 4));
  if (in_dtype == MOE_F32)
    hipLaunchKernelGGL(quantize_rows_kernel<float>, grid, dim3(256), 0, s, n, K,
                       static_cast<const float*>(x), q, scales);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, grid, dim3(256), 0, s, n, K,
                       static_cast<const uint16_t*>(x), q, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_blocks(int R, int C, int in_dtype, const void* w, uint8_t* q,
                                  float* scales, hipStream_t s) {
  const int64_t tiles = (int64_t)(R / 128) * (C / 128);
  if (tiles == 0) return hipSuccess;
  if (in_dtype == MOE_F32)
    hipLaunchKernelGGL(quantize_blocks_kernel<float>, dim3((unsigned)tiles), dim3(256), 0, s, R,
                       C, static_cast<const float*>(w), q, scales);
  else
    hipLaunchKernelGGL(quantize_blocks_kernel<uint16_t>, dim3((unsigned)tiles), dim3(256), 0, s,
                       R, C, static_cast<const uint16_t*>(w), q, scales);
  return hipGetLastError();
}

hipError_t launch_expert_up_fp8(const moe_config& c, const Fp8FfnArgs& a, hipStream_t s) {
  const int64_t d = c.d, F = c.d_ff;
  Fp8Args q{};
  GemmArgs& g = q.g;
  g.A = reinterpret_cast<const char*>(a.xq);
  g.a_rows = a.sorted_tok;
  g.lda = d;
  g.B = reinterpret_cast<const char*>(a.w13q);
  g.B_last = reinterpret_cast<const char*>(a.w13q_last);
  g.b_group = 2 * F * d;
  g.ldb = d;
  g.N = c.d_ff;
  g.up_row = c.d_ff;
  g.K = c.d;
  g.g_begin = a.g_begin;
  g.g_end = a.g_end;
  g.G = a.n_groups;
  g.C = reinterpret_cast<char*>(a.hq);
  g.ldc = F;
  g.n_tiles = c.d_ff / 128;
  g.a_bytes = (uint32_t)((int64_t)c.T * d);
  g.b_bytes = (uint32_t)(2 * F * d);
  q.a_scale = a.xs;
  q.b_scale = a.w13s;
  q.b_scale_last = a.w13s_last;
  q.b_scale_group = (2 * F / 128) * (d / 128);
  q.c_scale = a.hs;
  q.ldcs = c.d_ff / 128;
  q.as_bytes = (uint32_t)((int64_t)c.T * (d / 128) * 4);
  if (small_rows(a)) {
    g.tile_prefix = a.tile_prefix + tile_height_index(32) * (a.n_groups + 1);
    return launch_fp8<32, 256, 1, 4, EPI_SWIGLU8, 4>(q, tile_bound8(a.rows_bound, a.n_groups, 32), s);
  }
  g.tile_prefix = a.tile_prefix + tile_height_index(256) * (a.n_groups + 1);
  return launch_fp8<256, 256, 4, 4, EPI_SWIGLU8, 2>(q, tile_bound8(a.rows_bound, a.n_groups, 256), s);
}

hipError_t launch_expert_down_fp8(const moe_config& c, const Fp8FfnArgs& a, hipStream_t s) {
  const int64_t d = c.d, F = c.d_ff;
  Fp8Args q{};
  GemmArgs& g = q.g;
  g.A = reinterpret_cast<const char*>(a.hq);
  g.a_rows = nullptr;
  g.lda = F;
  g.B = reinterpret_cast<const char*>(a.w2q);
  g.B_last = reinterpret_cast<const char*>(a.w2q_last);
  g.b_group = d * F;
  g.ldb = F;
  g.N = c.d;
  g.K = c.d_ff;
  g.g_begin = a.g_begin;
  g.g_end = a.g_end;
  g.G = a.n_groups;
  g.C = static_cast<char*>(a.Y);
  g.ldc = d * 2;
  g.a_bytes = (uint32_t)((int64_t)a.rows_bound * F);
  g.b_bytes = (uint32_t)(d * F);
  q.a_scale = a.hs;
  q.b_scale = a.w2s;
  q.b_scale_last = a.w2s_last;
  q.b_scale_group = (d / 128) * (F / 128);
  q.as_bytes = (uint32_t)((int64_t)a.rows_bound * (F / 128) * 4);
  if (small_rows(a)) {
    g.n_tiles = ceil_div(c.d, 128);
    g.tile_prefix = a.tile_prefix + tile_height_index(32) * (a.n_groups + 1);
    return launch_fp8<32, 128, 1, 4, EPI_STORE, 4>(q, tile_bound8(a.rows_bound, a.n_groups, 32), s);
  }
  g.n_tiles = ceil_div(c.d, 256);
  g.tile_prefix = a.tile_prefix + tile_height_index(256) * (a.n_groups + 1);
  return launch_fp8<256, 256, 4, 4, EPI_STORE, 2>(q, tile_bound8(a.rows_bound, a.n_groups, 256), s);
}

}  // namespace moe
