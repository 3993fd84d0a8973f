// FP8 (E4M3) experts: the 1x128 and 128x128 quantizers and the launchers of
// the FP8 grouped GEMMs ("MoE 架构与路由策略", FP4 QAT section and table
// dsv4-moe-fp4-vs-fp8: E4M3, one scale per 128x128 weight tile; table
// dsv4-moe-stages: the FP8 cast after the activation; "MoE 的算量与通信" 五.2:
// FP8 dispatch of the hidden rows).
//
// A group of values x gets the power-of-two scale s = 2^e, the smallest with
// max |x| <= 448 s (e >= -126; s = 1 for an all-zero group), and the codes
// E4M3(x / s), nearest-even (the division by s is exact).
//
// MXFP4 weights (the same page's FP4 QAT section: E2M1 with one scale per 1x32
// sub-block): each 32 consecutive elements of a weight row get s = 2^e, the
// smallest with max |x| <= 6 s (e >= -126; 1 for an all-zero block), stored as
// the E8M0 byte e + 127, and the codes E2M1(x / s), nearest-even, two per byte
// with element 2j in the low nibble.  Scales are stored K-block-major
// ([C/128, R, 4] per matrix) so that one K block's scales of consecutive rows
// are contiguous for the GEMMs' loads.
#include "moe_gemm_fp8.h"

namespace moe {
namespace {

// workgroups of a grid-strided quantizer launch (256 per CU)
constexpr int64_t kQuantizeMaxGrid = 65536;
// most workgroups of 256 threads in one dispatch (2^32 work-items)
constexpr int64_t kMaxWorkgroups256 = (int64_t)1 << 24;

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

// 8 consecutive elements of a row as floats (16-byte loads)
template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// One wavefront per 512 consecutive elements of a row (four 128-column groups,
// fewer at a row's end): lane l holds elements 8l .. 8l+7, so group l/16 is
// reduced over 16 lanes.  Scales are stored K-block-major, [K/128, n], so that
// one group's scales of consecutive rows are contiguous for the GEMMs' loads.
template <typename TIn>
__global__ __launch_bounds__(256) void quantize_rows_kernel(int n, int K, const TIn* x,
                                                            uint8_t* q, float* scales) {
  const int JR = (K + 511) / 512;  // jobs per row
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= (int64_t)n * JR) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = job / JR;
  const int col = (int)(job - row * JR) * 512 + 8 * lane;
  const bool in = col < K;  // K is a multiple of 128: whole groups are in or out
  float v[8];
  if (in) {
    load8(x + row * K + col, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
  if (!in) return;
  const int e = fp8_scale_exp(m);
  const float inv = ldexpf(1.0f, -e);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 |= e4m3_code(v[i] * inv) << (8 * i);
    w1 |= e4m3_code(v[4 + i] * inv) << (8 * i);
  }
  *reinterpret_cast<uint2*>(q + row * K + col) = make_uint2(w0, w1);
  if ((lane & 15) == 0) scales[(int64_t)(col / 128) * n + row] = ldexpf(1.0f, e);
}

// E2M1 code of v, nearest with ties to the even mantissa, saturated to +-6: the
// magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6, and the code counts the midpoints
// below |v| (a midpoint that is a tie rounds to the even neighbour: strict
// comparison where the lower neighbour is even, inclusive where it is odd)
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.0f);
  return c | (signbit(v) ? 8u : 0u);
}

// Exponent of an MXFP4 block scale: the smallest e with amax <= 6 * 2^e.  With
// amax = m * 2^k, m in [0.5, 1), and 6 = 0.75 * 2^3: e = k - 3 if m <= 0.75,
// else k - 2; at least -126; 0 for an all-zero block.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (amax == 0.0f) return 0;
  int k;
  const float m = frexpf(amax, &k);
  const int e = k - 3 + (m > 0.75f ? 1 : 0);
  return e < -126 ? -126 : e;
}

// 16 lanes per 32-element block (two elements each, one output byte), four
// blocks per wavefront, blocks numbered over the row-major [n_mat * R, C]
// input (a row's C/32 blocks are consecutive).  Codes go to the paired-row
// layout: element (r, c) of matrix m at byte m*R*C/2 + (r/2)*C + (c/128)*128 +
// (r%2)*64 + (c%128)/2.  Scale of block b of row r of matrix m goes to
// scales[m][b / 4][r][b % 4].  A workgroup takes 16 blocks
// per pass and strides over the grid: a dispatch's work-item count is 32-bit,
// and all the experts' weights of a large layer (384 x 6144 x 7168 elements)
// would need more work-items than that at one thread per two elements.
template <typename TIn>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(int64_t nblocks, int R, int C,
                                                             const TIn* w, uint8_t* q,
                                                             uint8_t* scales) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int GB = C / 32;
  // the pass condition is the same for the whole workgroup, so every lane of
  // a 16-lane group takes part in its shuffles
  for (int64_t pass = blockIdx.x; pass * 16 < nblocks; pass += gridDim.x) {
    const int64_t blk = (pass * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const bool ok = blk < nblocks;
    const int64_t base = blk * 32 + 2 * sub;
    const float v0 = ok ? load_in(w, base) : 0.0f, v1 = ok ? load_in(w, base + 1) : 0.0f;
    float m = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
    if (!ok) continue;
    const int e = mx_scale_exp(m);
    const float inv = ldexpf(1.0f, -e);
    const int64_t row = blk / GB;  // over all matrices
    const int b = (int)(blk - row * GB);
    const int64_t mat = row / R, r = row - mat * R;
    // codes of rows 2i and 2i+1 share 128-byte lines per 128-element K block
    const int c = b * 32 + 2 * sub;  // element column of v0
    q[mat * ((int64_t)R * C / 2) + (r >> 1) * C + (c >> 7) * 128 + (r & 1) * 64 + ((c & 127) >> 1)] =
        (uint8_t)(e2m1_code(v0 * inv) | (e2m1_code(v1 * inv) << 4));
    if (sub == 0) scales[((mat * (C / 128) + b / 4) * R + r) * 4 + (b & 3)] = (uint8_t)(e + 127);
  }
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

template <int BM, int BN, int WM, int WN, int EPI, int ST, int WF = WF_E4M3, int SCHED = 0>
hipError_t launch_fp8(const Fp8Args& q, int m_tiles_bound, hipStream_t s) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDS = ST * fp8_stage_bytes<BM, BN, WF>();
  const int grid = xcd_grid((int64_t)m_tiles_bound * q.g.n_tiles);
  if (grid <= 0) return hipSuccess;
  auto kern = grouped_gemm_fp8<BM, BN, WM, WN, EPI, ST, WF, SCHED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), LDS, s, q);
  return hipGetLastError();
}

// The two tile lists of a skewed prefill-shaped batch in one launch
// (grouped_gemm_fp8_split): Small's 32-row streaming tiles of `small` on the
// first kSmallGroupBlocks blocks, one Big tile of `big` on each later block.
template <class Big, class Small, int EPI, int WF>
hipError_t launch_fp8_split(const Fp8Args& big, int big_m_tiles, const Fp8Args& small,
                            hipStream_t s) {
  constexpr int LDS_B = Big::ST * fp8_stage_bytes<Big::BM, Big::BN, WF>();
  constexpr int LDS_S = Small::ST * fp8_stage_bytes<32, Small::BN, WF>();
  constexpr int LDS = LDS_B > LDS_S ? LDS_B : LDS_S;
  const int grid = kSmallGroupBlocks + xcd_grid((int64_t)big_m_tiles * big.g.n_tiles);
  auto kern = grouped_gemm_fp8_split<Big, Small, EPI, WF>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * Big::WAVES), LDS, s, big, small,
                     kSmallGroupBlocks);
  return hipGetLastError();
}

int tile_bound8(int64_t rows, int groups, int bm) {
  const int64_t ne = rows < groups ? rows : groups;
  return (int)((rows + ne * (bm - 1)) / bm);
}

// 32-row streaming tiles when experts have a few rows each (decode), else
// 256x256 tiles (288x256 for the down GEMM of large groups; 128x256 for the
// other MXFP4 GEMMs, two blocks per CU; the E4M3 up GEMM stays at 256 rows, where
// the bf16 one takes 288: 288-row E4M3 up tiles measured 1.5% faster to 5%
// slower across the prefill shapes).  The decode tiles keep
// short LDS rings (2-3 stages, 40-80 KB) so that two to four blocks share a CU
// and one block's pipeline fill and epilogue overlap another's streaming:
// measured faster than one block per CU with a 4-12 stage ring.
bool small_rows(const Fp8FfnArgs& a) {
  return a.rows_bound / (a.n_groups > 0 ? a.n_groups : 1) < 48;
}

}  // namespace

hipError_t launch_quantize_rows(int n, int K, int in_dtype, const void* x, uint8_t* q,
                                float* scales, hipStream_t s) {
  const int64_t jobs = (int64_t)n * ((K + 511) / 512);
  if (jobs == 0) return hipSuccess;
  if ((jobs + 3) / 4 > kMaxWorkgroups256) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((jobs + 3) / 4));
  if (in_dtype == MOE_F32)
    hipLaunchKernelGGL(quantize_rows_kernel<float>, grid, dim3(256), 0, s, n, K,
                       static_cast<const float*>(x), q, scales);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, grid, dim3(256), 0, s, n, K,
                       static_cast<const uint16_t*>(x), q, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(int n_mat, int R, int C, int in_dtype, const void* w, uint8_t* q,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = (int64_t)n_mat * R * (C / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t passes = (nblocks + 15) / 16;
  const dim3 grid((unsigned)(passes < kQuantizeMaxGrid ? passes : kQuantizeMaxGrid));
  if (in_dtype == MOE_F32)
    hipLaunchKernelGGL(quantize_mxfp4_kernel<float>, grid, dim3(256), 0, s, nblocks, R, C,
                       static_cast<const float*>(w), q, scales);
  else
    hipLaunchKernelGGL(quantize_mxfp4_kernel<uint16_t>, grid, dim3(256), 0, s, nblocks, R, C,
                       static_cast<const uint16_t*>(w), q, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_blocks(int R, int C, int in_dtype, const void* w, uint8_t* q,
                                  float* scales, hipStream_t s) {
  const int64_t tiles = (int64_t)(R / 128) * (C / 128);
  if (tiles == 0) return hipSuccess;
  if (tiles > kMaxWorkgroups256) return hipErrorInvalidConfiguration;
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
  const bool mx = a.wfmt == kWeightMxfp4;
  Fp8Args q{};
  GemmArgs& g = q.g;
  g.A = reinterpret_cast<const char*>(a.xq);
  g.a_rows = a.sorted_tok;
  g.lda = d;
  g.B = reinterpret_cast<const char*>(a.w13q);
  g.B_last = reinterpret_cast<const char*>(a.w13q_last);
  g.ldb = mx ? d / 2 : d;
  g.b_group = 2 * F * g.ldb;
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
  g.b_bytes = (uint32_t)g.b_group;
  q.a_scale = a.xs;
  q.b_scale = a.w13s;
  q.b_scale_last = a.w13s_last;
  q.b_scale_group = mx ? 2 * F * (d / 32) : (2 * F / 128) * (d / 128) * 4;
  q.b_scale_kstride = mx ? (uint32_t)(2 * F * 4) : 4u;
  q.c_scale = a.hs;
  q.ldcs = a.rows_bound;
  q.as_bytes = (uint32_t)((int64_t)c.T * (d / 128) * 4);
  q.as_kstride = (uint32_t)(c.T * 4);
  if (small_rows(a)) {
    g.tile_prefix = a.tile_prefix + tile_height_index(32) * (a.n_groups + 1);
    const int mt = tile_bound8(a.rows_bound, a.n_groups, 32);
    return mx ? launch_fp8<32, 256, 1, 4, EPI_SWIGLU8, 3, WF_MXFP4>(q, mt, s)
              : launch_fp8<32, 256, 1, 4, EPI_SWIGLU8, 2>(q, mt, s);
  }
  if (mx) {
    // 128x256 tiles (8 waves of 64 x 64) in two 34 KB stages, so that two
    // blocks share a CU and one block's SwiGLU + FP8-cast epilogue (VALU work
    // with the matrix cores idle) overlaps the other's main loop: up GEMM
    // V4-Pro 4.42 -> 3.97 ms, Mixtral 0.97 -> 0.92 ms, DeepSeek-V3 2.23 ->
    // 2.07 ms against one block of 256x256 per CU.  (An E4M3 tile of the same
    // shape needs 100 KB: one block per CU.)
    // (these tiles keep the groups of a few rows: splitting those off onto
    // streaming tiles in the same launch, as for E4M3 below, measured neutral
    // on V4-Pro's up GEMM and 3% slower on its down GEMM)
    g.tile_prefix = a.tile_prefix + tile_height_index(128) * (a.n_groups + 1);
    return launch_fp8<128, 256, 2, 4, EPI_SWIGLU8, 2, WF_MXFP4>(
        q, tile_bound8(a.rows_bound, a.n_groups, 128), s);
  }
  const int mt = tile_bound8(a.rows_bound, a.n_groups, 256);
  // groups of a few rows on a skewed load: one 32-row streaming tile each,
  // walked by a few blocks of the same launch as the 256-row tiles (V4-Pro's
  // up GEMM 5.03-5.05 -> 4.91-4.92 ms; DeepSeek-V3, without such groups,
  // unchanged).  Scheduled main loop (0-2% faster).
  if (split_small_groups(a.rows_bound, a.n_groups)) {
    Fp8Args qs = q;
    qs.g.tile_prefix = a.tile_prefix + kListSmall32 * (a.n_groups + 1);
    g.tile_prefix = a.tile_prefix + kListLarge256 * (a.n_groups + 1);
    return launch_fp8_split<Fp8Tile<256, 256, 4, 2, 2, 1>, Fp8Tile<32, 256, 1, 4, 2>, EPI_SWIGLU8,
                            WF_E4M3>(q, mt, qs, s);
  }
  g.tile_prefix = a.tile_prefix + tile_height_index(256) * (a.n_groups + 1);
  return launch_fp8<256, 256, 4, 2, EPI_SWIGLU8, 2, WF_E4M3, 1>(q, mt, s);
}

hipError_t launch_expert_down_fp8(const moe_config& c, const Fp8FfnArgs& a, hipStream_t s) {
  const int64_t d = c.d, F = c.d_ff;
  const bool mx = a.wfmt == kWeightMxfp4;
  Fp8Args q{};
  GemmArgs& g = q.g;
  g.A = reinterpret_cast<const char*>(a.hq);
  g.a_rows = nullptr;
  g.lda = F;
  g.B = reinterpret_cast<const char*>(a.w2q);
  g.B_last = reinterpret_cast<const char*>(a.w2q_last);
  g.ldb = mx ? F / 2 : F;
  g.b_group = d * g.ldb;
  g.N = c.d;
  g.K = c.d_ff;
  g.g_begin = a.g_begin;
  g.g_end = a.g_end;
  g.G = a.n_groups;
  g.C = static_cast<char*>(a.Y);
  g.ldc = d * 2;
  g.a_bytes = (uint32_t)((int64_t)a.rows_bound * F);
  g.b_bytes = (uint32_t)g.b_group;
  q.a_scale = a.hs;
  q.b_scale = a.w2s;
  q.b_scale_last = a.w2s_last;
  q.b_scale_group = mx ? d * (F / 32) : (d / 128) * (F / 128) * 4;
  q.b_scale_kstride = mx ? (uint32_t)(d * 4) : 4u;
  q.as_bytes = (uint32_t)((int64_t)a.rows_bound * (F / 128) * 4);
  q.as_kstride = (uint32_t)(a.rows_bound * 4);
  if (small_rows(a)) {
    g.n_tiles = ceil_div(c.d, 128);
    g.tile_prefix = a.tile_prefix + tile_height_index(32) * (a.n_groups + 1);
    const int mt = tile_bound8(a.rows_bound, a.n_groups, 32);
    return mx ? launch_fp8<32, 128, 1, 4, EPI_STORE, 3, WF_MXFP4>(q, mt, s)
              : launch_fp8<32, 128, 1, 4, EPI_STORE, 3>(q, mt, s);
  }
  g.n_tiles = ceil_div(c.d, 256);
  if (tall_down_tiles(a.rows_bound, a.n_groups)) {
    g.tile_prefix = a.tile_prefix + tile_height_index(288) * (a.n_groups + 1);
    const int mt = tile_bound8(a.rows_bound, a.n_groups, 288);
    return mx ? launch_fp8<288, 256, 3, 4, EPI_STORE, 2, WF_MXFP4>(q, mt, s)
              : launch_fp8<288, 256, 3, 4, EPI_STORE, 2>(q, mt, s);
  }
  if (mx) {
    // 128x256 tiles, two blocks per CU as for the up GEMM: DeepSeek-V3's down
    // GEMM 1.24 -> 1.14 ms, V4-Pro's 2.31 -> 2.08 ms (not for the large
    // groups above: Mixtral's 288-row tiles 0.42 ms, 128-row 0.46 ms)
    g.tile_prefix = a.tile_prefix + tile_height_index(128) * (a.n_groups + 1);
    return launch_fp8<128, 256, 2, 4, EPI_STORE, 2, WF_MXFP4>(
        q, tile_bound8(a.rows_bound, a.n_groups, 128), s);
  }
  const int mt = tile_bound8(a.rows_bound, a.n_groups, 256);
  // scheduled main loop (within 1%; the 288-row tiles above keep the
  // compiler's order: their double-buffered fragments would not fit in the
  // registers of three waves per SIMD).  Groups of a few rows on a skewed
  // load: 32 x 128 streaming tiles in the same launch, as for the up GEMM
  // (V4-Pro's down GEMM 2.67 -> 2.60-2.63 ms).
  if (split_small_groups(a.rows_bound, a.n_groups)) {
    Fp8Args qs = q;
    qs.g.n_tiles = ceil_div(c.d, 128);
    qs.g.tile_prefix = a.tile_prefix + kListSmall32 * (a.n_groups + 1);
    g.tile_prefix = a.tile_prefix + kListLarge256 * (a.n_groups + 1);
    return launch_fp8_split<Fp8Tile<256, 256, 4, 4, 2, 1>, Fp8Tile<32, 128, 1, 4, 3>, EPI_STORE,
                            WF_E4M3>(q, mt, qs, s);
  }
  g.tile_prefix = a.tile_prefix + tile_height_index(256) * (a.n_groups + 1);
  return launch_fp8<256, 256, 4, 4, EPI_STORE, 2, WF_E4M3, 1>(q, mt, s);
}

}  // namespace moe
