// Grouped GEMMs of the MoE layer on gfx950 MFMA.
//
// Two kernel templates serve three contractions, all "TN" (both operands
// contiguous along the reduction dimension K):
//   router   logits[t, e]  = hidden[t] . W_r[e]            (+ logit offset), float out
//   GEMM 1   H[r, f]       = SiLU(x . W1_e[f]) * (x . W3_e[f]),  x = hidden[token of row r]
//   GEMM 2   Y[r, o]       = H[r] . W2_e[o]
// ("MoE 的算量与通信" chapter 二.1 SwiGLU and 六.2 grouped GEMM; "Mixture of Experts:
// Router, Token Dispatch, Grouped GEMM", sections Expert and Grouped GEMM; the
// fused gate/up weight w13 of "DeepSeek-V4 MoE" section 四.)
//
// Rows are grouped by expert ("group"); a group's rows are contiguous in the
// dispatch order and its row count is only known on the device.  The grid is
// sized on the host from an upper bound on the number of row tiles; each block
// reads the device-side tile prefix to find its (group, row tile), and blocks
// past the real tile count exit at once.
//
// grouped_gemm_dma (bf16): direct global -> LDS buffer loads into rings of
// LDS stages, MFMA 32x32x16.  When experts have many rows (MFMA-bound
// prefill): 288x256 tiles on 12 wavefronts for the up GEMM and for the down
// GEMM of large experts, else 256x256 tiles on 16 wavefronts; 32-row tiles
// with a four-stage ring when they have a few (each expert's weights streamed
// once, HBM-bound decode).
// grouped_gemm_staged (any element type): global -> registers -> LDS, two
// stages, MFMA 16x16; the router GEMM (split over K), the fp32 configurations
// and shapes the buffer-load kernel does not take.
#include "moe_gemm_kernels.h"

namespace moe {
namespace {
using namespace gemm;

template <typename TE, int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_gemm(GemmArgs p, int m_tiles_bound, hipStream_t s, int splits = 1) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDS = 2 * (BM + BN) * 128;
  const int grid = xcd_grid((int64_t)m_tiles_bound * p.n_tiles);
  if (grid <= 0) return hipSuccess;
  auto kern = grouped_gemm_staged<TE, BM, BN, WM, WN, EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid, splits), dim3(NT), LDS, s, p);
  return hipGetLastError();
}

// Direct-to-LDS bf16 kernel (ST LDS buffers of ROWB/2 K-elements).
template <int BM, int BN, int WM, int WN, int EPI, int ST, int ROWB, int SWZ, int SCHED = 0>
hipError_t launch_gemm_dma(GemmArgs p, int m_tiles_bound, hipStream_t s, int splits = 1) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDS = ST * (BM + BN) * ROWB;
  const int grid = xcd_grid((int64_t)m_tiles_bound * p.n_tiles);
  if (grid <= 0) return hipSuccess;
  auto kern = grouped_gemm_dma<BM, BN, WM, WN, EPI, ST, ROWB, SWZ, SCHED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid, splits), dim3(NT), LDS, s, p);
  return hipGetLastError();
}

// Upper bound on sum_g ceil(M_g / bm) given sum_g M_g <= rows over at most
// `groups` non-empty groups.
int tile_bound(int64_t rows, int groups, int bm) {
  const int64_t ne = rows < groups ? rows : groups;
  return (int)((rows + ne * (bm - 1)) / bm);
}

bool split_small_groups(const ExpertFfnArgs& a) {
  return moe::split_small_groups(a.rows_bound, a.n_groups);
}

// A grouped GEMM's two tile lists in one launch (grouped_gemm_dma_split): the
// 32 x 256 streaming tiles of `small` on the first kSmallGroupBlocks blocks,
// one 288 x 256 tile of `big` on each later block.
template <int EPI>
hipError_t launch_split(const GemmArgs& big, int big_m_tiles, const GemmArgs& small,
                        hipStream_t s) {
  const int big_grid = xcd_grid((int64_t)big_m_tiles * big.n_tiles);
  const int grid = kSmallGroupBlocks + big_grid;
  auto kern = grouped_gemm_dma_split<EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kSplitLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kSplitBigWaves), kSplitLds, s, big, small,
                     kSmallGroupBlocks);
  return hipGetLastError();
}

}  // namespace

int router_splits(const moe_config& c) {
  // Split K so that a small router GEMM still fills the chip (E = 8 or T = 64
  // give only a handful of 64x64 tiles), each split a whole number of 128-byte
  // K stages.  The count depends on d only, never on T: a token's logits are
  // then summed in the same order whatever batch it comes in.
  if (c.dtype == MOE_F32) return 1;
  const int stages = c.d / 64;
  int s = 1;
  while (s * 2 <= kRouterSplits && stages % (s * 2) == 0) s *= 2;
  return s;
}

hipError_t launch_router_gemm(const moe_config& c, const void* hidden, const void* w_router,
                              const float* logit_offset, float* out, int splits,
                              hipStream_t s) {
  GemmArgs p{};
  const int es = c.dtype == MOE_F32 ? 4 : 2;
  p.A = static_cast<const char*>(hidden);
  p.lda = (int64_t)c.d * es;
  p.B = static_cast<const char*>(w_router);
  p.ldb = (int64_t)c.d * es;
  p.N = c.E;
  p.K = c.d;
  p.G = 1;
  p.dense_rows = c.T;
  p.C = reinterpret_cast<char*>(out);
  p.ldc = (int64_t)c.E * 4;
  p.col_add = splits > 1 ? nullptr : logit_offset;  // with splits, added when summed
  if (c.dtype == MOE_F32) {
    p.n_tiles = ceil_div(c.E, 16);
    return launch_gemm<float, 16, 16, 1, 1, EPI_LOGITS>(p, ceil_div(c.T, 16), s);
  }
  if (splits > 1) {  // partial rows padded to whole 16-byte chunks
    p.k_chunk = c.d / splits;
    p.ldc = (int64_t)router_part_ld(c) * 4;
    p.c_split = (int64_t)c.T * p.ldc;
  }
  // The direct-to-LDS kernel (K slices of whole 64-element stages; hidden rows
  // and router weights addressed with 31-bit offsets): 128x128 tiles on 8
  // waves of 64x32 for large batches with many experts, 64x64 tiles on 4
  // waves otherwise, so that enough blocks run.  Both walk K in the same
  // order with the same MFMA for every output, so a token's logits are
  // bitwise the same whichever shape its batch takes.
  const int64_t lim = int64_t(1) << 31;
  if ((int64_t)c.T * c.d * 2 < lim && (int64_t)c.E * c.d * 2 < lim) {
    p.a_bytes = (uint32_t)((int64_t)c.T * c.d * 2);
    p.b_bytes = (uint32_t)((int64_t)c.E * c.d * 2);
    if (c.T >= 1024 && c.E >= 128) {
      p.n_tiles = ceil_div(c.E, 128);
      return launch_gemm_dma<128, 128, 2, 4, EPI_LOGITS, 2, 128, 3, 1>(p, ceil_div(c.T, 128),
                                                                       s, splits);
    }
    p.n_tiles = ceil_div(c.E, 64);
    return launch_gemm_dma<64, 64, 2, 2, EPI_LOGITS, 2, 128, 3, 1>(p, ceil_div(c.T, 64), s,
                                                                   splits);
  }
  // batches too large for 31-bit offsets: the register-staged kernel.  Large
  // batches with many experts: 128x128 tiles read the hidden rows half as
  // often, on 8 waves of 32x64; small batches 64x64 tiles.
  if (c.T >= 1024 && c.E >= 128) {
    p.n_tiles = ceil_div(c.E, 128);
    return launch_gemm<uint16_t, 128, 128, 4, 2, EPI_LOGITS>(p, ceil_div(c.T, 128), s, splits);
  }
  p.n_tiles = ceil_div(c.E, 64);
  return launch_gemm<uint16_t, 64, 64, 2, 2, EPI_LOGITS>(p, ceil_div(c.T, 64), s, splits);
}

namespace {

// Tile shape of the grouped expert GEMMs.  Rows per group on average (known on
// the host from T, k and the group count) picks 32-row tiles for
// decode-shaped batches and, for prefill-shaped ones, 288x256 tiles for the
// up GEMM and 256x256 tiles for the down GEMM (288x256 for large groups, see
// tall_down_tiles), all on the direct-to-LDS kernel when the shapes allow it (d_ff a multiple of 128 and
// operands addressable with 31-bit offsets), else 16- or 128-row tiles on the
// register-staged kernel.  The direct-to-LDS shapes accumulate K in the same
// order (64-element slabs, 16-element MFMA steps, one fp32 accumulator per
// output), so a row's result does not depend on which of them runs: with the
// router's T-independent split, the layer output of a token does not depend on
// the batch it is in.
enum class FfnTiles { F32_16, BF16_16, BF16_32, BF16_128, BF16_PREFILL };

FfnTiles pick_tiles(const moe_config& c, const ExpertFfnArgs& a) {
  if (c.dtype == MOE_F32) return FfnTiles::F32_16;
  const int64_t avg_rows = a.rows_bound / (a.n_groups > 0 ? a.n_groups : 1);
  // the buffer-load kernels address each operand, and a tile's rows of the
  // output (at most 288), with 32-bit offsets
  const int64_t lim = int64_t(1) << 31;
  const bool fits = c.d_ff % 128 == 0 && (int64_t)c.T * c.d * 2 < lim &&
                    (int64_t)a.rows_bound * c.d_ff * 2 < lim &&
                    (int64_t)2 * c.d_ff * c.d * 2 < lim && (int64_t)288 * c.d * 2 < lim;
  // a few rows per expert: the GEMMs stream each expert's weights once
  // (HBM-bound); 32-row tiles with a deep direct-to-LDS pipeline
  if (avg_rows < 48) return fits ? FfnTiles::BF16_32 : FfnTiles::BF16_16;
  return fits ? FfnTiles::BF16_PREFILL : FfnTiles::BF16_128;
}

int tile_rows(FfnTiles t) {
  return t == FfnTiles::BF16_PREFILL ? 288 : t == FfnTiles::BF16_128 ? 128
                                         : t == FfnTiles::BF16_32  ? 32 : 16;
}

}  // namespace

hipError_t launch_expert_up(const moe_config& c, const ExpertFfnArgs& a, hipStream_t s) {
  const int es = c.dtype == MOE_F32 ? 4 : 2;
  const int64_t d = c.d, F = c.d_ff;
  const FfnTiles tiles = pick_tiles(c, a);
  const int bm = tile_rows(tiles);
  GemmArgs g{};
  g.A = static_cast<const char*>(a.hidden);
  g.a_rows = a.sorted_tok;
  g.lda = d * es;
  g.B = static_cast<const char*>(a.w13);
  g.B_last = static_cast<const char*>(a.w13_last);
  g.b_group = 2 * F * d * es;
  g.ldb = d * es;
  g.N = c.d_ff;
  g.up_row = c.d_ff;
  g.K = c.d;
  g.g_begin = a.g_begin;
  g.g_end = a.g_end;
  g.G = a.n_groups;
  g.tile_prefix = a.tile_prefix + tile_height_index(bm) * (a.n_groups + 1);
  g.C = static_cast<char*>(a.H);
  g.ldc = F * es;
  const int mb = tile_bound(a.rows_bound, a.n_groups, bm);
  switch (tiles) {
    case FfnTiles::F32_16:
      g.n_tiles = c.d_ff / 32;
      return launch_gemm<float, 16, 64, 1, 2, EPI_SWIGLU>(g, mb, s);
    case FfnTiles::BF16_16:
      g.n_tiles = c.d_ff / 64;
      return launch_gemm<uint16_t, 16, 128, 1, 4, EPI_SWIGLU>(g, mb, s);
    case FfnTiles::BF16_32:
      g.n_tiles = c.d_ff / 128;
      g.a_bytes = (uint32_t)((int64_t)c.T * c.d * es);
      g.b_bytes = (uint32_t)(2 * F * d * es);
      return launch_gemm_dma<32, 256, 1, 4, EPI_SWIGLU, 4, 128, 3>(g, mb, s);
    case FfnTiles::BF16_PREFILL: {
      g.n_tiles = c.d_ff / 128;
      g.a_bytes = (uint32_t)((int64_t)c.T * c.d * es);
      g.b_bytes = (uint32_t)(2 * F * d * es);
      // the groups of more rows: 288-row tiles (3 x 4 waves of 96 x 64) with
      // the scheduled main loop (Mixtral's up GEMM 1.72 -> 1.67 ms and
      // DeepSeek-V3's 4.52 -> 4.33 ms against 256-row tiles)
      if (!split_small_groups(a))
        return launch_gemm_dma<288, 256, 3, 4, EPI_SWIGLU, 2, 128, 3, 1>(g, mb, s);
      // groups of a few rows: one 32-row streaming tile each, walked by a few
      // blocks of the same launch beside the 288-row tiles
      GemmArgs gs = g;
      gs.tile_prefix = a.tile_prefix + kListSmall32 * (a.n_groups + 1);
      g.tile_prefix = a.tile_prefix + kListLarge288 * (a.n_groups + 1);
      return launch_split<EPI_SWIGLU>(g, mb, gs, s);
    }
    default:
      g.n_tiles = c.d_ff / 64;
      return launch_gemm<uint16_t, 128, 128, 2, 2, EPI_SWIGLU>(g, mb, s);
  }
}

hipError_t launch_expert_down(const moe_config& c, const ExpertFfnArgs& a, hipStream_t s) {
  const int es = c.dtype == MOE_F32 ? 4 : 2;
  const int64_t d = c.d, F = c.d_ff;
  const FfnTiles tiles = pick_tiles(c, a);
  const int bm = tile_rows(tiles);
  GemmArgs g{};
  g.A = static_cast<const char*>(a.H);
  g.a_rows = nullptr;
  g.lda = F * es;
  g.B = static_cast<const char*>(a.w2);
  g.B_last = static_cast<const char*>(a.w2_last);
  g.b_group = d * F * es;
  g.ldb = F * es;
  g.N = c.d;
  g.K = c.d_ff;
  g.g_begin = a.g_begin;
  g.g_end = a.g_end;
  g.G = a.n_groups;
  g.tile_prefix = a.tile_prefix + tile_height_index(bm) * (a.n_groups + 1);
  g.C = static_cast<char*>(a.Y);
  g.ldc = d * es;
  const int mb = tile_bound(a.rows_bound, a.n_groups, bm);
  switch (tiles) {
    case FfnTiles::F32_16:
      g.n_tiles = ceil_div(c.d, 64);
      return launch_gemm<float, 16, 64, 1, 2, EPI_STORE>(g, mb, s);
    case FfnTiles::BF16_16:
      g.n_tiles = ceil_div(c.d, 128);
      return launch_gemm<uint16_t, 16, 128, 1, 4, EPI_STORE>(g, mb, s);
    case FfnTiles::BF16_32:
      g.n_tiles = ceil_div(c.d, 128);
      g.a_bytes = (uint32_t)((int64_t)a.rows_bound * F * es);
      g.b_bytes = (uint32_t)(d * F * es);
      return launch_gemm_dma<32, 128, 1, 2, EPI_STORE, 4, 128, 3>(g, mb, s);
    case FfnTiles::BF16_PREFILL: {
      g.a_bytes = (uint32_t)((int64_t)a.rows_bound * F * es);
      g.b_bytes = (uint32_t)(d * F * es);
      g.n_tiles = ceil_div(c.d, 256);
      // 288-row tiles with the scheduled main loop (Mixtral's down GEMM 0.88 ->
      // 0.83 ms against the compiler's order)
      if (!split_small_groups(a))
        return launch_gemm_dma<288, 256, 3, 4, EPI_STORE, 2, 128, 3, 1>(g, mb, s);
      // groups of a few rows: one 32-row streaming tile each, walked by a few
      // blocks of the same launch
      GemmArgs gs = g;
      gs.tile_prefix = a.tile_prefix + kListSmall32 * (a.n_groups + 1);
      g.tile_prefix = a.tile_prefix + kListLarge288 * (a.n_groups + 1);
      return launch_split<EPI_STORE>(g, mb, gs, s);
    }
    default:
      g.n_tiles = ceil_div(c.d, 128);
      return launch_gemm<uint16_t, 128, 128, 2, 2, EPI_STORE>(g, mb, s);
  }
}

}  // namespace moe
