// Internal declarations shared by the HIP sources of the MoE layer library.
// Nothing here is part of the C ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t align_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Row-tile heights for which the permutation builds tile lists.  List i < 6
// holds the cumulative m-tile count per group for BM = tile_height(i) over
// every group.  288 = 9 fragments: groups of up to 1152 rows in 4 tiles, up to
// 288 in one.
constexpr int kNumTileHeights = 6;  // 16, 32, 64, 128, 256, 288
__host__ __device__ constexpr int tile_height(int i) { return i < 5 ? 16 << i : 288; }
__host__ __device__ constexpr int tile_height_index(int bm) {
  return bm == 16 ? 0 : bm == 32 ? 1 : bm == 64 ? 2 : bm == 128 ? 3 : bm == 256 ? 4 : 5;
}

// Rows per tile of a group of M rows cut into tiles of at most BM rows: the
// group is split into ceil(M/BM) near-equal tiles, each rounded up to a
// multiple of min(32, BM) (whole MFMA fragments), so a group never ends in a
// sliver tile that costs a full tile's operand loads for a few rows, and the
// tiles of a group take about the same time.  The group then has
// ceil(M / group_tile_rows(M, BM)) <= ceil(M / BM) tiles.
__host__ __device__ constexpr int group_tile_rows(int M, int bm) {
  return M <= 0 ? bm
                : (int)align_up(ceil_div(M, ceil_div(M, bm)), bm < 32 ? bm : 32);
}
__host__ __device__ constexpr int group_tiles(int M, int bm) {
  return M <= 0 ? 0 : ceil_div(M, group_tile_rows(M, bm));
}

// More lists split the groups by size, for prefill-shaped batches whose
// routing leaves some experts a few rows (a skewed load): the groups with at
// most kSmallGroupRows rows get one 32-row tile each (list kListSmall32), run
// on the streaming tiles that keep a deep ring of weight loads in flight; the
// others get tiles of the GEMM's prefill height (bf16: 288 rows, list
// kListLarge288; E4M3: 256, kListLarge256).
constexpr int kSmallGroupRows = 32;
constexpr int kListLarge288 = kNumTileHeights, kListSmall32 = kNumTileHeights + 1;
constexpr int kListLarge256 = kNumTileHeights + 2;
constexpr int kNumTileLists = kNumTileHeights + 3;
__host__ __device__ constexpr int large_list_height(int list) {
  return list == kListLarge288 ? 288 : 256;
}
__host__ __device__ constexpr int list_tiles(int list, int M) {
  return list < kNumTileHeights ? group_tiles(M, tile_height(list))
         : list == kListSmall32 ? (M > kSmallGroupRows ? 0 : group_tiles(M, 32))
                                : (M > kSmallGroupRows ? group_tiles(M, large_list_height(list)) : 0);
}

// Consecutive tiles of a grouped GEMM's tile order that run on one XCD (see
// decode_tile); grids are whole multiples of 8 * kXcdChunk blocks.
constexpr int kXcdChunk = 16;
inline int xcd_grid(int64_t tiles) {
  const int64_t u = 8 * kXcdChunk;
  return tiles <= 0 ? 0 : (int)((tiles + u - 1) / u * u);
}

// FP8 / MXFP4 down GEMM of groups that average 512 rows or more: 288-row
// tiles (3 x 4 waves of 96 x 64).  A group of 4 x 256 rows plus the few percent that a
// random routing adds to about half of the groups still fits 4 of them, where
// 256-row tiles would add a fifth row of tiles to those groups and with it a
// partly filled extra round of blocks over the 256 CUs.  (The bf16 GEMMs run
// 288-row tiles on every prefill-shaped batch.)
inline bool tall_down_tiles(int64_t rows_bound, int n_groups) {
  return n_groups > 0 && rows_bound >= (int64_t)512 * n_groups;
}

// Whether a prefill-shaped batch's grouped GEMMs split off the groups of a few
// rows onto streaming tiles.  Not when the groups average 512 rows or more
// (Mixtral's 8 experts): few groups can be that small then, and the streaming
// blocks would mostly be empty; the large tiles then take every group.
inline bool split_small_groups(int64_t rows_bound, int n_groups) {
  return rows_bound < (int64_t)512 * n_groups;
}

// Blocks that walk the small groups' streaming tiles when they share a launch
// with the large tiles (a multiple of 8; one block per CU).  V4-Pro's bf16 up
// GEMM (127 groups of at most 32 rows): 9.11 ms with the two kinds of tile in
// two launches in sequence, 8.61 ms with the streaming tiles on 64 CUs beside
// the 288-row tiles (8.77 on 32, 8.69 on 128); its down GEMM 4.66-4.71 ->
// 4.57-4.63 ms (three rounds; 96 blocks: 4.63-4.64).
constexpr int kSmallGroupBlocks = 64;

// pairs handled by one histogram / scatter block of the permutation
constexpr int kPermuteChunk = 256;   // pairs per histogram / scatter chunk
constexpr int kPermuteSmall = 2048;  // up to this many pairs: one single-block kernel

// ---------------------------------------------------------------------------
// workspace carve-up (byte offsets from the workspace base), shared by the
// entry points so that moe_workspace_size is the maximum any of them needs
// ---------------------------------------------------------------------------
struct Workspace {
  int64_t logits, ids, weights;        // [splits*T*E] f32 partial logits, [T*k] i32, [T*k] f32
  int64_t blockcnt;                    // [nblk*E] i32
  int64_t counts, offsets;             // [E] i32, [E+1] i32
  int64_t groups;                      // [2*G] i32: first rows, then ends
  int64_t tile_prefix;                 // [kNumTileLists][G+1] i32
  int64_t sorted_tok, sorted_w;        // [P] i32, [R] f32
  int64_t dispatch;                    // [R] i32
  int64_t H, Y;                        // [P*d_ff], [P*d] elements of the layer dtype
  int64_t hs;                          // FP8 experts: H scales [P, d_ff/128] f32 (codes at H)
  int64_t xq, xs;                      // FP8 experts: hidden codes [T*d] u8, scales [T, d/128]
  int64_t total;
};

Workspace workspace_layout(const moe_config& c);

// ---------------------------------------------------------------------------
// launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
// Router logits = hidden W_r^T.  With splits == 1, `out` is [T,E] and holds the
// logits plus the offset; with splits > 1 (bf16 only), `out` is [splits,T,Ep]
// (Ep = router_part_ld(c), rows padded to 16 bytes) of partial sums over K
// slices, and the offset is added when the top-k kernel sums them.
// router_splits() is the split count moe_forward uses (at most kRouterSplits).
constexpr int kRouterSplits = 8;
inline int router_part_ld(const moe_config& c) { return align_up(c.E, 4); }
int router_splits(const moe_config& c);
hipError_t launch_router_gemm(const moe_config& c, const void* hidden, const void* w_router,
                              const float* logit_offset, float* out, int splits,
                              hipStream_t s);
// Scores, selection, gates from logits (learned or hash).  With nparts > 0 the
// logits are the sum of nparts partial rows (part s at parts + s*T*E, summed in
// order s = 0, 1, ...) plus logit_offset; else `logits` is read as is.
// logits_out (nullable) receives the summed logits.
hipError_t launch_topk(const moe_config& c, const float* logits, const float* parts, int nparts,
                       const float* logit_offset, const float* bias, const int32_t* token_ids,
                       const int32_t* tid2eid, int32_t* ids, float* weights, float* logits_out,
                       hipStream_t s);
// histogram + scan + stable scatter
hipError_t launch_permute(const moe_config& c, const int32_t* ids, const float* weights,
                          int32_t* blockcnt, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_tok, float* sorted_w, int32_t* dispatch,
                          hipStream_t s);
// Group row ranges and row-tile prefixes from the routed experts' offsets
// [E+1], clamped to [0, routed_limit].  With shared_rows > 0 the shared expert is group E, rows
// [shared_begin, shared_begin + shared_rows), and identity token ids are written
// to sorted_tok[shared_begin ..].  groups = [g_begin[G], g_end[G]].
hipError_t launch_build_tiles(const int32_t* offsets, int E, int routed_limit, int shared_begin,
                              int shared_rows, int32_t* groups, int32_t* tile_prefix,
                              int32_t* sorted_tok, hipStream_t s);

struct ExpertFfnArgs {
  const void* hidden;          // [T, d]
  const int32_t* sorted_tok;   // [rows] token of each dispatch row
  const int32_t* g_begin;      // [G] device: first dispatch row of each group
  const int32_t* g_end;        // [G] device: one past its last row
  const int32_t* tile_prefix;  // [kNumTileLists][G+1] device
  int n_groups;                // G (routed experts + shared)
  int rows_bound;              // host bound on the total number of rows (T*(k+S))
  int routed_groups;           // groups whose weights live in w13/w2 (E)
  const void* w13;             // [E, 2*d_ff, d]
  const void* w2;              // [E, d, d_ff]
  const void* w13_last;        // weights of group E (shared) or nullptr
  const void* w2_last;
  void* H;                     // [rows, d_ff] intermediate
  void* Y;                     // [rows, d] unweighted expert outputs
};
// GEMM 1 + SiLU(gate) * up -> H, and GEMM 2 -> Y
hipError_t launch_expert_up(const moe_config& c, const ExpertFfnArgs& a, hipStream_t s);
hipError_t launch_expert_down(const moe_config& c, const ExpertFfnArgs& a, hipStream_t s);

// FP8 experts: E4M3 codes with float32 block scales (see include/moe.h)
// The FP8 experts: E4M3 activations with 1x128 scales; weights in E4M3 with
// 128x128 float tile scales (kWeightE4M3) or MXFP4 with 1x32 E8M0 scales
// (kWeightMxfp4, codes packed two per byte)
enum { kWeightE4M3 = 0, kWeightMxfp4 = 1 };
struct Fp8FfnArgs {
  int wfmt;                    // kWeightE4M3 or kWeightMxfp4
  const uint8_t* xq;           // [T, d] codes of the hidden rows
  const float* xs;             // [d/128, T] (K-block-major)
  const int32_t* sorted_tok;   // [rows]
  const int32_t* g_begin;      // [G]
  const int32_t* g_end;        // [G]
  const int32_t* tile_prefix;  // [kNumTileLists][G+1]
  int n_groups, rows_bound, routed_groups;
  const uint8_t* w13q;         // E4M3: [E, 2*d_ff, d]; MXFP4: [E, 2*d_ff, d/2]
  const void* w13s;            // E4M3: [E, 2*d_ff/128, d/128] float; MXFP4: [E, d/128, 2*d_ff, 4] bytes
  const uint8_t* w2q;          // E4M3: [E, d, d_ff]; MXFP4: [E, d, d_ff/2]
  const void* w2s;             // E4M3: [E, d/128, d_ff/128] float; MXFP4: [E, d_ff/128, d, 4] bytes
  const uint8_t* w13q_last;    // group E (shared) or nullptr
  const void* w13s_last;
  const uint8_t* w2q_last;
  const void* w2s_last;
  uint8_t* hq;                 // [rows, d_ff]
  float* hs;                   // [d_ff/128, rows_bound] (K-block-major)
  void* Y;                     // [rows, d] bfloat16
};
hipError_t launch_expert_up_fp8(const moe_config& c, const Fp8FfnArgs& a, hipStream_t s);
hipError_t launch_expert_down_fp8(const moe_config& c, const Fp8FfnArgs& a, hipStream_t s);
// 1x128 row quantization (in_dtype MOE_F32 / MOE_BF16) and 128x128 tile quantization
hipError_t launch_quantize_rows(int n, int K, int in_dtype, const void* x, uint8_t* q,
                                float* scales, hipStream_t s);
hipError_t launch_quantize_blocks(int R, int C, int in_dtype, const void* w, uint8_t* q,
                                  float* scales, hipStream_t s);
// MXFP4: n_mat matrices [R, C] in 1x32 blocks -> q [n_mat, R, C/2] packed E2M1,
// scales [n_mat, C/128, R, 4] E8M0
hipError_t launch_quantize_mxfp4(int n_mat, int R, int C, int in_dtype, const void* w, uint8_t* q,
                                 uint8_t* scales, hipStream_t s);

hipError_t launch_combine(const moe_config& c, const void* expert_out, const int32_t* dispatch,
                          const float* weights, const void* shared_out, void* out,
                          hipStream_t s);

}  // namespace moe
