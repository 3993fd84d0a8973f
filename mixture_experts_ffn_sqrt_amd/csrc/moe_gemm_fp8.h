// Grouped GEMM with FP8 (E4M3) operands and block scales, for the FP8 experts.
// Instantiated by moe_fp8.hip.
//
// What it computes ("MoE 架构与路由策略": E4M3, one scale per 128x128 weight
// tile, table dsv4-moe-stages: activation + FP8 cast between Linear-1 and
// Linear-2; "MoE 的算量与通信" closing section: promotion to FP32 accumulation
// every 128 elements): for an output (row r, column o),
//   acc = sum_kb  sa[r, kb] * sb[o/128, kb] * sum_{k in block kb} A[r, k] * B[o, k]
// with A and B E4M3 codes, sa the operand row's scale per 128 columns and sb
// the weight tile's scale, all scales powers of two.  gfx950's scaled MFMA
// 32x32x64 takes a power-of-two (E8M0) scale per row of A and per column of B
// for each 32-element K sub-block and accumulates in float32, so each
// 128-element block (one LDS stage) is two scaled MFMA steps straight into the
// accumulator: the per-block promotion costs no vector instruction.
//
// MXFP4 weights (WF_MXFP4; the same page's FP4 QAT section: E2M1 with one
// scale per 1x32 sub-block, native FP4 weights at inference, FP4 x FP8
// products): B is packed E2M1 (two codes per byte; rows stored in pairs, so
// that one 128-element K block of rows 2i and 2i+1 fills one 128-byte line)
// with an E8M0 scale byte per weight row and 32-element K block, so
//   acc = sum_b  sa[r, b/4] * sb[o, b] * sum_{k in block b} A[r, k] * B[o, k]
// over 32-element blocks b.  The scaled MFMA takes FP8 A and FP4 B in one
// instruction, and its per-lane B scale is exactly one such block (a lane's
// column and K half), so the E8M0 bytes go to the matrix cores unchanged.
//
// Epilogues: EPI_SWIGLU8 (Linear-1): h = SiLU(g) * u in float32, then the FP8
// cast of h in 1x128 groups -- a tile holds exactly one 128-column group of H
// per row, so the group maximum is reduced across the tile's waves through
// LDS and the codes and scales are written straight from the tile.
// EPI_STORE (Linear-2): bfloat16 output rounded once.
#pragma once

#include "moe_gemm_kernels.h"

namespace moe {
namespace gemm {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

enum { EPI_SWIGLU8 = 3 };
enum { WF_E4M3 = 0, WF_MXFP4 = 1 };  // weight formats

struct Fp8Args {
  GemmArgs g;                 // operands as codes (1 byte per element); C: H codes or Y (bf16)
  const float* a_scale;       // [K/128, scale rows]: a K block's scales of all rows together
  // weight scales of group 0: E4M3 weights: [N_w/128, K/128] float tile scales
  // (N_w = weight rows); MXFP4: [K/128, N_w, 4] E8M0 bytes (per 128-column
  // block of K, each row's four 32-element block scales)
  const void* b_scale;
  const void* b_scale_last;   // the last group's, when it is not in b_scale (shared expert)
  int64_t b_scale_group;      // bytes between groups' weight scales (= one group's)
  uint32_t b_scale_kstride;   // bytes between the scales of consecutive K blocks of a row
  float* c_scale;             // EPI_SWIGLU8: [d_ff/128, rows] scales of H
  int ldcs;                   // floats between K blocks of c_scale (its rows)
  uint32_t as_bytes;          // bytes of a_scale (buffer range)
  uint32_t as_kstride;        // bytes between K blocks of a_scale
};

// E4M3 code of v (finite; saturated to +-448), nearest-even.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// Exponent of a group's scale: the smallest e with amax <= 448 * 2^e.  With
// amax = m * 2^k, m in [0.5, 1), and 448 = 0.875 * 2^9: e = k - 9 if m <= 0.875,
// else k - 8; at least -126 (a normal float); 0 for an all-zero group.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (amax == 0.0f) return 0;
  int k;
  const float m = frexpf(amax, &k);
  const int e = k - 9 + (m > 0.875f ? 1 : 0);
  return e < -126 ? -126 : e;
}

// E8M0 form of a power-of-two float scale: its biased exponent
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

// MFMA 32x32x64 with E8M0 scales, A in E4M3 and B in E4M3 (WF_E4M3) or E2M1
// (WF_MXFP4: B's 32 codes per lane in the first four registers): lane l's sa
// scales A row l % 32 and K half l / 32, lane l's sb scales B column l % 32 and
// K half l / 32
template <int WF>
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c,
                                           int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, WF == WF_MXFP4 ? 4 : 0, 0,
                                                         sa, 0, sb);
}

// BM x BN tile, WM x WN waves (wave tile 32*FM x 32*FN), STAGES LDS buffers of
// one 128-element K block each: A rows (128 bytes, chunks swizzled by
// (row >> 1) & 7), B rows (E4M3: 128 bytes, swizzled likewise; MXFP4: 64 bytes,
// chunks swizzled by (row >> 2) & 3), the block's A-row scales, and the
// block's weight scales (E4M3: of the tile's at most two 128-row weight
// blocks; MXFP4: one dword of four E8M0 bytes per B row).  Everything a stage
// needs arrives through the same direct-to-LDS loads, issued STAGES-1 stages
// ahead.
// LDS bytes of one pipeline stage of grouped_gemm_fp8: A rows (128 bytes), B
// rows (128 bytes E4M3, 64 MXFP4), A-row scales in whole 64-row loads, weight
// scales (E4M3: one 256-byte load; MXFP4: a dword per B row).
template <int BM, int BN, int WF>
__host__ __device__ constexpr int fp8_stage_bytes() {
  return BM * 128 + BN * (WF == WF_MXFP4 ? 64 : 128) + (BM + 63) / 64 * 256 +
         (WF == WF_MXFP4 ? BN * 4 : 256);
}

// Maxima of NV values per lane over the 32 lanes of a lane half, by recursive
// halving: at the step with lane distance D, a lane keeps the half of its N
// remaining values selected by bit D of its column and sends the other half to
// the lane D apart, which keeps the opposite half; the shuffles of one step are
// independent of one another.  After log2(NV) steps lane c holds the maximum
// of value c * NV / 32 (NV < 32: the remaining steps are plain exchanges, and
// 32 / NV neighbouring lanes hold the same maximum).  31 shuffles for 32
// values, where one butterfly per value takes 160.  A maximum is exact and
// independent of the order of its operands.
template <int NV, int D, int N = NV>
struct HalvingMax {
  template <int M>
  __device__ __forceinline__ static void run(float (&v)[M], int ccol) {
    if constexpr (D >= 1) {
      if constexpr (N > 1) {
        const bool b = (ccol & D) != 0;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
          const float send = b ? v[j] : v[j + N / 2];
          const float keep = b ? v[j + N / 2] : v[j];
          v[j] = fmaxf(keep, __shfl_xor(send, D, 32));
        }
        HalvingMax<NV, D / 2, N / 2>::run(v, ccol);
      } else {
        v[0] = fmaxf(v[0], __shfl_xor(v[0], D, 32));
        HalvingMax<NV, D / 2, 1>::run(v, ccol);
      }
    }
  }
};

// One tile of grouped_gemm_fp8 (below).
// SCHED = 1: fragments double-buffered in registers across the two k-steps of
// a stage, in the order sched_stage fixes (full tiles only).
template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int WF = WF_E4M3, int SCHED = 0>
__device__ __forceinline__ void gemm_fp8_tile(const Fp8Args& q, const TileCoord& tc) {
  const GemmArgs& p = q.g;
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr bool SW = EPI == EPI_SWIGLU8;
  constexpr bool MX = WF == WF_MXFP4;
  constexpr int ROWB = 128;                  // bytes (= K elements) of an A row per stage
  constexpr int BROWB = MX ? 64 : 128;       // bytes of a B row per stage
  constexpr int RPL = 1024 / ROWB;           // A rows filled by one wavefront load
  constexpr int RPLB = 1024 / BROWB;         // B rows filled by one wavefront load
  constexpr int BCH = BROWB / 16;            // 16-byte chunks per B row
  constexpr int NSA = (BM + 63) / 64;        // A-row scale loads per stage (one per wave < NSA)
  constexpr int SAB = NSA * 256;             // A-row scale bytes per stage
  constexpr int NSBL = MX ? BN / 64 : 1;     // weight-scale wavefront loads per stage
  constexpr int SBB = 256 * NSBL;            // weight-scale bytes per stage
  constexpr int OFF_B = BM * ROWB, OFF_SA = OFF_B + BN * BROWB, OFF_SB = OFF_SA + SAB;
  constexpr int STAGE = OFF_SB + SBB;
  static_assert(STAGE == fp8_stage_bytes<BM, BN, WF>(), "stage layout");
  constexpr int NSB = BN / 128;              // E4M3: weight blocks per tile (<= 2)
  // 1 KB operand loads per stage: NA of A rows, NB of B rows; wave w issues A
  // blocks w + NW*j (j < LA) and B blocks w + NW*j (j < LB, block < NB)
  constexpr int NA = BM / RPL, NB = BN / RPLB;
  constexpr int LA = NA / NW, LB = (NB + NW - 1) / NW;
  constexpr bool B_EVEN = NB % NW == 0;
  constexpr int B_POL = BM <= 32 ? kStreamWeightPolicy : 0;  // streaming tiles: whole lines
  constexpr int BKS = MX ? 128 : BROWB;  // bytes between consecutive K blocks of a weight row
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "whole 32x32 fragments");
  static_assert(NA * RPL == BM && NB * RPLB == BN && LA * NW == NA, "A loads must split evenly");
  static_assert(NSBL <= NW, "one weight-scale load per wave at most");
  static_assert(!SW || BN == 256, "SwiGLU8: one 128-column group of H per tile");
  static_assert(!SW || FN % 2 == 0, "SwiGLU waves hold gate and up fragments in pairs");
  static_assert(NSA <= NW, "one scale load per wave at most");
  static_assert(NSB >= 1 && NSB <= 2, "one or two weight blocks per tile");
  static_assert(STAGES >= 2 && STAGES * STAGE <= 160 * 1024, "LDS budget");
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool last = p.B_last && tc.grp == p.G - 1;
  const char* Bg = last ? p.B_last : p.B + (int64_t)tc.grp * p.b_group;
  const char* Sb = last ? static_cast<const char*>(q.b_scale_last)
                        : static_cast<const char*>(q.b_scale) + tc.grp * q.b_scale_group;
  constexpr uint32_t kOut = 0x80000000u;
  const __amdgpu_buffer_rsrc_t a_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.A), 0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Bg), 0, (int)p.b_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(q.a_scale), 0, (int)q.as_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t sb_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(Sb), 0, (int)q.b_scale_group, 0x00020000);
  const int KB = p.K / 128;  // K blocks (= stages of the loop)

  // operand rows: lane l of load j fills slot l % 8 of tile row RPL*(wave+NW*j) + l/8
  const int lr = lane / 8, lq = lane % 8;
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int row = RPL * (wave + NW * j) + lr;
    const int ch = lq ^ ((row >> 1) & 7);
    if (row < tc.nrows) {
      const int arow = p.a_rows ? p.a_rows[tc.row0 + row] : tc.row0 + row;
      a_off[j] = (uint32_t)arow * (uint32_t)p.lda + ch * 16;
    } else {
      a_off[j] = kOut;
    }
  }
  // weight row of tile row `row` (-1: past the weight rows)
  auto weight_row = [&](int row) -> int {
    if (SW) return row < BN / 2 ? tc.nt * (BN / 2) + row : p.up_row + tc.nt * (BN / 2) + (row - BN / 2);
    const int brow = tc.nt * BN + row;
    return brow < p.N ? brow : -1;
  };
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int row = RPLB * (wave + NW * j) + lane / BCH;
    const int ch = MX ? (lane % BCH) ^ ((row >> 2) & 3) : (lane % BCH) ^ ((row >> 1) & 7);
    const int brow = weight_row(row);
    // E2M1 codes: rows 2i, 2i+1 share each 128-byte line of a 128-element K block
    const uint32_t rowb = MX ? (uint32_t)(brow >> 1) * (uint32_t)(2 * p.ldb) + (uint32_t)(brow & 1) * 64u
                             : (uint32_t)brow * (uint32_t)p.ldb;
    b_off[j] = brow >= 0 ? rowb + ch * 16 : kOut;
  }
  // the last B slot exists on waves whose block wave + NW*(LB-1) is < NB
  const bool b_last = B_EVEN || wave + NW * (LB - 1) < NB;
  // A-row scales: wave w < NSA loads rows 64 w .. 64 w + 63 (4 bytes per lane;
  // the K-block-major layout keeps a stage's scales of ascending rows together)
  uint32_t s_off = kOut;
  {
    const int row = 64 * wave + lane;
    if (wave < NSA && row < tc.nrows) {
      const int arow = p.a_rows ? p.a_rows[tc.row0 + row] : tc.row0 + row;
      s_off = (uint32_t)arow * 4u;  // scales are indexed like the A rows
    }
  }
  // weight scales, loaded by the last NSBL waves.  E4M3: lane j < NSB loads
  // the scale row of the tile's weight block j (for SwiGLU: the gate block,
  // then the up block).  MXFP4: lane l of load i loads tile row 64 i + l's four
  // E8M0 bytes of the stage's K block (consecutive rows are consecutive words,
  // so a load reads 256 contiguous bytes).  Rows past the weight rows read zeros.
  uint32_t sb_off = kOut;
  if constexpr (MX) {
    const int brow = weight_row(64 * (wave - (NW - NSBL)) + lane);
    if (wave >= NW - NSBL && brow >= 0) sb_off = (uint32_t)brow * 4u;
  } else if (lane < NSB) {
    const int blk = SW ? (lane == 0 ? tc.nt : p.up_row / 128 + tc.nt) : tc.nt * NSB + lane;
    if (SW || blk * 128 < p.N) sb_off = (uint32_t)blk * (uint32_t)(KB * 4);
  }
  const bool has_sa = wave < NSA, has_sb = wave >= NW - NSBL;  // scale loads of this wave
#define MOE_FP8_ISSUE(kt_)                                                                 \
  do {                                                                                     \
    const int kc_ = (kt_) < KB ? (kt_) : KB - 1;                                           \
    char* buf_ = smem + ((kt_) % STAGES) * STAGE;                                          \
    _Pragma("unroll") for (int j = 0; j < LA; ++j)                                          \
        load_lds16(a_rs, buf_ + (RPL * (wave + NW * j)) * ROWB, a_off[j] + kc_ * ROWB);     \
    _Pragma("unroll") for (int j = 0; j < LB; ++j) {                                        \
      if (j == LB - 1 && !b_last) break;                                                   \
      load_lds16<B_POL>(b_rs, buf_ + OFF_B + (RPLB * (wave + NW * j)) * BROWB,             \
                 b_off[j] + kc_ * BKS);                                                    \
    }                                                                                      \
    if (has_sa)                                                                            \
      load_lds4(s_rs, buf_ + OFF_SA + 256 * wave, s_off + (uint32_t)kc_ * q.as_kstride);   \
    if (has_sb)                                                                            \
      load_lds4(sb_rs, buf_ + OFF_SB + 256 * (wave - (NW - NSBL)),                         \
                sb_off + (uint32_t)kc_ * q.b_scale_kstride);                                \
  } while (0)

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  // fragment reads: row lane % 32 of the K step kk (64 elements = four 16-byte
  // chunks 4 kk .. 4 kk + 3 of an A row).  E4M3 x E4M3: lane half fh holds K
  // 32 fh .. 32 fh + 31 of the step (chunks 2 fh, 2 fh + 1) on both sides.
  // E4M3 x E2M1: a lane half's 32 FP4 codes meet the A elements at step
  // positions 16 fh .. 16 fh + 15 and 32 + 16 fh .. 32 + 16 fh + 15, and its B
  // scale covers exactly those; so B lanes take K 32 fh .. 32 fh + 31 (one
  // 1x32 block, chunk 2 kk + fh of a 64-byte B row) and A lanes take chunks
  // fh and fh + 2 of the step.
  const int fr = lane & 31, fh = lane >> 5, fs = (fr >> 1) & 7;
  int rd0[2], rd1[2], rdb[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c0 = MX ? 4 * kk + fh : 4 * kk + 2 * fh;
    const int c1 = MX ? 4 * kk + fh + 2 : 4 * kk + 2 * fh + 1;
    rd0[kk] = fr * ROWB + ((c0 ^ fs) << 4);
    rd1[kk] = fr * ROWB + ((c1 ^ fs) << 4);
    rdb[kk] = fr * BROWB + (((2 * kk + fh) ^ ((fr >> 2) & 3)) << 4);
  }
  int b_row[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f)
    b_row[f] = SW ? ((f < FN / 2) ? wn * (WTN / 2) + 32 * f : BN / 2 + wn * (WTN / 2) + 32 * (f - FN / 2))
                  : wn * WTN + 32 * f;
  // weight tile (128-row block) of fragment f, as a row of the group's scale table
  // slot of fragment f's weight block among the stage's weight-block scales
  int sb_slot[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) sb_slot[f] = SW ? (f < FN / 2 ? 0 : 1) : b_row[f] / 128;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) MOE_FP8_ISSUE(s);

  const int live = min(FM, max(0, (tc.nrows - wm * WTM + 31) / 32));
  // fragment reads of k-step kk_ (64 elements) of the stage at cur into a_ / b_
#define MOE_FP8_FRAGS(a_, b_, kk_)                                                          \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                        \
      const char* src = cur + (wm * WTM + 32 * i) * ROWB;                                  \
      const u32x4 lo = *reinterpret_cast<const u32x4*>(src + rd0[kk_]);                    \
      const u32x4 hi = *reinterpret_cast<const u32x4*>(src + rd1[kk_]);                    \
      a_[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],                        \
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};                       \
    }                                                                                      \
    _Pragma("unroll") for (int f = 0; f < FN; ++f) {                                        \
      const char* src = cur + OFF_B + b_row[f] * BROWB;                                    \
      if constexpr (MX) {                                                                  \
        const u32x4 lo = *reinterpret_cast<const u32x4*>(src + rdb[kk_]);                  \
        b_[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};         \
      } else {                                                                             \
        const u32x4 lo = *reinterpret_cast<const u32x4*>(src + rd0[kk_]);                  \
        const u32x4 hi = *reinterpret_cast<const u32x4*>(src + rd1[kk_]);                  \
        b_[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],                      \
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};                     \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // k-step kk_'s scaled MFMAs (fragments with no valid row skipped when CHECK)
#define MOE_FP8_MMA(a_, b_, kk_, CHECK)                                                     \
  do {                                                                                     \
    int sbe[FN];                                                                           \
    _Pragma("unroll") for (int f = 0; f < FN; ++f)                                          \
        sbe[f] = MX ? (int)((sbw[f] >> (16 * (kk_))) & 0xFFu) : (int)sbw[f];               \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                        \
      if (CHECK && i >= live) continue;                                                    \
      _Pragma("unroll") for (int f = 0; f < FN; ++f)                                        \
          acc[i][f] = mfma_fp8<WF>(a_[i], b_[f], acc[i][f], sae[i], sbe[f]);               \
    }                                                                                      \
  } while (0)
#define MOE_FP8_MAIN(CHECK)                                                                 \
  for (int kt = 0; kt < KB; ++kt) {                                                        \
    /* at most (STAGES-2) later stages' loads may still be in flight: a wave's */         \
    /* loads per stage are its operand loads (one fewer without the last B */              \
    /* slot) plus one for each kind of scale it loads (wave-uniform, so each */            \
    /* wave waits for its own count) */                                                    \
    wait_loads_le<STAGES - 2, LA + LB - 1>(LA + LB - (b_last ? 0 : 1) + (has_sa ? 1 : 0) + \
                                           (has_sb ? 1 : 0));                              \
    __builtin_amdgcn_s_waitcnt(0xC07F);                                                    \
    lds_barrier();                                                                         \
    MOE_FP8_ISSUE(kt + STAGES - 1);                                                         \
    const char* cur = smem + (kt % STAGES) * STAGE;                                        \
    /* E4M3: the E8M0 form of the fragment's weight-block scale; MXFP4: the four */       \
    /* E8M0 bytes of the lane's B column, shifted so byte 2 kk is its K half's */          \
    uint32_t sbw[FN];                                                                      \
    _Pragma("unroll") for (int f = 0; f < FN; ++f) {                                        \
      if constexpr (MX)                                                                    \
        sbw[f] = *reinterpret_cast<const uint32_t*>(cur + OFF_SB + 4 * (b_row[f] + fr)) >> (8 * fh); \
      else                                                                                 \
        sbw[f] = e8m0_of(*reinterpret_cast<const float*>(cur + OFF_SB + 4 * sb_slot[f]));  \
    }                                                                                      \
    int sae[FM];                                                                           \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
        sae[i] = e8m0_of(*reinterpret_cast<const float*>(cur + OFF_SA + 4 * (wm * WTM + 32 * i + fr))); \
    if constexpr (SCHED) {                                                                 \
      i32x8 a[2][FM], b[2][FN];                                                            \
      MOE_FP8_FRAGS(a[0], b[0], 0);                                                        \
      MOE_FP8_FRAGS(a[1], b[1], 1);                                                        \
      MOE_FP8_MMA(a[0], b[0], 0, CHECK);                                                   \
      MOE_FP8_MMA(a[1], b[1], 1, CHECK);                                                   \
      if (!CHECK) sched_stage<2, FM * FN, 2 * FM + (MX ? 1 : 2) * FN,                      \
                              2 * FM + (MX ? 1 : 2) * FN + FM + FN>();                     \
    } else {                                                                               \
      _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                    \
        i32x8 a[FM], b[FN];                                                                \
        MOE_FP8_FRAGS(a, b, kk);                                                           \
        MOE_FP8_MMA(a, b, kk, CHECK);                                                      \
      }                                                                                    \
    }                                                                                      \
  }
  // Full tiles take a branch-free copy of the loop, except on the 32-row E4M3
  // tiles, whose one fragment per wave is always live (measured: the FP8
  // decode up GEMM 0.62 ms with one loop, 0.65 with two)
  if constexpr (FM > 1 || MX) {
    if (live == FM) {
      MOE_FP8_MAIN(false)
    } else {
      MOE_FP8_MAIN(true)
    }
  } else {
    MOE_FP8_MAIN(true)
  }
#undef MOE_FP8_MAIN
#undef MOE_FP8_MMA
#undef MOE_FP8_FRAGS
#undef MOE_FP8_ISSUE
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no LDS load may still be in flight

  // Stores go through buffer resources whose range is exactly the tile's valid
  // rows (consecutive rows of C and of the H scales), so a store to a row past
  // them, or given an offset outside the range, is dropped by the hardware: no
  // lane branches on its row, and addresses are 32-bit offsets from one base.
  const int ccol = lane & 31, crow = (lane >> 5) * 4;
  const __amdgpu_buffer_rsrc_t c_rs = __builtin_amdgcn_make_buffer_rsrc(
      p.C + (int64_t)tc.row0 * p.ldc, 0, tc.nrows * (int)p.ldc, 0x00020000);
  if constexpr (SW) {
    // h = SiLU(g) * u; the row maximum of |h| over this wave's columns, then over
    // the WN waves through LDS; scale 2^e = the smallest power of two with
    // max <= 448 * 2^e; codes E4M3(h * 2^-e)
    constexpr int HF = FN / 2;
    constexpr int NV = FM * 16;       // rows per lane half (lanes 0-31 / 32-63)
    constexpr int SPAN = 32 / NV;     // lanes that end up holding one row's maximum
    static_assert(NV == 16 || NV == 32, "one or two fragments of rows per wave");
    float h[FM][HF][16];
    float pmax[NV];                   // value q = 16 i + r: row 32 i + 8 (r / 4) + crow + r % 4
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float m = 0.0f;
#pragma unroll
        for (int f = 0; f < HF; ++f) {
          const float g = acc[i][f][r], u = acc[i][f + HF][r];
          h[i][f][r] = silu_mul(g, u);
          m = fmaxf(m, fabsf(h[i][f][r]));
        }
        pmax[16 * i + r] = m;
      }
    // the maxima over the 32 columns of each lane half: lane c ends with row
    // q = c / SPAN's maximum
    HalvingMax<NV, 16>::run(pmax, ccol);
    // all waves are past the main loop (their last LDS reads returned) before
    // the stage buffers are reused for the partial maxima
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
    float* part = reinterpret_cast<float*>(smem);  // [WN][BM]
    if (ccol % SPAN == 0) {
      const int q = ccol / SPAN;
      part[wn * BM + wm * WTM + 32 * (q >> 4) + 8 * ((q & 15) >> 2) + crow + (q & 3)] = pmax[0];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
    // the tile's H scales: rows row0 .. row0 + nrows - 1 of column block nt;
    // one lane per row (wave column 0, lane column 0) writes each
    const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
        q.c_scale + (int64_t)tc.nt * q.ldcs + tc.row0, 0, tc.nrows * 4, 0x00020000);
    const bool s_lane = wn == 0 && ccol == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrw = wm * WTM + 32 * i + 8 * (r >> 2) + crow + (r & 3);
        float m = 0.0f;
#pragma unroll
        for (int w = 0; w < WN; ++w) m = fmaxf(m, part[w * BM + lrw]);
        const int e = fp8_scale_exp(m);
        const float inv = ldexpf(1.0f, -e);  // exact: codes = E4M3(h * 2^-e)
        const uint32_t roff = (uint32_t)lrw * (uint32_t)p.ldc;
#pragma unroll
        for (int f = 0; f < HF; ++f) {
          const int col = tc.nt * (BN / 2) + wn * (WTN / 2) + 32 * f + ccol;
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)e4m3_code(h[i][f][r] * inv), c_rs,
                                               roff + col, 0, 0);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ldexpf(1.0f, e)), s_rs,
                                              s_lane ? (uint32_t)lrw * 4u : kOut, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrw = wm * WTM + 32 * i + 8 * (r >> 2) + crow + (r & 3);
        const uint32_t roff = (uint32_t)lrw * (uint32_t)p.ldc;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = tc.nt * BN + wn * WTN + 32 * f + ccol;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[i][f][r]), c_rs,
                                                col < p.N ? roff + col * 2 : kOut, 0, 0);
        }
      }
    }
  }
}

// FP8 / MXFP4 grouped GEMM: one tile per block.
template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int WF = WF_E4M3, int SCHED = 0>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_fp8(Fp8Args q) {
  TileCoord tc;
  if (!decode_tile<BM>(q.g, tc)) return;
  gemm_fp8_tile<BM, BN, WM, WN, EPI, STAGES, WF, SCHED>(q, tc);
}

// A tile shape of grouped_gemm_fp8_split: gemm_fp8_tile's parameters.
template <int BM_, int BN_, int WM_, int WN_, int ST_, int SCHED_ = 0>
struct Fp8Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, ST = ST_, SCHED = SCHED_;
  static constexpr int WAVES = WM_ * WN_;
};

// Both kinds of tile of a prefill-shaped batch with a skewed load in one
// launch, as grouped_gemm_dma_split does for bf16: blocks [0, n_small) walk the
// 32-row streaming tiles of `small` (Small's waves; the others end at once,
// and a barrier then waits only for the waves still running), every later
// block takes one Big tile of `big`.  The two roles write disjoint rows.
template <class Big, class Small, int EPI, int WF>
__global__ __launch_bounds__(64 * Big::WAVES, 1) void grouped_gemm_fp8_split(Fp8Args big,
                                                                            Fp8Args small,
                                                                            int n_small) {
  static_assert(Small::WAVES <= Big::WAVES && Small::BM == 32, "streaming role");
  TileCoord tc;
  const int bid = blockIdx.x;
  if (bid < n_small) {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= Small::WAVES) return;
    for (int vb = bid; decode_tile<32>(small.g, tc, vb); vb += n_small) {
      if (vb != bid) __syncthreads();
      gemm_fp8_tile<32, Small::BN, Small::WM, Small::WN, EPI, Small::ST, WF, Small::SCHED>(small, tc);
    }
    return;
  }
  if (!decode_tile<Big::BM>(big.g, tc, bid - n_small)) return;
  gemm_fp8_tile<Big::BM, Big::BN, Big::WM, Big::WN, EPI, Big::ST, WF, Big::SCHED>(big, tc);
}

}  // namespace gemm
}  // namespace moe
