// Grouped GEMMs of the MoE layer on gfx950 MFMA.
//
// One kernel template serves three contractions, all "TN" (both operands
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
// Tile pipeline: global -> registers -> LDS (XOR-swizzled 128-byte rows, two
// stages), MFMA 16x16x32 bf16 (or 16x16x4 f32) from LDS fragments, float32
// accumulation, epilogue straight from the accumulators.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

enum Epilogue { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_LOGITS = 2 };

struct GemmArgs {
  const char* A;              // operand rows (hidden or H)
  const int32_t* a_rows;      // dispatch row -> A row (nullptr: identity)
  int64_t lda;                // bytes between A rows
  const char* B;              // weights of group 0; group g at B + g * b_group
  const char* B_last;         // weights of the last group when it is not in B (shared expert)
  int64_t b_group;            // bytes between groups' weights
  int64_t ldb;                // bytes between weight rows
  int N;                      // output columns
  int up_row;                 // SwiGLU: first weight row of the up projection (d_ff)
  int K;                      // reduction length in elements
  const int32_t* g_begin;     // [G] first dispatch row of each group (nullptr: dense)
  const int32_t* g_end;       // [G] one past the last row
  const int32_t* tile_prefix; // [G+1] cumulative row-tile counts for this tile height
  int G;
  int dense_rows;             // dense mode: number of rows
  int n_tiles;                // column tiles
  char* C;                    // output rows (indexed by dispatch row)
  int64_t ldc;                // bytes between output rows
  const float* col_add;       // EPI_LOGITS: per-column addend (nullable)
};

// Byte offset of 16-byte chunk `ch` (0..7) of LDS tile row `row`.  The chunk is
// XOR-swizzled with the row so that the eight consecutive rows an MFMA fragment
// read touches at one K position fall in eight different bank groups.
__device__ __forceinline__ int lds_off(int row, int ch) {
  return (row << 7) + ((ch ^ (row & 7)) << 4);
}

template <typename TE>
struct Mma;

template <>
struct Mma<uint16_t> {  // bfloat16: one 16x16x32 step per 16-byte lane chunk
  __device__ __forceinline__ static void run(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {  // float32: four 16x16x4 steps; A and B take the same K order
  __device__ __forceinline__ static void run(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
  }
};

template <typename TE>
__device__ __forceinline__ void store_elem(char* p, float v);
template <>
__device__ __forceinline__ void store_elem<uint16_t>(char* p, float v) {
  *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void store_elem<float>(char* p, float v) {
  *reinterpret_cast<float*>(p) = v;
}

// BM x BN tile (BN = weight rows; for SwiGLU the first half are gate rows and
// the second half the matching up rows), WM x WN waves, 128 bytes of K per stage.
template <typename TE, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr bool SW = EPI == EPI_SWIGLU;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must hold whole fragments");
  static_assert(!SW || FN % 2 == 0, "SwiGLU waves hold gate and up fragments in pairs");
  constexpr int LA = ceil_div(BM * 8, NT), LB = ceil_div(BN * 8, NT);
  // whether every thread owns a chunk in every load slot (no per-thread guard)
  constexpr bool A_FULL = (BM * 8) % NT == 0, B_FULL = (BN * 8) % NT == 0;
  constexpr int STAGE = (BM + BN) * 128;
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- which tile is this block's -------------------------------------------
  const int total_m = p.g_begin ? p.tile_prefix[p.G] : ceil_div(p.dense_rows, BM);
  const int nact = total_m * p.n_tiles;
  const int bid = blockIdx.x;
  if (bid >= nact) return;
  // Blocks are handed to the 8 XCDs round-robin (block b -> XCD b % 8).  Give
  // each XCD a contiguous run of logical tiles, column tile fastest, so the
  // blocks sharing a row tile's operand rows share one L2.
  const int q8 = nact >> 3, r8 = nact & 7, xcd = bid & 7;
  const int logical = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int mt = logical / p.n_tiles, nt = logical - mt * p.n_tiles;
  int grp = 0, row0, nrows;
  if (p.g_begin) {
    int lo = 0, hi = p.G - 1;  // last group whose first tile is <= mt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tile_prefix[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    grp = lo;
    row0 = p.g_begin[grp] + (mt - p.tile_prefix[grp]) * BM;
    nrows = min(BM, p.g_end[grp] - row0);
  } else {
    row0 = mt * BM;
    nrows = min(BM, p.dense_rows - row0);
  }
  const char* Bg = (p.B_last && grp == p.G - 1) ? p.B_last : p.B + (int64_t)grp * p.b_group;

  // ---- per-thread global sources and LDS destinations ------------------------
  // Row slots past the tile's valid rows read the tile's first row: their
  // results are never stored, and every read stays inside the operand.
  const char* a_src[LA];
  int a_dst[LA];
  bool a_on[LA];
#pragma unroll
  for (int c = 0; c < LA; ++c) {
    const int lin = c * NT + tid, row = lin >> 3, ch = lin & 7;
    a_on[c] = A_FULL || lin < BM * 8;
    const int rr = (row < nrows) ? row : 0;
    const int arow = p.a_rows ? p.a_rows[row0 + rr] : row0 + rr;
    a_src[c] = p.A + (int64_t)arow * p.lda + ch * 16;
    a_dst[c] = lds_off(row, ch);
  }
  const char* b_src[LB];
  int b_dst[LB];
  bool b_on[LB];
#pragma unroll
  for (int c = 0; c < LB; ++c) {
    const int lin = c * NT + tid, row = lin >> 3, ch = lin & 7;
    b_on[c] = B_FULL || lin < BN * 8;
    int brow;
    if (SW) {
      brow = (row < BN / 2) ? nt * (BN / 2) + row : p.up_row + nt * (BN / 2) + (row - BN / 2);
    } else {
      brow = nt * BN + row;
      if (brow >= p.N) brow = p.N - 1;
    }
    b_src[c] = Bg + (int64_t)brow * p.ldb + ch * 16;
    b_dst[c] = BM * 128 + lds_off(row, ch);
  }

  const int KT = (p.K * (int)sizeof(TE)) >> 7;
  u32x4 ra[LA], rb[LB];
#pragma unroll
  for (int c = 0; c < LA; ++c)
    if (a_on[c]) ra[c] = *reinterpret_cast<const u32x4*>(a_src[c]);
#pragma unroll
  for (int c = 0; c < LB; ++c)
    if (b_on[c]) rb[c] = *reinterpret_cast<const u32x4*>(b_src[c]);
#pragma unroll
  for (int c = 0; c < LA; ++c)
    if (a_on[c]) *reinterpret_cast<u32x4*>(smem + a_dst[c]) = ra[c];
#pragma unroll
  for (int c = 0; c < LB; ++c)
    if (b_on[c]) *reinterpret_cast<u32x4*>(smem + b_dst[c]) = rb[c];
  __syncthreads();

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS rows of this lane's fragments
  const int frow = lane & 15, fq = lane >> 4;
  int a_row[FM], b_row[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_row[i] = wm * WTM + 16 * i + frow;
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    if (SW)
      b_row[f] = (f < FN / 2) ? wn * (WTN / 2) + 16 * f : BN / 2 + wn * (WTN / 2) + 16 * (f - FN / 2);
    else
      b_row[f] = wn * WTN + 16 * f;
    b_row[f] += frow;
  }

  for (int kt = 0; kt < KT; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE;
    const bool more = kt + 1 < KT;
    if (more) {
      const int off = (kt + 1) << 7;
#pragma unroll
      for (int c = 0; c < LA; ++c)
        if (a_on[c]) ra[c] = *reinterpret_cast<const u32x4*>(a_src[c] + off);
#pragma unroll
      for (int c = 0; c < LB; ++c)
        if (b_on[c]) rb[c] = *reinterpret_cast<const u32x4*>(b_src[c] + off);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + fq;
      u32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(cur + lds_off(a_row[i], ch));
#pragma unroll
      for (int f = 0; f < FN; ++f)
        fb[f] = *reinterpret_cast<const u32x4*>(cur + BM * 128 + lds_off(b_row[f], ch));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f) Mma<TE>::run(acc[i][f], fa[i], fb[f]);
    }
    if (more) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int c = 0; c < LA; ++c)
        if (a_on[c]) *reinterpret_cast<u32x4*>(nxt + a_dst[c]) = ra[c];
#pragma unroll
      for (int c = 0; c < LB; ++c)
        if (b_on[c]) *reinterpret_cast<u32x4*>(nxt + b_dst[c]) = rb[c];
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds C[4*(lane/16) + r][lane % 16] of each fragment ----
  const int ccol = lane & 15, crow = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = wm * WTM + 16 * i + crow + r;
      if (lr >= nrows) continue;
      char* crow_ptr = p.C + (int64_t)(row0 + lr) * p.ldc;
      if (SW) {
#pragma unroll
        for (int f = 0; f < FN / 2; ++f) {
          const float g = acc[i][f][r], u = acc[i][f + FN / 2][r];
          const float h = g / (1.0f + expf(-g)) * u;
          const int col = nt * (BN / 2) + wn * (WTN / 2) + 16 * f + ccol;
          store_elem<TE>(crow_ptr + (int64_t)col * sizeof(TE), h);
        }
      } else {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = nt * BN + wn * WTN + 16 * f + ccol;
          if (col >= p.N) continue;
          if (EPI == EPI_LOGITS) {
            const float v = acc[i][f][r] + (p.col_add ? p.col_add[col] : 0.0f);
            reinterpret_cast<float*>(crow_ptr)[col] = v;
          } else {
            store_elem<TE>(crow_ptr + (int64_t)col * sizeof(TE), acc[i][f][r]);
          }
        }
      }
    }
  }
}

template <typename TE, int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_gemm(const GemmArgs& p, int m_tiles_bound, hipStream_t s) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDS = 2 * (BM + BN) * 128;
  const int grid = m_tiles_bound * p.n_tiles;
  if (grid <= 0) return hipSuccess;
  auto kern = grouped_gemm_kernel<TE, BM, BN, WM, WN, EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), LDS, s, p);
  return hipGetLastError();
}

// Upper bound on sum_g ceil(M_g / bm) given sum_g M_g <= rows over at most
// `groups` non-empty groups.
int tile_bound(int64_t rows, int groups, int bm) {
  const int64_t ne = rows < groups ? rows : groups;
  return (int)((rows + ne * (bm - 1)) / bm);
}

}  // namespace

hipError_t launch_router_gemm(const moe_config& c, const void* hidden, const void* w_router,
                              const float* logit_offset, float* logits, hipStream_t s) {
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
  p.C = reinterpret_cast<char*>(logits);
  p.ldc = (int64_t)c.E * 4;
  p.col_add = logit_offset;
  if (c.dtype == MOE_F32) {
    p.n_tiles = ceil_div(c.E, 16);
    return launch_gemm<float, 16, 16, 1, 1, EPI_LOGITS>(p, ceil_div(c.T, 16), s);
  }
  p.n_tiles = ceil_div(c.E, 64);
  return launch_gemm<uint16_t, 64, 64, 2, 2, EPI_LOGITS>(p, ceil_div(c.T, 64), s);
}

namespace {

// Tile shape of the grouped expert GEMMs.  Rows per group on average (known on
// the host from T, k and the group count) picks skinny 16-row tiles for
// decode-shaped batches and 128-row tiles otherwise.
enum class FfnTiles { F32_16, BF16_16, BF16_128 };

FfnTiles pick_tiles(const moe_config& c, const ExpertFfnArgs& a) {
  if (c.dtype == MOE_F32) return FfnTiles::F32_16;
  const int64_t avg_rows = a.rows_bound / (a.n_groups > 0 ? a.n_groups : 1);
  return avg_rows < 48 ? FfnTiles::BF16_16 : FfnTiles::BF16_128;
}

int tile_rows(FfnTiles t) { return t == FfnTiles::BF16_128 ? 128 : 16; }

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
    default:
      g.n_tiles = ceil_div(c.d, 128);
      return launch_gemm<uint16_t, 128, 128, 2, 2, EPI_STORE>(g, mb, s);
  }
}

}  // namespace moe
