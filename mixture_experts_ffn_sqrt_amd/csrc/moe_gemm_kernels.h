// Grouped GEMM kernel templates (device code) of the MoE layer; instantiated by
// moe_gemm.hip.  See moe_gemm.hip for what the three contractions are.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace gemm {

// SiLU(g) * u = g * u / (1 + exp(-g)) with the hardware exp2 and reciprocal
// (each within about 1 ulp of float32; the result is rounded to bf16 or E4M3
// afterwards).  exp(-g) overflows to infinity for g below about -88, and the
// product is then -0, as the exact value rounds.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);  // exp(-g) = 2^(-g log2 e)
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

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
  char* C;                    // output rows: dispatch rows (grouped) or A rows (dense)
  int64_t ldc;                // bytes between output rows
  const float* col_add;       // EPI_LOGITS: per-column addend (nullable)
  int k_chunk;                // dense split-K: elements of K per grid row y (0: no split)
  int64_t c_split;            // dense split-K: bytes between the partial outputs of y and y+1
  uint32_t a_bytes;           // bytes of the A operand (buffer range; < 2^31)
  uint32_t b_bytes;           // bytes of one group's weights (buffer range; < 2^31)
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

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct TileCoord {
  int grp, row0, nrows, nt;
};

// Row tiles of one group that run next to each other on an XCD (see
// decode_tile).
constexpr int kSuperRows = 8;

// Which tile this block owns; false: nothing to do.
//
// Tiles: group g's rows are cut into tile_prefix[g+1] - tile_prefix[g] tiles
// of group_tile_rows(M_g, BM) rows (dense mode: one group of dense_rows rows),
// times n_tiles column tiles.  Order: group by group; inside a group, row tiles
// are taken in super-rows of at most kSuperRows (near-equal heights), and a
// super-row is walked column by column with its row tiles fastest.  So the
// tiles that run together share one weight panel per column and a handful of
// operand panels, and every tile of a super-row has about the same work,
// which keeps co-running blocks in step and their K slabs in L2.
//
// Blocks are handed to the 8 XCDs round-robin (block b -> XCD b % 8).
// Tiles of more than 32 rows reach them in chunks of kXcdChunk consecutive
// tiles of the order above: chunk c runs on XCD c % 8, so every part of the
// order, e.g. a shared expert's full tiles at its end, is spread over all
// XCDs and they take about the same work (measured on the DeepSeek-shaped
// prefill batches: 3-6% per layer over contiguous runs, 1% on Mixtral).
// 32-row (decode) tiles, which stream each expert's weights once, go in one
// contiguous run per XCD: XCD x takes tiles x*q + min(x, r) + b/8 (q, r: the
// tile count divided by 8), measured 4% faster there than chunks.  (The grid
// is a whole number of 8 * kXcdChunk blocks; blocks past the tiles exit.)
//
// `vbid` (default: the block index) is the block's number in this order: a
// persistent block walks virtual blocks vbid, vbid + n, ..., and a block of a
// launch that serves two tile lists counts from the first block of its list.
// Whenever vbid and the block index agree modulo 8, every tile runs on the XCD
// the mapping assumes.
template <int BM>
__device__ __forceinline__ bool decode_tile(const GemmArgs& p, TileCoord& tc, int vbid = -1) {
  const int nt_all = p.n_tiles;
  const int total_m = p.g_begin ? p.tile_prefix[p.G] : group_tiles(p.dense_rows, BM);
  const int nact = total_m * nt_all;
  const int bid = vbid < 0 ? (int)blockIdx.x : vbid, i = bid >> 3, xcd = bid & 7;
  int logical;
  if constexpr (BM > 32) {
    logical = ((i / kXcdChunk) * 8 + xcd) * kXcdChunk + i % kXcdChunk;
    if (logical >= nact) return false;
  } else {
    if (bid >= nact) return false;
    const int q8 = nact >> 3, r8 = nact & 7;
    logical = xcd * q8 + min(xcd, r8) + i;
  }

  int g = 0, t0 = 0, mt_g = total_m, M = p.dense_rows, rbeg = 0;
  if (p.g_begin) {
    // the group whose tiles [tile_prefix[g], tile_prefix[g+1]) * n_tiles hold it
    const int r = logical / nt_all;
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tile_prefix[mid] <= r) lo = mid; else hi = mid - 1;
    }
    g = lo;
    t0 = p.tile_prefix[g];
    mt_g = p.tile_prefix[g + 1] - t0;
    rbeg = p.g_begin[g];
    M = p.g_end[g] - rbeg;
  }
  const int l = logical - t0 * nt_all;  // tile index inside the group
  const int nsr = ceil_div(mt_g, kSuperRows);
  const int base = mt_g / nsr, extra = mt_g - base * nsr;  // first `extra` super-rows: base + 1
  const int rt = l / nt_all;
  int s0, h;
  if (rt < extra * (base + 1)) {
    h = base + 1;
    s0 = (rt / h) * h;
  } else {
    h = base;
    s0 = extra * (base + 1) + ((rt - extra * (base + 1)) / base) * base;
  }
  const int ls = l - s0 * nt_all;
  tc.nt = ls / h;
  const int mt = s0 + (ls - tc.nt * h);
  const int c = group_tile_rows(M, BM);
  tc.grp = g;
  tc.row0 = rbeg + mt * c;
  tc.nrows = min(c, M - mt * c);
  return true;
}

// Register-staged kernel (any element type; small tiles): BM x BN tile (BN =
// weight rows; for SwiGLU the first half are gate rows and the second half the
// matching up rows), WM x WN waves, MFMA 16x16, 128 bytes of K per stage, the
// next stage loaded to registers while the current one is multiplied from LDS.
template <typename TE, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm_staged(GemmArgs p) {
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

  TileCoord tc;
  if (!decode_tile<BM>(p, tc)) return;
  const int grp = tc.grp, row0 = tc.row0, nrows = tc.nrows, nt = tc.nt;
  if (p.k_chunk) {  // split-K over grid rows: this block's slice of K and its partial output
    const int64_t ko = (int64_t)blockIdx.y * p.k_chunk * (int64_t)sizeof(TE);
    p.A += ko;
    p.B += ko;
    p.C += (int64_t)blockIdx.y * p.c_split;
    p.K = p.k_chunk;
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
          const float h = silu_mul(g, u);
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


// ---------------------------------------------------------------------------
// Direct-to-LDS bf16 kernel: direct global->LDS buffer loads (16 bytes per lane;
// a wavefront's load fills 1 KB of LDS, lane l at byte 16*l), STAGES LDS
// buffers of ROWB/2 K-elements (ROWB bytes per tile row), loads issued
// STAGES-1 stages ahead, one barrier per stage, MFMA 32x32x16.
//
// LDS row layout: row r holds ROWB/16 16-byte chunks; logical chunk c sits in
// slot c ^ swz(r).  A fragment read (ds_read_b128) is served 16 lanes at a
// time, i.e. 16 consecutive rows at one K position; gfx950's LDS has 64 banks
// (256 bytes per cycle), so the swizzle must spread those 16 rows over all 16
// bank groups: (r >> 2) & 3 does for 64-byte rows and (r >> 1) & 7 for
// 128-byte rows (4 cycles per read, measured), while the plain layout costs 4x
// (64-byte rows) or 8x (128-byte rows).
// ---------------------------------------------------------------------------
// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding (vmcnt in bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their no-wait maxima)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Wait until at most MUL * n of this wave's vector-memory loads are in flight,
// for a wave-uniform n in [N0, N0 + 3] (s_waitcnt takes an immediate; an n
// below the range waits for MUL * N0, which is never too few).
template <int MUL, int N0>
__device__ __forceinline__ void wait_loads_le(int n) {
  static_assert(N0 >= 0 && MUL * (N0 + 3) <= 63, "vmcnt range");
  switch (n - N0) {
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(MUL * (N0 + 1))); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(MUL * (N0 + 2))); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(MUL * (N0 + 3))); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(MUL * N0)); break;
  }
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Workgroup barrier without a memory fence (so outstanding direct-to-LDS loads
// need not drain), fenced for the compiler: no LDS access may be moved across
// it, since the barrier is what orders one wave's LDS reads against another
// wave's loads into the same buffer.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// one 16-byte-per-lane buffer load straight into LDS at `dst` (+16 * lane),
// with cache policy POL (the buffer instruction's cache-policy bits)
template <int POL = 0>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 16, voff, 0, 0, POL);
}

// Cache policy of the weight loads of the 32-row streaming tiles (decode, and
// the groups of a few rows on a skewed prefill batch): they read every weight
// once, and the non-temporal bit (NT) lets the L2 let go of those lines first.
// A block-contiguous read stream runs at 6.9-7.0 TB/s with it against 6.2
// without; the decode GEMMs of V4-Flash shapes 6-7% faster (bf16 and E4M3),
// V4-Pro's bf16 up GEMM 1%.  Not for the larger tiles, whose co-running tiles
// share weight panels through the L2 (Mixtral and V4-Pro 3-5% slower with it).
// E2M1 weights take it only because their rows are stored in pairs: with
// row-major codes one K stage reads 64 bytes of each 128-byte line and leaves
// the rest to the next stage, which NT made 36% slower.
constexpr int kStreamWeightPolicy = 2;  // NT

// one 4-byte-per-lane buffer load straight into LDS at `dst` (+4 * lane)
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 4, voff, 0, 0, 0);
}

// Swizzle of the 16-byte chunks of an LDS row, from the row index modulo 32:
// SWZ 0 = none, 1 = (r>>1 ^ r>>3), 2 = r, 3 = r>>1, 4 = r>>2 (masked to the
// chunk count).
template <int ROWB, int SWZ>
__device__ __forceinline__ int swz_sel(int r) {
  constexpr int M = ROWB / 16 - 1;
  r &= 31;  // fragment reads see the row modulo 32: the writes must agree
  if constexpr (SWZ == 0) return 0;
  else if constexpr (SWZ == 1) return ((r >> 1) ^ (r >> 3)) & M;
  else if constexpr (SWZ == 2) return r & M;
  else if constexpr (SWZ == 3) return (r >> 1) & M;
  else return (r >> 2) & M;
}

// Instruction order of one stage of a scheduled main loop: the R0 LDS reads
// that come first (the first k-step's fragments, and any per-stage scale
// reads), then for every k-step but the last its M MFMAs, each followed by its
// share of the next k-step's R fragment reads, then the last k-step's MFMAs.
// A wave then multiplies one k-step while the next one's fragments are on
// their way from LDS, instead of waiting for each k-step's reads in turn.
// (Scheduling only: the compiler keeps every dependence whatever the groups
// say.  0x008: MFMA, 0x100: LDS read.)
template <int J, int M, int R>
struct SchedInterleave {
  __device__ __forceinline__ static void run() {
    constexpr int n = (R * (J + 1) + M - 1) / M - (R * J + M - 1) / M;  // reads after MFMA J
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
    SchedInterleave<J + 1, M, R>::run();
  }
};
template <int M, int R>
struct SchedInterleave<M, M, R> {
  __device__ __forceinline__ static void run() {}
};
template <int KS, int M, int R, int R0 = R>
__device__ __forceinline__ void sched_stage() {
  __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);
#pragma unroll
  for (int kk = 0; kk < KS - 1; ++kk) SchedInterleave<0, M, R>::run();
  __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
}

// One tile of grouped_gemm_dma (below).
// SCHED = 1: fragments double-buffered in registers across the k-steps of a
// stage, in the order sched_stage fixes (full tiles only).
template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int ROWB, int SWZ, int SCHED>
__device__ __forceinline__ void gemm_dma_tile(const GemmArgs& p, const TileCoord& tc) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr int KSTEPS = ROWB / 32;                 // MFMA k-steps of 16 bf16 per stage
  constexpr int CPR = ROWB / 16;                    // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;                  // rows filled by one wavefront load
  constexpr int A_STAGE = BM * ROWB, B_STAGE = BN * ROWB;
  constexpr int B_RING = STAGES * A_STAGE;          // LDS offset of the B ring
  // 1 KB loads per stage: NA of A rows, NB of B rows; wave w issues A blocks
  // w + NW*j (j < LA) and B blocks w + NW*j (j < LB, block < NB)
  constexpr int NA = BM / RPL, NB = BN / RPL;
  constexpr int LA = NA / NW, LB = (NB + NW - 1) / NW;
  constexpr bool B_EVEN = NB % NW == 0;
  constexpr int B_POL = BM <= 32 && ROWB == 128 ? kStreamWeightPolicy : 0;  // whole 128-byte lines
  static_assert(ROWB == 64 || ROWB == 128, "64- or 128-byte LDS rows");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "whole 32x32 fragments");
  static_assert(!SW || FN % 2 == 0, "SwiGLU waves hold gate and up fragments in pairs");
  static_assert(NA * RPL == BM && NB * RPL == BN && LA * NW == NA, "A loads must split evenly");
  static_assert(!SW || (BN / 2) % RPL == 0, "a load is all gate or all up rows");
  static_assert(STAGES >= 2 && B_RING + STAGES * B_STAGE <= 160 * 1024, "LDS budget");
  extern __shared__ __align__(16) char smem[];

  // the wavefront index is uniform: say so, so that everything derived from it
  // (LDS bases, fragment liveness) lives in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const char* Bg = (p.B_last && tc.grp == p.G - 1) ? p.B_last : p.B + (int64_t)tc.grp * p.b_group;
  constexpr uint32_t kOut = 0x80000000u;
  const __amdgpu_buffer_rsrc_t a_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.A), 0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Bg), 0, (int)p.b_bytes, 0x00020000);

  // Load slot j of this wave covers tile rows [RPL * (wave + NW * j), +RPL); lane
  // l fills LDS slot l % CPR of row l / CPR, i.e. logical chunk slot ^ swz(row).
  const int lr = lane / CPR, lq = lane % CPR;
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int row = RPL * (wave + NW * j) + lr;
    const int ch = lq ^ swz_sel<ROWB, SWZ>(row);
    if (row < tc.nrows) {
      const int arow = p.a_rows ? p.a_rows[tc.row0 + row] : tc.row0 + row;
      a_off[j] = (uint32_t)arow * (uint32_t)p.lda + ch * 16;
    } else {
      a_off[j] = kOut;
    }
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int row = RPL * (wave + NW * j) + lr;
    const int ch = lq ^ swz_sel<ROWB, SWZ>(row);
    int brow;
    bool ok = true;
    if (SW) {
      brow = (RPL * (wave + NW * j) < BN / 2) ? tc.nt * (BN / 2) + row
                                              : p.up_row + tc.nt * (BN / 2) + (row - BN / 2);
    } else {
      brow = tc.nt * BN + row;
      ok = brow < p.N;
    }
    b_off[j] = ok ? (uint32_t)brow * (uint32_t)p.ldb + ch * 16 : kOut;
  }
  // the last B slot exists on waves whose block wave + NW*(LB-1) is < NB
  const bool b_last = B_EVEN || wave + NW * (LB - 1) < NB;
  const int KT = p.K / (ROWB / 2);  // ROWB/2 bf16 per stage
  // Stage kt's A and B loads (A and B in rings of their own); stages past the
  // end reload the last one (never read; keeps the number of loads in flight
  // constant).
#define MOE_DMA_ISSUE_A(kt_)                                                              \
  do {                                                                                   \
    const int kc_ = (kt_) < KT ? (kt_) : KT - 1;                                         \
    char* buf_ = smem + ((kt_) % STAGES) * A_STAGE;                                      \
    const uint32_t ko_ = (uint32_t)kc_ * ROWB;                                           \
    _Pragma("unroll") for (int j = 0; j < LA; ++j)                                        \
        load_lds16(a_rs, buf_ + (RPL * (wave + NW * j)) * ROWB, a_off[j] + ko_);         \
  } while (0)
#define MOE_DMA_ISSUE_B(kt_)                                                              \
  do {                                                                                   \
    const int kc_ = (kt_) < KT ? (kt_) : KT - 1;                                         \
    char* buf_ = smem + B_RING + ((kt_) % STAGES) * B_STAGE;                             \
    const uint32_t ko_ = (uint32_t)kc_ * ROWB;                                           \
    _Pragma("unroll") for (int j = 0; j < LB; ++j) {                                      \
      if (j == LB - 1 && !b_last) break;                                                 \
      load_lds16<B_POL>(b_rs, buf_ + (RPL * (wave + NW * j)) * ROWB, b_off[j] + ko_);    \
    }                                                                                    \
  } while (0)

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  // fragment read offsets: row lane % 32 of each fragment, chunk 2*kk + lane/32
  const int fr = lane & 31, fh = lane >> 5, fs = swz_sel<ROWB, SWZ>(fr);
  int a_rd[KSTEPS], b_rd[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const int sl = ((2 * kk + fh) ^ fs) << 4;
    a_rd[kk] = (wm * WTM + fr) * ROWB + sl;
    b_rd[kk] = fr * ROWB + sl;
  }
  int b_row[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f)
    b_row[f] = SW ? ((f < FN / 2) ? wn * (WTN / 2) + 32 * f : BN / 2 + wn * (WTN / 2) + 32 * (f - FN / 2))
                  : wn * WTN + 32 * f;

  // Fragments of this wave whose 32 rows hold at least one valid row; a full
  // tile takes the branch-free loop.
  const int live = min(FM, max(0, (tc.nrows - wm * WTM + 31) / 32));

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) {
    MOE_DMA_ISSUE_A(st);
    MOE_DMA_ISSUE_B(st);
  }
  // fragment reads of k-step kk_ of the stage at cur into fa_ / fb_, and that
  // k-step's MFMAs (fragments with no valid row skipped when CHECK)
#define MOE_DMA_FRAGS(fa_, fb_, kk_)                                                          \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                            \
        fa_[i] = *reinterpret_cast<const u32x4*>(curA + a_rd[kk_] + i * 32 * ROWB);          \
    _Pragma("unroll") for (int f = 0; f < FN; ++f)                                            \
        fb_[f] = *reinterpret_cast<const u32x4*>(curB + b_rd[kk_] + b_row[f] * ROWB);        \
  } while (0)
#define MOE_DMA_MMA(fa_, fb_, CHECK)                                                          \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                          \
      if (CHECK && i >= live) continue;                                                      \
      _Pragma("unroll") for (int f = 0; f < FN; ++f)                                          \
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                               \
              __builtin_bit_cast(bf16x8, fa_[i]), __builtin_bit_cast(bf16x8, fb_[f]),        \
              acc[i][f], 0, 0, 0);                                                           \
    }                                                                                        \
  } while (0)
#define MOE_DMA_MAIN(CHECK)                                                                   \
  for (int kt = 0; kt < KT; ++kt) {                                                          \
    /* at most STAGES-2 later stages' loads in flight: LA + LB per stage, one */           \
    /* fewer on waves without the last B slot */                                             \
    wait_loads_le<STAGES - 2, LA + LB - 1>(LA + LB - (b_last ? 0 : 1));                      \
    __builtin_amdgcn_s_waitcnt(0xC07F);                                                      \
    lds_barrier();                                                                           \
    MOE_DMA_ISSUE_A(kt + STAGES - 1);                                                         \
    MOE_DMA_ISSUE_B(kt + STAGES - 1);                                                         \
    const char* curA = smem + (kt % STAGES) * A_STAGE;                                       \
    const char* curB = smem + B_RING + (kt % STAGES) * B_STAGE;                              \
    if constexpr (SCHED) {                                                                   \
      u32x4 fa[2][FM], fb[2][FN];                                                            \
      MOE_DMA_FRAGS(fa[0], fb[0], 0);                                                        \
      _Pragma("unroll") for (int kk = 0; kk < KSTEPS; ++kk) {                                \
        if (kk + 1 < KSTEPS)                                                                 \
          MOE_DMA_FRAGS(fa[(kk + 1) & 1], fb[(kk + 1) & 1], (kk + 1) % KSTEPS);              \
        MOE_DMA_MMA(fa[kk & 1], fb[kk & 1], CHECK);                                          \
      }                                                                                      \
      if (!CHECK) sched_stage<KSTEPS, FM * FN, FM + FN>();                                   \
    } else {                                                                                 \
      _Pragma("unroll") for (int kk = 0; kk < KSTEPS; ++kk) {                                \
        u32x4 fa[FM], fb[FN];                                                                \
        MOE_DMA_FRAGS(fa, fb, kk);                                                           \
        MOE_DMA_MMA(fa, fb, CHECK);                                                          \
      }                                                                                      \
    }                                                                                        \
  }
  if (live == FM) {
    MOE_DMA_MAIN(false)
  } else {
    MOE_DMA_MAIN(true)
  }
#undef MOE_DMA_MAIN
#undef MOE_DMA_MMA
#undef MOE_DMA_FRAGS
#undef MOE_DMA_ISSUE_A
#undef MOE_DMA_ISSUE_B
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no LDS load may still be in flight at exit

  // epilogue: lane holds C[8*(r/4) + 4*(lane/32) + r%4][lane % 32] of each
  // fragment.  The stores go through a buffer resource whose range is exactly
  // the tile's valid rows (they are consecutive rows of C), so a store to a row
  // past them, or to a column past N (given an offset outside the range), is
  // dropped by the hardware: no lane branches on its row or column, and every
  // address is a 32-bit offset from one base.
  const int ccol = lane & 31, crow = (lane >> 5) * 4;
  const __amdgpu_buffer_rsrc_t c_rs = __builtin_amdgcn_make_buffer_rsrc(
      p.C + (int64_t)tc.row0 * p.ldc, 0, tc.nrows * (int)p.ldc, 0x00020000);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lrw = wm * WTM + 32 * i + 8 * (r >> 2) + crow + (r & 3);
      const uint32_t roff = (uint32_t)lrw * (uint32_t)p.ldc;
      if (SW) {
#pragma unroll
        for (int f = 0; f < FN / 2; ++f) {
          const float g = acc[i][f][r], u = acc[i][f + FN / 2][r];
          const float h = silu_mul(g, u);
          const int col = tc.nt * (BN / 2) + wn * (WTN / 2) + 32 * f + ccol;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(h), c_rs, roff + col * 2, 0, 0);
        }
      } else {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = tc.nt * BN + wn * WTN + 32 * f + ccol;
          if (EPI == EPI_LOGITS) {
            const float v = acc[i][f][r] + (p.col_add && col < p.N ? p.col_add[col] : 0.0f);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), c_rs,
                                                  col < p.N ? roff + col * 4 : kOut, 0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[i][f][r]), c_rs,
                                                  col < p.N ? roff + col * 2 : kOut, 0, 0);
          }
        }
      }
    }
  }
}

// Direct-to-LDS grouped GEMM: one tile per block.
template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int ROWB, int SWZ, int SCHED = 0>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_dma(GemmArgs p) {
  TileCoord tc;
  if (!decode_tile<BM>(p, tc)) return;
  if (p.k_chunk) {  // split-K over grid rows (dense bf16): K slice y, partial output y
    const uint32_t ko = (uint32_t)blockIdx.y * (uint32_t)p.k_chunk * 2u;
    p.A += ko;
    p.B += ko;
    p.a_bytes -= ko;  // the buffer ranges still end where the operands end
    p.b_bytes -= ko;
    p.C += (int64_t)blockIdx.y * p.c_split;
    p.K = p.k_chunk;
  }
  gemm_dma_tile<BM, BN, WM, WN, EPI, STAGES, ROWB, SWZ, SCHED>(p, tc);
}

// Tile shapes of the two roles of grouped_gemm_dma_split (the grouped GEMMs of
// a prefill-shaped batch with a skewed load): 288 x 256 tiles on 12 waves with
// the scheduled main loop for the groups of more than 32 rows, and 32 x 256
// streaming tiles (4 waves, a four-stage ring of weight loads) for the others.
constexpr int kSplitBigWaves = 12, kSplitSmallWaves = 4;
constexpr int kSplitLds = 4 * (32 + 256) * 128;  // the larger of the two rings
static_assert(kSplitLds >= 2 * (288 + 256) * 128, "LDS of the 288-row role");

// Both kinds of tile in one launch: blocks [0, n_small) walk the streaming
// tiles of `small` in turn (block b takes the tiles of virtual blocks b,
// b + n_small, ..., which keeps each on the XCD the tile order assumes, since
// n_small is a multiple of 8), and every later block takes one 288-row tile of
// `big`.  The hardware dispatches blocks in index order, so the streaming
// blocks start first on n_small CUs and the 288-row tiles fill the others and,
// as the streaming blocks finish, theirs too.  The streaming tiles use 4 of
// the 12 waves; the other 8 end at once, and a barrier then waits only for the
// waves still running (S_BARRIER in the CDNA ISA).  The two roles write
// disjoint output rows.
template <int EPI>
__global__ __launch_bounds__(64 * kSplitBigWaves, 1) void grouped_gemm_dma_split(
    GemmArgs big, GemmArgs small, int n_small) {
  TileCoord tc;
  const int bid = blockIdx.x;
  if (bid < n_small) {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kSplitSmallWaves) return;
    for (int vb = bid; decode_tile<32>(small, tc, vb); vb += n_small) {
      if (vb != bid) __syncthreads();
      gemm_dma_tile<32, 256, 1, kSplitSmallWaves, EPI, 4, 128, 3, 0>(small, tc);
    }
    return;
  }
  if (!decode_tile<288>(big, tc, bid - n_small)) return;
  gemm_dma_tile<288, 256, 3, 4, EPI, 2, 128, 3, 1>(big, tc);
}

}  // namespace gemm
}  // namespace moe
