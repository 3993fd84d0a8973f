// Routing: affinity scores, selection key, optional group stage, top-k and gates.
//
// Affinity ("MoE 架构与路由策略", equation dsv4-moe-softplus; "MoE 的算量与通信" 二.2):
//   softmax      selection on the logit, gates = softmax over the selected logits
//   sigmoid      s = 1 / (1 + e^-l)
//   sqrt(softplus) s = sqrt(ln(1 + e^l)), evaluated as sqrt(max(l,0) + log1p(e^-|l|))
// Selection key = s + bias (bias picks experts, gates use the unbiased s:
// "MoE 的算量与通信" 七.3).  Group stage (DeepSeek-V3 node-limited routing, same
// pages' V3 section and 五.3): a group scores the sum, largest first, of its
// group_topk largest keys; the topk_group best groups stay eligible.  Top-k in
// descending key order, equal keys to the lower expert id.  Gates: selected s
// over their sum (1/k when the sum is 0).
// Hash routing ("DeepSeek-V4 MoE" 二, HashTopK): ids = tid2eid[token id]; gates
// from the affinities at those ids.
//
// One 64-lane wavefront per token.  Lane l holds experts l, l+64, ... (up to 16
// per lane, E <= 1024).  Each top-k round is a wavefront max over 64-bit keys
// (order-preserving float bits above, inverted expert id below).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxPerLane = 16;  // E <= 1024: experts e = lane + 64 i, i < 16
constexpr int kWavesPerBlock = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TopkArgs {
  const float* logits;   // [T, E] (when nparts == 0)
  const float* parts;    // [nparts, T, part_ld] partial logits (when nparts > 0)
  int nparts, part_ld;
  const float* offset;   // [E] added to summed partials, or nullptr
  float* logits_out;     // [T, E] summed logits, or nullptr
  const float* bias;     // [E] or nullptr
  const int32_t* token_ids;
  const int32_t* tid2eid;
  int32_t* ids;          // [T, k]
  float* weights;        // [T, k]
  int T, E, k, scoring, mode, n_group, topk_group, group_topk, vocab;
};

__device__ __forceinline__ float affinity(float l, int scoring) {
  if (scoring == MOE_SCORE_SIGMOID) return 1.0f / (1.0f + expf(-l));
  if (scoring == MOE_SCORE_SQRTSOFTPLUS) return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));
  return l;
}

// float -> uint32 with the same order (finite and infinite values); -0 and +0
// compare equal as floats, so both map to the bits of +0
__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
  return (static_cast<uint64_t>(order_bits(key)) << 32) | static_cast<uint32_t>(~idx);
}

// the float whose order_bits are b (-0 comes back as +0)
__device__ __forceinline__ float from_order_bits(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
}

// maximum over each aligned segment of `width` lanes (a power of two <= 64)
__device__ __forceinline__ uint64_t segment_max_u64(uint64_t v, int width) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    if (off >= width) continue;  // uniform
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off);
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off);
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Gates for the expert `e` held by lane j < k (e < 0: an invalid slot), and the
// output stores.
__device__ __forceinline__ void write_gates(const TopkArgs& p, const float* l, int t, int lane,
                                            int e) {
  const bool mine = lane < p.k && e >= 0;
  const float lg = mine ? l[e] : 0.0f;
  float g;
  if (p.scoring == MOE_SCORE_SOFTMAX) {
    const float lmax = wave_max(mine ? lg : -INFINITY);
    const float ex = mine ? expf(lg - lmax) : 0.0f;
    g = ex / wave_sum(ex);
  } else {
    const float s = mine ? affinity(lg, p.scoring) : 0.0f;
    const float sum = wave_sum(s);
    g = sum > 0.0f ? s / sum : 1.0f / static_cast<float>(p.k);
  }
  if (lane < p.k) {
    p.ids[static_cast<int64_t>(t) * p.k + lane] = mine ? e : -1;
    p.weights[static_cast<int64_t>(t) * p.k + lane] = mine ? g : 0.0f;
  }
}

// NS = experts per lane (E <= 64 NS), so that the selection rounds touch only
// the slots that hold experts
template <int NS>
__global__ __launch_bounds__(64 * kWavesPerBlock) void topk_kernel(TopkArgs p) {
  // per wavefront: the token's logits and (group stage) its keys, E <= 64 NS
  __shared__ float skey[kWavesPerBlock][64 * NS];
  __shared__ float slog[kWavesPerBlock][64 * NS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kWavesPerBlock + wave;
  if (t >= p.T) return;  // whole wavefronts only; no block barrier below
  // this token's logits row, in LDS: the given row, or the sum of the split-K
  // partials taken in a fixed order (part 0 first) plus the offset
  float* l = slog[wave];
  if (p.nparts > 0) {
    const int64_t pstride = static_cast<int64_t>(p.T) * p.part_ld;
    const float* prow = p.parts + static_cast<int64_t>(t) * p.part_ld;
    for (int c = lane; c * 4 < p.E; c += 64) {
      f32x4 acc = *reinterpret_cast<const f32x4*>(prow + 4 * c);
      for (int q0 = 1; q0 < p.nparts; q0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (q0 + j < p.nparts)
            v[j] = *reinterpret_cast<const f32x4*>(prow + (q0 + j) * pstride + 4 * c);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (q0 + j < p.nparts) acc += v[j];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 4 * c + u;
        if (e < p.E) {
          const float x = p.offset ? acc[u] + p.offset[e] : acc[u];
          l[e] = x;
          if (p.logits_out) p.logits_out[static_cast<int64_t>(t) * p.E + e] = x;
        }
      }
    }
  } else {
    const float* lrow = p.logits + static_cast<int64_t>(t) * p.E;
    for (int e = lane; e < p.E; e += 64) {
      l[e] = lrow[e];
      if (p.logits_out) p.logits_out[static_cast<int64_t>(t) * p.E + e] = lrow[e];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  if (p.mode == MOE_ROUTE_HASH) {
    int e = -1;
    if (lane < p.k) {
      const int tok = p.token_ids[t];
      if (tok >= 0 && tok < p.vocab) {
        const int v = p.tid2eid[static_cast<int64_t>(tok) * p.k + lane];
        if (v >= 0 && v < p.E) e = v;
      }
    }
    write_gates(p, l, t, lane, e);
    return;
  }

  float key[NS];
  bool ok[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + 64 * i;
    ok[i] = e < p.E;
    key[i] = 0.0f;
    if (ok[i]) {
      const float s = affinity(l[e], p.scoring);
      key[i] = p.bias ? s + p.bias[e] : s;
    }
  }

  if (p.n_group > 1) {
    const int G = p.E / p.n_group;
    float* kw = skey[wave];
    uint64_t gk = 0;
    if ((G & (G - 1)) == 0 && G <= 64) {
      // a group is G consecutive lanes of one slot: its score is the sum of the
      // group_topk largest keys, largest first, taken by segment maxima over
      // the packed (key, index) words; ties go to the lower index, as below
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (64 * i >= p.E) continue;  // uniform
        uint64_t cur = ok[i] ? pack_key(key[i], lane + 64 * i) : 0;
        float acc = 0.0f;
        for (int r = 0; r < p.group_topk; ++r) {
          const uint64_t m = segment_max_u64(cur, G);
          const float v = from_order_bits(static_cast<uint32_t>(m >> 32));
          acc = (r == 0) ? v : acc + v;
          if (cur == m) cur = 0;
        }
        if ((lane & (G - 1)) == 0) kw[(64 * i + lane) / G] = acc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < p.n_group) gk = pack_key(kw[lane], lane);
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (ok[i]) kw[lane + 64 * i] = key[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // lane g scores group g: sum of its group_topk largest keys, largest first
      if (lane < p.n_group) {
        const float* gkey = kw + lane * G;
        // round r takes the best member that comes after round r-1's pick in the
        // (key descending, index ascending) order, i.e. selection without removal
        float acc = 0.0f, pv = 0.0f;
        int pi = -1;
        for (int r = 0; r < p.group_topk; ++r) {
          int b = -1;
          float bv = 0.0f;
          for (int i = 0; i < G; ++i) {
            const float v = gkey[i];
            const bool after = r == 0 || v < pv || (v == pv && i > pi);
            if (after && (b < 0 || v > bv)) { b = i; bv = v; }
          }
          pv = bv;
          pi = b;
          acc = (r == 0) ? bv : acc + bv;
        }
        gk = pack_key(acc, lane);
      }
    }
    uint64_t keep = 0;  // bit g set: group g stays eligible
    for (int r = 0; r < p.topk_group; ++r) {
      const uint64_t best = wave_max_u64(gk);
      const int g = static_cast<int>(~static_cast<uint32_t>(best));
      keep |= 1ull << g;
      if (lane == g) gk = 0;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (ok[i]) ok[i] = (keep >> ((lane + 64 * i) / G)) & 1ull;
  }

  int my_e = -1;  // lane j keeps the id of slot j
  for (int r = 0; r < p.k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (ok[i]) {
        const uint64_t pk = pack_key(key[i], lane + 64 * i);
        best = pk > best ? pk : best;
      }
    best = wave_max_u64(best);
    const int e = static_cast<int>(~static_cast<uint32_t>(best));
    if (lane == r) my_e = e;
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (i == (e >> 6)) ok[i] = false;
    }
  }
  write_gates(p, l, t, lane, my_e);
}

}  // namespace

hipError_t launch_topk(const moe_config& c, const float* logits, const float* parts, int nparts,
                       const float* logit_offset, const float* bias, const int32_t* token_ids,
                       const int32_t* tid2eid, int32_t* ids, float* weights, float* logits_out,
                       hipStream_t s) {
  TopkArgs p{logits, parts, nparts, router_part_ld(c), logit_offset, logits_out, bias, token_ids, tid2eid, ids,
             weights, c.T, c.E, c.k, c.scoring, c.route_mode, c.n_group, c.topk_group,
             c.group_topk, c.vocab};
  const dim3 grid(ceil_div(c.T, kWavesPerBlock)), block(64 * kWavesPerBlock);
  static_assert(kMaxPerLane == 16, "slot counts below");
  if (c.E <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, p);
  else if (c.E <= 128)
    hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, p);
  else if (c.E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, p);
  else if (c.E <= 512)
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
