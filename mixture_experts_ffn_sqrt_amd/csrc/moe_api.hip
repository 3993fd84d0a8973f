// C ABI entry points (include/moe.h): argument checks on the host, workspace
// carve-up, and the launch sequence on the caller's stream.  The library never
// allocates or synchronises; the only state it keeps is, per device, the
// address of moe_forward_noalloc's static scratch array.
#include <algorithm>
#include <mutex>

#include "moe_internal.h"

namespace moe {

Workspace workspace_layout(const moe_config& c) {
  const int64_t T = c.T, E = c.E, k = c.k, S = c.n_shared;
  const int64_t R = T * k, P = R + S * T, G = E + S;
  const int64_t es = c.dtype == MOE_F32 ? 4 : 2;
  const int64_t nblk = std::max<int64_t>(1, (R + kPermuteChunk - 1) / kPermuteChunk);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align_up(off + std::max<int64_t>(bytes, 1), 256);
    return o;
  };
  Workspace w;
  const int splits = router_splits(c);
  w.logits = take(splits > 1 ? (int64_t)splits * T * router_part_ld(c) * 4 : (int64_t)T * E * 4);
  w.ids = take(R * 4);
  w.weights = take(R * 4);
  w.blockcnt = take(nblk * E * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.groups = take(2 * G * 4);
  w.tile_prefix = take(kNumTileLists * (G + 1) * 4);
  w.sorted_tok = take(P * 4);
  w.sorted_w = take(R * 4);
  w.dispatch = take(R * 4);
  // H holds the bf16/f32 intermediate, or the FP8 codes followed by their scales
  const int64_t h_codes = align_up(P * c.d_ff, 256);
  w.H = take(std::max(P * c.d_ff * es, h_codes + P * (c.d_ff / 128) * 4));
  w.hs = w.H + h_codes;
  w.Y = take(P * c.d * es);
  w.xq = take(T * c.d);
  w.xs = take(T * (c.d / 128) * 4);
  w.total = off;
  return w;
}

namespace {

int check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->d < 1 || c->E < 1 || c->k < 1 || c->d_ff < 1) return MOE_ERR_INVALID_ARG;
  if (c->n_shared < 0 || c->n_shared > 1) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->scoring < MOE_SCORE_SOFTMAX || c->scoring > MOE_SCORE_SQRTSOFTPLUS)
    return MOE_ERR_INVALID_ARG;
  if (c->route_mode != MOE_ROUTE_LEARNED && c->route_mode != MOE_ROUTE_HASH)
    return MOE_ERR_INVALID_ARG;
  if (c->k > c->E) return MOE_ERR_INVALID_ARG;
  if (c->E > 1024 || c->k > 16) return MOE_ERR_UNSUPPORTED;
  if (c->d % 64 || c->d_ff % 64) return MOE_ERR_UNSUPPORTED;
  if (c->n_group < 1) return MOE_ERR_INVALID_ARG;
  if (c->n_group > 1) {
    if (c->n_group > 64) return MOE_ERR_UNSUPPORTED;
    if (c->E % c->n_group) return MOE_ERR_INVALID_ARG;
    const int G = c->E / c->n_group;
    if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_INVALID_ARG;
    if (c->group_topk < 1 || c->group_topk > G) return MOE_ERR_INVALID_ARG;
    if (c->k > c->topk_group * G) return MOE_ERR_INVALID_ARG;
  }
  if (c->route_mode == MOE_ROUTE_HASH && c->vocab < 1) return MOE_ERR_INVALID_ARG;
  const int64_t P = static_cast<int64_t>(c->T) * (c->k + c->n_shared);
  const int64_t width = std::max(c->d, c->d_ff);
  if (P * width >= (int64_t(1) << 31) * 64 || P >= (int64_t(1) << 30) ||
      static_cast<int64_t>(c->T) * c->E >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The FP8 entry points: bf16 activations, 128-multiples, and operands the
// buffer-load kernels address with 31-bit offsets.
int check_fp8(const moe_config* c) {
  const int st = check_cfg(c);
  if (st) return st;
  if (c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->d % 128 || c->d_ff % 128) return MOE_ERR_UNSUPPORTED;
  const int64_t lim = int64_t(1) << 31;
  const int64_t T = c->T, d = c->d, F = c->d_ff;
  const int64_t P = T * (c->k + c->n_shared);
  if (T * d >= lim || P * F >= lim || 2 * F * d >= lim || P * (F / 128) * 4 >= lim ||
      288 * d * 2 >= lim)  // a tile's rows of Y (bf16) through one buffer range
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The workspace of moe_forward_noalloc: a static device array (one copy on
// every GPU the library runs on, held until the process ends).  Host code
// never passes the array's name to a kernel: its address on a device comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

template <typename T>
T* at(void* ws, int64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Tile lists for the routed experts of the staged API (E groups, rows from the
// caller's offsets) and the matching launch arguments.
int staged_groups(const moe_config& c, const int32_t* expert_offsets, void* workspace,
                  const Workspace& w, hipStream_t s, ExpertFfnArgs* a) {
  int32_t* groups = at<int32_t>(workspace, w.groups);
  int32_t* tiles = at<int32_t>(workspace, w.tile_prefix);
  const int st = hip_status(
      launch_build_tiles(expert_offsets, c.E, c.T * c.k, 0, 0, groups, tiles, nullptr, s));
  *a = ExpertFfnArgs{};
  a->g_begin = groups;
  a->g_end = groups + c.E;
  a->tile_prefix = tiles;
  a->n_groups = c.E;
  a->rows_bound = c.T * c.k;
  a->routed_groups = c.E;
  return st;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  const int st = check_cfg(cfg);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = static_cast<size_t>(workspace_layout(*cfg).total);
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const void* hidden, const void* w_router,
              const float* logit_offset, const float* bias, const int32_t* token_ids,
              const int32_t* tid2eid, float* logits, int32_t* topk_ids, float* topk_weights,
              void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARG;
  if (!c.logits_given && (!hidden || !w_router)) return MOE_ERR_INVALID_ARG;
  if (c.route_mode == MOE_ROUTE_HASH && (!token_ids || !tid2eid)) return MOE_ERR_INVALID_ARG;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!c.logits_given) {
    st = hip_status(launch_router_gemm(c, hidden, w_router, logit_offset, logits, 1, s));
    if (st) return st;
  }
  return hip_status(launch_topk(c, logits, nullptr, 0, nullptr, bias, token_ids, tid2eid,
                                topk_ids, topk_weights, nullptr, s));
}

int moe_permute(const moe_config* cfg, const int32_t* topk_ids, const float* topk_weights,
                int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token_ids,
                float* sorted_weights, int32_t* dispatch_index, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int st = check_cfg(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!topk_ids || !topk_weights || !expert_counts || !expert_offsets || !sorted_token_ids ||
      !sorted_weights || !dispatch_index || !workspace)
    return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  return hip_status(launch_permute(c, topk_ids, topk_weights, at<int32_t>(workspace, w.blockcnt),
                                   expert_counts, expert_offsets, sorted_token_ids,
                                   sorted_weights, dispatch_index,
                                   static_cast<hipStream_t>(stream)));
}

int moe_expert_up(const moe_config* cfg, const void* hidden, const int32_t* sorted_token_ids,
                  const int32_t* expert_offsets, const void* w13, void* h_out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!hidden || !sorted_token_ids || !expert_offsets || !w13 || !h_out || !workspace)
    return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertFfnArgs a;
  if ((st = staged_groups(c, expert_offsets, workspace, w, s, &a))) return st;
  a.hidden = hidden;
  a.sorted_tok = sorted_token_ids;
  a.w13 = w13;
  a.H = h_out;
  return hip_status(launch_expert_up(c, a, s));
}

int moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                    const void* w2, void* expert_out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!h || !expert_offsets || !w2 || !expert_out || !workspace) return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertFfnArgs a;
  if ((st = staged_groups(c, expert_offsets, workspace, w, s, &a))) return st;
  a.H = const_cast<void*>(h);
  a.w2 = w2;
  a.Y = expert_out;
  return hip_status(launch_expert_down(c, a, s));
}

int moe_expert_ffn(const moe_config* cfg, const void* hidden, const int32_t* sorted_token_ids,
                   const int32_t* expert_offsets, const void* w13, const void* w2,
                   void* expert_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!hidden || !sorted_token_ids || !expert_offsets || !w13 || !w2 || !expert_out ||
      !workspace)
    return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertFfnArgs a;
  if ((st = staged_groups(c, expert_offsets, workspace, w, s, &a))) return st;
  a.hidden = hidden;
  a.sorted_tok = sorted_token_ids;
  a.w13 = w13;
  a.w2 = w2;
  a.H = at<char>(workspace, w.H);
  a.Y = expert_out;
  if ((st = hip_status(launch_expert_up(c, a, s)))) return st;
  return hip_status(launch_expert_down(c, a, s));
}

int moe_combine(const moe_config* cfg, const void* expert_out, const int32_t* dispatch_index,
                const float* topk_weights, const void* shared_out, void* out, void* stream) {
  const int st = check_cfg(cfg);
  if (st) return st;
  if (!expert_out || !dispatch_index || !topk_weights || !out) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(launch_combine(*cfg, expert_out, dispatch_index, topk_weights, shared_out,
                                   out, static_cast<hipStream_t>(stream)));
}

int moe_forward(const moe_config* cfg, const void* hidden, const void* w_router,
                const float* logit_offset, const float* bias, const int32_t* token_ids,
                const int32_t* tid2eid, const void* w13, const void* w2, const void* w13_shared,
                const void* w2_shared, void* out, int32_t* topk_ids_out,
                float* topk_weights_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!hidden || !w_router || !w13 || !w2 || !out || !workspace) return MOE_ERR_INVALID_ARG;
  if (c.n_shared && (!w13_shared || !w2_shared)) return MOE_ERR_INVALID_ARG;
  if (c.route_mode == MOE_ROUTE_HASH && (!token_ids || !tid2eid)) return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe_config rc = c;
  rc.logits_given = 0;
  const int R = c.T * c.k;
  float* logits = at<float>(workspace, w.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, w.ids);
  float* gates = topk_weights_out ? topk_weights_out : at<float>(workspace, w.weights);
  int32_t* sorted_tok = at<int32_t>(workspace, w.sorted_tok);
  int32_t* dispatch = at<int32_t>(workspace, w.dispatch);
  int32_t* offsets = at<int32_t>(workspace, w.offsets);
  int32_t* groups = at<int32_t>(workspace, w.groups);
  int32_t* tiles = at<int32_t>(workspace, w.tile_prefix);
  const int G = c.E + c.n_shared;
  const int splits = router_splits(rc);
  if ((st = hip_status(launch_router_gemm(rc, hidden, w_router, logit_offset, logits, splits, s))))
    return st;
  if ((st = hip_status(launch_topk(rc, splits > 1 ? nullptr : logits, splits > 1 ? logits : nullptr,
                                   splits > 1 ? splits : 0, logit_offset, bias, token_ids, tid2eid,
                                   ids, gates, nullptr, s))))
    return st;
  if ((st = hip_status(launch_permute(rc, ids, gates, at<int32_t>(workspace, w.blockcnt),
                                      at<int32_t>(workspace, w.counts), offsets, sorted_tok,
                                      at<float>(workspace, w.sorted_w), dispatch, s))))
    return st;
  if ((st = hip_status(launch_build_tiles(offsets, c.E, R, R, c.n_shared ? c.T : 0, groups,
                                          tiles, sorted_tok, s))))
    return st;
  ExpertFfnArgs a{};
  a.hidden = hidden;
  a.sorted_tok = sorted_tok;
  a.g_begin = groups;
  a.g_end = groups + G;
  a.tile_prefix = tiles;
  a.n_groups = G;
  a.rows_bound = R + c.n_shared * c.T;
  a.routed_groups = c.E;
  a.w13 = w13;
  a.w2 = w2;
  a.w13_last = c.n_shared ? w13_shared : nullptr;
  a.w2_last = c.n_shared ? w2_shared : nullptr;
  a.H = at<char>(workspace, w.H);
  a.Y = at<char>(workspace, w.Y);
  if ((st = hip_status(launch_expert_up(c, a, s)))) return st;
  if ((st = hip_status(launch_expert_down(c, a, s)))) return st;
  const int64_t es = c.dtype == MOE_F32 ? 4 : 2;
  const char* shared_rows = c.n_shared ? at<char>(workspace, w.Y) + (int64_t)R * c.d * es : nullptr;
  return hip_status(launch_combine(c, a.Y, dispatch, gates, shared_rows, out, s));
}

int moe_forward_noalloc(const moe_config* cfg, const void* hidden, const void* w_router,
                        const float* logit_offset, const float* bias, const int32_t* token_ids,
                        const int32_t* tid2eid, const void* w13, const void* w2,
                        const void* w13_shared, const void* w2_shared, void* out,
                        int32_t* topk_ids_out, float* topk_weights_out, void* stream) {
  const int st = check_cfg(cfg);
  if (st) return st;
  if (workspace_layout(*cfg).total > (int64_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  if (cfg->T == 0) return MOE_OK;
  void* ws = nullptr;
  const int sst = noalloc_scratch(&ws);
  if (sst) return sst;
  return moe_forward(cfg, hidden, w_router, logit_offset, bias, token_ids, tid2eid, w13, w2,
                     w13_shared, w2_shared, out, topk_ids_out, topk_weights_out, ws,
                     MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_quantize_fp8_rows(int n, int K, int in_dtype, const void* x, uint8_t* q, float* scales,
                          void* stream) {
  if (n < 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (K % 128) return MOE_ERR_UNSUPPORTED;
  if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_rows(n, K, in_dtype, x, q, scales,
                                         static_cast<hipStream_t>(stream)));
}

int moe_quantize_fp8_blocks(int R, int C, int in_dtype, const void* w, uint8_t* q, float* scales,
                            void* stream) {
  if (R < 0 || C < 0) return MOE_ERR_INVALID_ARG;
  if (R % 128 || C % 128) return MOE_ERR_UNSUPPORTED;
  if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (R == 0 || C == 0) return MOE_OK;
  if (!w || !q || !scales) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_blocks(R, C, in_dtype, w, q, scales,
                                           static_cast<hipStream_t>(stream)));
}

namespace {
Fp8FfnArgs fp8_args_of(const ExpertFfnArgs& a) {
  Fp8FfnArgs f{};
  f.sorted_tok = a.sorted_tok;
  f.g_begin = a.g_begin;
  f.g_end = a.g_end;
  f.tile_prefix = a.tile_prefix;
  f.n_groups = a.n_groups;
  f.rows_bound = a.rows_bound;
  f.routed_groups = a.routed_groups;
  return f;
}
}  // namespace

namespace {
int expert_up_lowp(const moe_config* cfg, int wfmt, const uint8_t* xq, const float* xs,
                   const int32_t* sorted_token_ids, const int32_t* expert_offsets,
                   const uint8_t* w13q, const void* w13s, uint8_t* hq, float* hs,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_fp8(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!xq || !xs || !sorted_token_ids || !expert_offsets || !w13q || !w13s || !hq || !hs ||
      !workspace)
    return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertFfnArgs a;
  if ((st = staged_groups(c, expert_offsets, workspace, w, s, &a))) return st;
  a.sorted_tok = sorted_token_ids;
  Fp8FfnArgs f = fp8_args_of(a);
  f.wfmt = wfmt;
  f.xq = xq;
  f.xs = xs;
  f.w13q = w13q;
  f.w13s = w13s;
  f.hq = hq;
  f.hs = hs;
  return hip_status(launch_expert_up_fp8(c, f, s));
}

int expert_down_lowp(const moe_config* cfg, int wfmt, const uint8_t* hq, const float* hs,
                     const int32_t* expert_offsets, const uint8_t* w2q, const void* w2s,
                     void* expert_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_fp8(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!hq || !hs || !expert_offsets || !w2q || !w2s || !expert_out || !workspace)
    return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertFfnArgs a;
  if ((st = staged_groups(c, expert_offsets, workspace, w, s, &a))) return st;
  Fp8FfnArgs f = fp8_args_of(a);
  f.wfmt = wfmt;
  f.hq = const_cast<uint8_t*>(hq);
  f.hs = const_cast<float*>(hs);
  f.w2q = w2q;
  f.w2s = w2s;
  f.Y = expert_out;
  return hip_status(launch_expert_down_fp8(c, f, s));
}

// router -> top-k -> FP8 cast of the hidden rows -> permute -> tiles -> GEMM 1
// (+ SwiGLU + FP8 cast of H) -> GEMM 2 -> combine, for either weight format
int forward_lowp(const moe_config* cfg, int wfmt, const void* hidden, const void* w_router,
                 const float* logit_offset, const float* bias, const int32_t* token_ids,
                 const int32_t* tid2eid, const uint8_t* w13q, const void* w13s,
                 const uint8_t* w2q, const void* w2s, const uint8_t* w13q_shared,
                 const void* w13s_shared, const uint8_t* w2q_shared, const void* w2s_shared,
                 void* out, int32_t* topk_ids_out, float* topk_weights_out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int st = check_fp8(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (!hidden || !w_router || !w13q || !w13s || !w2q || !w2s || !out || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (c.n_shared && (!w13q_shared || !w13s_shared || !w2q_shared || !w2s_shared))
    return MOE_ERR_INVALID_ARG;
  if (c.route_mode == MOE_ROUTE_HASH && (!token_ids || !tid2eid)) return MOE_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(c);
  if (workspace_bytes < static_cast<size_t>(w.total)) return MOE_ERR_WORKSPACE;
  if (c.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe_config rc = c;
  rc.logits_given = 0;
  const int R = c.T * c.k;
  float* logits = at<float>(workspace, w.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, w.ids);
  float* gates = topk_weights_out ? topk_weights_out : at<float>(workspace, w.weights);
  int32_t* sorted_tok = at<int32_t>(workspace, w.sorted_tok);
  int32_t* dispatch = at<int32_t>(workspace, w.dispatch);
  int32_t* offsets = at<int32_t>(workspace, w.offsets);
  int32_t* groups = at<int32_t>(workspace, w.groups);
  int32_t* tiles = at<int32_t>(workspace, w.tile_prefix);
  uint8_t* xq = at<uint8_t>(workspace, w.xq);
  float* xs = at<float>(workspace, w.xs);
  const int G = c.E + c.n_shared;
  const int splits = router_splits(rc);
  if ((st = hip_status(launch_router_gemm(rc, hidden, w_router, logit_offset, logits, splits, s))))
    return st;
  if ((st = hip_status(launch_topk(rc, splits > 1 ? nullptr : logits, splits > 1 ? logits : nullptr,
                                   splits > 1 ? splits : 0, logit_offset, bias, token_ids, tid2eid,
                                   ids, gates, nullptr, s))))
    return st;
  if ((st = hip_status(launch_quantize_rows(c.T, c.d, MOE_BF16, hidden, xq, xs, s)))) return st;
  if ((st = hip_status(launch_permute(rc, ids, gates, at<int32_t>(workspace, w.blockcnt),
                                      at<int32_t>(workspace, w.counts), offsets, sorted_tok,
                                      at<float>(workspace, w.sorted_w), dispatch, s))))
    return st;
  if ((st = hip_status(launch_build_tiles(offsets, c.E, R, R, c.n_shared ? c.T : 0, groups,
                                          tiles, sorted_tok, s))))
    return st;
  Fp8FfnArgs f{};
  f.wfmt = wfmt;
  f.xq = xq;
  f.xs = xs;
  f.sorted_tok = sorted_tok;
  f.g_begin = groups;
  f.g_end = groups + G;
  f.tile_prefix = tiles;
  f.n_groups = G;
  f.rows_bound = R + c.n_shared * c.T;
  f.routed_groups = c.E;
  f.w13q = w13q;
  f.w13s = w13s;
  f.w2q = w2q;
  f.w2s = w2s;
  f.w13q_last = c.n_shared ? w13q_shared : nullptr;
  f.w13s_last = c.n_shared ? w13s_shared : nullptr;
  f.w2q_last = c.n_shared ? w2q_shared : nullptr;
  f.w2s_last = c.n_shared ? w2s_shared : nullptr;
  f.hq = at<uint8_t>(workspace, w.H);
  f.hs = at<float>(workspace, w.hs);
  f.Y = at<char>(workspace, w.Y);
  if ((st = hip_status(launch_expert_up_fp8(c, f, s)))) return st;
  if ((st = hip_status(launch_expert_down_fp8(c, f, s)))) return st;
  const char* shared_rows = c.n_shared ? at<char>(workspace, w.Y) + (int64_t)R * c.d * 2 : nullptr;
  return hip_status(launch_combine(c, f.Y, dispatch, gates, shared_rows, out, s));
}
}  // namespace

int moe_expert_up_fp8(const moe_config* cfg, const uint8_t* xq, const float* xs,
                      const int32_t* sorted_token_ids, const int32_t* expert_offsets,
                      const uint8_t* w13q, const float* w13s, uint8_t* hq, float* hs,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return expert_up_lowp(cfg, kWeightE4M3, xq, xs, sorted_token_ids, expert_offsets, w13q, w13s,
                        hq, hs, workspace, workspace_bytes, stream);
}

int moe_expert_down_fp8(const moe_config* cfg, const uint8_t* hq, const float* hs,
                        const int32_t* expert_offsets, const uint8_t* w2q, const float* w2s,
                        void* expert_out, void* workspace, size_t workspace_bytes, void* stream) {
  return expert_down_lowp(cfg, kWeightE4M3, hq, hs, expert_offsets, w2q, w2s, expert_out,
                          workspace, workspace_bytes, stream);
}

int moe_forward_fp8(const moe_config* cfg, const void* hidden, const void* w_router,
                    const float* logit_offset, const float* bias, const int32_t* token_ids,
                    const int32_t* tid2eid, const uint8_t* w13q, const float* w13s,
                    const uint8_t* w2q, const float* w2s, const uint8_t* w13q_shared,
                    const float* w13s_shared, const uint8_t* w2q_shared, const float* w2s_shared,
                    void* out, int32_t* topk_ids_out, float* topk_weights_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return forward_lowp(cfg, kWeightE4M3, hidden, w_router, logit_offset, bias, token_ids, tid2eid,
                      w13q, w13s, w2q, w2s, w13q_shared, w13s_shared, w2q_shared, w2s_shared, out,
                      topk_ids_out, topk_weights_out, workspace, workspace_bytes, stream);
}

int moe_quantize_mxfp4(int n_mat, int R, int C, int in_dtype, const void* w, uint8_t* q,
                       uint8_t* scales, void* stream) {
  if (n_mat < 0 || R < 0 || C < 0) return MOE_ERR_INVALID_ARG;
  if (C % 128 || R % 2) return MOE_ERR_UNSUPPORTED;
  if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (n_mat == 0 || R == 0 || C == 0) return MOE_OK;
  if (!w || !q || !scales) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_mxfp4(n_mat, R, C, in_dtype, w, q, scales,
                                          static_cast<hipStream_t>(stream)));
}

int moe_expert_up_mxfp4(const moe_config* cfg, const uint8_t* xq, const float* xs,
                        const int32_t* sorted_token_ids, const int32_t* expert_offsets,
                        const uint8_t* w13q, const uint8_t* w13s, uint8_t* hq, float* hs,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return expert_up_lowp(cfg, kWeightMxfp4, xq, xs, sorted_token_ids, expert_offsets, w13q, w13s,
                        hq, hs, workspace, workspace_bytes, stream);
}

int moe_expert_down_mxfp4(const moe_config* cfg, const uint8_t* hq, const float* hs,
                          const int32_t* expert_offsets, const uint8_t* w2q, const uint8_t* w2s,
                          void* expert_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return expert_down_lowp(cfg, kWeightMxfp4, hq, hs, expert_offsets, w2q, w2s, expert_out,
                          workspace, workspace_bytes, stream);
}

int moe_forward_mxfp4(const moe_config* cfg, const void* hidden, const void* w_router,
                      const float* logit_offset, const float* bias, const int32_t* token_ids,
                      const int32_t* tid2eid, const uint8_t* w13q, const uint8_t* w13s,
                      const uint8_t* w2q, const uint8_t* w2s, const uint8_t* w13q_shared,
                      const uint8_t* w13s_shared, const uint8_t* w2q_shared,
                      const uint8_t* w2s_shared, void* out, int32_t* topk_ids_out,
                      float* topk_weights_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return forward_lowp(cfg, kWeightMxfp4, hidden, w_router, logit_offset, bias, token_ids, tid2eid,
                      w13q, w13s, w2q, w2s, w13q_shared, w13s_shared, w2q_shared, w2s_shared, out,
                      topk_ids_out, topk_weights_out, workspace, workspace_bytes, stream);
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_TOO_LARGE: return "workspace larger than the no-alloc entry point's scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
