"""Thin Python binding of libmoe.so (include/moe.h), same names as the C ABI.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  Each wrapper
checks on the host that every tensor has the shape, dtype, device and layout the
kernels assume before the call is made; the library itself sees only pointers.
If libmoe.so is missing the wrappers raise: there is no fallback path.
"""
import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_TOO_LARGE = -5
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SQRTSOFTPLUS = 0, 1, 2
MOE_ROUTE_LEARNED, MOE_ROUTE_HASH = 0, 1

EXPORTS = ("moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_up",
           "moe_expert_down", "moe_combine", "moe_forward", "moe_forward_noalloc",
           "moe_quantize_fp8_rows",
           "moe_quantize_fp8_blocks", "moe_expert_up_fp8", "moe_expert_down_fp8",
           "moe_forward_fp8", "moe_quantize_mxfp4", "moe_expert_up_mxfp4",
           "moe_expert_down_mxfp4", "moe_forward_mxfp4", "moe_strerror")


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, _strerror(status), status))
        self.status = status


class MoeConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "T", "d", "E", "k", "d_ff", "n_shared", "dtype", "scoring", "route_mode",
        "n_group", "topk_group", "group_topk", "vocab", "logits_given")]

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == MOE_F32 else torch.bfloat16


def make_config(T, d, E, k, d_ff, n_shared=0, dtype="bf16", scoring=MOE_SCORE_SOFTMAX,
                route_mode=MOE_ROUTE_LEARNED, n_group=1, topk_group=1, group_topk=0, vocab=0,
                logits_given=0) -> MoeConfig:
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, MOE_F32: MOE_F32, MOE_BF16: MOE_BF16}[dtype]
    return MoeConfig(T, d, E, k, d_ff, n_shared, dt, scoring, route_mode, n_group, topk_group,
                     group_topk, vocab, logits_given)


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmoe.so (built in-tree by mixture_experts_ffn_sqrt_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe.so is not built (%s); run `python -m "
                           "mixture_experts_ffn_sqrt_amd.build`" % path)
    L = C.CDLL(path)
    P, S, I = C.c_void_p, C.c_size_t, C.c_int
    cfg = C.POINTER(MoeConfig)
    L.moe_workspace_size.argtypes = [cfg, C.POINTER(C.c_size_t)]
    L.moe_route.argtypes = [cfg, P, P, P, P, P, P, P, P, P, P]
    L.moe_permute.argtypes = [cfg, P, P, P, P, P, P, P, P, S, P]
    L.moe_expert_ffn.argtypes = [cfg, P, P, P, P, P, P, P, S, P]
    L.moe_expert_up.argtypes = [cfg, P, P, P, P, P, P, S, P]
    L.moe_expert_down.argtypes = [cfg, P, P, P, P, P, S, P]
    L.moe_combine.argtypes = [cfg, P, P, P, P, P, P]
    L.moe_forward.argtypes = [cfg, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    L.moe_forward_noalloc.argtypes = [cfg, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    L.moe_quantize_fp8_rows.argtypes = [I, I, I, P, P, P, P]
    L.moe_quantize_fp8_blocks.argtypes = [I, I, I, P, P, P, P]
    L.moe_expert_up_fp8.argtypes = [cfg, P, P, P, P, P, P, P, P, P, S, P]
    L.moe_expert_down_fp8.argtypes = [cfg, P, P, P, P, P, P, P, S, P]
    L.moe_forward_fp8.argtypes = [cfg] + [P] * 18 + [S, P]
    L.moe_quantize_mxfp4.argtypes = [I, I, I, I, P, P, P, P]
    L.moe_expert_up_mxfp4.argtypes = [cfg, P, P, P, P, P, P, P, P, P, S, P]
    L.moe_expert_down_mxfp4.argtypes = [cfg, P, P, P, P, P, P, P, S, P]
    L.moe_forward_mxfp4.argtypes = [cfg] + [P] * 18 + [S, P]
    L.moe_strerror.argtypes = [I]
    L.moe_strerror.restype = C.c_char_p
    for n in EXPORTS[:-1]:
        getattr(L, n).restype = I
    _lib = L
    return L


def _strerror(status):
    try:
        return load_library().moe_strerror(int(status)).decode()
    except Exception:
        return "status %d" % status


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _t(name, t, shape, dtype, required=True):
    """Pointer of a device tensor after checking shape, dtype, device, layout."""
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() and t.data_ptr() % 16:
        raise ValueError("%s must be 16-byte aligned" % name)
    return C.c_void_p(t.data_ptr()) if t.numel() else C.c_void_p(0)


def moe_workspace_size(cfg: MoeConfig) -> int:
    n = C.c_size_t(0)
    _check("moe_workspace_size", load_library().moe_workspace_size(C.byref(cfg), C.byref(n)))
    return n.value


def _ws(cfg, workspace):
    need = moe_workspace_size(cfg)
    if workspace is None:
        raise ValueError("workspace is required (moe_workspace_size = %d bytes)" % need)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError("workspace has %d bytes, needs %d" % (have, need))
    return C.c_void_p(workspace.data_ptr()), C.c_size_t(have)


def moe_route(cfg, hidden, w_router, logit_offset, bias, token_ids, tid2eid, logits, topk_ids,
              topk_weights, stream=None):
    dt, T, d, E, k = cfg.torch_dtype, cfg.T, cfg.d, cfg.E, cfg.k
    given = bool(cfg.logits_given)
    hsh = cfg.route_mode == MOE_ROUTE_HASH
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), dt, not given),
            _t("w_router", w_router, (E, d), dt, not given),
            _t("logit_offset", logit_offset, (E,), torch.float32, False),
            _t("bias", bias, (E,), torch.float32, False),
            _t("token_ids", token_ids, (T,), torch.int32, hsh),
            _t("tid2eid", tid2eid, (cfg.vocab, k), torch.int32, hsh),
            _t("logits", logits, (T, E), torch.float32),
            _t("topk_ids", topk_ids, (T, k), torch.int32),
            _t("topk_weights", topk_weights, (T, k), torch.float32),
            _stream(stream)]
    _check("moe_route", load_library().moe_route(*args))


def moe_permute(cfg, topk_ids, topk_weights, expert_counts, expert_offsets, sorted_token_ids,
                sorted_weights, dispatch_index, workspace, stream=None):
    T, E, k = cfg.T, cfg.E, cfg.k
    i32, f32 = torch.int32, torch.float32
    args = [C.byref(cfg),
            _t("topk_ids", topk_ids, (T, k), i32), _t("topk_weights", topk_weights, (T, k), f32),
            _t("expert_counts", expert_counts, (E,), i32),
            _t("expert_offsets", expert_offsets, (E + 1,), i32),
            _t("sorted_token_ids", sorted_token_ids, (T * k,), i32),
            _t("sorted_weights", sorted_weights, (T * k,), f32),
            _t("dispatch_index", dispatch_index, (T, k), i32),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_permute", load_library().moe_permute(*args))


def moe_expert_ffn(cfg, hidden, sorted_token_ids, expert_offsets, w13, w2, expert_out, workspace,
                   stream=None):
    dt, T, d, E, k, F = cfg.torch_dtype, cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), dt),
            _t("sorted_token_ids", sorted_token_ids, (T * k,), torch.int32),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w13", w13, (E, 2 * F, d), dt), _t("w2", w2, (E, d, F), dt),
            _t("expert_out", expert_out, (T * k, d), dt),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_ffn", load_library().moe_expert_ffn(*args))


def moe_expert_up(cfg, hidden, sorted_token_ids, expert_offsets, w13, h_out, workspace,
                  stream=None):
    dt, T, d, E, k, F = cfg.torch_dtype, cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), dt),
            _t("sorted_token_ids", sorted_token_ids, (T * k,), torch.int32),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w13", w13, (E, 2 * F, d), dt),
            _t("h_out", h_out, (T * k, F), dt),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_up", load_library().moe_expert_up(*args))


def moe_expert_down(cfg, h, expert_offsets, w2, expert_out, workspace, stream=None):
    dt, T, d, E, k, F = cfg.torch_dtype, cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    args = [C.byref(cfg),
            _t("h", h, (T * k, F), dt),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w2", w2, (E, d, F), dt),
            _t("expert_out", expert_out, (T * k, d), dt),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_down", load_library().moe_expert_down(*args))


def moe_combine(cfg, expert_out, dispatch_index, topk_weights, shared_out, out, stream=None):
    dt, T, d, k = cfg.torch_dtype, cfg.T, cfg.d, cfg.k
    args = [C.byref(cfg),
            _t("expert_out", expert_out, (T * k, d), dt),
            _t("dispatch_index", dispatch_index, (T, k), torch.int32),
            _t("topk_weights", topk_weights, (T, k), torch.float32),
            _t("shared_out", shared_out, (T, d), dt, False),
            _t("out", out, (T, d), dt), _stream(stream)]
    _check("moe_combine", load_library().moe_combine(*args))


def moe_forward(cfg, hidden, w_router, logit_offset, bias, token_ids, tid2eid, w13, w2,
                w13_shared, w2_shared, out, topk_ids_out, topk_weights_out, workspace,
                stream=None):
    dt, T, d, E, k, F = cfg.torch_dtype, cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    hsh = cfg.route_mode == MOE_ROUTE_HASH
    sh = bool(cfg.n_shared)
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), dt), _t("w_router", w_router, (E, d), dt),
            _t("logit_offset", logit_offset, (E,), torch.float32, False),
            _t("bias", bias, (E,), torch.float32, False),
            _t("token_ids", token_ids, (T,), torch.int32, hsh),
            _t("tid2eid", tid2eid, (cfg.vocab, k), torch.int32, hsh),
            _t("w13", w13, (E, 2 * F, d), dt), _t("w2", w2, (E, d, F), dt),
            _t("w13_shared", w13_shared, (2 * F, d), dt, sh),
            _t("w2_shared", w2_shared, (d, F), dt, sh),
            _t("out", out, (T, d), dt),
            _t("topk_ids_out", topk_ids_out, (T, k), torch.int32, False),
            _t("topk_weights_out", topk_weights_out, (T, k), torch.float32, False),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_forward", load_library().moe_forward(*args))


def moe_forward_noalloc(cfg, hidden, w_router, logit_offset, bias, token_ids, tid2eid, w13, w2,
                        w13_shared, w2_shared, out, topk_ids_out, topk_weights_out,
                        stream=None):
    """moe_forward with the library's static scratch as its workspace (no
    allocation); configurations needing more than MOE_NOALLOC_SCRATCH_BYTES of
    workspace raise with MOE_ERR_TOO_LARGE."""
    dt, T, d, E, k, F = cfg.torch_dtype, cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    hsh = cfg.route_mode == MOE_ROUTE_HASH
    sh = bool(cfg.n_shared)
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), dt), _t("w_router", w_router, (E, d), dt),
            _t("logit_offset", logit_offset, (E,), torch.float32, False),
            _t("bias", bias, (E,), torch.float32, False),
            _t("token_ids", token_ids, (T,), torch.int32, hsh),
            _t("tid2eid", tid2eid, (cfg.vocab, k), torch.int32, hsh),
            _t("w13", w13, (E, 2 * F, d), dt), _t("w2", w2, (E, d, F), dt),
            _t("w13_shared", w13_shared, (2 * F, d), dt, sh),
            _t("w2_shared", w2_shared, (d, F), dt, sh),
            _t("out", out, (T, d), dt),
            _t("topk_ids_out", topk_ids_out, (T, k), torch.int32, False),
            _t("topk_weights_out", topk_weights_out, (T, k), torch.float32, False),
            _stream(stream)]
    _check("moe_forward_noalloc", load_library().moe_forward_noalloc(*args))


_IN_DTYPES = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


def moe_quantize_fp8_rows(x, q, scales, stream=None):
    """x [n, K] float32/bfloat16 -> q [n, K] uint8 E4M3 codes, scales [K/128, n]
    (K-block-major)."""
    if x.dtype not in _IN_DTYPES:
        raise ValueError("x must be float32 or bfloat16, got %s" % x.dtype)
    n, K = x.shape
    args = [n, K, _IN_DTYPES[x.dtype], _t("x", x, (n, K), x.dtype),
            _t("q", q, (n, K), torch.uint8), _t("scales", scales, (K // 128, n), torch.float32),
            _stream(stream)]
    _check("moe_quantize_fp8_rows", load_library().moe_quantize_fp8_rows(*args))


def moe_quantize_fp8_blocks(w, q, scales, stream=None):
    """w [R, C] (or [E, R, C], quantized as E*R rows) -> codes of the same shape,
    scales [R/128, C/128] (or [E, R/128, C/128])."""
    if w.dtype not in _IN_DTYPES:
        raise ValueError("w must be float32 or bfloat16, got %s" % w.dtype)
    C_ = w.shape[-1]
    R = w.numel() // C_ if C_ else 0
    sshape = tuple(w.shape[:-2]) + (w.shape[-2] // 128, C_ // 128)
    args = [R, C_, _IN_DTYPES[w.dtype], _t("w", w, tuple(w.shape), w.dtype),
            _t("q", q, tuple(w.shape), torch.uint8), _t("scales", scales, sshape, torch.float32),
            _stream(stream)]
    _check("moe_quantize_fp8_blocks", load_library().moe_quantize_fp8_blocks(*args))


def moe_expert_up_fp8(cfg, xq, xs, sorted_token_ids, expert_offsets, w13q, w13s, hq, hs,
                      workspace, stream=None):
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    u8, f32 = torch.uint8, torch.float32
    args = [C.byref(cfg),
            _t("xq", xq, (T, d), u8), _t("xs", xs, (d // 128, T), f32),
            _t("sorted_token_ids", sorted_token_ids, (T * k,), torch.int32),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w13q", w13q, (E, 2 * F, d), u8), _t("w13s", w13s, (E, 2 * F // 128, d // 128), f32),
            _t("hq", hq, (T * k, F), u8), _t("hs", hs, (F // 128, T * k), f32),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_up_fp8", load_library().moe_expert_up_fp8(*args))


def moe_expert_down_fp8(cfg, hq, hs, expert_offsets, w2q, w2s, expert_out, workspace,
                        stream=None):
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    u8, f32 = torch.uint8, torch.float32
    args = [C.byref(cfg),
            _t("hq", hq, (T * k, F), u8), _t("hs", hs, (F // 128, T * k), f32),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w2q", w2q, (E, d, F), u8), _t("w2s", w2s, (E, d // 128, F // 128), f32),
            _t("expert_out", expert_out, (T * k, d), torch.bfloat16),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_down_fp8", load_library().moe_expert_down_fp8(*args))


def moe_forward_fp8(cfg, hidden, w_router, logit_offset, bias, token_ids, tid2eid, w13q, w13s,
                    w2q, w2s, w13q_shared, w13s_shared, w2q_shared, w2s_shared, out,
                    topk_ids_out, topk_weights_out, workspace, stream=None):
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    hsh = cfg.route_mode == MOE_ROUTE_HASH
    sh = bool(cfg.n_shared)
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), bf), _t("w_router", w_router, (E, d), bf),
            _t("logit_offset", logit_offset, (E,), f32, False),
            _t("bias", bias, (E,), f32, False),
            _t("token_ids", token_ids, (T,), torch.int32, hsh),
            _t("tid2eid", tid2eid, (cfg.vocab, k), torch.int32, hsh),
            _t("w13q", w13q, (E, 2 * F, d), u8), _t("w13s", w13s, (E, 2 * F // 128, d // 128), f32),
            _t("w2q", w2q, (E, d, F), u8), _t("w2s", w2s, (E, d // 128, F // 128), f32),
            _t("w13q_shared", w13q_shared, (2 * F, d), u8, sh),
            _t("w13s_shared", w13s_shared, (2 * F // 128, d // 128), f32, sh),
            _t("w2q_shared", w2q_shared, (d, F), u8, sh),
            _t("w2s_shared", w2s_shared, (d // 128, F // 128), f32, sh),
            _t("out", out, (T, d), bf),
            _t("topk_ids_out", topk_ids_out, (T, k), torch.int32, False),
            _t("topk_weights_out", topk_weights_out, (T, k), f32, False),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_forward_fp8", load_library().moe_forward_fp8(*args))


def quantize_fp8_weights(inp, stream=None):
    """FP8 copies of the expert weights of an input dict (w13, w2 and the shared
    expert's), quantized on the GPU in 128x128 tiles: returns a dict with w13q,
    w13s, w2q, w2s (and *_shared when present)."""
    out = {}
    for name in ("w13", "w2", "w13_shared", "w2_shared"):
        w = inp.get(name)
        if w is None:
            continue
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
        s = torch.empty(tuple(w.shape[:-2]) + (w.shape[-2] // 128, w.shape[-1] // 128),
                        dtype=torch.float32, device=w.device)
        moe_quantize_fp8_blocks(w, q, s, stream)
        base = name.replace("_shared", "")
        suffix = "_shared" if name.endswith("_shared") else ""
        out[base + "q" + suffix] = q
        out[base + "s" + suffix] = s
    return out


def moe_quantize_mxfp4(w, q, scales, stream=None):
    """w [R, C] or [n, R, C] float32/bfloat16 (C a multiple of 128, R even) ->
    q [..., R/2, C] uint8 packed E2M1 in row pairs (row pair i, 128-column block j:
    64 bytes of row 2i, then 64 of row 2i+1), scales [..., C/128, R, 4] uint8 E8M0
    (K-block-major)."""
    if w.dtype not in _IN_DTYPES:
        raise ValueError("w must be float32 or bfloat16, got %s" % w.dtype)
    if w.dim() not in (2, 3):
        raise ValueError("w must be [R, C] or [n, R, C]")
    R, C_ = w.shape[-2], w.shape[-1]
    n = w.shape[0] if w.dim() == 3 else 1
    lead = tuple(w.shape[:-2])
    args = [n, R, C_, _IN_DTYPES[w.dtype], _t("w", w, tuple(w.shape), w.dtype),
            _t("q", q, lead + (R // 2, C_), torch.uint8),
            _t("scales", scales, lead + (C_ // 128, R, 4), torch.uint8), _stream(stream)]
    _check("moe_quantize_mxfp4", load_library().moe_quantize_mxfp4(*args))


def moe_expert_up_mxfp4(cfg, xq, xs, sorted_token_ids, expert_offsets, w13q, w13s, hq, hs,
                        workspace, stream=None):
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    u8, f32 = torch.uint8, torch.float32
    args = [C.byref(cfg),
            _t("xq", xq, (T, d), u8), _t("xs", xs, (d // 128, T), f32),
            _t("sorted_token_ids", sorted_token_ids, (T * k,), torch.int32),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w13q", w13q, (E, F, d), u8),
            _t("w13s", w13s, (E, d // 128, 2 * F, 4), u8),
            _t("hq", hq, (T * k, F), u8), _t("hs", hs, (F // 128, T * k), f32),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_up_mxfp4", load_library().moe_expert_up_mxfp4(*args))


def moe_expert_down_mxfp4(cfg, hq, hs, expert_offsets, w2q, w2s, expert_out, workspace,
                          stream=None):
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    u8, f32 = torch.uint8, torch.float32
    args = [C.byref(cfg),
            _t("hq", hq, (T * k, F), u8), _t("hs", hs, (F // 128, T * k), f32),
            _t("expert_offsets", expert_offsets, (E + 1,), torch.int32),
            _t("w2q", w2q, (E, d // 2, F), u8), _t("w2s", w2s, (E, F // 128, d, 4), u8),
            _t("expert_out", expert_out, (T * k, d), torch.bfloat16),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_expert_down_mxfp4", load_library().moe_expert_down_mxfp4(*args))


def moe_forward_mxfp4(cfg, hidden, w_router, logit_offset, bias, token_ids, tid2eid, w13q, w13s,
                      w2q, w2s, w13q_shared, w13s_shared, w2q_shared, w2s_shared, out,
                      topk_ids_out, topk_weights_out, workspace, stream=None):
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    hsh = cfg.route_mode == MOE_ROUTE_HASH
    sh = bool(cfg.n_shared)
    args = [C.byref(cfg),
            _t("hidden", hidden, (T, d), bf), _t("w_router", w_router, (E, d), bf),
            _t("logit_offset", logit_offset, (E,), f32, False),
            _t("bias", bias, (E,), f32, False),
            _t("token_ids", token_ids, (T,), torch.int32, hsh),
            _t("tid2eid", tid2eid, (cfg.vocab, k), torch.int32, hsh),
            _t("w13q", w13q, (E, F, d), u8),
            _t("w13s", w13s, (E, d // 128, 2 * F, 4), u8),
            _t("w2q", w2q, (E, d // 2, F), u8), _t("w2s", w2s, (E, F // 128, d, 4), u8),
            _t("w13q_shared", w13q_shared, (F, d), u8, sh),
            _t("w13s_shared", w13s_shared, (d // 128, 2 * F, 4), u8, sh),
            _t("w2q_shared", w2q_shared, (d // 2, F), u8, sh),
            _t("w2s_shared", w2s_shared, (F // 128, d, 4), u8, sh),
            _t("out", out, (T, d), bf),
            _t("topk_ids_out", topk_ids_out, (T, k), torch.int32, False),
            _t("topk_weights_out", topk_weights_out, (T, k), f32, False),
            *_ws(cfg, workspace), _stream(stream)]
    _check("moe_forward_mxfp4", load_library().moe_forward_mxfp4(*args))


def quantize_mxfp4_weights(inp, stream=None):
    """MXFP4 copies of the expert weights of an input dict (w13, w2 and the
    shared expert's), quantized on the GPU in 1x32 blocks: returns a dict with
    w13q, w13s, w2q, w2s (and *_shared when present)."""
    out = {}
    for name in ("w13", "w2", "w13_shared", "w2_shared"):
        w = inp.get(name)
        if w is None:
            continue
        lead, R, C_ = tuple(w.shape[:-2]), w.shape[-2], w.shape[-1]
        q = torch.empty(lead + (R // 2, C_), dtype=torch.uint8, device=w.device)
        s = torch.empty(lead + (C_ // 128, R, 4), dtype=torch.uint8, device=w.device)
        moe_quantize_mxfp4(w, q, s, stream)
        base = name.replace("_shared", "")
        suffix = "_shared" if name.endswith("_shared") else ""
        out[base + "q" + suffix] = q
        out[base + "s" + suffix] = s
    return out


def moe_strerror(status: int) -> str:
    return load_library().moe_strerror(int(status)).decode()


class MoELayer:
    """Convenience holder: weights, a workspace and moe_forward on the current stream."""

    def __init__(self, cfg: MoeConfig, inputs: dict, device="cuda"):
        self.cfg = cfg
        self.inp = inputs
        self.workspace = torch.empty(moe_workspace_size(cfg), dtype=torch.uint8, device=device)
        self.out = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=device)
        self.ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=device)
        self.gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=device)

    def forward(self, stream=None):
        i = self.inp
        moe_forward(self.cfg, i["hidden"], i["w_router"], i.get("logit_offset"), i.get("bias"),
                    i.get("token_ids"), i.get("tid2eid"), i["w13"], i["w2"], i.get("w13_shared"),
                    i.get("w2_shared"), self.out, self.ids, self.gates, self.workspace, stream)
        return self.out

    def forward_fp8(self, fp8, stream=None):
        """The layer with FP8 experts; fp8 = quantize_fp8_weights(inputs)."""
        i = self.inp
        moe_forward_fp8(self.cfg, i["hidden"], i["w_router"], i.get("logit_offset"), i.get("bias"),
                        i.get("token_ids"), i.get("tid2eid"), fp8["w13q"], fp8["w13s"],
                        fp8["w2q"], fp8["w2s"], fp8.get("w13q_shared"), fp8.get("w13s_shared"),
                        fp8.get("w2q_shared"), fp8.get("w2s_shared"), self.out, self.ids,
                        self.gates, self.workspace, stream)
        return self.out

    def forward_mxfp4(self, mx, stream=None):
        """The layer with MXFP4 expert weights; mx = quantize_mxfp4_weights(inputs)."""
        i = self.inp
        moe_forward_mxfp4(self.cfg, i["hidden"], i["w_router"], i.get("logit_offset"),
                          i.get("bias"), i.get("token_ids"), i.get("tid2eid"), mx["w13q"],
                          mx["w13s"], mx["w2q"], mx["w2s"], mx.get("w13q_shared"),
                          mx.get("w13s_shared"), mx.get("w2q_shared"), mx.get("w2s_shared"),
                          self.out, self.ids, self.gates, self.workspace, stream)
        return self.out
