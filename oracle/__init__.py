"""The oracle: TEST INFRASTRUCTURE ONLY.

A plain CPU statement of the single-GPU MoE FFN layer (moe_oracle.c), loaded
through ctypes.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product path never does.  It shares no
code with the HIP library.  Arrays in, arrays out (numpy); bf16 tensors are
passed as their raw uint16 bit patterns.

See moe_oracle.c for the pages and sections each function follows.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

SOFTMAX, SIGMOID, SQRTSOFTPLUS = 0, 1, 2
LEARNED, HASH = 0, 1
F32, BF16 = 0, 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        # MOE_ORACLE_LIB: a library built from a modified copy of moe_oracle.c,
        # so that a test can plant a mistake in the oracle and see the pins fail
        path = os.environ.get("MOE_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and (not os.path.exists(path) or
                                   os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = C.CDLL(path)
        P, I, F = C.c_void_p, C.c_int, C.c_float
        L.oracle_affinity.argtypes = [F, I]
        L.oracle_affinity.restype = F
        L.oracle_route.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P]
        L.oracle_hash_route.argtypes = [I, I, I, I, P, P, P, I, P, P]
        L.oracle_permute.argtypes = [I, I, I, P, P, P, P, P, P, P]
        L.oracle_combine.argtypes = [I, I, P, P, P, P]
        L.oracle_combine.restype = None
        L.oracle_expert_ffn.argtypes = [I, I, P, P, P, I, P]
        L.oracle_expert_ffn.restype = None
        L.oracle_logits.argtypes = [I, P, I, I, P, P, I, P, P]
        L.oracle_logits.restype = None
        L.oracle_layer.argtypes = [I, P, I, I, I, I, I, I, I, I, I, I, I,
                                   P, P, P, P, P, P, I, P, P, P, P, P, P, P, P]
        L.oracle_expert_rows.argtypes = [I, P, I, I, P, I, P, P, P]
        L.oracle_expert_rows.restype = None
        L.oracle_expert_rows_lowp.argtypes = [I, I, P, I, I, P, I, P, P, P, P, P]
        L.oracle_expert_rows_lowp.restype = None
        L.oracle_set_num_threads.argtypes = [I]
        L.oracle_set_num_threads.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_decode.restype = C.c_double
        L.oracle_e4m3_encode.argtypes = [F]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_quantize_rows.argtypes = [I, I, P, P, P]
        L.oracle_quantize_rows.restype = None
        L.oracle_quantize_blocks.argtypes = [I, I, P, I, P, P]
        L.oracle_quantize_blocks.restype = None
        L.oracle_expert_ffn_fp8.argtypes = [I, I, P, P, P, P, P, P, P]
        L.oracle_expert_up_fp8.argtypes = [I, I, P, P, P, P, P, P]
        L.oracle_expert_up_fp8.restype = None
        L.oracle_expert_ffn_fp8.restype = None
        L.oracle_layer_fp8.argtypes = [I, P, I, I, I, I, I, I, I, I, I, I, I,
                                       P, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, P]
        L.oracle_layer_fp8.restype = I
        L.oracle_e2m1_decode.argtypes = [C.c_uint8]
        L.oracle_e2m1_decode.restype = C.c_double
        L.oracle_e2m1_encode.argtypes = [F]
        L.oracle_e2m1_encode.restype = C.c_uint8
        L.oracle_quantize_mxfp4.argtypes = [I, I, P, I, P, P]
        L.oracle_quantize_mxfp4.restype = None
        L.oracle_expert_up_mxfp4.argtypes = [I, I, P, P, P, P, P, P]
        L.oracle_expert_up_mxfp4.restype = None
        L.oracle_expert_ffn_mxfp4.argtypes = [I, I, P, P, P, P, P, P, P]
        L.oracle_expert_ffn_mxfp4.restype = None
        L.oracle_layer_mxfp4.argtypes = L.oracle_layer_fp8.argtypes
        L.oracle_layer_mxfp4.restype = I
        for name in ("oracle_route", "oracle_hash_route", "oracle_permute",
                     "oracle_layer", "oracle_num_threads"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _tensor(a):
    """float32 array -> (array, F32); uint16 (bf16 bits) -> (array, BF16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("oracle tensors are float32 or uint16 bf16 bit patterns, got %s" % a.dtype)


def affinity(l, scoring):
    """Affinity of one float logit (float arithmetic, C library exp/log1p/sqrt)."""
    return lib().oracle_affinity(float(l), int(scoring))


def route(logits, k, scoring, bias=None, n_group=1, topk_group=1, group_topk=0):
    """Learned routing from given float logits [T, E] -> (ids [T,k] int32,
    gates [T,k] float32, margin [T] float32)."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float32)
    margin = np.zeros(T, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    rc = lib().oracle_route(T, E, k, scoring, n_group, topk_group, group_topk,
                            _p(lg), _p(b), _p(ids), _p(gates), _p(margin))
    if rc:
        raise ValueError("oracle_route rejected its arguments")
    return ids, gates, margin


def hash_route(logits, token_ids, tid2eid, scoring):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    tab = _c(tid2eid, np.int32)
    vocab, k = tab.shape
    tok = _c(token_ids, np.int32)
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float32)
    rc = lib().oracle_hash_route(T, E, k, scoring, _p(lg), _p(tok), _p(tab), vocab,
                                 _p(ids), _p(gates))
    if rc:
        raise ValueError("oracle_hash_route rejected its arguments")
    return ids, gates


def permute(ids, gates, E):
    """Expert-major dispatch -> dict(counts, offsets, sorted_token_ids,
    sorted_weights, dispatch_index)."""
    ids = _c(ids, np.int32)
    gates = _c(gates, np.float32)
    T, k = ids.shape
    out = dict(counts=np.zeros(E, np.int32), offsets=np.zeros(E + 1, np.int32),
               sorted_token_ids=np.zeros(T * k, np.int32),
               sorted_weights=np.zeros(T * k, np.float32),
               dispatch_index=np.zeros((T, k), np.int32))
    rc = lib().oracle_permute(T, k, E, _p(ids), _p(gates), _p(out["counts"]),
                              _p(out["offsets"]), _p(out["sorted_token_ids"]),
                              _p(out["sorted_weights"]), _p(out["dispatch_index"]))
    if rc:
        raise ValueError("oracle_permute: an id lies outside [0, E)")
    return out


def combine(expert_out, token_of_row, weight_of_row, T, out=None):
    """index_add_-style combine of dispatch rows into T output rows (double)."""
    eo = _c(expert_out, np.float64)
    P, d = eo.shape
    tok = _c(token_of_row, np.int32)
    w = _c(weight_of_row, np.float32)
    o = np.zeros((T, d), np.float64) if out is None else _c(out, np.float64).copy()
    lib().oracle_combine(P, d, _p(eo), _p(tok), _p(w), _p(o))
    return o


def expert_ffn(x, w13_e, w2_e):
    """One SwiGLU expert on one row x [d] (double result)."""
    w13_e, dt = _tensor(w13_e)
    w2_e, dt2 = _tensor(w2_e)
    assert dt == dt2
    d_ff2, d = w13_e.shape
    xx = _c(x, np.float64)
    y = np.zeros(d, np.float64)
    lib().oracle_expert_ffn(d, d_ff2 // 2, _p(xx), _p(w13_e), _p(w2_e), dt, _p(y))
    return y


def expert_rows(hidden, tokens, w13_e, w2_e):
    """One SwiGLU expert on the listed token rows of hidden [T, d]: [n, d] double,
    row q = expert_ffn(hidden[tokens[q]], w13_e, w2_e)."""
    h, dt = _tensor(hidden)
    w13_e, dt2 = _tensor(w13_e)
    w2_e, dt3 = _tensor(w2_e)
    assert dt == dt2 == dt3
    d = h.shape[1]
    d_ff = w13_e.shape[0] // 2
    tok = _c(tokens, np.int32)
    y = np.zeros((len(tok), d), np.float64)
    lib().oracle_expert_rows(len(tok), _p(tok), d, d_ff, _p(h), dt, _p(w13_e), _p(w2_e), _p(y))
    return y


def logits(hidden, w_router, rows=None, logit_offset=None):
    h, dt = _tensor(hidden)
    w, dt2 = _tensor(w_router)
    assert dt == dt2
    T, d = h.shape
    E = w.shape[0]
    r = np.arange(T, dtype=np.int32) if rows is None else _c(rows, np.int32)
    out = np.zeros((len(r), E), np.float64)
    off = None if logit_offset is None else _c(logit_offset, np.float32)
    lib().oracle_logits(len(r), _p(r), d, E, _p(h), _p(w), dt, _p(off), _p(out))
    return out


def layer(hidden, w_router, w13, w2, k, scoring, rows=None, bias=None,
          logit_offset=None, n_group=1, topk_group=1, group_topk=0,
          w13_shared=None, w2_shared=None, route_mode=LEARNED, token_ids=None,
          tid2eid=None):
    """The whole layer for the listed token rows.

    w13 / w2 are either stacked arrays [E, ...] or sequences of per-expert arrays
    (None for experts no listed token selects).  Returns dict(out [n, d] double,
    ids [n, k], gates [n, k], margin [n])."""
    h, dt = _tensor(hidden)
    wr, _ = _tensor(w_router)
    T, d = h.shape
    E = wr.shape[0]
    keep = []

    def ptrs(ws):
        arr = (C.c_void_p * E)()
        for e in range(E):
            w = ws[e]
            if w is None:
                arr[e] = None
            else:
                w, dte = _tensor(w)
                assert dte == dt
                keep.append(w)
                arr[e] = w.ctypes.data
        return arr

    p13, p2 = ptrs(w13), ptrs(w2)
    first = next(w for w in w13 if w is not None)
    d_ff = np.asarray(first).shape[0] // 2
    n_shared = 0 if w13_shared is None else 1
    s13 = s2 = None
    if n_shared:
        s13, _ = _tensor(w13_shared)
        s2, _ = _tensor(w2_shared)
    r = np.arange(T, dtype=np.int32) if rows is None else _c(rows, np.int32)
    n = len(r)
    out = np.zeros((n, d), np.float64)
    ids = np.zeros((n, k), np.int32)
    gates = np.zeros((n, k), np.float32)
    margin = np.zeros(n, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    off = None if logit_offset is None else _c(logit_offset, np.float32)
    tok = None if token_ids is None else _c(token_ids, np.int32)
    tab = None if tid2eid is None else _c(tid2eid, np.int32)
    vocab = 0 if tab is None else tab.shape[0]
    rc = lib().oracle_layer(n, _p(r), d, E, k, d_ff, n_shared, dt, scoring, route_mode,
                            n_group, topk_group, group_topk, _p(h), _p(wr), _p(b), _p(off),
                            _p(tok), _p(tab), vocab,
                            C.cast(p13, C.c_void_p), C.cast(p2, C.c_void_p),
                            _p(s13), _p(s2), _p(out), _p(ids), _p(gates), _p(margin))
    if rc:
        raise ValueError("oracle_layer rejected its arguments (missing expert weights?)")
    return dict(out=out, ids=ids, gates=gates, margin=margin)


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    """Threads of the oracle's later parallel loops (for a single-core timing)."""
    lib().oracle_set_num_threads(int(n))


# ----------------------------------------------------------------------------
# FP8 (E4M3) experts
# ----------------------------------------------------------------------------
def e4m3_decode(codes):
    """E4M3 codes (uint8 array or int) -> float64 values."""
    c = np.asarray(codes, np.uint8)
    f = np.vectorize(lambda v: lib().oracle_e4m3_decode(int(v)), otypes=[np.float64])
    return f(c)


def e4m3_encode(values):
    """float32 values -> nearest E4M3 codes (ties to even, saturated to +-448)."""
    v = np.asarray(values, np.float32)
    f = np.vectorize(lambda x: lib().oracle_e4m3_encode(float(x)), otypes=[np.uint8])
    return f(v)


def quantize_rows(x):
    """float32 [n, K] (K a multiple of 128) -> (codes uint8 [n, K], scales float32 [n, K/128])."""
    x = _c(x, np.float32)
    n, K = x.shape
    q = np.zeros((n, K), np.uint8)
    s = np.zeros((n, K // 128), np.float32)
    lib().oracle_quantize_rows(n, K, _p(x), _p(q), _p(s))
    return q, s


def quantize_blocks(w):
    """[R, C] float32 or bf16 bits (both multiples of 128) -> (codes uint8 [R, C],
    scales float32 [R/128, C/128]), one scale per 128x128 tile."""
    w, dt = _tensor(w)
    R, Cc = w.shape
    q = np.zeros((R, Cc), np.uint8)
    s = np.zeros((R // 128, Cc // 128), np.float32)
    lib().oracle_quantize_blocks(R, Cc, _p(w), dt, _p(q), _p(s))
    return q, s


def expert_ffn_fp8(xq, xs, w13q, w13s, w2q, w2s):
    """One FP8 SwiGLU expert on one quantized row (codes xq [d], scales xs [d/128])."""
    xq, xs = _c(xq, np.uint8), _c(xs, np.float32)
    w13q, w13s, w2q, w2s = (_c(w13q, np.uint8), _c(w13s, np.float32), _c(w2q, np.uint8),
                            _c(w2s, np.float32))
    d = xq.shape[0]
    d_ff = w13q.shape[0] // 2
    y = np.zeros(d, np.float64)
    lib().oracle_expert_ffn_fp8(d, d_ff, _p(xq), _p(xs), _p(w13q), _p(w13s), _p(w2q), _p(w2s),
                                _p(y))
    return y


def expert_up_fp8(xq, xs, w13q, w13s):
    """The up half of an FP8 expert on one quantized row: (hq [d_ff] codes, hs [d_ff/128])."""
    xq, xs = _c(xq, np.uint8), _c(xs, np.float32)
    w13q, w13s = _c(w13q, np.uint8), _c(w13s, np.float32)
    d = xq.shape[0]
    d_ff = w13q.shape[0] // 2
    hq = np.zeros(d_ff, np.uint8)
    hs = np.zeros(d_ff // 128, np.float32)
    lib().oracle_expert_up_fp8(d, d_ff, _p(xq), _p(xs), _p(w13q), _p(w13s), _p(hq), _p(hs))
    return hq, hs


def layer_fp8(hidden, w_router, w13q, w13s, w2q, w2s, k, scoring, **kw):
    """The layer with FP8 experts for the listed token rows.  w13q/w13s/w2q/w2s:
    sequences over experts of per-expert arrays (None where not needed); keyword
    arguments as for layer_mxfp4.  Returns dict(out, ids, gates, margin)."""
    return _layer_lowp("oracle_layer_fp8", np.float32, hidden, w_router, w13q, w13s, w2q, w2s,
                       k, scoring, **kw)


def _layer_lowp(fn, scale_dtype, hidden, w_router, w13q, w13s, w2q, w2s, k, scoring, rows=None,
                bias=None, logit_offset=None, n_group=1, topk_group=1, group_topk=0, shared=None,
                route_mode=LEARNED, token_ids=None, tid2eid=None, d_ff=None):
    h, dt = _tensor(hidden)
    wr, _ = _tensor(w_router)
    T, d = h.shape
    E = wr.shape[0]
    keep = []

    def ptrs(ws, dtype):
        arr = (C.c_void_p * E)()
        for e in range(E):
            if ws[e] is None:
                arr[e] = None
            else:
                a = _c(ws[e], dtype)
                keep.append(a)
                arr[e] = a.ctypes.data
        return arr

    pq13, ps13 = ptrs(w13q, np.uint8), ptrs(w13s, scale_dtype)
    pq2, ps2 = ptrs(w2q, np.uint8), ptrs(w2s, scale_dtype)
    if d_ff is None:
        first = next(w for w in w13q if w is not None)
        d_ff = np.asarray(first).shape[0] // 2
    sh = [None] * 4
    if shared is not None:
        sh = [_c(shared[0], np.uint8), _c(shared[1], scale_dtype), _c(shared[2], np.uint8),
              _c(shared[3], scale_dtype)]
    r = np.arange(T, dtype=np.int32) if rows is None else _c(rows, np.int32)
    n = len(r)
    out = np.zeros((n, d), np.float64)
    ids = np.zeros((n, k), np.int32)
    gates = np.zeros((n, k), np.float32)
    margin = np.zeros(n, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    off = None if logit_offset is None else _c(logit_offset, np.float32)
    tok = None if token_ids is None else _c(token_ids, np.int32)
    tab = None if tid2eid is None else _c(tid2eid, np.int32)
    vocab = 0 if tab is None else tab.shape[0]
    rc = getattr(lib(), fn)(n, _p(r), d, E, k, d_ff, 0 if shared is None else 1, dt,
                            scoring, route_mode, n_group, topk_group, group_topk, _p(h),
                            _p(wr), _p(b), _p(off), _p(tok), _p(tab), vocab,
                            C.cast(pq13, C.c_void_p), C.cast(ps13, C.c_void_p),
                            C.cast(pq2, C.c_void_p), C.cast(ps2, C.c_void_p),
                            _p(sh[0]), _p(sh[1]), _p(sh[2]), _p(sh[3]),
                            _p(out), _p(ids), _p(gates), _p(margin))
    if rc:
        raise ValueError("%s rejected its arguments (missing expert weights?)" % fn)
    return dict(out=out, ids=ids, gates=gates, margin=margin)


# ----------------------------------------------------------------------------
# MXFP4 (E2M1, 1x32 E8M0 scales) expert weights
# ----------------------------------------------------------------------------
def e2m1_decode(codes):
    """E2M1 codes (0..15, uint8 array or int) -> float64 values."""
    c = np.asarray(codes, np.uint8)
    f = np.vectorize(lambda v: lib().oracle_e2m1_decode(int(v)), otypes=[np.float64])
    return f(c)


def e2m1_encode(values):
    """float32 values -> nearest E2M1 codes (ties to even, saturated to +-6)."""
    v = np.asarray(values, np.float32)
    f = np.vectorize(lambda x: lib().oracle_e2m1_encode(float(x)), otypes=[np.uint8])
    return f(v)


def quantize_mxfp4(w):
    """[R, C] float32 or bf16 bits (C a multiple of 32) -> (packed codes uint8
    [R, C/2], element 2j in the low nibble; E8M0 scale bytes uint8 [R, C/32])."""
    w, dt = _tensor(w)
    R, Cc = w.shape
    q = np.zeros((R, Cc // 2), np.uint8)
    s = np.zeros((R, Cc // 32), np.uint8)
    lib().oracle_quantize_mxfp4(R, Cc, _p(w), dt, _p(q), _p(s))
    return q, s


def mxfp4_dequantize(q, s):
    """(packed codes [R, C/2], E8M0 bytes [R, C/32]) -> float64 [R, C]."""
    q, s = np.asarray(q, np.uint8), np.asarray(s, np.uint8)
    R = q.shape[0]
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(R, -1)
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    return e2m1_decode(codes) * np.repeat(scale, 32, axis=1)


def expert_up_mxfp4(xq, xs, w13q, w13s):
    """The up half of an MXFP4 expert on one FP8 row: (hq [d_ff] codes, hs [d_ff/128])."""
    xq, xs = _c(xq, np.uint8), _c(xs, np.float32)
    w13q, w13s = _c(w13q, np.uint8), _c(w13s, np.uint8)
    d = xq.shape[0]
    d_ff = w13q.shape[0] // 2
    hq = np.zeros(d_ff, np.uint8)
    hs = np.zeros(d_ff // 128, np.float32)
    lib().oracle_expert_up_mxfp4(d, d_ff, _p(xq), _p(xs), _p(w13q), _p(w13s), _p(hq), _p(hs))
    return hq, hs


def expert_ffn_mxfp4(xq, xs, w13q, w13s, w2q, w2s):
    """One SwiGLU expert with MXFP4 weights on one FP8 row (codes xq [d], scales xs [d/128])."""
    xq, xs = _c(xq, np.uint8), _c(xs, np.float32)
    w13q, w13s, w2q, w2s = (_c(w13q, np.uint8), _c(w13s, np.uint8), _c(w2q, np.uint8),
                            _c(w2s, np.uint8))
    d = xq.shape[0]
    d_ff = w13q.shape[0] // 2
    y = np.zeros(d, np.float64)
    lib().oracle_expert_ffn_mxfp4(d, d_ff, _p(xq), _p(xs), _p(w13q), _p(w13s), _p(w2q),
                                  _p(w2s), _p(y))
    return y


def expert_rows_lowp(fmt, hidden, tokens, w13q, w13s, w2q, w2s):
    """One low-precision expert on the listed token rows of hidden [T, d] (bf16
    bits or float32): each row is quantized 1x128 as in the FP8 layer, then
    expert_ffn_fp8 (fmt "fp8": float tile scales) or expert_ffn_mxfp4 (fmt
    "mxfp4": E8M0 block scales [R, C/32]).  Returns [n, d] double."""
    h, dt = _tensor(hidden)
    sd = np.float32 if fmt == "fp8" else np.uint8
    w13q, w13s, w2q, w2s = (_c(w13q, np.uint8), _c(w13s, sd), _c(w2q, np.uint8), _c(w2s, sd))
    d = h.shape[1]
    d_ff = w13q.shape[0] // 2
    tok = _c(tokens, np.int32)
    y = np.zeros((len(tok), d), np.float64)
    lib().oracle_expert_rows_lowp(0 if fmt == "fp8" else 1, len(tok), _p(tok), d, d_ff, _p(h),
                                  dt, _p(w13q), _p(w13s), _p(w2q), _p(w2s), _p(y))
    return y


def layer_mxfp4(hidden, w_router, w13q, w13s, w2q, w2s, k, scoring, **kw):
    """The layer with MXFP4 expert weights for the listed token rows (keyword
    arguments: rows, bias, logit_offset, n_group, topk_group, group_topk, shared =
    (w13q, w13s, w2q, w2s), route_mode, token_ids, tid2eid).  Returns
    dict(out, ids, gates, margin)."""
    return _layer_lowp("oracle_layer_mxfp4", np.uint8, hidden, w_router, w13q, w13s, w2q, w2s,
                       k, scoring, **kw)
