"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on host copies of the same input buffers, compare.

Tolerances (written here once, used by every parity test):
  * routing ids, permutation, offsets, dispatch index: bit-exact; a token whose
    deciding key gap (oracle margin) is <= TIE_GIVEN (identical logits) or
    <= TIE_LAYER (each side computes its own logits) is a near-tie: its ids are
    checked for validity instead of equality.
  * gates: absolute 1e-6.
  * layer / expert outputs, per token row: max |gpu - oracle| / max(max |oracle|, 1e-6)
    <= 2e-2 for bf16, <= 1e-4 for fp32.
"""
import numpy as np
import torch

import mixture_experts_ffn_sqrt_amd as moe
import oracle as O
from mixture_experts_ffn_sqrt_amd.synth import to_host_bits

TIE_GIVEN = 1e-6
TIE_LAYER = 2e-5
GATE_TOL = 1e-6


def out_tol(dtype):
    return 1e-4 if dtype == "f32" else 2e-2


def row_rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(gpu - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-6)
    return num / den


def to_f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def cfg_of(lc, **over):
    """C-ABI config from a synth.LayerConfig."""
    kw = dict(T=lc.T, d=lc.d, E=lc.E, k=lc.k, d_ff=lc.d_ff, n_shared=lc.n_shared,
              dtype=lc.dtype, scoring=lc.scoring, n_group=lc.n_group, topk_group=lc.topk_group,
              group_topk=lc.group_topk, vocab=lc.hash_vocab)
    kw.update(over)
    return moe.make_config(**kw)


def gpu_forward(c, inp):
    layer = moe.MoELayer(c, inp)
    out = layer.forward()
    torch.cuda.synchronize()
    return out, layer.ids, layer.gates


def oracle_layer_rows(lc, inp, rows, route_mode=O.LEARNED, w13_host=None, w2_host=None):
    """Oracle outputs for the listed token rows, on host copies of `inp`.
    Only the experts the listed tokens select are copied to the host."""
    h = to_host_bits(inp["hidden"])
    wr = to_host_bits(inp["w_router"])
    bias = to_host_bits(inp.get("bias"))
    off = to_host_bits(inp.get("logit_offset"))
    tok = to_host_bits(inp.get("token_ids"))
    tab = to_host_bits(inp.get("tid2eid"))
    rows = np.asarray(rows, np.int32)
    grp = dict(n_group=lc.n_group, topk_group=lc.topk_group, group_topk=lc.group_topk)
    # pass 1: routing only (no expert weights needed) to learn which experts to copy
    if w13_host is None:
        lg = O.logits(h, wr, rows=rows, logit_offset=off).astype(np.float32)
        if route_mode == O.HASH:
            ids, _ = O.hash_route(lg, tok[rows], tab, lc.scoring)
        else:
            ids, _, _ = O.route(lg, lc.k, lc.scoring, bias=bias, **grp)
        need = sorted(set(ids.ravel().tolist()))
        w13_host = [None] * lc.E
        w2_host = [None] * lc.E
        for e in need:
            w13_host[e] = to_host_bits(inp["w13"][e])
            w2_host[e] = to_host_bits(inp["w2"][e])
    s13 = to_host_bits(inp.get("w13_shared"))
    s2 = to_host_bits(inp.get("w2_shared"))
    return O.layer(h, wr, w13_host, w2_host, k=lc.k, scoring=lc.scoring, rows=rows, bias=bias,
                   logit_offset=off, w13_shared=s13, w2_shared=s2, route_mode=route_mode,
                   token_ids=tok, tid2eid=tab, **grp)


def check_layer(lc, inp, gpu_out, gpu_ids, gpu_gates, rows, route_mode=O.LEARNED,
                max_tie_frac=0.02):
    """Compare GPU layer outputs with the oracle on the listed rows.  Returns a
    dict of summary numbers."""
    ref = oracle_layer_rows(lc, inp, rows, route_mode)
    rows = np.asarray(rows)
    g_ids = gpu_ids.cpu().numpy()[rows]
    g_gates = gpu_gates.cpu().numpy()[rows]
    g_out = to_f64(gpu_out)[rows]
    tie = (ref["margin"] <= TIE_LAYER) if route_mode == O.LEARNED else np.zeros(len(rows), bool)
    ok = ~tie
    assert tie.sum() <= max(2, max_tie_frac * len(rows)), \
        "too many near-ties: %d of %d" % (tie.sum(), len(rows))
    assert np.array_equal(g_ids[ok], ref["ids"][ok]), "topk_ids differ on non-tie tokens"
    assert np.abs(g_gates[ok] - ref["gates"][ok]).max(initial=0) <= 1e-5
    err = row_rel_err(g_out[ok], ref["out"][ok])
    tol = out_tol(lc.dtype)
    assert err.max(initial=0) <= tol, "max row rel err %.3g > %.3g" % (err.max(), tol)
    fro = np.linalg.norm(g_out[ok] - ref["out"][ok]) / max(np.linalg.norm(ref["out"][ok]), 1e-30)
    return dict(max_row_rel_err=float(err.max(initial=0)), fro_rel_err=float(fro),
                ties=int(tie.sum()), rows=int(len(rows)))


def check_routing(ids, gates, ref_ids, ref_gates, margin, keys=None, tie=TIE_GIVEN):
    """ids bit-exact except near-ties; near-tie tokens must pick keys within `tie`
    of the oracle's selected keys (valid alternative choices)."""
    ok = margin > tie
    assert np.array_equal(ids[ok], ref_ids[ok])
    assert np.abs(gates[ok] - ref_gates[ok]).max(initial=0) <= GATE_TOL
    if keys is not None:
        for t in np.nonzero(~ok)[0]:
            a = np.sort(keys[t, ids[t]])
            b = np.sort(keys[t, ref_ids[t]])
            assert np.all(np.abs(a - b) <= tie * 4)
    return int((~ok).sum())


def hot_cold_rows(ids, counts, n=2):
    """Token rows routed to the expert with the most rows and to the expert with
    the fewest (but some) rows: on a skewed workload the first runs on the
    288-row tiles, the second on the small-group streaming tiles."""
    hot = int(np.argmax(counts))
    cold = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    return np.r_[np.nonzero((ids == hot).any(1))[0][:n], np.nonzero((ids == cold).any(1))[0][:n]]
