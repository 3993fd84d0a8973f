"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on host copies of the same input buffers, compare.

Tolerances (written here once, used by every parity test):
  * routing ids, permutation, offsets, dispatch index: bit-exact.  A token
    whose deciding key gap (the oracle's margin: the smallest gap between a
    kept and a dropped key or group score, or between consecutive selected
    keys) is <= TIE_GIVEN (both sides route the same logits) or <= TIE_LAYER
    (each side computes its own logits) is a near-tie.  For a near-tie token
    the GPU's ids must be a valid alternative choice: keys (and, with groups,
    group scores) that the rule would pick if the near-tied decision went the
    other way, within TIE_VALID.  Its output row is then checked against the
    oracle routed on the GPU's ids, with the same row tolerance as any other.
  * near-ties are rare: a deciding gap below TIE_LAYER has probability about
    (number of deciding gaps) * TIE_LAYER / (typical gap), about 2% of tokens
    for DeepSeek-V3-shaped routing (9 deciding gaps of ~0.01 among 128 kept
    keys); MAX_TIE_FRAC bounds the count at 5% (plus 3 rows).
  * gates: absolute GATE_TOL_GIVEN = 1e-6 from identical logits,
    GATE_TOL_LAYER = 1e-5 when each side computes its own logits (the float32
    logits then differ by ~1e-6).
  * layer / expert outputs, per token row: max |gpu - oracle| / max(max |oracle|, 1e-6)
    <= 2e-2 for bf16, <= 1e-4 for fp32 (the low-precision experts' bounds are
    in their test modules).

The oracle side of a layer check is assembled from the oracle's own pieces
(logits, routing, one expert over many rows, combine), one expert's weights on
the host at a time, so that a full-size workload can be checked on thousands
of rows without copying every expert at once.
"""
import itertools

import numpy as np
import torch

import mixture_experts_ffn_sqrt_amd as moe
import oracle as O
from mixture_experts_ffn_sqrt_amd.synth import to_host_bits

TIE_GIVEN = 1e-6
TIE_LAYER = 2e-5
TIE_VALID = 2 * TIE_LAYER
GATE_TOL_GIVEN = 1e-6
GATE_TOL_LAYER = 1e-5
GATE_TOL = GATE_TOL_GIVEN
MAX_TIE_FRAC, MAX_TIE_EXTRA = 0.05, 3


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


def rows_f64(t, rows):
    """Listed rows of a device tensor as float64 host rows (only those rows move)."""
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=t.device)
    return t.index_select(0, idx).to("cpu", torch.float64).numpy()


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


def np_keys(logits, scoring, bias):
    """Selection keys in float64 from float32 logits: affinity + bias."""
    l = np.asarray(logits, np.float64)
    if scoring == O.SIGMOID:
        s = 1 / (1 + np.exp(-l))
    elif scoring == O.SQRTSOFTPLUS:
        s = np.sqrt(np.logaddexp(0, l))
    else:
        s = l
    return s + (0 if bias is None else np.asarray(bias, np.float64))


def valid_alternative(keys, ids, ref_ids, k, n_group=1, topk_group=1, group_topk=0,
                      tol=TIE_VALID):
    """Whether `ids` (one token's k experts, in slot order) is a choice the routing
    rule could make if near-tied decisions (within `tol`) went either way.

    Without groups: the selected keys equal the oracle's selected keys up to
    `tol`, in non-increasing order up to `tol`.  With groups: some set of
    topk_group groups, each scoring within `tol` of the kept groups' cut and
    holding every group that scores clearly above it, contains the selection,
    and the selection's keys are the top k keys of those groups up to `tol`."""
    ids = np.asarray(ids)
    E = len(keys)
    if len(set(ids.tolist())) != k or ids.min() < 0 or ids.max() >= E:
        return False
    sel = keys[ids]
    if np.any(np.diff(sel) > tol):  # slot order: descending keys
        return False
    want = np.sort(sel)[::-1]
    if n_group <= 1:
        return bool(np.all(np.abs(want - np.sort(keys[ref_ids])[::-1]) <= tol))
    G = E // n_group
    kg = keys.reshape(n_group, G)
    gscore = np.sort(kg, axis=1)[:, ::-1][:, :group_topk].sum(1)
    cut = np.sort(gscore)[::-1][topk_group - 1]
    near = [g for g in range(n_group) if gscore[g] >= cut - tol]
    must = {g for g in range(n_group) if gscore[g] > cut + tol}
    used = set((ids // G).tolist())
    for combo in itertools.combinations(near, topk_group):
        cs = set(combo)
        if not (used <= cs and must <= cs):
            continue
        cand = np.concatenate([kg[g] for g in combo])
        top = np.sort(cand)[::-1][:k]
        if np.all(np.abs(want - top) <= tol):
            return True
    return False


def check_routing(ids, gates, ref_ids, ref_gates, margin, keys=None, tie=TIE_GIVEN, grp=None):
    """Routing from identical logits: ids bit-exact except near-ties (margin <=
    `tie`), gates within GATE_TOL_GIVEN; a near-tie token must pick a valid
    alternative (keys within 4 * tie of a choice the rule could make)."""
    ok = margin > tie
    assert np.array_equal(ids[ok], ref_ids[ok])
    assert np.abs(gates[ok] - ref_gates[ok]).max(initial=0) <= GATE_TOL_GIVEN
    if keys is not None:
        grp = grp or {}
        k = ids.shape[1]
        for t in np.nonzero(~ok)[0]:
            assert valid_alternative(keys[t], ids[t], ref_ids[t], k, tol=4 * tie, **grp), t
    return int((~ok).sum())


# ----------------------------------------------------------------------------
# the oracle's layer, expert by expert
# ----------------------------------------------------------------------------
class HostInputs:
    """Host copies of the small inputs (expert weights are fetched per expert)."""

    def __init__(self, inp):
        self.inp = inp
        self.h = to_host_bits(inp["hidden"])
        self.wr = to_host_bits(inp["w_router"])
        self.bias = to_host_bits(inp.get("bias"))
        self.off = to_host_bits(inp.get("logit_offset"))
        self.tok = to_host_bits(inp.get("token_ids"))
        self.tab = to_host_bits(inp.get("tid2eid"))


def expert_weights(inp, e, fmt):
    """Oracle-side weights of expert e (or e = "shared"): the bf16 / fp32 masters,
    or the oracle's own FP8 (128x128 tiles) or MXFP4 (1x32 blocks) quantization of
    them.  Only this expert is copied to the host."""
    if e == "shared":
        w13, w2 = inp["w13_shared"], inp["w2_shared"]
    else:
        w13, w2 = inp["w13"][e], inp["w2"][e]
    b13, b2 = to_host_bits(w13), to_host_bits(w2)
    if fmt == "fp8":
        return O.quantize_blocks(b13) + O.quantize_blocks(b2)
    if fmt == "mxfp4":
        return O.quantize_mxfp4(b13) + O.quantize_mxfp4(b2)
    return b13, b2


def expert_eval(h, tokens, wts, fmt):
    if fmt in ("fp8", "mxfp4"):
        return O.expert_rows_lowp(fmt, h, tokens, *wts)
    return O.expert_rows(h, tokens, *wts)


def oracle_outputs(lc, inp, hi, rows, ids, gates, fmt):
    """y_t = sum_j g[t,j] FFN_{ids[t,j]}(x_t) (+ the shared expert) for the listed
    token rows, from the given routing: every (token, slot) pair's expert output
    from the oracle, expert by expert, then the oracle's combine in slot order
    and the shared expert's rows with weight 1."""
    rows = np.asarray(rows, np.int32)
    n, k = ids.shape
    eo = np.zeros((n * k, lc.d), np.float64)
    flat = ids.ravel()
    for e in np.unique(flat):
        sel = np.nonzero(flat == e)[0]
        eo[sel] = expert_eval(hi.h, rows[sel // k], expert_weights(inp, int(e), fmt), fmt)
    out = O.combine(eo, np.repeat(np.arange(n, dtype=np.int32), k),
                    np.asarray(gates, np.float32).ravel(), n)
    del eo
    if lc.n_shared:
        ys = expert_eval(hi.h, rows, expert_weights(inp, "shared", fmt), fmt)
        out = O.combine(ys, np.arange(n, dtype=np.int32), np.ones(n, np.float32), n, out=out)
    return out


def max_ties(n):
    return MAX_TIE_EXTRA + MAX_TIE_FRAC * n


def check_layer(lc, inp, gpu_out, gpu_ids, gpu_gates, rows, route_mode=O.LEARNED, fmt=None,
                tol=None, median_tol=None):
    """Compare the GPU layer's outputs, ids and gates with the oracle on the
    listed token rows; returns a dict of summary numbers.

    The oracle routes each row from its own logits (float64 sums rounded to
    float32).  Ids must match bit for bit except near-ties, whose GPU ids must
    be a valid alternative; their rows are then checked against the oracle
    routed on the GPU's ids (gates from the oracle's affinities at those ids).
    Every listed row's output is compared."""
    fmt = fmt or lc.dtype
    tol = out_tol(lc.dtype) if tol is None else tol
    rows = np.asarray(rows, np.int32)
    n, k = len(rows), lc.k
    hi = HostInputs(inp)
    grp = dict(n_group=lc.n_group, topk_group=lc.topk_group, group_topk=lc.group_topk)
    lg = O.logits(hi.h, hi.wr, rows=rows, logit_offset=hi.off).astype(np.float32)
    g_ids = gpu_ids.cpu().numpy()[rows]
    g_gates = gpu_gates.cpu().numpy()[rows]
    if route_mode == O.HASH:
        ids, gates = O.hash_route(lg, hi.tok[rows], hi.tab, lc.scoring)
        tie = np.zeros(n, bool)
    else:
        ids, gates, margin = O.route(lg, k, lc.scoring, bias=hi.bias, **grp)
        tie = margin <= TIE_LAYER
    n_tie = int(tie.sum())
    assert n_tie <= max_ties(n), "too many near-ties: %d of %d" % (n_tie, n)
    ok = ~tie
    assert np.array_equal(g_ids[ok], ids[ok]), "topk_ids differ on non-tie tokens"
    assert np.abs(g_gates[ok] - gates[ok]).max(initial=0) <= GATE_TOL_LAYER
    if n_tie:
        keys = np_keys(lg[tie], lc.scoring, hi.bias)
        for q, (kt, gi, ri) in enumerate(zip(keys, g_ids[tie], ids[tie])):
            assert valid_alternative(kt, gi, ri, k, **grp), \
                "near-tie token %d: GPU ids %s are not a valid choice" % (rows[tie][q], gi)
        # the oracle's gates for the GPU's choice: the token's affinities at
        # those ids, renormalised (the rule the hash route applies to given ids)
        _, tie_gates = O.hash_route(lg[tie], np.arange(n_tie, dtype=np.int32),
                                    g_ids[tie].astype(np.int32), lc.scoring)
        assert np.abs(g_gates[tie] - tie_gates).max() <= GATE_TOL_LAYER
        ids = ids.copy()
        gates = gates.copy()
        ids[tie] = g_ids[tie]
        gates[tie] = tie_gates
    ref = oracle_outputs(lc, inp, hi, rows, ids, gates, fmt)
    g_out = rows_f64(gpu_out, rows)
    err = row_rel_err(g_out, ref)
    assert err.max(initial=0) <= tol, "max row rel err %.3g > %.3g (row %d)" % (
        err.max(), tol, rows[int(np.argmax(err))])
    if median_tol is not None:
        assert np.median(err) <= median_tol, np.median(err)
    fro = np.linalg.norm(g_out - ref) / max(np.linalg.norm(ref), 1e-30)
    return dict(max_row_rel_err=float(err.max(initial=0)), fro_rel_err=float(fro),
                ties=n_tie, rows=n, err=err)


# ----------------------------------------------------------------------------
# row choice at full size
# ----------------------------------------------------------------------------
FRAG = 32  # rows of an MFMA fragment; every expert tile is a whole number of them


def dispatch_of(gpu_ids, E):
    """Expert-major dispatch order of a routing (the oracle's permutation)."""
    ids = np.asarray(gpu_ids, np.int32)
    return O.permute(ids, np.zeros(ids.shape, np.float32), E)


def stratified_rows(gpu_ids, E, T, n_shared, seed, experts=None):
    """Token rows such that every 32-row fragment of every expert's dispatch rows
    (and of the shared expert's T rows) holds one of them: one random row per
    fragment, plus each group's last row (its ragged tail).  Expert tiles start
    at the group's first row and are whole fragments, so every (expert, row
    tile) of both grouped GEMMs is covered, whatever the tile height.
    `experts` restricts the routed experts covered."""
    perm = dispatch_of(gpu_ids, E)
    off, tok = perm["offsets"], perm["sorted_token_ids"]
    rng = np.random.default_rng(seed)
    pick = []
    for e in (range(E) if experts is None else experts):
        a, b = int(off[e]), int(off[e + 1])
        for f0 in range(a, b, FRAG):
            pick.append(tok[rng.integers(f0, min(b, f0 + FRAG))])
        if b > a:
            pick.append(tok[b - 1])
    if n_shared:
        for f0 in range(0, T, FRAG):
            pick.append(rng.integers(f0, min(T, f0 + FRAG)))
        pick.append(T - 1)
    return np.unique(np.asarray(pick, np.int64)).astype(np.int32)


def expert_sample(counts, seed, n_random=12, n_hot=6, n_cold=6):
    """A spread of experts with rows: the hottest, the smallest non-empty (on a
    skewed load the streaming-tile ones) and a seeded random set of the rest."""
    counts = np.asarray(counts)
    active = np.nonzero(counts > 0)[0]
    order = active[np.argsort(counts[active], kind="stable")]
    pick = set(order[::-1][:n_hot].tolist()) | set(order[:n_cold].tolist())
    rest = np.setdiff1d(active, np.fromiter(pick, int, len(pick)))
    rng = np.random.default_rng(seed)
    pick |= set(rng.choice(rest, min(n_random, len(rest)), replace=False).tolist())
    return sorted(pick)


def hot_cold_rows(ids, counts, n=2):
    """Token rows routed to the expert with the most rows and to the expert with
    the fewest (but some) rows: on a skewed workload the first runs on the
    288-row tiles, the second on the small-group streaming tiles."""
    hot = int(np.argmax(counts))
    cold = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    return np.r_[np.nonzero((ids == hot).any(1))[0][:n], np.nonzero((ids == cold).any(1))[0][:n]]


# ----------------------------------------------------------------------------
# low-precision experts at full size
# ----------------------------------------------------------------------------
def check_lowp_stages(lc, inp, fmt, wq, ids, gates, tol, median_tol, seed):
    """The FP8 / MXFP4 expert stages (moe_expert_up_* then moe_expert_down_*) on
    the layer's own routing at full size, against the oracle's low-precision
    expert (which quantizes the bf16 masters and the hidden rows itself): one
    dispatch row in every 32-row fragment of a spread of experts (the hottest,
    the smallest and a random set), i.e. every (expert, row tile) of both
    GEMMs for those experts.  Returns the per-row errors."""
    c = cfg_of(lc)
    T, k, E, d, F = lc.T, lc.k, lc.E, lc.d, lc.d_ff
    dev = "cuda"
    ws = torch.empty(moe.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    perm = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                tok=torch.empty(T * k, dtype=torch.int32, device=dev),
                w=torch.empty(T * k, dtype=torch.float32, device=dev),
                disp=torch.empty((T, k), dtype=torch.int32, device=dev))
    moe.moe_permute(c, ids, gates, perm["counts"], perm["offsets"], perm["tok"], perm["w"],
                    perm["disp"], ws)
    xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
    xs = torch.empty((d // 128, T), dtype=torch.float32, device=dev)
    moe.moe_quantize_fp8_rows(inp["hidden"], xq, xs)
    hq = torch.empty((T * k, F), dtype=torch.uint8, device=dev)
    hs = torch.empty((F // 128, T * k), dtype=torch.float32, device=dev)
    y = torch.empty((T * k, d), dtype=torch.bfloat16, device=dev)
    up = moe.moe_expert_up_fp8 if fmt == "fp8" else moe.moe_expert_up_mxfp4
    down = moe.moe_expert_down_fp8 if fmt == "fp8" else moe.moe_expert_down_mxfp4
    up(c, xq, xs, perm["tok"], perm["offsets"], wq["w13q"], wq["w13s"], hq, hs, ws)
    down(c, hq, hs, perm["offsets"], wq["w2q"], wq["w2s"], y, ws)
    torch.cuda.synchronize()
    counts = perm["counts"].cpu().numpy()
    off = perm["offsets"].cpu().numpy()
    tok = perm["tok"].cpu().numpy()
    h = to_host_bits(inp["hidden"])
    rng = np.random.default_rng(seed)
    errs = []
    for e in expert_sample(counts, seed):
        a, b = int(off[e]), int(off[e + 1])
        rws = np.unique([rng.integers(f0, min(b, f0 + FRAG)) for f0 in range(a, b, FRAG)] +
                        [b - 1])
        ref = expert_eval(h, tok[rws], expert_weights(inp, e, fmt), fmt)
        errs.append(row_rel_err(rows_f64(y, rws), ref))
    err = np.concatenate(errs)
    assert err.max() <= tol, err.max()
    assert np.median(err) <= median_tol, np.median(err)
    return err


def check_quantized_tiles(inp, wq, fmt, seed):
    """Every expert's quantized weights (and the shared expert's) at full size:
    one random 128 x 128 region of w13 and of w2 per expert, codes and scales
    bit-exact against the oracle's quantizer on the same bf16 region (catches a
    quantizer launch that leaves later experts untouched)."""
    rng = np.random.default_rng(seed)
    for name in ("w13", "w2", "w13_shared", "w2_shared"):
        w = inp.get(name)
        if w is None:
            continue
        base = name.replace("_shared", "")
        sfx = "_shared" if name.endswith("_shared") else ""
        q, s = wq[base + "q" + sfx], wq[base + "s" + sfx]
        if w.dim() == 2:
            w, q, s = w.unsqueeze(0), q.unsqueeze(0), s.unsqueeze(0)
        n, R, C_ = w.shape
        for e in range(n):
            r0, c0 = 128 * int(rng.integers(R // 128)), 128 * int(rng.integers(C_ // 128))
            region = to_host_bits(w[e, r0:r0 + 128, c0:c0 + 128])
            if fmt == "fp8":
                rq, rs = O.quantize_blocks(region)
                gq = q[e, r0:r0 + 128, c0:c0 + 128].cpu().numpy()
                gs = s[e, r0 // 128, c0 // 128].reshape(1, 1).cpu().numpy()
            else:
                rq, rs = O.quantize_mxfp4(region)  # [128, 64] codes, [128, 4] E8M0
                gq = mxfp4_rows(q[e, r0 // 2:r0 // 2 + 64, c0:c0 + 128].cpu().numpy())
                gs = s[e, c0 // 128, r0:r0 + 128, :].cpu().numpy()
            assert np.array_equal(gs, rs), (name, e, r0, c0)
            assert np.array_equal(gq, rq), (name, e, r0, c0)


def mxfp4_rows(q):
    """E2M1 codes in the library's paired-row layout, [..., R/2, C] bytes (row
    pair i, 128-column block j: 64 bytes of row 2i, then 64 of row 2i+1) ->
    the row-major [..., R, C/2] that the oracle's quantizer returns."""
    q = np.asarray(q)
    *lead, P, C_ = q.shape
    t = q.reshape(*lead, P, C_ // 128, 2, 64)
    return np.ascontiguousarray(np.moveaxis(t, -2, -3)).reshape(*lead, 2 * P, C_ // 2)


def dequantized(fmt, q, s):
    """A weight matrix as the oracle's quantizer left it, in float64: E4M3 codes
    times their 128x128 tile scales ("fp8"), or E2M1 codes times their 1x32
    block scales ("mxfp4")."""
    if fmt == "mxfp4":
        return np.asarray(O.mxfp4_dequantize(q, s), np.float64)
    w = O.e4m3_decode(q).astype(np.float64)
    return w * np.kron(np.asarray(s, np.float64), np.ones((128, 128)))
