"""GPU parity: every entry point of the C ABI against the oracle, on the same
seeded inputs.  Small cases span several tiles and ragged tails; the full-size
cases run the workloads' real shapes through moe_forward and compare sampled
token rows.  Tolerances are in parity_helpers."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import mixture_experts_ffn_sqrt_amd as moe
import oracle as O
from mixture_experts_ffn_sqrt_amd.synth import CONFIGS, make_inputs, random_logits, to_host_bits

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity_helpers as H  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()  # raises if the HIP library is not built
    yield
    torch.cuda.synchronize()


def dev(x, dtype=None):
    t = torch.as_tensor(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


# ----------------------------------------------------------------------------
# routing from identical logits
# ----------------------------------------------------------------------------
def gpu_route_given(logits, k, scoring, bias=None, n_group=1, topk_group=1, group_topk=0):
    T, E = logits.shape
    c = moe.make_config(T=T, d=64, E=E, k=k, d_ff=64, scoring=scoring, n_group=n_group,
                        topk_group=topk_group, group_topk=group_topk, logits_given=1)
    lg = dev(logits, torch.float32)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(c, None, None, None, None if bias is None else dev(bias), None, None, lg, ids,
                  gates)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gates.cpu().numpy()


def test_router_worked_example(golden):
    g = golden("router_worked_example.json")
    ids, gates = gpu_route_given(np.array([g["scores"]], np.float32), g["k"], O.SOFTMAX)
    assert ids[0].tolist() == g["expected_ids"]
    assert np.all(np.abs(gates[0] - g["expected_weights_printed"]) <= 0.005)
    _, ref, _ = O.route(np.array([g["scores"]], np.float32), g["k"], O.SOFTMAX)
    assert np.abs(gates - ref).max() <= H.GATE_TOL


ROUTE_CASES = [
    dict(T=1, E=8, k=2, scoring=O.SOFTMAX),
    dict(T=7, E=8, k=2, scoring=O.SOFTMAX),
    dict(T=1000, E=64, k=6, scoring=O.SOFTMAX),
    dict(T=513, E=256, k=8, scoring=O.SIGMOID, bias=True, n_group=8, topk_group=4, group_topk=2),
    dict(T=300, E=256, k=6, scoring=O.SQRTSOFTPLUS, bias=True),
    dict(T=300, E=384, k=6, scoring=O.SQRTSOFTPLUS, bias=True),
    dict(T=200, E=1024, k=16, scoring=O.SIGMOID, bias=True),
    dict(T=200, E=1024, k=16, scoring=O.SQRTSOFTPLUS, bias=True, n_group=64, topk_group=3,
         group_topk=3),
    dict(T=64, E=3, k=3, scoring=O.SOFTMAX),
    dict(T=64, E=257, k=1, scoring=O.SIGMOID),
    dict(T=100, E=16, k=4, scoring=O.SOFTMAX, quantised=True),  # many exact ties
    # group sizes: 64 and 1 (lane segments), 24 and 96 (the serial group scan),
    # and exact ties inside groups
    dict(T=300, E=256, k=8, scoring=O.SIGMOID, bias=True, n_group=4, topk_group=2, group_topk=3),
    dict(T=100, E=16, k=4, scoring=O.SIGMOID, bias=True, n_group=16, topk_group=6, group_topk=1),
    dict(T=300, E=96, k=6, scoring=O.SIGMOID, bias=True, n_group=4, topk_group=2, group_topk=2),
    dict(T=300, E=384, k=6, scoring=O.SQRTSOFTPLUS, bias=True, n_group=4, topk_group=3,
         group_topk=4),
    dict(T=200, E=64, k=6, scoring=O.SIGMOID, n_group=8, topk_group=3, group_topk=2,
         quantised=True),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: "T%(T)d-E%(E)d-k%(k)d-s%(scoring)d" % c)
def test_route_from_given_logits(case):
    rng = np.random.default_rng(case["T"] * 31 + case["E"])
    T, E, k = case["T"], case["E"], case["k"]
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if case.get("quantised"):
        lg = np.round(lg * 2) / 2  # exact ties: lower expert id must win on both sides
    bias = (0.01 * rng.standard_normal(E)).astype(np.float32) if case.get("bias") else None
    grp = {kk: case[kk] for kk in ("n_group", "topk_group", "group_topk") if kk in case}
    ids, gates = gpu_route_given(lg, k, case["scoring"], bias, **grp)
    rid, rg, margin = O.route(lg, k, case["scoring"], bias=bias, **grp)
    if case.get("quantised"):
        # keys are exactly representable: no near-tie excuse, ids must agree everywhere
        assert np.array_equal(ids, rid)
        assert np.abs(gates - rg).max() <= H.GATE_TOL
        return
    H.check_routing(ids, gates, rid, rg, margin, keys=H.np_keys(lg, case["scoring"], bias),
                    grp=grp)
    if grp:
        G = E // grp["n_group"]
        assert max(len(np.unique(r // G)) for r in ids) <= grp["topk_group"]


@pytest.mark.parametrize("scoring", [O.SOFTMAX, O.SIGMOID])
def test_group_limited_routing_worked_example(golden, scoring):
    """The hand-built node-limited routing example of [P3] 五.3 (1 + 3 + 2 + 2
    experts over the 4 kept groups), from given logits (see the oracle pin)."""
    g = golden("group_limited_routing_example.json")
    keys = np.array([g["keys"]], np.float32)
    grp = dict(n_group=g["n_group"], topk_group=g["topk_group"], group_topk=g["group_topk"])
    if scoring == O.SOFTMAX:
        ids, _ = gpu_route_given(keys, g["k"], scoring, **grp)
    else:
        ids, gates = gpu_route_given(np.full_like(keys, -200.0), g["k"], scoring, bias=keys[0],
                                     **grp)
        assert np.all(gates == np.float32(1.0 / g["k"]))
    assert ids[0].tolist() == g["expected_ids"]


def test_zero_denominator_gates():
    lg = np.full((3, 8), -200.0, np.float32)
    ids, gates = gpu_route_given(lg, 2, O.SQRTSOFTPLUS)
    assert ids.tolist() == [[0, 1]] * 3
    assert np.all(gates == 0.5)


def test_hash_route():
    rng = np.random.default_rng(5)
    V, E, k, T = 1000, 256, 6, 64
    tab = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    tok = rng.integers(0, V, T).astype(np.int32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    c = moe.make_config(T=T, d=64, E=E, k=k, d_ff=64, scoring=O.SQRTSOFTPLUS, route_mode=1,
                        vocab=V, logits_given=1)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(c, None, None, None, None, dev(tok), dev(tab), dev(lg), ids, gates)
    rid, rg = O.hash_route(lg, tok, tab, O.SQRTSOFTPLUS)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(gates.cpu().numpy() - rg).max() <= H.GATE_TOL


@pytest.mark.parametrize("dtype, T, d, E", [("f32", 16, 64, 8), ("f32", 70, 128, 40),
                                           ("bf16", 200, 512, 64), ("bf16", 64, 7168, 384)])
def test_router_gemm_logits(dtype, T, d, E):
    lc = CONFIGS["tiny_fp32"].with_(T=T, d=d, E=E, d_ff=64, dtype=dtype, seed=17)
    inp = make_inputs(lc, "cuda")
    off = torch.linspace(-1, 1, E, device="cuda", dtype=torch.float32)
    c = H.cfg_of(lc)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, lc.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, lc.k), dtype=torch.float32, device="cuda")
    moe.moe_route(c, inp["hidden"], inp["w_router"], off, None, None, None, logits, ids, gates)
    torch.cuda.synchronize()
    h, wr = to_host_bits(inp["hidden"]), to_host_bits(inp["w_router"])
    ref = O.logits(h, wr, logit_offset=off.cpu().numpy())
    # float32 accumulation bound: d * 2^-24 * sum |x_i w_i|
    habs = np.abs(inp["hidden"].double().cpu().numpy())
    wabs = np.abs(inp["w_router"].double().cpu().numpy())
    bound = d * 2.0 ** -24 * (habs @ wabs.T) + 1e-6
    assert np.all(np.abs(logits.double().cpu().numpy() - ref) <= bound)


# ----------------------------------------------------------------------------
# permutation
# ----------------------------------------------------------------------------
def gpu_permute(ids, gates, E):
    T, k = ids.shape
    c = moe.make_config(T=T, d=64, E=E, k=k, d_ff=64)
    ws = torch.empty(moe.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    out = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
               offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               sorted_token_ids=torch.empty(T * k, dtype=torch.int32, device="cuda"),
               sorted_weights=torch.empty(T * k, dtype=torch.float32, device="cuda"),
               dispatch_index=torch.empty((T, k), dtype=torch.int32, device="cuda"))
    moe.moe_permute(c, dev(ids, torch.int32), dev(gates, torch.float32), out["counts"],
                    out["offsets"], out["sorted_token_ids"], out["sorted_weights"],
                    out["dispatch_index"], ws)
    torch.cuda.synchronize()
    return {kk: v.cpu().numpy() for kk, v in out.items()}


def assert_permute_equal(g, ref):
    for kk in ("counts", "offsets", "sorted_token_ids", "sorted_weights", "dispatch_index"):
        assert np.array_equal(g[kk], ref[kk]), kk


@pytest.mark.parametrize("name", ["two_token_toy.json", "dispatch_combine_toy.json",
                                  "ep4_counts.json"])
def test_permute_worked_examples(golden, name):
    g = golden(name)
    ids = np.array(g["ids"], np.int32)
    w = np.array(g.get("weights", np.ones(ids.shape)), np.float32)
    got = gpu_permute(ids, w, g["E"])
    assert_permute_equal(got, O.permute(ids, w, g["E"]))
    if "expected_permuted_token_ids" in g:
        assert got["sorted_token_ids"].tolist() == g["expected_permuted_token_ids"]


@pytest.mark.parametrize("T, k, E, mode", [
    (1, 1, 1, "uniform"), (3, 2, 8, "uniform"), (1000, 8, 256, "uniform"),
    (4097, 6, 384, "zipf"), (9000, 2, 8, "uniform"), (5000, 6, 1024, "uniform"),
    (3000, 4, 64, "one_hot"), (16384, 6, 384, "zipf")])
def test_permute_random(T, k, E, mode):
    rng = np.random.default_rng(T + k + E)
    if mode == "uniform":
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    elif mode == "one_hot":  # every token picks expert 5 first: one huge group, many empty
        rest = np.array([e for e in range(E) if e != 5])
        ids = np.stack([np.r_[5, rng.choice(rest[:k + 2], k - 1, replace=False)]
                        for _ in range(T)])
    else:
        w = 1.0 / np.arange(1, E + 1) ** 1.1
        ids = np.stack([rng.choice(E, k, replace=False, p=w / w.sum()) for _ in range(T)])
    ids = ids.astype(np.int32)
    assert all(len(set(r)) == k for r in ids)
    gates = rng.random((T, k)).astype(np.float32)
    assert_permute_equal(gpu_permute(ids, gates, E), O.permute(ids, gates, E))


# ----------------------------------------------------------------------------
# grouped experts and combine (staged API)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype, T, d, E, k, d_ff", [
    ("f32", 16, 64, 8, 2, 128),
    ("f32", 50, 128, 5, 3, 192),
    ("bf16", 300, 256, 5, 2, 192),     # ~120 rows/expert, d_ff not a multiple of 128: 128-row tiles
    ("bf16", 40, 256, 64, 6, 128),     # ~4 rows/expert: 32-row streaming tiles
    ("bf16", 200, 256, 16, 2, 256),    # ~25 rows/expert: 32-row tiles, some experts span two
    ("bf16", 40, 256, 64, 6, 192),     # ~4 rows/expert, d_ff not a multiple of 128: 16-row tiles
    ("bf16", 1, 512, 16, 4, 256),      # single token
    ("bf16", 700, 128, 3, 3, 64),      # k = E: every expert gets every token
    ("bf16", 700, 320, 4, 2, 256),     # prefill (288x256) tiles: ragged rows, partial last column tile
    ("bf16", 2000, 512, 8, 2, 384),    # prefill tiles, several row tiles per expert
    ("bf16", 2100, 320, 4, 2, 256),    # ~1050 rows per expert: 4 row tiles each, partial column
    ("bf16", 1300, 256, 2, 1, 128),    # ~650 rows per expert: 3 row tiles each, ragged last tile
    ("bf16", 600, 64, 4, 2, 128),      # prefill tiles with K shorter than the LDS ring:
                                       # one K stage up, two down, partial column tile
    ("bf16", 900, 128, 3, 2, 128),     # two K stages up
])
def test_expert_ffn_and_combine(dtype, T, d, E, k, d_ff):
    lc = CONFIGS["tiny_fp32"].with_(T=T, d=d, E=E, k=k, d_ff=d_ff, dtype=dtype, seed=23)
    inp = make_inputs(lc, "cuda")
    rng = np.random.default_rng(T)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    perm = O.permute(ids, gates, E)
    c = H.cfg_of(lc)
    ws = torch.empty(moe.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    eo = torch.empty((T * k, d), dtype=lc.torch_dtype, device="cuda")
    moe.moe_expert_ffn(c, inp["hidden"], dev(perm["sorted_token_ids"]), dev(perm["offsets"]),
                       inp["w13"], inp["w2"], eo, ws)
    out = torch.empty((T, d), dtype=lc.torch_dtype, device="cuda")
    moe.moe_combine(c, eo, dev(perm["dispatch_index"]), dev(gates), None, out)
    torch.cuda.synchronize()
    h = to_host_bits(inp["hidden"])
    w13, w2 = to_host_bits(inp["w13"]), to_host_bits(inp["w2"])
    x = h.astype(np.float64) if dtype == "f32" else inp["hidden"].double().cpu().numpy()
    expert_of_row = np.repeat(np.arange(E), perm["counts"])
    ref_eo = np.stack([O.expert_ffn(x[t], w13[e], w2[e])
                       for t, e in zip(perm["sorted_token_ids"], expert_of_row)])
    err = H.row_rel_err(H.to_f64(eo), ref_eo)
    assert err.max() <= H.out_tol(dtype), err.max()
    ref_out = O.combine(ref_eo, perm["sorted_token_ids"], perm["sorted_weights"], T)
    err = H.row_rel_err(H.to_f64(out), ref_out)
    assert err.max() <= H.out_tol(dtype), err.max()


@pytest.mark.parametrize("d, d_ff", [(256, 256), (320, 128)])
def test_expert_ffn_mixed_group_sizes(d, d_ff):
    """A prefill-shaped batch (195 rows per expert on average) whose routing
    leaves some experts a few rows: groups of 0, 1, 31 and 32 rows take one
    32-row streaming tile each, groups of 33 rows and more take 288-row tiles
    (the boundary on both sides, and ragged tails)."""
    sizes = [0, 1, 31, 32, 33, 64, 300, 1100]
    E, k, T = len(sizes), 1, sum(sizes)
    lc = CONFIGS["tiny_fp32"].with_(T=T, d=d, E=E, k=k, d_ff=d_ff, dtype="bf16", seed=31)
    inp = make_inputs(lc, "cuda")
    rng = np.random.default_rng(31)
    ids = rng.permutation(np.repeat(np.arange(E), sizes)).astype(np.int32)[:, None]
    gates = np.ones((T, k), np.float32)
    perm = O.permute(ids, gates, E)
    assert list(perm["counts"]) == sizes
    c = H.cfg_of(lc)
    ws = torch.empty(moe.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    eo = torch.empty((T * k, d), dtype=lc.torch_dtype, device="cuda")
    moe.moe_expert_ffn(c, inp["hidden"], dev(perm["sorted_token_ids"]), dev(perm["offsets"]),
                       inp["w13"], inp["w2"], eo, ws)
    torch.cuda.synchronize()
    w13, w2 = to_host_bits(inp["w13"]), to_host_bits(inp["w2"])
    x = inp["hidden"].double().cpu().numpy()
    expert_of_row = np.repeat(np.arange(E), perm["counts"])
    ref_eo = np.stack([O.expert_ffn(x[t], w13[e], w2[e])
                       for t, e in zip(perm["sorted_token_ids"], expert_of_row)])
    err = H.row_rel_err(H.to_f64(eo), ref_eo)
    assert err.max() <= H.out_tol("bf16"), err.max()


def test_combine_worked_example(golden):
    g = golden("dispatch_combine_toy.json")
    ids = np.array(g["ids"], np.int32)
    w = np.array(g["weights"], np.float32)
    perm = O.permute(ids, w, g["E"])
    expert_of_row = np.repeat(np.arange(g["E"]), perm["counts"])
    d = 64
    # expert output of a dispatch row: the constant 10*expert + token
    eo = np.array([[10.0 * e + t] * d for e, t in zip(expert_of_row, perm["sorted_token_ids"])],
                  np.float32)
    c = moe.make_config(T=4, d=d, E=g["E"], k=2, d_ff=64, dtype="f32")
    shared = np.full((4, d), 0.5, np.float32)
    out = torch.empty((4, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(c, dev(eo), dev(perm["dispatch_index"]), dev(w), dev(shared), out)
    got = out.cpu().numpy()
    for t, terms in g["expected_combine"].items():
        want = sum(wt * (10.0 * e + int(t)) for e, wt in terms) + 0.5
        assert np.allclose(got[int(t)], want, rtol=1e-6)


# ----------------------------------------------------------------------------
# the whole layer (moe_forward)
# ----------------------------------------------------------------------------
SMALL_LAYERS = {
    "tiny_fp32": CONFIGS["tiny_fp32"],
    "mixtral_small": CONFIGS["mixtral_prefill"].with_(T=512, d=512, d_ff=1024),
    "dsv3_small": CONFIGS["dsv3_prefill"].with_(T=384, d=256, d_ff=128),
    "v4flash_small": CONFIGS["v4flash_decode"].with_(d=512, d_ff=256),
    "v4pro_skew_small": CONFIGS["v4pro_skew_prefill"].with_(T=600, d=256, E=96, d_ff=192),
    "tiny_fp32_shared_sig": CONFIGS["tiny_fp32"].with_(T=33, n_shared=1, scoring=O.SIGMOID,
                                                       bias_std=0.01, E=16, k=3),
    "grouped_square_tiles": CONFIGS["dsv3_prefill"].with_(T=1024, d=256, E=16, k=4, d_ff=128,
                                                          n_group=4, topk_group=2, group_topk=2),
    "v4pro_skew_square_tiles": CONFIGS["v4pro_skew_prefill"].with_(T=2048, d=256, E=16, k=4,
                                                                   d_ff=256),
    "single_dense_expert": CONFIGS["mixtral_prefill"].with_(T=130, d=256, E=1, k=1, d_ff=128),
    "decode_T1": CONFIGS["v4flash_decode"].with_(T=1, d=256, d_ff=128),
    # 512 rows per expert: the down GEMM runs 288-row tiles
    "mixtral_tall_tiles": CONFIGS["mixtral_prefill"].with_(T=2048, d=256, d_ff=256),
    # 128 rows per expert on average with a skewed load: the experts with at
    # most 32 rows run on streaming tiles, the others on 288-row tiles
    "v4pro_skew_split": CONFIGS["v4pro_skew_prefill"].with_(T=1024, d=256, E=32, k=4, d_ff=128),
    # about 70 experts of at most 32 rows x 8 column tiles: the up GEMM's
    # streaming launch (64 persistent blocks beside the 288-row tiles) walks
    # several tiles per block
    "v4pro_skew_many_small": CONFIGS["v4pro_skew_prefill"].with_(T=4096, d=256, E=128, k=6,
                                                                 d_ff=1024),
}


@pytest.mark.parametrize("name", list(SMALL_LAYERS))
def test_forward_small(name):
    lc = SMALL_LAYERS[name]
    inp = make_inputs(lc, "cuda")
    out, ids, gates = H.gpu_forward(H.cfg_of(lc), inp)
    H.check_layer(lc, inp, out, ids, gates, rows=np.arange(lc.T))
    again, _, _ = H.gpu_forward(H.cfg_of(lc), inp)
    assert torch.equal(out, again), "moe_forward is not deterministic"


def test_forward_hash_pass_small():
    lc = CONFIGS["v4flash_decode"].with_(d=256, d_ff=128, hash_vocab=5000)
    inp = make_inputs(lc, "cuda", hash_pass=True)
    out, ids, gates = H.gpu_forward(H.cfg_of(lc, route_mode=1), inp)
    assert np.array_equal(ids.cpu().numpy(),
                          inp["tid2eid"].cpu().numpy()[inp["token_ids"].cpu().numpy()])
    H.check_layer(lc, inp, out, ids, gates, rows=np.arange(lc.T), route_mode=O.HASH)


def test_forward_all_tokens_to_one_expert():
    """A logit offset that sends every token to expert 0 first: one group holds all
    T rows, most experts hold none."""
    lc = CONFIGS["v4pro_skew_prefill"].with_(T=300, d=256, E=32, k=2, d_ff=128, zipf_s=0.0)
    inp = make_inputs(lc, "cuda")
    off = torch.zeros(lc.E, dtype=torch.float32, device="cuda")
    off[0] = 50.0
    inp["logit_offset"] = off
    out, ids, gates = H.gpu_forward(H.cfg_of(lc), inp)
    assert (ids[:, 0] == 0).all()
    H.check_layer(lc, inp, out, ids, gates, rows=np.arange(lc.T))


FULL = ["tiny_fp32", "mixtral_prefill", "dsv3_prefill", "v4flash_decode", "v4pro_skew_prefill"]


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size_stratified(name):
    """The workload at its full size, in the launch configuration the bench
    times.  The oracle recomputes, from its own routing, one token row in every
    32-row fragment of every expert's dispatch rows (and of the shared expert's):
    every (expert, row tile) of both grouped GEMMs and every combine path is
    compared, near-tie tokens included."""
    lc = CONFIGS[name]
    inp = make_inputs(lc, "cuda")
    out, ids, gates = H.gpu_forward(H.cfg_of(lc), inp)
    T = lc.T
    ids_np = ids.cpu().numpy()
    # properties at any size
    assert ((ids_np >= 0) & (ids_np < lc.E)).all()
    assert all(len(set(r)) == lc.k for r in ids_np)
    g = gates.cpu().numpy()
    assert np.allclose(g.sum(1), 1.0, atol=1e-5)
    counts = np.bincount(ids_np.ravel(), minlength=lc.E)
    assert counts.sum() == T * lc.k
    if lc.zipf_s > 0:  # the skewed workload must actually be skewed
        assert counts.max() > 10 * counts.mean() and (counts == 0).any()
    rows = H.stratified_rows(ids_np, lc.E, T, lc.n_shared, seed=lc.seed)
    res = H.check_layer(lc, inp, out, ids, gates, rows=rows)
    print("%s: %d rows checked, %d near-ties, max row rel err %.3g, frobenius %.3g" % (
        name, res["rows"], res["ties"], res["max_row_rel_err"], res["fro_rel_err"]))


def test_forward_hash_pass_full_size():
    """The decode workload's hash-routed pass at its real shape: tid2eid
    [129280, 6] indexed by uniform random token ids, d = 4096, d_ff = 2048."""
    lc = CONFIGS["v4flash_decode"]
    inp = make_inputs(lc, "cuda", hash_pass=True)
    assert tuple(inp["tid2eid"].shape) == (129280, 6)
    out, ids, gates = H.gpu_forward(H.cfg_of(lc, route_mode=1), inp)
    assert np.array_equal(ids.cpu().numpy(),
                          inp["tid2eid"].cpu().numpy()[inp["token_ids"].cpu().numpy()])
    H.check_layer(lc, inp, out, ids, gates, rows=np.arange(lc.T), route_mode=O.HASH)


# ----------------------------------------------------------------------------
# batch invariance: a token's output, ids and gates do not depend on the batch
# it is computed in ("MoE 架构与路由策略", table dsv4-moe-batch-invariance: the
# MoE reduction order is fixed, no split-K whose split depends on the batch)
# ----------------------------------------------------------------------------
BATCH_INVARIANT = {
    # the full batch runs 288-row prefill tiles, the slices 32-row tiles
    "mixtral_small": CONFIGS["mixtral_prefill"].with_(T=512, d=512, d_ff=1024),
    "dsv3_groups_shared": CONFIGS["dsv3_prefill"].with_(T=1024, d=256, E=16, k=4, d_ff=128,
                                                        n_group=4, topk_group=2, group_topk=2),
    "v4pro_skew": CONFIGS["v4pro_skew_prefill"].with_(T=2048, d=512, E=16, k=4, d_ff=256),
    "tiny_fp32": CONFIGS["tiny_fp32"].with_(T=64),
    # the full batch's router GEMM runs 128x128 tiles (T >= 1024, E >= 128), the
    # slices' 64x64 tiles
    "dsv3_router_tiles": CONFIGS["dsv3_prefill"].with_(T=1024, d=256, E=128, k=8, d_ff=128,
                                                       n_group=8, topk_group=4, group_topk=2),
    # the full batch's down GEMM runs 288-row tiles (512 rows per expert)
    "mixtral_tall_tiles": CONFIGS["mixtral_prefill"].with_(T=2048, d=256, d_ff=256),
    # the full batch runs its small experts on streaming tiles, the rest on
    # 288-row tiles
    "v4pro_skew_split": CONFIGS["v4pro_skew_prefill"].with_(T=1024, d=256, E=32, k=4, d_ff=128),
    # the full batch runs the small groups on the persistent streaming launch
    "v4pro_skew_many_small": CONFIGS["v4pro_skew_prefill"].with_(T=4096, d=256, E=128, k=6,
                                                                 d_ff=1024),
}


def test_forward_on_a_caller_stream():
    # the up GEMM runs its small groups on a stream of the library's own,
    # forked from and joined to the caller's: on a non-default caller stream,
    # three calls in a row (sharing one workspace) whose outputs are copied on
    # that stream right after each call, with no host synchronisation between
    # them, equal the default stream's result bitwise
    lc = SMALL_LAYERS["v4pro_skew_many_small"]
    inp = make_inputs(lc, "cuda")
    ref = [t.clone() for t in H.gpu_forward(H.cfg_of(lc), inp)]
    layer = moe.MoELayer(H.cfg_of(lc), inp)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    got = []
    with torch.cuda.stream(st):
        for _ in range(3):
            layer.forward()
            got.append([layer.out.clone(), layer.ids.clone(), layer.gates.clone()])
    st.synchronize()
    for outs in got:
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("name", list(BATCH_INVARIANT))
def test_forward_batch_invariant(name):
    lc = BATCH_INVARIANT[name]
    inp = make_inputs(lc, "cuda")
    full, full_ids, full_gates = (t.clone() for t in H.gpu_forward(H.cfg_of(lc), inp))
    T = lc.T
    for a, b in [(0, 1), (5, 42), (T // 2, min(T, T // 2 + 64)), (T - 3, T)]:
        sub = dict(inp)
        sub["hidden"] = inp["hidden"][a:b].contiguous()
        if inp.get("token_ids") is not None:
            sub["token_ids"] = inp["token_ids"][a:b].contiguous()
        out, ids, gates = H.gpu_forward(H.cfg_of(lc, T=b - a), sub)
        assert torch.equal(ids, full_ids[a:b]), (a, b)
        assert torch.equal(gates, full_gates[a:b]), (a, b)
        assert torch.equal(out, full[a:b]), (a, b, (out.float() - full[a:b].float()).abs().max())
