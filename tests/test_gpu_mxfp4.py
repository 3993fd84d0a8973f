"""GPU parity of the MXFP4 expert weights (E2M1 codes, 1x32 E8M0 scales) against
the oracle.

The GPU quantizes the bf16 master weights with moe_quantize_mxfp4 and the hidden
rows inside the layer; the oracle quantizes the same masters itself (pinned on
the CPU), so no oracle input comes from the GPU.  Quantizer codes and scales
must match bit for bit.  The expert stages and the layer then differ from the
oracle only by float32 sums on the GPU against float64 in the oracle, which can
flip an H code at a rounding boundary: the FP8 experts' bounds apply unchanged
(decoded H within one E4M3 step or 4 subnormal steps, flips under 1%, a group
scale one power of two away in at most 1% of groups; expert rows <= 2e-2; layer
rows <= 5e-2 and median <= 1e-2).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_sqrt_amd as moe
import oracle as O
from mixture_experts_ffn_sqrt_amd.synth import CONFIGS, make_inputs, to_host_bits

import parity_helpers as H

pytestmark = pytest.mark.gpu

MIXED_SIZES = [0, 1, 31, 32, 33, 64, 300, 1100]

TOL = 2e-2
LAYER_TOL, LAYER_MEDIAN_TOL = 5e-2, 1e-2


def gpu_mx(w):
    lead, R, C_ = tuple(w.shape[:-2]), w.shape[-2], w.shape[-1]
    q = torch.empty(lead + (R // 2, C_), dtype=torch.uint8, device="cuda")
    s = torch.empty(lead + (C_ // 128, R, 4), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp4(w, q, s)
    torch.cuda.synchronize()
    return H.mxfp4_rows(q.cpu().numpy()), s.cpu().numpy()


def kmajor(s):
    """Oracle scales [R, C/32] -> the library's K-block-major layout [C/128, R, 4]."""
    R, G = s.shape
    return np.ascontiguousarray(s.reshape(R, G // 4, 4).transpose(1, 0, 2))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_mxfp4_bit_exact(dtype):
    g = torch.Generator().manual_seed(41)
    w = torch.randn((70, 384), generator=g) * torch.logspace(-5, 4, 70).unsqueeze(1)
    w[3, 64:96] = 0.0                                    # an all-zero block
    ties = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    w[4, :32] = ties.repeat(4)                           # exact ties, scale 1
    w[5, :32] = -ties.repeat(4) * 2.0 ** -7              # the same at scale 2^-7
    w[6, :] = 1e-30                                      # tiny blocks
    w[7, 32:64] = 3.0e38 * torch.linspace(-1, 1, 32)     # near the float range
    w = w.to(dtype)
    q, s = gpu_mx(w.cuda())
    rq, rs = O.quantize_mxfp4(to_host_bits(w))
    assert np.array_equal(s, kmajor(rs)), np.argwhere(s != kmajor(rs))[:5]
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:5]


def test_quantize_mxfp4_expert_stack_bit_exact():
    g = torch.Generator().manual_seed(42)
    w = (torch.randn((3, 256, 384), generator=g) * 0.02).to(torch.bfloat16)
    w[1, :, 32:64] *= 50
    q, s = gpu_mx(w.cuda())
    for e in range(3):   # each matrix has its own scale table
        rq, rs = O.quantize_mxfp4(to_host_bits(w[e]))
        assert np.array_equal(s[e], kmajor(rs)), e
        assert np.array_equal(q[e], rq), e


def test_quantize_mxfp4_grid_stride_bit_exact():
    # 5 x 1662 x 132 = 1 096 920 blocks: more than one pass of the capped grid
    # (65 536 workgroups x 16 blocks), and a last pass that ends inside a
    # workgroup; each matrix's scale table still lands in its own place
    g = torch.Generator().manual_seed(43)
    w = (torch.randn((5, 1662, 4224), generator=g) * 0.02).to(torch.bfloat16)
    w[4, -1, -32:] = 0.0                                 # the very last block all zero
    w[3, :, :128] *= 300
    q, s = gpu_mx(w.cuda())
    for e in range(5):
        rq, rs = O.quantize_mxfp4(to_host_bits(w[e]))
        assert np.array_equal(s[e], kmajor(rs)), e
        assert np.array_equal(q[e], rq), e


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("T, d, E, k, d_ff", [
    (40, 256, 16, 4, 256),      # a few rows per expert: 32-row streaming tiles
    (700, 256, 4, 2, 384),      # 128x256 tiles (two blocks per CU), ragged rows per expert
    (300, 384, 3, 3, 128),      # k = E, d not a multiple of 256 (partial column tile)
    (1100, 256, 8, 2, 256),     # ~275 rows per expert: three 128-row tiles, a ragged third
    (1, 512, 8, 2, 256),        # one token
    (2100, 384, 4, 2, 128),     # ~1050 rows per expert: 288x256 down tiles, partial column tile
    (1300, 256, 2, 1, 128),     # ~650 rows per expert: 288-row down tiles, ragged last row tile
    # groups of 0, 1, 31, 32, 33, 64, 300 and 1100 rows (195 on average): the
    # groups of at most 32 rows on 32-row streaming tiles, in the same launch as
    # the large tiles of the others (E4M3)
    (1561, 256, 8, 1, 256),
])
def test_expert_up_down_mxfp4(T, d, E, k, d_ff):
    lc = CONFIGS["mixtral_prefill"].with_(T=T, d=d, E=E, k=k, d_ff=d_ff, seed=37)
    inp = make_inputs(lc, "cuda")
    rng = np.random.default_rng(T + 1)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if T == 1561:  # explicit group sizes (see the case list)
        ids = rng.permutation(np.repeat(np.arange(E), MIXED_SIZES)).astype(np.int32)[:, None]
    perm = O.permute(ids, np.ones((T, k), np.float32), E)
    c = H.cfg_of(lc)
    ws = torch.empty(moe.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    xq = torch.empty((T, d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((d // 128, T), dtype=torch.float32, device="cuda")
    moe.moe_quantize_fp8_rows(inp["hidden"], xq, xs)
    mx = moe.quantize_mxfp4_weights(inp)
    hq = torch.zeros((T * k, d_ff), dtype=torch.uint8, device="cuda")
    hs = torch.zeros((d_ff // 128, T * k), dtype=torch.float32, device="cuda")
    y = torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda")
    st, off = _dev(perm["sorted_token_ids"]), _dev(perm["offsets"])
    moe.moe_expert_up_mxfp4(c, xq, xs, st, off, mx["w13q"], mx["w13s"], hq, hs, ws)
    moe.moe_expert_down_mxfp4(c, hq, hs, off, mx["w2q"], mx["w2s"], y, ws)
    torch.cuda.synchronize()
    x_f = inp["hidden"].float().cpu().numpy()
    rxq, rxs = O.quantize_rows(x_f)
    assert np.array_equal(rxq, xq.cpu().numpy()) and np.array_equal(rxs.T, xs.cpu().numpy())
    q13 = [O.quantize_mxfp4(to_host_bits(inp["w13"][e])) for e in range(E)]
    q2 = [O.quantize_mxfp4(to_host_bits(inp["w2"][e])) for e in range(E)]
    for e in range(E):   # the GPU's weight codes and scales are the oracle's
        assert np.array_equal(H.mxfp4_rows(mx["w13q"][e].cpu().numpy()), q13[e][0])
        assert np.array_equal(mx["w13s"][e].cpu().numpy(), kmajor(q13[e][1]))
        assert np.array_equal(H.mxfp4_rows(mx["w2q"][e].cpu().numpy()), q2[e][0])
        assert np.array_equal(mx["w2s"][e].cpu().numpy(), kmajor(q2[e][1]))
    expert_of_row = np.repeat(np.arange(E), perm["counts"])
    g_hq, g_hs = hq.cpu().numpy(), hs.cpu().numpy().T   # scales back to [rows, d_ff/128]
    flips, scale_moves, ref_y, ref_hq, ref_hs, h_differs = 0, 0, [], [], [], []
    dh = {}  # row -> (expert, H_gpu - H_oracle) for the rows whose H differs
    for r, (t, e) in enumerate(zip(perm["sorted_token_ids"], expert_of_row)):
        rhq, rhs = O.expert_up_mxfp4(rxq[t], rxs[t], *q13[e])
        ratio = g_hs[r] / rhs
        assert np.all((ratio == 1) | (ratio == 2) | (ratio == 0.5)), (r, g_hs[r], rhs)
        scale_moves += int((ratio != 1).sum())
        ref_hq.append(rhq)
        ref_hs.append(rhs)
        hg = O.e4m3_decode(g_hq[r]).reshape(-1, 128) * g_hs[r][:, None]
        hr = O.e4m3_decode(rhq).reshape(-1, 128) * rhs[:, None]
        flips += int((hg != hr)[ratio == 1].sum())
        h_differs.append(bool((hg != hr).any()))
        if (hg != hr).any():
            dh[r] = (e, (hg - hr).ravel())
        smax = np.maximum(g_hs[r], rhs)[:, None]
        assert np.all(np.abs(hg - hr) <= np.abs(hr) / 8 + 4 * 2.0 ** -9 * smax), r
        ref_y.append(O.expert_ffn_mxfp4(rxq[t], rxs[t], *q13[e], *q2[e]))
    assert flips <= max(4, 1e-2 * g_hq.size), flips
    assert scale_moves <= max(1, 1e-2 * g_hs.size), scale_moves
    ref_y = np.stack(ref_y)
    # end to end: rows whose H equals the oracle's (an H value one E4M3 step
    # off, or a scale one power of two off, moves y by that step's share)
    err = H.row_rel_err(H.to_f64(y), ref_y)
    keep = ~np.array(h_differs)
    assert not keep.any() or err[keep].max() <= TOL, err[keep].max()
    # rows whose H differs: the down stage is linear in H, so the row may move
    # by at most max_o sum_f |W2[o, f]| |dH_f| (W2 as the oracle dequantizes
    # it) beyond the same tolerance
    yg = H.to_f64(y)
    for r, (e, d_h) in dh.items():
        shift = (np.abs(H.dequantized("mxfp4", *q2[e])) @ np.abs(d_h)).max()
        assert np.abs(yg[r] - ref_y[r]).max() <= TOL * np.abs(ref_y[r]).max() + shift, r
    # the down stage alone: run again on the oracle's H codes and scales
    hq_o = torch.from_numpy(np.stack(ref_hq)).to("cuda")
    hs_o = torch.from_numpy(np.ascontiguousarray(np.stack(ref_hs).T)).to("cuda")
    y.zero_()
    moe.moe_expert_down_mxfp4(c, hq_o, hs_o, off, mx["w2q"], mx["w2s"], y, ws)
    torch.cuda.synchronize()
    err = H.row_rel_err(H.to_f64(y), ref_y)
    assert err.max() <= TOL, err.max()


MX_LAYERS = {
    "mixtral_small": CONFIGS["mixtral_prefill"].with_(T=512, d=512, d_ff=1024),
    "dsv3_groups_shared": CONFIGS["dsv3_prefill"].with_(T=1024, d=256, E=16, k=4, d_ff=128,
                                                        n_group=4, topk_group=2, group_topk=2),
    "v4flash_decode_small": CONFIGS["v4flash_decode"].with_(d=512, d_ff=256),
    "v4pro_skew_small": CONFIGS["v4pro_skew_prefill"].with_(T=2048, d=256, E=16, k=4, d_ff=256),
    "decode_T1": CONFIGS["v4flash_decode"].with_(T=1, d=256, d_ff=128),
    "single_expert": CONFIGS["mixtral_prefill"].with_(T=100, d=256, E=1, k=1, d_ff=128),
    "mixtral_tall_tiles": CONFIGS["mixtral_prefill"].with_(T=2048, d=256, d_ff=256),
    "v4pro_skew_many_small": CONFIGS["v4pro_skew_prefill"].with_(T=4096, d=256, E=128, k=6,
                                                                 d_ff=1024),
}


def check_layer_mx(lc, inp, out, ids, gates, rows, route_mode=O.LEARNED):
    """The MXFP4 layer on the listed rows against the oracle's MXFP4 layer (which
    quantizes the bf16 masters itself), near-tie tokens included."""
    return H.check_layer(lc, inp, out, ids, gates, rows, route_mode=route_mode, fmt="mxfp4",
                         tol=LAYER_TOL, median_tol=LAYER_MEDIAN_TOL)


@pytest.mark.parametrize("name", list(MX_LAYERS))
def test_forward_mxfp4_small(name):
    lc = MX_LAYERS[name]
    inp = make_inputs(lc, "cuda")
    layer = moe.MoELayer(H.cfg_of(lc), inp)
    out = layer.forward_mxfp4(moe.quantize_mxfp4_weights(inp))
    torch.cuda.synchronize()
    check_layer_mx(lc, inp, out, layer.ids, layer.gates, rows=np.arange(lc.T))


def test_forward_mxfp4_hash_pass():
    lc = CONFIGS["v4flash_decode"].with_(d=256, d_ff=256)
    inp = make_inputs(lc, "cuda", hash_pass=True)
    c = H.cfg_of(lc, route_mode=moe.MOE_ROUTE_HASH, vocab=lc.hash_vocab)
    layer = moe.MoELayer(c, inp)
    out = layer.forward_mxfp4(moe.quantize_mxfp4_weights(inp))
    torch.cuda.synchronize()
    check_layer_mx(lc, inp, out, layer.ids, layer.gates, rows=np.arange(lc.T), route_mode=O.HASH)


@pytest.mark.parametrize("name, n_rows", [("mixtral_prefill", 24), ("v4flash_decode", 64),
                                          ("dsv3_prefill", 6), ("v4pro_skew_prefill", 6)])
def test_forward_mxfp4_full_size(name, n_rows):
    """Full size, in the launch configuration the bench times: the layer on
    sampled rows (hottest and coldest experts' included), the two expert stages
    on every row tile of a spread of experts, and every expert's quantized
    weights spot-checked against the oracle's quantizer."""
    lc = CONFIGS[name]
    inp = make_inputs(lc, "cuda")
    layer = moe.MoELayer(H.cfg_of(lc), inp)
    mx = moe.quantize_mxfp4_weights(inp)
    out = layer.forward_mxfp4(mx)
    torch.cuda.synchronize()
    ids_np = layer.ids.cpu().numpy()
    counts = np.bincount(ids_np.ravel(), minlength=lc.E)
    rows = np.random.default_rng(6).choice(lc.T, min(n_rows, lc.T), replace=False)
    rows = np.unique(np.r_[rows, H.hot_cold_rows(ids_np, counts)])
    check_layer_mx(lc, inp, out, layer.ids, layer.gates, rows=rows)
    H.check_lowp_stages(lc, inp, "mxfp4", mx, layer.ids, layer.gates, LAYER_TOL,
                        LAYER_MEDIAN_TOL, seed=lc.seed)
    H.check_quantized_tiles(inp, mx, "mxfp4", seed=lc.seed)


@pytest.mark.parametrize("name", ["mixtral_small", "mixtral_tall_tiles", "dsv3_groups_shared"])
def test_forward_mxfp4_batch_invariant(name):
    # mixtral_tall_tiles: the full batch's down GEMM runs 288-row tiles;
    # dsv3_groups_shared: both of its GEMMs run 128-row tiles (two blocks per
    # CU), the slices 32-row tiles
    lc = MX_LAYERS[name]
    inp = make_inputs(lc, "cuda")
    mx = moe.quantize_mxfp4_weights(inp)
    layer = moe.MoELayer(H.cfg_of(lc), inp)
    full = layer.forward_mxfp4(mx).clone()
    for a, b in [(0, 1), (7, 60), (400, 512), (lc.T - 3, lc.T)]:
        sub = dict(inp)
        sub["hidden"] = inp["hidden"][a:b].contiguous()
        part = moe.MoELayer(H.cfg_of(lc, T=b - a), sub).forward_mxfp4(mx)
        torch.cuda.synchronize()
        assert torch.equal(part, full[a:b]), (a, b)
