"""CPU checks of the parity checker itself (no GPU): the layer the checker
assembles from the oracle's pieces equals the oracle's own layer, a planted
output error or routing error is caught, near-tie alternatives are judged
correctly, and the stratified row choice covers every 32-row fragment."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_ffn_sqrt_amd.synth import CONFIGS, make_inputs, to_host_bits

import parity_helpers as H

LAYERS = {
    "grouped_shared_bf16": CONFIGS["dsv3_prefill"].with_(T=48, d=128, E=16, k=4, d_ff=128,
                                                         n_group=4, topk_group=2, group_topk=2),
    "softmax_f32": CONFIGS["tiny_fp32"].with_(T=24),
    "skew_shared_bf16": CONFIGS["v4pro_skew_prefill"].with_(T=40, d=128, E=12, k=3, d_ff=128),
}


def oracle_as_gpu(lc, inp, route_mode=O.LEARNED):
    """The oracle's whole layer in the shape of the GPU results (torch tensors)."""
    grp = dict(n_group=lc.n_group, topk_group=lc.topk_group, group_topk=lc.group_topk)
    r = O.layer(to_host_bits(inp["hidden"]), to_host_bits(inp["w_router"]),
                to_host_bits(inp["w13"]), to_host_bits(inp["w2"]), k=lc.k, scoring=lc.scoring,
                bias=to_host_bits(inp["bias"]), logit_offset=to_host_bits(inp["logit_offset"]),
                w13_shared=to_host_bits(inp["w13_shared"]),
                w2_shared=to_host_bits(inp["w2_shared"]), route_mode=route_mode,
                token_ids=to_host_bits(inp["token_ids"]), tid2eid=to_host_bits(inp["tid2eid"]),
                **grp)
    return torch.from_numpy(r["out"]), torch.from_numpy(r["ids"]), torch.from_numpy(r["gates"])


@pytest.mark.parametrize("name", list(LAYERS))
def test_assembled_layer_equals_oracle_layer(name):
    lc = LAYERS[name]
    inp = make_inputs(lc, "cpu")
    out, ids, gates = oracle_as_gpu(lc, inp)
    res = H.check_layer(lc, inp, out, ids, gates, rows=np.arange(lc.T), tol=1e-12)
    assert res["max_row_rel_err"] <= 1e-12


def test_assembled_hash_layer_equals_oracle_layer():
    lc = CONFIGS["v4flash_decode"].with_(T=20, d=128, d_ff=128, hash_vocab=300)
    inp = make_inputs(lc, "cpu", hash_pass=True)
    out, ids, gates = oracle_as_gpu(lc, inp, route_mode=O.HASH)
    H.check_layer(lc, inp, out, ids, gates, rows=np.arange(lc.T), route_mode=O.HASH, tol=1e-12)


def test_planted_output_error_is_caught():
    lc = LAYERS["grouped_shared_bf16"]
    inp = make_inputs(lc, "cpu")
    out, ids, gates = oracle_as_gpu(lc, inp)
    bad = out.clone()
    bad[7] *= 1.05
    with pytest.raises(AssertionError):
        H.check_layer(lc, inp, bad, ids, gates, rows=np.arange(lc.T))


def test_planted_routing_error_is_caught():
    lc = LAYERS["skew_shared_bf16"]
    inp = make_inputs(lc, "cpu")
    out, ids, gates = oracle_as_gpu(lc, inp)
    bad = ids.clone()
    bad[3, [0, 1]] = bad[3, [1, 0]]  # slot order swapped on a (non-tie) token
    with pytest.raises(AssertionError):
        H.check_layer(lc, inp, out, bad, gates, rows=np.arange(lc.T))


def test_valid_alternative_without_groups():
    keys = np.array([0.9, 0.5, 0.50001, 0.1, 0.7], np.float64)
    ref = np.array([0, 4, 2])
    assert H.valid_alternative(keys, ref, ref, 3)
    assert H.valid_alternative(keys, np.array([0, 4, 1]), ref, 3)      # the near-tie went the other way
    assert not H.valid_alternative(keys, np.array([0, 4, 3]), ref, 3)  # a clearly smaller key
    assert not H.valid_alternative(keys, np.array([4, 0, 2]), ref, 3)  # slot order wrong
    assert not H.valid_alternative(keys, np.array([0, 0, 2]), ref, 3)  # repeated id


def test_valid_alternative_with_groups():
    # 4 groups of 3, top-2 groups by the sum of their top-2 keys, then top-2
    keys = np.array([0.9, 0.8, 0.0,    # group 0: 1.7
                     0.6, 0.5, 0.0,    # group 1: 1.1
                     0.6, 0.49999, 0.0,  # group 2: 1.09999 (near-tie with group 1)
                     0.1, 0.1, 0.0])   # group 3: 0.2
    grp = dict(n_group=4, topk_group=2, group_topk=2)
    ref = np.array([0, 1])
    assert H.valid_alternative(keys, ref, ref, 2, **grp)
    # with k = 3 the third key comes from the second kept group: either near-tied one
    assert H.valid_alternative(keys, np.array([0, 1, 3]), np.array([0, 1, 3]), 3, **grp)
    assert H.valid_alternative(keys, np.array([0, 1, 6]), np.array([0, 1, 3]), 3, **grp)
    # group 3 is never a valid second group
    assert not H.valid_alternative(keys, np.array([0, 1, 9]), np.array([0, 1, 3]), 3, **grp)


def test_stratified_rows_cover_every_fragment():
    rng = np.random.default_rng(0)
    T, E, k = 3000, 10, 2
    w = np.array([40.0, 20, 10, 5, 2, 1, 0.5, 0.2, 0.1, 0.0])
    ids = np.stack([rng.choice(E, k, replace=False, p=w / w.sum()) for _ in range(T)])
    rows = set(H.stratified_rows(ids, E, T, n_shared=1, seed=1).tolist())
    perm = H.dispatch_of(ids, E)
    off, tok = perm["offsets"], perm["sorted_token_ids"]
    for e in range(E):
        a, b = off[e], off[e + 1]
        for f0 in range(a, b, H.FRAG):
            assert rows & set(tok[f0:min(b, f0 + H.FRAG)].tolist()), (e, f0)
        if b > a:
            assert tok[b - 1] in rows
    for f0 in range(0, T, H.FRAG):  # shared expert: identity rows
        assert rows & set(range(f0, min(T, f0 + H.FRAG)))


def test_dequantized_weights_within_one_rounding_step():
    """The helper the low-precision stage tests use to bound a row's move from
    its H differences: codes times scales, each element within half a step of
    the bf16 master (E4M3: 3 mantissa bits; E2M1: 1 bit; plus the subnormal
    step near zero)."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((256, 384)) * np.exp(rng.standard_normal((256, 1)))).astype(np.float32)
    q, s = O.quantize_blocks(w)
    tile_s = np.kron(s, np.ones((128, 128)))
    deq = H.dequantized("fp8", q, s)
    assert np.all(np.abs(deq - w) <= np.abs(w) / 16 + 2.0 ** -10 * tile_s)
    q, s = O.quantize_mxfp4(w)
    blk_s = np.repeat(np.ldexp(1.0, s.astype(np.int32) - 127), 32, axis=1)
    deq = H.dequantized("mxfp4", q, s)
    assert np.all(np.abs(deq - w) <= np.abs(w) / 4 + 0.25 * blk_s)


def test_mxfp4_rows_inverts_the_paired_row_layout():
    """The paired-row code layout, built byte by byte from its definition
    (element (r, c) at byte (r/2)*C + (c/128)*128 + (r%2)*64 + (c%128)/2),
    maps back to the row-major codes."""
    rng = np.random.default_rng(5)
    R, C_ = 6, 384
    rowmajor = rng.integers(0, 256, (R, C_ // 2), dtype=np.uint8)
    flat = np.zeros(R * C_ // 2, np.uint8)
    for r in range(R):
        for c in range(0, C_, 2):
            flat[(r // 2) * C_ + (c // 128) * 128 + (r % 2) * 64 + (c % 128) // 2] = \
                rowmajor[r, c // 2]
    paired = flat.reshape(R // 2, C_)
    assert np.array_equal(H.mxfp4_rows(paired), rowmajor)
    stacked = np.stack([paired, paired[::-1]])
    assert np.array_equal(H.mxfp4_rows(stacked)[0], rowmajor)
