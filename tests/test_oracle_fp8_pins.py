"""Pins of the oracle's FP8 (E4M3) part against the format's definition, an
independent library conversion (torch.float8_e4m3fn), closed-form invariants and
array reformulations.  CPU only.

Sources: "MoE 架构与路由策略" (FP4 QAT section, table dsv4-moe-fp4-vs-fp8: E4M3
with 4 exponent and 3 mantissa bits, one scale per 128x128 weight tile; table
dsv4-moe-stages: activation + FP8 cast); "MoE 的算量与通信" 五.2 (FP8 dispatch).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]  # 0x7F / 0xFF are NaN


def test_e4m3_decode_table():
    dec = O.e4m3_decode(np.arange(256))
    assert dec[0x00] == 0.0 and dec[0x80] == 0.0 and math.copysign(1, dec[0x80]) < 0
    assert dec[0x01] == 2.0 ** -9          # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert dec[0x08] == 2.0 ** -6          # smallest normal
    assert dec[0x38] == 1.0
    assert dec[0x39] == 1.125
    assert dec[0x7E] == 448.0              # largest finite, (1 + 6/8) * 2^8
    assert dec[0xFE] == -448.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert len(FINITE) == 254
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes decode to increasing values"


def test_e4m3_round_trip_every_code():
    vals = O.e4m3_decode(FINITE).astype(np.float32)
    assert list(O.e4m3_encode(vals)) == FINITE


def test_e4m3_matches_torch_conversion():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * 30.0,
        rng.standard_normal(5000) * 2.0 ** -7,     # subnormal range
        rng.uniform(-463.9, 463.9, 5000),          # up to the last value that rounds to 448
        O.e4m3_decode(FINITE[:0x7E]),              # exact codes
    ]).astype(np.float32)
    x = x[np.abs(x) < 463.9]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_e4m3_ties_go_to_even_mantissa():
    dec = O.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):
        mid = np.float32((dec[c] + dec[c + 1]) / 2)   # exact in float32
        want = c if c % 2 == 0 else c + 1
        assert O.e4m3_encode(mid) == want, hex(c)
        lo, hi = np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))
        assert O.e4m3_encode(lo) == c and O.e4m3_encode(hi) == c + 1


def test_e4m3_saturates():
    assert list(O.e4m3_encode([448.0, 463.9, 464.0, 1e6, -1e30])) == [0x7E] * 4 + [0xFE]


def _dequant_rows(q, s):
    return O.e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)


def _scale_of(amax):
    """The smallest power of two 2^e with amax <= 448 * 2^e (e >= -126), by search."""
    out = np.ones_like(amax, dtype=np.float64)
    for idx, a in np.ndenumerate(amax):
        if a == 0:
            continue
        e = -126
        while a > 448.0 * 2.0 ** e:
            e += 1
        out[idx] = 2.0 ** e
    return out.astype(np.float32)


def test_quantize_rows_bounds_and_extremes():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 512)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    x[5, 128:256] = 0.0                                # an all-zero group
    x[6, 0:128] = np.float32(448.0) * np.float32(2.0 ** -3)   # amax exactly 448 * 2^-3
    q, s = O.quantize_rows(x)
    g = x.reshape(64, 4, 128)
    amax = np.abs(g).max(axis=2)
    assert np.array_equal(s, _scale_of(amax))
    assert s[6, 0] == 2.0 ** -3
    assert s[5, 1] == 1.0 and not q[5, 128:256].any()
    # the largest element of every non-zero group lands in the top binade (224, 448]
    idx = np.abs(g).argmax(axis=2)
    top = np.take_along_axis(q.reshape(64, 4, 128), idx[..., None], 2)[..., 0]
    tv = np.abs(O.e4m3_decode(top[amax > 0]))
    assert np.all((tv >= 224) & (tv <= 448))
    # error bound: half a step of E4M3 (2^-4 relative for normals, 2^-10 * s absolute below)
    err = np.abs(_dequant_rows(q, s) - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(s, 128, axis=1) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))


def test_quantize_rows_power_of_two_invariance():
    """Scales are powers of two: scaling the input by 8 scales the scale by 8
    and leaves every code unchanged."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q1, s1 = O.quantize_rows(x)
    q2, s2 = O.quantize_rows(x * np.float32(8.0))
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * np.float32(8.0))


def test_quantize_blocks_against_torch_formulation():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[128:256, 0:128] *= 50.0                          # tiles with different ranges
    q, s = O.quantize_blocks(w)
    assert s.shape == (2, 3)
    for br in range(2):
        for bc in range(3):
            blk = w[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
            sc = _scale_of(np.array([np.abs(blk).max()]))[0]
            v = (blk / sc).astype(np.float32)          # exact: sc is a power of two
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert s[br, bc] == sc
            assert np.array_equal(q[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128], ref)


def test_fp4_to_fp8_tile_dequantization_is_lossless():
    """The page's claim: MXFP4 weights (E2M1 values with a power-of-two scale per
    1x32 sub-block) re-quantized to FP8 128x128 tiles lose nothing as long as the
    sub-block scales of a tile span little enough of the FP8 exponent range."""
    rng = np.random.default_rng(13)
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    vals = rng.choice(e2m1, (256, 256)) * rng.choice([-1, 1], (256, 256))
    sub = 2.0 ** rng.integers(-3, 4, (256, 256 // 32))          # a 2^6 spread per tile
    w = (vals * np.repeat(sub, 32, axis=1)).astype(np.float32)
    q, s = O.quantize_blocks(w)
    assert np.array_equal(_dequant_blocks(q, s), w.astype(np.float64))


def _dequant_blocks(q, s):
    return O.e4m3_decode(q) * np.kron(s.astype(np.float64), np.ones((128, 128)))


def test_expert_ffn_fp8_against_dequantized_arrays():
    """Per-block scaled sums equal the dot products of the dequantized operands;
    wrong scale indexing or a transposed scale layout fails here."""
    rng = np.random.default_rng(6)
    d, d_ff = 256, 384
    w13 = (rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32)
    w13[:, 128:] *= 7.0
    w2 = (rng.standard_normal((d, d_ff)) / 20).astype(np.float32)
    w2[128:, :] *= 0.1
    w13q, w13s = O.quantize_blocks(w13)
    w2q, w2s = O.quantize_blocks(w2)
    x = rng.standard_normal((1, d)).astype(np.float32)
    x[0, :128] *= 100.0
    xq, xs = O.quantize_rows(x)
    y = O.expert_ffn_fp8(xq[0], xs[0], w13q, w13s, w2q, w2s)
    xd = _dequant_rows(xq, xs)[0]
    gu = _dequant_blocks(w13q, w13s) @ xd
    g, u = gu[:d_ff], gu[d_ff:]
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    hq, hs = O.quantize_rows(h[None, :])
    ref = _dequant_blocks(w2q, w2s) @ _dequant_rows(hq, hs)[0]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_expert_rows_lowp_fp8_equal_single_rows():
    """The batched helper quantizes each listed row 1x128 and runs the FP8 expert
    on it, exactly as quantize_rows followed by expert_ffn_fp8."""
    rng = np.random.default_rng(8)
    d, d_ff = 256, 128
    x = rng.standard_normal((5, d)).astype(np.float32)
    w13q, w13s = O.quantize_blocks((rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32))
    w2q, w2s = O.quantize_blocks((rng.standard_normal((d, d_ff)) / 11).astype(np.float32))
    tokens = np.array([4, 1, 4, 0], np.int32)
    y = O.expert_rows_lowp("fp8", x, tokens, w13q, w13s, w2q, w2s)
    xq, xs = O.quantize_rows(x)
    for q, t in enumerate(tokens):
        assert np.array_equal(y[q], O.expert_ffn_fp8(xq[t], xs[t], w13q, w13s, w2q, w2s))


def test_expert_ffn_fp8_exact_on_small_integers():
    """Codes of small integers with unit scales: every sum is an exact integer."""
    rng = np.random.default_rng(8)
    d, d_ff = 128, 128
    ints = np.array([-3, -2, -1, 0, 1, 2, 3], np.float32)
    w13 = rng.choice(ints, (2 * d_ff, d))
    w2 = rng.choice(ints, (d, d_ff))
    w13[0, 0] = w13[d_ff, 0] = w2[0, 0] = 448.0    # every tile: max 448, scale 1
    x = rng.choice(ints, (1, d))
    x[0, 0] = 448.0
    w13q, w13s = O.quantize_blocks(w13)
    w2q, w2s = O.quantize_blocks(w2)
    xq, xs = O.quantize_rows(x)
    assert np.all(w13s == 1) and np.all(w2s == 1) and np.all(xs == 1)
    y = O.expert_ffn_fp8(xq[0], xs[0], w13q, w13s, w2q, w2s)
    g = w13[:d_ff].astype(np.float64) @ x[0]
    u = w13[d_ff:].astype(np.float64) @ x[0]
    assert np.all(g == np.round(g)) and np.all(u == np.round(u))
    with np.errstate(over="ignore"):   # SiLU of a large negative g is -0
        h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    hq, hs = O.quantize_rows(h[None, :])
    assert np.allclose(y, w2.astype(np.float64) @ _dequant_rows(hq, hs)[0], rtol=1e-13)


def test_layer_fp8_close_to_bf16_layer():
    """Same routing as the bf16 layer; FP8 experts change each output by a few
    percent at most (3 mantissa bits, errors averaging over d and d_ff)."""
    rng = np.random.default_rng(9)
    T, d, E, k, d_ff = 24, 256, 6, 2, 256
    h = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / 16).astype(np.float32)
    w13 = [(rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32) for _ in range(E)]
    w2 = [(rng.standard_normal((d, d_ff)) / 16).astype(np.float32) for _ in range(E)]
    sh = ((rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32),
          (rng.standard_normal((d, d_ff)) / 16).astype(np.float32))
    ref = O.layer(h, wr, w13, w2, k, O.SOFTMAX, w13_shared=sh[0], w2_shared=sh[1])
    q13 = [O.quantize_blocks(w) for w in w13]
    q2 = [O.quantize_blocks(w) for w in w2]
    qs13, qs2 = O.quantize_blocks(sh[0]), O.quantize_blocks(sh[1])
    got = O.layer_fp8(h, wr, [a for a, _ in q13], [b for _, b in q13], [a for a, _ in q2],
                      [b for _, b in q2], k, O.SOFTMAX, shared=(qs13[0], qs13[1], qs2[0], qs2[1]))
    assert np.array_equal(got["ids"], ref["ids"]) and np.array_equal(got["gates"], ref["gates"])
    rel = np.linalg.norm(got["out"] - ref["out"]) / np.linalg.norm(ref["out"])
    assert 1e-4 < rel < 0.08, rel


@pytest.mark.parametrize("which", ["rows", "blocks"])
def test_quantizers_on_zeros(which):
    z = np.zeros((128, 256), np.float32)
    q, s = O.quantize_rows(z) if which == "rows" else O.quantize_blocks(z)
    assert not q.any() and np.all(s == 1.0)
