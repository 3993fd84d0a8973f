"""Pins of the oracle's MXFP4 (E2M1 weights with 1x32 power-of-two scales) part
against the format's definition, an independent rounding formulation
(numpy's half-to-even rounding on each binade's uniform step), closed-form
bounds, the pages' lossless FP4 -> FP8 claim and dense dequantized arithmetic.
CPU only.

Sources: "MoE 架构与路由策略", FP4 QAT section and table dsv4-moe-fp4-vs-fp8
(E2M1: 2 exponent bits, 1 mantissa bit; one scale per 1x32 sub-block; FP8 tiles
of 128x128; FP4 -> FP8 dequantization lossless while a tile's sub-block scales
stay within the FP8 exponent headroom; native FP4 weights at inference).
"""
import math

import numpy as np
import pytest

import oracle as O

# E2M1 magnitudes by code 0..7 (OCP MX: exponent bias 1, one mantissa bit)
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _round_e2m1(a):
    """|v| -> nearest E2M1 magnitude, ties to the even mantissa: on [0, 2) the
    values are the multiples of 0.5, on [2, 4) of 1, on [4, 6] of 2, so
    half-to-even rounding of a / step (numpy's rule) picks the even code."""
    a = np.minimum(np.abs(np.asarray(a, np.float64)), 6.0)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    return np.minimum(np.round(a / step) * step, 6.0)


def _unpack(q):
    q = np.asarray(q, np.uint8)
    return np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)


def _dequant(q, s):
    """Packed codes [R, C/2] and E8M0 bytes [R, C/32] -> float64 [R, C] (table
    lookup from the format's value list, independent of the oracle)."""
    c = _unpack(q)
    mag = GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    return mag * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)


def test_e2m1_decode_table():
    dec = O.e2m1_decode(np.arange(16))
    assert np.array_equal(dec[:8], GRID)
    assert np.array_equal(dec[8:], -GRID)
    assert math.copysign(1, dec[8]) < 0          # code 8 is -0


def test_e2m1_round_trip_every_code():
    vals = O.e2m1_decode(np.arange(16)).astype(np.float32)
    assert list(O.e2m1_encode(vals)) == list(range(16))


def test_e2m1_ties_go_to_even_mantissa():
    # midpoints between neighbours and the code each must give
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in ties.items():
        assert O.e2m1_encode(v) == c, v
        assert O.e2m1_encode(-v) == 8 | c, -v
        lo, hi = np.nextafter(np.float32(v), np.float32(0)), np.nextafter(np.float32(v), np.float32(9))
        below = [g for g in range(8) if GRID[g] < v][-1]
        above = [g for g in range(8) if GRID[g] > v][0]
        assert O.e2m1_encode(lo) == below and O.e2m1_encode(hi) == above


def test_e2m1_matches_half_even_rounding():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.uniform(-7, 7, 20000), rng.standard_normal(5000) * 0.3,
                        np.arange(-28, 29) / 4.0]).astype(np.float32)
    got = O.e2m1_decode(O.e2m1_encode(x))
    want = _round_e2m1(x) * np.where(np.signbit(x), -1.0, 1.0)
    assert np.array_equal(got, want)


def test_e2m1_saturates():
    assert list(O.e2m1_encode([6.0, 6.5, 100.0, 1e30, -7.0])) == [7, 7, 7, 7, 15]


def _exp_of(amax):
    """The smallest e with amax <= 6 * 2^e (e >= -126), by search."""
    if amax == 0:
        return 0
    e = -126
    while amax > 6.0 * 2.0 ** e:
        e += 1
    return e


def test_quantize_mxfp4_scales_codes_and_bounds():
    rng = np.random.default_rng(22)
    R, C = 40, 256
    w = (rng.standard_normal((R, C)) * rng.uniform(1e-4, 1e3, (R, 1))).astype(np.float32)
    w[3, 64:96] = 0.0                                   # an all-zero block
    w[4, :32] = np.float32(6.0 * 2.0 ** -5)             # amax exactly 6 * 2^-5
    w[5, :32] = np.float32(6.0 * 2.0 ** -5) * np.float32(1.0000001)  # just above: next scale
    q, s = O.quantize_mxfp4(w)
    assert q.shape == (R, C // 2) and s.shape == (R, C // 32)
    blocks = w.reshape(R, C // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    want_e = np.vectorize(_exp_of)(amax)
    assert np.array_equal(s.astype(np.int64) - 127, want_e)
    assert s[4, 0] == 127 - 5 and s[5, 0] == 127 - 4 and s[3, 2] == 127
    assert not _unpack(q)[3, 64:96].any()
    # codes are the half-to-even rounding of w / scale (exact power-of-two scaling)
    sc = np.repeat(np.ldexp(1.0, want_e), 32, axis=1)
    want = _round_e2m1(w / sc) * np.where(np.signbit(w), -1.0, 1.0) * sc
    assert np.array_equal(_dequant(q, s), want)
    # every block's largest magnitude lands in the top binade (3, 6] of the grid
    top = np.abs(want).reshape(R, C // 32, 32).max(axis=2) / np.ldexp(1.0, want_e)
    assert np.all((top[amax > 0] >= 3.0) & (top[amax > 0] <= 6.0))
    # error: at most half a step of the value's binade (the step is 1/2 to 1/4 of
    # the value in the normal range, 0.5 * scale below 1 * scale)
    err = np.abs(_dequant(q, s) - w)
    assert np.all(err <= np.maximum(np.abs(w) / 4, sc / 4) * (1 + 1e-12))


def test_quantize_mxfp4_nibble_order():
    """Element 2j in the low nibble, 2j+1 in the high nibble."""
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1], w[0, 30], w[0, 31] = 6.0, 1.0, -0.5, 3.0
    q, s = O.quantize_mxfp4(w)
    assert s[0, 0] == 127
    assert q[0, 0] == (7 | (2 << 4)) and q[0, 15] == (9 | (5 << 4))


def test_fp4_to_fp8_dequantization_lossless_on_quantized_weights():
    """The page's claim on the oracle's own MXFP4 output: re-quantizing the
    dequantized FP4 weights into FP8 128x128 tiles is exact while the 1x32 scales
    of a tile span at most 2^14 (E4M3 reaches 2^-9 below its 2^8 top binade);
    a tile whose scales span 2^20 is not."""
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[:, 32:64] *= 30.0                                 # sub-block scales vary inside tiles
    q, s = O.quantize_mxfp4(w)
    deq = _dequant(q, s).astype(np.float32)             # exact in float32
    spans = [np.ptp(s[r0:r0 + 128, c0 // 32:(c0 + 128) // 32].astype(int))
             for r0 in range(0, 256, 128) for c0 in range(0, 384, 128)]
    assert max(spans) <= 14
    q8, s8 = O.quantize_blocks(deq)
    back = O.e4m3_decode(q8) * np.kron(s8.astype(np.float64), np.ones((128, 128)))
    assert np.array_equal(back, deq.astype(np.float64))
    bad = deq.copy()
    bad[:128, 96:128] *= np.float32(2.0 ** -20)          # one tile: scales spanning 2^20+
    q8, s8 = O.quantize_blocks(bad)
    back = O.e4m3_decode(q8) * np.kron(s8.astype(np.float64), np.ones((128, 128)))
    assert not np.array_equal(back, bad.astype(np.float64))


def _dq_rows(q, s):
    return O.e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)


def test_expert_ffn_mxfp4_against_dequantized_arrays():
    """32-element block sums scaled by the weight's E8M0 scale and the
    activation's 1x128 scale equal the dense products of the dequantized
    operands; a wrong nibble order, scale index or block size fails here."""
    rng = np.random.default_rng(24)
    d, d_ff = 256, 384
    w13 = (rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32)
    w13[:, 32:64] *= 9.0
    w2 = (rng.standard_normal((d, d_ff)) / 20).astype(np.float32)
    w2[:, 128:160] *= 0.05
    w13q, w13s = O.quantize_mxfp4(w13)
    w2q, w2s = O.quantize_mxfp4(w2)
    x = rng.standard_normal((1, d)).astype(np.float32)
    x[0, :128] *= 100.0
    xq, xs = O.quantize_rows(x)
    y = O.expert_ffn_mxfp4(xq[0], xs[0], w13q, w13s, w2q, w2s)
    gu = _dequant(w13q, w13s) @ _dq_rows(xq, xs)[0]
    g, u = gu[:d_ff], gu[d_ff:]
    with np.errstate(over="ignore"):   # SiLU of a large negative g is -0
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    hq, hs = O.quantize_rows(h[None, :])
    rhq, rhs = O.expert_up_mxfp4(xq[0], xs[0], w13q, w13s)
    assert np.array_equal(rhq, hq[0]) and np.array_equal(rhs, hs[0])
    ref = _dequant(w2q, w2s) @ _dq_rows(hq, hs)[0]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_expert_rows_lowp_mxfp4_equal_single_rows():
    """The batched helper quantizes each listed row 1x128 and runs the MXFP4
    expert on it, exactly as quantize_rows followed by expert_ffn_mxfp4."""
    rng = np.random.default_rng(9)
    d, d_ff = 256, 128
    x = rng.standard_normal((5, d)).astype(np.float32)
    w13q, w13s = O.quantize_mxfp4((rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32))
    w2q, w2s = O.quantize_mxfp4((rng.standard_normal((d, d_ff)) / 11).astype(np.float32))
    tokens = np.array([2, 2, 4, 0], np.int32)
    y = O.expert_rows_lowp("mxfp4", x, tokens, w13q, w13s, w2q, w2s)
    xq, xs = O.quantize_rows(x)
    for q, t in enumerate(tokens):
        assert np.array_equal(y[q], O.expert_ffn_mxfp4(xq[t], xs[t], w13q, w13s, w2q, w2s))


def test_expert_ffn_mxfp4_exact_on_grid_weights():
    """Weights drawn from the E2M1 grid with a 6 in every block (scale 1) are
    stored exactly: the expert equals the dense float64 expert on those weights
    up to the FP8 cast of x and h, which is exact for small integers."""
    rng = np.random.default_rng(25)
    d, d_ff = 128, 128
    signs = lambda shape: rng.choice([-1.0, 1.0], shape)
    w13 = (rng.choice(GRID, (2 * d_ff, d)) * signs((2 * d_ff, d))).astype(np.float32)
    w2 = (rng.choice(GRID, (d, d_ff)) * signs((d, d_ff))).astype(np.float32)
    w13[:, ::32] = 6.0
    w2[:, ::32] = 6.0
    x = rng.choice(np.array([-2, -1, 0, 1, 2], np.float32), (1, d))
    x[0, 0] = 448.0
    w13q, w13s = O.quantize_mxfp4(w13)
    w2q, w2s = O.quantize_mxfp4(w2)
    assert np.all(w13s == 127) and np.all(w2s == 127)
    assert np.array_equal(_dequant(w13q, w13s), w13) and np.array_equal(_dequant(w2q, w2s), w2)
    xq, xs = O.quantize_rows(x)
    assert np.all(xs == 1)
    y = O.expert_ffn_mxfp4(xq[0], xs[0], w13q, w13s, w2q, w2s)
    g = w13[:d_ff].astype(np.float64) @ x[0]
    u = w13[d_ff:].astype(np.float64) @ x[0]
    with np.errstate(over="ignore"):
        h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    hq, hs = O.quantize_rows(h[None, :])
    assert np.allclose(y, w2.astype(np.float64) @ _dq_rows(hq, hs)[0], rtol=1e-13)


def test_layer_mxfp4_close_to_bf16_layer():
    """Same routing as the bf16 layer; E2M1 weights (1 mantissa bit) move the
    output by roughly the weights' relative quantization error, ~10%."""
    rng = np.random.default_rng(26)
    T, d, E, k, d_ff = 24, 256, 6, 2, 256
    h = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / 16).astype(np.float32)
    w13 = [(rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32) for _ in range(E)]
    w2 = [(rng.standard_normal((d, d_ff)) / 16).astype(np.float32) for _ in range(E)]
    sh = ((rng.standard_normal((2 * d_ff, d)) / 16).astype(np.float32),
          (rng.standard_normal((d, d_ff)) / 16).astype(np.float32))
    ref = O.layer(h, wr, w13, w2, k, O.SOFTMAX, w13_shared=sh[0], w2_shared=sh[1])
    q13 = [O.quantize_mxfp4(w) for w in w13]
    q2 = [O.quantize_mxfp4(w) for w in w2]
    qs13, qs2 = O.quantize_mxfp4(sh[0]), O.quantize_mxfp4(sh[1])
    got = O.layer_mxfp4(h, wr, [a for a, _ in q13], [b for _, b in q13], [a for a, _ in q2],
                        [b for _, b in q2], k, O.SOFTMAX,
                        shared=(qs13[0], qs13[1], qs2[0], qs2[1]))
    assert np.array_equal(got["ids"], ref["ids"]) and np.array_equal(got["gates"], ref["gates"])
    rel = np.linalg.norm(got["out"] - ref["out"]) / np.linalg.norm(ref["out"])
    assert 0.02 < rel < 0.25, rel
    # the same layer through the FP8 oracle on the dequantized MXFP4 weights is
    # the same computation (FP4 values are exact in FP8 here) up to summation order
    fp8_13 = [O.quantize_blocks(_dequant(a, b).astype(np.float32)) for a, b in q13]
    fp8_2 = [O.quantize_blocks(_dequant(a, b).astype(np.float32)) for a, b in q2]
    f13 = O.quantize_blocks(_dequant(*qs13).astype(np.float32))
    f2 = O.quantize_blocks(_dequant(*qs2).astype(np.float32))
    via8 = O.layer_fp8(h, wr, [a for a, _ in fp8_13], [b for _, b in fp8_13],
                       [a for a, _ in fp8_2], [b for _, b in fp8_2], k, O.SOFTMAX,
                       shared=(f13[0], f13[1], f2[0], f2[1]))
    assert np.allclose(via8["out"], got["out"], rtol=1e-9, atol=1e-12 * np.abs(got["out"]).max())


def test_quantize_mxfp4_on_zeros():
    q, s = O.quantize_mxfp4(np.zeros((4, 64), np.float32))
    assert not q.any() and np.all(s == 127)
