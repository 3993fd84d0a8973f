#!/usr/bin/env python3
"""Benchmark: one MoE FFN layer step on one MI355X.

A step is one moe_forward call (router GEMM, scores + top-k, permutation,
grouped SwiGLU GEMM 1, grouped GEMM 2, combine) over one batch of synthetic
inputs already resident in HBM.  Prints ONE JSON line with tokens/s of the
headline workload (DeepSeek-V4-Pro-shaped prefill with a Zipf-skewed load,
T=16384, d=7168, E=384+1, top-6, d_ff=3072: the largest configuration), the
roofline of its dominant kernel (grouped GEMM 1 + SwiGLU), the chip's measured
ceilings, and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--side NAMES|none]

Beside the headline the line carries the other prefill workloads (DeepSeek-V3
and Mixtral shapes) and the decode workload (V4-Flash shapes, learned and
hash-routed passes), and the FP8 / MXFP4 expert variants of every workload,
each with the roofline of its GEMM 1.  A roofline's bound is the one that the
kernel's algorithmic FLOPs and bytes make binding at the published peaks
(matrix cores for large groups, HBM where the weights outweigh the rows that
use them); the other bound's fraction rides along.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM % bf16 MFMA peak (prefill), % HBM BW (decode)"
DEFAULT_WORKLOAD = "v4pro_skew_prefill"  # T=16384, d=7168, E=384+1, top-6, d_ff=3072, bf16
SIDE_WORKLOADS = ("dsv3_prefill", "mixtral_prefill", "v4flash_decode")
SIDE_CPU_SECONDS = 3.0  # oracle on one host thread per side workload

# MI355X published peaks
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}  # dense MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--side", default=",".join(SIDE_WORKLOADS),
                    help="comma-separated workloads reported beside the headline, or 'none'")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the workload, copy 1 GiB three times (counter calibration)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured ceilings and the vendor-library reference points")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8-expert measurements reported beside the bf16 ones")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the MXFP4-weight measurements reported beside the bf16 ones")
    return ap.parse_args()


KERNEL_SOURCES = {
    "bf16": ("mixture_experts_ffn_sqrt_amd/csrc/moe_gemm_kernels.h",
             "mixture_experts_ffn_sqrt_amd/csrc/moe_gemm.hip"),
    "fp8": ("mixture_experts_ffn_sqrt_amd/csrc/moe_gemm_kernels.h",
            "mixture_experts_ffn_sqrt_amd/csrc/moe_gemm_fp8.h",
            "mixture_experts_ffn_sqrt_amd/csrc/moe_fp8.hip"),
}
KERNEL_SOURCES["mxfp4"] = KERNEL_SOURCES["fp8"]


def code_text(src):
    """C/HIP source with its comments removed and its whitespace collapsed, so
    that an edit of the comments alone leaves the code's hash unchanged."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_sha(kind="bf16"):
    """SHA-256 of the code (comments aside) of the sources a GEMM kind is built
    from: the key under which its counter-derived traffic is stored."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def measured_traffic(workload, kind="bf16"):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/traffic.json, keyed "<workload>" for bf16 and
    "<workload>_fp8"), or None when it is absent or was taken on different
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(workload if kind == "bf16" else workload + "_" + kind)
    if not ent or ent.get("kernel_source_sha") != kernel_source_sha(kind):
        return None
    return int(ent["fetch_bytes_per_launch"] + ent["write_bytes_per_launch"])


def accounting(lc, counts):
    """Algorithmic work of the grouped expert GEMMs from the realised routing.
    Units: one dispatch row = one (token, expert) pair, shared expert included.
      GEMM 1 (+SwiGLU): 4*d*d_ff FLOPs per row; bytes = w13 of every expert with
      rows (2*d_ff*d elements) + gathered rows read (d) + H written (d_ff) per row
      GEMM 2: 2*d*d_ff FLOPs per row; bytes = w2 of active experts + H read + Y written
    Layer FLOPs per row: 6*d*d_ff (the SwiGLU count)."""
    import numpy as np
    es = 4 if lc.dtype == "f32" else 2
    d, F, T, k, S = lc.d, lc.d_ff, lc.T, lc.k, lc.n_shared
    active = int((np.asarray(counts) > 0).sum()) + S
    rows = T * k + S * T
    routed_rows = T * k
    routed_active = int((np.asarray(counts) > 0).sum())
    up_flops = 4 * d * F * rows
    up_bytes = (active * 2 * F * d + rows * d + rows * F) * es
    up_routed_flops = 4 * d * F * routed_rows
    up_routed_bytes = (routed_active * 2 * F * d + routed_rows * d + routed_rows * F) * es
    layer_flops = 6 * d * F * rows + 2 * T * d * lc.E
    layer_bytes = (active * 3 * F * d + 2 * T * d + 2 * rows * F) * es + T * lc.E * 4
    return dict(active_experts=active, rows=rows, up_flops=up_flops, up_bytes=up_bytes,
                up_routed_flops=up_routed_flops, up_routed_bytes=up_routed_bytes,
                layer_flops=layer_flops, layer_bytes=layer_bytes)


def time_gpu(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall


def step_percentiles(fn, steps, stream):
    """Each of `steps` further steps timed on its own (HIP events on the launch
    stream): p10 / p50 / p90 in ms.  Outside the timed region of `value`."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return [round(float(np.percentile(t, q)), 4) for q in (10, 50, 90)]


def input_digests(inp):
    """Digests of every input buffer's bytes, so that a result can be tied to the
    exact synthetic inputs whatever generator produced them: SHA-256 of the
    small tensors, XXH3-128 of the expert weight stacks (tens of GB, streamed
    to the host one expert at a time)."""
    import hashlib

    import torch
    import xxhash
    sha, xxh = {}, {}
    for name in sorted(inp):
        t = inp[name]
        if t is None:
            continue
        if name in ("w13", "w2"):
            h = xxhash.xxh3_128()
            for e in range(t.shape[0]):
                h.update(t[e].detach().contiguous().view(torch.uint8).cpu().numpy().tobytes())
            xxh[name] = h.hexdigest()
        else:
            b_ = t.detach().contiguous().view(torch.uint8).cpu().numpy()
            sha[name] = hashlib.sha256(b_.tobytes()).hexdigest()
    return dict(sha256=sha, xxh3_128=xxh)


def output_digest(t):
    """XXH3-128 of a layer output's bytes (after the timed region, from one more
    step on the same inputs): two runs computed the same output bitwise exactly
    when their digests agree."""
    import torch
    import xxhash
    torch.cuda.synchronize()
    return xxhash.xxh3_128(t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()


def lowp_accounting(lc, counts, kind):
    """Algorithmic work of the low-precision expert GEMM 1 (routed rows): the same
    FLOPs as bf16; bytes = every active expert's w13 codes and scales (FP8: 1
    byte per weight and a float per 128x128 tile; MXFP4: half a byte per weight
    and a byte per 32), the gathered rows' E4M3 codes and 1x128 scales, and H's
    codes and scales."""
    import numpy as np
    d, F, T, k = lc.d, lc.d_ff, lc.T, lc.k
    act = int((np.asarray(counts) > 0).sum())
    rows = T * k
    flops = 4 * d * F * rows
    if kind == "mxfp4":
        wbytes = 2 * F * d // 2 + 2 * F * (d // 32)
    else:
        wbytes = 2 * F * d + (2 * F // 128) * (d // 128) * 4
    nbytes = act * wbytes + rows * (d + d // 128 * 4) + rows * (F + F // 128 * 4)
    return flops, nbytes


def layer_roofline(flops, nbytes, ms, dtype):
    """The whole layer step against its roofline: rates, each as a fraction of
    its published peak, and roof_frac = t_roof / t_measured with t_roof =
    max(FLOPs / MFMA peak, bytes / HBM peak) (the larger of the two fractions)."""
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    mfma_frac, hbm_frac = tflops / PEAK_TFLOPS[dtype], gbs / PEAK_HBM_GBS
    return dict(tflops=round(tflops, 1), gbs=round(gbs, 1), hbm_frac=round(hbm_frac, 4),
                mfma_frac=round(mfma_frac, 4), roof_frac=round(max(mfma_frac, hbm_frac), 4))


def roofline_of(flops, nbytes, ms, mfma_peak, mfma_ceiling, hbm_ceiling):
    """Roofline of one kernel launch: its algorithmic FLOPs and bytes over its
    measured duration.  The bound is the one whose ideal time at the published
    peaks is longer (FLOPs / MFMA peak against bytes / HBM peak: the ridge
    point), so a batch whose experts see few rows is priced against the HBM
    it streams the weights from, and a batch of large groups against the
    matrix cores; the other bound's fraction is reported beside it."""
    s = ms * 1e-3
    tflops, gbs = flops / s / 1e12, nbytes / s / 1e9
    mfma = dict(achieved=round(tflops, 1), peak=mfma_peak, unit="TFLOP/s",
                frac=round(tflops / mfma_peak, 4))
    hbm = dict(achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
               frac=round(gbs / PEAK_HBM_GBS, 4))
    if nbytes / PEAK_HBM_GBS / 1e9 > flops / mfma_peak / 1e12:
        roof, other, ceil = dict(bound="hbm", **hbm), dict(bound="mfma", **mfma), hbm_ceiling
        ach = gbs
    else:
        roof, other, ceil = dict(bound="mfma", **mfma), dict(bound="hbm", **hbm), mfma_ceiling
        ach = tflops
    roof["other_bound"] = other
    roof["measured_peak"] = ceil
    roof["frac_of_measured_peak"] = round(ach / ceil, 4) if ceil else None
    roof["kernel_ms"] = round(ms, 4)
    return roof


def up_roofline(acct, ms_up, dtype, measured, name):
    """Roofline of the dominant kernel (grouped GEMM 1 + SwiGLU, routed rows),
    against the published peaks and the chip's measured ceilings."""
    m = measured or {}
    roof = roofline_of(acct["up_routed_flops"], acct["up_routed_bytes"], ms_up,
                       PEAK_TFLOPS[dtype],
                       m.get("mfma_bf16_random_tflops") if dtype == "bf16" else None,
                       m.get("hbm_read_stream_gbs"))
    roof["traffic"] = measured_traffic(name)
    roof["kernel"] = "grouped GEMM 1 + SwiGLU (moe_expert_up, routed rows)"
    return roof


def run_workload(name, steps, warmup, with_cpu, cpu_seconds, with_fp8=True, with_mx=True,
                 measured=None, cpu_single=0.0):
    import numpy as np
    import torch

    import mixture_experts_ffn_sqrt_amd as moe
    from mixture_experts_ffn_sqrt_amd.synth import CONFIGS, make_inputs

    lc = CONFIGS[name]
    stream = torch.cuda.current_stream()
    with_hash = lc.hash_vocab > 0
    inp = make_inputs(lc, "cuda", hash_pass=with_hash)
    c = moe.make_config(T=lc.T, d=lc.d, E=lc.E, k=lc.k, d_ff=lc.d_ff, n_shared=lc.n_shared,
                        dtype=lc.dtype, scoring=lc.scoring, n_group=lc.n_group,
                        topk_group=lc.topk_group, group_topk=lc.group_topk)
    # the learned-route layer does not take the hash pass's table
    layer = moe.MoELayer(c, dict(inp, token_ids=None, tid2eid=None))
    print("[bench] %s: inputs ready, workspace %.1f MB" % (name, layer.workspace.numel() / 1e6),
          file=sys.stderr, flush=True)

    ms_step, wall = time_gpu(layer.forward, steps, warmup, stream)
    print("[bench] %s: %.3f ms/step" % (name, ms_step), file=sys.stderr, flush=True)
    pct = step_percentiles(layer.forward, steps, stream)

    # staged pieces on the same stream: routing decision of the last step
    ids = layer.ids
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=lc.E)
    acct = accounting(lc, counts)
    T, k, E = lc.T, lc.k, lc.E
    ws = layer.workspace
    perm = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                tok=torch.empty(T * k, dtype=torch.int32, device="cuda"),
                w=torch.empty(T * k, dtype=torch.float32, device="cuda"),
                disp=torch.empty((T, k), dtype=torch.int32, device="cuda"))
    moe.moe_permute(c, ids, layer.gates, perm["counts"], perm["offsets"], perm["tok"], perm["w"],
                    perm["disp"], ws)
    H = torch.empty((T * k, lc.d_ff), dtype=lc.torch_dtype, device="cuda")
    Y = torch.empty((T * k, lc.d), dtype=lc.torch_dtype, device="cuda")
    out = torch.empty((T, lc.d), dtype=lc.torch_dtype, device="cuda")

    def up():
        moe.moe_expert_up(c, inp["hidden"], perm["tok"], perm["offsets"], inp["w13"], H, ws)

    def down():
        moe.moe_expert_down(c, H, perm["offsets"], inp["w2"], Y, ws)

    def combine():
        moe.moe_combine(c, Y, perm["disp"], layer.gates, None, out)

    ms_up, _ = time_gpu(up, steps, warmup, stream)
    ms_down, _ = time_gpu(down, steps, warmup, stream)
    ms_combine, _ = time_gpu(combine, steps, warmup, stream)

    roof = up_roofline(acct, ms_up, lc.dtype, measured, name)
    gemm_tflops = 6 * lc.d * lc.d_ff * T * k / ((ms_up + ms_down) * 1e-3) / 1e12
    res = dict(
        workload=name, ms_per_step=ms_step, tokens_per_s=T / (ms_step * 1e-3), wall_s=wall,
        step_ms_p10_p50_p90=pct,
        roofline=roof,
        grouped_gemm=dict(ms_up=round(ms_up, 4), ms_down=round(ms_down, 4),
                          tflops=round(gemm_tflops, 1),
                          frac_bf16_peak=round(gemm_tflops / PEAK_TFLOPS[lc.dtype], 4)),
        # the combine of the routed rows on its own (the GEMM 2 output read back
        # and the gated sum written): the cost of keeping the weighted sum out
        # of the GEMM 2 epilogue
        combine=dict(ms=round(ms_combine, 4), share_of_step=round(ms_combine / ms_step, 4)),
        layer=layer_roofline(acct["layer_flops"], acct["layer_bytes"], ms_step, lc.dtype),
        routing=dict(active_experts=acct["active_experts"], max_rows=int(counts.max()),
                     mean_rows=float(counts.mean()), empty_experts=int((counts == 0).sum())),
    )
    res["output_xxh3_128"] = output_digest(layer.forward())
    if with_hash:
        # the hash-routed pass: ids from tid2eid[token_ids], same experts and shapes
        hc = moe.make_config(T=lc.T, d=lc.d, E=lc.E, k=lc.k, d_ff=lc.d_ff,
                             n_shared=lc.n_shared, dtype=lc.dtype, scoring=lc.scoring,
                             route_mode=moe.MOE_ROUTE_HASH, vocab=lc.hash_vocab)
        hl = moe.MoELayer(hc, inp)
        ms_hash, _ = time_gpu(hl.forward, steps, warmup, stream)
        hcounts = np.bincount(hl.ids.cpu().numpy().ravel(), minlength=lc.E)
        hacct = accounting(lc, hcounts)
        res["hash_pass"] = dict(
            ms_per_step=round(ms_hash, 4), tokens_per_s=round(T / (ms_hash * 1e-3), 1),
            vocab=lc.hash_vocab, active_experts=hacct["active_experts"],
            layer_gbs=round(hacct["layer_bytes"] / (ms_hash * 1e-3) / 1e9, 1),
            layer_hbm_frac=round(hacct["layer_bytes"] / (ms_hash * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        print("[bench] %s hash pass: %.3f ms/step" % (name, ms_hash), file=sys.stderr, flush=True)
        del hl
    lowp_ok = lc.dtype == "bf16" and lc.d % 128 == 0 and lc.d_ff % 128 == 0
    for kind, on in (("fp8", with_fp8), ("mxfp4", with_mx)):
        if on and lowp_ok:
            res[kind] = run_lowp(kind, lc, c, layer, inp, perm, ws, Y, counts, steps,
                                 warmup, stream, measured)
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(lc, inp, cpu_seconds)
        res["input_digests"] = input_digests(inp)
    elif cpu_single > 0:
        res["cpu_single_core"] = cpu_single_core(lc, inp, cpu_single)
    del layer, inp, H, Y, out, perm
    torch.cuda.empty_cache()
    return res


def run_lowp(kind, lc, c, layer, inp, perm, ws, Y, counts, steps, warmup, stream,
             measured=None):
    """The same step with FP8 activations and FP8 (E4M3, kind "fp8") or MXFP4
    (kind "mxfp4") expert weights (moe_forward_fp8 / moe_forward_mxfp4), and its
    two grouped GEMMs on their own; weights quantized once on the GPU beforehand.
    The peak is the FP8 matrix rate in both cases: the activations are E4M3, so
    every MFMA has an FP8 operand."""
    import torch

    import mixture_experts_ffn_sqrt_amd as moe
    T, k, d, F = lc.T, lc.k, lc.d, lc.d_ff
    mx = kind == "mxfp4"
    wq = moe.quantize_mxfp4_weights(inp) if mx else moe.quantize_fp8_weights(inp)
    fwd = layer.forward_mxfp4 if mx else layer.forward_fp8
    ms_step, _ = time_gpu(lambda: fwd(wq), steps, warmup, stream)
    print("[bench] %s %s: %.3f ms/step" % (lc.name, kind, ms_step), file=sys.stderr, flush=True)
    xq = torch.empty((T, d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((d // 128, T), dtype=torch.float32, device="cuda")
    moe.moe_quantize_fp8_rows(inp["hidden"], xq, xs)
    hq = torch.empty((T * k, F), dtype=torch.uint8, device="cuda")
    hs = torch.empty((F // 128, T * k), dtype=torch.float32, device="cuda")
    up_fn = moe.moe_expert_up_mxfp4 if mx else moe.moe_expert_up_fp8
    down_fn = moe.moe_expert_down_mxfp4 if mx else moe.moe_expert_down_fp8

    def up():
        up_fn(c, xq, xs, perm["tok"], perm["offsets"], wq["w13q"], wq["w13s"], hq, hs, ws)

    def down():
        down_fn(c, hq, hs, perm["offsets"], wq["w2q"], wq["w2s"], Y, ws)

    ms_up, _ = time_gpu(up, steps, warmup, stream)
    ms_down, _ = time_gpu(down, steps, warmup, stream)
    flops, nbytes = lowp_accounting(lc, counts, kind)
    m = measured or {}
    roof = roofline_of(flops, nbytes, ms_up, PEAK_TFLOPS["fp8"], m.get("mfma_fp8_random_tflops"),
                       m.get("hbm_read_stream_gbs"))
    roof["traffic"] = measured_traffic(lc.name, kind)
    roof["kernel"] = "%s grouped GEMM 1 + SwiGLU + FP8 cast (%s, routed rows)" % (
        "MXFP4-weight" if mx else "FP8", up_fn.__name__)
    gemm_tflops = 6 * d * F * T * k / ((ms_up + ms_down) * 1e-3) / 1e12
    digest = output_digest(fwd(wq))
    del wq, xq, xs, hq, hs
    return dict(ms_per_step=round(ms_step, 4), tokens_per_s=round(T / (ms_step * 1e-3), 1),
                roofline=roof, output_xxh3_128=digest,
                grouped_gemm=dict(ms_up=round(ms_up, 4), ms_down=round(ms_down, 4),
                                  tflops=round(gemm_tflops, 1),
                                  frac_fp8_peak=round(gemm_tflops / PEAK_TFLOPS["fp8"], 4)))


def measured_ceilings():
    """The chip's ceilings measured by the committed microbenchmarks
    (include/moe_peaks.h): matrix-core rates on random operands, HBM read stream."""
    from mixture_experts_ffn_sqrt_amd import peaks as P
    m = P.measure()
    print("[bench] measured ceilings: %s" % m, file=sys.stderr, flush=True)
    return m


def peaks():
    """Reference points on random N(0,1) data: the vendor BLAS (torch.mm and
    torch._scaled_mm -> hipBLASLt) on an 8192^3 GEMM in bf16 and in E4M3, and a
    device-to-device copy."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    n = 8192
    a = torch.randn((n, n), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    ms, _ = time_gpu(lambda: torch.mm(a, b), 10, 3, torch.cuda.current_stream())
    gemm = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    # the same shape in E4M3 with per-tensor scales (torch._scaled_mm -> hipBLASLt)
    fp8 = None
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.t().contiguous().to(torch.float8_e4m3fn)   # [N, K] row-major = column-major B
        one = torch.ones((), device="cuda", dtype=torch.float32)
        ms8, _ = time_gpu(lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one,
                                                   out_dtype=torch.bfloat16),
                          10, 3, torch.cuda.current_stream())
        fp8 = round(2.0 * n ** 3 / (ms8 * 1e-3) / 1e12, 1)
        del a8, b8
    except (RuntimeError, TypeError, AttributeError) as e:  # not offered by this torch build
        print("[bench] vendor fp8 GEMM unavailable: %s" % str(e)[:120], file=sys.stderr)
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms, _ = time_gpu(lambda: dst.copy_(src), 10, 3, torch.cuda.current_stream())
    copy = 2 * (1 << 30) / (ms * 1e-3) / 1e9
    return dict(vendor_bf16_gemm_8192_tflops=round(gemm, 1),
                vendor_bf16_gemm_frac_of_spec=round(gemm / PEAK_TFLOPS["bf16"], 4),
                vendor_fp8_gemm_8192_tflops=fp8,
                copy_1gib_gbs_read_plus_write=round(copy, 1))


def calibrate_copy():
    """A plain copy of known size for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("[bench] calibration copy: 3 x %d bytes" % (1 << 30), file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family and model numbers
    (a virtualised host may report only the brand) and the logical CPUs seen."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key in ("model name", "cpu family", "model") and key not in info:
                    info[key] = val.strip()
    except OSError:
        return None
    if "model name" not in info:
        return None
    return "%s (family %s, model %s; %d logical CPUs)" % (
        info["model name"], info.get("cpu family", "?"), info.get("model", "?"), os.cpu_count() or 0)


def oracle_runner(lc, inp):
    """run(rows) -> seconds: the oracle's whole layer (float64 FFN) on the listed
    token rows of this workload's inputs, on the threads OpenMP currently gives
    it.  Only the experts the listed rows select are copied to the host (the
    oracle's own routing of those rows decides which)."""
    import numpy as np

    import oracle as O
    from mixture_experts_ffn_sqrt_amd.synth import to_host_bits

    h = to_host_bits(inp["hidden"])
    wr = to_host_bits(inp["w_router"])
    bias = to_host_bits(inp.get("bias"))
    off = to_host_bits(inp.get("logit_offset"))
    s13 = to_host_bits(inp.get("w13_shared"))
    s2 = to_host_bits(inp.get("w2_shared"))
    grp = dict(n_group=lc.n_group, topk_group=lc.topk_group, group_topk=lc.group_topk)
    w13 = [None] * lc.E
    w2 = [None] * lc.E

    def fetch(rows):
        lg = O.logits(h, wr, rows=rows, logit_offset=off).astype(np.float32)
        ids, _, _ = O.route(lg, lc.k, lc.scoring, bias=bias, **grp)
        for e in sorted(set(ids.ravel().tolist())):
            if w13[e] is None:
                w13[e] = to_host_bits(inp["w13"][e])
                w2[e] = to_host_bits(inp["w2"][e])

    def run(rows):
        fetch(rows)
        t0 = time.perf_counter()
        O.layer(h, wr, w13, w2, k=lc.k, scoring=lc.scoring, rows=rows, bias=bias,
                logit_offset=off, w13_shared=s13, w2_shared=s2, **grp)
        return time.perf_counter() - t0

    return run


def cpu_baseline(lc, inp, seconds):
    """The oracle as it stands, on a bounded sample of this workload's tokens (the
    first n rows, n sized from a probe to about `seconds` of work), on all the
    host threads OpenMP gives it, and on one thread for a smaller sample.
    Reported in tokens/s."""
    import numpy as np

    import oracle as O

    threads = O.num_threads()
    run = oracle_runner(lc, inp)
    probe = np.arange(min(threads, lc.T), dtype=np.int32)
    tp = run(probe)
    n = int(min(lc.T, max(len(probe), seconds / max(tp, 1e-4) * len(probe))))
    n = max(len(probe), n // len(probe) * len(probe))
    rows = np.arange(n, dtype=np.int32)
    t = run(rows)
    # one thread: a sample of about a quarter of the time budget
    single = cpu_single_core(lc, inp, 0.25 * seconds, run, tp * threads / len(probe))
    return dict(value=round(len(rows) / t, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample="first %d of %d tokens of %s, full layer per token (float64 FFN), "
                       "%.1f s on %d threads" % (len(rows), lc.T, lc.name, t, threads),
                cpu_model=cpu_model(), single_core=single)


def cpu_single_core(lc, inp, seconds, run=None, per_token=None):
    """The oracle on one host thread, on the first n tokens of the workload (n
    sized to about `seconds` of work from one probe token unless the per-token
    time is given), in tokens/s."""
    import numpy as np

    import oracle as O

    threads = O.num_threads()
    run = run or oracle_runner(lc, inp)
    O.set_num_threads(1)
    try:
        if per_token is None:
            per_token = run(np.arange(1, dtype=np.int32))
        n1 = int(min(lc.T, max(1, seconds / max(per_token, 1e-6))))
        rows1 = np.arange(n1, dtype=np.int32)
        t1 = run(rows1)
        reps = 1
        if n1 == lc.T and t1 < 0.25 * seconds:  # a whole small batch: repeat it
            reps = int(min(1000, seconds / max(t1, 1e-6)))
            t1 = sum(run(rows1) for _ in range(reps))
    finally:
        O.set_num_threads(threads)
    return dict(value=round(reps * n1 / t1, 3), unit="tokens/s", cores=1, kind="oracle",
                sample="first %d of %d tokens of %s%s, %.2f s" % (
                    n1, lc.T, lc.name, " x %d" % reps if reps > 1 else "", t1))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X and this "
              "build has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import mixture_experts_ffn_sqrt_amd as moe
    moe.load_library()

    measured = None if args.no_peaks else measured_ceilings()
    head = run_workload(args.workload, args.steps, args.warmup, not args.no_cpu, args.cpu_seconds,
                        not args.no_fp8, not args.no_mxfp4, measured)
    from mixture_experts_ffn_sqrt_amd.synth import CONFIGS
    lc = CONFIGS[args.workload]
    line = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": lc.dtype,
        "data": "synthetic (seeded N(0,1) hidden, N(0,1/fan_in) weights)",
        "config": {"workload": lc.name, "T": lc.T, "d": lc.d, "E": lc.E, "k": lc.k,
                   "d_ff": lc.d_ff, "n_shared": lc.n_shared, "scoring": lc.scoring,
                   "n_group": lc.n_group, "topk_group": lc.topk_group,
                   "group_topk": lc.group_topk, "zipf_s": lc.zipf_s,
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "grouped_gemm": head["grouped_gemm"],
        "combine": head["combine"],
        "layer": head["layer"],
        "routing": head["routing"],
        "step_ms_p10_p50_p90": head["step_ms_p10_p50_p90"],
        "input_digests": head.get("input_digests"),
        "output_xxh3_128": head.get("output_xxh3_128"),
        "fp8": head.get("fp8"),
        "mxfp4": head.get("mxfp4"),
        "measured_peaks": measured,
    }
    keep = ("ms_per_step", "tokens_per_s", "roofline", "grouped_gemm", "combine", "layer",
            "routing", "step_ms_p10_p50_p90", "hash_pass", "fp8", "mxfp4", "cpu_single_core",
            "output_xxh3_128")
    side = [] if args.side in ("", "none") else [w for w in args.side.split(",")
                                                 if w != args.workload]
    others = {}
    for name in side:
        r = run_workload(name, args.steps, args.warmup, False, 0, not args.no_fp8,
                         not args.no_mxfp4, measured,
                         cpu_single=0.0 if args.no_cpu else SIDE_CPU_SECONDS)
        others[name] = {kk: r.get(kk) for kk in keep if r.get(kk) is not None}
    if others:
        line["workloads"] = others
    if not args.no_cpu:
        # the fp32 toy configuration is a parity case, never timed on the GPU;
        # its oracle time on one thread is the one figure it contributes
        from mixture_experts_ffn_sqrt_amd.synth import make_inputs
        tl = CONFIGS["tiny_fp32"]
        line["cpu_single_core_tiny_fp32"] = cpu_single_core(tl, make_inputs(tl, "cpu"), 0.5)
    if not args.no_peaks:
        line["context"] = peaks()
    if args.calibrate_copy:
        calibrate_copy()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
