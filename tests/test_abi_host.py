"""Host-side checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch (these
calls never reach the GPU)."""
import ctypes as C
import os
import re

import pytest

import mixture_experts_ffn_sqrt_amd as moe
from mixture_experts_ffn_sqrt_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_entry_points() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.load_library()
    for name in declared_entry_points():
        assert hasattr(L, name), name
    assert moe.moe_strerror(0) == "ok"
    assert "workspace" in moe.moe_strerror(-3)


def cfg(**kw):
    base = dict(T=16, d=64, E=8, k=2, d_ff=128, dtype="f32")
    base.update(kw)
    return moe.make_config(**base)


def ws_status(c):
    n = C.c_size_t(0)
    return moe.load_library().moe_workspace_size(C.byref(c), C.byref(n)), n.value


@pytest.mark.parametrize("kw, status", [
    (dict(), 0),
    (dict(T=0), 0),
    (dict(T=-1), -1),
    (dict(k=9), -1),                       # k > E
    (dict(k=0), -1),
    (dict(E=2000, k=2), -2),               # E > 1024
    (dict(E=32, k=17), -2),                # k > 16
    (dict(d=96), -2),                      # d not a multiple of 64
    (dict(d_ff=100), -2),
    (dict(n_shared=2), -1),
    (dict(dtype=7), None),                 # make_config rejects unknown dtype names
    (dict(scoring=5), -1),
    (dict(route_mode=3), -1),
    (dict(n_group=3), -1),                 # E % n_group
    (dict(n_group=4, topk_group=5, group_topk=1), -1),
    (dict(n_group=4, topk_group=2, group_topk=3), -1),   # group_topk > E/n_group
    (dict(n_group=4, topk_group=1, group_topk=1, k=3), -1),  # k > topk_group*E/n_group
    (dict(n_group=4, topk_group=2, group_topk=2, k=4), 0),
    (dict(route_mode=1, vocab=0), -1),
    (dict(n_group=0), -1),
])
def test_config_validation(kw, status):
    if status is None:
        with pytest.raises(KeyError):
            cfg(**kw)
        return
    st, n = ws_status(cfg(**kw))
    assert st == status
    if st == 0:
        assert n > 0


def test_workspace_size_covers_buffers():
    c = cfg(T=100, d=128, E=8, k=2, d_ff=256, n_shared=1, dtype="bf16")
    _, n = ws_status(c)
    P = 100 * 3
    assert n >= P * 128 * 2 + P * 256 * 2 + 100 * 8 * 4


def test_null_pointers_rejected_before_launch():
    L = moe.load_library()
    c = cfg()
    z = None
    bogus = C.c_void_p(0x1000)  # never dereferenced: every call below fails its checks
    assert L.moe_route(C.byref(c), z, z, z, z, z, z, z, z, z, z) == -1
    assert L.moe_route(C.byref(c), bogus, z, z, z, z, z, bogus, bogus, bogus, z) == -1
    hc = cfg(route_mode=1, vocab=10)
    assert L.moe_route(C.byref(hc), bogus, bogus, z, z, z, z, bogus, bogus, bogus, z) == -1
    assert L.moe_permute(C.byref(c), z, z, z, z, z, z, z, z, 0, z) == -1
    assert L.moe_permute(C.byref(c), *([bogus] * 8), 16, z) == -3  # workspace too small
    assert L.moe_expert_ffn(C.byref(c), z, z, z, z, z, z, z, 0, z) == -1
    assert L.moe_expert_ffn(C.byref(c), *([bogus] * 7), 16, z) == -3
    assert L.moe_combine(C.byref(c), z, z, z, z, z, z) == -1
    args = [bogus] * 2 + [z] * 4 + [bogus] * 2 + [z] * 2 + [bogus] + [z] * 2 + [bogus]
    assert L.moe_forward(C.byref(c), *args, 16, z) == -3
    sc = cfg(n_shared=1)
    assert L.moe_forward(C.byref(sc), *args, 1 << 40, z) == -1  # shared weights missing
    assert L.moe_forward(None, *args, 1 << 40, z) == -1


def test_empty_batch_queues_nothing():
    L = moe.load_library()
    c = cfg(T=0)
    bogus = C.c_void_p(0x1000)
    assert L.moe_route(C.byref(c), bogus, bogus, None, None, None, None, bogus, bogus, bogus,
                       None) == 0
    assert L.moe_combine(C.byref(c), bogus, bogus, bogus, None, bogus, None) == 0


def test_fp8_entry_points_check_on_host():
    L = moe.load_library()
    z = None
    bogus = C.c_void_p(0x1000)
    # quantizers: sizes and dtype first, then pointers
    assert L.moe_quantize_fp8_rows(4, 192, 1, bogus, bogus, bogus, z) == -2   # K % 128
    assert L.moe_quantize_fp8_rows(-1, 128, 1, bogus, bogus, bogus, z) == -1
    assert L.moe_quantize_fp8_rows(4, 128, 7, bogus, bogus, bogus, z) == -1   # dtype
    assert L.moe_quantize_fp8_rows(4, 128, 1, z, bogus, bogus, z) == -1
    assert L.moe_quantize_fp8_rows(0, 128, 1, z, z, z, z) == 0               # nothing to do
    assert L.moe_quantize_fp8_blocks(128, 200, 1, bogus, bogus, bogus, z) == -2
    assert L.moe_quantize_fp8_blocks(128, 128, 0, bogus, z, bogus, z) == -1
    # the FP8 layer needs bf16 activations and d, d_ff multiples of 128
    fwd = [bogus] * 2 + [z] * 4 + [bogus] * 4 + [z] * 4 + [bogus] + [z] * 2 + [bogus]
    c = cfg(d=256, d_ff=256, dtype="bf16")
    assert L.moe_forward_fp8(C.byref(c), *fwd, 16, z) == -3                   # workspace
    assert L.moe_forward_fp8(C.byref(cfg(d=192, d_ff=256, dtype="bf16")), *fwd, 1 << 40, z) == -2
    assert L.moe_forward_fp8(C.byref(cfg(d=256, d_ff=256, dtype="f32")), *fwd, 1 << 40, z) == -2
    assert L.moe_forward_fp8(C.byref(cfg(d=256, d_ff=256, dtype="bf16", n_shared=1)), *fwd,
                             1 << 40, z) == -1
    missing = list(fwd)
    missing[8] = z                                                            # w2q
    assert L.moe_forward_fp8(C.byref(c), *missing, 1 << 40, z) == -1
    assert L.moe_expert_up_fp8(C.byref(c), *([bogus] * 8), z, 1 << 40, z) == -1  # workspace null
    assert L.moe_expert_down_fp8(C.byref(c), *([bogus] * 6), bogus, 16, z) == -3


def test_mxfp4_entry_points_check_on_host():
    L = moe.load_library()
    z = None
    bogus = C.c_void_p(0x1000)
    assert L.moe_quantize_mxfp4(1, 4, 96, 1, bogus, bogus, bogus, z) == -2    # C % 128
    assert L.moe_quantize_mxfp4(1, 5, 128, 1, bogus, bogus, bogus, z) == -2   # odd R
    assert L.moe_quantize_mxfp4(1, -1, 128, 1, bogus, bogus, bogus, z) == -1
    assert L.moe_quantize_mxfp4(-1, 4, 128, 1, bogus, bogus, bogus, z) == -1
    assert L.moe_quantize_mxfp4(1, 4, 128, 5, bogus, bogus, bogus, z) == -1   # dtype
    assert L.moe_quantize_mxfp4(1, 4, 128, 1, bogus, z, bogus, z) == -1
    assert L.moe_quantize_mxfp4(0, 4, 128, 1, z, z, z, z) == 0               # nothing to do
    assert L.moe_quantize_mxfp4(2, 0, 128, 1, z, z, z, z) == 0
    fwd = [bogus] * 2 + [z] * 4 + [bogus] * 4 + [z] * 4 + [bogus] + [z] * 2 + [bogus]
    c = cfg(d=256, d_ff=256, dtype="bf16")
    assert L.moe_forward_mxfp4(C.byref(c), *fwd, 16, z) == -3                 # workspace
    assert L.moe_forward_mxfp4(C.byref(cfg(d=256, d_ff=160, dtype="bf16")), *fwd, 1 << 40, z) == -2
    assert L.moe_forward_mxfp4(C.byref(cfg(d=256, d_ff=256, dtype="f32")), *fwd, 1 << 40, z) == -2
    assert L.moe_forward_mxfp4(C.byref(cfg(d=256, d_ff=256, dtype="bf16", n_shared=1)), *fwd,
                               1 << 40, z) == -1                              # shared missing
    missing = list(fwd)
    missing[7] = z                                                            # w13s
    assert L.moe_forward_mxfp4(C.byref(c), *missing, 1 << 40, z) == -1
    assert L.moe_expert_up_mxfp4(C.byref(c), *([bogus] * 8), z, 1 << 40, z) == -1
    assert L.moe_expert_down_mxfp4(C.byref(c), *([bogus] * 6), bogus, 16, z) == -3


@pytest.mark.parametrize("fn", ["moe_forward_fp8", "moe_forward_mxfp4"])
def test_low_precision_forward_empty_batch(fn):
    """T == 0 returns before any launch (the pointers are never dereferenced)."""
    L = moe.load_library()
    bogus = C.c_void_p(0x1000)
    c = cfg(T=0, d=256, d_ff=256, dtype="bf16")
    args = [bogus] * 2 + [None] * 4 + [bogus] * 4 + [None] * 4 + [bogus] + [None] * 2 + [bogus]
    assert getattr(L, fn)(C.byref(c), *args, 1 << 40, None) == 0
    assert L.moe_expert_up_fp8(C.byref(c), *([bogus] * 8), bogus, 1 << 40, None) == 0
    assert L.moe_expert_down_mxfp4(C.byref(c), *([bogus] * 6), bogus, 1 << 40, None) == 0


def test_peaks_library_exports_every_declared_symbol():
    from mixture_experts_ffn_sqrt_amd import peaks
    text = open(os.path.join(ROOT, "include", "moe_peaks.h")).read()
    declared = sorted(set(re.findall(r"^(?:int|size_t|double)\s*(moe_peaks_\w+)\s*\(", text, re.M)))
    assert declared == sorted(peaks.EXPORTS)
    L = peaks.load_library()
    for name in declared:
        assert hasattr(L, name), name
    assert L.moe_peaks_operand_bytes() == 16 << 20
    assert L.moe_peaks_mfma_flops(0, 1, 4) == 2.0 * 32 * 32 * 16 * 8 * 4 * 4


def test_peaks_reject_bad_arguments_on_the_host():
    from mixture_experts_ffn_sqrt_amd import peaks
    L = peaks.load_library()
    p = C.c_void_p(16)  # never dereferenced: every call below fails its host checks
    assert L.moe_peaks_mfma(2, p, 1, 4, p, None) == -1      # unknown kind
    assert L.moe_peaks_mfma(0, p, 1, 6, p, None) == -1      # iters not a multiple of 4
    assert L.moe_peaks_mfma(0, None, 1, 4, p, None) == -1
    assert L.moe_peaks_read(p, 4095, 1, p, None) == -1      # not a multiple of 4096
    assert L.moe_peaks_read(p, 4096, 0, p, None) == -1
    assert L.moe_peaks_read(p, 3 * 4096, 2, p, None) == -1  # chunks not whole 4 KB blocks


def test_noalloc_rejects_on_the_host():
    """moe_forward_noalloc: argument errors and a workspace beyond its static
    scratch are reported before any launch (no GPU is touched here)."""
    L = moe.load_library()
    p = C.c_void_p(16)  # never dereferenced
    args = [p] * 13 + [None]
    big = cfg(T=4096, d=4096, E=8, k=2, d_ff=14336, dtype="bf16")
    assert L.moe_forward_noalloc(C.byref(big), *args) == B.MOE_ERR_TOO_LARGE
    n = C.c_size_t(0)
    assert L.moe_workspace_size(C.byref(big), C.byref(n)) == 0 and n.value > B.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(C.byref(cfg(k=9)), *args) == -1
    assert L.moe_forward_noalloc(C.byref(cfg(d=96)), *args) == -2
    assert L.moe_forward_noalloc(C.byref(cfg(T=0)), *args) == 0  # nothing to do, nothing queued
    assert "scratch" in moe.moe_strerror(B.MOE_ERR_TOO_LARGE)
