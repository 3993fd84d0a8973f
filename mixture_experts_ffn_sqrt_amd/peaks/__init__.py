"""Chip-ceiling microbenchmarks: a thin binding of libmoe_peaks.so
(include/moe_peaks.h) and their measurement with HIP events on the launch
stream.  Not part of the MoE layer; the benchmark reports the layer's kernels
against these measured ceilings beside the published peaks.

    python -m mixture_experts_ffn_sqrt_amd.peaks     (prints one JSON line)
"""
import ctypes as C
import json
import os

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(HERE, "libmoe_peaks.so")
EXPORTS = ("moe_peaks_operand_bytes", "moe_peaks_mfma_flops", "moe_peaks_mfma", "moe_peaks_read")

_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe_peaks.so is not built (%s); run `python -m "
                           "mixture_experts_ffn_sqrt_amd.build`" % path)
    L = C.CDLL(path)
    P, I = C.c_void_p, C.c_int
    L.moe_peaks_operand_bytes.argtypes = []
    L.moe_peaks_operand_bytes.restype = C.c_size_t
    L.moe_peaks_mfma_flops.argtypes = [I, I, I]
    L.moe_peaks_mfma_flops.restype = C.c_double
    L.moe_peaks_mfma.argtypes = [I, P, I, I, P, P]
    L.moe_peaks_mfma.restype = I
    L.moe_peaks_read.argtypes = [P, C.c_size_t, I, P, P]
    L.moe_peaks_read.restype = I
    _lib = L
    return L


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _timed(fn, reps):
    """Mean ms of `reps` calls after one warm-up, HIP events on the current stream."""
    import torch
    fn()
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def mfma_tflops(kind, cus=256, iters=32768, reps=3):
    """Matrix-core rate (TFLOP/s) on random operands: kind 0 bf16 32x32x16,
    kind 1 E4M3 32x32x64; four 256-thread blocks per CU."""
    import torch
    L = load_library()
    g = torch.Generator(device="cuda").manual_seed(7)
    n = L.moe_peaks_operand_bytes()
    if kind == 0:
        ops = torch.randn(n // 2, generator=g, device="cuda").to(torch.bfloat16)
    else:
        ops = torch.randn(n, generator=g, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8)
    blocks = 4 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def run():
        rc = L.moe_peaks_mfma(kind, C.c_void_p(ops.data_ptr()), blocks, iters,
                              C.c_void_p(out.data_ptr()), _stream())
        if rc:
            raise RuntimeError("moe_peaks_mfma failed (%d)" % rc)

    ms = _timed(run, reps)
    return L.moe_peaks_mfma_flops(kind, blocks, iters) / (ms * 1e-3) / 1e12


def read_gbs(gib=4, blocks=256 * 4, reps=5):
    """HBM read-stream rate (GB/s) over a `gib` GiB buffer (16 times the
    Infinity Cache)."""
    import torch
    L = load_library()
    nbytes = gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    out = torch.empty(blocks, dtype=torch.int32, device="cuda")

    def run():
        rc = L.moe_peaks_read(C.c_void_p(src.data_ptr()), nbytes, blocks,
                              C.c_void_p(out.data_ptr()), _stream())
        if rc:
            raise RuntimeError("moe_peaks_read failed (%d)" % rc)

    ms = _timed(run, reps)
    return nbytes / (ms * 1e-3) / 1e9


def measure():
    """Measured ceilings of this chip: bf16 and E4M3 matrix-core rates on random
    operands, HBM read stream."""
    return dict(mfma_bf16_random_tflops=round(mfma_tflops(0), 1),
                mfma_fp8_random_tflops=round(mfma_tflops(1), 1),
                hbm_read_stream_gbs=round(read_gbs(), 1))


if __name__ == "__main__":
    print(json.dumps(measure()))
