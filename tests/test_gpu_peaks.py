"""The chip-ceiling microbenchmarks (include/moe_peaks.h) on the GPU: the read
stream covers every byte exactly once (each block's XOR equals the XOR of its
chunk computed on the host), and the matrix-core loop returns finite sums."""
import ctypes as C

import numpy as np
import pytest
import torch

from mixture_experts_ffn_sqrt_amd import peaks as P

pytestmark = pytest.mark.gpu


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("blocks, mib", [(64, 64), (8, 4), (1024, 16)])
def test_read_stream_reads_each_chunk_once(blocks, mib):
    L = P.load_library()
    nbytes = mib << 20
    g = torch.Generator(device="cpu").manual_seed(blocks)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = host.to("cuda")
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    rc = L.moe_peaks_read(C.c_void_p(src.data_ptr()), nbytes, blocks, C.c_void_p(out.data_ptr()),
                          _stream())
    assert rc == 0
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32).reshape(blocks, -1)
    expect = np.bitwise_xor.reduce(words, axis=1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), expect)


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_loop_returns_finite_sums(kind):
    L = P.load_library()
    n = L.moe_peaks_operand_bytes()
    g = torch.Generator(device="cuda").manual_seed(3)
    if kind == 0:
        ops = torch.randn(n // 2, generator=g, device="cuda").to(torch.bfloat16)
    else:
        ops = torch.randn(n, generator=g, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8)
    blocks, iters = 8, 64
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.moe_peaks_mfma(kind, C.c_void_p(ops.data_ptr()), blocks, iters,
                          C.c_void_p(out.data_ptr()), _stream())
    assert rc == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all() and np.abs(o).max() > 0
