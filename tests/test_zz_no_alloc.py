"""moe_forward_noalloc (the library's static device scratch as the workspace)
against moe_forward (a caller workspace), through the C ABI: outputs, ids and
gates bitwise equal, on two calls in a row, the second with a smaller batch;
and a configuration beyond the scratch rejected before any launch."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_sqrt_amd as moe
from mixture_experts_ffn_sqrt_amd.synth import CONFIGS, make_inputs

import parity_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield
    torch.cuda.synchronize()


def run_noalloc(c, inp):
    out = torch.empty((c.T, c.d), dtype=c.torch_dtype, device="cuda")
    ids = torch.empty((c.T, c.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((c.T, c.k), dtype=torch.float32, device="cuda")
    moe.moe_forward_noalloc(c, inp["hidden"], inp["w_router"], inp.get("logit_offset"),
                            inp.get("bias"), inp.get("token_ids"), inp.get("tid2eid"), inp["w13"],
                            inp["w2"], inp.get("w13_shared"), inp.get("w2_shared"), out, ids, gates)
    torch.cuda.synchronize()
    return out, ids, gates


@pytest.mark.parametrize("big, small", [
    # the decode workload at its full size (T = 64), then 9 tokens
    (CONFIGS["v4flash_decode"], CONFIGS["v4flash_decode"].with_(T=9)),
    # grouped sigmoid routing with a shared expert, 288-row prefill tiles, then 33 tokens
    (CONFIGS["dsv3_prefill"].with_(T=700, d=512, E=16, k=4, d_ff=256, n_group=4, topk_group=2,
                                   group_topk=2),
     CONFIGS["dsv3_prefill"].with_(T=33, d=512, E=16, k=4, d_ff=256, n_group=4, topk_group=2,
                                   group_topk=2)),
])
def test_noalloc_equals_forward_two_calls(big, small):
    for lc in (big, small):
        c = H.cfg_of(lc)
        n = moe.moe_workspace_size(c)
        assert n <= moe.binding.MOE_NOALLOC_SCRATCH_BYTES, n
        inp = make_inputs(lc, "cuda")
        ref = [t.clone() for t in H.gpu_forward(c, inp)]
        got = run_noalloc(c, inp)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), lc
    # and the first shape again after the smaller one: the scratch keeps the
    # last call's contents, and nothing in it needs clearing
    c = H.cfg_of(big)
    inp = make_inputs(big, "cuda")
    ref = [t.clone() for t in H.gpu_forward(c, inp)]
    for a, b in zip(run_noalloc(c, inp), ref):
        assert torch.equal(a, b)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    lc = CONFIGS["mixtral_prefill"]
    c = H.cfg_of(lc)
    assert moe.moe_workspace_size(c) > moe.binding.MOE_NOALLOC_SCRATCH_BYTES
    # never read: the call is rejected on the host before any launch
    inp = {"hidden": torch.empty((lc.T, lc.d), dtype=torch.bfloat16, device="cuda"),
           "w_router": torch.empty((lc.E, lc.d), dtype=torch.bfloat16, device="cuda"),
           "w13": torch.empty((lc.E, 2 * lc.d_ff, lc.d), dtype=torch.bfloat16, device="cuda"),
           "w2": torch.empty((lc.E, lc.d, lc.d_ff), dtype=torch.bfloat16, device="cuda")}
    with pytest.raises(moe.MoeError) as ei:
        run_noalloc(c, inp)
    assert ei.value.status == moe.binding.MOE_ERR_TOO_LARGE
