"""Seeded synthetic inputs for the MoE FFN layer.

This module only draws random numbers: it holds none of the layer's arithmetic.
Both the GPU path and the CPU oracle are fed the same buffers it produces
(tensors on the GPU are copied to the host for the oracle).

Workload shapes follow the pages' model families (Mixtral 8x7B, DeepSeek-V3,
DeepSeek-V4 Flash/Pro); no dataset or trained weight is involved.
  hidden        N(0, 1)                                  [T, d]
  w_router      N(0, 1/d)   (a uniformly random router)  [E, d]
  w13           N(0, 1/d)   rows [0,d_ff) gate, [d_ff,2d_ff) up   [E, 2*d_ff, d]
  w2            N(0, 1/d_ff)                             [E, d, d_ff]
  shared        same laws as one routed expert           [2*d_ff, d], [d, d_ff]
  bias          N(0, sigma^2), sigma = bias_std          [E] float32
  logit_offset  -s * ln(r_e), r a seeded permutation of 1..E (Zipf(s) weights
                put on the logit scale), when zipf_s is set   [E] float32
  token_ids     uniform in [0, vocab)                    [T] int32
  tid2eid       each row k distinct experts, uniform     [vocab, k] int32
bf16 tensors are rounded to nearest-even from float32 draws.
"""
import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

SOFTMAX, SIGMOID, SQRTSOFTPLUS = 0, 1, 2


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    n_shared: int = 0
    dtype: str = "bf16"          # "bf16" or "f32": storage and MFMA input type
    scoring: int = SOFTMAX
    n_group: int = 1
    topk_group: int = 1
    group_topk: int = 0
    bias_std: float = 0.0        # 0 = no selection bias
    zipf_s: float = 0.0          # 0 = no logit offset
    hash_vocab: int = 0          # >0: a hash-routed second pass exists
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "tiny_fp32": LayerConfig(
        "tiny_fp32", T=16, d=64, E=8, k=2, d_ff=128, dtype="f32", scoring=SOFTMAX, seed=1,
        note="tiny layer in float32: top-2 on raw logits, softmax over the pair"),
    "mixtral_prefill": LayerConfig(
        "mixtral_prefill", T=4096, d=4096, E=8, k=2, d_ff=14336, scoring=SOFTMAX, seed=2,
        note="Mixtral-shaped prefill, softmax top-2 renormalised"),
    "dsv3_prefill": LayerConfig(
        "dsv3_prefill", T=8192, d=7168, E=256, k=8, d_ff=2048, n_shared=1, scoring=SIGMOID,
        n_group=8, topk_group=4, group_topk=2, bias_std=0.01, seed=3,
        note="DeepSeek-V3-shaped prefill: sigmoid + bias, 8 groups, top-4 groups, top-8"),
    "v4flash_decode": LayerConfig(
        "v4flash_decode", T=64, d=4096, E=256, k=6, d_ff=2048, n_shared=1,
        scoring=SQRTSOFTPLUS, bias_std=0.01, hash_vocab=129280, seed=4,
        note="DeepSeek-V4-Flash-shaped decode: sqrt(softplus) + bias, top-6; hash pass"),
    "v4pro_skew_prefill": LayerConfig(
        "v4pro_skew_prefill", T=16384, d=7168, E=384, k=6, d_ff=3072, n_shared=1,
        scoring=SQRTSOFTPLUS, bias_std=0.01, zipf_s=1.1, seed=5,
        note="DeepSeek-V4-Pro-shaped prefill with Zipf(1.1)-skewed expert load"),
}

# tensor ids for the per-tensor streams
_HIDDEN, _ROUTER, _W13, _W2, _S13, _S2, _BIAS, _ZIPF, _TOK, _TAB = range(10)


def _gen(cfg_seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * cfg_seed + 7919 * tensor_id + 17)
    return g


def _normal(shape, std, g, device, dtype, out=None):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if out is not None:
        out.copy_(x)
        return out
    return x.to(dtype)


def make_inputs(cfg: LayerConfig, device="cpu", hash_pass: bool = False,
                experts_on_device: bool = True):
    """All inputs of one layer call, seeded by cfg.seed, on `device`.

    Returns a dict of tensors: hidden, w_router, w13, w2, (w13_shared, w2_shared),
    bias, logit_offset, token_ids, tid2eid (None where the workload has none)."""
    dev = torch.device(device)
    dt = cfg.torch_dtype
    s = cfg.seed
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    inp = {}
    inp["hidden"] = _normal((T, d), 1.0, _gen(s, _HIDDEN, dev), dev, dt)
    inp["w_router"] = _normal((E, d), 1.0 / math.sqrt(d), _gen(s, _ROUTER, dev), dev, dt)
    w13 = torch.empty((E, 2 * F, d), device=dev, dtype=dt)
    w2 = torch.empty((E, d, F), device=dev, dtype=dt)
    g13, g2 = _gen(s, _W13, dev), _gen(s, _W2, dev)
    for e in range(E):  # one expert at a time bounds the float32 temporaries
        _normal((2 * F, d), 1.0 / math.sqrt(d), g13, dev, dt, out=w13[e])
        _normal((d, F), 1.0 / math.sqrt(F), g2, dev, dt, out=w2[e])
    inp["w13"], inp["w2"] = w13, w2
    if cfg.n_shared:
        inp["w13_shared"] = _normal((2 * F, d), 1.0 / math.sqrt(d), _gen(s, _S13, dev), dev, dt)
        inp["w2_shared"] = _normal((d, F), 1.0 / math.sqrt(F), _gen(s, _S2, dev), dev, dt)
    else:
        inp["w13_shared"] = inp["w2_shared"] = None
    inp["bias"] = (_normal((E,), cfg.bias_std, _gen(s, _BIAS, dev), dev, torch.float32)
                   if cfg.bias_std > 0 else None)
    if cfg.zipf_s > 0:
        g = _gen(s, _ZIPF, torch.device("cpu"))
        ranks = torch.randperm(E, generator=g).to(torch.float64) + 1.0
        inp["logit_offset"] = (-cfg.zipf_s * torch.log(ranks)).to(torch.float32).to(dev)
    else:
        inp["logit_offset"] = None
    if hash_pass:
        assert cfg.hash_vocab > 0
        V = cfg.hash_vocab
        gt = _gen(s, _TOK, dev)
        inp["token_ids"] = torch.randint(0, V, (T,), generator=gt, device=dev, dtype=torch.int64).to(torch.int32)
        gtab = _gen(s, _TAB, dev)
        keys = torch.rand((V, E), generator=gtab, device=dev)
        inp["tid2eid"] = keys.argsort(dim=1)[:, :k].to(torch.int32).contiguous()
        del keys
    else:
        inp["token_ids"] = inp["tid2eid"] = None
    return inp


def random_logits(T, E, seed, device="cpu", scale=1.0):
    """Seeded float32 logits N(0, scale^2) [T, E], for routing checks from given logits."""
    g = _gen(seed, 99, torch.device(device))
    return torch.randn((T, E), generator=g, device=device, dtype=torch.float32) * scale


def to_host_bits(t: Optional[torch.Tensor]):
    """A tensor as a host numpy array: bf16 as its uint16 bit pattern, others as is."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
