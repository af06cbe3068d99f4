"""Seeded synthetic inputs and layer configurations for the MoE layer.

This module is the only code shared between the HIP path's tests/bench and the
CPU oracle.  It holds shapes, the routing hyper-parameters of each workload and
seeded random tensors -- none of the layer's arithmetic.

Workloads (shapes and value distributions of the pages' model families; the
pages' own training data is not reported, so every tensor is synthetic):

  tiny             T=128  d=64   E=8   k=2  f=128   fp32, softmax+renorm, fwd
  mixtral          T=4096 d=4096 E=8   k=2  f=14336 bf16, softmax+renorm, fwd
  qwen3_235b       T=8192 d=4096 E=128 k=8  f=1536  bf16, softmax+renorm, aux 1e-3, fwd+bwd
  deepseek_v3      T=4096 d=7168 E=256 k=8  f=2048  bf16, sigmoid+bias, 8 groups top-4,
                                                     renorm x2.5, shared f=2048, fwd+bwd
  deepseek_v3_skew same as deepseek_v3, Zipf(1.2) skewed bias, MXFP8 expert GEMMs
                   (deepseek_v3_skew_mxfp4: the same with MXFP4 expert GEMMs;
                   deepseek_v3_skew_bf16: the same routing with bf16 expert GEMMs)

Distributions ("N(0, v)" read as a variance when v is 1/d or 1/fan_in, as a
standard deviation when v is 0.02 or 0.01):
  x ~ N(0,1); router W ~ N(0, 1/d) (tiny/mixtral/qwen3) or std 0.02 (deepseek);
  experts ~ N(0, 1/fan_in) (tiny) or std 0.02; bias std 0.01 (deepseek_v3);
  upstream gradient dy ~ N(0,1).

Every tensor is drawn from its own torch.Generator seeded with
(seed, tensor id[, expert]) so that one expert's weights can be generated
without the others and host and device draws are each reproducible.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

SCORE_SOFTMAX = "softmax"
SCORE_SIGMOID = "sigmoid"


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens (batch x sequence, flattened batch-major)
    d: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    f: int            # routed expert FFN width
    f_shared: int = 0  # shared-expert FFN width (0: none)
    score: str = SCORE_SOFTMAX
    n_group: int = 1
    topk_group: int = 1
    renorm: bool = True
    scale: float = 1.0
    aux_coeff: float = 0.0
    dtype: str = "bf16"        # storage dtype: "f32" | "bf16" | "mxfp8" | "mxfp4"
    backward: bool = False
    router_std: float = 0.0    # 0: 1/sqrt(d)
    expert_std: float = 0.0    # 0: 1/sqrt(fan_in)
    bias: str = "none"         # "none" | "normal" | "zipf"
    bias_std: float = 0.0
    # layer modes (the C ABI's moe_cfg.flags)
    force_balanced: bool = False   # round-robin expert assignment instead of top-k
    fold_gates: bool = False       # gates applied to the SwiGLU output before the down projection
    recompute_act: bool = False    # act formed from the stored H, U and re-formed in the backward

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def rows(self) -> int:
        return self.T * self.k


TINY = MoEConfig("tiny", T=128, d=64, E=8, k=2, f=128, dtype="f32")
MIXTRAL = MoEConfig("mixtral", T=4096, d=4096, E=8, k=2, f=14336,
                    expert_std=0.02)
QWEN3 = MoEConfig("qwen3_235b", T=8192, d=4096, E=128, k=8, f=1536,
                  aux_coeff=1e-3, backward=True, expert_std=0.02)
DSV3 = MoEConfig("deepseek_v3", T=4096, d=7168, E=256, k=8, f=2048, f_shared=2048,
                 score=SCORE_SIGMOID, n_group=8, topk_group=4, scale=2.5,
                 backward=True, router_std=0.02, expert_std=0.02,
                 bias="normal", bias_std=0.01)
DSV3_SKEW = DSV3.with_(name="deepseek_v3_skew_mxfp8", dtype="mxfp8", bias="zipf")
# the same skewed layer with MXFP4 expert GEMMs (e2m1 codes, 1x32 e8m0 scales)
DSV3_SKEW_MX4 = DSV3.with_(name="deepseek_v3_skew_mxfp4", dtype="mxfp4", bias="zipf")
# and with bf16 expert GEMMs: the unquantised layer on the same routing
DSV3_SKEW_BF16 = DSV3.with_(name="deepseek_v3_skew_bf16", bias="zipf")
# one GPU's share of the DeepSeek-V3 layer under 64-way expert parallelism: 4
# local experts of 8192 rows each (every token reaches all four), no shared
# expert; times the expert GEMMs at the per-GPU shape of an EP deployment
DSV3_EP_SHARE = MoEConfig("deepseek_v3_ep_share", T=8192, d=7168, E=4, k=4, f=2048,
                          backward=True, router_std=0.02, expert_std=0.02)

CONFIGS = {c.name: c for c in (TINY, MIXTRAL, QWEN3, DSV3, DSV3_SKEW, DSV3_SKEW_MX4, DSV3_SKEW_BF16,
                                DSV3_EP_SHARE)}

# tensor ids for per-tensor seeding
_TID = {"x": 1, "w_router": 2, "bias": 3, "w13": 4, "w2": 5, "ws13": 6,
        "ws2": 7, "dy": 8, "zipf_perm": 9}


def _gen(seed: int, tid: str, sub: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TID[tid] * 10_007 + sub) & 0x7FFF_FFFF_FFFF)
    return g


def _normal(shape, std, seed, tid, sub, device, dtype):
    g = _gen(seed, tid, sub, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def storage_dtype(cfg: MoEConfig) -> torch.dtype:
    # MXFP8 layers keep bf16 master tensors; the codes are derived from them
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def router_std(cfg: MoEConfig) -> float:
    return cfg.router_std if cfg.router_std > 0 else 1.0 / math.sqrt(cfg.d)


def expert_std(cfg: MoEConfig, fan_in: int) -> float:
    return cfg.expert_std if cfg.expert_std > 0 else 1.0 / math.sqrt(fan_in)


def zipf_bias(cfg: MoEConfig, seed: int, lam: float = 0.07) -> torch.Tensor:
    """Bias b_e = -1.2 * lam * ln(r_e), r_e the 1-based rank of expert e in a
    seeded permutation, so expert popularity falls off like a Zipf(1.2) law."""
    g = _gen(seed, "zipf_perm", 0, "cpu")
    perm = torch.randperm(cfg.E, generator=g)
    rank = torch.empty(cfg.E, dtype=torch.float64)
    rank[perm] = torch.arange(1, cfg.E + 1, dtype=torch.float64)
    return (-1.2 * lam * torch.log(rank)).to(torch.float32)


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu",
                with_grad_inputs: bool | None = None, experts: bool = True) -> dict:
    """All layer inputs for `cfg`, generated on `device`.

    Returns x [T,d], w_router [E,d], bias [E] fp32 or None, w13 [E,2f,d]
    (rows 0..f-1 gate, f..2f-1 up), w2 [E,d,f], ws13 [2fs,d] / ws2 [d,fs] or
    None, and dy [T,d] when a backward pass is wanted.  experts=False skips
    the expert weights (routing-only uses).
    """
    dt = storage_dtype(cfg)
    dev = torch.device(device)
    out = {}
    out["x"] = _normal((cfg.T, cfg.d), 1.0, seed, "x", 0, dev, dt)
    out["w_router"] = _normal((cfg.E, cfg.d), router_std(cfg), seed, "w_router", 0, dev, dt)
    if cfg.bias == "normal":
        out["bias"] = _normal((cfg.E,), cfg.bias_std, seed, "bias", 0, dev, torch.float32)
    elif cfg.bias == "zipf":
        out["bias"] = zipf_bias(cfg, seed).to(dev)
    else:
        out["bias"] = None
    if not experts:
        out["w13"] = out["w2"] = out["ws13"] = out["ws2"] = None
        want_dy = cfg.backward if with_grad_inputs is None else with_grad_inputs
        out["dy"] = _normal((cfg.T, cfg.d), 1.0, seed, "dy", 0, dev, dt) if want_dy else None
        return out
    s13, s2 = expert_std(cfg, cfg.d), expert_std(cfg, cfg.f)
    w13 = torch.empty((cfg.E, 2 * cfg.f, cfg.d), dtype=dt, device=dev)
    w2 = torch.empty((cfg.E, cfg.d, cfg.f), dtype=dt, device=dev)
    for e in range(cfg.E):
        w13[e] = _normal((2 * cfg.f, cfg.d), s13, seed, "w13", e, dev, dt)
        w2[e] = _normal((cfg.d, cfg.f), s2, seed, "w2", e, dev, dt)
    out["w13"], out["w2"] = w13, w2
    if cfg.f_shared > 0:
        out["ws13"] = _normal((2 * cfg.f_shared, cfg.d), expert_std(cfg, cfg.d), seed, "ws13", 0, dev, dt)
        out["ws2"] = _normal((cfg.d, cfg.f_shared), expert_std(cfg, cfg.f_shared), seed, "ws2", 0, dev, dt)
    else:
        out["ws13"] = out["ws2"] = None
    want_dy = cfg.backward if with_grad_inputs is None else with_grad_inputs
    out["dy"] = _normal((cfg.T, cfg.d), 1.0, seed, "dy", 0, dev, dt) if want_dy else None
    return out


def exact_grid_inputs(cfg: MoEConfig, seed: int = 0, device="cpu") -> dict:
    """Inputs whose router logits are exact in fp32 in any summation order.

    x and w_router take values a/8 with integer a in [-8, 8], so every product
    is a multiple of 1/64 with |a*b| <= 64 and every partial sum over d <= 2^17
    terms stays an integer multiple of 1/64 below 2^24/64: fp32 accumulation is
    exact whatever the order, and the routing decision is the same on any
    correct implementation.  Used to make layer-level routing bit-comparable.
    """
    assert cfg.d * 64 < (1 << 24)
    inp = make_inputs(cfg, seed, device)
    dt = storage_dtype(cfg)
    dev = torch.device(device)
    g = _gen(seed, "x", 77, dev)
    inp["x"] = (torch.randint(-8, 9, (cfg.T, cfg.d), generator=g, device=dev).to(torch.float32) / 8).to(dt)
    g = _gen(seed, "w_router", 77, dev)
    inp["w_router"] = (torch.randint(-8, 9, (cfg.E, cfg.d), generator=g, device=dev).to(torch.float32) / 8).to(dt)
    if inp["bias"] is not None:
        # multiples of 2^-10 keep score+bias sums well conditioned
        g = _gen(seed, "bias", 77, dev)
        inp["bias"] = (torch.randint(-64, 65, (cfg.E,), generator=g, device=dev).to(torch.float32) / 1024)
    return inp


def fixed_logits(T: int, E: int, seed: int = 0, device="cpu", std: float = 1.0,
                 ties: bool = False) -> torch.Tensor:
    """fp32 router logits [T,E] for the routing kernels' bit-exact tests.

    With ties=True the values are drawn from a coarse grid so that equal keys
    (and equal group scores) are frequent and the lower-id tie rule is exercised.
    """
    g = _gen(seed, "x", 99, torch.device(device))
    if ties:
        return (torch.randint(-6, 7, (T, E), generator=g, device=device).to(torch.float32) / 4) * std
    return torch.randn((T, E), generator=g, device=device, dtype=torch.float32) * std
