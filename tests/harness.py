"""Helpers shared by the GPU parity tests: run the HIP layer through the C ABI
on seeded inputs, run the oracle on the same inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi
from mixture_experts_layer_limited_amd import LayerShape, MoELayer
from oracle import moe_oracle as O

# relative L2 bound for floating outputs (MXFP8: against an oracle applying the
# same quantisation)
TOL = {"f32": 1e-5, "bf16": 1e-2, "mxfp8": 1e-2}


def shape_of(cfg: mi.MoEConfig) -> LayerShape:
    return LayerShape(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, f=cfg.f, f_shared=cfg.f_shared,
                      score=cfg.score, n_group=cfg.n_group, topk_group=cfg.topk_group,
                      renorm=cfg.renorm, scale=cfg.scale, aux_coeff=cfg.aux_coeff,
                      dtype=cfg.dtype if cfg.dtype in ("f32", "mxfp8") else "bf16")


def to_dev(inp: dict, dev="cuda") -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def host(t) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        t = t.float()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    return t.double().numpy()


def run_gpu(cfg: mi.MoEConfig, inp: dict, backward: bool, d_aux: float = 1.0) -> dict:
    dev = to_dev(inp)
    layer = MoELayer(shape_of(cfg), "cuda", backward=backward)
    layer.forward(dev["x"], dev["w_router"], dev["bias"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    if backward:
        layer.backward(dev["dy"], dev["x"], dev["w_router"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"],
                       d_aux=d_aux)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in layer.buf.t.items() if v is not None}


def run_gpu_tensors(cfg: mi.MoEConfig, dev: dict, backward: bool, d_aux: float = 1.0) -> dict:
    """Run the layer on device inputs; return its device buffers (no copies)."""
    layer = MoELayer(shape_of(cfg), "cuda", backward=backward)
    layer.forward(dev["x"], dev["w_router"], dev["bias"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    if backward:
        layer.backward(dev["dy"], dev["x"], dev["w_router"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"],
                       d_aux=d_aux)
    torch.cuda.synchronize()
    return {k: v for k, v in layer.buf.t.items() if v is not None}


def run_oracle(cfg: mi.MoEConfig, inp: dict, backward: bool, d_aux: float = 1.0) -> dict:
    fwd = O.layer_forward(inp, cfg)
    out = dict(fwd)
    out["hu"] = np.concatenate([fwd["H"], fwd["U"]], axis=1)
    if cfg.f_shared:
        out["hu_s"] = np.concatenate([fwd["Hs"], fwd["Us"]], axis=1)
    if backward:
        out.update(O.layer_backward(inp, fwd, cfg, d_aux=d_aux))
    return out


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return float(num)
    return float(num / den)


# GPU buffer name -> oracle name
FWD_PAIRS = [("logits", "logits"), ("gates", "gates"), ("x_perm", "Xp"), ("act", "A"),
             ("y_perm", "Yp"), ("y", "y")]
SHARED_PAIRS = [("act_s", "As"), ("y_s", "Ys")]
BWD_PAIRS = [("hu", "hu"), ("dy_perm", "dYp"), ("d_gates", "d_gates"), ("dhu", "dHU"), ("dx_perm", "dXp"),
             ("dw13", "dw13"), ("dw2", "dw2"), ("d_logits", "d_logits"), ("dw_router", "dw_router"),
             ("dx", "dx")]
SHARED_BWD_PAIRS = [("hu_s", "hu_s"), ("dhu_s", "dHUs"), ("dws13", "dws13"), ("dws2", "dws2")]
EXACT_PAIRS = [("idx", "idx"), ("counts", "counts"), ("offsets", "offsets"), ("row_id_map", "row_id_map"),
               ("src_token", "src_token")]


def compare_layer(cfg: mi.MoEConfig, g: dict, o: dict, backward: bool, tol: float | None = None) -> dict:
    """Assert every output of the layer against the oracle; returns the errors."""
    tol = tol if tol is not None else TOL.get(cfg.dtype, TOL["bf16"])
    for gk, ok in EXACT_PAIRS:
        assert np.array_equal(g[gk].reshape(-1), np.asarray(o[ok]).reshape(-1)), f"{gk} differs"
    pairs = list(FWD_PAIRS)
    if cfg.f_shared:
        pairs += SHARED_PAIRS
    if backward:
        pairs += BWD_PAIRS + (SHARED_BWD_PAIRS if cfg.f_shared else [])
    errs = {}
    for gk, ok in pairs:
        errs[gk] = rel_l2(g[gk].reshape(np.shape(o[ok])), o[ok])
    if cfg.aux_coeff:
        errs["aux"] = abs(float(g["aux"][0]) - o["aux"]) / abs(o["aux"])
    print(f"{cfg.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"relative L2 above {tol}: {bad}"
    if backward:
        # experts that received no rows get exact zero weight gradients
        empty = np.flatnonzero(np.asarray(o["counts"]) == 0)
        for e in empty:
            assert not np.any(g["dw13"][e]) and not np.any(g["dw2"][e]), f"expert {e} is empty"
    return errs
