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
TOL = {"f32": 1e-5, "bf16": 1e-2, "mxfp8": 1e-2, "mxfp4": 1e-2}
# Bound on any single row (last axis) of an output, as a multiple of TOL.  A
# whole-tensor relative L2 lets one wrong element or a small wrong patch of a
# large tensor through; every row is held to twice the tensor bound instead.
# Stored bf16 values differ from the oracle's by at most one rounding step
# (2^-8 relative) plus what a one-step difference in their bf16 inputs carries
# through one product, so a correct row stays near 2^-8.  Along a chain of
# MXFP8 products a one-step bf16 difference upstream can move an e4m3 code by
# one step (2^-3 relative at the bottom of a binade) or a whole 32-value block
# scale by 2x, so a row of a later product may move by several percent while
# the tensor stays within 1e-2.  For MXFP8 layers the rows are therefore held
# to twice the bound only where both sides start from the same bits (the
# router, the permutation, the first expert product and the scaled upstream
# gradient); every other product is checked row by row on the GPU's own inputs
# by mx_stepwise_check below.  Element errors are held to ELEM_FACTOR * TOL of
# the element (or of its row's RMS): a few bf16 rounding steps at most.
ROW_FACTOR = 2.0
ELEM_FACTOR = 4.0
MX_ROW_CHECKED = {"logits", "gates", "x_perm", "act", "hu", "act_s", "hu_s", "dy_perm"}


def shape_of(cfg: mi.MoEConfig) -> LayerShape:
    return LayerShape(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, f=cfg.f, f_shared=cfg.f_shared,
                      score=cfg.score, n_group=cfg.n_group, topk_group=cfg.topk_group,
                      renorm=cfg.renorm, scale=cfg.scale, aux_coeff=cfg.aux_coeff,
                      dtype=cfg.dtype if cfg.dtype in ("f32", "mxfp8", "mxfp4") else "bf16",
                      force_balanced=cfg.force_balanced, fold_gates=cfg.fold_gates,
                      recompute_act=cfg.recompute_act)


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


def row_errors(got, want) -> tuple[float, float]:
    """Worst row and worst element of an output against the oracle, rows along
    the last axis.

    A row's scale is the larger of its own L2 norm and the tensor's RMS row
    norm, so a row whose exact value is tiny through cancellation (a gate
    gradient of two nearly equal experts, say) is judged against a typical row
    rather than against its own near-zero norm.  Returns
      row:  max over rows of ||got_r - want_r|| / scale_r
      elem: max over elements of |got - want| / (|want| + scale_r / sqrt(n)),
            i.e. against the element or, if smaller, the row's RMS -- one
            wrong element of a long row shows here, not in the row norm."""
    want = np.asarray(want, np.float64)
    n = want.shape[-1] if want.ndim else 1
    w = want.reshape(-1, n)
    g = np.asarray(got, np.float64).reshape(-1, n)
    if w.shape[0] == 0:
        return 0.0, 0.0
    norms = np.linalg.norm(w, axis=1)
    scale = np.maximum(norms, np.linalg.norm(w) / np.sqrt(w.shape[0]))
    diff = np.abs(g - w)
    if not np.all(scale > 0):                  # an all-zero tensor: got must be zero too
        return (0.0, 0.0) if not np.any(diff) else (np.inf, np.inf)
    row = float(np.max(np.linalg.norm(diff, axis=1) / scale))
    elem = float(np.max(diff / (np.abs(w) + (scale / np.sqrt(n))[:, None])))
    return row, elem


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
    if cfg.fold_gates:
        pairs += [("row_gates", "row_gates")]
    if cfg.f_shared:
        pairs += SHARED_PAIRS
    if backward:
        pairs += BWD_PAIRS + (SHARED_BWD_PAIRS if cfg.f_shared else [])
    errs, rows, elems = {}, {}, {}
    for gk, ok in pairs:
        got = g[gk].reshape(np.shape(o[ok]))
        errs[gk] = rel_l2(got, o[ok])
        rows[gk], elems[gk] = row_errors(got, o[ok])
    if cfg.aux_coeff:
        errs["aux"] = abs(float(g["aux"][0]) - o["aux"]) / abs(o["aux"])
    print(f"{cfg.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    print(f"{cfg.name} worst row/element: " + " ".join(f"{k}={rows[k]:.1e}/{elems[k]:.1e}" for k in rows),
          flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"relative L2 above {tol}: {bad}"
    checked = lambda k: cfg.dtype not in ("mxfp8", "mxfp4") or k in MX_ROW_CHECKED
    bad = {k: v for k, v in rows.items() if not v <= ROW_FACTOR * tol and checked(k)}
    assert not bad, f"a row's relative L2 above {ROW_FACTOR * tol}: {bad}"
    bad = {k: v for k, v in elems.items() if not v <= ELEM_FACTOR * tol and checked(k)}
    assert not bad, f"an element's error above {ELEM_FACTOR * tol}: {bad}"
    if backward:
        # experts that received no rows get exact zero weight gradients
        empty = np.flatnonzero(np.asarray(o["counts"]) == 0)
        for e in empty:
            assert not np.any(g["dw13"][e]) and not np.any(g["dw2"][e]), f"expert {e} is empty"
    return errs


def mx_stepwise_check(cfg: mi.MoEConfig, inp: dict, g: dict) -> dict:
    """Every MXFP8 / MXFP4 expert product of every expert, row by row, recomputed by the
    oracle from the GPU's own upstream tensors (so both sides quantise the same
    bits): A and H, U from x_perm; Y from act; dH, dU from dy_perm and the
    saved H, U, act; dX from the GPU's dH, dU; the weight gradients over all of
    the expert's rows; the shared expert likewise.  Tensor bound TOL, row bound
    ROW_FACTOR * TOL.  Returns the worst errors.

    Beside each check it also measures what the microscaling itself costs that
    product: the same-quantisation oracle against the product of the same
    (unquantised) bf16 operands, relative L2 over the whole product; the
    table `quant` of the return value (and the printed line) holds the worst
    over the experts."""
    tol = TOL[cfg.dtype]
    f = cfg.f
    fmt = O.mx_format_of(cfg.dtype)
    q = lambda a, axis: O.mx_qdq(a, axis, fmt)
    w13, w2 = inp["w13"], inp["w2"]
    worst, worst_row, quant = {}, {}, {}

    def chk(name, got, want, plain=None):
        e = rel_l2(got, want)
        r, el = row_errors(got, want)
        worst[name] = max(worst.get(name, 0.0), e)
        worst_row[name] = max(worst_row.get(name, 0.0), r, el)
        if plain is not None:
            quant[name] = max(quant.get(name, 0.0), rel_l2(want, plain))
        assert e <= tol and r <= ROW_FACTOR * tol and el <= ELEM_FACTOR * tol, (name, e, r, el)

    def expert(xe, hu, act, dyp, dhu, dxp, dw13, dw2, W13, W2, fe, tag, gate=None):
        o = O.swiglu_ffn_fwd_mx(xe, W13, W2, "bf16", gate=gate, act_from_stored=cfg.recompute_act, fmt=fmt)
        p = O.swiglu_ffn_fwd(xe, W13, W2, "bf16", gate=gate, act_from_stored=cfg.recompute_act)
        chk(tag + "H", hu[:, :fe], o["H"], p["H"])
        chk(tag + "U", hu[:, fe:], o["U"], p["U"])
        chk(tag + "A", act, o["A"])
        H, U = hu[:, :fe], hu[:, fe:]
        b = O.swiglu_ffn_bwd_mx(xe, H, U, act, dyp, W13, W2, "bf16", gate=gate, fmt=fmt)
        pb = O.swiglu_ffn_bwd(xe, H, U, act, dyp, W13, W2, "bf16", gate=gate)
        chk(tag + "dH", dhu[:, :fe], b["dH"], pb["dH"])
        chk(tag + "dU", dhu[:, fe:], b["dU"], pb["dU"])
        n64 = lambda a: np.asarray(a, np.float64)
        chk(tag + "dW2", dw2, O.store(q(dyp, 0).T @ q(act, 0), "bf16"), O.store(n64(dyp).T @ n64(act), "bf16"))
        chk(tag + "dW13", dw13, O.store(q(dhu, 0).T @ q(xe, 0), "bf16"), O.store(n64(dhu).T @ n64(xe), "bf16"))
        if dxp is not None:
            chk(tag + "dX", dxp, O.store(q(dhu, 1) @ q(W13, 0), "bf16"), O.store(n64(dhu) @ n64(W13), "bf16"))
        return o

    off = np.asarray(g["offsets"])
    for e in range(cfg.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        sl = slice(lo, hi)
        W13, W2 = O._np(w13[e]), O._np(w2[e])
        expert(g["x_perm"][sl], g["hu"][sl], g["act"][sl], g["dy_perm"][sl], g["dhu"][sl], g["dx_perm"][sl],
               g["dw13"][e], g["dw2"][e], W13, W2, f, "", gate=g["row_gates"][sl] if cfg.fold_gates else None)
        a = g["act"][sl]
        chk("Y", g["y_perm"][sl], O.store(q(a, 1) @ q(W2, 1).T, "bf16"),
            O.store(np.asarray(a, np.float64) @ np.asarray(W2, np.float64).T, "bf16"))
    if cfg.f_shared:
        x, dy = O._np(inp["x"]), O._np(inp["dy"])
        Ws13, Ws2 = O._np(inp["ws13"]), O._np(inp["ws2"])
        expert(x, g["hu_s"], g["act_s"], dy, g["dhu_s"], None, g["dws13"], g["dws2"], Ws13, Ws2,
               cfg.f_shared, "shared_")
        a = g["act_s"]
        chk("shared_Y", g["y_s"], O.store(q(a, 1) @ q(Ws2, 1).T, "bf16"),
            O.store(np.asarray(a, np.float64) @ np.asarray(Ws2, np.float64).T, "bf16"))
    print(f"{cfg.name} stepwise: " + " ".join(f"{k}={v:.1e}/{worst_row[k]:.1e}" for k, v in worst.items()),
          flush=True)
    print(f"{cfg.name} {fmt} quantisation error per product (same-quantisation oracle vs bf16 operands): "
          + " ".join(f"{k}={v:.2e}" for k, v in quant.items()), flush=True)
    # the rule rounds each operand to 4 (e4m3) or 2 (e2m1) significant bits:
    # an RMS relative error of at most 2^-4/sqrt(3) or 2^-2/sqrt(3) per operand,
    # about sqrt(2) of that on a product of two; bounds with a margin of 1.6
    qb = 1.6 * 2 ** 0.5 * (2.0 ** -4 if fmt == "e4m3" else 2.0 ** -2) / 3 ** 0.5
    assert all(v <= qb for v in quant.values()), (qb, quant)
    return {"worst": worst, "quant": quant}
