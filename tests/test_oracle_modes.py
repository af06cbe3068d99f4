"""Pins of the oracle's layer modes to facts outside them.

* Gate folding (the gate multiplies the SwiGLU output before the linear down
  projection, so the combine sums unweighted rows) and act recomputation (act
  formed from the stored H, U) change only where rounding happens: in exact
  arithmetic ("f64" storage) every output and gradient must equal the standard
  layer's, which the finite-difference pins already fix.
* Force-balanced routing: each token's k choices are distinct, every expert
  gets T k / E rows when E divides T k, gates keep their sums, and where the
  logits make the top-k choice coincide with the round-robin one the two
  routers agree exactly.
* The aux-loss-free bias update moves the selection toward balance: applied
  step after step to a skewed router it shrinks the hottest expert's excess
  load, leaves a balanced load alone, and moves each bias by exactly one step.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O

LAYER_OUTS = ["y"]
GRAD_OUTS = ["dx", "dw13", "dw2", "d_gates", "d_logits", "dw_router"]


def _cfg(**kw):
    base = dict(T=24, d=16, E=8, k=2, f=12, dtype="f32", backward=True, expert_std=0.3)
    base.update(kw)
    return mi.MoEConfig("modes", **base)


def _run(cfg, inp, storage):
    fwd = O.layer_forward(inp, cfg, storage=storage)
    bwd = O.layer_backward(inp, fwd, cfg, d_aux=0.7, storage=storage)
    return fwd, bwd


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


MODE_CASES = [
    _cfg(aux_coeff=1e-2),
    _cfg(score="sigmoid", n_group=4, topk_group=2, scale=2.5, bias="normal", bias_std=0.05, f_shared=8),
    _cfg(renorm=False, k=3),
]


@pytest.mark.parametrize("base", MODE_CASES, ids=["softmax_aux", "sigmoid_groups_shared", "softmax_norenorm"])
@pytest.mark.parametrize("mode", ["fold_gates", "recompute_act", "both"])
def test_modes_equal_the_standard_layer_in_exact_arithmetic(base, mode):
    flags = dict(fold_gates=mode in ("fold_gates", "both"), recompute_act=mode in ("recompute_act", "both"))
    inp = mi.make_inputs(base, seed=3)
    f_std, b_std = _run(base, inp, "f64")
    f_mod, b_mod = _run(base.with_(**flags), inp, "f64")
    np.testing.assert_array_equal(f_mod["idx"], f_std["idx"])
    for k in LAYER_OUTS:
        assert _rel(f_mod[k], f_std[k]) < 1e-12, k
    for k in GRAD_OUTS:
        assert _rel(b_mod[k], b_std[k]) < 1e-12, k
    if flags["fold_gates"]:
        # the folded rows are the unfolded ones times their gates
        g = f_std["row_gates"][:, None]
        assert _rel(f_mod["A"], g * f_std["A"]) < 1e-12 and _rel(f_mod["Yp"], g * f_std["Yp"]) < 1e-12


def test_fold_in_storage_precision_stays_close_and_differs_only_by_rounding():
    """In bf16 storage the folded layer rounds g*act instead of act: the outputs
    move by rounding only (well inside the bf16 tolerance) and not at all in
    exact arithmetic (above)."""
    cfg = _cfg(dtype="bf16", T=64, d=64, E=8, k=2, f=64)
    inp = mi.make_inputs(cfg, seed=4)
    f_std, b_std = _run(cfg, inp, None)
    f_mod, b_mod = _run(cfg.with_(fold_gates=True), inp, None)
    assert 0 < _rel(f_mod["y"], f_std["y"]) < 4e-3
    for k in GRAD_OUTS:
        assert _rel(b_mod[k], b_std[k]) < 1e-2, k


def test_recompute_reforms_the_forward_act_bit_for_bit():
    """With recomputation the forward forms act from the stored H, U, so the
    backward's act (formed again from the same stored values) is the same bits;
    the standard forward forms it from the unrounded H, U."""
    cfg = _cfg(dtype="bf16", T=64, d=64, E=8, k=2, f=64, fold_gates=True, recompute_act=True)
    inp = mi.make_inputs(cfg, seed=5)
    fwd = O.layer_forward(inp, cfg)
    again = O.store(O._act(fwd["H"], fwd["U"], fwd["row_gates"]), "bf16")
    np.testing.assert_array_equal(again, fwd["A"])
    std = O.layer_forward(inp, cfg.with_(recompute_act=False))
    assert np.any(std["A"] != fwd["A"])


# ---------------------------------------------------------------------------
# force-balanced routing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (40, 16, 8), (7, 5, 5), (33, 256, 8)])
def test_balanced_selection_invariants(T, E, k):
    idx = O.select_balanced(T, E, k)
    assert idx.shape == (T, k)
    assert all(len(set(row)) == k for row in idx.tolist())
    c = O.expert_counts(idx, E)
    assert c.sum() == T * k
    if (T * k) % E == 0:
        assert np.all(c == T * k // E)
    else:
        assert c.max() - c.min() == 1
    p = O.permutation(idx, E)
    assert np.array_equal(np.sort(p["row_id_map"].ravel()), np.arange(T * k))


def _identity_router_inputs(T, E, logits):
    """x = the wanted logits, W_r = identity (d = E): the router's logits are x."""
    return {"x": torch.tensor(logits), "w_router": torch.eye(E, dtype=torch.float64), "bias": None}


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_balanced_routing_equals_topk_where_topk_picks_the_same_experts(score):
    T, E, k = 12, 8, 3
    rng = np.random.default_rng(6)
    logits = rng.normal(-3.0, 0.3, (T, E))
    for t in range(T):                                   # the round-robin experts lead, in order
        for j in range(k):
            logits[t, (t * k + j) % E] = 2.0 - 0.5 * j + rng.normal(0, 0.05)
    base = _cfg(T=T, d=E, E=E, k=k, score=score, scale=2.5 if score == "sigmoid" else 1.0)
    inp = _identity_router_inputs(T, E, logits)
    a = O.route(O._np(inp["x"]), O._np(inp["w_router"]), None, base)
    b = O.route(O._np(inp["x"]), O._np(inp["w_router"]), None, base.with_(force_balanced=True))
    np.testing.assert_array_equal(a["idx"], O.select_balanced(T, E, k))
    np.testing.assert_array_equal(b["idx"], a["idx"])
    np.testing.assert_array_equal(b["gates"], a["gates"])


def test_balanced_gates_sum_to_the_scale():
    cfg = _cfg(T=50, d=32, E=16, k=4, score="sigmoid", scale=2.5, force_balanced=True)
    inp = mi.make_inputs(cfg, seed=7)
    r = O.route(O._np(inp["x"]), O._np(inp["w_router"]), None, cfg)
    assert np.allclose(np.asarray(r["gates"], np.float64).sum(axis=1), 2.5, rtol=4 * 2.0 ** -23)
    cfg = cfg.with_(score="softmax", scale=1.0)
    r = O.route(O._np(inp["x"]), O._np(inp["w_router"]), None, cfg)
    assert np.allclose(np.asarray(r["gates"], np.float64).sum(axis=1), 1.0, rtol=4 * 2.0 ** -23)


# ---------------------------------------------------------------------------
# aux-loss-free bias update
# ---------------------------------------------------------------------------
def test_bias_update_moves_each_bias_one_step_toward_balance():
    T, k, E = 16, 2, 8                                    # mean load 4
    counts = np.array([4, 0, 9, 4, 3, 5, 7, 0], np.int32)
    counts[0] += T * k - counts.sum()
    b = np.linspace(-0.1, 0.1, E).astype(np.float32)
    nb = O.bias_update(b, counts, T, k, 1e-3)
    mean = T * k / E
    for e in range(E):
        want = np.float32(b[e] + np.float32(1e-3) * np.float32(np.sign(mean - counts[e])))
        assert nb[e] == want
    assert np.array_equal(O.bias_update(b, np.full(E, T * k // E, np.int32), T, k, 1e-3), b)


def test_bias_update_balances_a_skewed_router():
    """A sigmoid router with a strongly skewed selection bias: repeated updates
    (rate 2e-3, routing recomputed each step on the same tokens) bring the
    hottest expert from several times the mean load to within 50% of it."""
    cfg = _cfg(T=256, d=32, E=16, k=2, score="sigmoid", router_std=0.05, dtype="f32")
    inp = mi.make_inputs(cfg, seed=8, experts=False)
    x, wr = O._np(inp["x"]), O._np(inp["w_router"])
    bias = (-0.05 * np.log(np.arange(1, cfg.E + 1))).astype(np.float32)
    mean = cfg.T * cfg.k / cfg.E
    first = None
    for step in range(120):
        r = O.route(x, wr, bias, cfg)
        c = O.expert_counts(r["idx"], cfg.E)
        if first is None:
            first = c.max() / mean
        bias = O.bias_update(bias, c, cfg.T, cfg.k, 2e-3)
    last = c.max() / mean
    assert first > 2.5 and last < 1.5, (first, last)
