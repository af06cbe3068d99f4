"""Pins of the CPU oracle against facts outside itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix:
an invariant, a closed form, a special case that reduces to a library routine
(torch's silu / matmul / autograd, torch's bf16 conversion), brute-force
enumeration, or central finite differences.  The pages print no worked example
of the layer, so no value below is taken from them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O


def _small(**kw):
    base = dict(name="t", T=64, d=32, E=8, k=2, f=24, dtype="bf16", expert_std=0.2)
    base.update(kw)
    return mi.MoEConfig(**base)


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------
def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40]]).astype(np.float32)
    # exact halfway cases: a bf16 value plus half an ulp, both parities of the kept lsb
    base = (rng.integers(0x3F80, 0x4000, 2000).astype(np.uint32) << 16)
    v = np.concatenate([v, (base | 0x8000).view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# P1/P2: counts, offsets, bijection, gate sums
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [
    _small(),
    _small(E=16, k=4, score="sigmoid", n_group=4, topk_group=2, scale=2.5, bias="normal", bias_std=0.01),
    mi.DSV3.with_(T=256),
])
def test_counts_offsets_bijection_gate_sums(cfg):
    inp = mi.make_inputs(cfg, seed=1, experts=False)
    r = O.route(O._np(inp["x"]), O._np(inp["w_router"]), O._np(inp["bias"]), cfg)
    p = O.permutation(r["idx"], cfg.E)
    T, k = cfg.T, cfg.k
    assert int(p["counts"].sum()) == T * k
    assert p["offsets"][0] == 0 and p["offsets"][-1] == T * k
    assert np.all(np.diff(p["offsets"]) == p["counts"])
    rows = np.sort(p["row_id_map"].ravel())
    assert np.array_equal(rows, np.arange(T * k))
    # src_token inverts row_id_map; rows are expert-major, tokens ascending inside an expert
    for t in range(T):
        for j in range(k):
            assert p["src_token"][p["row_id_map"][t, j]] == t
    for e in range(cfg.E):
        seg = p["src_token"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(np.any(r["idx"][seg] == e, axis=1))
    # each token picks k distinct experts
    assert all(len(set(row)) == k for row in r["idx"].tolist())
    gsum = r["gates"].astype(np.float64).sum(axis=1)
    assert np.allclose(gsum, cfg.scale, rtol=k * 2.0 ** -23 * 4, atol=0)


# --------------------------------------------------------------------------
# P3: permute -> identity experts -> unpermute with unit gates = k * x exactly
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k", [2, 8])
def test_permute_identity_unpermute_is_k_times_x(k):
    cfg = _small(E=16, k=k, T=96)
    inp = mi.make_inputs(cfg, seed=3)
    x = O._np(inp["x"])
    r = O.route(x, O._np(inp["w_router"]), None, cfg)
    p = O.permutation(r["idx"], cfg.E)
    Xp = O.permute_rows(x, p["src_token"])
    y = O.combine(Xp, np.ones((cfg.T, k), np.float32), p["row_id_map"], None, "bf16")
    assert np.array_equal(y, k * x)


# --------------------------------------------------------------------------
# P4: k = E with softmax equals the dense gate-weighted mixture
# --------------------------------------------------------------------------
def test_k_equals_E_softmax_is_dense_mixture():
    cfg = _small(E=6, k=6, T=40, f=16)
    inp = mi.make_inputs(cfg, seed=4)
    out = O.layer_forward(inp, cfg, storage="f64")
    x = O._np(inp["x"])
    probs = O.softmax_probs(x @ O._np(inp["w_router"]).T)
    dense = np.zeros_like(x)
    for e in range(cfg.E):            # every expert on every token, no routing machinery
        ye = O.swiglu_ffn_fwd(x, O._np(inp["w13"][e]), O._np(inp["w2"][e]), "f64")["Y"]
        dense += probs[:, e:e + 1] * ye
    assert np.allclose(out["y"], dense, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P5: E = k = 1 is a plain SwiGLU MLP (torch library routines, incl. autograd)
# --------------------------------------------------------------------------
def test_single_expert_is_swiglu_mlp_fwd_and_bwd():
    cfg = _small(E=1, k=1, T=20, d=16, f=12, backward=True)
    inp = mi.make_inputs(cfg, seed=5)
    fwd = O.layer_forward(inp, cfg, storage="f64")
    bwd = O.layer_backward(inp, fwd, cfg, storage="f64")
    x = inp["x"].double().requires_grad_(True)
    w13 = inp["w13"][0].double().requires_grad_(True)
    w2 = inp["w2"][0].double().requires_grad_(True)
    f = cfg.f
    y = torch.nn.functional.silu(x @ w13[:f].T) * (x @ w13[f:].T) @ w2.T
    (y * inp["dy"].double()).sum().backward()
    assert np.allclose(fwd["y"], y.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(bwd["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(bwd["dw13"][0], w13.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(bwd["dw2"][0], w2.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(bwd["dw_router"] == 0)    # a single expert's gate is constant 1


# --------------------------------------------------------------------------
# P6: sharding one SwiGLU MLP of width F into E experts of width F/E (the
# granular-upcycling construction, Figure 42 step 1) with all experts
# selected and unit gates reproduces the dense MLP
# --------------------------------------------------------------------------
@pytest.mark.parametrize("score", ["sigmoid", "softmax"])
def test_sharded_mlp_identity(score):
    E, F, d, T = 4, 32, 16, 24
    rng = np.random.default_rng(6)
    x = rng.standard_normal((T, d))
    wg, wu = rng.standard_normal((F, d)) * 0.3, rng.standard_normal((F, d)) * 0.3
    wd = rng.standard_normal((d, F)) * 0.3
    tx = torch.from_numpy(x)
    dense = (torch.nn.functional.silu(tx @ torch.from_numpy(wg).T) * (tx @ torch.from_numpy(wu).T)
             @ torch.from_numpy(wd).T).numpy()
    fs = F // E
    w13 = np.stack([np.concatenate([wg[e * fs:(e + 1) * fs], wu[e * fs:(e + 1) * fs]]) for e in range(E)])
    # softmax gives gate 1/E to each expert: fold the factor E into the down projection
    gain = 1.0 if score == "sigmoid" else float(E)
    w2 = np.stack([wd[:, e * fs:(e + 1) * fs] * gain for e in range(E)])
    cfg = mi.MoEConfig("shard", T=T, d=d, E=E, k=E, f=fs, score=score,
                       scale=float(E) if score == "sigmoid" else 1.0)
    inp = {"x": x, "w_router": np.zeros((E, d)), "bias": None, "w13": w13, "w2": w2}
    out = O.layer_forward(inp, cfg, storage="f64")
    assert np.allclose(out["gates"], 1.0 if score == "sigmoid" else 1.0 / E)
    assert np.allclose(out["y"], dense, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P7: brute force top-k and group-limited selection on tiny inputs
# --------------------------------------------------------------------------
def _brute_topk(keys, cand, k):
    best, best_set = None, None
    for sub in itertools.combinations(sorted(cand), k):     # lexicographic order
        s = sum(float(keys[i]) for i in sub)
        if best is None or s > best:
            best, best_set = s, sub
    return best_set


@pytest.mark.parametrize("ties", [False, True])
def test_topk_brute_force(ties):
    cfg = mi.MoEConfig("b", T=300, d=8, E=8, k=3, f=8)
    # keys on a dyadic grid are exact in fp32 so subset sums compare exactly
    logits = mi.fixed_logits(cfg.T, cfg.E, seed=7, ties=ties).numpy()
    if not ties:
        logits = np.round(logits * 256) / 256
    idx = O.select_topk(O.selection_keys(logits, cfg), cfg)
    for t in range(cfg.T):
        want = _brute_topk(logits[t], range(cfg.E), cfg.k)
        assert tuple(sorted(idx[t].tolist())) == want
        # order: key descending, equal keys by lower id
        order = sorted(idx[t].tolist(), key=lambda e: (-logits[t, e], e))
        assert idx[t].tolist() == order


@pytest.mark.parametrize("ties", [False, True])
def test_group_limited_brute_force(ties):
    cfg = mi.MoEConfig("g", T=300, d=8, E=16, k=3, f=8, score="sigmoid",
                       n_group=4, topk_group=2)
    keys = mi.fixed_logits(cfg.T, cfg.E, seed=8, ties=ties).numpy()
    keys = np.round(keys * 64) / 64                          # dyadic: sums exact
    # select_topk sees the keys directly (the score transform is pinned elsewhere)
    idx = O.select_topk(keys.astype(np.float32), cfg)
    per = cfg.E // cfg.n_group
    for t in range(cfg.T):
        gs = []
        for g in range(cfg.n_group):
            mem = keys[t, g * per:(g + 1) * per]
            gs.append(max(mem[a] + mem[b] for a, b in itertools.combinations(range(per), 2)))
        best, best_groups = None, None
        for sub in itertools.combinations(range(cfg.n_group), cfg.topk_group):
            s = sum(gs[g] for g in sub)
            if best is None or s > best:
                best, best_groups = s, sub
        cand = [e for g in best_groups for e in range(g * per, (g + 1) * per)]
        assert tuple(sorted(idx[t].tolist())) == _brute_topk(keys[t], cand, cfg.k)


def _rank(v, i):
    """sort key of (value, id) under R27: numbers descending (infinities
    included), then NaN, ties by id"""
    return (1, 0.0, i) if np.isnan(v) else (0, -float(v), i)


def test_nonfinite_keys_rank_last_and_choices_stay_valid():
    """R27: NaN keys rank after every number, a NaN-holding group after every
    numeric group; the choices are always k distinct eligible ids."""
    rng = np.random.default_rng(11)
    for E, k, n_group, topk_group in [(8, 3, 1, 1), (16, 3, 4, 2), (16, 5, 16, 8), (12, 12, 1, 1)]:
        cfg = mi.MoEConfig("nf", T=200, d=8, E=E, k=k, f=8, score="sigmoid", n_group=n_group,
                           topk_group=topk_group)
        keys = np.round(rng.standard_normal((cfg.T, E)) * 8) / 8
        pick = rng.random((cfg.T, E))
        keys[pick < 0.15] = np.nan
        keys[(pick >= 0.15) & (pick < 0.22)] = np.inf
        keys[(pick >= 0.22) & (pick < 0.30)] = -np.inf
        keys[0] = np.nan                                  # a row of NaN only
        keys[1] = -np.inf                                 # a row of -inf only
        keys = keys.astype(np.float32)
        idx = O.select_topk(keys, cfg)
        per = E // n_group
        for t in range(cfg.T):
            if n_group > 1:
                gs = []
                for g in range(n_group):
                    mem = sorted(keys[t, g * per:(g + 1) * per].tolist(), reverse=True)
                    bad = any(np.isnan(m) for m in mem)
                    gs.append(np.nan if bad else (mem[0] + mem[1] if per >= 2 else mem[0]))
                groups = sorted(range(n_group), key=lambda g: _rank(gs[g], g))[:topk_group]
                cand = [e for g in groups for e in range(g * per, (g + 1) * per)]
            else:
                cand = list(range(E))
            want = sorted(cand, key=lambda e: _rank(keys[t, e], e))[:k]
            assert idx[t].tolist() == want, t
            assert len(set(want)) == k and all(0 <= e < E for e in want)
        assert idx[0].tolist() == (list(range(k)) if n_group == 1 else idx[0].tolist())
        assert idx[1].tolist() == (list(range(k)) if n_group == 1 else idx[1].tolist())


def test_sigmoid_score_rounding_and_bias_is_selection_only():
    from scipy.special import expit
    l = mi.fixed_logits(64, 32, seed=9, std=3.0).numpy()
    assert np.array_equal(O.sigmoid_scores(l), expit(l.astype(np.float64)).astype(np.float32))
    cfg = mi.MoEConfig("s", T=64, d=8, E=32, k=4, f=8, score="sigmoid", scale=2.5)
    idx0 = O.select_topk(O.selection_keys(l, cfg), cfg)
    g0 = O.gates_from_selection(l, idx0, cfg)
    # a constant bias shifts every key alike: same selection and same gates
    idx1 = O.select_topk(O.selection_keys(l, cfg, np.full(32, 0.125, np.float32)), cfg)
    assert np.array_equal(idx0, idx1)
    assert np.array_equal(g0, O.gates_from_selection(l, idx1, cfg))


# --------------------------------------------------------------------------
# P8: every gradient against float64 central finite differences
# --------------------------------------------------------------------------
FD_CFGS = [
    mi.MoEConfig("fd_softmax_aux", T=6, d=8, E=4, k=2, f=6, aux_coeff=0.3,
                 backward=True, expert_std=0.5),
    mi.MoEConfig("fd_sigmoid_groups_shared", T=6, d=8, E=8, k=3, f=6, f_shared=4,
                 score="sigmoid", n_group=4, topk_group=2, scale=2.5, bias="normal",
                 bias_std=0.3, backward=True, expert_std=0.5, router_std=0.5),
    mi.MoEConfig("fd_softmax_norenorm", T=6, d=8, E=4, k=2, f=6, renorm=False,
                 backward=True, expert_std=0.5),
]


def _loss(inp, cfg, d_aux):
    fwd = O.layer_forward(inp, cfg, storage="f64")
    L = float(np.sum(fwd["y"] * O._np(inp["dy"])))
    if cfg.aux_coeff:
        L += d_aux * fwd["aux"]
    return L, fwd


def _margin(fwd, cfg, bias):
    """Smallest gap between a selected and an unselected eligible key / group."""
    keys = np.asarray(fwd["keys"], np.float64)
    m = np.inf
    for t in range(keys.shape[0]):
        sel = set(fwd["idx"][t].tolist())
        cand = range(cfg.E)
        if cfg.n_group > 1:
            per = cfg.E // cfg.n_group
            gsc = [np.sort(keys[t, g * per:(g + 1) * per])[-2:].sum() for g in range(cfg.n_group)]
            srt = np.sort(gsc)[::-1]
            m = min(m, srt[cfg.topk_group - 1] - srt[cfg.topk_group])
            kept = O.eligible_groups(keys[t], cfg.n_group, cfg.topk_group)
            cand = [e for g in kept for e in range(g * per, (g + 1) * per)]
        ins = [keys[t, e] for e in cand if e in sel]
        outs = [keys[t, e] for e in cand if e not in sel]
        if outs:
            m = min(m, min(ins) - max(outs))
    return m


@pytest.mark.parametrize("cfg", FD_CFGS, ids=lambda c: c.name)
def test_gradients_match_finite_differences(cfg):
    inp = {k: O._np(v) for k, v in mi.make_inputs(cfg, seed=11).items()}
    d_aux = 0.7
    L0, fwd = _loss(inp, cfg, d_aux)
    h = 1e-6
    # one entry moved by h moves a key by at most ~h*|other operand| (< 5h here)
    assert _margin(fwd, cfg, inp["bias"]) > 20 * h
    g = O.layer_backward(inp, fwd, cfg, d_aux=d_aux, storage="f64")
    rng = np.random.default_rng(0)
    names = [("x", "dx"), ("w_router", "dw_router"), ("w13", "dw13"), ("w2", "dw2")]
    if cfg.f_shared:
        names += [("ws13", "dws13"), ("ws2", "dws2")]
    for pname, gname in names:
        arr = inp[pname]
        for _ in range(12):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[pos]
            arr[pos] = old + h
            lp, _ = _loss(inp, cfg, d_aux)
            arr[pos] = old - h
            lm, _ = _loss(inp, cfg, d_aux)
            arr[pos] = old
            fd = (lp - lm) / (2 * h)
            an = g[gname][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (pname, pos, fd, an)
    if inp["bias"] is not None:       # selection-only bias: zero gradient
        b = inp["bias"]
        b[0] += h
        lp, _ = _loss(inp, cfg, d_aux)
        b[0] -= 2 * h
        lm, _ = _loss(inp, cfg, d_aux)
        b[0] += h
        assert abs(lp - lm) < 1e-12


def test_router_backward_against_autograd_of_gates():
    """d_logits for all three gate rules against torch autograd of the gate
    formulas on a fixed selection (autograd differentiates independently)."""
    rng = np.random.default_rng(12)
    T, E, k = 10, 8, 3
    logits = rng.standard_normal((T, E))
    dg = rng.standard_normal((T, k))
    for cfg in [mi.MoEConfig("a", T=T, d=4, E=E, k=k, f=4),
                mi.MoEConfig("b", T=T, d=4, E=E, k=k, f=4, renorm=False),
                mi.MoEConfig("c", T=T, d=4, E=E, k=k, f=4, score="sigmoid", scale=2.5)]:
        idx = O.select_topk(O.selection_keys(logits, cfg, exact=True), cfg)
        gates = O.gates_from_selection(logits, idx, cfg, exact=True)
        dl = O.router_backward(logits, idx, gates, dg, None, cfg, exact=True)
        tl = torch.from_numpy(logits).requires_grad_(True)
        ti = torch.from_numpy(idx.astype(np.int64))
        if cfg.score == "softmax":
            p = torch.softmax(tl, dim=1)
            sel = torch.gather(p, 1, ti)
            g = sel / sel.sum(1, keepdim=True) if cfg.renorm else sel
        else:
            s = torch.sigmoid(tl)
            sel = torch.gather(s, 1, ti)
            g = 2.5 * sel / sel.sum(1, keepdim=True)
        (g * torch.from_numpy(dg)).sum().backward()
        assert np.allclose(dl, tl.grad.numpy(), rtol=1e-12, atol=1e-13), cfg.name


def test_router_backward_peaked_softmax_fp32_gates():
    """With one selected logit far above the others the renormalised gates
    stored in fp32 round to (1, ~1e-8, ...) and no longer sum to 1; the gate
    derivative must still be that of the gate function (autograd in float64
    from the logits), not of the rounded values."""
    rng = np.random.default_rng(13)
    T, E, k = 6, 16, 3
    logits = rng.standard_normal((T, E))
    logits[np.arange(T), rng.integers(0, E, T)] += 18.0 + np.arange(T)
    dg = rng.standard_normal((T, k))
    cfg = mi.MoEConfig("peak", T=T, d=4, E=E, k=k, f=4, scale=2.5)
    idx = O.select_topk(O.selection_keys(logits, cfg, exact=True), cfg)
    gates32 = O.gates_from_selection(logits.astype(np.float32), idx, cfg).astype(np.float32)
    assert np.any(gates32.astype(np.float64).sum(1) != 2.5)     # the rounded gates do not sum to the scale
    dl = O.router_backward(logits, idx, gates32, dg, None, cfg)
    tl = torch.from_numpy(logits).requires_grad_(True)
    sel = torch.gather(torch.softmax(tl, dim=1), 1, torch.from_numpy(idx.astype(np.int64)))
    (2.5 * sel / sel.sum(1, keepdim=True) * torch.from_numpy(dg)).sum().backward()
    want = tl.grad.numpy()
    # float64 itself keeps ~1e-16 / |result| of relative precision in either
    # form (results down to ~1e-11 here); rounding the gates to fp32 would be off by ~1e-8 absolute
    assert np.allclose(dl, want, rtol=1e-5, atol=1e-22)     # (autograd leaves ~1e-26 off the selection)


# --------------------------------------------------------------------------
# P9: aux-loss closed forms
# --------------------------------------------------------------------------
def test_aux_loss_closed_forms():
    T, E, k, a = 32, 8, 2, 1e-3
    # uniform probabilities (equal logits): L = coeff, whatever the counts
    p = O.softmax_probs(np.zeros((T, E)))
    counts = O.expert_counts(O.select_topk(np.zeros((T, E), np.float32),
                                           mi.MoEConfig("z", T=T, d=1, E=E, k=k, f=1)), E)
    assert counts[0] == T and counts[1] == T           # ties -> lowest ids
    assert math.isclose(O.aux_loss(p, counts, T, k, a), a, rel_tol=1e-15)
    # uniform load f_e = 1/E: L = coeff, whatever the probabilities
    rng = np.random.default_rng(13)
    p = O.softmax_probs(rng.standard_normal((T, E)))
    counts = np.full(E, T * k // E)
    assert math.isclose(O.aux_loss(p, counts, T, k, a), a, rel_tol=1e-12)
