"""Parity at the full workload sizes, in the launch configuration bench.py
times (default kernels), on outputs the oracle can compute one by one.

The layer runs once, forward and backward, on the GPU at full size.  Every
check then feeds the oracle the GPU's own upstream tensors for the sampled
rows (so errors do not compound across steps) and compares:

* router: logits of sampled tokens; selection, gates and the permutation of
  every token, bit-exact from the GPU's fp32 logits;
* permute: the whole x_perm as a bit copy of x;
* experts: every row of sampled experts (H, U, A, Y and dH, dU, dX), sampled
  rows of their weight gradients (each row contracts over all of the expert's
  rows);
* shared expert, combine, combine backward, router backward and dx on sampled
  tokens; sampled rows of dW_router and of the shared weight gradients.

The MXFP8 workload (skewed DeepSeek-V3 routing with empty experts) is checked
against the same oracle steps with MXFP8 GEMM operands.

Tolerances: bf16 storage rel-L2 1e-2 (spec bound; MXFP8 against the
same-quantisation oracle likewise), and 2e-2 on every single row of the
expert products; fp32 outputs 1e-5.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.harness import rel_l2, row_errors, run_gpu_tensors

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
F32_TOL = 1e-5
# every row of a product computed from the GPU's own upstream tensors (both
# sides round and quantise the same bits) stays within twice the tensor bound,
# and every element within 4e-2 of itself or its row's RMS
ROW_TOL = 2e-2
ELEM_TOL = 4e-2


def _h(t) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        t = t.float()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    return t.double().numpy()


def _pick(rng, n, m):
    return np.sort(rng.choice(n, size=min(n, m), replace=False))


def _sample_experts(counts, rng, n=4):
    """The smallest and largest non-empty experts plus random non-empty ones."""
    ok = np.nonzero(counts > 0)[0]
    pick = {int(ok[np.argmin(counts[ok])]), int(ok[np.argmax(counts[ok])])}
    rest = [e for e in ok if e not in pick]
    if rest:
        pick.update(int(e) for e in rng.choice(rest, size=min(len(rest), n - len(pick)), replace=False))
    return sorted(pick)


class _Ops:
    """The oracle's expert arithmetic for one dtype: bf16 GEMMs, or MXFP8 /
    MXFP4 GEMMs whose operands are quantised along each contraction
    (weight-gradient operands along the rows, blocks starting at the expert's
    first row)."""

    def __init__(self, dtype: str):
        self.mx = dtype in ("mxfp8", "mxfp4")
        fmt = O.mx_format_of(dtype) if self.mx else None
        self.fmt = fmt
        if self.mx:
            self.ffn_fwd = lambda *a, **k: O.swiglu_ffn_fwd_mx(*a, fmt=fmt, **k)
            self.ffn_bwd = lambda *a, **k: O.swiglu_ffn_bwd_mx(*a, fmt=fmt, **k)
        else:
            self.ffn_fwd, self.ffn_bwd = O.swiglu_ffn_fwd, O.swiglu_ffn_bwd

    def q(self, a, axis):
        return O.mx_qdq(a, axis, self.fmt) if self.mx else a

    def nt(self, a, w):          # a @ w.T, contraction along both last axes
        return self.q(a, 1) @ self.q(w, 1).T

    def nn(self, a, w):          # a @ w, contraction along a's columns and w's rows
        return self.q(a, 1) @ self.q(w, 0)

    def wgrad_rows(self, p, q, ridx):   # (p^T q)[ridx], contraction over all rows
        return self.q(p, 0)[:, ridx].T @ self.q(q, 0)


FULL = [mi.CONFIGS["deepseek_v3"], mi.CONFIGS["qwen3_235b"], mi.CONFIGS["mixtral"],
        mi.CONFIGS["deepseek_v3_skew_mxfp8"], mi.CONFIGS["deepseek_v3_skew_mxfp4"], mi.CONFIGS["deepseek_v3_ep_share"]]


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_fullsize_sampled_parity(cfg):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[fullsize] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} fs={cfg.f_shared}",
          flush=True)
    rng = np.random.default_rng(1234)
    inp = mi.make_inputs(cfg, seed=0, device="cuda")
    bwd = cfg.backward
    b = run_gpu_tensors(cfg, inp, backward=bwd)
    T, d, E, k, f, fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.f_shared
    st = "bf16"
    ops = _Ops(cfg.dtype)

    # -- router -------------------------------------------------------------
    toks = _pick(rng, T, 48)
    x_s = _h(inp["x"][torch.as_tensor(toks, device="cuda")])
    wr = _h(inp["w_router"])
    want = O.router_logits(x_s, wr)
    assert rel_l2(_h(b["logits"][torch.as_tensor(toks, device="cuda")]), want) < F32_TOL
    logits = b["logits"].cpu().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    keys = O.selection_keys(logits, cfg, bias)
    idx = O.select_topk(keys, cfg)
    np.testing.assert_array_equal(b["idx"].cpu().numpy(), idx)
    gates = O.gates_from_selection(logits, idx, cfg)
    assert rel_l2(b["gates"].cpu().numpy(), gates) < F32_TOL
    counts = O.expert_counts(idx, E)
    np.testing.assert_array_equal(b["counts"].cpu().numpy(), counts)
    perm = O.permutation(idx, E)
    for name in ("offsets", "row_id_map", "src_token"):
        np.testing.assert_array_equal(b[name].cpu().numpy(), perm[name])
    src = torch.as_tensor(perm["src_token"].astype(np.int64), device="cuda")
    assert torch.equal(b["x_perm"], inp["x"][src]), "x_perm is not a bit copy of x"

    if cfg.bias == "zipf":
        # the skewed workload: several experts without tokens, the hottest one
        # above ten times the mean load
        n_empty = int((counts == 0).sum())
        print(f"  skew: {n_empty} empty experts, hottest {counts.max()} rows = "
              f"{counts.max() / counts.mean():.1f} x mean", flush=True)
        assert counts.min() == 0 and n_empty >= 3 and counts.max() > 10 * counts.mean()

    # -- routed experts -----------------------------------------------------
    off = perm["offsets"]
    experts = _sample_experts(counts, rng, n=3 if ops.mx else 4)
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = lo + _pick(rng, hi - lo, 48)                    # row-wise checks
        rt = torch.as_tensor(rows, device="cuda")
        xe = _h(b["x_perm"][rt])
        w13, w2 = _h(inp["w13"][e]), _h(inp["w2"][e])
        o = ops.ffn_fwd(xe, w13, w2, st)
        err, rows_err, elem_err = {}, {}, {}

        def cmp(name, got, want):
            err[name] = rel_l2(got, want)
            rows_err[name], elem_err[name] = row_errors(got, want)

        got_act, got_y = _h(b["act"][rt]), _h(b["y_perm"][rt])
        cmp("A", got_act, o["A"])
        cmp("Y", got_y, O.store(ops.nt(got_act, w2), st))
        if bwd:
            hu = _h(b["hu"][rt])
            cmp("H", hu[:, :f], o["H"])
            cmp("U", hu[:, f:], o["U"])
            ob = ops.ffn_bwd(xe, hu[:, :f], hu[:, f:], got_act, _h(b["dy_perm"][rt]), w13, w2, st)
            dhu = _h(b["dhu"][rt])
            cmp("dH", dhu[:, :f], ob["dH"])
            cmp("dU", dhu[:, f:], ob["dU"])
            cmp("dX", _h(b["dx_perm"][rt]), O.store(ops.nn(dhu, w13), st))   # from the GPU's own dH, dU
            # weight-gradient rows contract over every row of the expert
            sl = slice(lo, hi)
            r13 = _pick(rng, 2 * f, 48)
            r2 = _pick(rng, d, 48)
            w_dw13 = O.store(ops.wgrad_rows(_h(b["dhu"][sl]), _h(b["x_perm"][sl]), r13), st)
            w_dw2 = O.store(ops.wgrad_rows(_h(b["dy_perm"][sl]), _h(b["act"][sl]), r2), st)
            cmp("dW13", _h(b["dw13"][e][torch.as_tensor(r13, device="cuda")]), w_dw13)
            cmp("dW2", _h(b["dw2"][e][torch.as_tensor(r2, device="cuda")]), w_dw2)
        print(f"  expert {e} rows {hi - lo}: " + " ".join(f"{k_}={v:.2e}" for k_, v in err.items()), flush=True)
        print(f"  expert {e} worst row/element: " + " ".join(f"{k_}={rows_err[k_]:.1e}/{elem_err[k_]:.1e}"
                                                         for k_ in rows_err), flush=True)
        for k_, v in err.items():
            assert v < BF16_TOL, (cfg.name, e, k_, v)
        for k_ in rows_err:
            assert rows_err[k_] < ROW_TOL and elem_err[k_] < ELEM_TOL, (cfg.name, e, k_, rows_err[k_], elem_err[k_])
    if bwd:
        # every expert without rows has exact zero weight gradients
        empty = np.nonzero(counts == 0)[0]
        if len(empty):
            et = torch.as_tensor(empty, device="cuda")
            assert int(torch.count_nonzero(b["dw13"][et])) == 0 and int(torch.count_nonzero(b["dw2"][et])) == 0

    # -- shared expert, combine ---------------------------------------------
    tt = torch.as_tensor(toks, device="cuda")
    ys = None
    if fs:
        ws13, ws2 = _h(inp["ws13"]), _h(inp["ws2"])
        o = ops.ffn_fwd(x_s, ws13, ws2, st)
        a_s = _h(b["act_s"][tt])
        assert rel_l2(a_s, o["A"]) < BF16_TOL
        ys = _h(b["y_s"][tt])
        assert rel_l2(ys, O.store(ops.nt(a_s, ws2), st)) < BF16_TOL
    rmap = perm["row_id_map"][toks]
    y_perm_rows = {int(r): _h(b["y_perm"][int(r)]) for r in np.unique(rmap)}
    yp_local = np.stack([y_perm_rows[int(r)] for r in rmap.ravel()]).reshape(len(toks), k, d)
    g_s = b["gates"][tt].cpu().numpy()
    want_y = O.store(sum(g_s[:, j:j + 1].astype(np.float64) * yp_local[:, j] for j in range(k))
                     + (ys if ys is not None else 0.0), st)
    assert rel_l2(_h(b["y"][tt]), want_y) < BF16_TOL

    if not bwd:
        return

    # -- combine backward, router backward, dx --------------------------------
    dy_s = _h(inp["dy"][tt])
    want_dyp = O.store(g_s[:, :, None].astype(np.float64) * dy_s[:, None, :], st)
    got_dyp = np.stack([_h(b["dy_perm"][int(r)]) for r in rmap.ravel()]).reshape(len(toks), k, d)
    assert rel_l2(got_dyp, want_dyp) < BF16_TOL
    want_dg = np.einsum("td,tjd->tj", dy_s, yp_local)
    dg_s = b["d_gates"][tt].cpu().numpy()
    assert rel_l2(dg_s, want_dg) < F32_TOL
    want_dl = O.router_backward(logits[toks], idx[toks], gates[toks], dg_s, counts, cfg)
    if cfg.aux_coeff:
        # the aux term of a token needs the full-batch statistics: recompute them on all tokens
        full = O.router_backward(logits, idx, b["gates"].cpu().numpy(), b["d_gates"].cpu().numpy(), counts, cfg)
        want_dl = full[toks]
    assert rel_l2(b["d_logits"][tt].cpu().numpy(), want_dl) < F32_TOL
    dl_all = b["d_logits"].cpu().numpy().astype(np.float64)
    re_ = _pick(rng, E, 16)
    x_all = _h(inp["x"])
    want_dwr = O.store(dl_all[:, re_].T @ x_all, st)
    assert rel_l2(_h(b["dw_router"][torch.as_tensor(re_, device="cuda")]), want_dwr) < BF16_TOL
    part = dl_all[toks] @ wr
    if fs:
        hus = _h(b["hu_s"][tt])
        obs = ops.ffn_bwd(x_s, hus[:, :fs], hus[:, fs:], _h(b["act_s"][tt]), dy_s, ws13, ws2, st)
        dhus = _h(b["dhu_s"][tt])
        assert rel_l2(dhus[:, :fs], obs["dH"]) < BF16_TOL and rel_l2(dhus[:, fs:], obs["dU"]) < BF16_TOL
        part = part + ops.nn(dhus, ws13)
        dhus_all = _h(b["dhu_s"])
        rs13 = _pick(rng, 2 * fs, 32)
        assert rel_l2(_h(b["dws13"][torch.as_tensor(rs13, device="cuda")]),
                      O.store(ops.wgrad_rows(dhus_all, x_all, rs13), st)) < BF16_TOL
        rs2 = _pick(rng, d, 32)
        assert rel_l2(_h(b["dws2"][torch.as_tensor(rs2, device="cuda")]),
                      O.store(ops.wgrad_rows(_h(inp["dy"]), _h(b["act_s"]), rs2), st)) < BF16_TOL
    got_part = b["dx_partial"][tt].cpu().numpy().astype(np.float64)
    # fp32 sum of the shared dX and the router term (its d_logits enter the GEMM as bf16)
    assert rel_l2(got_part, part) < BF16_TOL
    dxp_local = np.stack([_h(b["dx_perm"][int(r)]) for r in rmap.ravel()]).reshape(len(toks), k, d)
    want_dx = O.store(got_part + dxp_local.sum(axis=1), st)
    assert rel_l2(_h(b["dx"][tt]), want_dx) < BF16_TOL
