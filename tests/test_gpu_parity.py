"""HIP path vs the CPU oracle, through the C ABI, on seeded inputs.

Integer results (top-k ids, counts, offsets, row maps) are compared bit for
bit; floating outputs and gradients by relative L2 error (1e-5 fp32, 1e-2
bf16) over each whole tensor and, at twice that bound, over every row.  Layer-level cases use inputs on an exact grid (moe_inputs.
exact_grid_inputs) so that the fp32 router logits -- and therefore every routing
decision -- are the same on both sides whatever the summation order.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from mixture_experts_layer_limited_amd import _abi as abi
from oracle import moe_oracle as O

from harness import compare_layer, host, rel_l2, run_gpu, run_oracle, shape_of

pytestmark = pytest.mark.gpu


def _cfg(name, **kw):
    base = dict(T=256, d=128, E=8, k=2, f=128, dtype="bf16", expert_std=0.05)
    base.update(kw)
    return mi.MoEConfig(name, **base)


# ---------------------------------------------------------------------------
# router: identical fp32 logits -> identical choices, counts; gates and aux
# ---------------------------------------------------------------------------
ROUTER_CASES = [
    _cfg("softmax_e8_k2", T=300),
    _cfg("softmax_e128_k8_aux", T=300, E=128, k=8, aux_coeff=1e-3),
    _cfg("sigmoid_e256_groups", T=300, E=256, k=8, score="sigmoid", n_group=8, topk_group=4,
         scale=2.5, bias="normal", bias_std=0.01),
    _cfg("softmax_k_eq_E_norenorm", T=70, E=6, k=6, renorm=False),
    _cfg("sigmoid_one_expert_groups", T=130, E=16, k=3, score="sigmoid", n_group=16, topk_group=4),
    _cfg("softmax_e200_k17", T=65, E=200, k=17),
    # force-balanced routing: (t k + j) mod E whatever the keys; groups and bias ignored
    _cfg("balanced_sigmoid_groups", T=300, E=256, k=8, score="sigmoid", n_group=8, topk_group=4, scale=2.5,
         bias="normal", bias_std=0.01, force_balanced=True),
    _cfg("balanced_softmax_aux", T=77, E=12, k=5, aux_coeff=1e-3, force_balanced=True),
]


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("cfg", ROUTER_CASES, ids=lambda c: c.name)
def test_router_topk_from_logits_bitexact(cfg, ties):
    print(f"case router {cfg.name} ties={ties}", flush=True)
    logits = mi.fixed_logits(cfg.T, cfg.E, seed=5, std=2.0, ties=ties)
    bias = mi.make_inputs(cfg, seed=5, experts=False)["bias"]
    o_keys = O.selection_keys(logits.numpy(), cfg, None if bias is None else bias.numpy())
    o_idx = O.select_balanced(cfg.T, cfg.E, cfg.k) if cfg.force_balanced else O.select_topk(o_keys, cfg)
    o_g = O.gates_from_selection(logits.numpy(), o_idx, cfg)
    o_cnt = O.expert_counts(o_idx, cfg.E)
    c = shape_of(cfg).cfg()
    dev = "cuda"
    L = logits.to(dev)
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    gates = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    cnt = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(abi.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    abi.moe_router_topk(c, None, None, None if bias is None else bias.to(dev), L, idx, gates, cnt,
                        aux if cfg.aux_coeff else None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), o_idx)
    assert np.array_equal(host(cnt), o_cnt)
    assert np.max(np.abs(host(gates) - o_g)) <= 2e-6 * cfg.scale
    if cfg.aux_coeff:
        want = O.aux_loss(O.softmax_probs(logits.numpy()), o_cnt, cfg.T, cfg.k, cfg.aux_coeff)
        assert abs(float(host(aux)[0]) - want) <= 1e-5 * want


NONFINITE_CASES = [ROUTER_CASES[i] for i in (0, 1, 2, 4, 5)]


@pytest.mark.parametrize("cfg", NONFINITE_CASES, ids=lambda c: c.name)
def test_router_topk_nonfinite_logits(cfg):
    """Caller logits holding NaN and infinities: NaN keys rank after every
    number and NaN-holding groups after every numeric group, so the ids stay
    k distinct eligible experts, equal to the oracle's bit for bit."""
    print(f"case router nonfinite {cfg.name}", flush=True)
    logits = mi.fixed_logits(cfg.T, cfg.E, seed=9, std=2.0, ties=True).numpy()
    pick = np.random.default_rng(3).random(logits.shape)
    logits[pick < 0.15] = np.nan
    logits[(pick >= 0.15) & (pick < 0.2)] = np.inf
    logits[(pick >= 0.2) & (pick < 0.26)] = -np.inf
    logits[0] = np.nan
    logits[1] = -np.inf
    logits[2] = np.inf
    bias = mi.make_inputs(cfg, seed=5, experts=False)["bias"]
    o_keys = O.selection_keys(logits, cfg, None if bias is None else bias.numpy())
    o_idx = O.select_topk(o_keys, cfg)
    c = shape_of(cfg).cfg()
    dev = "cuda"
    L = torch.from_numpy(logits).to(dev)
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    gates = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    cnt = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(abi.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    abi.moe_router_topk(c, None, None, None if bias is None else bias.to(dev), L, idx, gates, cnt,
                        aux if cfg.aux_coeff else None, ws)
    torch.cuda.synchronize()
    got = host(idx)
    assert got.min() >= 0 and got.max() < cfg.E
    assert np.array_equal(got, o_idx)
    assert np.array_equal(host(cnt), O.expert_counts(o_idx, cfg.E))


def test_router_zero_tokens_writes_zero_counts_and_aux():
    """T = 0: every count is 0 and the aux loss is exactly 0 (the per-block
    partial sums are empty)."""
    cfg = _cfg("softmax_aux_T0", T=0, E=128, k=8, aux_coeff=1e-3)
    print("case router T=0", flush=True)
    c = shape_of(cfg).cfg()
    dev = "cuda"
    # one-row buffers: the calls want non-NULL pointers, and T = 0 reads none of them
    L = torch.empty(1, cfg.E, dtype=torch.float32, device=dev)
    idx = torch.empty(1, cfg.k, dtype=torch.int32, device=dev)
    gates = torch.empty(1, cfg.k, dtype=torch.float32, device=dev)
    cnt = torch.full((cfg.E,), 7, dtype=torch.int32, device=dev)
    aux = torch.full((1,), 3.0, dtype=torch.float32, device=dev)
    ws = torch.empty(max(abi.moe_workspace_size(c), 1), dtype=torch.uint8, device=dev)
    abi.moe_router_topk(c, None, None, None, L, idx, gates, cnt, aux, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(cnt), np.zeros(cfg.E, np.int32))
    assert float(host(aux)[0]) == 0.0


# ---------------------------------------------------------------------------
# permute: stable counting sort and row gather, bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (1000, 256, 8), (64, 64, 2), (5, 16, 16), (0, 8, 2)])
def test_permute_bitexact(T, E, k):
    print(f"case permute T={T} E={E} k={k}", flush=True)
    cfg = _cfg("perm", T=T, E=E, k=k, d=72)
    logits = mi.fixed_logits(max(T, 1), E, seed=6)[:T]
    o_idx = O.select_topk(O.selection_keys(logits.numpy(), cfg), cfg)
    p = O.permutation(o_idx, E)
    x = mi.make_inputs(cfg.with_(T=max(T, 1)), seed=6, experts=False)["x"][:T]
    c = shape_of(cfg).cfg()
    dev = "cuda"
    n = max(T * k, 1)
    idx = torch.from_numpy(o_idx.astype(np.int32)).to(dev) if T else torch.zeros(1, dtype=torch.int32, device=dev)
    xd = x.to(dev) if T else torch.zeros(1, cfg.d, dtype=torch.bfloat16, device=dev)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    rmap = torch.empty(n, dtype=torch.int32, device=dev)
    src = torch.empty(n, dtype=torch.int32, device=dev)
    xp = torch.empty(n, cfg.d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(abi.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    abi.moe_permute(c, xd, idx, None, off, rmap, src, None, xp, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(off), p["offsets"])
    if T:
        assert np.array_equal(host(rmap).reshape(T, k), p["row_id_map"])
        assert np.array_equal(host(src), p["src_token"])
        assert torch.equal(xp.cpu(), x[torch.from_numpy(p["src_token"].astype(np.int64))])


# ---------------------------------------------------------------------------
# the whole layer, forward (+ backward), every output against the oracle
# ---------------------------------------------------------------------------
LAYER_CASES = [
    # the tiny fp32 workload exactly as specified (normal inputs)
    (mi.TINY, False, False),
    _cfg("f32_sigmoid_groups_shared_bwd", T=160, d=64, E=16, k=4, f=48, f_shared=32, dtype="f32",
         score="sigmoid", n_group=4, topk_group=2, scale=2.5, bias="normal", bias_std=0.05,
         backward=True),
    _cfg("f32_softmax_aux_bwd", T=130, d=32, E=8, k=2, f=40, dtype="f32", aux_coeff=1e-2, backward=True),
    _cfg("f32_softmax_norenorm_bwd", T=96, d=40, E=6, k=3, f=24, dtype="f32", renorm=False, backward=True),
    _cfg("bf16_qwen3_like_bwd", T=300, d=256, E=16, k=4, f=192, aux_coeff=1e-3, backward=True),
    _cfg("bf16_dsv3_like_bwd", T=256, d=384, E=32, k=8, f=256, f_shared=256, score="sigmoid", n_group=8,
         topk_group=4, scale=2.5, bias="normal", bias_std=0.01, backward=True, expert_std=0.02,
         router_std=0.02),
    _cfg("bf16_mostly_empty_experts_bwd", T=40, d=128, E=64, k=2, f=64, backward=True),
    _cfg("bf16_mixtral_like_fwd", T=512, d=512, E=8, k=2, f=512),
    # grids of fewer workgroups than XCDs (the per-XCD tile runs of the
    # persistent kernels then split over G < 8 workgroups)
    _cfg("bf16_two_experts_bwd", T=48, d=64, E=2, k=1, f=64, backward=True),
    _cfg("bf16_one_expert_bwd", T=33, d=64, E=1, k=1, f=64, f_shared=64, backward=True),
    # experts of >= 512 rows on average and a wide dense shared expert: the
    # forward products run on 256-row tiles (with their own tile prefix)
    _cfg("bf16_big_experts_bwd", T=1024, d=128, E=2, k=2, f=256, f_shared=1024, backward=True),
    # a single token: one row per chosen expert, the rest empty; dense shared
    # products over one row
    _cfg("bf16_one_token_bwd", T=1, d=128, E=8, k=2, f=64, aux_coeff=1e-3, backward=True),
    _cfg("bf16_one_token_sigmoid_shared_bwd", T=1, d=128, E=16, k=4, f=64, f_shared=64, score="sigmoid",
         n_group=4, topk_group=2, scale=2.5, bias="normal", bias_std=0.01, backward=True),
    _cfg("f32_one_token_bwd", T=1, d=32, E=4, k=2, f=16, dtype="f32", backward=True),
    # layer modes: gates folded into act (unweighted combine, gate gradient from the
    # experts' backward), act formed again in the backward, force-balanced routing
    _cfg("f32_fold_recompute_sigmoid_shared_bwd", T=160, d=64, E=16, k=4, f=48, f_shared=32, dtype="f32",
         score="sigmoid", n_group=4, topk_group=2, scale=2.5, bias="normal", bias_std=0.05, backward=True,
         fold_gates=True, recompute_act=True),
    _cfg("f32_fold_softmax_aux_bwd", T=130, d=32, E=8, k=2, f=40, dtype="f32", aux_coeff=1e-2, backward=True,
         fold_gates=True),
    _cfg("bf16_fold_dsv3_like_bwd", T=256, d=384, E=32, k=8, f=256, f_shared=256, score="sigmoid", n_group=8,
         topk_group=4, scale=2.5, bias="normal", bias_std=0.01, backward=True, expert_std=0.02,
         router_std=0.02, fold_gates=True),
    _cfg("bf16_recompute_dsv3_like_bwd", T=256, d=384, E=32, k=8, f=256, f_shared=256, score="sigmoid",
         n_group=8, topk_group=4, scale=2.5, bias="normal", bias_std=0.01, backward=True, expert_std=0.02,
         router_std=0.02, recompute_act=True),
    _cfg("bf16_fold_recompute_qwen3_like_bwd", T=300, d=256, E=16, k=4, f=192, aux_coeff=1e-3, backward=True,
         fold_gates=True, recompute_act=True),
    _cfg("bf16_fold_mostly_empty_bwd", T=40, d=128, E=64, k=2, f=64, backward=True, fold_gates=True,
         recompute_act=True),
    _cfg("bf16_fold_big_experts_bwd", T=1024, d=128, E=2, k=2, f=256, f_shared=1024, backward=True,
         fold_gates=True, recompute_act=True),
    _cfg("bf16_fold_one_token_bwd", T=1, d=128, E=8, k=2, f=64, backward=True, fold_gates=True,
         recompute_act=True),
    # d >= 1024: the router logits run split-K (3 and 2 parts of 512) and
    # sum their parts in order
    _cfg("bf16_router_split_k_bwd", T=200, d=1536, E=64, k=4, f=64, score="sigmoid", n_group=8, topk_group=4,
         scale=2.5, bias="normal", bias_std=0.01, backward=True),
    _cfg("bf16_router_split_k_one_token_bwd", T=1, d=1024, E=16, k=2, f=64, aux_coeff=1e-3, backward=True),
    _cfg("bf16_balanced_sigmoid_shared_bwd", T=256, d=256, E=32, k=8, f=128, f_shared=128, score="sigmoid",
         n_group=8, topk_group=4, scale=2.5, bias="normal", bias_std=0.01, backward=True,
         force_balanced=True),
    _cfg("bf16_balanced_fold_recompute_bwd", T=200, d=192, E=10, k=3, f=128, aux_coeff=1e-3, backward=True,
         force_balanced=True, fold_gates=True, recompute_act=True),
]


def _case(c):
    if isinstance(c, tuple):
        return c[0], c[1], c[2]
    return c, c.backward, True


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: _case(c)[0].name)
def test_layer_parity(case):
    cfg, backward, grid = _case(case)
    print(f"case layer {cfg.name} backward={backward}", flush=True)
    inp = mi.exact_grid_inputs(cfg, seed=0) if grid else mi.make_inputs(cfg, seed=0)
    g = run_gpu(cfg, inp, backward, d_aux=0.5)
    o = run_oracle(cfg, inp, backward, d_aux=0.5)
    compare_layer(cfg, g, o, backward)


def test_layer_deterministic():
    cfg = _cfg("det", T=300, d=256, E=16, k=4, f=192, f_shared=64, score="sigmoid", n_group=4,
               topk_group=2, bias="normal", bias_std=0.01, backward=True)
    print("case determinism", flush=True)
    inp = mi.make_inputs(cfg, seed=3)
    a = run_gpu(cfg, inp, True)
    b = run_gpu(cfg, inp, True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_router_bias_update_bitexact():
    """moe_router_bias_update against the oracle's rule, bit for bit, on counts
    below, at and above the mean load."""
    print("case router bias update", flush=True)
    T, k, E = 96, 4, 24                                 # mean load 16
    rng = np.random.default_rng(9)
    counts = rng.integers(0, 40, E).astype(np.int32)
    counts[:3] = 16
    bias = rng.normal(0, 0.05, E).astype(np.float32)
    cfg = abi.make_cfg(T, 64, E, k, 64, score="sigmoid")
    b = torch.from_numpy(bias).cuda()
    abi.moe_router_bias_update(cfg, torch.from_numpy(counts).cuda(), 1e-3, b)
    torch.cuda.synchronize()
    want = O.bias_update(bias, counts, T, k, 1e-3)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert np.array_equal(b.cpu().numpy()[:3], bias[:3])


def test_recompute_reforms_the_forward_act_bit_for_bit():
    """With act recomputation the forward forms act from the stored H, U and the
    backward forms it again into its workspace: the backward's results must be
    the same bits as a backward that reads the forward's act (same kernels
    otherwise), with and without folded gates."""
    from mixture_experts_layer_limited_amd import MoELayer
    from harness import to_dev
    for fold in (False, True):
        cfg = _cfg("recompute_bits", T=300, d=256, E=16, k=4, f=192, f_shared=128, score="sigmoid", n_group=4,
                   topk_group=2, scale=2.5, bias="normal", bias_std=0.01, backward=True, fold_gates=fold,
                   recompute_act=True)
        print(f"case recompute bit-exact fold={fold}", flush=True)
        dev = to_dev(mi.make_inputs(cfg, seed=2))
        layer = MoELayer(shape_of(cfg), "cuda", backward=True)
        layer.forward(dev["x"], dev["w_router"], dev["bias"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
        layer.backward(dev["dy"], dev["x"], dev["w_router"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
        torch.cuda.synchronize()
        got = {k: layer.buf[k].clone() for k in ("dw2", "dws2", "dw13", "dhu", "dx_perm")}
        b = layer.buf
        plain = shape_of(cfg.with_(recompute_act=False)).cfg()
        abi.moe_grouped_gemm_swiglu_bwd(
            plain, b["dy_perm"], b["x_perm"], b["offsets"], b["row_gates"] if fold else None,
            b["row_id_map"] if fold else None, b["hu"], b["act"], dev["w13"], dev["w2"], b["dhu"], b["dx_perm"],
            b["dw13"], b["dw2"], b["d_gates"] if fold else None, dev["dy"], dev["x"], b["hu_s"], b["act_s"],
            dev["ws13"], dev["ws2"], b["dhu_s"], b["dx_partial"], b["dws13"], b["dws2"], layer.ws)
        torch.cuda.synchronize()
        for k, v in got.items():
            assert torch.equal(v, layer.buf[k]), k
