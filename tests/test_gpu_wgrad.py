"""Expert weight gradients on chosen expert sizes, through the C ABI.

moe_grouped_gemm_swiglu_bwd takes the expert offsets as an input, so the
expert sizes here are picked by hand rather than by a router: empty experts,
one row, sizes on and off the 64-row slice boundary, on both sides of 192
rows (the band kernel's wide and narrow units), up to 384 rows (the
stationary-band kernel) and beyond (the DMA ring kernel), with output
shapes wide enough (N >= 512 columns) for the band kernel to run.  Every
expert's dW13 and dW2, and dHU, are compared with the oracle's SwiGLU backward
(bf16 storage, rel-L2 1e-2); dW13 is also compared with the oracle's product
of the GPU's own dHU, so that the weight-gradient kernel is checked on its
exact inputs.  Experts without rows must give exact zeros.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from mixture_experts_layer_limited_amd import _abi as abi
from oracle import moe_oracle as O

from harness import host, rel_l2, shape_of

pytestmark = pytest.mark.gpu

TOL = 1e-2

SIZES = {
    "mixed_sizes": [0, 1, 37, 64, 65, 192, 193, 200, 256, 300, 320, 321, 384, 385, 400],
    "random_sizes_e40": [int(v) if v > 20 else 0
                         for v in np.random.default_rng(7).integers(0, 420, size=40)],
}


# (d, f): with d = 768, f = 512 both weight gradients (gate/up 1024 x 768, down
# 768 x 512) are taller than wide and keep the band on their row side; with
# d = 1024, f = 256 the gate/up gradient (512 x 1024) keeps it on its column side
SHAPES = [(768, 512), (1024, 256)]


@pytest.mark.parametrize("d,f", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("name", list(SIZES))
def test_expert_wgrad_parity(name, d, f):
    sizes = np.asarray(SIZES[name], np.int64)
    E, rows = len(sizes), int(sizes.sum())
    print(f"case wgrad {name} E={E} rows={rows} d={d} f={f}", flush=True)
    cfg = mi.MoEConfig(f"wgrad_{name}", T=rows, d=d, E=E, k=1, f=f, dtype="bf16", backward=True)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    g = torch.Generator().manual_seed(11)

    def bf(*shape, std=1.0):
        return (torch.randn(*shape, generator=g) * std).to(torch.bfloat16)

    x_perm, dy_perm = bf(rows, d), bf(rows, d)
    hu, act = bf(rows, 2 * f), bf(rows, f)
    w13, w2 = bf(E, 2 * f, d, std=0.02), bf(E, d, f, std=0.02)

    dev = "cuda"
    c = shape_of(cfg).cfg()
    D = {k: v.to(dev) for k, v in dict(x_perm=x_perm, dy_perm=dy_perm, hu=hu, act=act, w13=w13, w2=w2).items()}
    off = torch.from_numpy(offsets).to(dev)
    dhu = torch.empty(rows, 2 * f, dtype=torch.bfloat16, device=dev)
    dx_perm = torch.empty(rows, d, dtype=torch.bfloat16, device=dev)
    # start from garbage so that unwritten outputs show
    dw13 = torch.full((E, 2 * f, d), 7.0, dtype=torch.bfloat16, device=dev)
    dw2 = torch.full((E, d, f), 7.0, dtype=torch.bfloat16, device=dev)
    dx_partial = torch.empty(rows, d, dtype=torch.float32, device=dev)   # zero-filled by the call
    ws = torch.empty(abi.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    abi.moe_grouped_gemm_swiglu_bwd(c, D["dy_perm"], D["x_perm"], off, None, None, D["hu"], D["act"], D["w13"],
                                    D["w2"], dhu, dx_perm, dw13, dw2, None, None, None, None, None, None, None,
                                    None, dx_partial, None, None, ws)
    torch.cuda.synchronize()

    g_dhu, g_dw13, g_dw2 = host(dhu), host(dw13), host(dw2)
    f64 = lambda t: t.float().double().numpy()
    X, DY, HU, A = f64(x_perm), f64(dy_perm), f64(hu), f64(act)
    W13, W2 = f64(w13), f64(w2)
    worst = {}
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            assert np.all(g_dw13[e] == 0) and np.all(g_dw2[e] == 0), f"expert {e} without rows"
            continue
        o = O.swiglu_ffn_bwd(X[lo:hi], HU[lo:hi, :f], HU[lo:hi, f:], A[lo:hi], DY[lo:hi], W13[e], W2[e], "bf16")
        errs = {
            "dW2": rel_l2(g_dw2[e], o["dW2"]),
            "dHU": rel_l2(g_dhu[lo:hi], np.concatenate([o["dH"], o["dU"]], axis=1)),
            "dW13": rel_l2(g_dw13[e], o["dW13"]),
            "dW13_own_dHU": rel_l2(g_dw13[e], O.store(g_dhu[lo:hi].T @ X[lo:hi], "bf16")),
        }
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
            assert v <= TOL, f"expert {e} ({hi - lo} rows): {k} rel-L2 {v:.3e}"
    print(f"  worst rel-L2: {worst}", flush=True)


def test_shared_expert_dense_wgrad():
    """The shared expert's weight gradients contract over every token.  At T = 1024, d = 7168,
    f_s = 2048 both of them (4096 x 7168 and 7168 x 2048 outputs, 448 and 224 tiles of 256 x 256)
    run on 256 x 256 tiles, one per workgroup; every element of dWs13, dWs2 and dHU_s, and the fp32
    shared dX, is compared with the oracle's SwiGLU backward.  The routed part is one expert
    holding every row, with the identity as the permutation."""
    T, d, fs, f = 1024, 7168, 2048, 256
    print(f"case shared dense wgrad T={T} d={d} fs={fs}", flush=True)
    cfg = mi.MoEConfig("shared_dense_wgrad", T=T, d=d, E=1, k=1, f=f, f_shared=fs, dtype="bf16",
                       backward=True)
    g = torch.Generator().manual_seed(13)

    def bf(*shape, std=1.0):
        return (torch.randn(*shape, generator=g) * std).to(torch.bfloat16)

    x, dy = bf(T, d), bf(T, d)
    hu_s, act_s = bf(T, 2 * fs), bf(T, fs)
    ws13, ws2 = bf(2 * fs, d, std=0.02), bf(d, fs, std=0.02)
    hu, act = bf(T, 2 * f), bf(T, f)
    w13, w2 = bf(1, 2 * f, d, std=0.02), bf(1, d, f, std=0.02)

    dev = "cuda"
    c = shape_of(cfg).cfg()
    D = {k: v.to(dev) for k, v in dict(x=x, dy=dy, hu_s=hu_s, act_s=act_s, ws13=ws13, ws2=ws2,
                                       hu=hu, act=act, w13=w13, w2=w2).items()}
    off = torch.tensor([0, T], dtype=torch.int32, device=dev)
    e = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
    dhu, dx_perm, dw13, dw2 = e(T, 2 * f), e(T, d), e(1, 2 * f, d), e(1, d, f)
    dhu_s = e(T, 2 * fs)
    dws13 = torch.full((2 * fs, d), 7.0, dtype=torch.bfloat16, device=dev)
    dws2 = torch.full((d, fs), 7.0, dtype=torch.bfloat16, device=dev)
    dx_partial = torch.empty(T, d, dtype=torch.float32, device=dev)
    ws = torch.empty(abi.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    abi.moe_grouped_gemm_swiglu_bwd(c, D["dy"], D["x"], off, None, None, D["hu"], D["act"], D["w13"], D["w2"],
                                    dhu, dx_perm, dw13, dw2, None, D["dy"], D["x"], D["hu_s"], D["act_s"],
                                    D["ws13"], D["ws2"], dhu_s, dx_partial, dws13, dws2, ws)
    torch.cuda.synchronize()

    f64 = lambda t: t.float().double().numpy()
    HU = f64(hu_s)
    o = O.swiglu_ffn_bwd(f64(x), HU[:, :fs], HU[:, fs:], f64(act_s), f64(dy), f64(ws13), f64(ws2), "bf16")
    errs = {
        "dWs13": rel_l2(host(dws13), o["dW13"]),
        "dWs2": rel_l2(host(dws2), o["dW2"]),
        "dHU_s": rel_l2(host(dhu_s), np.concatenate([o["dH"], o["dU"]], axis=1)),
        "dX_s": rel_l2(host(dx_partial), o["dX32"]),
    }
    print(f"  rel-L2: {errs}", flush=True)
    for k, v in errs.items():
        assert v <= TOL, f"{k} rel-L2 {v:.3e}"
