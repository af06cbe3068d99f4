"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/moe.h declares, and rejects bad arguments on the host before
touching a device."""
import ctypes
import os
import re

import pytest
import torch

import mixture_experts_layer_limited_amd as m
from mixture_experts_layer_limited_amd import _abi as abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    names = _declared_symbols()
    assert {"moe_router_topk", "moe_permute", "moe_grouped_gemm_swiglu", "moe_unpermute_combine",
            "moe_unpermute_combine_bwd", "moe_grouped_gemm_swiglu_bwd", "moe_router_topk_bwd",
            "moe_permute_bwd"} <= names
    for n in sorted(names):
        assert hasattr(L, n), f"{n} declared in include/ but not exported"
    # the binding wraps every declared call under the same name
    for n in names:
        assert hasattr(m, n), f"binding lacks {n}"


def test_binding_signatures_match_header():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    decls = dict(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", src))
    abi.lib()
    for name, params in decls.items():
        params = [p.strip() for p in params.split(",") if p.strip() and p.strip() != "void"]
        res, args = abi._SIGS[name]
        assert len(args) == len(params), f"{name}: header has {len(params)} parameters, binding {len(args)}"
        for p, a in zip(params, args):
            if re.match(r"(const\s+)?float\s+\w+$", p):
                assert a is ctypes.c_float, f"{name}: {p}"
            elif "*" in p:
                assert a in (ctypes.c_void_p,) or hasattr(a, "_type_"), f"{name}: {p}"


def test_status_strings():
    assert abi.moe_status_string(0) == "MOE_OK"
    assert abi.moe_status_string(3) == "MOE_ERR_WORKSPACE_TOO_SMALL"
    assert abi.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def test_workspace_size_and_invalid_cfg():
    c = abi.make_cfg(4096, 7168, 256, 8, 2048, 2048, "sigmoid", 8, 4, True, 2.5)
    assert abi.moe_workspace_size(c) >= 4096 * 256 * 2
    bad = abi.make_cfg(16, 64, 8, 9, 128)                  # k > E
    with pytest.raises(abi.MoEError) as ei:
        abi.moe_workspace_size(bad)
    assert "cfg.k" in str(ei.value)


# The calls below pass dummy non-NULL device addresses.  They must fail in
# host-side validation, before any launch; to stay safe even if a validation
# bug let one through, they only run where no GPU is visible.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="dummy pointers: CPU-only test")
FAKE = 0x100000


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(k=9), abi.MOE_ERR_INVALID_ARGUMENT, "cfg.k"),
    (dict(E=300, k=2), abi.MOE_ERR_INVALID_ARGUMENT, "cfg.E"),
    (dict(d=60), abi.MOE_ERR_INVALID_ARGUMENT, "cfg.d"),
    (dict(f=100), abi.MOE_ERR_INVALID_ARGUMENT, "cfg.f"),
    (dict(n_group=3), abi.MOE_ERR_INVALID_ARGUMENT, "n_group"),
    (dict(n_group=4, topk_group=1, k=3), abi.MOE_ERR_INVALID_ARGUMENT, "topk_group"),
    (dict(score="sigmoid", aux_coeff=1e-3), abi.MOE_ERR_UNSUPPORTED, "aux"),
])
def test_router_rejects_bad_cfg(kw, status, needle):
    base = dict(T=16, d=64, E=8, k=2, f=128)
    base.update(kw)
    cfg = abi.make_cfg(**base)
    st = abi.lib().moe_router_topk(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, 1 << 20, None)
    assert st == status
    assert needle in abi.moe_last_error()


@no_gpu
def test_rejects_null_misaligned_and_small_workspace():
    cfg = abi.make_cfg(16, 64, 8, 2, 128)
    L = abi.lib()
    ws = abi.moe_workspace_size(cfg)
    st = L.moe_router_topk(ctypes.byref(cfg), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "logits" in abi.moe_last_error()
    st = L.moe_router_topk(ctypes.byref(cfg), FAKE + 2, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "aligned" in abi.moe_last_error()
    st = L.moe_router_topk(ctypes.byref(cfg), FAKE, None, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "both" in abi.moe_last_error()
    st = L.moe_router_topk(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws - 1, None)
    assert st == abi.MOE_ERR_WORKSPACE_TOO_SMALL
    st = L.moe_permute(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "src_token" in abi.moe_last_error()
    st = L.moe_permute(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "both" in abi.moe_last_error()
    folded = abi.make_cfg(16, 64, 8, 2, 128, fold_gates=True)
    st = L.moe_permute(ctypes.byref(folded), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "topk_gates" in abi.moe_last_error()
    shared = abi.make_cfg(16, 64, 8, 2, 128, f_shared=64)
    st = L.moe_grouped_gemm_swiglu(ctypes.byref(shared), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None,
                                   FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "'x'" in abi.moe_last_error()
    cfg.dtype = 7
    st = L.moe_permute(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None)
    assert st == abi.MOE_ERR_UNSUPPORTED
    cfg.dtype, cfg.flags = abi.MOE_BF16, 8
    st = L.moe_permute(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "flags" in abi.moe_last_error()


@no_gpu
def test_valid_call_without_gpu_reports_device_error():
    cfg = abi.make_cfg(16, 64, 8, 2, 128)
    ws = abi.moe_workspace_size(cfg)
    st = abi.lib().moe_unpermute_combine(ctypes.byref(cfg), FAKE, FAKE, FAKE, None, FAKE, None)
    assert st == abi.MOE_ERR_DEVICE
    assert abi.lib().moe_init(0) == abi.MOE_ERR_DEVICE
    del ws


@no_gpu
@pytest.mark.parametrize("shape", [
    dict(T=65536, d=8192, E=64, k=8, f=2048),          # 524288 rows x 8192 x 2 B = 8 GiB of x_perm
    dict(T=1024, d=16384, E=8, k=2, f=32768),          # one expert's W13: 65536 x 16384 x 2 B
])
def test_gemm_calls_reject_shapes_past_32bit_offsets(shape):
    """The MFMA kernels address each expert's rows and weights with 32-bit
    buffer ranges: shapes whose spans reach 2^31 bytes are rejected on the host."""
    cfg = abi.make_cfg(**shape)
    L = abi.lib()
    st = L.moe_grouped_gemm_swiglu(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None, None,
                                   None, None, None, None, FAKE, 1 << 40, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "32-bit" in abi.moe_last_error()
    st = L.moe_grouped_gemm_swiglu_bwd(ctypes.byref(cfg), FAKE, FAKE, FAKE, None, None, *([FAKE] * 8), None,
                                       *([None] * 7), FAKE, None, None, FAKE, 1 << 40, None)
    assert st == abi.MOE_ERR_INVALID_ARGUMENT and "32-bit" in abi.moe_last_error()
    # the same shape scaled down passes validation and only fails for want of a device
    small = abi.make_cfg(**dict(shape, T=64))
    if 2 * shape["f"] * shape["d"] * 2 < (1 << 31):
        st = L.moe_grouped_gemm_swiglu(ctypes.byref(small), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None,
                                       None, None, None, None, None, FAKE, 1 << 40, None)
        assert st == abi.MOE_ERR_DEVICE


def test_binding_refuses_views_host_tensors_and_wrong_dtypes():
    """The binding passes raw addresses: a strided view, a host tensor or a
    tensor of the wrong element type would be misread, so it is refused."""
    with pytest.raises(ValueError, match="contiguous"):
        abi._ptr(torch.zeros(8, 4).t())
    with pytest.raises(ValueError, match="contiguous"):
        abi._ptr(torch.zeros(8, 8)[:, :4])
    with pytest.raises(ValueError, match="device"):
        abi._ptr(torch.zeros(8))
    assert abi._ptr(None) is None and abi._ptr(1234) == 1234
    cfg = abi.make_cfg(16, 64, 8, 2, 128)
    with pytest.raises(ValueError):
        abi.moe_permute(cfg, torch.zeros(16, 64, dtype=torch.bfloat16).t(), None, None, None, None, None, None,
                        None, None)
