"""One MoE layer's forward and backward driven through libmoe_gfx950.

This module only allocates device buffers (torch) and sequences the C calls:
Route (moe_router_topk) -> Dispatch (moe_permute) -> Compute
(moe_grouped_gemm_swiglu) -> Combine (moe_unpermute_combine), and the
backward counterparts in reverse.  Every number is produced by the HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _abi as abi


@dataclass
class LayerShape:
    T: int
    d: int
    E: int
    k: int
    f: int
    f_shared: int = 0
    score: str = "softmax"
    n_group: int = 1
    topk_group: int = 1
    renorm: bool = True
    scale: float = 1.0
    aux_coeff: float = 0.0
    dtype: str = "bf16"
    force_balanced: bool = False   # round-robin expert assignment (moe_cfg.flags)
    fold_gates: bool = False       # gates applied to act before the down projection
    recompute_act: bool = False    # the backward forms act again from the saved H, U

    def cfg(self) -> abi.moe_cfg:
        return abi.make_cfg(self.T, self.d, self.E, self.k, self.f, self.f_shared, self.score,
                            self.n_group, self.topk_group, self.renorm, self.scale,
                            self.aux_coeff, self.dtype, self.force_balanced, self.fold_gates,
                            self.recompute_act)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


@dataclass
class Buffers:
    """Every tensor the layer reads or writes, allocated once and reused."""
    t: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.t[k]

    def get(self, k):
        return self.t.get(k)


class MoELayer:
    def __init__(self, shape: LayerShape, device="cuda", backward: bool = True):
        self.s = shape
        self.cfg = shape.cfg()
        self.device = torch.device(device)
        self.backward_enabled = backward
        abi.moe_init(self.device.index or 0)
        self.ws = torch.empty(abi.moe_workspace_size(self.cfg), dtype=torch.uint8, device=self.device)
        self.buf = self._alloc()

    def _alloc(self) -> Buffers:
        s, dev, dt = self.s, self.device, self.s.torch_dtype
        rows = s.T * s.k
        e = lambda *shape, dtype=dt: torch.empty(shape, dtype=dtype, device=dev)
        b = {
            "logits": e(s.T, s.E, dtype=torch.float32),
            "idx": e(s.T, s.k, dtype=torch.int32),
            "gates": e(s.T, s.k, dtype=torch.float32),
            "counts": e(s.E, dtype=torch.int32),
            "aux": e(1, dtype=torch.float32) if s.aux_coeff else None,
            "offsets": e(s.E + 1, dtype=torch.int32),
            "row_id_map": e(s.T, s.k, dtype=torch.int32),
            "src_token": e(rows, dtype=torch.int32),
            "row_gates": e(rows, dtype=torch.float32) if s.fold_gates else None,
            "x_perm": e(rows, s.d),
            "hu": e(rows, 2 * s.f) if self.backward_enabled else None,
            "act": e(rows, s.f),
            "y_perm": e(rows, s.d),
            "y": e(s.T, s.d),
        }
        if s.f_shared:
            b.update({"hu_s": e(s.T, 2 * s.f_shared) if self.backward_enabled else None,
                      "act_s": e(s.T, s.f_shared), "y_s": e(s.T, s.d)})
        if self.backward_enabled:
            b.update({
                "dy_perm": e(rows, s.d), "d_gates": e(s.T, s.k, dtype=torch.float32),
                "dhu": e(rows, 2 * s.f), "dx_perm": e(rows, s.d),
                "dw13": e(s.E, 2 * s.f, s.d), "dw2": e(s.E, s.d, s.f),
                "dx_partial": e(s.T, s.d, dtype=torch.float32),
                "d_logits": e(s.T, s.E, dtype=torch.float32),
                "dw_router": e(s.E, s.d), "dx": e(s.T, s.d),
            })
            if s.f_shared:
                b.update({"dhu_s": e(s.T, 2 * s.f_shared), "dws13": e(2 * s.f_shared, s.d),
                          "dws2": e(s.d, s.f_shared)})
        return Buffers(b)

    # -- forward ------------------------------------------------------------
    def route(self, x, w_router, bias, stream=None):
        b = self.buf
        abi.moe_router_topk(self.cfg, x, w_router, bias, b["logits"], b["idx"], b["gates"], b["counts"],
                            b["aux"] if self.s.aux_coeff else None, self.ws, stream)

    def permute(self, x, stream=None):
        b = self.buf
        fold = self.s.fold_gates
        abi.moe_permute(self.cfg, x, b["idx"], b["gates"] if fold else None, b["offsets"], b["row_id_map"],
                        b["src_token"], b.get("row_gates"), b["x_perm"], self.ws, stream)

    # -- MXFP8 / MXFP4 weights ----------------------------------------------
    @staticmethod
    def _mx_source_key(*ws):
        """Identity of the bf16 weights the quantised copies were made from:
        each tensor's address, shape and torch's in-place version counter
        (shared by all views of a storage).  The layer also holds references to
        those tensors (mx_sources), so their memory cannot be freed and handed
        to other tensors while the copies exist: an equal address is the same
        memory, and an in-place update (e.g. an optimizer step) bumps the
        version.  Writes that bypass the version counter (through .data or a raw
        pointer) are not seen: call prepare_mx_weights after those."""
        return tuple(None if w is None else (w.data_ptr(), w._version, tuple(w.shape), tuple(w.stride()))
                     for w in ws)

    def _ensure_mx_weights(self, w13, w2, ws13, ws2, stream):
        if getattr(self, "mx_key", None) != self._mx_source_key(w13, w2, ws13, ws2):
            self.prepare_mx_weights(w13, w2, ws13, ws2, stream)

    def prepare_mx_weights(self, w13, w2, ws13=None, ws2=None, stream=None):
        """Quantise the expert weights (once per weight update) in the two
        orientations the microscaled GEMMs contract them in (MXFP4 codes two
        per byte).  The copies are reused by later forward and backward calls
        for as long as they are given the same, unmodified weight tensors;
        other weights are quantised anew."""
        s, dev = self.s, self.device
        u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=dev)
        q = {}
        fp4 = s.dtype == "mxfp4"
        per_byte = 2 if fp4 else 1
        quantize_both = abi.moe_quantize_mxfp4_both if fp4 else abi.moe_quantize_mxfp8_both

        def quant(name, w, batch, rows, cols):
            # the row form (name) and the transposed form (name_t) in one
            # pass, scales grouped as the microscaled GEMMs read them
            c, sc = u8(batch, rows, cols // per_byte), u8(batch, rows, cols // 32)
            ct, sct = u8(batch, cols, rows // per_byte), u8(batch, cols, rows // 32)
            quantize_both(w, batch, rows, cols, c, sc, ct, sct, abi.MOE_MX_GROUPED, stream)
            q[name], q[name + "_t"] = (c, sc), (ct, sct)

        quant("w13", w13, s.E, 2 * s.f, s.d)
        quant("w2", w2, s.E, s.d, s.f)
        if s.f_shared:
            quant("ws13", ws13, 1, 2 * s.f_shared, s.d)
            quant("ws2", ws2, 1, s.d, s.f_shared)
        self.mx_tensors = q                          # keeps the device memory alive
        self.mx_weights = abi.mx_weights(**q)
        self.mx_sources = (w13, w2, ws13, ws2)       # their memory stays theirs while the copies exist
        self.mx_key = self._mx_source_key(w13, w2, ws13, ws2)

    def experts(self, x, w13, w2, ws13=None, ws2=None, stream=None):
        b = self.buf
        if self.s.dtype in ("mxfp8", "mxfp4"):
            self._ensure_mx_weights(w13, w2, ws13, ws2, stream)
            call = abi.moe_grouped_gemm_swiglu_mxfp4 if self.s.dtype == "mxfp4" else abi.moe_grouped_gemm_swiglu_mxfp8
            call(self.cfg, b["x_perm"], b["offsets"], b.get("row_gates"), self.mx_weights, b.get("hu"), b["act"],
                 b["y_perm"], x if self.s.f_shared else None, b.get("hu_s"), b.get("act_s"), b.get("y_s"), self.ws,
                 stream)
            return
        abi.moe_grouped_gemm_swiglu(self.cfg, b["x_perm"], b["offsets"], b.get("row_gates"), w13, w2, b.get("hu"),
                                    b["act"],
                                    b["y_perm"], x if self.s.f_shared else None, ws13, ws2, b.get("hu_s"),
                                    b.get("act_s"), b.get("y_s"), self.ws, stream)

    def combine(self, stream=None):
        b = self.buf
        abi.moe_unpermute_combine(self.cfg, b["y_perm"], b["row_id_map"], None if self.s.fold_gates else b["gates"],
                                  b.get("y_s"), b["y"], stream)

    def forward(self, x, w_router, bias, w13, w2, ws13=None, ws2=None, stream=None):
        self.route(x, w_router, bias, stream)
        self.permute(x, stream)
        self.experts(x, w13, w2, ws13, ws2, stream)
        self.combine(stream)
        return self.buf["y"]

    # -- backward -----------------------------------------------------------
    def backward(self, dy, x, w_router, w13, w2, ws13=None, ws2=None, d_aux: float = 1.0, stream=None):
        """Gradients of <y, dy>.  With fold_gates the combine's backward only
        copies dy to the permuted rows and the experts' backward forms d_gates;
        with recompute_act the experts' backward does not read act."""
        b, s = self.buf, self.s
        fold = s.fold_gates
        abi.moe_unpermute_combine_bwd(self.cfg, dy, None if fold else b["y_perm"], b["row_id_map"],
                                      None if fold else b["gates"], b["dy_perm"], None if fold else b["d_gates"],
                                      stream)
        sh = bool(s.f_shared)
        act = None if s.recompute_act else b["act"]
        act_s = None if s.recompute_act else b.get("act_s")
        rg = (b["row_gates"], b["row_id_map"], b["d_gates"]) if fold else (None, None, None)
        if s.dtype in ("mxfp8", "mxfp4"):
            self._ensure_mx_weights(w13, w2, ws13, ws2, stream)
            call = abi.moe_grouped_gemm_swiglu_bwd_mxfp4 if s.dtype == "mxfp4" else abi.moe_grouped_gemm_swiglu_bwd_mxfp8
            call(
                self.cfg, b["dy_perm"], b["x_perm"], b["offsets"], rg[0], rg[1], b["hu"], act, self.mx_weights,
                b["dhu"], b["dx_perm"], b["dw13"], b["dw2"], rg[2], dy if sh else None, x if sh else None,
                b.get("hu_s"), act_s, b.get("dhu_s"), b["dx_partial"], b.get("dws13"), b.get("dws2"), self.ws,
                stream)
        else:
            self._gemm_bwd_bf16(dy, x, w13, w2, ws13, ws2, stream)
        abi.moe_router_topk_bwd(self.cfg, x, w_router, b["logits"], b["idx"], b["gates"], b["counts"],
                                b["d_gates"], d_aux, b["d_logits"], b["dw_router"], b["dx_partial"],
                                self.ws, stream)
        abi.moe_permute_bwd(self.cfg, b["dx_perm"], b["row_id_map"], b["dx_partial"], b["dx"], stream)
        return b["dx"]

    def _gemm_bwd_bf16(self, dy, x, w13, w2, ws13, ws2, stream):
        b, s = self.buf, self.s
        sh = bool(s.f_shared)
        fold = s.fold_gates
        act = None if s.recompute_act else b["act"]
        act_s = None if s.recompute_act else b.get("act_s")
        abi.moe_grouped_gemm_swiglu_bwd(
            self.cfg, b["dy_perm"], b["x_perm"], b["offsets"], b["row_gates"] if fold else None,
            b["row_id_map"] if fold else None, b["hu"], act, w13, w2, b["dhu"], b["dx_perm"], b["dw13"], b["dw2"],
            b["d_gates"] if fold else None, dy if sh else None, x if sh else None, b.get("hu_s"), act_s, ws13, ws2,
            b.get("dhu_s"), b["dx_partial"], b.get("dws13"), b.get("dws2"), self.ws, stream)
