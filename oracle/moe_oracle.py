"""CPU oracle for one GPU's mixture-of-experts layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module.  The product path (the HIP library and its Python binding) never
calls it and shares no code with it; both sides only share the seeded input
generators of moe_inputs.py.

What it computes is the plain definition of the layer, evaluated in float64
with numpy (a matmul is the only library primitive used), following the pages
"Scalable Training of Mixture-of-Experts Models with Megatron Core":

* the layer output y = sum over the top-k experts of g(x)_i * E_i(x)
  (papers.lunadong.com summary, "Problem Definition");
* the stage order Router -> Dispatcher -> Experts -> Combiner
  (same page, "Pipeline Flow"; thelatestinai.com page, Figure 1);
* the router as a learned linear projection, a score function, top-k selection
  and load balancing (summary page, "System Modules: Router"; Figure 2);
* the combiner putting rows back in their original token position and forming
  the gate-weighted sum (summary page, "System Modules: Combiner");
* SwiGLU experts (Table 4 names "Activation Function (SwiGLU)"; the GLU-variants
  paper is in the citation list);
* a shared expert that sees every token (Table 1 "Shared Experts", Figure 40).

The pages give no formula for scores, groups, gates, the aux loss or the
backward pass.  Those follow the workload descriptions (sigmoid + selection-only
bias, 8 groups / top-4 by top-2 sum, renormalise then x2.5, aux coefficient
1e-3) and, where both are silent, the plainest readings; the ones this module
depends on:

  R3  softmax selection key = fp32 logit (softmax is monotone), ties -> lower id
  R4  sigmoid score s = fp32(1 / (1 + exp(-(double) l))); key = fp32(s + b)
  R5  contiguous groups of E/n_group experts; group score = fp32 sum of the two
      largest keys; group ties -> lower group id
  R7  gates divide by the sum of the unbiased selected scores, then x scale
  R8  aux = coeff * E * sum_e f_e * Pbar_e, f_e = c_e / (T k), Pbar_e = mean
      full-softmax probability; only Pbar carries gradient
  R9  dropless: every (token, choice) gets a row, T*k rows in all
  R10 rows are expert-major, ascending token id inside an expert
  R12 storage rounding (bf16 round-to-nearest-even) where a tensor is
      materialised; everything in between is float64 here
  R13 combine sums j = 0..k-1 in selection order, then the shared output
  R15 MXFP8: fp8 e4m3fn codes, one e8m0 power-of-two scale 2^e per 32
      consecutive values along the contraction dimension, e the smallest
      integer with 448 * 2^e >= block amax (clamped to [-127, 127]; amax 0
      gives e = -127 and zero codes); element = RNE(v / 2^e), saturating
  R16 MXFP8 along a ragged row range: blocks of 32 rows start at the range's
      first row, rows past its end count as zeros
  R17 expert weights enter the MXFP8 GEMMs quantised along whichever of their
      dimensions the GEMM contracts
  R25 MXFP4 (the gfx950 counterpart of the NVFP4 the pages support): the R15
      block structure with fp4 e2m1 elements (largest magnitude 6), e the
      smallest integer with 6 * 2^e >= block amax; the same seven expert
      products as MXFP8; codes stored two per byte, element 2i in the low
      nibble
  R21 force-balanced routing (the benchmark condition of Table 11): choice j of
      token t goes to expert (t k + j) mod E, so every expert gets T k / E rows
      when E divides T k; gates come from the scores of the assigned experts
      by the usual rule
  R22 bias update without an auxiliary loss (Figure 39, load balancing): after
      a step, b_e <- fp32(b_e + rate * sign(T k / E - c_e)), the sign taken
      on the integers T k - E c_e
  R23 gate folding (a reading of memory-efficient permutation, Figure 7 and
      Table 6): the gate of each permuted row multiplies the SwiGLU output
      before the down projection, A_g = g silu(H) U, so the combine is an
      unweighted sum; the backward gets dg = <dA, silu(H) U> with dA = dy W2
      and silu(H) U formed from the stored H, U
  R24 SwiGLU recomputation (Figure 8, Table 4): act is formed from the stored
      (rounded) H and U in the forward, and the backward forms it again from
      them, so it is not kept between the passes and both forms agree bit for
      bit
  R27 non-finite keys (the pages are silent): -inf and +inf order as numbers;
      a NaN key ranks after every number, NaN keys among themselves by lower
      id; a group holding a NaN key scores NaN and ranks after every group
      with a numeric score.  So the k choices are k distinct eligible experts
      whatever the logits hold

Pins that tie this oracle to facts outside itself live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------
def round_bf16(a) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), via fp32; returned as fp64.

    bfloat16 keeps the top 16 bits of an IEEE binary32; rounding to nearest even
    adds 0x7FFF plus the lowest kept bit before truncating the low 16 bits.
    """
    a32 = np.ascontiguousarray(np.asarray(a, dtype=F64).astype(F32))
    u = a32.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(F32).astype(F64)


def store(a, storage: str) -> np.ndarray:
    """Value of `a` after it is materialised in the layer's storage dtype."""
    if storage == "bf16":
        return round_bf16(a)
    if storage == "f32":
        return np.asarray(a, dtype=F64).astype(F32).astype(F64)
    if storage == "f64":          # exact mode used by the finite-difference pins
        return np.asarray(a, dtype=F64)
    raise ValueError(storage)


def storage_of(cfg) -> str:
    return "f32" if cfg.dtype == "f32" else "bf16"


# ----------------------------------------------------------------------------
# Router: projection, score, (group-limited) top-k, gates, statistics
# ----------------------------------------------------------------------------
def router_logits(x, w_router, storage: str = "f32") -> np.ndarray:
    """logits[t,e] = sum_i x[t,i] * W_r[e,i]  (learned linear projection).
    Stored as fp32 (or kept exact in "f64" mode)."""
    l = np.asarray(x, F64) @ np.asarray(w_router, F64).T
    return l if storage == "f64" else l.astype(F32)


def sigmoid_scores(logits, exact: bool = False) -> np.ndarray:
    """s = 1/(1+exp(-l)) evaluated in float64 and rounded once to fp32 (R4)."""
    s = 1.0 / (1.0 + np.exp(-np.asarray(logits, F64)))
    return s if exact else s.astype(F32)


def softmax_probs(logits) -> np.ndarray:
    """Full softmax over all E experts, float64."""
    l = np.asarray(logits, F64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def selection_keys(logits, cfg, bias=None, exact: bool = False) -> np.ndarray:
    """Key each expert is ranked by.  Softmax: the logit itself (R3).
    Sigmoid: fp32(s + b), the bias steering selection only (R4)."""
    if cfg.score == "softmax":
        return np.asarray(logits, F64 if exact else F32)
    s = sigmoid_scores(logits, exact)
    if bias is None:
        return s
    b = np.asarray(bias, F32)
    return (s + b) if not exact else (np.asarray(s, F64) + b.astype(F64))


def _desc_order(values, ids) -> np.ndarray:
    """ids sorted by value descending, equal values by id ascending; NaN values
    after every number (-inf included), among themselves by id (R27)."""
    values = np.asarray(values)
    ids = np.asarray(ids)
    o = np.argsort(ids, kind="stable")               # ids ascending first
    v = values[o]
    num = ~np.isnan(v)
    o_num = o[num][np.argsort(-v[num], kind="stable")]   # numbers: stable sort by value desc
    return np.concatenate([ids[o_num], ids[o[~num]]])


def eligible_groups(keys_row, n_group: int, topk_group: int) -> np.ndarray:
    """Group-limited routing for one token (R5): split the E experts into
    n_group contiguous groups, score each group by the sum of its two largest
    keys (one fp32 add; a single-expert group scores its only key), keep the
    topk_group best groups.  Returns the kept group ids in rank order.  A group
    holding a NaN key scores NaN and so ranks after every numeric score (R27)."""
    E = keys_row.shape[0]
    per = E // n_group
    gscore = np.empty(n_group, dtype=keys_row.dtype)
    for g in range(n_group):
        member = keys_row[g * per:(g + 1) * per]
        if np.isnan(member).any():
            gscore[g] = np.nan
            continue
        member = np.sort(member)[::-1]
        gscore[g] = member[0] + member[1] if per >= 2 else member[0]
    return _desc_order(gscore, np.arange(n_group))[:topk_group]


def select_topk(keys, cfg) -> np.ndarray:
    """idx[t, :] = the k eligible experts with the largest keys, in descending
    key order, equal keys by lower expert id (R6)."""
    T, E = keys.shape
    idx = np.empty((T, cfg.k), dtype=np.int32)
    per = E // cfg.n_group
    for t in range(T):
        if cfg.n_group > 1:
            groups = eligible_groups(keys[t], cfg.n_group, cfg.topk_group)
            cand = np.concatenate([np.arange(g * per, (g + 1) * per) for g in groups])
        else:
            cand = np.arange(E)
        idx[t] = _desc_order(keys[t][cand], cand)[:cfg.k]
    return idx


def select_balanced(T: int, E: int, k: int) -> np.ndarray:
    """Force-balanced routing (R21): choice j of token t is expert (t k + j) mod E.
    The k choices of a token are k consecutive experts modulo E, so they are
    distinct for k <= E."""
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        for j in range(k):
            idx[t, j] = (t * k + j) % E
    return idx


def bias_update(bias, counts, T: int, k: int, rate: float) -> np.ndarray:
    """Aux-loss-free balancing step (R22): raise the selection bias of experts
    below the mean load T k / E by `rate`, lower it for those above, leave it
    where the load is exactly the mean.  One fp32 add per expert."""
    b = np.asarray(bias, F32).copy()
    c = np.asarray(counts, np.int64)
    E = b.shape[0]
    sign = np.sign(T * k - E * c)                      # integer: no rounding in the comparison
    for e in range(E):
        b[e] = F32(b[e] + F32(rate) * F32(sign[e]))
    return b


def gates_from_selection(logits, idx, cfg, exact: bool = False) -> np.ndarray:
    """Gate weights g[t, j] of the selected experts (R7).
    softmax + renorm: softmax restricted to the selection;
    softmax without renorm: the full-softmax probability;
    sigmoid: s / sum of selected s (if renorm), times cfg.scale."""
    l = np.asarray(logits, F64)
    sel_l = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    if cfg.score == "softmax":
        if cfg.renorm:
            z = np.exp(sel_l - sel_l.max(axis=1, keepdims=True))
            g = z / z.sum(axis=1, keepdims=True)
        else:
            g = np.take_along_axis(softmax_probs(l), idx.astype(np.int64), axis=1)
    else:
        s = np.asarray(sigmoid_scores(l, exact), F64)
        sel_s = np.take_along_axis(s, idx.astype(np.int64), axis=1)
        g = sel_s / sel_s.sum(axis=1, keepdims=True) if cfg.renorm else sel_s
    g = g * cfg.scale
    return g if exact else g.astype(F32)


def route(x, w_router, bias, cfg, storage: str = None) -> dict:
    """Router stage on the tokens in x: logits, idx, gates (and full softmax
    probabilities when the score is softmax)."""
    exact = storage == "f64"
    logits = router_logits(x, w_router, "f64" if exact else "f32")
    keys = selection_keys(logits, cfg, bias, exact)
    if getattr(cfg, "force_balanced", False):
        idx = select_balanced(logits.shape[0], logits.shape[1], cfg.k)
    else:
        idx = select_topk(keys, cfg)
    gates = gates_from_selection(logits, idx, cfg, exact)
    out = {"logits": logits, "keys": keys, "idx": idx, "gates": gates}
    if cfg.score == "softmax":
        out["probs"] = softmax_probs(logits)
    else:
        out["scores"] = sigmoid_scores(logits, exact)
    return out


def expert_counts(idx, E: int) -> np.ndarray:
    c = np.zeros(E, dtype=np.int64)
    for e in np.asarray(idx).ravel():
        c[e] += 1
    return c.astype(np.int32)


def aux_loss(probs, counts, T: int, k: int, coeff: float) -> float:
    """Load-balancing loss (R8): coeff * E * sum_e f_e * Pbar_e with
    f_e = c_e/(T k) the fraction of assignments and Pbar_e the mean probability."""
    E = probs.shape[1]
    if T == 0:
        return 0.0
    f = np.asarray(counts, F64) / (T * k)
    pbar = np.asarray(probs, F64).sum(axis=0) / T
    return float(coeff * E * np.sum(f * pbar))


# ----------------------------------------------------------------------------
# Dispatch on one GPU: permutation into expert-contiguous rows
# ----------------------------------------------------------------------------
def permutation(idx, E: int) -> dict:
    """Stable counting sort of (token, choice) pairs by expert (R9, R10).

    offsets[e] = number of assignments to experts < e; the rows of expert e are
    offsets[e] .. offsets[e+1]-1, filled by ascending token id;
    row_id_map[t, j] = row of (t, j); src_token[row] = t.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = expert_counts(idx, E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    next_row = offsets[:E].copy()
    row_id_map = np.empty((T, k), dtype=np.int32)
    src_token = np.empty(T * k, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            row_id_map[t, j] = next_row[e]
            src_token[next_row[e]] = t
            next_row[e] += 1
    return {"counts": counts, "offsets": offsets.astype(np.int32),
            "row_id_map": row_id_map, "src_token": src_token}


def permute_rows(x, src_token) -> np.ndarray:
    """Xp[row] = x[src_token[row]]: the one permuted copy of the activations."""
    return np.asarray(x)[np.asarray(src_token, dtype=np.int64)]


# ----------------------------------------------------------------------------
# Experts: SwiGLU FFNs
# ----------------------------------------------------------------------------
def silu(h):
    return h / (1.0 + np.exp(-h))


def _act(h, u, gate):
    """SwiGLU output silu(h) * u, times the row's gate when gates are folded (R23)."""
    a = silu(h) * u
    return a if gate is None else np.asarray(gate, F64)[:, None] * a


def swiglu_ffn_fwd(xe, w13_e, w2_e, storage: str, gate=None, act_from_stored: bool = False) -> dict:
    """One SwiGLU FFN on rows xe [n, d] with W13 [2f, d] (gate rows then up
    rows) and W2 [d, f]:  H = xe Wg^T, U = xe Wu^T, A = silu(H) * U, Y = A W2^T.
    H and U are kept as stored (for backward); A is formed from the unrounded
    H, U (from the stored ones with act_from_stored, R24), times the row gates
    `gate` [n] if given (R23), and then stored; Y is stored."""
    f = w2_e.shape[1]
    xe = np.asarray(xe, F64)
    w13_e = np.asarray(w13_e, F64)
    h = xe @ w13_e[:f].T
    u = xe @ w13_e[f:].T
    H, U = store(h, storage), store(u, storage)
    a = store(_act(H, U, gate) if act_from_stored else _act(h, u, gate), storage)
    y = store(a @ np.asarray(w2_e, F64).T, storage)
    return {"H": H, "U": U, "A": a, "Y": y}


def swiglu_ffn_bwd(xe, H, U, A, dY, w13_e, w2_e, storage: str, gate=None) -> dict:
    """Backward of swiglu_ffn_fwd given the stored H, U, A and the incoming dY:
      dA  = dY W2                       dW2 = dY^T A
      dH  = dA * U * sig(H) * (1 + H (1 - sig(H)))      (d silu)
      dU  = dA * silu(H)
      dX  = dH Wg + dU Wu               dWg = dH^T X,  dWu = dU^T X
    With folded gates (R23, `gate` [n]) A holds g silu(H) U and dY the
    unweighted upstream rows: the gate gradient of each row is
    dg = <dY W2, silu(H) U> and dH, dU take dA = g (dY W2).
    dA stays unrounded (it lives only inside the producing kernel); dH, dU, dX
    and the weight gradients are stored; dg is returned unrounded."""
    f = w2_e.shape[1]
    dY = np.asarray(dY, F64)
    H = np.asarray(H, F64)
    U = np.asarray(U, F64)
    w13_e = np.asarray(w13_e, F64)
    dA = dY @ np.asarray(w2_e, F64)
    dg = None
    if gate is not None:
        dg = np.sum(dA * (silu(H) * U), axis=1)
        dA = np.asarray(gate, F64)[:, None] * dA
    dW2 = store(dY.T @ np.asarray(A, F64), storage)
    sig = 1.0 / (1.0 + np.exp(-H))
    dH = store(dA * U * sig * (1.0 + H * (1.0 - sig)), storage)
    dU = store(dA * H * sig, storage)
    dHU = np.concatenate([dH, dU], axis=1)
    xe = np.asarray(xe, F64)
    dX_unrounded = dHU @ w13_e
    dW13 = store(dHU.T @ xe, storage)
    return {"dA": dA, "dH": dH, "dU": dU, "dX32": dX_unrounded,
            "dX": store(dX_unrounded, storage), "dW13": dW13, "dW2": dW2, "dg": dg}


# ----------------------------------------------------------------------------
# MXFP8 (DeepSeek-V3 workload with skewed load: expert GEMM operands in fp8
# e4m3 with 1x32 e8m0 block scales along the contraction, fp32+ accumulation,
# bf16 outputs)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3fn byte: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN (the format
    has no infinities)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sgn = np.where(c >> 7, -1.0, 1.0)
    ex = (c >> 3) & 15
    man = c & 7
    mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    mag = np.where((ex == 15) & (man == 7), np.nan, mag)
    return sgn * mag


def _e4m3_table():
    """The 127 non-negative finite magnitudes of e4m3fn, ascending, and their
    codes (codes 0x00 .. 0x7E)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return e4m3_decode(codes), codes


def e4m3_encode(v) -> np.ndarray:
    """Round each finite value to the nearest e4m3fn value (ties to the code
    with an even mantissa, i.e. an even code), saturating at +-448; the sign
    of zero is kept.  Found by searching the table of representable values."""
    v = np.asarray(v, F64)
    mags, codes = _e4m3_table()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, len(mags) - 1)
    lo = np.clip(hi - 1, 0, len(mags) - 1)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return np.where(np.signbit(v), c | np.uint8(0x80), c).astype(np.uint8)


# ----------------------------------------------------------------------------
# MXFP4 (R25): the same block structure with fp4 e2m1 elements -- one sign
# bit, two exponent bits (bias 1), one mantissa bit, no infinities or NaN;
# magnitudes 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6
# ----------------------------------------------------------------------------
E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit e2m1 code (the low nibble of the byte): exponent
    field 0 is subnormal, m/2; otherwise (1 + m/2) * 2^(ex - 1)."""
    c = np.asarray(codes, np.uint8).astype(np.int64) & 15
    sgn = np.where(c >> 3, -1.0, 1.0)
    ex = (c >> 1) & 3
    man = c & 1
    mag = np.where(ex == 0, man / 2.0, (1.0 + man / 2.0) * np.exp2(ex - 1.0))
    return sgn * mag


def e2m1_encode(v) -> np.ndarray:
    """Round each finite value to the nearest e2m1 value (ties to the code
    with an even mantissa bit, i.e. an even code), saturating at +-6; the sign
    of zero is kept.  Found by searching the table of the 8 magnitudes."""
    v = np.asarray(v, F64)
    codes = np.arange(8, dtype=np.uint8)
    mags = e2m1_decode(codes)
    a = np.minimum(np.abs(v), E2M1_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, len(mags) - 1)
    lo = np.clip(hi - 1, 0, len(mags) - 1)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return np.where(np.signbit(v), c | np.uint8(0x8), c).astype(np.uint8)


def pack_e2m1(codes) -> np.ndarray:
    """Two codes per byte along the last axis (even length): element 2i in the
    low nibble, 2i+1 in the high nibble -- the storage form of MXFP4 codes."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_e2m1(packed) -> np.ndarray:
    b = np.asarray(packed, np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


# element formats of the microscaled GEMM operands: largest magnitude, encoder, decoder
MX_FORMATS = {
    "e4m3": (E4M3_MAX, e4m3_encode, e4m3_decode),   # MXFP8 (R15)
    "e2m1": (E2M1_MAX, e2m1_encode, e2m1_decode),   # MXFP4 (R25)
}


def mx_scale_exp(amax, fmt: str = "e4m3") -> np.ndarray:
    """Smallest integer e with emax * 2^e >= amax (emax: the format's largest
    magnitude, 448 for e4m3 and 6 for e2m1), clamped to [-127, 127] (amax = 0
    gives -127).  Stored as the e8m0 byte e + 127."""
    top = MX_FORMATS[fmt][0]
    amax = np.asarray(amax, F64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / top))
    # the float log2 may sit one off near powers of two: settle on the exact rule
    e = np.where(top * np.exp2(e) < amax, e + 1, e)
    e = np.where(top * np.exp2(e - 1) >= amax, e - 1, e)
    e = np.where(amax > 0, e, -127.0)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(a, axis: int, fmt: str = "e4m3"):
    """Codes (one per value, unpacked) and e8m0 scale bytes of `a` with blocks
    of 32 consecutive values along `axis`, the first block starting at index 0
    of that axis and a short last block padded with zeros.  Returns (codes
    shaped like a, scale bytes with the blocked axis of length ceil(n/32))."""
    encode = MX_FORMATS[fmt][1]
    a = np.moveaxis(np.asarray(a, F64), axis, -1)
    n = a.shape[-1]
    nb = -(-n // MX_BLOCK)
    pad = np.zeros(a.shape[:-1] + (nb * MX_BLOCK,))
    pad[..., :n] = a
    blk = pad.reshape(a.shape[:-1] + (nb, MX_BLOCK))
    e = mx_scale_exp(np.max(np.abs(blk), axis=-1), fmt)
    codes = encode(blk / np.exp2(e)[..., None]).reshape(pad.shape)[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis((e + 127).astype(np.uint8), -1, axis)


def mx_dequantize(codes, scale_bytes, axis: int, fmt: str = "e4m3") -> np.ndarray:
    decode = MX_FORMATS[fmt][2]
    c = np.moveaxis(np.asarray(codes, np.uint8), axis, -1)
    sb = np.moveaxis(np.asarray(scale_bytes, np.uint8), axis, -1).astype(np.int64)
    n = c.shape[-1]
    scale = np.repeat(np.exp2(sb - 127.0), MX_BLOCK, axis=-1)[..., :n]
    return np.moveaxis(decode(c) * scale, -1, axis)


def mx_qdq(a, axis: int, fmt: str = "e4m3") -> np.ndarray:
    """What a microscaled GEMM sees of `a` when it contracts along `axis`."""
    return mx_dequantize(*mx_quantize(a, axis, fmt), axis, fmt)


def mx_format_of(dtype: str) -> str:
    return {"mxfp8": "e4m3", "mxfp4": "e2m1"}[dtype]


def swiglu_ffn_fwd_mx(xe, w13_e, w2_e, storage: str, gate=None, act_from_stored: bool = False,
                      fmt: str = "e4m3") -> dict:
    """swiglu_ffn_fwd with microscaled GEMM operands (MXFP8: fmt e4m3,
    MXFP4: e2m1): X and W13 quantised along d, A (after its bf16 store) and
    W2 along f."""
    f = w2_e.shape[1]
    xq = mx_qdq(xe, 1, fmt)
    wq = mx_qdq(w13_e, 1, fmt)
    h = xq @ wq[:f].T
    u = xq @ wq[f:].T
    H, U = store(h, storage), store(u, storage)
    a = store(_act(H, U, gate) if act_from_stored else _act(h, u, gate), storage)
    y = store(mx_qdq(a, 1, fmt) @ mx_qdq(w2_e, 1, fmt).T, storage)
    return {"H": H, "U": U, "A": a, "Y": y}


def swiglu_ffn_bwd_mx(xe, H, U, A, dY, w13_e, w2_e, storage: str, gate=None, fmt: str = "e4m3") -> dict:
    """swiglu_ffn_bwd with microscaled GEMM operands, each quantised along the
    dimension its GEMM contracts: dA = dY W2 (d), dW2 = dY^T A (rows),
    dX = dHU W13 (2f), dW13 = dHU^T X (rows; blocks start at the first row).
    Folded gates (`gate`) as in swiglu_ffn_bwd."""
    H = np.asarray(H, F64)
    U = np.asarray(U, F64)
    dY = np.asarray(dY, F64)
    dA = mx_qdq(dY, 1, fmt) @ mx_qdq(w2_e, 0, fmt)
    dg = None
    if gate is not None:
        dg = np.sum(dA * (silu(H) * U), axis=1)
        dA = np.asarray(gate, F64)[:, None] * dA
    dW2 = store(mx_qdq(dY, 0, fmt).T @ mx_qdq(A, 0, fmt), storage)
    sig = 1.0 / (1.0 + np.exp(-H))
    dH = store(dA * U * sig * (1.0 + H * (1.0 - sig)), storage)
    dU = store(dA * H * sig, storage)
    dHU = np.concatenate([dH, dU], axis=1)
    dX_unrounded = mx_qdq(dHU, 1, fmt) @ mx_qdq(w13_e, 0, fmt)
    dW13 = store(mx_qdq(dHU, 0, fmt).T @ mx_qdq(xe, 0, fmt), storage)
    return {"dA": dA, "dH": dH, "dU": dU, "dX32": dX_unrounded,
            "dX": store(dX_unrounded, storage), "dW13": dW13, "dW2": dW2, "dg": dg}


def _ffn_fns(dtype: str):
    """(forward, backward) expert FFN of a layer of storage mode `dtype`."""
    if dtype in ("mxfp8", "mxfp4"):
        fmt = mx_format_of(dtype)
        return (lambda *a, **k: swiglu_ffn_fwd_mx(*a, fmt=fmt, **k),
                lambda *a, **k: swiglu_ffn_bwd_mx(*a, fmt=fmt, **k))
    return swiglu_ffn_fwd, swiglu_ffn_bwd


# ----------------------------------------------------------------------------
# Combine and the whole layer
# ----------------------------------------------------------------------------
def combine(Yp, gates, row_id_map, Ys, storage: str) -> np.ndarray:
    """y[t] = sum_{j<k} g[t,j] * Yp[row(t,j)]  (+ Ys[t]), summed in j order and
    stored once (R13).  gates = None: the rows already carry their gates (R23)
    and are summed unweighted."""
    T, k = row_id_map.shape
    y = np.zeros((T, Yp.shape[1]), F64)
    for j in range(k):
        w = 1.0 if gates is None else np.asarray(gates, F64)[:, j:j + 1]
        y += w * Yp[row_id_map[:, j].astype(np.int64)]
    if Ys is not None:
        y += Ys
    return store(y, storage)


def layer_forward(inp: dict, cfg, storage: str = None) -> dict:
    """The whole layer: Route -> permute -> grouped SwiGLU experts (+ shared
    expert) -> unpermute/combine.  `inp` holds numpy/torch CPU arrays as made
    by moe_inputs.make_inputs."""
    storage = storage or storage_of(cfg)
    ffn_fwd = _ffn_fns(cfg.dtype)[0]
    fold = getattr(cfg, "fold_gates", False)
    from_stored = getattr(cfg, "recompute_act", False)
    x = _np(inp["x"])
    T = x.shape[0]
    r = route(x, _np(inp["w_router"]), _np(inp.get("bias")), cfg, storage)
    p = permutation(r["idx"], cfg.E)
    Xp = permute_rows(x, p["src_token"])
    rows, f = T * cfg.k, cfg.f
    # gate of each permuted row: row_gates[row(t, j)] = gates[t, j]
    row_gates = np.zeros(rows)
    row_gates[p["row_id_map"].reshape(-1).astype(np.int64)] = np.asarray(r["gates"], F64).reshape(-1)
    H = np.zeros((rows, f)); U = np.zeros((rows, f)); A = np.zeros((rows, f))
    Yp = np.zeros((rows, cfg.d))
    w13, w2 = inp["w13"], inp["w2"]
    off = p["offsets"]
    for e in range(cfg.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        o = ffn_fwd(Xp[lo:hi], _np(w13[e]), _np(w2[e]), storage,
                    gate=row_gates[lo:hi] if fold else None, act_from_stored=from_stored)
        H[lo:hi], U[lo:hi], A[lo:hi], Yp[lo:hi] = o["H"], o["U"], o["A"], o["Y"]
    out = dict(r)
    out.update(p)
    out.update({"Xp": Xp, "H": H, "U": U, "A": A, "Yp": Yp, "row_gates": row_gates})
    Ys = None
    if cfg.f_shared > 0:
        s = ffn_fwd(x, _np(inp["ws13"]), _np(inp["ws2"]), storage, act_from_stored=from_stored)
        out.update({"Hs": s["H"], "Us": s["U"], "As": s["A"], "Ys": s["Y"]})
        Ys = s["Y"]
    out["y"] = combine(Yp, None if fold else r["gates"], p["row_id_map"], Ys, storage)
    if cfg.aux_coeff != 0.0:
        out["aux"] = aux_loss(r["probs"], p["counts"], T, cfg.k, cfg.aux_coeff)
    return out


def router_backward(logits, idx, gates, d_gates, counts, cfg, d_aux: float = 1.0,
                    exact: bool = False) -> np.ndarray:
    """d loss / d logits, routing held fixed (top-k is piecewise constant and the
    selection bias receives no gradient).

    softmax + renorm:  dl_m = q_m (dg_m - sum_j q_j dg_j) on the selection, q the
                       softmax of the selected logits (the gates before the
                       scale), evaluated here from the logits: the stored fp32
                       gates sum to 1 only to fp32 precision, and with one gate
                       near 1 the centred form turns that into an error of the
                       size of the result
    softmax, no renorm: dl = p * (dg_full - sum_e p_e dg_full_e)
    aux (softmax):     dl[t,e] += d_aux * p[t,e] * (a_e - sum_e' p[t,e'] a_e'),
                       a_e = coeff * E * f_e / T
    sigmoid:           S = sum s_sel, ds_m = (scale/S) (dg_m - sum_j dg_j s_j / S)
                       (renorm), ds_m = scale * dg_m (no renorm); dl = ds s (1-s)
    """
    l = np.asarray(logits, F64)
    T, E = l.shape
    ii = idx.astype(np.int64)
    dg = np.asarray(d_gates, F64)
    dgs = dg * cfg.scale                            # gradient w.r.t. unscaled gates
    dl = np.zeros((T, E), F64)
    if cfg.score == "softmax":
        if cfg.renorm:
            sl = np.take_along_axis(l, ii, axis=1)
            q = np.exp(sl - sl.max(axis=1, keepdims=True)) if T else sl
            q = q / q.sum(axis=1, keepdims=True) if T else q
            inner = np.sum(q * dgs, axis=1, keepdims=True)
            np.put_along_axis(dl, ii, q * (dgs - inner), axis=1)
        else:
            p = softmax_probs(l)
            full = np.zeros((T, E), F64)
            np.put_along_axis(full, ii, dgs, axis=1)
            dl = p * (full - np.sum(p * full, axis=1, keepdims=True))
        if cfg.aux_coeff != 0.0 and T > 0:
            p = softmax_probs(l)
            a = cfg.aux_coeff * E * (np.asarray(counts, F64) / (T * cfg.k)) / T
            dl += d_aux * p * (a[None, :] - np.sum(p * a[None, :], axis=1, keepdims=True))
    else:
        s = np.asarray(sigmoid_scores(l, exact), F64)
        sel = np.take_along_axis(s, ii, axis=1)
        if cfg.renorm:
            S = sel.sum(axis=1, keepdims=True)
            ds_sel = (dgs - np.sum(dgs * sel, axis=1, keepdims=True) / S) / S
        else:
            ds_sel = dgs
        ds = np.zeros((T, E), F64)
        np.put_along_axis(ds, ii, ds_sel, axis=1)
        dl = ds * s * (1.0 - s)
    return dl


def layer_backward(inp: dict, fwd: dict, cfg, d_aux: float = 1.0,
                   storage: str = None, dense: bool = True) -> dict:
    """Gradients of <y, dy> (+ d_aux * aux) w.r.t. x, the router weight and all
    expert weights, for the forward pass `fwd` of layer_forward.  With
    dense=False the expert weight gradients come back as {expert: array} for
    the experts that received rows only (all others are exactly zero)."""
    storage = storage or storage_of(cfg)
    ffn_bwd = _ffn_fns(cfg.dtype)[1]
    fold = getattr(cfg, "fold_gates", False)
    recompute = getattr(cfg, "recompute_act", False)
    exact = storage == "f64"
    x = _np(inp["x"])
    dy = _np(inp["dy"])
    T, d = x.shape
    rmap = fwd["row_id_map"].astype(np.int64)
    gates = np.asarray(fwd["gates"], F64)
    Yp = fwd["Yp"]
    rows = T * cfg.k
    # combine backward: dYp[row(t,j)] = g[t,j] dy[t]; dg[t,j] = <dy[t], Yp[row]>.
    # With folded gates the rows already carry g: dYp[row(t,j)] = dy[t], and dg
    # comes from the experts' backward (R23).
    dYp = np.zeros_like(Yp)
    d_gates = np.zeros((T, cfg.k), F64)
    for j in range(cfg.k):
        dYp[rmap[:, j]] = dy if fold else gates[:, j:j + 1] * dy
        if not fold:
            d_gates[:, j] = np.sum(dy * Yp[rmap[:, j]], axis=1)
    dYp = store(dYp, storage)
    row_dg = np.zeros(rows)
    dHU = np.zeros((rows, 2 * cfg.f))
    dXp32 = np.zeros((rows, d))
    dXp = np.zeros((rows, d))
    dw13 = np.zeros(inp["w13"].shape) if dense else {}
    dw2 = np.zeros(inp["w2"].shape) if dense else {}
    off = fwd["offsets"]
    Xp = fwd["Xp"]

    def act_for_bwd(H, U, gate, A_fwd):
        # with recomputation the backward forms act again from the stored H, U (R24)
        return store(_act(H, U, gate), storage) if recompute else A_fwd

    for e in range(cfg.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue            # empty expert: exact zero weight gradients
        g_rows = fwd["row_gates"][lo:hi] if fold else None
        A_e = act_for_bwd(fwd["H"][lo:hi], fwd["U"][lo:hi], g_rows, fwd["A"][lo:hi])
        b = ffn_bwd(Xp[lo:hi], fwd["H"][lo:hi], fwd["U"][lo:hi], A_e,
                    dYp[lo:hi], _np(inp["w13"][e]), _np(inp["w2"][e]), storage, gate=g_rows)
        dHU[lo:hi] = np.concatenate([b["dH"], b["dU"]], axis=1)
        dXp32[lo:hi], dXp[lo:hi] = b["dX32"], b["dX"]
        dw13[e], dw2[e] = b["dW13"], b["dW2"]
        if fold:
            row_dg[lo:hi] = b["dg"]
    if fold:
        d_gates = row_dg[rmap]
    if not exact:
        d_gates = d_gates.astype(F32)
    out = {"dYp": dYp, "d_gates": d_gates, "dHU": dHU, "dXp": dXp,
           "dw13": dw13, "dw2": dw2}
    dx_partial = np.zeros((T, d))
    if cfg.f_shared > 0:
        As = act_for_bwd(fwd["Hs"], fwd["Us"], None, fwd["As"])
        s = ffn_bwd(x, fwd["Hs"], fwd["Us"], As, dy,
                    _np(inp["ws13"]), _np(inp["ws2"]), storage)
        out.update({"dHUs": np.concatenate([s["dH"], s["dU"]], axis=1),
                    "dws13": s["dW13"], "dws2": s["dW2"]})
        dx_partial += s["dX32"]
    dl = router_backward(fwd["logits"], fwd["idx"], fwd["gates"], d_gates,
                         fwd["counts"], cfg, d_aux, exact)
    out["d_logits"] = dl if exact else dl.astype(F32)
    out["dw_router"] = store(dl.T @ x, storage)
    dx_partial += dl @ _np(inp["w_router"])
    # permute backward: dx[t] = partial[t] + sum_j dXp[row(t,j)], stored once
    dx = dx_partial.copy()
    for j in range(cfg.k):
        dx += dXp[rmap[:, j]]
    out["dx"] = store(dx, storage)
    return out


def _np(a):
    """torch tensor / numpy array -> float64 numpy array (None passes through)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu")
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.double().numpy()
    return np.asarray(a, F64)
