"""Plain CPU oracle for the local Mixture-of-Experts FFN forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library.

What it computes (ruDNN user guide, "3. MoE workflow"): logits -> fp32 softmax
over all experts -> top-k -> compact dispatch -> bias-free SwiGLU experts ->
weighted combine in token order; plus the fused combine + residual Add +
RMSNorm epilogue of the CANN page aclnnMoeDistributeCombineAddRmsNormV2
("function description", formula). Also the next steps built on the same
data structures: grouped sigmoid routing (ruDNN user guide, "10."), special
experts and the activity mask (the CANN combine page), weight-only INT8/INT4
experts (aclnnFFN, pseudo-quantization scenario) and first-order training
(ruDNN user guide, "12. MoE first-order training": router weights for a fixed
selection and their backward, combine_backward, the experts' training cache
and backward, dispatch_backward).

Precision policy:
  * softmax: computed exactly (fp64) from the fp32-widened logits and rounded
    once to fp32, which is the most accurate result an fp32 softmax can give;
    top-k selection compares these fp32 probabilities (routing contract: the
    softmax over all experts is fp32 and precedes the top-k);
  * expert GEMMs, SiLU, combine and RMSNorm: fp64, with one round-to-nearest-
    even into the model dtype at each tensor the API returns (h inside the
    experts, expert_out, out, x_out, y) and fp32 for rstd;
  * bf16 values travel as uint16 bit patterns; fp16 as numpy float16.

Every function is a direct statement of the definition, vectorised with numpy
where that keeps it readable. Library primitives used: exp, sum, matmul,
lexsort.

Parity pins for every function live in tests/test_oracle_pins.py and
tests/test_oracle_training_pins.py; no function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"


# --------------------------------------------------------------------------
# storage dtypes
# --------------------------------------------------------------------------
def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> exact fp64 values."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == F16:
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == BF16:
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest, ties to even, in one step.

    bf16 keeps 8 significant bits and fp32's exponent range. For |x| in
    [2^(e-1), 2^e) the spacing of bf16 values is 2^(e-8); below 2^-126
    (subnormal) it is fixed at 2^-133. Dividing by a power of two is exact,
    so np.round (half to even) of x / spacing is the RNE integer multiple."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    r = np.round(xf / q) * q
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)  # exact, or +-inf past the largest bf16
    out[fin] = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = 0x7FC0
    out[np.isposinf(x)] = 0x7F80
    out[np.isneginf(x)] = 0xFF80
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> storage dtype, one rounding to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        if dtype == F32:
            return x.astype(np.float32)
        if dtype == F16:
            return x.astype(np.float16)
    if dtype == BF16:
        return _round_bf16(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# routing  (ruDNN user guide, "4. Routing contract")
# --------------------------------------------------------------------------
def invalid_rows(z: np.ndarray) -> np.ndarray:
    """Rows that contain NaN, contain +inf, or are entirely -inf. The routing
    contract keeps NaN weights for these rows instead of a uniform fallback."""
    return np.isnan(z).any(axis=1) | np.isposinf(z).any(axis=1) | np.isneginf(z).all(axis=1)


def softmax_fp32(logits: np.ndarray, logits_dtype: str) -> np.ndarray:
    """p[t, e] = exp(z[t, e]) / sum_j exp(z[t, j]) over all E experts, delivered
    in fp32. Computed as exp(z - max) in fp64 and rounded once."""
    z = decode(logits, logits_dtype)
    T, E = z.shape
    p = np.full((T, E), np.nan, dtype=np.float32)
    ok = ~invalid_rows(z)
    if ok.any():
        zo = z[ok]
        a = np.exp(zo - zo.max(axis=1, keepdims=True))
        p[ok] = (a / a.sum(axis=1, keepdims=True)).astype(np.float32)
    return p


def route(logits: np.ndarray, logits_dtype: str, top_k: int, renormalize: bool):
    """Routing plan: (indices uint32 [T, k], weights [T, k] in logits dtype).

    Selection: the k largest fp32 probabilities, largest first; equal
    probabilities favour the lower expert id. Rows that are invalid (see
    invalid_rows) have all probabilities NaN; NaNs tie with each other, so the
    tie rule selects ids 0..k-1, and every weight is NaN.
    With renormalize the selected probabilities are divided by their sum, then
    cast to the logits dtype; without it they are cast as they are."""
    z = decode(logits, logits_dtype)
    T, E = z.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k must satisfy 1 <= top_k <= E")
    p = softmax_fp32(logits, logits_dtype)
    bad = invalid_rows(z)
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -p.astype(np.float64)), axis=-1)  # key 1: -p, key 2: id
    order[bad] = np.arange(E)
    idx = order[:, :top_k]
    psel = np.take_along_axis(p, idx, axis=1).astype(np.float64)
    if renormalize:
        w = psel / psel.sum(axis=1, keepdims=True)
    else:
        w = psel
    w[bad] = np.nan
    return idx.astype(np.uint32), round_to(w, logits_dtype)


# --------------------------------------------------------------------------
# grouped-limited sigmoid routing  (ruDNN user guide, "10. Grouped-limited
# sigmoid MoE routing")
# --------------------------------------------------------------------------
def sigmoid_fp32(logits: np.ndarray, logits_dtype: str) -> np.ndarray:
    """s = 1 / (1 + exp(-z)) delivered in fp32: computed in fp64 and rounded
    once. sigmoid(+inf) = 1, sigmoid(-inf) = 0, NaN stays NaN."""
    z = decode(logits, logits_dtype)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s.astype(np.float32)


def grouped_sigmoid_scores(logits, logits_dtype, bias, groups, group_top_two):
    """The quantities the grouped router decides on, all fp32 [T, ...]:
    s (raw sigmoid scores, [T, E]), c = s + bias (the corrected scores used
    for selection only, one fp32 addition, [T, E]) and the group scores
    [T, groups]: the sum of the two largest corrected scores of each group
    (one fp32 addition of the largest and the second largest), or the
    group's largest corrected score. Expert e belongs to group e // (E/groups)."""
    s = sigmoid_fp32(logits, logits_dtype)
    T, E = s.shape
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    c = s + b  # float32 + float32: IEEE fp32 addition
    c = c + np.float32(0.0)  # -0 -> +0, so equal scores compare as ties
    cg = np.sort(c.reshape(T, groups, E // groups), axis=-1)[..., ::-1]
    if group_top_two:
        g = cg[..., 0] + cg[..., 1]
    else:
        g = cg[..., 0].copy()
    return s, c, g


def route_sigmoid_grouped(logits, logits_dtype, bias, top_k, groups, selected_groups,
                          group_top_two, renormalize, scale):
    """Routing plan (indices uint32 [T, k], weights [T, k] in logits dtype).

    1. s = sigmoid(z) in fp32; c = s + bias (bias [E] fp32, absent = 0).
    2. Experts are split into `groups` equal contiguous groups; each group is
       scored by its two largest c summed (group_top_two) or its largest c.
    3. The `selected_groups` best groups are kept (equal scores: lower group
       first); experts of the other groups cannot be chosen.
    4. Among the kept experts the k largest c are chosen, largest first,
       equal scores favouring the lower expert id.
    5. Weights use the raw s of the chosen experts (the bias only steers the
       choice): divided by their sum when renormalize is set, then times
       scale, then cast to the logits dtype.
    A row whose corrected scores contain a NaN (a NaN logit or bias) has all
    scores tied as NaN: its indices are 0..k-1 and every weight is NaN, as
    for the softmax router."""
    z = decode(logits, logits_dtype)
    T, E = z.shape
    if not (1 <= groups <= 128 and E % groups == 0 and 1 <= E <= 1024):
        raise ValueError("groups must divide E, 1 <= groups <= 128, 1 <= E <= 1024")
    gs = E // groups
    if not (1 <= selected_groups <= groups) or not (1 <= top_k <= min(64, selected_groups * gs)):
        raise ValueError("need 1 <= selected_groups <= groups and 1 <= top_k <= min(64, selected experts)")
    if group_top_two and gs < 2:
        raise ValueError("group_top_two needs at least two experts per group")
    if not (np.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and positive")
    s, c, g = grouped_sigmoid_scores(logits, logits_dtype, bias, groups, group_top_two)
    bad = np.isnan(c).any(axis=1)
    gid = np.broadcast_to(np.arange(groups), (T, groups))
    gorder = np.lexsort((gid, -g.astype(np.float64)), axis=-1)  # key 1: -score, key 2: group id
    kept = np.zeros((T, groups), bool)
    np.put_along_axis(kept, gorder[:, :selected_groups], True, axis=1)
    masked = np.where(np.repeat(kept, gs, axis=1), c.astype(np.float64), -np.inf)
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -masked), axis=-1)
    order[bad] = np.arange(E)
    idx = order[:, :top_k].astype(np.uint32)
    w = _grouped_weights_f64(logits, logits_dtype, idx, renormalize, scale)
    w[bad] = np.nan
    return idx, round_to(w, logits_dtype)


def _grouped_weights_f64(logits, logits_dtype, indices, renormalize, scale):
    s = sigmoid_fp32(logits, logits_dtype)
    w = np.take_along_axis(s, np.asarray(indices).astype(np.int64), axis=1).astype(np.float64)
    if renormalize:
        with np.errstate(invalid="ignore"):  # NaN rows, marked by the caller
            w = w / w.sum(axis=1, keepdims=True)
    return w * float(scale)


def grouped_selection_weights(logits, logits_dtype, indices, renormalize, scale):
    """Step 5 of route_sigmoid_grouped for a given selection: the raw fp32
    sigmoid scores s of the selected experts (the correction bias steers the
    choice only), divided by their sum when renormalize is set, then times
    scale, cast to the logits dtype. Any valid selection of a row (one that
    the grouped rule could have produced) gets its weights from here; rows
    whose scores hold a NaN are route_sigmoid_grouped's to mark."""
    return round_to(_grouped_weights_f64(logits, logits_dtype, indices, renormalize, scale), logits_dtype)


def route_sigmoid_grouped_margins(logits, logits_dtype, bias, top_k, groups, selected_groups,
                                  group_top_two):
    """Per row, the smallest gap the grouped router's decisions rest on: between
    the last kept and the first dropped group score, and between consecutive
    corrected scores among the k+1 best kept experts. Rows with a margin of a
    few fp32 ulps may legitimately differ between two fp32 implementations."""
    s, c, g = grouped_sigmoid_scores(logits, logits_dtype, bias, groups, group_top_two)
    T, E = c.shape
    gs = E // groups
    gsorted = -np.sort(-g.astype(np.float64), axis=1)
    gm = (gsorted[:, selected_groups - 1] - gsorted[:, selected_groups]) if selected_groups < groups \
        else np.full(T, np.inf)
    gid = np.broadcast_to(np.arange(groups), (T, groups))
    gorder = np.lexsort((gid, -g.astype(np.float64)), axis=-1)
    kept = np.zeros((T, groups), bool)
    np.put_along_axis(kept, gorder[:, :selected_groups], True, axis=1)
    masked = np.where(np.repeat(kept, gs, axis=1), c.astype(np.float64), -np.inf)
    top = -np.sort(-masked, axis=1)[:, :min(top_k + 1, selected_groups * gs)]
    em = np.diff(-top, axis=1).min(axis=1) if top.shape[1] > 1 else np.full(T, np.inf)
    return np.minimum(gm, em)


# --------------------------------------------------------------------------
# dispatch  (ruDNN user guide, "5. Expert weights and dispatch")
# --------------------------------------------------------------------------
def dispatch(indices: np.ndarray, E: int, x: np.ndarray | None = None, active=None):
    """Compact grouping of the T*k (token, slot) pairs by expert, no capacity
    drop. Within an expert, pairs keep (token, slot) order (the pages leave
    this order free; it is fixed here so results repeat). Returns
      offsets     int32 [E+1]  rows of expert e are offsets[e]:offsets[e+1]
      slot_of_row int32 [R]    flat slot t*k+j held by dispatched row r
      row_of_slot int32 [T*k]  inverse map; -1 for an out-of-range expert id
      x_disp      [R, H]       x_disp[r] = x[slot_of_row[r] // k]   (if x given)
    where R = number of in-range pairs. active (optional, the xActiveMaskOptional
    input of aclnnMoeDistributeCombineAddRmsNormV2): bool [T] per token or
    [T, k] per slot; inactive pairs are not dispatched either."""
    T, k = indices.shape
    flat = indices.reshape(-1).astype(np.int64)
    if active is not None:
        a = np.asarray(active, bool)
        on = np.repeat(a, k) if a.ndim == 1 else a.reshape(-1)
        flat = np.where(on, flat, -1)
    slots_by_expert = [np.nonzero(flat == e)[0] for e in range(E)]
    counts = np.array([len(s) for s in slots_by_expert], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    slot_of_row = (np.concatenate(slots_by_expert) if E else np.zeros(0, np.int64)).astype(np.int32)
    row_of_slot = np.full(T * k, -1, dtype=np.int32)
    row_of_slot[slot_of_row] = np.arange(len(slot_of_row), dtype=np.int32)
    out = dict(offsets=offsets, slot_of_row=slot_of_row, row_of_slot=row_of_slot)
    if x is not None:
        out["x_disp"] = x[slot_of_row // k]
    return out


# --------------------------------------------------------------------------
# experts  (ruDNN user guide, "3. MoE workflow" and "5. Expert weights")
# --------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_expert(x_rows: np.ndarray, w_gate_e: np.ndarray, w_up_e: np.ndarray,
                  w_down_e: np.ndarray, dtype: str) -> np.ndarray:
    """One bias-free SwiGLU expert on its rows.
    x_rows [n, H]; gate/up [I, H]; down [H, I] (all stored in dtype).
      g = x W_gate^T, u = x W_up^T            (fp64)
      h = round(SiLU(g) * u)                  (stored in the model dtype)
      y = round(h W_down^T)                   [n, H]"""
    x = decode(x_rows, dtype)
    g = x @ decode(w_gate_e, dtype).T
    u = x @ decode(w_up_e, dtype).T
    h = decode(round_to(silu(g) * u, dtype), dtype)
    return round_to(h @ decode(w_down_e, dtype).T, dtype)


def swiglu_expert_f64(x_rows, w_gate, w_up, w_down, dtype):
    """swiglu_expert with the three weight matrices given as fp64 arrays (the
    decoded dequantised weights); x_rows stored in dtype; same roundings of h
    and y."""
    x = decode(x_rows, dtype)
    g = x @ w_gate.T
    u = x @ w_up.T
    h = decode(round_to(silu(g) * u, dtype), dtype)
    return round_to(h @ w_down.T, dtype)


# --------------------------------------------------------------------------
# weight-only quantised experts  (aclnnFFN, "Formula", pseudo-quantization
# scenario: W enters as (W + antiquantOffset) * antiquantScale)
# --------------------------------------------------------------------------
def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] integers: element k lives in byte k // 2,
    low nibble for even k, as a two's complement 4-bit value (-8 .. 7)."""
    b = np.asarray(packed, np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    out = np.stack([lo, hi], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2)
    return np.where(out >= 8, out - 16, out)


def dequant_weight(q, bits, scale, offset, groups, dtype, round_weights=False):
    """One expert's dequantised weight matrix [N, K] as fp64 values:
        w[n, k] = (q[n, k] + offset[n, j]) * scale[n, j],  j = k // (K / groups)
    (the pseudo-quantization formula of aclnnFFN, per channel or per group).
    round_weights=False (the reading used for parity): the formula in exact
    arithmetic. The page states the formula and the storage dtypes of the
    codes, antiquantScale and antiquantOffset (the activation dtype), not a
    rounding of the bracketed product, so w is the exact value and only the
    GEMMs' results are rounded, as in the unquantised path.
    round_weights=True (an alternative reading, for comparison): w held as a
    tensor of the activation dtype, the exact value rounded once.
    q: int8 [N, K] (bits 8) or packed int4 bytes [N, K/2] (bits 4); scale,
    offset: [N, groups] stored in dtype (offset None = 0)."""
    qi = unpack_int4(q) if bits == 4 else np.asarray(q).view(np.int8).astype(np.int16)
    N, K = qi.shape
    gs = K // groups
    sc = np.repeat(decode(scale, dtype).reshape(N, groups), gs, axis=1)
    off = 0.0 if offset is None else np.repeat(decode(offset, dtype).reshape(N, groups), gs, axis=1)
    w = (qi.astype(np.float64) + off) * sc
    return decode(round_to(w, dtype), dtype) if round_weights else w


def experts_forward_quant(x_disp, offsets, quant_of, bits, groups, dtype, round_weights=False):
    """Expert outputs for every dispatched row with quantised weights: the
    SwiGLU expert of swiglu_expert_f64 on the dequantised weights of
    dequant_weight (round_weights as there).
    quant_of(e) -> ((q_gate, s_gate, o_gate), (q_up, s_up, o_up),
    (q_down, s_down, o_down)) for expert e."""
    def weights_f64(e):
        return [dequant_weight(q, bits, sc, off, groups, dtype, round_weights) for q, sc, off in quant_of(e)]
    R = int(offsets[-1])
    out = None
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        y = swiglu_expert_f64(x_disp[a:b], *weights_f64(e), dtype)
        if out is None:
            out = np.empty((R, y.shape[1]), dtype=y.dtype)
        out[a:b] = y
    return out


def experts_forward_dispatched(x_disp: np.ndarray, offsets: np.ndarray, weights_of, dtype: str):
    """Expert outputs for every dispatched row, in dispatched order.
    weights_of(e) -> (gate [I,H], up [I,H], down [H,I]) for expert e."""
    R = int(offsets[-1])
    E = len(offsets) - 1
    out = None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        y = swiglu_expert(x_disp[a:b], *weights_of(e), dtype)
        if out is None:
            out = np.empty((R, y.shape[1]), dtype=y.dtype)
        out[a:b] = y
    return out


# --------------------------------------------------------------------------
# combine  (ruDNN user guide, "6. Calling MoE": combine restores token order
# with the saved map and merges expert outputs using the routing weights)
# --------------------------------------------------------------------------
def combine_fp64(expert_out, row_of_slot, weights, w_dtype, T, k, dtype):
    """c[t] = sum_{j<k} w[t,j] * expert_out[row_of_slot[t*k+j]] in fp64; a token
    with an unassigned slot (row -1) gets a NaN row."""
    rows = row_of_slot.reshape(T, k).astype(np.int64)
    w = decode(weights, w_dtype).reshape(T, k)
    H = expert_out.shape[1] if expert_out is not None and expert_out.ndim == 2 else 0
    c = np.zeros((T, H), dtype=np.float64)
    y = decode(expert_out, dtype) if H else None
    for j in range(k):
        rj = rows[:, j]
        good = rj >= 0
        contrib = np.full((T, H), np.nan)
        contrib[good] = w[good, j][:, None] * y[rj[good]]
        c += contrib
    return c


def combine(expert_out, row_of_slot, weights, w_dtype, T, k, dtype):
    """out [T, H] in the model dtype."""
    return round_to(combine_fp64(expert_out, row_of_slot, weights, w_dtype, T, k, dtype), dtype)


def combine_add_rmsnorm(expert_out, row_of_slot, weights, w_dtype, shared, residual,
                        gamma, eps, T, k, dtype):
    """aclnnMoeDistributeCombineAddRmsNormV2, formula (local part):
      combineOut = sum_j (w_j * y_j + w_j * s)      s = shared-expert row (0 if absent)
      x          = combineOut + residual
      rstd       = 1 / sqrt(mean_H(x^2) + eps)
      y          = x * rstd * gamma
    Returns (y, x_out) in the model dtype and rstd fp32 [T]. Statistics use the
    unrounded x; gamma is fp32 (ruDNN user guide, "7. LayerNorm, RMSNorm and
    Softmax": affine parameters stay F32)."""
    c = combine_fp64(expert_out, row_of_slot, weights, w_dtype, T, k, dtype)
    if shared is not None:
        wsum = decode(weights, w_dtype).reshape(T, k).sum(axis=1)
        c = c + wsum[:, None] * decode(shared, dtype)
    x = c + decode(residual, dtype)
    rstd = 1.0 / np.sqrt((x * x).mean(axis=1) + float(eps))
    y = x * rstd[:, None] * np.asarray(gamma, dtype=np.float32).astype(np.float64)[None, :]
    return round_to(y, dtype), round_to(x, dtype), rstd.astype(np.float32)


def combine_special_fp64(expert_out, row_of_slot, indices, weights, w_dtype, T, k, dtype, E,
                         zero_num=0, copy_num=0, const_num=0, ori_x=None, alpha1=None,
                         alpha2=None, const_v=None, active=None, shared=None):
    """aclnnMoeDistributeCombineAddRmsNormV2 with special experts and the
    activity mask (local part), in fp64:
      c[t] = sum over active slots j of w[t,j] * (Moe_j + s[t])
    where, for e = indices[t, j]:
      e < E                      Moe = expert_out[row_of_slot[t*k+j]]
      E <= e < E+zero_num        Moe = 0                         (zero expert)
      next copy_num ids          Moe = ori_x[t]                  (copy expert)
      next const_num ids (q)     Moe = alpha1[q]*ori_x[t] + alpha2[q]*V[q]
    Any other id, or a real-expert slot that was not dispatched (row -1), makes
    the row NaN. A token with no active slot combines to 0."""
    idx = np.asarray(indices).reshape(T, k).astype(np.int64)
    rows = np.asarray(row_of_slot).reshape(T, k).astype(np.int64)
    w = decode(weights, w_dtype).reshape(T, k)
    H = expert_out.shape[1]
    y = decode(expert_out, dtype)
    ox = decode(ori_x, dtype) if ori_x is not None else None
    a1 = decode(alpha1, dtype) if const_num else None
    a2 = decode(alpha2, dtype) if const_num else None
    V = decode(const_v, dtype) if const_num else None
    sh = decode(shared, dtype) if shared is not None else None
    if active is None:
        on = np.ones((T, k), bool)
    else:
        a = np.asarray(active, bool)
        on = np.repeat(a[:, None], k, axis=1) if a.ndim == 1 else a.reshape(T, k)
    c = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if not on[t, j]:
                continue
            e, d = idx[t, j], idx[t, j] - E
            if d < 0:
                m = y[rows[t, j]] if rows[t, j] >= 0 else np.full(H, np.nan)
            elif d < zero_num:
                m = np.zeros(H)
            elif d < zero_num + copy_num:
                m = ox[t]
            elif d < zero_num + copy_num + const_num:
                q = d - zero_num - copy_num
                m = a1[q] * ox[t] + a2[q] * V[q]
            else:
                m = np.full(H, np.nan)
            c[t] += w[t, j] * (m + (sh[t] if sh is not None else 0.0))
    return c


def combine_special(*args, **kw):
    """out [T, H] in the model dtype; arguments as combine_special_fp64."""
    dtype = args[7] if len(args) > 7 else kw["dtype"]
    return round_to(combine_special_fp64(*args, **kw), dtype)


def combine_add_rmsnorm_special(residual, gamma, eps, *args, **kw):
    """The whole aclnnMoeDistributeCombineAddRmsNormV2 formula with special
    experts and the activity mask: x = combine_special_fp64(...) + residual,
    rstd = 1/sqrt(mean_H(x^2) + eps), y = x * rstd * gamma. Returns (y, x_out)
    in the model dtype and rstd fp32 [T]."""
    dtype = args[7] if len(args) > 7 else kw["dtype"]
    x = combine_special_fp64(*args, **kw) + decode(residual, dtype)
    rstd = 1.0 / np.sqrt((x * x).mean(axis=1) + float(eps))
    y = x * rstd[:, None] * np.asarray(gamma, dtype=np.float32).astype(np.float64)[None, :]
    return round_to(y, dtype), round_to(x, dtype), rstd.astype(np.float32)


# --------------------------------------------------------------------------
# whole local forward  (ruDNN user guide, "6. Calling MoE": forward(input,
# logits, options) = route -> dispatch -> forward_dispatched -> combine)
# --------------------------------------------------------------------------
def forward(x, logits, logits_dtype, top_k, renormalize, weights_of, E, dtype):
    idx, w = route(logits, logits_dtype, top_k, renormalize)
    d = dispatch(idx, E, x)
    T = x.shape[0]
    y = experts_forward_dispatched(d["x_disp"], d["offsets"], weights_of, dtype)
    if y is None:
        return idx, w, d, None, round_to(np.zeros((T, x.shape[1])), dtype)
    return idx, w, d, y, combine(y, d["row_of_slot"], w, logits_dtype, T, top_k, dtype)


def forward_sigmoid_grouped(x, logits, logits_dtype, bias, top_k, groups, selected_groups,
                            group_top_two, renormalize, scale, weights_of, E, dtype):
    """SwiGluExperts::forward_sigmoid_grouped (ruDNN user guide, "10. Grouped-
    limited sigmoid MoE routing"): the grouped sigmoid routing plan, then the
    same dispatch, experts and combine as forward()."""
    idx, w = route_sigmoid_grouped(logits, logits_dtype, bias, top_k, groups, selected_groups,
                                   group_top_two, renormalize, scale)
    d = dispatch(idx, E, x)
    T = x.shape[0]
    y = experts_forward_dispatched(d["x_disp"], d["offsets"], weights_of, dtype)
    if y is None:
        return idx, w, d, None, round_to(np.zeros((T, x.shape[1])), dtype)
    return idx, w, d, y, combine(y, d["row_of_slot"], w, logits_dtype, T, top_k, dtype)


def expert_out_rows(x, indices, tokens, weights_of, dtype):
    """Expert outputs for the (token, slot) pairs of the given tokens only:
    returns {(t, j): y row} computed one by one, for sampled checks at sizes
    where the full forward is too slow. x [T, H]; indices [T, k]."""
    need = {}
    for t in tokens:
        for j, e in enumerate(indices[t]):
            need.setdefault(int(e), []).append((int(t), j))
    out = {}
    for e, pairs in sorted(need.items()):
        wg, wu, wd = weights_of(e)
        rows = np.stack([x[t] for t, _ in pairs])
        y = swiglu_expert(rows, wg, wu, wd, dtype)
        for (t, j), yr in zip(pairs, y):
            out[(t, j)] = yr
    return out


# --------------------------------------------------------------------------
# training: weights for a fixed selection and the backward pass  (ruDNN
# user guide, "12. MoE first-order training")
# --------------------------------------------------------------------------
SOFTMAX, SIGMOID = 0, 1


def _index_rows_invalid(indices, E):
    """Rows holding an index outside [0, E): their weights and gradients are NaN."""
    i = np.asarray(indices).astype(np.int64)
    return ((i < 0) | (i >= E)).any(axis=1)


def router_selected_weights(logits, logits_dtype, indices, scoring, normalize, scale):
    """selected_router_weights: fp32 [T, k] weights of a fixed selection.
    scoring SOFTMAX: the fp32 softmax over all E gathered at the indices;
    SIGMOID: the fp32 sigmoid of the selected logits. Repeated indices gather
    the same score again. With normalize the k gathered scores are divided by
    their sum; then every weight is multiplied by scale. A row holding an
    index outside [0, E) is NaN throughout."""
    z = decode(logits, logits_dtype)
    T, E = z.shape
    idx = np.asarray(indices).astype(np.int64)
    bad = _index_rows_invalid(idx, E)
    safe = np.where(bad[:, None], 0, idx)
    score = softmax_fp32(logits, logits_dtype) if scoring == SOFTMAX else sigmoid_fp32(logits, logits_dtype)
    s = np.take_along_axis(score, safe, axis=1).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        w = s / s.sum(axis=1, keepdims=True) if normalize else s
    w = w * float(np.float32(scale))
    w[bad] = np.nan
    return w.astype(np.float32)


def router_selected_backward(logits, logits_dtype, indices, grad_weights, scoring, normalize, scale):
    """selected_router_backward: d loss / d logits [T, E] in the logits dtype,
    for the weights of router_selected_weights with the selection held fixed.
    By the chain rule, with a the gathered score of slot j, S the sum of the
    gathered scores (normalize) and c the scale:
        w_j = c * a_j / S            (S = 1 without normalize)
        dw_j/dz_e = c * (da_j/dz_e / S - a_j / S^2 * sum_m da_m/dz_e)
    where for the softmax da_j/dz_e = p_{i_j} (delta(i_j, e) - p_e) and for
    the sigmoid da_j/dz_e = delta(i_j, e) s_e (1 - s_e). The scores are the
    exact fp64 ones; the Jacobian is formed explicitly, token by token."""
    z = decode(logits, logits_dtype)
    T, E = z.shape
    idx = np.asarray(indices).astype(np.int64)
    k = idx.shape[1]
    g = np.asarray(grad_weights, np.float32).astype(np.float64).reshape(T, k)
    c = float(np.float32(scale))
    bad = _index_rows_invalid(idx, E)
    out = np.full((T, E), np.nan)
    for t in range(T):
        if bad[t]:
            continue
        zt = z[t]
        if scoring == SOFTMAX:
            if invalid_rows(zt[None, :])[0]:
                continue
            a_all = np.exp(zt - zt.max())
            p = a_all / a_all.sum()
            dscore = np.diag(p) - np.outer(p, p)      # d p_a / d z_e
            score = p
        else:
            with np.errstate(over="ignore"):
                s = 1.0 / (1.0 + np.exp(-zt))
            dscore = np.diag(s * (1.0 - s))
            score = s
        a = score[idx[t]]                              # [k]
        da = dscore[idx[t]]                            # [k, E]
        if normalize:
            S = a.sum()
            with np.errstate(invalid="ignore", divide="ignore"):
                jac = c * (da / S - np.outer(a, da.sum(axis=0)) / S ** 2)
        else:
            jac = c * da
        out[t] = g[t] @ jac
    return round_to(out, logits_dtype)


def combine_backward(expert_out, row_of_slot, weights, w_dtype, grad_out, T, k, dtype):
    """combine_backward of out[t] = sum_j w[t,j] y[row(t,j)]:
      dexpert[row(t,j)] = w[t,j] * grad_out[t]          (model dtype, one rounding)
      dweights[t, j]    = sum_h grad_out[t,h] y[row(t,j),h]   (fp32)
    A slot without a dispatched row has dweights NaN (the forward made that
    token's row NaN) and no dexpert row."""
    rows = np.asarray(row_of_slot).astype(np.int64).reshape(T, k)
    w = decode(weights, w_dtype).reshape(T, k)
    go = decode(grad_out, dtype)
    y = decode(expert_out, dtype)
    R, H = y.shape
    dexp = np.zeros((R, H))
    dw = np.full((T, k), np.nan)
    for t in range(T):
        for j in range(k):
            r = rows[t, j]
            if r < 0:
                continue
            dexp[r] = w[t, j] * go[t]
            dw[t, j] = go[t] @ y[r]
    return round_to(dexp, dtype), dw.astype(np.float32)


def swiglu_expert_training(x_rows, w_gate_e, w_up_e, w_down_e, dtype):
    """Training forward of one expert: returns (y, g, u, h), all in the model
    dtype. The cache keeps the gate and up projections rounded to the model
    dtype, and h is formed from those cached values:
      g = round(x W_gate^T), u = round(x W_up^T), h = round(SiLU(g) u),
      y = round(h W_down^T)."""
    x = decode(x_rows, dtype)
    g = round_to(x @ decode(w_gate_e, dtype).T, dtype)
    u = round_to(x @ decode(w_up_e, dtype).T, dtype)
    h = round_to(silu(decode(g, dtype)) * decode(u, dtype), dtype)
    y = round_to(decode(h, dtype) @ decode(w_down_e, dtype).T, dtype)
    return y, g, u, h


def swiglu_expert_backward(x_rows, w_gate_e, w_up_e, w_down_e, g, u, h, dy, dtype, terms=False):
    """cache.backward of one expert, from its training cache (g, u, h) and the
    gradient dy of its output rows:
      dh = dy W_down                                   (not rounded)
      sigma = 1 / (1 + exp(-g)),  SiLU'(g) = sigma (1 + g (1 - sigma))
      dg = round(dh * u * SiLU'(g)),  du = round(dh * SiLU(g))
      dinput = round(dg W_gate + du W_up)              [n, H], model dtype
      dgate = dg^T x, dup = du^T x, ddown = dy^T h     fp32
    Returns (dinput, dgate [I, H], dup [I, H], ddown [H, I]), and with
    terms=True also the rounded dg and du as fp64 values."""
    x = decode(x_rows, dtype)
    wg, wu, wd = decode(w_gate_e, dtype), decode(w_up_e, dtype), decode(w_down_e, dtype)
    gv, uv, hv, dyv = decode(g, dtype), decode(u, dtype), decode(h, dtype), decode(dy, dtype)
    dh = dyv @ wd
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-gv))
    dg = decode(round_to(dh * uv * sig * (1.0 + gv * (1.0 - sig)), dtype), dtype)
    du = decode(round_to(dh * gv * sig, dtype), dtype)
    dinput = round_to(dg @ wg + du @ wu, dtype)
    out = (dinput, (dg.T @ x).astype(np.float32), (du.T @ x).astype(np.float32),
           (dyv.T @ hv).astype(np.float32))
    return out + (dg, du) if terms else out


def experts_forward_training(x_disp, offsets, weights_of, dtype):
    """forward_dispatched_training over all experts: (expert_out [R, H],
    g [R, I], u [R, I], h [R, I]), rows in dispatched order."""
    R = int(offsets[-1])
    parts = None
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        outs = swiglu_expert_training(x_disp[a:b], *weights_of(e), dtype)
        if parts is None:
            parts = [np.empty((R,) + o.shape[1:], dtype=o.dtype) for o in outs]
        for p, o in zip(parts, outs):
            p[a:b] = o
    return parts


def experts_backward(x_disp, offsets, weights_of, g, u, h, dexpert, dtype, terms=False):
    """cache.backward over all experts: (dinput [R, H] model dtype, dgate
    [E, I, H], dup [E, I, H], ddown [E, H, I] fp32), and with terms=True also
    dg, du [R, I] (fp64 values of the rounded terms). Experts without rows
    get zero weight gradients."""
    E = len(offsets) - 1
    R = int(offsets[-1])
    H = x_disp.shape[1] if R else 0
    dinput = None
    dgate = dup = ddown = None
    for e in range(E):
        wg, wu, wd = weights_of(e)
        if dgate is None:
            I_, Hh = wg.shape
            dgate = np.zeros((E, I_, Hh), np.float32)
            dup = np.zeros((E, I_, Hh), np.float32)
            ddown = np.zeros((E, Hh, I_), np.float32)
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        di, dgt, dut, ddn, dgv, duv = swiglu_expert_backward(x_disp[a:b], wg, wu, wd, g[a:b], u[a:b], h[a:b],
                                                             dexpert[a:b], dtype, terms=True)
        if dinput is None:
            dinput = np.empty((R, H), dtype=di.dtype)
            dg_all, du_all = np.zeros((R, I_)), np.zeros((R, I_))
        dinput[a:b] = di
        dg_all[a:b], du_all[a:b] = dgv, duv
        dgate[e], dup[e], ddown[e] = dgt, dut, ddn
    if terms:
        if dinput is None:
            dg_all = du_all = np.zeros((0, dgate.shape[1] if dgate is not None else 0))
        return dinput, dgate, dup, ddown, dg_all, du_all
    return dinput, dgate, dup, ddown


def dispatch_backward(dinput, row_of_slot, T, k, H, dtype):
    """dispatch_backward: dx[t] = sum over the slots j of token t that have a
    dispatched row of dinput[row(t,j)], without the routing weight (the
    weight was applied in combine_backward); one rounding to the model dtype.
    A token with no dispatched slot gets zeros."""
    rows = np.asarray(row_of_slot).astype(np.int64).reshape(T, k)
    d = decode(dinput, dtype) if dinput is not None and len(dinput) else np.zeros((0, H))
    dx = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if rows[t, j] >= 0:
                dx[t] += d[rows[t, j]]
    return round_to(dx, dtype)
