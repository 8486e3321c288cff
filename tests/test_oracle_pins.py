"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms
(tests/golden), brute force on tiny inputs, special cases that reduce to a
library routine (torch softmax, torch rms_norm, torch bf16 cast, stable
argsort, bincount), and invariants. The cases are chosen so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(s):
    if s.startswith("ln"):
        return math.log(int(s[2:]))
    return float(s)


def _frac(s):
    if s == "nan":
        return float("nan")
    return float(Fraction(s))


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- rounding --
def test_bf16_round_matches_torch_on_fp32_inputs():
    x = torch.randn(200000, dtype=torch.float32) * torch.exp(torch.randn(200000) * 20)
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = O.round_to(x.numpy().astype(np.float64), "bf16")
    assert (ref == got).all()


def test_bf16_round_ties_and_specials():
    # 1 + 2^-8 is exactly between 1 and 1+2^-7: ties to even -> 1.0 (0x3F80)
    # 1 + 3*2^-8 is between 1+2^-7 and 1+2^-6: ties to even -> 1+2^-6 (0x3F82)
    cases = [(1.0 + 2**-8, 0x3F80), (1.0 + 3 * 2**-8, 0x3F82),
             # just above the tie, in fp64 only (fp32 would round to the tie first)
             (1.0 + 2**-8 + 2**-40, 0x3F81),
             (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
             (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
             (3.4e38, 0x7F80),  # past the largest finite bf16 once rounded
             (2.0**-133, 0x0001),  # smallest bf16 subnormal
             (2.0**-134, 0x0000),  # tie between 0 and 2^-133 -> even (0)
             (3 * 2.0**-134, 0x0002)]
    for v, bits in cases:
        assert int(O.round_to(np.array([v]), "bf16")[0]) == bits, v
    assert np.isnan(O.decode(O.round_to(np.array([np.nan]), "bf16"), "bf16")[0])


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert (O.decode(bits, "bf16") == ref).all()


# ----------------------------------------------------------------- routing --
def test_routing_golden_closed_forms():
    spec = json.load(open(os.path.join(GOLDEN, "routing_closed_form.json")))
    for case in spec["cases"]:
        z = np.array([[_num(s) for s in case["logits"]]], dtype=np.float32)
        idx, w = O.route(z, "f32", case["top_k"], case["renormalize"])
        assert idx[0].tolist() == case["indices"], case["name"]
        exp = np.array([_frac(s) for s in case["weights"]])
        got = w[0].astype(np.float64)
        assert (np.isnan(got) == np.isnan(exp)).all(), case["name"]
        ok = ~np.isnan(exp)
        # fp32 softmax, one renormalisation and one cast: a few fp32 ulps
        assert np.allclose(got[ok], exp[ok], rtol=4e-7, atol=0), (case["name"], got, exp)


def test_softmax_matches_torch():
    z = rng(1).standard_normal((300, 37)).astype(np.float32) * 4
    ref = torch.softmax(torch.from_numpy(z).double(), dim=-1).float().numpy()
    got = O.softmax_fp32(z, "f32")
    assert np.array_equal(got, ref) or np.abs(got - ref).max() <= 1e-7 * ref.max()
    assert np.allclose(got.sum(axis=1), 1.0, atol=1e-6)


def test_topk_equals_E_is_sorted_softmax():
    z = rng(2).standard_normal((64, 16)).astype(np.float32)
    idx, w = O.route(z, "f32", 16, False)
    p = torch.softmax(torch.from_numpy(z).double(), dim=-1).float()
    vals, order = torch.sort(p, dim=-1, descending=True, stable=True)
    assert (idx.astype(np.int64) == order.numpy()).all()
    assert np.array_equal(w, vals.numpy())


def _brute_topk(p, k):
    """Exhaustive: the k-subset with the largest probabilities in
    (p desc, id asc) order is the one whose sorted key list is
    lexicographically best; listed best first."""
    E = len(p)
    best = None
    for sub in itertools.combinations(range(E), k):
        key = sorted(((-p[i], i) for i in sub))
        if best is None or key < best:
            best = key
    return [i for _, i in best]


@pytest.mark.parametrize("E", [1, 2, 3, 5, 6])
def test_topk_brute_force_tiny(E):
    g = rng(10 + E)
    for trial in range(40):
        # quantised logits force many exact ties
        z = (g.integers(-3, 4, size=(1, E)) * 0.5).astype(np.float32)
        p = O.softmax_fp32(z, "f32")[0]
        for k in range(1, E + 1):
            idx, _ = O.route(z, "f32", k, False)
            assert idx[0].tolist() == _brute_topk(p.tolist(), k)


def test_renormalize_invariants():
    z = rng(3).standard_normal((500, 64)).astype(np.float32)
    for k in (1, 2, 8, 64):
        idx, w = O.route(z, "f32", k, True)
        assert np.abs(w.astype(np.float64).sum(axis=1) - 1).max() <= k * 2.0**-23
        assert (np.diff(w.astype(np.float64), axis=1) <= 0).all()
        idx2, w2 = O.route(z, "f32", k, False)
        assert (idx == idx2).all()
        assert (w2.astype(np.float64).sum(axis=1) <= 1 + 64 * 2.0**-24).all()
        # renormalised = plain / sum(plain)
        ratio = w2.astype(np.float64) / w2.astype(np.float64).sum(axis=1, keepdims=True)
        assert np.allclose(w, ratio, rtol=3e-7, atol=0)


def test_k1_renormalized_weight_is_exactly_one():
    z = rng(4).standard_normal((200, 9)).astype(np.float32)
    idx, w = O.route(z, "f32", 1, True)
    assert (w == 1.0).all()
    assert (idx[:, 0] == z.argmax(axis=1)).all()


def test_nan_contract_rows_isolated():
    z = rng(5).standard_normal((6, 10)).astype(np.float32)
    idx0, w0 = O.route(z, "f32", 3, True)
    z2 = z.copy()
    z2[1, 4] = np.nan
    z2[3, 0] = np.inf
    z2[5, :] = -np.inf
    idx, w = O.route(z2, "f32", 3, True)
    for r in (1, 3, 5):
        assert idx[r].tolist() == [0, 1, 2]
        assert np.isnan(w[r]).all()
    for r in (0, 2, 4):
        assert (idx[r] == idx0[r]).all() and np.array_equal(w[r], w0[r])


def test_weights_take_logits_dtype():
    z32 = rng(6).standard_normal((50, 8)).astype(np.float32)
    zb = O.round_to(z32.astype(np.float64), "bf16")
    idx, w = O.route(zb, "bf16", 2, True)
    assert w.dtype == np.uint16
    zf = O.decode(zb, "bf16").astype(np.float32)
    idx_f, w_f = O.route(zf, "f32", 2, True)
    assert (idx == idx_f).all()
    # one rounding into bf16: within half a bf16 ulp, i.e. 2^-8 relative (plus fp32 rounding)
    wd = O.decode(w, "bf16")
    assert (np.abs(wd - w_f) <= (2.0**-8 + 2.0**-23) * np.abs(w_f)).all()
    z16 = z32.astype(np.float16)
    idx16, w16 = O.route(z16, "f16", 2, False)
    assert w16.dtype == np.float16


def test_route_rejects_bad_top_k():
    z = np.zeros((2, 4), np.float32)
    for k in (0, 5):
        with pytest.raises(ValueError):
            O.route(z, "f32", k, True)


# ---------------------------------------------------------------- dispatch --
def test_dispatch_invariants():
    g = rng(7)
    T, k, E, H = 97, 3, 11, 5
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.uint32)
    x = g.standard_normal((T, H)).astype(np.float32)
    d = O.dispatch(idx, E, x)
    counts = np.bincount(idx.ravel().astype(np.int64), minlength=E)
    assert (np.diff(d["offsets"]) == counts).all() and d["offsets"][0] == 0
    assert d["offsets"][-1] == T * k
    order = np.argsort(idx.ravel(), kind="stable")
    assert (d["slot_of_row"] == order).all()
    assert (d["row_of_slot"][d["slot_of_row"]] == np.arange(T * k)).all()
    assert np.array_equal(d["x_disp"], x[order // k])
    # every row of expert e holds a slot routed to e
    for e in range(E):
        sl = d["slot_of_row"][d["offsets"][e]:d["offsets"][e + 1]]
        assert (idx.ravel()[sl] == e).all()


def test_dispatch_out_of_range_ids_are_dropped():
    idx = np.array([[0, 5], [2, 1], [9, 0]], dtype=np.uint32)
    d = O.dispatch(idx, 3)
    assert d["offsets"].tolist() == [0, 2, 3, 4]
    assert d["row_of_slot"].tolist() == [0, -1, 3, 2, -1, 1]
    assert d["slot_of_row"].tolist() == [0, 5, 3, 2]


# ----------------------------------------------------------------- experts --
def _torch_swiglu(x, wg, wu, wd):
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def test_swiglu_expert_fp32_matches_dense_torch():
    g = rng(8)
    n, H, I = 7, 12, 20  # H != I so a transposed operand cannot pass
    x = g.standard_normal((n, H)).astype(np.float32)
    wg = g.standard_normal((I, H)).astype(np.float32) / np.sqrt(H)
    wu = g.standard_normal((I, H)).astype(np.float32) / np.sqrt(H)
    wd = g.standard_normal((H, I)).astype(np.float32) / np.sqrt(I)
    got = O.swiglu_expert(x, wg, wu, wd, "f32").astype(np.float64)
    ref = _torch_swiglu(x, wg, wu, wd).numpy()
    # the oracle rounds h to fp32 once; that bounds the difference
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)
    # swapping gate and up changes the result (SiLU applies to the gate)
    swapped = O.swiglu_expert(x, wu, wg, wd, "f32").astype(np.float64)
    assert not np.allclose(swapped, ref, rtol=1e-3, atol=1e-3)


def test_swiglu_expert_bf16_rounding_points():
    g = rng(9)
    n, H, I = 5, 16, 24
    b = lambda a: O.round_to(a, "bf16")  # noqa: E731
    x, wg, wu = b(g.standard_normal((n, H))), b(g.standard_normal((I, H)) / 4), b(g.standard_normal((I, H)) / 4)
    wd = b(g.standard_normal((H, I)) / 5)
    got = O.swiglu_expert(x, wg, wu, wd, "bf16")
    xt, wgt, wut, wdt = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double() for a in (x, wg, wu, wd))
    h = (torch.nn.functional.silu(xt @ wgt.T) * (xt @ wut.T)).to(torch.bfloat16).double()
    ref = (h @ wdt.T).numpy()
    gotd = O.decode(got, "bf16")
    # torch's double->bf16 cast passes through fp32; allow one bf16 ulp
    assert np.allclose(gotd, ref, rtol=2.0**-7, atol=1e-30)


def test_power_of_two_linearity_of_down_projection():
    g = rng(10)
    n, H, I = 6, 8, 12
    b = lambda a: O.round_to(a, "bf16")  # noqa: E731
    x, wg, wu, wd = b(g.standard_normal((n, H))), b(g.standard_normal((I, H))), b(g.standard_normal((I, H))), b(g.standard_normal((H, I)))
    y1 = O.decode(O.swiglu_expert(x, wg, wu, wd, "bf16"), "bf16")
    wd2 = O.round_to(2 * O.decode(wd, "bf16"), "bf16")
    y2 = O.decode(O.swiglu_expert(x, wg, wu, wd2, "bf16"), "bf16")
    assert np.array_equal(2 * y1, y2)


def _weights(g, E, H, I):
    wg = g.standard_normal((E, I, H)).astype(np.float32) / np.sqrt(H)
    wu = g.standard_normal((E, I, H)).astype(np.float32) / np.sqrt(H)
    wd = g.standard_normal((E, H, I)).astype(np.float32) / np.sqrt(I)
    return wg, wu, wd


def test_forward_one_hot_equals_dense_swiglu_of_argmax_expert():
    g = rng(11)
    T, H, I, E = 33, 10, 14, 5
    x = g.standard_normal((T, H)).astype(np.float32)
    z = g.standard_normal((T, E)).astype(np.float32)
    wg, wu, wd = _weights(g, E, H, I)
    idx, w, d, y, out = O.forward(x, z, "f32", 1, True, lambda e: (wg[e], wu[e], wd[e]), E, "f32")
    assert (w == 1.0).all()
    am = z.argmax(axis=1)
    ref = np.stack([_torch_swiglu(x[t:t + 1], wg[am[t]], wu[am[t]], wd[am[t]]).numpy()[0] for t in range(T)])
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_single_expert_reduces_to_dense_swiglu():
    g = rng(12)
    T, H, I = 9, 6, 10
    x = g.standard_normal((T, H)).astype(np.float32)
    z = g.standard_normal((T, 1)).astype(np.float32)
    wg, wu, wd = _weights(g, 1, H, I)
    _, _, _, _, out = O.forward(x, z, "f32", 1, False, lambda e: (wg[e], wu[e], wd[e]), 1, "f32")
    ref = _torch_swiglu(x, wg[0], wu[0], wd[0]).numpy()
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_forward_top2_matches_weighted_dense_mixture():
    """Dense reference: every expert on every token, weighted by the routing
    weights of the selected experts (zero elsewhere)."""
    g = rng(13)
    T, H, I, E, k = 21, 8, 12, 6, 2
    x = g.standard_normal((T, H)).astype(np.float32)
    z = g.standard_normal((T, E)).astype(np.float32)
    wg, wu, wd = _weights(g, E, H, I)
    idx, w, d, y, out = O.forward(x, z, "f32", k, True, lambda e: (wg[e], wu[e], wd[e]), E, "f32")
    dense = np.stack([_torch_swiglu(x, wg[e], wu[e], wd[e]).numpy() for e in range(E)], 1)  # [T,E,H]
    gate = np.zeros((T, E))
    p = torch.softmax(torch.from_numpy(z).double(), -1).numpy()
    top = np.argsort(-p, axis=1, kind="stable")[:, :k]
    for t in range(T):
        gate[t, top[t]] = p[t, top[t]] / p[t, top[t]].sum()
    ref = np.einsum("te,teh->th", gate, dense)
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-6)


def test_expert_out_rows_matches_full_forward():
    g = rng(14)
    T, H, I, E, k = 40, 8, 12, 5, 2
    x = g.standard_normal((T, H)).astype(np.float32)
    z = g.standard_normal((T, E)).astype(np.float32)
    wg, wu, wd = _weights(g, E, H, I)
    wo = lambda e: (wg[e], wu[e], wd[e])  # noqa: E731
    idx, w, d, y, out = O.forward(x, z, "f32", k, True, wo, E, "f32")
    rows = O.expert_out_rows(x, idx, [0, 7, 39], wo, "f32")
    for (t, j), yr in rows.items():
        assert np.array_equal(yr, y[d["row_of_slot"][t * k + j]])


# ----------------------------------------------------------------- combine --
def test_combine_k1_unit_weight_is_exact_gather():
    g = rng(15)
    T, H = 12, 9
    y = O.round_to(g.standard_normal((T, H)), "bf16")
    perm = g.permutation(T).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    out = O.combine(y, perm, w, "f32", T, 1, "bf16")
    assert np.array_equal(out, y[perm])


def test_combine_weighted_sum_matches_torch():
    g = rng(16)
    T, k, H = 10, 3, 7
    y = g.standard_normal((T * k, H)).astype(np.float32)
    ros = g.permutation(T * k).astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    out = O.combine(y, ros, w, "f32", T, k, "f32")
    ref = torch.einsum("tj,tjh->th", torch.from_numpy(w).double(),
                       torch.from_numpy(y).double()[torch.from_numpy(ros).long()].reshape(T, k, H))
    assert np.allclose(out, ref.numpy(), rtol=1e-7, atol=1e-7)


def test_combine_unassigned_slot_gives_nan_row():
    y = np.ones((3, 4), np.float32)
    out = O.combine(y, np.array([0, -1, 1, 2], np.int32), np.ones((2, 2), np.float32), "f32", 2, 2, "f32")
    assert np.isnan(out[0]).all() and (out[1] == 2).all()


def test_rmsnorm_matches_torch_rms_norm():
    g = rng(17)
    T, k, H = 6, 2, 32
    y = g.standard_normal((T * k, H)).astype(np.float32)
    ros = np.arange(T * k, dtype=np.int32)
    w = np.full((T, k), 0.5, np.float32)
    res = g.standard_normal((T, H)).astype(np.float32)
    gamma = g.uniform(0.5, 1.5, H).astype(np.float32)
    yo, xo, rstd = O.combine_add_rmsnorm(y, ros, w, "f32", None, res, gamma, 1e-6, T, k, "f32")
    x = torch.from_numpy(y).double().reshape(T, k, H).mul(0.5).sum(1) + torch.from_numpy(res).double()
    ref = torch.nn.functional.rms_norm(x, (H,), torch.from_numpy(gamma).double(), 1e-6)
    assert np.allclose(yo, ref.numpy(), rtol=1e-6, atol=1e-6)
    assert np.allclose(xo, x.numpy(), rtol=1e-7, atol=1e-7)
    assert np.allclose(rstd, torch.rsqrt(x.pow(2).mean(-1) + 1e-6).numpy(), rtol=1e-7)


def test_rmsnorm_constant_rows_closed_form():
    T, H, c, eps = 3, 16, 0.75, 1e-6
    y = np.zeros((T, H), np.float32)
    res = np.full((T, H), c, np.float32)
    gamma = np.full(H, 2.0, np.float32)
    yo, xo, rstd = O.combine_add_rmsnorm(y, np.arange(T, dtype=np.int32), np.ones((T, 1), np.float32),
                                         "f32", None, res, gamma, eps, T, 1, "f32")
    r = 1 / math.sqrt(c * c + eps)
    assert np.allclose(rstd, r, rtol=1e-7)
    assert np.allclose(yo, 2 * c * r, rtol=1e-7)
    assert (xo == c).all()


def test_shared_term_reading_equals_sum_plus_shared_when_renormalized():
    g = rng(18)
    T, k, H = 8, 3, 10
    y = g.standard_normal((T * k, H)).astype(np.float32)
    ros = np.arange(T * k, dtype=np.int32)
    z = g.standard_normal((T, 6)).astype(np.float32)
    _, w = O.route(z, "f32", k, True)
    s = g.standard_normal((T, H)).astype(np.float32)
    r = g.standard_normal((T, H)).astype(np.float32)
    gamma = np.ones(H, np.float32)
    _, xo, _ = O.combine_add_rmsnorm(y, ros, w, "f32", s, r, gamma, 1e-6, T, k, "f32")
    ref = np.einsum("tj,tjh->th", w.astype(np.float64), y.reshape(T, k, H).astype(np.float64)) + s + r
    assert np.allclose(xo, ref, rtol=1e-6, atol=1e-6)


def test_rmsnorm_nan_weights_propagate_to_row_only():
    T, k, H = 3, 2, 8
    y = np.ones((T * k, H), np.float32)
    w = np.full((T, k), 0.5, np.float32)
    w[1] = np.nan
    yo, xo, rstd = O.combine_add_rmsnorm(y, np.arange(T * k, dtype=np.int32), w, "f32", None,
                                         np.zeros((T, H), np.float32), np.ones(H, np.float32), 1e-6, T, k, "f32")
    assert np.isnan(yo[1]).all() and np.isnan(rstd[1])
    assert np.isfinite(yo[[0, 2]]).all()


# --------------------------------------------------------------------------
# grouped-limited sigmoid routing (ruDNN user guide, "10. Grouped-limited
# sigmoid MoE routing")
# --------------------------------------------------------------------------
def _sig(z):
    return torch.sigmoid(torch.tensor(z, dtype=torch.float64)).float().numpy()


def test_grouped_sigmoid_one_group_is_topk_of_sigmoid():
    """One group holding every expert: selection is the plain top-k of the
    sigmoid scores (torch.topk on torch.sigmoid); weights are those scores,
    divided by their sum when renormalised, times scale."""
    rng = np.random.default_rng(11)
    z = rng.standard_normal((64, 48)).astype(np.float32)
    for renorm, scale in ((True, 2.5), (False, 1.0)):
        idx, w = O.route_sigmoid_grouped(z, "f32", None, 6, 1, 1, False, renorm, scale)
        s = _sig(z)
        ref_w, ref_i = torch.topk(torch.tensor(s), 6, dim=1)
        np.testing.assert_array_equal(idx, ref_i.numpy())
        rw = ref_w.double().numpy()
        if renorm:
            rw = rw / rw.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(w, rw * scale, rtol=2e-7, atol=0)


def test_grouped_sigmoid_bias_steers_choice_not_weight():
    """With one group, selection is the top-k of sigmoid + bias (torch.topk on
    the corrected scores) while the weights stay the uncorrected sigmoid."""
    rng = np.random.default_rng(12)
    z = rng.standard_normal((32, 40)).astype(np.float32)
    bias = (rng.standard_normal(40) * 0.3).astype(np.float32)
    idx, w = O.route_sigmoid_grouped(z, "f32", bias, 5, 1, 1, False, False, 1.0)
    s = _sig(z)
    _, ref_i = torch.topk(torch.tensor(s) + torch.tensor(bias), 5, dim=1)
    np.testing.assert_array_equal(idx, ref_i.numpy())
    np.testing.assert_array_equal(w, np.take_along_axis(s, idx.astype(np.int64), axis=1))
    # the bias really changes the choice on these rows
    plain, _ = O.route_sigmoid_grouped(z, "f32", None, 5, 1, 1, False, False, 1.0)
    assert (plain != idx).any()


def test_grouped_sigmoid_all_ties_closed_form():
    """All logits 0, no bias: every score is 1/2 and every group ties, so the
    lowest groups and the lowest ids win; weights are 1/k (renormalised) or
    1/2, times scale."""
    z = np.zeros((3, 8), np.float32)
    idx, w = O.route_sigmoid_grouped(z, "f32", None, 3, 4, 2, True, True, 3.0)
    np.testing.assert_array_equal(idx, np.tile([0, 1, 2], (3, 1)))
    np.testing.assert_array_equal(w, np.full((3, 3), np.float32(1.0)))
    idx, w = O.route_sigmoid_grouped(z, "f32", None, 3, 4, 2, True, False, 3.0)
    np.testing.assert_array_equal(w, np.full((3, 3), np.float32(1.5)))


def test_grouped_sigmoid_group_score_definitions():
    """Hand-built row where the two group scores disagree. Group 0 = experts
    {0, 1} with z = (3, -3): top-two sum sigmoid(3)+sigmoid(-3) = 1, max 0.9526.
    Group 1 = {2, 3} with z = (2, 2): sum 1.7616, max 0.8808. Others z = -5.
    Keeping one group, the sum picks group 1 (expert 2, the lower of a tie),
    the max picks group 0 (expert 0)."""
    z = np.array([[3, -3, 2, 2, -5, -5, -5, -5]], np.float32)
    i2, w2 = O.route_sigmoid_grouped(z, "f32", None, 1, 4, 1, True, True, 1.0)
    i1, _ = O.route_sigmoid_grouped(z, "f32", None, 1, 4, 1, False, True, 1.0)
    assert i2.tolist() == [[2]] and i1.tolist() == [[0]]
    assert w2.tolist() == [[1.0]]
    # k = 2 inside the kept group: the tied pair, lower id first
    i, w = O.route_sigmoid_grouped(z, "f32", None, 2, 4, 1, True, False, 1.0)
    assert i.tolist() == [[2, 3]]
    np.testing.assert_allclose(w, [[1 / (1 + np.exp(-2.0))] * 2], rtol=1e-7)


def test_grouped_sigmoid_group_boundary_tie_goes_to_lower_group():
    """Groups 1 and 3 tie for the last kept slot (equal logits); group 0 is
    best. The lower of the tied groups (1) is kept."""
    z = np.array([[4, 4, 1, 1, -3, -3, 1, 1]], np.float32)
    idx, _ = O.route_sigmoid_grouped(z, "f32", None, 4, 4, 2, True, True, 1.0)
    assert idx.tolist() == [[0, 1, 2, 3]]


def test_grouped_sigmoid_invariants_random():
    """On random rows: the kept groups are the best by group score (checked by
    an independent sort), every chosen expert lies in a kept group, no
    unchosen kept expert beats a chosen one, weights are proportional to the
    sigmoid and sum to scale when renormalised."""
    rng = np.random.default_rng(13)
    T, E, G, SG, k = 200, 64, 8, 3, 7
    z = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    idx, w = O.route_sigmoid_grouped(z, "f32", bias, k, G, SG, True, True, 1.7)
    s = _sig(z)
    c = (s + bias).astype(np.float32)
    gs = E // G
    for t in range(T):
        top2 = [np.sort(c[t, g * gs:(g + 1) * gs])[-2:].sum(dtype=np.float32) for g in range(G)]
        kept = sorted(range(G), key=lambda g: (-top2[g], g))[:SG]
        chosen = idx[t].astype(int)
        assert all(e // gs in kept for e in chosen)
        pool = [e for e in range(E) if e // gs in kept and e not in chosen]
        assert max(c[t, pool]) <= min(c[t, chosen])
        assert list(c[t, chosen]) == sorted(c[t, chosen], reverse=True)
        np.testing.assert_allclose(w[t], s[t, chosen] / s[t, chosen].astype(np.float64).sum() * 1.7,
                                   rtol=1e-6)
        assert abs(w[t].astype(np.float64).sum() - 1.7) < 1e-5


def test_grouped_sigmoid_special_values():
    """A NaN logit makes its row's scores NaN: ids 0..k-1, NaN weights; other
    rows are untouched. +inf and -inf are ordinary inputs (scores 1 and 0)."""
    z = np.zeros((3, 8), np.float32)
    z[0, 5] = np.nan
    z[1, 6] = np.inf
    z[2, :] = -np.inf
    z[2, 3] = 0.0
    idx, w = O.route_sigmoid_grouped(z, "f32", None, 2, 4, 2, True, False, 1.0)
    assert idx[0].tolist() == [0, 1] and np.isnan(w[0]).all()
    assert idx[1, 0] == 6 and w[1, 0] == 1.0
    assert idx[2, 0] == 3 and w[2, 0] == 0.5 and w[2, 1] == 0.0


@pytest.mark.parametrize("ldt", ["bf16", "f16"])
def test_grouped_sigmoid_half_logits(ldt):
    """bf16 / fp16 logits: the choice equals the fp32 router's on the same
    (exactly widened) values, the weights are the fp32 router's within one
    rounding to the logits dtype, and a NaN row keeps ids 0..k-1 with NaN
    weights in the logits dtype."""
    rng_ = rng(67)
    z = O.round_to(rng_.standard_normal((40, 32)), ldt)
    z32 = O.decode(z, ldt).astype(np.float32)
    if ldt == "bf16":
        z[5, 20] = 0x7FC0
    else:
        z[5, 20] = np.float16(np.nan)
    z32[5, 20] = np.nan
    bias = (rng_.standard_normal(32) * 0.05).astype(np.float32)
    idx, w = O.route_sigmoid_grouped(z, ldt, bias, 4, 4, 2, True, True, 2.5)
    i32, w32 = O.route_sigmoid_grouped(z32, "f32", bias, 4, 4, 2, True, True, 2.5)
    np.testing.assert_array_equal(idx, i32)
    assert idx[5].tolist() == [0, 1, 2, 3]
    wd = O.decode(w, ldt)
    assert np.isnan(wd[5]).all() and not np.isnan(np.delete(wd, 5, axis=0)).any()
    ok = np.arange(40) != 5
    ulp = 2.0 ** -8 if ldt == "bf16" else 2.0 ** -11
    np.testing.assert_allclose(wd[ok], w32[ok].astype(np.float64), rtol=ulp, atol=0)


def test_grouped_sigmoid_argument_checks():
    z = np.zeros((1, 12), np.float32)
    bad = [dict(groups=5), dict(groups=0), dict(selected_groups=0), dict(selected_groups=5),
           dict(top_k=7, selected_groups=2), dict(top_k=0), dict(scale=0.0), dict(scale=np.inf),
           dict(groups=12, group_top_two=True)]
    for b in bad:
        a = dict(top_k=2, groups=4, selected_groups=2, group_top_two=True, renormalize=True, scale=1.0)
        a.update(b)
        with pytest.raises(ValueError):
            O.route_sigmoid_grouped(z, "f32", None, a["top_k"], a["groups"], a["selected_groups"],
                                    a["group_top_two"], a["renormalize"], a["scale"])


# --------------------------------------------------------------------------
# special experts and the activity mask (aclnnMoeDistributeCombineAddRmsNormV2:
# zero / copy / constant experts, xActiveMaskOptional)
# --------------------------------------------------------------------------
def _bf16(a):
    return O.round_to(np.asarray(a, np.float64), "bf16")


def test_masked_dispatch_counts_and_broadcast():
    rng = np.random.default_rng(31)
    T, k, E = 50, 3, 6
    idx = rng.integers(0, E + 3, size=(T, k)).astype(np.uint32)  # some ids past E
    act2 = rng.random((T, k)) < 0.7
    d = O.dispatch(idx, E, active=act2)
    flat = np.where(act2.reshape(-1) & (idx.reshape(-1) < E), idx.reshape(-1).astype(np.int64), E)
    np.testing.assert_array_equal(np.diff(d["offsets"]), np.bincount(flat, minlength=E + 1)[:E])
    # same as the unmasked dispatch of ids with the inactive slots pointed past E
    ref = O.dispatch(np.where(act2, idx, E).astype(np.uint32), E)
    for key in ("offsets", "slot_of_row", "row_of_slot"):
        np.testing.assert_array_equal(d[key], ref[key])
    act1 = rng.random(T) < 0.6
    np.testing.assert_array_equal(O.dispatch(idx, E, active=act1)["row_of_slot"],
                                  O.dispatch(idx, E, active=np.repeat(act1[:, None], k, 1))["row_of_slot"])
    np.testing.assert_array_equal(O.dispatch(idx, E, active=np.ones((T, k), bool))["row_of_slot"],
                                  O.dispatch(idx, E)["row_of_slot"])


def test_special_combine_reduces_to_plain_combine():
    rng = np.random.default_rng(32)
    T, k, E, H = 40, 2, 5, 16
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.uint32)
    d = O.dispatch(idx, E)
    y = _bf16(rng.standard_normal((T * k, H)))
    w = rng.random((T, k)).astype(np.float32)
    a = O.combine_special_fp64(y, d["row_of_slot"], idx, w, "f32", T, k, "bf16", E)
    b = O.combine_fp64(y, d["row_of_slot"], w, "f32", T, k, "bf16")
    np.testing.assert_array_equal(a, b)


def test_special_experts_closed_forms():
    rng = np.random.default_rng(33)
    T, H, E = 6, 24, 4
    ori = _bf16(rng.standard_normal((T, H)))
    V = _bf16(rng.standard_normal((2, H)))
    a1 = _bf16([0.0, 1.0])
    a2 = _bf16([1.0, 0.0])
    y = _bf16(np.zeros((1, H)))
    nores = np.full(T, -1, np.int32)
    one = np.ones((T, 1), np.float32)
    # copy expert (id E + zero_num), weight 1: the token itself, bit for bit
    idx = np.full((T, 1), E + 2, np.uint32)
    out = O.combine_special(y, nores, idx, one, "f32", T, 1, "bf16", E, 2, 1, 2, ori, a1, a2, V)
    np.testing.assert_array_equal(out, ori)
    # constant expert 0 (alpha1 = 0, alpha2 = 1): V[0]; constant 1 (1, 0): the token
    idx[:] = E + 3
    out = O.combine_special(y, nores, idx, one, "f32", T, 1, "bf16", E, 2, 1, 2, ori, a1, a2, V)
    np.testing.assert_array_equal(out, np.repeat(V[:1], T, 0))
    idx[:] = E + 4
    out = O.combine_special(y, nores, idx, one, "f32", T, 1, "bf16", E, 2, 1, 2, ori, a1, a2, V)
    np.testing.assert_array_equal(out, ori)
    # zero experts: nothing, except the shared term w * s of their slot
    idx = np.full((T, 2), E, np.uint32)
    w2 = np.full((T, 2), 0.25, np.float32)
    c = O.combine_special_fp64(y, np.full(2 * T, -1, np.int32), idx, w2, "f32", T, 2, "bf16", E, 2,
                               0, 0, shared=ori)
    np.testing.assert_array_equal(c, 0.5 * O.decode(ori, "bf16"))
    # an id past every range: NaN row
    idx = np.full((T, 1), E + 5, np.uint32)
    c = O.combine_special_fp64(y, nores, idx, one, "f32", T, 1, "bf16", E, 2, 1, 2, ori, a1, a2, V)
    assert np.isnan(c).all()


def test_activity_mask_is_a_zero_weight_and_empty_token_normalises_residual():
    rng = np.random.default_rng(34)
    T, k, E, H = 30, 3, 6, 32
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.uint32)
    act = rng.random((T, k)) < 0.6
    act[0] = False
    d = O.dispatch(idx, E, active=act)
    y = _bf16(rng.standard_normal((T * k, H)))
    w = rng.random((T, k)).astype(np.float32)
    c = O.combine_special_fp64(y, d["row_of_slot"], idx, w, "f32", T, k, "bf16", E, active=act)
    dfull = O.dispatch(idx, E)
    # rows of active slots agree between the two dispatches only through the slot map, so
    # compare against the unmasked combine with inactive weights zeroed on the same rows
    y_full = np.zeros((T * k, H), np.uint16)
    for s_ in range(T * k):
        r = d["row_of_slot"][s_]
        if r >= 0:
            y_full[dfull["row_of_slot"][s_]] = y[r]
    ref = O.combine_fp64(y_full, dfull["row_of_slot"], np.where(act, w, 0).astype(np.float32), "f32",
                         T, k, "bf16")
    np.testing.assert_allclose(c, ref, rtol=1e-12, atol=1e-12)
    assert (c[0] == 0).all()
    res = _bf16(rng.standard_normal((T, H)))
    gamma = rng.uniform(0.5, 1.5, H).astype(np.float32)
    yo, xo, rs = O.combine_add_rmsnorm_special(res, gamma, 1e-6, y, d["row_of_slot"], idx, w, "f32", T,
                                               k, "bf16", E, active=act)
    np.testing.assert_array_equal(xo[0], res[0])
    ref0 = torch.nn.functional.rms_norm(torch.tensor(O.decode(res[:1], "bf16")), (H,),
                                        torch.tensor(gamma.astype(np.float64)), 1e-6)
    np.testing.assert_array_equal(yo[0], O.round_to(ref0.numpy()[0], "bf16"))


# --------------------------------------------------------------------------
# weight-only quantised experts (aclnnFFN, pseudo-quantization scenario)
# --------------------------------------------------------------------------
def test_int4_unpacking_hand_values():
    """Bytes 0x21, 0x8F, 0x7F: low nibble first, two's complement."""
    got = O.unpack_int4(np.array([[0x21, 0x8F, 0x7F]], np.uint8))
    assert got.tolist() == [[1, 2, -1, -8, -1, 7]]


def test_dequant_closed_forms():
    # INT8 per channel: (q + o) * s with s = 0.5, o = -1 on row 0; s = 2, no offset on row 1
    q = np.array([[3, -4, 127, -128], [1, 2, 3, 4]], np.int8)
    sc = _bf16([[0.5], [2.0]])
    off = _bf16([[-1.0], [0.0]])
    w = O.dequant_weight(q.view(np.uint8), 8, sc, off, 1, "bf16")
    np.testing.assert_array_equal(w, [[1.0, -2.5, 63.0, -64.5], [2, 4, 6, 8]])
    # INT4 per group: two groups of two channels with scales 1 and 0.25
    packed = np.array([[0x21, 0x8F]], np.uint8)  # values 1, 2, -1, -8
    w = O.dequant_weight(packed, 4, _bf16([[1.0, 0.25]]), None, 2, "bf16")
    np.testing.assert_array_equal(w, [[1.0, 2.0, -0.25, -2.0]])


def test_dequant_rounds_once_to_model_dtype():
    """The rounded reading (round_weights=True, kept for comparison).
    Scale 1 + 2^-7 (exact in bf16). bf16 spacing is 2^-6 in [2, 4), 2^-5
    in [4, 8) and 2^-1 in [64, 128):
    127 * s = 127.9921875 -> 128;  2 * s = 2.015625 exact;
    -5 * s = -5.0390625 (-161.25 steps of 2^-5) -> -5.03125;
    3 * s = 3.0234375 is a tie (193.5 steps of 2^-6) -> even, 3.03125.
    With offset 0.5: 2.5 * s = 2.51953125 -> 2.515625; -4.5 * s =
    -4.53515625 -> -4.53125; 3.5 * s = 3.52734375 (225.75 steps) -> 3.53125.
    In fp16 (spacing 2^-9 in [2, 4)) 3 * s = 3.0234375 is exact, while
    127 * s still rounds to 128 (spacing 2^-4 in [64, 128))."""
    q = np.array([[127, 2, -5, 3]], np.int8)
    sc = _bf16([[1.0 + 2.0 ** -7]])
    w = O.dequant_weight(q.view(np.uint8), 8, sc, None, 1, "bf16", round_weights=True)
    np.testing.assert_array_equal(w, [[128.0, 2.015625, -5.03125, 3.03125]])
    w = O.dequant_weight(q.view(np.uint8), 8, sc, _bf16([[0.5]]), 1, "bf16", round_weights=True)
    np.testing.assert_array_equal(w, [[128.0, 2.515625, -4.53125, 3.53125]])
    w = O.dequant_weight(q.view(np.uint8), 8, np.array([[1.0 + 2.0 ** -7]], np.float16), None, 1, "f16",
                         round_weights=True)
    np.testing.assert_array_equal(w[0, [0, 3]], [128.0, 3.0234375])
    # the parity reading keeps the exact products: 127 * (1 + 2^-7) = 127.9921875, 3.5 * s = 3.52734375
    w = O.dequant_weight(q.view(np.uint8), 8, sc, _bf16([[0.5]]), 1, "bf16")
    np.testing.assert_array_equal(w, [[127.5 * (1 + 2.0 ** -7), 2.5 * (1 + 2.0 ** -7), -4.5 * (1 + 2.0 ** -7),
                                       3.5 * (1 + 2.0 ** -7)]])


def test_quant_expert_reduces_to_plain_expert():
    """Integer weights with scale 1 and offset 0 are the same expert as the
    bf16 weights holding those integers (exact in bf16)."""
    rng = np.random.default_rng(41)
    H, I_ = 32, 48
    x = _bf16(rng.standard_normal((7, H)))
    qs = [rng.integers(-8, 8, size=s).astype(np.int8) for s in ((I_, H), (I_, H), (H, I_))]
    packs = [((q[:, 0::2] & 0xF) | ((q[:, 1::2] & 0xF) << 4)).astype(np.uint8) for q in qs]
    ones = [_bf16(np.ones((q.shape[0], 1))) for q in qs]
    y4 = O.swiglu_expert_f64(x, *[O.dequant_weight(p, 4, o, None, 1, "bf16") for p, o in zip(packs, ones)],
                             "bf16")
    ref = O.swiglu_expert(x, *[_bf16(q.astype(np.float64)) for q in qs], "bf16")
    np.testing.assert_array_equal(y4, ref)
    y8 = O.swiglu_expert_f64(x, *[O.dequant_weight(q.view(np.uint8), 8, o, None, 1, "bf16")
                                  for q, o in zip(qs, ones)], "bf16")
    np.testing.assert_array_equal(y8, ref)


# --------------------------------------------------------------------------
# pins added for the grouped router's decision margins, the grouped forward
# and the quantised experts as whole functions
# --------------------------------------------------------------------------
# All logits 0 give s = sigmoid(0) = 1/2 exactly, so with dyadic biases every
# corrected score c = 1/2 + bias and every group score is exact in fp32:
# c = [0.75, 0.625, 0.5625, 1.0, 0.25, 0.375, 0.875, 0.5] (groups of two:
# {0,1} {2,3} {4,5} {6,7}); top-two group scores 1.375, 1.5625, 0.625, 1.375;
# largest-score group scores 0.75, 1.0, 0.375, 0.875.
_DYADIC_BIAS = np.array([0.25, 0.125, 0.0625, 0.5, -0.25, -0.125, 0.375, 0.0], np.float32)


@pytest.mark.parametrize("k,SG,two,margin", [
    (1, 1, True, 0.1875),   # groups: 1.5625 - 1.375; experts of group 1: 1.0 - 0.5625 = 0.4375
    (2, 1, True, 0.1875),   # k + 1 = 3 exceeds the two kept experts: only their gap counts
    (2, 2, True, 0.0),      # groups 0 and 3 tie (1.375) for the second kept place
    (3, 3, True, 0.125),    # groups: 1.375 - 0.625 = 0.75; experts 1.0 .875 .75 .625: 0.125
    (4, 4, True, 0.0625),   # every group kept (no group gap); top five c: ... .625 .5625
    (1, 1, False, 0.125),   # largest-score groups: 1.0 - 0.875
])
def test_grouped_margins_closed_form(k, SG, two, margin):
    z = np.zeros((1, 8), np.float32)
    got = O.route_sigmoid_grouped_margins(z, "f32", _DYADIC_BIAS, k, 4, SG, two)
    assert got.tolist() == [margin]


def test_grouped_margins_scale_with_a_gap_planted_in_the_logits():
    """Planting a logit gap d between the k-th and (k+1)-th expert of a row
    (all in one group, no bias) gives a margin of at most s(a) - s(a - d),
    which shrinks with d; the row without a planted gap keeps the larger
    margin of its own spacing (also the margin of the d = 0.5 row, whose
    planted gap is not its smallest)."""
    E, k = 8, 3
    base = np.array([3.0, 2.0, 1.0, 0.0, -1.0, -2.0, -3.0, -4.0], np.float32)
    z = np.tile(base, (4, 1))
    for r, d in enumerate((0.5, 0.05, 0.005)):
        z[r, 3] = np.float32(1.0 - d)  # the 4th best now sits d below the 3rd
    got = O.route_sigmoid_grouped_margins(z, "f32", None, k, 1, 1, False)
    s = torch.sigmoid(torch.tensor(z, dtype=torch.float64)).float().double().numpy()
    for r in range(4):
        top = np.sort(s[r])[::-1][:k + 1]
        assert got[r] == pytest.approx(np.diff(-top).min(), rel=0, abs=0)
    assert got[2] < got[1] < got[0] == got[3]


def test_grouped_forward_matches_weighted_dense_mixture():
    """forward_sigmoid_grouped against a dense reference built without the
    oracle's router or dispatch: with one group the choice is torch.topk of
    sigmoid + bias, the weights the selected sigmoid scores normalised and
    scaled, and the output the weighted sum of every selected expert's dense
    SwiGLU (fp32 model dtype: only the rounding of h and of the output to
    fp32 separate the two)."""
    g = rng(61)
    T, H, I, E, k, scale = 19, 8, 12, 6, 3, 2.5
    x = g.standard_normal((T, H)).astype(np.float32)
    z = g.standard_normal((T, E)).astype(np.float32)
    bias = (g.standard_normal(E) * 0.5).astype(np.float32)
    wg, wu, wd = _weights(g, E, H, I)
    idx, w, d, y, out = O.forward_sigmoid_grouped(x, z, "f32", bias, k, 1, 1, False, True, scale,
                                                  lambda e: (wg[e], wu[e], wd[e]), E, "f32")
    s = torch.sigmoid(torch.from_numpy(z).double())
    _, top = torch.topk(s.float() + torch.from_numpy(bias), k, dim=1)
    np.testing.assert_array_equal(idx, top.numpy())
    dense = np.stack([_torch_swiglu(x, wg[e], wu[e], wd[e]).numpy() for e in range(E)], 1)  # [T, E, H]
    gate = np.zeros((T, E))
    for t in range(T):
        sel = top[t].numpy()
        gate[t, sel] = s[t, sel].numpy() / s[t, sel].numpy().sum() * scale
    ref = np.einsum("te,teh->th", gate, dense)
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-6)
    # with three groups of two, keeping one: every token's experts share one group
    idx3, _, _, _, _ = O.forward_sigmoid_grouped(x, z, "f32", bias, 2, 3, 1, True, True, 1.0,
                                                 lambda e: (wg[e], wu[e], wd[e]), E, "f32")
    assert (idx3[:, 0] // 2 == idx3[:, 1] // 2).all()


def _quant_case(g, E, H, I_, bits, groups):
    """Integer codes (as the kernel stores them) and power-of-two scales, so
    that every dequantised weight is exact in bf16."""
    def one(N, K):
        v = g.integers(-8, 8, size=(E, N, K)).astype(np.int16)
        if bits == 8:
            q = v.astype(np.int8).view(np.uint8)
        else:
            q = ((v[..., 0::2] & 0xF) | ((v[..., 1::2] & 0xF) << 4)).astype(np.uint8)
        sc = 2.0 ** g.integers(-6, -2, size=(E, N, groups))
        off = g.integers(-2, 3, size=(E, N, groups)).astype(np.float64)
        w = (v + np.repeat(off, K // groups, axis=2)) * np.repeat(sc, K // groups, axis=2)
        return (q, _bf16(sc), _bf16(off)), _bf16(w)
    return [one(I_, H), one(I_, H), one(H, I_)]


@pytest.mark.parametrize("bits,groups", [(8, 1), (4, 1), (4, 2)])
def test_experts_forward_quant_equals_plain_experts_on_exact_weights(bits, groups):
    """experts_forward_quant on several experts, with the dispatch's offsets
    (empty experts included), equals experts_forward_dispatched on the bf16
    weights holding (q + offset) * scale, which are exact here: the codes,
    offsets and scales must meet in the right expert, channel and group
    (per-group scales differ between the two halves of K)."""
    g = rng(62 + bits + groups)
    E, H, I_, T, k = 5, 32, 48, 11, 2
    case = _quant_case(g, E, H, I_, bits, groups)
    x = _bf16(g.standard_normal((T, H)))
    idx = np.stack([g.choice([0, 2, 3, 4], 2, replace=False) for _ in range(T)]).astype(np.uint32)
    d = O.dispatch(idx, E, x)
    assert d["offsets"][2] == d["offsets"][1]  # expert 1 gets no rows
    quant_of = lambda e: tuple((c[0][0][e], c[0][1][e], c[0][2][e]) for c in case)  # noqa: E731
    plain = lambda e: tuple(c[1][e] for c in case)  # noqa: E731
    ref = O.experts_forward_dispatched(d["x_disp"], d["offsets"], plain, "bf16")
    for rw in (True, False):
        got = O.experts_forward_quant(d["x_disp"], d["offsets"], quant_of, bits, groups, "bf16", rw)
        np.testing.assert_array_equal(got, ref)


def test_experts_forward_quant_exact_variant_keeps_unrounded_weights():
    """With scales that make (q + offset) * scale inexact in bf16, the exact
    variant equals the SwiGLU expert on the fp64 dequantised weights, and the
    rounded variant the same expert on those weights rounded to bf16."""
    g = rng(66)
    E, H, I_, T = 2, 16, 24, 6
    qs = [g.integers(-127, 128, size=s).astype(np.int8) for s in ((E, I_, H), (E, I_, H), (E, H, I_))]
    scs = [_bf16(1.0 + np.abs(g.standard_normal((E, q.shape[1], 1))) / 7) for q in qs]
    offs = [_bf16(g.standard_normal((E, q.shape[1], 1))) for q in qs]  # not integers
    x = _bf16(g.standard_normal((T, H)))
    d = O.dispatch(np.array([[0], [1]] * (T // 2), np.uint32), E, x)
    quant_of = lambda e: tuple((q[e].view(np.uint8), s[e], o[e]) for q, s, o in zip(qs, scs, offs))  # noqa: E731
    exact = O.experts_forward_quant(d["x_disp"], d["offsets"], quant_of, 8, 1, "bf16", False)
    rounded = O.experts_forward_quant(d["x_disp"], d["offsets"], quant_of, 8, 1, "bf16", True)
    for e in range(E):
        lo, hi = int(d["offsets"][e]), int(d["offsets"][e + 1])
        wf = [(q[e].astype(np.float64) + O.decode(o[e], "bf16")) * O.decode(s[e], "bf16")
              for q, s, o in zip(qs, scs, offs)]
        np.testing.assert_array_equal(exact[lo:hi], O.swiglu_expert_f64(x[e::2], *wf, "bf16"))
        wr = [O.decode(_bf16(a), "bf16") for a in wf]
        np.testing.assert_array_equal(rounded[lo:hi], O.swiglu_expert_f64(x[e::2], *wr, "bf16"))
    assert not np.array_equal(exact, rounded)  # the weights' rounding is visible here
