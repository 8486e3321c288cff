"""Pins of the oracle's training functions (ruDNN user guide, "12. MoE
first-order training"): router weights for a fixed selection and their
backward, combine_backward, the experts' training forward and backward, and
dispatch_backward.

The backward formulas are checked against torch autograd in fp64 applied to
forward definitions written independently here with torch ops, against
closed forms and against invariants (softmax shift invariance, zero gradient
of unselected logits under normalisation). Shapes use H != I so that a
transposed weight or gradient cannot pass.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

F64 = torch.float64


def _f32(a):
    return np.asarray(a, np.float64).astype(np.float32)


# ------------------------------------------------------------------ router --
def _torch_router_weights(z, idx, scoring, normalize, scale):
    """Forward definition in torch fp64, differentiable in z."""
    score = torch.softmax(z, dim=1) if scoring == O.SOFTMAX else torch.sigmoid(z)
    a = torch.gather(score, 1, idx)
    if normalize:
        a = a / a.sum(dim=1, keepdim=True)
    return a * scale


@pytest.mark.parametrize("scoring", [O.SOFTMAX, O.SIGMOID])
@pytest.mark.parametrize("normalize", [False, True])
def test_router_weights_match_torch(scoring, normalize):
    r = np.random.default_rng(5 + scoring * 2 + normalize)
    T, E, k = 40, 12, 4
    z = _f32(r.standard_normal((T, E)) * 2)
    idx = np.stack([r.choice(E, k, replace=bool(t % 5 == 0)) for t in range(T)])  # some repeats
    w = O.router_selected_weights(z, "f32", idx.astype(np.uint32), scoring, normalize, 1.5)
    ref = _torch_router_weights(torch.tensor(z.astype(np.float64)), torch.tensor(idx), scoring, normalize, 1.5)
    assert w.dtype == np.float32
    np.testing.assert_allclose(w, ref.numpy(), rtol=2e-7, atol=0)


def test_router_weights_closed_forms():
    # all-zero logits: softmax 1/E everywhere, sigmoid 1/2
    z = np.zeros((2, 8), np.float32)
    idx = np.array([[0, 3, 3], [7, 1, 2]], np.uint32)
    w = O.router_selected_weights(z, "f32", idx, O.SOFTMAX, False, 2.0)
    np.testing.assert_array_equal(w, np.full((2, 3), 0.25, np.float32))
    w = O.router_selected_weights(z, "f32", idx, O.SIGMOID, True, 3.0)
    np.testing.assert_array_equal(w, np.full((2, 3), 1.0, np.float32))
    # k = E without normalisation: the softmax weights of a row sum to scale
    r = np.random.default_rng(2)
    z = _f32(r.standard_normal((5, 6)))
    w = O.router_selected_weights(z, "f32", np.tile(np.arange(6), (5, 1)), O.SOFTMAX, False, 0.5)
    np.testing.assert_allclose(w.sum(axis=1), 0.5, rtol=1e-6)


def test_router_invalid_index_row_is_nan():
    z = np.zeros((3, 4), np.float32)
    idx = np.array([[0, 1], [2, 4], [3, 3]], np.int64)
    idx[0, 1] = -1
    for scoring in (O.SOFTMAX, O.SIGMOID):
        w = O.router_selected_weights(z, "f32", idx, scoring, True, 1.0)
        assert np.isnan(w[:2]).all() and not np.isnan(w[2]).any()
        d = O.router_selected_backward(z, "f32", idx, np.ones((3, 2), np.float32), scoring, True, 1.0)
        assert np.isnan(d[:2]).all() and not np.isnan(d[2]).any()


@pytest.mark.parametrize("scoring", [O.SOFTMAX, O.SIGMOID])
@pytest.mark.parametrize("normalize", [False, True])
def test_router_backward_matches_autograd(scoring, normalize):
    r = np.random.default_rng(11 + scoring * 2 + normalize)
    T, E, k = 30, 10, 3
    z = _f32(r.standard_normal((T, E)) * 2)
    idx = np.stack([r.choice(E, k, replace=bool(t % 4 == 0)) for t in range(T)])
    gw = _f32(r.standard_normal((T, k)))
    d = O.router_selected_backward(z, "f32", idx.astype(np.uint32), gw, scoring, normalize, 0.75)
    zt = torch.tensor(z.astype(np.float64), requires_grad=True)
    w = _torch_router_weights(zt, torch.tensor(idx), scoring, normalize, 0.75)
    w.backward(torch.tensor(gw.astype(np.float64)))
    np.testing.assert_allclose(d, zt.grad.numpy(), rtol=1e-6, atol=1e-7)


def test_router_backward_invariants():
    r = np.random.default_rng(17)
    T, E, k = 20, 9, 3
    z = _f32(r.standard_normal((T, E)))
    idx = np.stack([r.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    gw = _f32(r.standard_normal((T, k)))
    for normalize in (False, True):
        d = O.router_selected_backward(z, "f32", idx, gw, O.SOFTMAX, normalize, 1.0).astype(np.float64)
        # softmax is invariant to adding a constant to a row of logits
        np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-6)
    # normalised weights depend only on the selected logits
    for scoring in (O.SOFTMAX, O.SIGMOID):
        d = O.router_selected_backward(z, "f32", idx, gw, scoring, True, 1.0)
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert np.abs(d[mask]).max() < 1e-12  # zero up to fp64 cancellation
    # sigmoid without normalisation: c * g * s (1 - s) at the selected ids
    d = O.router_selected_backward(z, "f32", idx, gw, O.SIGMOID, False, 2.0).astype(np.float64)
    s = 1 / (1 + np.exp(-z.astype(np.float64)))
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(d, idx.astype(np.int64), axis=1),
                               2.0 * gw * sel * (1 - sel), rtol=1e-6)


# ----------------------------------------------------------------- combine --
def test_combine_backward_matches_autograd():
    r = np.random.default_rng(23)
    T, k, E, H = 16, 3, 5, 24
    idx = np.stack([r.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    d = O.dispatch(idx, E)
    R = int(d["offsets"][-1])
    y = _f32(r.standard_normal((R, H)))
    w = _f32(r.random((T, k)))
    go = _f32(r.standard_normal((T, H)))
    dexp, dw = O.combine_backward(y, d["row_of_slot"], w, "f32", go, T, k, "f32")
    yt = torch.tensor(y.astype(np.float64), requires_grad=True)
    wt = torch.tensor(w.astype(np.float64), requires_grad=True)
    rows = torch.tensor(d["row_of_slot"].astype(np.int64)).reshape(T, k)
    out = (wt[:, :, None] * yt[rows]).sum(dim=1)
    out.backward(torch.tensor(go.astype(np.float64)))
    np.testing.assert_allclose(dexp, yt.grad.numpy(), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-6, atol=1e-6)


def test_combine_backward_dropped_slot():
    idx = np.array([[0, 9], [1, 0]], np.uint32)  # id 9 is outside E = 2
    d = O.dispatch(idx, 2)
    y = np.ones((3, 4), np.float32)
    dexp, dw = O.combine_backward(y, d["row_of_slot"], np.ones((2, 2), np.float32), "f32",
                                  np.ones((2, 4), np.float32), 2, 2, "f32")
    assert np.isnan(dw[0, 1]) and not np.isnan(dw[0, 0]) and not np.isnan(dw[1]).any()
    np.testing.assert_array_equal(dw[1], [4.0, 4.0])
    assert dexp.shape == (3, 4)


# ----------------------------------------------------------------- experts --
def _torch_swiglu(x, wg, wu, wd):
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def test_expert_training_forward_is_the_swiglu():
    r = np.random.default_rng(29)
    n, H, I_ = 9, 24, 40
    x, wg, wu, wd = (_f32(r.standard_normal(s) / np.sqrt(s[-1])) for s in ((n, H), (I_, H), (I_, H), (H, I_)))
    y, g, u, h = O.swiglu_expert_training(x, wg, wu, wd, "f32")
    t = [torch.tensor(a.astype(np.float64)) for a in (x, wg, wu, wd)]
    np.testing.assert_allclose(y, _torch_swiglu(*t).numpy(), rtol=2e-5, atol=1e-6)
    np.testing.assert_allclose(g, (t[0] @ t[1].T).numpy(), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(u, (t[0] @ t[2].T).numpy(), rtol=1e-6, atol=1e-7)
    # the inference expert computes the same function (no rounding of g, u)
    np.testing.assert_allclose(y, O.swiglu_expert(x, wg, wu, wd, "f32"), rtol=2e-5, atol=1e-6)


def test_expert_backward_matches_autograd():
    r = np.random.default_rng(31)
    n, H, I_ = 11, 24, 40
    x, wg, wu, wd = (_f32(r.standard_normal(s) / np.sqrt(s[-1])) for s in ((n, H), (I_, H), (I_, H), (H, I_)))
    dy = _f32(r.standard_normal((n, H)))
    y, g, u, h = O.swiglu_expert_training(x, wg, wu, wd, "f32")
    dinput, dgate, dup, ddown = O.swiglu_expert_backward(x, wg, wu, wd, g, u, h, dy, "f32")
    t = [torch.tensor(a.astype(np.float64), requires_grad=True) for a in (x, wg, wu, wd)]
    _torch_swiglu(*t).backward(torch.tensor(dy.astype(np.float64)))
    for got, ref in zip((dinput, dgate, dup, ddown), t):
        assert got.shape == ref.grad.shape
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=1e-4, atol=1e-5)


def test_experts_backward_blocks_and_empty_experts():
    r = np.random.default_rng(37)
    T, k, E, H, I_ = 10, 2, 4, 16, 24
    idx = np.stack([r.choice([0, 2, 3], k, replace=False) for _ in range(T)]).astype(np.uint32)  # expert 1 empty
    x = _f32(r.standard_normal((T, H)))
    d = O.dispatch(idx, E, x)
    W = [tuple(_f32(r.standard_normal(s) / np.sqrt(s[-1])) for s in ((I_, H), (I_, H), (H, I_))) for _ in range(E)]
    y, g, u, h = O.experts_forward_training(d["x_disp"], d["offsets"], lambda e: W[e], "f32")
    dy = _f32(r.standard_normal(y.shape))
    dinput, dgate, dup, ddown = O.experts_backward(d["x_disp"], d["offsets"], lambda e: W[e], g, u, h, dy, "f32")
    assert not dgate[1].any() and not dup[1].any() and not ddown[1].any()
    for e in (0, 2, 3):
        a, b = d["offsets"][e], d["offsets"][e + 1]
        one = O.swiglu_expert_backward(d["x_disp"][a:b], *W[e], g[a:b], u[a:b], h[a:b], dy[a:b], "f32")
        np.testing.assert_array_equal(dinput[a:b], one[0])
        np.testing.assert_array_equal(dgate[e], one[1])
        np.testing.assert_array_equal(ddown[e], one[3])


def test_expert_backward_rounding_points_bf16():
    """In bf16, dg and du are rounded before the weight-gradient products:
    dgate equals dg^T x formed from the rounded dg exactly (fp32 of an fp64
    sum of bf16 products), and differs from the unrounded dg^T x."""
    r = np.random.default_rng(41)
    n, H, I_ = 7, 16, 24
    bf = lambda a: O.round_to(np.asarray(a, np.float64), "bf16")  # noqa: E731
    x, wg, wu, wd = (bf(r.standard_normal(s) / np.sqrt(s[-1])) for s in ((n, H), (I_, H), (I_, H), (H, I_)))
    dy = bf(r.standard_normal((n, H)))
    y, g, u, h = O.swiglu_expert_training(x, wg, wu, wd, "bf16")
    di, dgt, dut, ddn = O.swiglu_expert_backward(x, wg, wu, wd, g, u, h, dy, "bf16")
    dec = lambda a: O.decode(a, "bf16")  # noqa: E731
    dh = dec(dy) @ dec(wd)
    gv = dec(g)
    s = 1 / (1 + np.exp(-gv))
    du_exact = dh * gv * s
    assert np.abs(dut - (du_exact.T @ dec(x))).max() > 0  # rounding of du matters
    np.testing.assert_allclose(dut, (dec(bf(du_exact)).T @ dec(x)).astype(np.float32), rtol=0, atol=0)
    np.testing.assert_array_equal(ddn, (dec(dy).T @ dec(h)).astype(np.float32))


# ---------------------------------------------------------------- dispatch --
def test_dispatch_backward_is_the_gather_adjoint():
    r = np.random.default_rng(43)
    T, k, E, H = 12, 3, 4, 8
    idx = r.integers(0, E + 1, size=(T, k)).astype(np.uint32)  # id E is not dispatched
    d = O.dispatch(idx, E)
    R = int(d["offsets"][-1])
    dinput = _f32(r.standard_normal((R, H)))
    dx = O.dispatch_backward(dinput, d["row_of_slot"], T, k, H, "f32")
    xt = torch.zeros((T, H), dtype=F64, requires_grad=True)
    tok = torch.tensor(d["slot_of_row"].astype(np.int64) // k)
    (xt[tok] * torch.tensor(dinput.astype(np.float64))).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-6, atol=1e-7)


# -------------------------------------------------------------- end to end --
@pytest.mark.parametrize("scoring,normalize", [(O.SOFTMAX, True), (O.SIGMOID, False)])
def test_training_chain_matches_autograd(scoring, normalize):
    """logits, x, weights -> fixed selection -> dispatch -> experts -> combine;
    the four backward steps in the pages' order give the gradients autograd
    finds for the whole composition."""
    r = np.random.default_rng(47 + scoring)
    T, k, E, H, I_ = 14, 2, 4, 12, 20
    z = _f32(r.standard_normal((T, E)))
    idx = np.stack([r.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    x = _f32(r.standard_normal((T, H)))
    W = [tuple(_f32(r.standard_normal(s) / np.sqrt(s[-1])) for s in ((I_, H), (I_, H), (H, I_))) for _ in range(E)]
    go = _f32(r.standard_normal((T, H)))
    # oracle chain
    w = O.router_selected_weights(z, "f32", idx, scoring, normalize, 1.25)
    d = O.dispatch(idx, E, x)
    y, g, u, h = O.experts_forward_training(d["x_disp"], d["offsets"], lambda e: W[e], "f32")
    dexp, dw = O.combine_backward(y, d["row_of_slot"], w, "f32", go, T, k, "f32")
    dinput, dgate, dup, ddown = O.experts_backward(d["x_disp"], d["offsets"], lambda e: W[e], g, u, h, dexp, "f32")
    dx = O.dispatch_backward(dinput, d["row_of_slot"], T, k, H, "f32")
    dz = O.router_selected_backward(z, "f32", idx, dw, scoring, normalize, 1.25)
    # autograd of the composition
    zt = torch.tensor(z.astype(np.float64), requires_grad=True)
    xt = torch.tensor(x.astype(np.float64), requires_grad=True)
    Wt = [[torch.tensor(a.astype(np.float64), requires_grad=True) for a in We] for We in W]
    wt = _torch_router_weights(zt, torch.tensor(idx.astype(np.int64)), scoring, normalize, 1.25)
    out = torch.zeros((T, H), dtype=F64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            out[t] = out[t] + wt[t, j] * _torch_swiglu(xt[t:t + 1], *Wt[e])[0]
    out.backward(torch.tensor(go.astype(np.float64)))
    tol = dict(rtol=2e-4, atol=2e-5)
    np.testing.assert_allclose(dz, zt.grad.numpy(), **tol)
    np.testing.assert_allclose(dx, xt.grad.numpy(), **tol)
    for e in range(E):
        np.testing.assert_allclose(dgate[e], Wt[e][0].grad.numpy(), **tol)
        np.testing.assert_allclose(dup[e], Wt[e][1].grad.numpy(), **tol)
        np.testing.assert_allclose(ddown[e], Wt[e][2].grad.numpy(), **tol)
