"""GPU parity of the first-order training path (ruDNN user guide, "12. MoE
first-order training"): the HIP library through its C ABI against the CPU
oracle on the same seeded inputs.

Tolerances (|gpu - ref| <= atol + rtol |ref|, NaN positions identical):
  * outputs in the model or logits dtype: as the forward (fp32 1e-4 / 1e-4,
    bf16 1e-2 / 2e-2, fp16 1e-3 / 2e-3);
  * router weights (fp32): 1e-4 / 1e-4;
  * dweights (fp32 dot products over H): |err| <= H * 2^-23 * sum_h |go_h y_h|
    plus 1e-6, the textbook bound of an fp32 sum of H products;
  * weight gradients C = A^T B (fp32 sums over an expert's n rows of
    products of model-dtype operands): both sides round the terms (dg, du,
    and where the GPU's own cache and dexpert feed in, h and dexpert too) from
    values that differ by accumulation error, so a term may land one ulp of
    the model dtype away; the bar is that ulp times the other operand, summed
    over the rows, plus the fp32 accumulation bound n 2^-23 sum |a b|;
  * dweights likewise (expert outputs one ulp apart, summed over H) and
    dlogits through the router's Jacobian of those (|dw/dz| <= 2 scale).
"""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_top_amd import inputs as I
from mixture_experts_ffn_top_amd import moe
from oracle import moe_oracle as O
from parity_helpers import TOL, assert_close, decode, dev, host, upload_expert_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def _store(a, dtype):
    return O.round_to(np.asarray(a, np.float64), dtype)


def _idx_dev(idx, kind):
    """kind: 'u32' (int32 storage read as uint32), 'i32' or 'i64'."""
    if kind == "i64":
        return torch.from_numpy(np.ascontiguousarray(idx).astype(np.int64)).cuda(), False
    return torch.from_numpy(np.ascontiguousarray(idx).astype(np.int64).astype(np.int32)).cuda(), kind == "i32"


def _ulp(v, dtype):
    """Spacing of the model dtype at |v| (subnormal spacing near zero)."""
    frac_bits, emin = {"bf16": (7, -126), "f16": (10, -14)}[dtype]
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, emin), emin)
    return 2.0 ** (e - frac_bits)


def _wgrad_bound(a, b, dtype, ma, mb):
    """Bound on |C_gpu - C_ref| for C = a^T b (a [n, P], b [n, Q] fp64 values)
    summed in fp32, when elements of a may be ma ulps of the model dtype away
    from the oracle's and elements of b mb ulps (0: identical inputs). One ulp
    for a term both sides round once from values a little apart (dg, du from
    the same cache; dexpert); three for h formed from a cache whose g and u
    may each sit one ulp away; four for dg, du whose cache and dexpert both
    come from the GPU."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    n = a.shape[0]
    bound = n * 2.0 ** -23 * (np.abs(a).T @ np.abs(b))
    if ma:
        bound = bound + ma * (_ulp(a, dtype).T @ np.abs(b))
    if mb:
        bound = bound + mb * (np.abs(a).T @ _ulp(b, dtype))
    return bound


def _assert_bound(gpu, ref, bound, what):
    g, r = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert not np.isnan(g).any() and not np.isnan(r).any(), what
    err = np.abs(g - r)
    bad = err > bound + 1e-30
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {bad.sum()} of {r.size} outside the bound; worst gpu={g.flat[i]} "
                             f"ref={r.flat[i]} err={err.flat[i]:.3g} bound={bound.flat[i]:.3g}")


# ------------------------------------------------------------------ router --
def _router_case(seed, T, E, k, ldt, repeats=True, specials=True):
    r = np.random.default_rng(seed)
    z = r.standard_normal((T, E)) * 2
    idx = np.stack([r.choice(E, k, replace=bool(repeats and t % 7 == 3)) for t in range(T)]).astype(np.int64)
    if specials and T >= 12:
        z[1, idx[1, 0]] = np.nan            # NaN at a selected expert
        z[2, (idx[2, 0] + 1) % E] = np.nan  # NaN at an expert that may not be selected
        z[3, :] = -np.inf                   # all -inf
        z[4, idx[4, 0]] = np.inf            # +inf at a selected expert
        z[5, :E // 2] = -np.inf             # partly -inf
        idx[6, k - 1] = E + 3               # an index outside [0, E)
    return _store(z, ldt), idx


ROUTER_SHAPES = [(8, 1), (8, 2), (64, 8), (256, 8), (1000, 17), (128, 64)]


@pytest.mark.parametrize("scoring", [O.SOFTMAX, O.SIGMOID])
@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("E,k", ROUTER_SHAPES)
def test_router_weights_and_backward(E, k, scoring, normalize):
    say("router", E, k, scoring, normalize)
    T = 200
    for ldt, kind in (("f32", "u32"), ("bf16", "i64"), ("f16", "i32")):
        z, idx = _router_case(E * 7 + k + scoring * 3 + normalize, T, E, k, ldt)
        idx_t, signed = _idx_dev(idx, kind)
        if kind == "i32":
            idx_t[6, k - 1] = -1  # negative ids are invalid for signed indices
            idx_h = host(idx_t).astype(np.int64)
        else:
            idx_h = idx
        scale = 1.75
        w = moe.moe_router_weights(dev(z, ldt), idx_t, scoring, normalize, scale, unsigned=not signed)
        gw = np.random.default_rng(E + k).standard_normal((T, k)).astype(np.float32)
        dz = moe.moe_router_backward(dev(z, ldt), idx_t, dev(gw, "f32"), scoring, normalize, scale,
                                     unsigned=not signed)
        torch.cuda.synchronize()
        w_ref = O.router_selected_weights(z, ldt, idx_h, scoring, normalize, scale)
        dz_ref = O.router_selected_backward(z, ldt, idx_h, gw, scoring, normalize, scale)
        assert_close(host(w), w_ref, "f32", f"router weights {ldt} {kind}")
        assert_close(host(dz), dz_ref, ldt, f"router backward {ldt} {kind}")


def test_router_empty_batch():
    z = torch.zeros((0, 8), device="cuda")
    idx = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    assert moe.moe_router_weights(z, idx, O.SOFTMAX, True).shape == (0, 2)
    assert moe.moe_router_backward(z, idx, torch.zeros((0, 2), device="cuda"), O.SIGMOID, False).shape == (0, 8)


# ------------------------------------------------------- combine / dispatch --
@pytest.mark.parametrize("dtype,wdt", [("bf16", "f32"), ("f16", "f16"), ("f32", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("T,k,E,H", [(300, 4, 16, 520), (5, 1, 2, 8), (64, 70, 80, 64)])
def test_combine_and_dispatch_backward(T, k, E, H, dtype, wdt):
    say("combine/dispatch backward", T, k, E, H, dtype, wdt)
    r = np.random.default_rng(T + k + H)
    idx = np.stack([r.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    if T > 10:
        idx[3, 0] = E + 1  # not dispatched: NaN dweight, no dexpert row, nothing summed back
    d = O.dispatch(idx, E)
    R = int(d["offsets"][-1])
    y = _store(r.standard_normal((R, H)), dtype)
    w = _store(r.random((T, k)), wdt)
    go = _store(r.standard_normal((T, H)), dtype)
    ros = dev(d["row_of_slot"])
    dexp, dw = moe.moe_combine_backward(dev(y, dtype), ros, dev(w, wdt), dev(go, dtype), k)
    torch.cuda.synchronize()
    dexp_ref, dw_ref = O.combine_backward(y, d["row_of_slot"], w, wdt, go, T, k, dtype)
    assert_close(host(dexp)[:R], dexp_ref, dtype, "dexpert")
    # dweights: fp32 sum of H products
    rows = d["row_of_slot"].reshape(T, k)
    mag = np.array([[np.abs(decode(go, dtype)[t] * decode(y, dtype)[rows[t, j]]).sum() if rows[t, j] >= 0 else 0
                     for j in range(k)] for t in range(T)])
    g, rf = host(dw).astype(np.float64), dw_ref.astype(np.float64)
    assert (np.isnan(g) == np.isnan(rf)).all(), "dweights NaN positions"
    ok = ~np.isnan(rf)
    assert (np.abs(g[ok] - rf[ok]) <= H * 2.0 ** -23 * mag[ok] + 1e-6).all(), "dweights"
    # dispatch backward of a dinput in dispatched order
    dinput = _store(r.standard_normal((R, H)), dtype)
    dx = moe.moe_dispatch_backward(dev(dinput, dtype), ros, T, k)
    torch.cuda.synchronize()
    assert_close(host(dx), O.dispatch_backward(dinput, d["row_of_slot"], T, k, H, dtype), dtype, "dx")


# ----------------------------------------------------------------- experts --
def _experts_case(seed, E, H, I_, counts, dtype):
    r = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    x = _store(r.standard_normal((R, H)), dtype)
    W = [tuple(_store(r.standard_normal(s) / np.sqrt(s[-1]), dtype) for s in ((I_, H), (I_, H), (H, I_)))
         for _ in range(E)]
    dy = _store(r.standard_normal((R, H)), dtype)
    return offsets, x, W, dy


def _stack(W, j, dtype):
    return dev(np.stack([w[j] for w in W]), dtype)


EXPERT_CASES = [
    # E, H, I, rows per expert, dtype
    (4, 264, 200, [130, 0, 37, 257], "bf16"),   # ragged K, N and M tails, an empty expert
    (8, 512, 384, [64] * 8, "f16"),
    (3, 128, 136, [1, 300, 5], "bf16"),
    (16, 256, 512, list(range(0, 160, 10)), "bf16"),
    (1, 392, 328, [513], "bf16"),               # one expert takes every row
    (5, 256, 264, [0, 0, 600, 0, 0], "bf16"),   # every row on one of several experts
    (2, 1032, 1544, [200, 311], "f16"),         # larger and ragged, fp16
    # several tiles per persistent workgroup in the training forward, ragged tails
    (256, 264, 200, [int(c) for c in np.random.default_rng(3).integers(0, 80, 256)], "bf16"),
    (96, 136, 328, [int(c) for c in np.random.default_rng(4).integers(150, 350, 96)], "f16"),
]


@pytest.mark.parametrize("E,H,I_,counts,dtype", EXPERT_CASES)
def test_experts_training_forward_and_backward(E, H, I_, counts, dtype):
    say("experts training", E, H, I_, sum(counts), dtype)
    offsets, x, W, dy = _experts_case(E * 31 + H + I_, E, H, I_, counts, dtype)
    R = int(offsets[-1])
    wg, wu, wd = (_stack(W, j, dtype) for j in range(3))
    xo = dev(x, dtype)
    off = dev(offsets)
    y, cache = moe.moe_experts_forward_training(xo, off, wg, wu, wd)
    dinput, dgate, dup, ddown = moe.moe_experts_backward(xo, off, wg, wu, wd, cache, dev(dy, dtype))
    torch.cuda.synchronize()
    y_ref, g_ref, u_ref, h_ref = O.experts_forward_training(x, offsets, lambda e: W[e], dtype)
    c = host(cache)
    gu = c[:R * 2 * I_].reshape(R, 2 * I_)
    assert_close(gu[:, :I_], g_ref, dtype, "cache g")
    assert_close(gu[:, I_:], u_ref, dtype, "cache u")
    assert_close(c[R * 2 * I_:].reshape(R, I_), h_ref, dtype, "cache h")
    assert_close(host(y), y_ref, dtype, "training expert_out")
    # backward from the oracle's own cache, so the comparison isolates the backward
    di_ref, dg_ref, du_ref, dd_ref, dg_t, du_t = O.experts_backward(x, offsets, lambda e: W[e], g_ref, u_ref,
                                                                    h_ref, dy, dtype, terms=True)
    cache_ref = np.concatenate([np.concatenate([g_ref, u_ref], axis=1).reshape(-1), h_ref.reshape(-1)])
    dinput2, dgate2, dup2, ddown2 = moe.moe_experts_backward(xo, off, wg, wu, wd, dev(cache_ref, dtype),
                                                             dev(dy, dtype))
    torch.cuda.synchronize()
    assert_close(host(dinput2), di_ref, dtype, "dinput")
    xv, dyv, hv = decode(x, dtype), decode(dy, dtype), decode(h_ref, dtype)
    hg = decode(c[R * 2 * I_:].reshape(R, I_), dtype)
    gg, gu_, gd, gd_own = host(dgate2), host(dup2), host(ddown2), host(ddown)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            for nm, t in (("dgate", gg), ("dup", gu_), ("ddown", gd), ("ddown (gpu cache)", gd_own)):
                assert not t[e].any(), f"{nm}: expert {e} without rows must be zero"
            continue
        _assert_bound(gg[e], dg_ref[e], _wgrad_bound(dg_t[a:b], xv[a:b], dtype, 1, 0), f"dgate e={e}")
        _assert_bound(gu_[e], du_ref[e], _wgrad_bound(du_t[a:b], xv[a:b], dtype, 1, 0), f"dup e={e}")
        _assert_bound(gd[e], dd_ref[e], _wgrad_bound(dyv[a:b], hv[a:b], dtype, 0, 0), f"ddown e={e}")
        # from the GPU's own cache: h may sit one ulp away
        _assert_bound(gd_own[e], dd_ref[e], _wgrad_bound(dyv[a:b], hg[a:b], dtype, 0, 3),
                      f"ddown (gpu cache) e={e}")
    assert_close(host(dinput), di_ref, dtype, "dinput (gpu cache)")


def test_experts_backward_deterministic_and_no_rows():
    E, H, I_, counts, dtype = 4, 264, 200, [130, 0, 37, 257], "bf16"
    offsets, x, W, dy = _experts_case(7, E, H, I_, counts, dtype)
    wg, wu, wd = (_stack(W, j, dtype) for j in range(3))
    xo, off = dev(x, dtype), dev(offsets)
    _, cache = moe.moe_experts_forward_training(xo, off, wg, wu, wd)
    a = moe.moe_experts_backward(xo, off, wg, wu, wd, cache, dev(dy, dtype))
    b = moe.moe_experts_backward(xo, off, wg, wu, wd, cache, dev(dy, dtype))
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert torch.equal(p.view(torch.uint8) if p.dtype != torch.float32 else p, q.view(torch.uint8)
                           if q.dtype != torch.float32 else q)
    # no rows at all: every weight gradient is zero
    z_off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    empty = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    dgate = torch.full((E, I_, H), 7.0, device="cuda")
    dup, ddown = torch.full_like(dgate, 7.0), torch.full((E, H, I_), 7.0, device="cuda")
    moe.moe_experts_backward(empty, z_off, wg, wu, wd, torch.empty(0, dtype=torch.bfloat16, device="cuda"),
                             empty, rows=0, dgate=dgate, dup=dup, ddown=ddown)
    torch.cuda.synchronize()
    assert not dgate.any() and not dup.any() and not ddown.any()


# -------------------------------------------------------------- whole chain --
@pytest.mark.parametrize("scoring,normalize,k", [(O.SOFTMAX, True, 2), (O.SIGMOID, False, 2), (O.SOFTMAX, False, 1),
                                                 (O.SIGMOID, True, 3)])
def test_training_step_chain(scoring, normalize, k):
    """route (fixed selection) -> weights -> dispatch -> experts (training)
    -> combine; then combine_backward -> experts backward -> dispatch_backward
    -> router backward, each step through the C ABI, against the oracle chain."""
    say("training chain", scoring, normalize, k)
    r = np.random.default_rng(5 + scoring + 10 * k)
    T, E, H, I_, dtype = 96, 8, 256, 384, "bf16"
    z = _store(r.standard_normal((T, E)), "f32")
    x = _store(r.standard_normal((T, H)), dtype)
    W = [tuple(_store(r.standard_normal(s) / np.sqrt(s[-1]), dtype) for s in ((I_, H), (I_, H), (H, I_)))
         for _ in range(E)]
    go = _store(r.standard_normal((T, H)), dtype)
    idx_ref, _ = O.route(z, "f32", k, True)
    # GPU chain
    zd = dev(z, "f32")
    idx, _ = moe.moe_route(zd, k, True)
    w = moe.moe_router_weights(zd, idx, scoring, normalize, 1.0)
    d = moe.moe_dispatch(idx, E, dev(x, dtype))
    wg, wu, wd = (_stack(W, j, dtype) for j in range(3))
    y, cache = moe.moe_experts_forward_training(d["x_disp"], d["offsets"], wg, wu, wd, rows=T * k)
    out = moe.moe_combine(y, d["row_of_slot"], w)
    dexp, dw = moe.moe_combine_backward(y, d["row_of_slot"], w, dev(go, dtype), k)
    dinput, dgate, dup, ddown = moe.moe_experts_backward(d["x_disp"], d["offsets"], wg, wu, wd, cache, dexp,
                                                         rows=T * k)
    dx = moe.moe_dispatch_backward(dinput, d["row_of_slot"], T, k)
    dz = moe.moe_router_backward(zd, idx, dw, scoring, normalize, 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx).astype(np.uint32), idx_ref)
    # oracle chain
    w_ref = O.router_selected_weights(z, "f32", idx_ref, scoring, normalize, 1.0)
    od = O.dispatch(idx_ref, E, x)
    y_ref, g_ref, u_ref, h_ref = O.experts_forward_training(od["x_disp"], od["offsets"], lambda e: W[e], dtype)
    dexp_ref, dw_ref = O.combine_backward(y_ref, od["row_of_slot"], w_ref, "f32", go, T, k, dtype)
    di_ref, dg_ref, du_ref, dd_ref, dg_t, du_t = O.experts_backward(od["x_disp"], od["offsets"], lambda e: W[e],
                                                                    g_ref, u_ref, h_ref, dexp_ref, dtype, terms=True)
    dx_ref = O.dispatch_backward(di_ref, od["row_of_slot"], T, k, H, dtype)
    dz_ref = O.router_selected_backward(z, "f32", idx_ref, dw_ref, scoring, normalize, 1.0)
    assert_close(host(w), w_ref, "f32", "weights")
    assert_close(host(out), O.combine(y_ref, od["row_of_slot"], w_ref, "f32", T, k, dtype), dtype, "out")
    assert_close(host(dx), dx_ref, dtype, "dx")
    # the GPU's own expert outputs, dexpert and cache feed its backward
    xv, hv = decode(od["x_disp"], dtype), decode(h_ref, dtype)
    dyv = decode(dexp_ref, dtype)
    for e in range(E):
        a, b = int(od["offsets"][e]), int(od["offsets"][e + 1])
        if a == b:
            continue
        _assert_bound(host(dgate)[e], dg_ref[e], _wgrad_bound(dg_t[a:b], xv[a:b], dtype, 4, 0), "dgate")
        _assert_bound(host(dup)[e], du_ref[e], _wgrad_bound(du_t[a:b], xv[a:b], dtype, 4, 0), "dup")
        _assert_bound(host(ddown)[e], dd_ref[e], _wgrad_bound(dyv[a:b], hv[a:b], dtype, 1, 3), "ddown")
    # dweights: <grad_out, y> with y one ulp away
    yv, gov = decode(y_ref, dtype), decode(go, dtype)
    rows = od["row_of_slot"].reshape(T, k)
    bw = np.array([[(np.abs(gov[t]) @ _ulp(yv[rows[t, j]], dtype) + H * 2.0 ** -23 * np.abs(gov[t]) @ np.abs(yv[rows[t, j]]))
                    for j in range(k)] for t in range(T)])
    _assert_bound(host(dw), dw_ref, bw, "dweights")
    # dlogits: the router's Jacobian (entries at most 2 x scale in size) applied to those differences
    bz = 2.0 * bw.sum(axis=1, keepdims=True) + 1e-4 * np.abs(dz_ref.astype(np.float64)) + 1e-6
    _assert_bound(host(dz), dz_ref, np.broadcast_to(bz, dz_ref.shape), "dlogits")


# ------------------------------------------------- full-size training step --
def test_training_step_mixtral_shape_sampled():
    """The Mixtral-shaped workload (T=4096, H=4096, I=14336, E=8, top-2) through
    the same entry points the training benchmark times. Routing weights,
    offsets and maps are compared in full; expert outputs, the cache, dexpert,
    dweights, dinput, dx and dlogits on sampled tokens (first, middle, last,
    random); weight gradients on sampled columns of I for three experts, from
    all of each expert's rows (the oracle's experts are separable over I)."""
    w = I.workload("mixtral_8x_bf16")
    T, H, I_, E, k, dt = w.T, w.H, w.I, w.E, w.top_k, w.dtype
    R = T * k
    say("training mixtral-shaped: inputs")
    z = I.logits_for(w)
    x = I.tokens_for(w)
    go = I.grad_output_for(w)
    wg, wu, wd, W = upload_expert_weights(w, keep=range(E))
    zd, xd, god = dev(z, "f32"), dev(x, dt), dev(go, dt)
    say("training mixtral-shaped: gpu step")
    idx, _ = moe.moe_route(zd, k, True)
    wts = moe.moe_router_weights(zd, idx, O.SOFTMAX, True, 1.0)
    d = moe.moe_dispatch(idx, E, xd)
    y, cache = moe.moe_experts_forward_training(d["x_disp"], d["offsets"], wg, wu, wd, rows=R)
    dexp, dw = moe.moe_combine_backward(y, d["row_of_slot"], wts, god, k)
    dinput, dgate, dup, ddown = moe.moe_experts_backward(d["x_disp"], d["offsets"], wg, wu, wd, cache, dexp,
                                                         rows=R)
    dx = moe.moe_dispatch_backward(dinput, d["row_of_slot"], T, k)
    dz = moe.moe_router_backward(zd, idx, dw, O.SOFTMAX, True, 1.0)
    torch.cuda.synchronize()
    say("training mixtral-shaped: oracle")
    idx_ref, _ = O.route(z, "f32", k, True)
    assert np.array_equal(host(idx).astype(np.uint32), idx_ref)
    w_ref = O.router_selected_weights(z, "f32", idx_ref, O.SOFTMAX, True, 1.0)
    assert_close(host(wts), w_ref, "f32", "weights")
    od = O.dispatch(idx_ref, E)
    for key in ("offsets", "slot_of_row", "row_of_slot"):
        assert np.array_equal(host(d[key]), od[key]), key
    c = host(cache)
    gu_gpu, h_gpu = c[:R * 2 * I_].reshape(R, 2 * I_), c[R * 2 * I_:].reshape(R, I_)
    y_g, dexp_g, dinput_g = host(y), host(dexp), host(dinput)
    rng = np.random.default_rng(3)
    tokens = sorted({0, 1, T // 2, T - 1, *rng.integers(0, T, 4).tolist()})
    pairs = [(t, j) for t in tokens for j in range(k)]
    by_e = {}
    for t, j in pairs:
        by_e.setdefault(int(idx_ref[t, j]), []).append((t, j))
    fwd = {}
    for e, pj in by_e.items():  # one oracle call per expert over its sampled rows
        outs = O.swiglu_expert_training(x[[t for t, _ in pj]], *W[e], dt)
        for n, tj in enumerate(pj):
            fwd[tj] = tuple(o[n:n + 1] for o in outs)
    de, dwt = {}, {}
    for t in tokens:
        y_rows = np.concatenate([fwd[(t, j)][0] for j in range(k)])
        d_, w_ = O.combine_backward(y_rows, np.arange(k, dtype=np.int32), w_ref[t:t + 1], "f32", go[t:t + 1],
                                    1, k, dt)
        dwt[t] = w_
        for j in range(k):
            de[(t, j)] = d_[j:j + 1]
    di = {}
    for e, pj in by_e.items():
        cat = lambda i: np.concatenate([fwd[tj][i] for tj in pj])  # noqa: E731
        d_in = O.swiglu_expert_backward(x[[t for t, _ in pj]], *W[e], cat(1), cat(2), cat(3),
                                        np.concatenate([de[tj] for tj in pj]), dt)[0]
        for n, tj in enumerate(pj):
            di[tj] = d_in[n:n + 1]
    for t in tokens:
        for j in range(k):
            r = od["row_of_slot"][t * k + j]
            yr, g_, u_, h_ = fwd[(t, j)]
            assert_close(y_g[r:r + 1], yr, dt, f"expert_out t={t}")
            assert_close(gu_gpu[r:r + 1, :I_], g_, dt, f"cache g t={t}")
            assert_close(gu_gpu[r:r + 1, I_:], u_, dt, f"cache u t={t}")
            assert_close(h_gpu[r:r + 1], h_, dt, f"cache h t={t}")
            assert_close(dexp_g[r:r + 1], de[(t, j)], dt, f"dexpert t={t}")
            assert_close(dinput_g[r:r + 1], di[(t, j)], dt, f"dinput t={t}")
        # dweights: <grad_out, y> with y one ulp away; dlogits through the Jacobian
        gov = decode(go[t], dt)
        bw = np.array([np.abs(gov) @ _ulp(decode(fwd[(t, j)][0][0], dt), dt)
                       + H * 2.0 ** -23 * np.abs(gov) @ np.abs(decode(fwd[(t, j)][0][0], dt)) for j in range(k)])
        _assert_bound(host(dw)[t], dwt[t][0], bw, f"dweights t={t}")
        dx_ref = O.dispatch_backward(np.concatenate([di[(t, j)] for j in range(k)]),
                                     np.arange(k, dtype=np.int32), 1, k, H, dt)
        assert_close(host(dx)[t:t + 1], dx_ref, dt, f"dx t={t}")
        dz_ref = O.router_selected_backward(z[t:t + 1], "f32", idx_ref[t:t + 1], dwt[t], O.SOFTMAX, True, 1.0)
        _assert_bound(host(dz)[t], dz_ref[0], 2.0 * bw.sum() + 1e-4 * np.abs(dz_ref[0].astype(np.float64)) + 1e-6,
                      f"dlogits t={t}")
    # weight gradients: sampled columns of I, all rows of the expert
    dexp_all, _ = O.combine_backward(np.zeros((R, H), np.uint16), od["row_of_slot"], w_ref, "f32", go, T, k, dt)
    for e in (0, 3, E - 1):
        a, b = int(od["offsets"][e]), int(od["offsets"][e + 1])
        xe = x[od["slot_of_row"][a:b] // k]
        isel = np.sort(rng.choice(I_, 8, replace=False))
        wge, wue, wde = W[e][0][isel], W[e][1][isel], np.ascontiguousarray(W[e][2][:, isel])
        _, g_, u_, h_ = O.swiglu_expert_training(xe, wge, wue, wde, dt)
        _, dg_ref, du_ref, dd_ref, dg_t, du_t = O.swiglu_expert_backward(xe, wge, wue, wde, g_, u_, h_,
                                                                         dexp_all[a:b], dt, terms=True)
        xv, hv, dyv = decode(xe, dt), decode(h_, dt), decode(dexp_all[a:b], dt)
        _assert_bound(host(dgate[e])[isel], dg_ref, _wgrad_bound(dg_t, xv, dt, 4, 0), f"dgate e={e}")
        _assert_bound(host(dup[e])[isel], du_ref, _wgrad_bound(du_t, xv, dt, 4, 0), f"dup e={e}")
        _assert_bound(host(ddown[e])[:, isel], dd_ref, _wgrad_bound(dyv, hv, dt, 1, 3), f"ddown e={e}")
