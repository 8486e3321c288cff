"""Shared helpers for the GPU parity tests: moving seeded host arrays (oracle
representation: fp32 / float16 / bf16 as uint16 bits) to device tensors and
back, and the element-wise tolerance check."""
from __future__ import annotations

import numpy as np
import torch

from mixture_experts_ffn_top_amd import inputs as I

# |gpu - ref| <= atol + rtol * |ref|, NaN exactly where the oracle has NaN.
TOL = {"f32": (1e-4, 1e-4), "bf16": (1e-2, 2e-2), "f16": (1e-3, 2e-3)}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def dev(a: np.ndarray, dtype: str | None = None, device="cuda") -> torch.Tensor:
    """Host array -> device tensor. dtype names the element type of `a`
    ("bf16" means uint16 bit patterns); None keeps integer arrays as int32."""
    if dtype is None:
        return torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array in the oracle's representation."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def count_outside(gpu: np.ndarray, ref: np.ndarray, dtype: str, tol=None) -> int:
    """Elements outside the tolerance, NaN mismatches included."""
    g, r = decode(gpu, dtype), decode(ref, dtype)
    gn, rn = np.isnan(g), np.isnan(r)
    atol, rtol = tol or TOL[dtype]
    ok = ~rn & ~gn
    return int((gn != rn).sum() + (np.abs(g[ok] - r[ok]) > atol + rtol * np.abs(r[ok])).sum())


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", tol=None):
    g, r = decode(gpu, dtype), decode(ref, dtype)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gn, rn = np.isnan(g), np.isnan(r)
    assert (gn == rn).all(), f"{what}: NaN positions differ ({(gn != rn).sum()} elements)"
    atol, rtol = tol or TOL[dtype]
    ok = ~rn
    err = np.abs(g[ok] - r[ok])
    bound = atol + rtol * np.abs(r[ok])
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {bad.sum()} of {ok.sum()} outside tolerance; worst "
                             f"gpu={g[ok][i]} ref={r[ok][i]} err={err[i]:.3g} bound={bound[i]:.3g}")


def upload_expert_weights(w: I.Workload, keep=(), device="cuda", chunk: int = 16):
    """Generate the three weight tensors expert by expert (bounded host memory)
    and copy them to the device. Returns (gate, up, down) device tensors and a
    dict {e: (gate_e, up_e, down_e)} of host arrays for the experts in keep."""
    td = TORCH[w.dtype]
    out = {n: torch.empty(((w.E, w.I, w.H) if n != "w_down" else (w.E, w.H, w.I)), dtype=td, device=device)
           for n in ("w_gate", "w_up", "w_down")}
    kept = {e: [None, None, None] for e in keep}
    for e0 in range(0, w.E, chunk):
        ex = list(range(e0, min(w.E, e0 + chunk)))
        for j, n in enumerate(("w_gate", "w_up", "w_down")):
            a = I.expert_weights(w, n, ex)
            out[n][ex[0]:ex[-1] + 1].copy_(dev(a, w.dtype, device="cpu"))
            for i, e in enumerate(ex):
                if e in kept:
                    kept[e][j] = a[i].copy()
            del a
    torch.cuda.synchronize()
    return out["w_gate"], out["w_up"], out["w_down"], {e: tuple(v) for e, v in kept.items()}


def grouped_choice_valid(c, gsc, chosen, G, SG, margin):
    """Whether `chosen` (one row's expert ids, in slot order) is a choice the
    grouped rule could make, within `margin`, given the oracle's fp32 corrected
    scores c [E] and group scores gsc [G]: k distinct experts in at most SG
    groups; some set of SG kept groups containing theirs, no better than any
    dropped group by more than the margin (the best such set is theirs plus
    the best groups not excluded below); every unchosen expert that beats the
    weakest chosen one by more than the margin lies in a dropped group; and
    the slots run in descending c up to the margin."""
    E = c.shape[0]
    gs = E // G
    chosen = [int(e) for e in chosen]
    if len(set(chosen)) != len(chosen) or max(chosen) >= E:
        return False
    cg = {e // gs for e in chosen}
    cmin = min(c[e] for e in chosen)
    must_drop = {e // gs for e in range(E) if e not in chosen and c[e] > cmin + margin}
    if must_drop & cg or len(cg) > SG:
        return False
    rest = sorted((g for g in range(G) if g not in cg and g not in must_drop), key=lambda g: (-gsc[g], g))
    if len(rest) < SG - len(cg):
        return False
    kept = cg | set(rest[:SG - len(cg)])
    dropped = [gsc[g] for g in range(G) if g not in kept]
    if dropped and min(gsc[g] for g in kept) < max(dropped) - margin:
        return False
    return all(c[a] >= c[b] - margin for a, b in zip(chosen, chosen[1:]))
