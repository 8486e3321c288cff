"""Seeded synthetic inputs for the local MoE FFN forward.

This module is the only code shared between the GPU path's callers (tests,
benchmark, smoke check) and the CPU oracle's callers. It draws random numbers
and stores them in the tensor dtypes the method consumes; it performs none of
the method's arithmetic (no softmax, no top-k, no GEMM, no normalisation).

Layouts follow the ruDNN user guide, "Expert weights and dispatch" and
"Routing contract" sections: tokens ``x`` are ``[T, H]``, ``gate``/``up`` are
``[E, I, H]``, ``down`` is ``[E, H, I]``, ``logits`` are ``[T, E]``.

Randomness: numpy PCG64 streams seeded with ``SeedSequence([seed,
crc32(name), *extra])`` so every tensor (and every expert's slice of a weight
tensor) is reproducible on its own. bf16 tensors are returned as ``uint16`` bit
patterns (numpy has no bf16), rounded from fp32 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Workloads: named by what they are, with their sizes. Logits are fp32 in all
# of them; x, weights, shared-expert output and residual use ``dtype``.
WORKLOADS = {
    "tiny_fp32": dict(T=64, H=128, I=256, E=8, top_k=2, renormalize=True,
                      dtype="f32", seed=0),
    "mixtral_8x_bf16": dict(T=4096, H=4096, I=14336, E=8, top_k=2, renormalize=True,
                            dtype="bf16", seed=1),
    "many_expert_zipf_bf16": dict(T=8192, H=2048, I=768, E=128, top_k=8,
                                  renormalize=True, dtype="bf16", seed=2,
                                  zipf_bias=True),
    "dsv3_share_rmsnorm_bf16": dict(T=2048, H=7168, I=2048, E=256, top_k=8,
                                    renormalize=True, dtype="bf16", seed=3,
                                    epilogue=True, eps=1e-6),
    "decode_nan_rows_bf16": dict(T=16, H=4096, I=1536, E=128, top_k=8,
                                 renormalize=False, dtype="bf16", seed=4,
                                 special_rows=True),
}

GAP = 1e-3  # minimum spacing among each row's top (k+1) logits


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    renormalize: bool
    dtype: str  # "f32" | "bf16"
    seed: int
    zipf_bias: bool = False
    epilogue: bool = False
    eps: float = 1e-6
    special_rows: bool = False


def workload(name: str, **override) -> Workload:
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    return Workload(name=name, **cfg)


def stream(seed: int, name: str, *extra: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), zlib.crc32(name.encode())] + [int(e) for e in extra])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest-even); returns uint16 bits.

    Used only to store generated data; NaN payloads are passed through as a
    quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


def normal(seed: int, name: str, shape, std: float = 1.0, *extra: int) -> np.ndarray:
    g = stream(seed, name, *extra)
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _logits_row_ok(rows: np.ndarray, k: int) -> np.ndarray:
    E = rows.shape[1]
    m = min(k + 1, E)
    top = -np.sort(-rows.astype(np.float64), axis=1)[:, :m]
    if m < 2:
        return np.ones(rows.shape[0], dtype=bool)
    return (np.diff(-top, axis=1) >= GAP).all(axis=1)


def gapped_logits(seed: int, T: int, E: int, k: int, bias: np.ndarray | None = None,
                  name: str = "logits") -> np.ndarray:
    """fp32 logits [T, E] ~ N(0,1) (+ bias) whose top (k+1) values in every row are
    pairwise at least GAP apart, so the selected set and its order are unique.
    Failing rows are redrawn, in row order, from the same stream."""
    g = stream(seed, name)
    bias32 = None if bias is None else np.asarray(bias, dtype=np.float32)

    def draw(n):
        r = g.standard_normal((n, E), dtype=np.float32)
        if bias32 is not None:
            r = (r + bias32).astype(np.float32)
        return r

    z = draw(T)
    bad = np.nonzero(~_logits_row_ok(z, k))[0]
    while bad.size:
        z[bad] = draw(bad.size)
        bad = bad[~_logits_row_ok(z[bad], k)]
    return z


def zipf_bias(E: int) -> np.ndarray:
    """Per-expert popularity bias 2*log(1/rank) with rank(e) = e + 1."""
    return (-2.0 * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def special_logit_rows(z: np.ndarray) -> np.ndarray:
    """Rows 3, 7 and 11 get a NaN, a +inf and all -inf respectively (the routing
    contract's NaN-weight cases); positions chosen away from lanes 0 and E-1."""
    z = z.copy()
    E = z.shape[1]
    z[3, min(37, E - 1)] = np.nan
    z[7, min(101, E - 1)] = np.inf
    z[11, :] = -np.inf
    return z


def logits_for(w: Workload) -> np.ndarray:
    bias = zipf_bias(w.E) if w.zipf_bias else None
    z = gapped_logits(w.seed, w.T, w.E, w.top_k, bias)
    if w.special_rows:
        z = special_logit_rows(z)
    return z


def tokens_for(w: Workload) -> np.ndarray:
    return store(normal(w.seed, "x", (w.T, w.H)), w.dtype)


def expert_weight(w: Workload, which: str, e: int) -> np.ndarray:
    """One expert's slice: gate/up [I, H] with std H^-1/2, down [H, I] with std I^-1/2."""
    if which in ("w_gate", "w_up"):
        shape, fan_in = (w.I, w.H), w.H
    elif which == "w_down":
        shape, fan_in = (w.H, w.I), w.I
    else:
        raise ValueError(which)
    return store(normal(w.seed, which, shape, 1.0 / math.sqrt(fan_in), e), w.dtype)


def expert_weights(w: Workload, which: str, experts=None, threads: int | None = None) -> np.ndarray:
    """Stacked weights [len(experts), ...] generated expert by expert in parallel."""
    ex = list(range(w.E)) if experts is None else list(experts)
    first = expert_weight(w, which, ex[0]) if ex else None
    if not ex:
        return np.zeros((0,), dtype=np.float32 if w.dtype == "f32" else np.uint16)
    out = np.empty((len(ex),) + first.shape, dtype=first.dtype)
    out[0] = first

    def fill(i):
        out[i] = expert_weight(w, which, ex[i])

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(fill, range(1, len(ex))))
    return out


def quant_expert_weights(w: Workload, which: str, bits: int, groups: int):
    """Synthetic weight-only quantised weights of all experts for one
    projection: integer codes [E, N, K] (bits 8: one int8 per byte; bits 4:
    two codes per byte along K, uniform over all byte values) and positive
    scales [E, N, groups] in the model dtype, |N(0, 1)| / (spread * sqrt(K)) +
    1e-5 with spread 73 (int8) or 4.6 (int4), so that dequantised products
    keep activations O(1). No offsets."""
    N, K = (w.I, w.H) if which in ("w_gate", "w_up") else (w.H, w.I)
    g = stream(w.seed, "quant_" + which, bits, groups)
    q = g.integers(0, 256, size=(w.E, N, K * bits // 8), dtype=np.uint8)
    spread = 73.0 if bits == 8 else 4.6
    sc = np.abs(g.standard_normal((w.E, N, groups), dtype=np.float32)) / np.float32(spread * np.sqrt(K))
    return q, store(sc + np.float32(1e-5), w.dtype)


def grad_output_for(w: Workload) -> np.ndarray:
    """Gradient of the MoE output for a training step: [T, H] ~ N(0, 1) in the model dtype."""
    return store(normal(w.seed, "grad_out", (w.T, w.H)), w.dtype)


def epilogue_inputs(w: Workload):
    """Shared-expert output and residual [T, H] ~ N(0,1); gamma fp32 [H] ~ U(0.5, 1.5)."""
    shared = store(normal(w.seed, "shared", (w.T, w.H)), w.dtype)
    residual = store(normal(w.seed, "residual", (w.T, w.H)), w.dtype)
    gamma = stream(w.seed, "gamma").uniform(0.5, 1.5, w.H).astype(np.float32)
    return shared, residual, gamma


def router_bias(w: Workload) -> np.ndarray:
    """Correction bias of the grouped-limited sigmoid router: fp32 [E] ~ N(0, 0.05^2)."""
    return (stream(w.seed, "router_bias").standard_normal(w.E) * 0.05).astype(np.float32)


def special_expert_inputs(w: Workload, n_zero: int, n_copy: int, n_const: int,
                          active_frac: float = 0.875):
    """Routing over the E experts plus n_zero zero, n_copy copy and n_const
    constant experts (ids E ..), for a forward with special experts:
    logits fp32 [T, E + n_zero + n_copy + n_const] (gapped like logits_for),
    alpha1 and alpha2 [n_const] ~ U(0.5, 1.5) and v [n_const, H] ~ N(0, 1) in
    the model dtype, and a per-token activity mask (uint8 [T]) whose first
    round(active_frac * T) tokens are active."""
    n_ids = w.E + n_zero + n_copy + n_const
    z = gapped_logits(w.seed, w.T, n_ids, w.top_k, name="logits_special")
    g = stream(w.seed, "special_consts", n_zero, n_copy, n_const)
    a1 = store(g.uniform(0.5, 1.5, n_const).astype(np.float32), w.dtype)
    a2 = store(g.uniform(0.5, 1.5, n_const).astype(np.float32), w.dtype)
    v = store(normal(w.seed, "special_v", (n_const, w.H)), w.dtype)
    active = np.zeros(w.T, dtype=np.uint8)
    active[: int(round(active_frac * w.T))] = 1
    return z, a1, a2, v, active

