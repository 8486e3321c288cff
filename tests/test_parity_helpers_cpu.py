"""CPU checks of the parity tests' own helpers."""
import numpy as np

from mixture_experts_ffn_top_amd import inputs as I
from oracle import moe_oracle as O
from parity_helpers import assert_close, grouped_choice_valid

MARGIN = 1e-6


def test_grouped_choice_validity_on_hand_built_scores():
    """Accepts the best choice and a swap inside a near tie; rejects a skipped
    better expert, a kept group beaten by a dropped one, a wrong slot order and
    a repeated expert."""
    c = np.array([0.9, 0.5, 0.8, 0.8 - 5e-7, 0.1, 0.2], np.float32)  # groups {0,1} {2,3} {4,5}
    gsc = np.array([1.4, 1.6 - 5e-7, 0.3], np.float32)                # top-two sums
    assert grouped_choice_valid(c, gsc, [0, 2], 3, 2, MARGIN)
    assert grouped_choice_valid(c, gsc, [0, 3], 3, 2, MARGIN)         # 2 and 3 tie within the margin
    assert not grouped_choice_valid(c, gsc, [0, 1], 3, 2, MARGIN)     # skips expert 2 (0.8 > 0.5)
    assert not grouped_choice_valid(c, gsc, [0, 4], 3, 2, MARGIN)     # keeps group 2 over group 1
    assert not grouped_choice_valid(c, gsc, [2, 0], 3, 2, MARGIN)     # slot order
    assert not grouped_choice_valid(c, gsc, [0, 0], 3, 2, MARGIN)
    assert grouped_choice_valid(c, gsc, [2, 3], 3, 1, MARGIN)         # one group kept: group 1 (1.6)
    assert not grouped_choice_valid(c, gsc, [0, 1], 3, 1, MARGIN)     # group 0 (1.4) is not the best
    assert grouped_choice_valid(c, gsc, [0, 1], 3, 1, 0.3)            # unless within a wide margin


def test_grouped_choice_validity_accepts_the_oracle_and_rejects_perturbations():
    """On random DeepSeek-V3-shaped rows the oracle's own choice is always
    valid; replacing its last expert by the best unchosen expert of a dropped
    group, or swapping its first two slots, is rejected wherever the decision
    it overturns has a margin above MARGIN."""
    g = np.random.default_rng(3)
    T, E, G, SG, k = 400, 256, 8, 4, 8
    z = g.standard_normal((T, E)).astype(np.float32)
    bias = (g.standard_normal(E) * 0.05).astype(np.float32)
    idx, _ = O.route_sigmoid_grouped(z, "f32", bias, k, G, SG, True, True, 2.5)
    _, c, gsc = O.grouped_sigmoid_scores(z, "f32", bias, G, True)
    margin = O.route_sigmoid_grouped_margins(z, "f32", bias, k, G, SG, True)
    gs = E // G
    rejected = 0
    for t in range(T):
        assert grouped_choice_valid(c[t], gsc[t], idx[t], G, SG, MARGIN)
        if margin[t] < MARGIN:
            continue
        kept = {int(e) // gs for e in idx[t]}
        others = [e for e in range(E) if e // gs not in kept]
        if len(kept) == SG and others:
            alt = idx[t].copy()
            alt[-1] = max(others, key=lambda e: c[t, e])
            rejected += not grouped_choice_valid(c[t], gsc[t], alt, G, SG, MARGIN)
        sw = idx[t].copy()
        sw[[0, 1]] = sw[[1, 0]]
        assert not grouped_choice_valid(c[t], gsc[t], sw, G, SG, MARGIN)
    assert rejected > T // 2


def test_assert_close_rejects_outside_tolerance_and_nan_mismatch():
    ref = I.store(np.array([1.0, 2.0, -3.0], np.float32), "bf16")
    assert_close(ref, ref, "bf16")
    bad = I.store(np.array([1.0, 2.1, -3.0], np.float32), "bf16")
    try:
        assert_close(bad, ref, "bf16")
        raise RuntimeError("not rejected")
    except AssertionError:
        pass
    nan = I.store(np.array([1.0, np.nan, -3.0], np.float32), "bf16")
    try:
        assert_close(nan, ref, "bf16")
        raise RuntimeError("not rejected")
    except AssertionError:
        pass
