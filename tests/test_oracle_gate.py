"""Pins of the oracle's SkipGS backward gate: the worked example the SkipGS
notes print (tests/golden/skipgs_worked_example.json, cited there), the
warm-up calibration of the floor on a constructed loss sequence, and the
floor as an invariant of any loss sequence."""
import json
import math
import os

from hypothesis import given, settings, strategies as st

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "skipgs_worked_example.json")))


def test_worked_example_floor_and_decisions():
    rho_min = oracle.rho_min_of(GOLD["warmup_rebound_fraction"], GOLD["rho_lo"])
    assert abs(rho_min - GOLD["rho_min"]) < 1e-15
    ex = GOLD["normal_skip"]
    score = ex["loss"] / (ex["ema"] + 1e-8)
    assert round(score, 3) == ex["score_3dp"] and score <= 1.0
    assert oracle.gate_decide(score, ex["rho_cum"], rho_min) == (ex["backward"], ex["forced"])
    fx = GOLD["forced_backward"]
    assert oracle.gate_decide(fx["score"], fx["rho_cum"], rho_min) == (fx["backward"], fx["forced"])
    # a loss above the view's baseline asks for its backward whatever the ratio
    assert oracle.gate_decide(1.01, 0.99, rho_min) == (True, False)


def test_worked_example_through_the_gate_state():
    """View A at the step of the example: baseline 0.0420, loss 0.0415, the
    backward ratio so far 0.68 over the floor 0.65 -> skipped, and the
    baseline moves to 0.95 * 0.0420 + 0.05 * 0.0415 all the same."""
    g = oracle.SkipGate(n_views=2, warmup=500)
    g.rho_min = GOLD["rho_min"]
    g.ema[0] = GOLD["normal_skip"]["ema"]
    g.t, g.b = 1999, round(0.68 * 1999)   # the step below is t = 2000: rho_cum = b / 1999
    r = g.step(0, GOLD["normal_skip"]["loss"])
    assert abs(r["rho_cum"] - 0.68) < 1e-3 and r["rho_cum"] > g.rho_min
    assert (r["backward"], r["forced"]) == (False, False) and g.b == round(0.68 * 1999)
    assert abs(g.ema[0] - (0.95 * 0.0420 + 0.05 * 0.0415)) < 1e-18
    # the forced case: ratio 0.648 under the floor, score 0.97
    g.ema[1] = 1.0
    g.t, g.b = 7999, round(0.648 * 7999)
    r = g.step(1, 0.97 * (1.0 + 1e-8))
    assert r["rho_cum"] < g.rho_min and (r["backward"], r["forced"]) == (True, True)


def test_warmup_calibrates_the_floor():
    """Ten views in turn for the 500 warm-up steps: the first visit of each
    has no baseline (always a backward, not counted); of the other 490 steps
    147 see a loss above their view's baseline, so rho_hat = 0.30 and
    rho_min = 0.65, fixed at step 501."""
    g = oracle.SkipGate(n_views=10, warmup=500)
    counted = 0
    rebounds = 0
    for t in range(1, 501):
        v = (t - 1) % 10
        if g.ema[v] is None:
            loss = 1.0
        else:
            counted += 1
            up = rebounds < 147 and counted % 10 < 3
            rebounds += 1 if up else 0
            loss = g.ema[v] * (1.5 if up else 0.5)
        r = g.step(v, loss)
        assert r["backward"] and not r["forced"]
    assert (counted, rebounds, g.warm_n, g.warm_hits) == (490, 147, 490, 147)
    assert g.rho_min is None
    g.step(0, 0.0)
    assert abs(g.rho_min - 0.65) < 1e-15 and g.b == 500


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 6), st.integers(0, 40), st.lists(st.floats(0.01, 2.0), min_size=50, max_size=400),
       st.integers(0, 2**31 - 1))
def test_floor_holds_for_any_loss_sequence(n_views, warmup, losses, seed):
    import numpy as np
    rng = np.random.default_rng(seed)
    g = oracle.SkipGate(n_views=n_views, warmup=warmup)
    seen = set()
    for t, loss in enumerate(losses, start=1):
        v = int(rng.integers(0, n_views))
        r = g.step(v, loss)
        if v not in seen:
            assert r["backward"] and math.isinf(r["score"])
            seen.add(v)
        if t <= warmup:
            assert r["backward"]
        elif not r["backward"]:
            # a skip is only allowed while the ratio so far is at the floor
            assert r["rho_cum"] >= g.rho_min and r["score"] <= 1.0
        if t > warmup + 1:
            assert g.b / t >= g.rho_min - 1.0 / t - 1e-12
