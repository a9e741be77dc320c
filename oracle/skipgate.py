"""SkipGS backward gate, written from the SkipGS notes ("key design" items
1-3 and the "worked example").  TEST INFRASTRUCTURE ONLY (part of the
oracle): only the tests, the smoke check and the benchmark's CPU baseline
use it.

Per training view v the gate keeps an EMA of that view's loss.  At step t
(counted from the start of the gated phase) with view v and forward loss L:
  s = L / (ema_v + eps), or +inf if v has no EMA yet;
  the gate proposes a backward iff s > 1;
  the EMA is updated whatever the decision: ema_v = beta ema_v + (1 - beta) L
  (the first loss of a view starts its EMA: reading, the notes give no
  initial value);
  during the first W steps (warm-up) every step runs its backward, and the
  proposals of the steps whose view already had an EMA are counted;
  at step W + 1 the floor rho_min = rho_lo + (1 - rho_lo) rho_hat is fixed,
  rho_hat = the fraction of those counted proposals that asked for a backward
  (reading: 0 when none was counted);
  after the warm-up a proposed skip is overridden when the backward ratio so
  far, rho_cum = b / max(t - 1, 1) with b the backwards run in steps 1..t-1,
  is below rho_min.
Defaults W = 500, beta = 0.95, rho_lo = 0.5, eps = 1e-8 (the notes' values).
"""
import math


def rho_min_of(rho_hat, rho_lo=0.5):
    """The calibrated floor of the backward ratio."""
    return rho_lo + (1.0 - rho_lo) * rho_hat


def decide(score, rho_cum, rho_min):
    """After the warm-up: (run the backward, forced by the floor)."""
    proposed = score > 1.0
    if proposed:
        return True, False
    if rho_cum < rho_min:
        return True, True
    return False, False


class SkipGate:
    def __init__(self, n_views, warmup=500, beta=0.95, rho_lo=0.5, eps=1e-8):
        self.ema = [None] * n_views
        self.W, self.beta, self.rho_lo, self.eps = warmup, beta, rho_lo, eps
        self.t = 0          # steps taken
        self.b = 0          # backwards run
        self.warm_hits = 0  # warm-up proposals for a backward (views with an EMA)
        self.warm_n = 0     # warm-up steps whose view had an EMA
        self.rho_min = None

    def step(self, view, loss):
        """One step: returns dict(backward, forced, score, rho_cum)."""
        self.t += 1
        e = self.ema[view]
        score = math.inf if e is None else loss / (e + self.eps)
        proposed = score > 1.0
        rho_cum = self.b / max(self.t - 1, 1)
        if self.t <= self.W:
            if e is not None:
                self.warm_n += 1
                self.warm_hits += 1 if proposed else 0
            backward, forced = True, False
        else:
            if self.rho_min is None:
                rho_hat = self.warm_hits / self.warm_n if self.warm_n > 0 else 0.0
                self.rho_min = rho_min_of(rho_hat, self.rho_lo)
            backward, forced = decide(score, rho_cum, self.rho_min)
        self.ema[view] = loss if e is None else self.beta * e + (1.0 - self.beta) * loss
        if backward:
            self.b += 1
        return dict(backward=backward, forced=forced, score=score, rho_cum=rho_cum)
