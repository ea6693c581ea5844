"""GOOSE's confidence-adaptive spine topology, a host policy over the spine build.

GOOSE page, section 2 (A: adaptive allocation; B: Proposition 2; C: bypass mode and dynamic
spine ratio). A step spends a fixed budget of B draft nodes: a spine of L nodes and B - L
branch nodes. Readings where the page gives the shape but no constants:

* spine acceptance rate: an exponential moving average (weight ``beta`` on the past,
  start ``ema0``) of the step's per-token estimate k / (k + 1) when the spine broke after
  k accepted tokens, or 1 when all L were accepted;
* spine share: L = round(r B) with r the average clamped to [r_min, r_max], L >= 1;
* branch widths fall linearly with depth (Proposition 2): fork j of the spine (j = 0 the
  root, j = 1.. L-1 spine nodes) gets weight L - j, and the B - L branch nodes go to the
  forks by largest remainder of their shares (ties: the shallower fork);
* bypass: once the average reaches ``bypass``, the step drafts the chain alone (L = B, every
  width 0), i.e. verifies the context match linearly.
"""
from __future__ import annotations


def linear_widths(L: int, branch: int) -> list:
    """Widths of forks 0..L-1 summing to ``branch``, proportional to L - j (largest remainder)."""
    if L <= 0 or branch <= 0:
        return [0] * max(L, 0)
    weights = [L - j for j in range(L)]
    total = sum(weights)
    shares = [branch * w / total for w in weights]
    base = [int(x) for x in shares]
    rest = branch - sum(base)
    order = sorted(range(L), key=lambda j: (-(shares[j] - base[j]), j))
    for j in order[:rest]:
        base[j] += 1
    return base


class SpineTopology:
    def __init__(self, budget: int, beta: float = 0.8, ema0: float = 0.5, r_min: float = 0.1,
                 r_max: float = 0.9, bypass: float = 0.9):
        self.B = budget
        self.beta, self.ema = beta, ema0
        self.r_min, self.r_max, self.bypass = r_min, r_max, bypass

    def plan(self) -> tuple:
        """(L, widths of forks 0..L-1) for the next step."""
        if self.ema >= self.bypass:
            return self.B, [0] * self.B
        r = min(max(self.ema, self.r_min), self.r_max)
        L = min(max(int(round(r * self.B)), 1), self.B)
        return L, linear_widths(L, self.B - L)

    def observe(self, accepted, L: int) -> float:
        """Update the average with a step whose spine of L nodes had its first k accepted
        (``accepted``: k, or one k per sequence of a batch, whose estimates are averaged)."""
        ks = [int(accepted)] if isinstance(accepted, (int,)) else [int(k) for k in accepted]
        est = sum(1.0 if k >= L else k / (k + 1.0) for k in ks) / len(ks)
        self.ema = self.beta * self.ema + (1.0 - self.beta) * est
        return self.ema


def spine_accepted(path, L: int) -> int:
    """Accepted spine tokens of a step: path nodes in the spine slots 1..L (the spine is a
    chain from the root, so they are the path's first nodes)."""
    return sum(1 for v in list(path)[1:] if 1 <= int(v) <= L)
