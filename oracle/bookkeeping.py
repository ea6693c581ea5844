"""Draft-efficiency bookkeeping (TALON page, section 5.3).

Logged quantities: N_v verification passes, N_d draft steps, L output tokens, and the
draft-to-target cost ratio gamma. The page defines the draft efficiency
eta = N_d / N_v and the wall-clock speedup Speedup ~ E[A] / (1 + gamma * eta).

Reading: E[A] is the mean number of tokens one verification pass emits, L / N_v,
where each pass emits its A_t accepted draft tokens plus the bonus token, so
L = sum_t (A_t + 1) and a step with no draft work (N_d = 0, A_t = 0) gives
Speedup = 1. The concept page's L/(1 + L*c) equals this when eta = E[A].

Parity: pinned by closed forms only (no page prints a worked example of these
numbers); beyond them this function is "parity unpinned".
"""
from __future__ import annotations


def bookkeeping(accepted, draft_steps: int, gamma: float) -> dict:
    """accepted: A_t per verification pass; draft_steps: N_d; gamma: cost ratio."""
    N_v = len(accepted)
    if N_v == 0:
        raise ValueError("need at least one verification pass")
    L = sum(int(a) + 1 for a in accepted)
    EA = L / N_v
    eta = draft_steps / N_v
    return {"N_v": N_v, "N_d": int(draft_steps), "L": L, "E_A": EA, "eta": eta,
            "speedup": EA / (1.0 + gamma * eta)}
