"""Verification-cost model of speculative decoding on the measured kernels.

The pages ("Speculative Decoding" survey, the trade-off paragraph before
"Speculative Decoding이란?") put the speed-up of speculative decoding over
plain decoding at

    accepted tokens per verification / (verification cost + draft cost),

with both costs in units of one plain decoding step.  Here the verification
cost of a pass over M rows is the measured t(M) / t(1) of the int4 verify
sweep (a sequence draft verifies M = 5 rows, a tree draft M = 64), the draft
cost is an assumed multiple of t(1), and "accepted tokens per verification"
(the tokens a verification emits: the accepted drafts plus the target's own
next token) is swept, since acceptance depends on trained drafters that are
not part of this work.  Host-side arithmetic only.
"""
from __future__ import annotations


def speedup(accepted: float, t_ratio: float, draft_cost: float) -> float:
    """accepted / (t_ratio + draft_cost): tokens per unit of plain-decode time."""
    if accepted < 0 or t_ratio <= 0 or draft_cost < 0:
        raise ValueError("accepted >= 0, t_ratio > 0, draft_cost >= 0")
    return accepted / (t_ratio + draft_cost)


def break_even(t_ratio: float, draft_cost: float) -> float:
    """Accepted tokens per verification at which speculation only breaks even."""
    return t_ratio + draft_cost


def table(us_per_pass: dict, accepted=(1, 2, 3, 4, 5, 6, 8), draft_costs=(0.0, 0.1, 0.25, 0.5)) -> dict:
    """Speed-up grid for every measured M > 1 from the per-pass microseconds
    {M: us} of the sweep (M = 1 must be present)."""
    t1 = float(us_per_pass[1] if 1 in us_per_pass else us_per_pass["1"])
    out = {"accepted": list(accepted), "draft_cost": list(draft_costs), "t_over_t1": {}, "speedup": {},
           "break_even_accepted": {}}
    for key, us in us_per_pass.items():
        M = int(key)
        if M == 1:
            continue
        r = float(us) / t1
        out["t_over_t1"][str(M)] = round(r, 4)
        out["speedup"][str(M)] = [[round(speedup(a, r, d), 3) for a in accepted] for d in draft_costs]
        out["break_even_accepted"][str(M)] = [round(break_even(r, d), 3) for d in draft_costs]
    return out
