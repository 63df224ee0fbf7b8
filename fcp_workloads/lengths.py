"""Lognormal sequence-length draws that fill a token budget.

The FCP paper (Sec. 2.1, Figure 2) describes context lengths as long-tailed and roughly
lognormal; its traces are not public, so lengths are drawn here as ln L ~ N(ln median,
sigma^2), rounded to the nearest integer and redrawn when outside [lo, hi]. The draw
continues until the budget is met and the sequence crossing the budget is cut to fit,
which is the split rule of the packing simulation in "Another View on Context Parallel
for LLMs" (section "Computational Simulation").
"""
import numpy as np


def lognormal_lengths(rng: np.random.Generator, median: float, sigma: float,
                      lo: int, hi: int, budget: int) -> list:
    out, total = [], 0
    mu = float(np.log(median))
    while total < budget:
        while True:
            length = int(np.rint(np.exp(rng.normal(mu, sigma))))
            if lo <= length <= hi:
                break
        if total + length > budget:
            length = budget - total
        out.append(length)
        total += length
    return out
