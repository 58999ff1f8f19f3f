"""Closed forms the source pages state for speculative sampling (test pins).

These are consequences of the method, not the method: they predict the
statistics that many seeded runs of the walk must reproduce.
"""
from __future__ import annotations

import numpy as np


def tv(p, q) -> float:
    """Total variation distance 1/2 sum |p - q| ([LOSSY] section 3.1)."""
    return 0.5 * float(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum())


def acceptance(p, q) -> float:
    """Probability that a draft x ~ q is accepted: sum_x min(p, q) ([LOSSY] G.1)."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def chain_expected_emitted(alphas) -> float:
    """1 + sum_i prod_{j<=i} alpha_j: expected tokens per step of a chain
    ([SPEED] acceptance-length formula; [SD] E[tau] product form)."""
    total, prod = 1.0, 1.0
    for a in alphas:
        prod *= a
        total += prod
    return total


def chain_expected_emitted_iid(alpha: float, K: int) -> float:
    """(1 - alpha^(K+1)) / (1 - alpha) ([SD] '1. Chain / Linear Speculative Decoding')."""
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def sibling_rejection_chain(p, q, k: int) -> tuple[float, list]:
    """Probability that k i.i.d. draws from q at one position are all rejected
    when the i-th is tested against the (i-1)-times-renormalised residual:
    prod_i (1 - sum min(p_{i-1}, q)). Returns it and the residual sequence."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    seq = [p]
    prob = 1.0
    cur = p
    for _ in range(k):
        prob *= 1.0 - np.minimum(cur, q).sum()
        pos = np.maximum(cur - q, 0.0)
        cur = pos / pos.sum()
        seq.append(cur)
    return prob, seq
