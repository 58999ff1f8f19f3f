"""Builders of small sampler batches shared by the oracle and GPU sampler tests.

They only arrange inputs (rows of logits and draft probabilities, trees,
draft tokens drawn from q with numpy); no verification arithmetic lives here.
"""
from __future__ import annotations

import numpy as np


def draw(rng: np.random.Generator, q: np.ndarray, n: int) -> np.ndarray:
    """n independent tokens from the fp32 distribution q (inverse CDF in fp64)."""
    c = np.cumsum(q.astype(np.float64))
    return np.minimum(np.searchsorted(c, rng.random(n) * c[-1], side="right"), q.size - 1).astype(np.int32)


def replicated_batch(rng, parent, logit_rows, q_rows, n_req: int):
    """n_req copies of one tree whose rows (root row first, then one per node)
    are `logit_rows`/`q_rows` [T+1, V]; each copy draws its own draft tokens:
    node j's token ~ q at its parent's row. Returns (cu, parent, tokens, logits, q)."""
    parent = np.asarray(parent, np.int32)
    T = parent.size
    V = logit_rows.shape[1]
    cu = (np.arange(n_req + 1, dtype=np.int64) * T).astype(np.int32)
    par = np.tile(parent, n_req)
    toks = np.empty((n_req, T), np.int32)
    for j in range(T):
        toks[:, j] = draw(rng, q_rows[parent[j] + 1], n_req)
    logits = np.tile(logit_rows.astype(np.float32), (n_req, 1))
    q = np.tile(q_rows.astype(np.float32), (n_req, 1))
    assert logits.shape == (n_req * (T + 1), V)
    return cu, par, toks.reshape(-1), logits, q


def rows_from_probs(rng, V: int, n_rows: int, sharp: float = 1.0, draft_noise: float = 0.7):
    """Random target logits and a perturbed, renormalised draft distribution per row."""
    logits = (rng.standard_normal((n_rows, V)) * sharp).astype(np.float32)
    d = logits.astype(np.float64) + rng.standard_normal((n_rows, V)) * draft_noise
    q = np.exp(d - d.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    return logits, q.astype(np.float32)


def softmax64(logits_row, T=1.0):
    z = np.asarray(logits_row, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()
