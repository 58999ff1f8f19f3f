"""Oracle pins of min-p truncation sampling + speculative verification.

[LOSSY] section 2.3 defines the min-p allowed set A = {x : p(x) >= p_base *
max p} and the truncated target p_Theta = p / Z on A; appendix G.2/G.3 state
that "truncation sampling + SD" (the lossless walk run against p_Theta) emits
p_Theta exactly and accepts one candidate with probability sum min(p_Theta,
q). The pins: hand values of the set, the identity as p_base -> 0, the
emitted distribution (chi-square), the acceptance rate, and that no emitted
token lies outside A. The test computes p_Theta itself, in fp64 from the
definition, independently of the oracle's fp32 membership rule (the random
rows used here have no logit near the cutoff).
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from sampler_cases import replicated_batch, rows_from_probs, softmax64


def p_theta(logits_row, T, p_base):
    p = softmax64(logits_row, T)
    keep = p >= p_base * p.max()
    out = np.where(keep, p, 0.0)
    return out / out.sum()


def _run(cu, par, toks, logits, q, T=1.0, seed=5, min_p=0.0):
    return oracle.verify(cu, par, toks, logits, q, temperature=T, seed=seed, max_depth=int(np.diff(cu).max()),
                         min_p=min_p)


def test_min_p_hand_values():
    lg = np.log(np.array([1.0, 2.0, 4.0, 8.0], np.float32)).astype(np.float32)
    p = oracle.target_probs(lg, 1.0)
    # p = [1, 2, 4, 8] / 15; cutoff 0.3 * 8/15 keeps 4 and 8
    pt = oracle.truncate_min_p(lg, p, oracle.min_p_theta(1.0, 0.3))
    np.testing.assert_allclose(pt, [0.0, 0.0, 4 / 12, 8 / 12], rtol=1e-6)  # logits are fp32 logs
    # at T = 2 the weights are sqrt([1, 2, 4, 8]); 0.3 * sqrt(8) < 1 keeps all
    p2 = oracle.target_probs(lg, 2.0)
    np.testing.assert_allclose(oracle.truncate_min_p(lg, p2, oracle.min_p_theta(2.0, 0.3)), p2, rtol=1e-15)
    # 0.6 * sqrt(8) = 1.70 keeps sqrt(4) and sqrt(8) only
    w = np.array([0.0, 0.0, 2.0, math.sqrt(8.0)])
    np.testing.assert_allclose(oracle.truncate_min_p(lg, p2, oracle.min_p_theta(2.0, 0.6)), w / w.sum(), rtol=1e-7)
    # the maximum always stays; min_p off gives -inf
    assert oracle.min_p_theta(1.0, 0.0) == float("-inf") and oracle.min_p_theta(0.0, 0.5) == float("-inf")
    pt1 = oracle.truncate_min_p(lg, p, oracle.min_p_theta(1.0, 0.999))
    np.testing.assert_allclose(pt1, [0.0, 0.0, 0.0, 1.0])


def test_min_p_tiny_is_identity():
    rng = np.random.default_rng(41)
    V, n = 40, 2000
    parent = np.array([-1, 0, 0, 1, -1], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.5, draft_noise=0.8)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    a = _run(cu, par, toks, logits, qq)
    b = _run(cu, par, toks, logits, qq, min_p=1e-30)
    for k in ("accept_len", "accepted_nodes", "out_tokens", "n_rejections"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("p_base", [0.1, 0.4])
def test_min_p_lossless_first_token_chi_square(p_base):
    """Truncation sampling + SD emits p_Theta ([LOSSY] G.3)."""
    rng = np.random.default_rng(51 if p_base < 0.2 else 52)
    V, n = 8, 600_000
    parent = np.array([-1, -1, 0], np.int32)  # two root children, one grandchild
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.2, draft_noise=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    out = _run(cu, par, toks, logits, qq, min_p=p_base, seed=9)
    pt = p_theta(lg[0], 1.0, p_base)
    counts = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert (counts[pt == 0] == 0).all()
    keep = pt > 0
    assert stats.chisquare(counts[keep], pt[keep] * n).pvalue > 1e-3, (counts, pt * n)
    # given root child 0 accepted, the next token ~ p_Theta at row(node 0)
    sel = out["accepted_nodes"][:, 0] == 0
    pt1 = p_theta(lg[1], 1.0, p_base)
    c1 = np.bincount(out["out_tokens"][sel, 1], minlength=V)
    assert (c1[pt1 == 0] == 0).all()
    assert stats.chisquare(c1[pt1 > 0], pt1[pt1 > 0] * sel.sum()).pvalue > 1e-3


def test_min_p_acceptance_rate():
    rng = np.random.default_rng(61)
    V, n, p_base = 8, 400_000, 0.25
    lg, q = rows_from_probs(rng, V, 2, sharp=1.0, draft_noise=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1], lg, q, n)
    out = _run(cu, par, toks, logits, qq, min_p=p_base, seed=13)
    alpha = float(np.minimum(p_theta(lg[0], 1.0, p_base), q[0].astype(np.float64)).sum())
    freq = out["accept_len"].mean()
    assert abs(freq - alpha) < 5 * math.sqrt(alpha * (1 - alpha) / n)


def test_min_p_emits_only_allowed_tokens():
    rng = np.random.default_rng(71)
    V, n, p_base, T = 50, 20_000, 0.2, 0.8
    parent = np.array([-1, -1, -1, 0, 0, 1, 3], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=2.0, draft_noise=1.5)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    out = _run(cu, par, toks, logits, qq, T=T, min_p=p_base)
    allowed = np.stack([p_theta(lg[r], T, p_base) > 0 for r in range(parent.size + 1)])
    for b in range(0, n, 97):
        pos, d = -1, int(out["accept_len"][b])
        for k in range(d + 1):
            tok = int(out["out_tokens"][b, k])
            assert allowed[pos + 1, tok], (b, k)
            if k < d:
                pos = int(out["accepted_nodes"][b, k])


def test_min_p_greedy_unaffected():
    rng = np.random.default_rng(81)
    V, n = 30, 500
    parent = np.array([-1, 0, 1, -1], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    a = oracle.verify(cu, par, toks, logits, None, temperature=0.0, seed=1, max_depth=4)
    b = oracle.verify(cu, par, toks, logits, None, temperature=0.0, seed=1, max_depth=4, min_p=0.5)
    for k in ("accept_len", "accepted_nodes", "out_tokens"):
        assert np.array_equal(a[k], b[k]), k
