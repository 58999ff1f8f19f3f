"""Oracle pins of the deterministic-candidate sibling rule.

[LOSSY] appendix G.3 analyses a position whose candidates x^(1), x^(2), ...
are fixed (not drawn from q): x^(i) is tried only if all earlier ones were
rejected, and is accepted with probability p~_i(x^(i)), where p~_i is the
target with x^(1..i-1) removed and renormalised. Its telescoping product gives
Pr[reach x^(i)] = 1 - sum_{l<i} p(x^(l)) and Pr[accept x^(i)] = p(x^(i)); with
a final draw from the target without the candidates the emitted token follows
p exactly (with p_Theta in place of p under min-p truncation).

Pins: hand values of the removal; the G.3 closed forms for reaching and
accepting each candidate (Monte Carlo within 5 sigma); the emitted law
(chi-square) at the root and one level down; a repeated candidate is never
accepted; on a chain it coincides bit for bit with the sampled-draft rule fed
a one-hot q (a special case of [SD]'s rule: accept iff u <= p(x), residual =
p without x); greedy is unchanged. The expected laws are computed here in
fp64 from the definition of softmax, not by the oracle.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from sampler_cases import rows_from_probs, softmax64


def p_theta(logits_row, T, p_base=0.0):
    p = softmax64(logits_row, T)
    if p_base <= 0:
        return p
    keep = p >= p_base * p.max()
    out = np.where(keep, p, 0.0)
    return out / out.sum()


def fixed_batch(parent, tokens, logit_rows, n_req):
    """n_req copies of one tree whose node tokens are fixed (deterministic
    candidates); rows are the root row then one per node, as in the packing."""
    parent = np.asarray(parent, np.int32)
    T = parent.size
    cu = (np.arange(n_req + 1, dtype=np.int64) * T).astype(np.int32)
    par = np.tile(parent, n_req)
    toks = np.tile(np.asarray(tokens, np.int32), n_req)
    logits = np.tile(logit_rows.astype(np.float32), (n_req, 1))
    return cu, par, toks, logits


def _det(cu, par, toks, logits, T=1.0, seed=7, min_p=0.0, q=None):
    return oracle.verify(cu, par, toks, logits, q, temperature=T, seed=seed, max_depth=int(np.diff(cu).max()),
                         min_p=min_p, siblings="deterministic")


def test_remove_candidate_hand_values():
    out, R = oracle.remove_candidate([0.5, 0.3, 0.2], 0)
    assert R == pytest.approx(0.5, abs=1e-15)
    np.testing.assert_allclose(out, [0.0, 0.6, 0.4], rtol=1e-15)
    out2, R2 = oracle.remove_candidate(out, 0)  # already removed: unchanged
    assert R2 == pytest.approx(1.0, abs=1e-15)
    np.testing.assert_allclose(out2, out, rtol=1e-15)
    out3, R3 = oracle.remove_candidate([0.0, 1.0, 0.0], 1)  # nothing left: kept
    assert R3 == 0.0
    np.testing.assert_array_equal(out3, [0.0, 1.0, 0.0])


@pytest.mark.parametrize("p_base", [0.0, 0.15])
def test_g3_reach_and_accept_probabilities(p_base):
    """Pr[accept x^(i)] = p(x^(i)) and Pr[reach x^(i)] = 1 - sum_{l<i} p(x^(l))."""
    rng = np.random.default_rng(301 if p_base == 0 else 302)
    V, n = 8, 400_000
    parent = np.array([-1, -1, -1], np.int32)
    lg, _ = rows_from_probs(rng, V, parent.size + 1, sharp=1.0)
    pt = p_theta(lg[0], 1.0, p_base)
    cands = np.argsort(-pt, kind="stable")[:3]  # the three most likely tokens
    cu, par, toks, logits = fixed_batch(parent, cands, lg, n)
    out = _det(cu, par, toks, logits, min_p=p_base, seed=17)
    first = np.where(out["accept_len"] > 0, out["accepted_nodes"][:, 0], -1)
    reach = 1.0
    for i in range(3):
        a = pt[cands[i]]
        freq = (first == i).mean()
        assert abs(freq - a) < 5 * math.sqrt(a * (1 - a) / n) + 1e-12, (i, freq, a)
        reached = (out["n_rejections"] >= i).mean()  # rejections before node i (no accept earlier)
        assert abs(reached - reach) < 5 * math.sqrt(max(reach * (1 - reach), 1e-12) / n), (i, reached, reach)
        reach -= a


@pytest.mark.parametrize("p_base", [0.0, 0.2])
def test_deterministic_rule_is_lossless(p_base):
    """The emitted token follows p (p_Theta) at the root and, below an
    accepted candidate, at that candidate's row."""
    rng = np.random.default_rng(311 if p_base == 0 else 312)
    V, n = 8, 600_000
    parent = np.array([-1, -1, 0, 0], np.int32)  # two root candidates, two below node 0
    lg, _ = rows_from_probs(rng, V, parent.size + 1, sharp=1.2)
    p0, p1 = p_theta(lg[0], 1.0, p_base), p_theta(lg[1], 1.0, p_base)
    o0, o1 = np.argsort(-p0, kind="stable"), np.argsort(-p1, kind="stable")
    tokens = [o0[0], o0[1], o1[0], o1[2]]
    cu, par, toks, logits = fixed_batch(parent, tokens, lg, n)
    out = _det(cu, par, toks, logits, min_p=p_base, seed=23)
    c0 = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert (c0[p0 == 0] == 0).all()
    assert stats.chisquare(c0[p0 > 0], p0[p0 > 0] * n).pvalue > 1e-3, (c0, p0 * n)
    sel = out["accepted_nodes"][:, 0] == 0
    c1 = np.bincount(out["out_tokens"][sel, 1], minlength=V)
    assert (c1[p1 == 0] == 0).all()
    assert stats.chisquare(c1[p1 > 0], p1[p1 > 0] * sel.sum()).pvalue > 1e-3


def test_repeated_candidate_is_never_accepted():
    rng = np.random.default_rng(321)
    V, n = 6, 100_000
    parent = np.array([-1, -1, -1], np.int32)
    lg, _ = rows_from_probs(rng, V, 4, sharp=1.0)
    p = softmax64(lg[0])
    x = int(np.argmax(p))
    cu, par, toks, logits = fixed_batch(parent, [x, x, (x + 1) % V], lg, n)
    out = _det(cu, par, toks, logits, seed=29)
    first = np.where(out["accept_len"] > 0, out["accepted_nodes"][:, 0], -1)
    assert not (first == 1).any()
    # the third candidate is reached with 1 - p(x) and accepted with p(x + 1)
    a = p[(x + 1) % V]
    assert abs((first == 2).mean() - a) < 5 * math.sqrt(a * (1 - a) / n)
    c = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(c, p * n).pvalue > 1e-3


def test_chain_matches_sampled_rule_with_one_hot_q():
    """On a chain every position has one candidate; [SD]'s rule with
    q = one-hot(candidate) accepts iff u <= p(x) and leaves p without x as the
    residual, which is exactly the deterministic rule."""
    rng = np.random.default_rng(331)
    V, n, K = 40, 3000, 4
    parent = np.arange(-1, K - 1, dtype=np.int32)
    lg, _ = rows_from_probs(rng, V, K + 1, sharp=1.5)
    tokens = rng.integers(0, V, size=K).astype(np.int32)
    cu, par, toks, logits = fixed_batch(parent, tokens, lg, n)
    q1 = np.zeros((K + 1, V), np.float32)
    for r in range(K):
        q1[r, tokens[r]] = 1.0  # row r (position before node r) drafts node r's token
    qq = np.tile(q1, (n, 1))
    a = _det(cu, par, toks, logits, seed=31)
    b = oracle.verify(cu, par, toks, logits, qq, temperature=1.0, seed=31, max_depth=K)
    for k in ("accept_len", "accepted_nodes", "out_tokens", "n_rejections"):
        assert np.array_equal(a[k], b[k]), k


def test_deterministic_greedy_unaffected():
    rng = np.random.default_rng(341)
    V, n = 30, 400
    parent = np.array([-1, 0, 1, -1], np.int32)
    lg, _ = rows_from_probs(rng, V, parent.size + 1, sharp=1.0)
    tokens = rng.integers(0, V, size=parent.size)
    cu, par, toks, logits = fixed_batch(parent, tokens, lg, n)
    a = oracle.verify(cu, par, toks, logits, None, temperature=0.0, seed=1, max_depth=4)
    b = oracle.verify(cu, par, toks, logits, None, temperature=0.0, seed=1, max_depth=4, siblings="deterministic")
    for k in ("accept_len", "accepted_nodes", "out_tokens"):
        assert np.array_equal(a[k], b[k]), k
