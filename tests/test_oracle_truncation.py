"""Oracle pins of the eta allowed set and of truncation-based verification.

[LOSSY] section 2.3 defines eta-sampling's allowed set
A = {x : p(x) >= min(eps, delta exp(-H(p)))}; section 3.2 defines
truncation-based verification (SpecCascade with the min-p set, typical
acceptance with the eta set): h(x) = 1{x in A}, which generates
q(x) / Z_A(q) on A and 0 elsewhere; appendix G.3 states that truncation
sampling + SD emits p_Theta exactly.

Pins: hand values of the eta set on a three-token row (entropy, threshold,
set), the entropy against scipy's routine, the invariants that the argmax is
always allowed (p_max >= exp(-H)) and that a uniform row is wholly allowed;
the emitted law of truncation-based verification against the pages' q/Z_A(q)
by chi-square with one child and with three i.i.d. siblings, its per-position
acceptance 1 - (1 - Z_A(q))^k, a leaf's bonus token from p_Theta, the chain's
expected accepted length from the per-position Z_A(q) (weakly above the
lossless rate sum min(p_Theta, q), appendix G.5), and truncation sampling + SD
with the eta set emitting p_Theta. The test computes every expected law
itself, in fp64, from the definitions.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from sampler_cases import replicated_batch, rows_from_probs, softmax64


def eta_set(logits_row, T, eps, delta):
    p = softmax64(logits_row, T)
    H = float(stats.entropy(p))
    return p >= min(eps, delta * math.exp(-H)), p


def min_p_set(logits_row, T, p_base):
    p = softmax64(logits_row, T)
    return p >= p_base * p.max(), p


def _run(cu, par, toks, logits, q, *, rule="lossless", seed=5, T=1.0, min_p=0.0, eta=None, **kw):
    return oracle.verify(cu, par, toks, logits, q, temperature=T, seed=seed, max_depth=int(np.diff(cu).max()),
                         rule=rule, min_p=min_p, eta=eta, **kw)


def test_eta_hand_values():
    lg = np.log(np.array([0.7, 0.2, 0.1], np.float64)).astype(np.float32)
    p = oracle.target_probs(lg, 1.0)
    # H = -(0.7 ln 0.7 + 0.2 ln 0.2 + 0.1 ln 0.1) = 0.8018185 nats, exp(-H) = 0.4485150
    assert abs(oracle.row_entropy(lg, 1.0) - 0.8018185) < 1e-6
    # eps 0.15, delta 0.3: tau = min(0.15, 0.1345545) keeps 0.7 and 0.2;
    # threshold on l - l_max: ln S + ln tau = -ln 0.7 + ln 0.3 - H = -1.6491164
    pt, th, margin = oracle.truncate_eta(lg, p, 1.0, 0.15, 0.3)
    np.testing.assert_allclose(pt, [0.7 / 0.9, 0.2 / 0.9, 0.0], rtol=1e-6)
    assert abs(th - (-1.6491164)) < 1e-6
    # nearest token: ln 0.1 - ln 0.7 = -1.9459101, 0.2967937 below the threshold
    # (ln 0.2 - ln 0.7 = -1.2527630 is 0.3963534 above it)
    assert abs(margin - 0.2967937) < 1e-6
    # eps 0.25, delta 1: tau = 0.25 keeps only 0.7
    pt, _, _ = oracle.truncate_eta(lg, p, 1.0, 0.25, 1.0)
    np.testing.assert_allclose(pt, [1.0, 0.0, 0.0])
    # eps 0.05: tau = 0.05 keeps all
    pt, _, _ = oracle.truncate_eta(lg, p, 1.0, 0.05, 1.0)
    np.testing.assert_allclose(pt, p, rtol=1e-15)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_eta_entropy_and_invariants(T):
    rng = np.random.default_rng(601 + int(10 * T))
    for _ in range(20):
        V = int(rng.integers(2, 300))
        lg = (rng.standard_normal(V) * 3).astype(np.float32)
        p64 = softmax64(lg, T)
        assert abs(oracle.row_entropy(lg, T) - stats.entropy(p64)) < 1e-10
        eps, delta = float(rng.uniform(0.001, 0.5)), float(rng.uniform(0.05, 1.0))
        p = oracle.target_probs(lg, T)
        pt, _, margin = oracle.truncate_eta(lg, p, T, eps, delta)
        assert pt[int(np.argmax(lg))] > 0.0  # p_max >= exp(-H) >= delta exp(-H)
        assert abs(pt.sum() - 1.0) < 1e-12
        keep, _ = eta_set(lg, T, eps, delta)
        if margin > 1e-9:  # away from the boundary the set is the definition's
            assert np.array_equal(pt > 0, keep)
    lg = np.zeros(50, np.float32)
    pt, _, _ = oracle.truncate_eta(lg, oracle.target_probs(lg, 1.0), 1.0, 0.4, 1.0)
    np.testing.assert_allclose(pt, np.full(50, 0.02), rtol=1e-12)  # uniform: tau <= 1/V


def _sets(kind, lg, T=1.0):
    if kind == "min_p":
        return {"min_p": 0.2}, min_p_set(lg, T, np.float32(0.2))
    eps, delta = oracle.eta_params((0.1, 0.4))
    return {"eta": (0.1, 0.4)}, eta_set(lg, T, eps, delta)


@pytest.mark.parametrize("kind", ["min_p", "eta"])
@pytest.mark.parametrize("k", [1, 3])
def test_truncation_verification_law(kind, k):
    V, n = 8, 600_000
    for s in range(611 + 10 * k + (0 if kind == "min_p" else 5), 700):  # first seed with a proper allowed set
        rng = np.random.default_rng(s)
        lg, q = rows_from_probs(rng, V, k + 1, sharp=1.6, draft_noise=1.2)
        args, (keep, _) = _sets(kind, lg[0])
        if 2 < keep.sum() < V:
            break
    cu, par, toks, logits, qq = replicated_batch(rng, [-1] * k, lg, q, n)
    out = _run(cu, par, toks, logits, qq, rule="truncation", seed=17, **args)
    assert (out["status"] == 0).all() and (out["flag_kind"] != 2).all()
    q0 = q[0].astype(np.float64)
    ZA = float(q0[keep].sum())
    law = np.where(keep, q0, 0.0) / ZA
    c = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert c[~keep].sum() == 0
    e = law[keep] * n
    assert stats.chisquare(c[keep], e).pvalue > 1e-3, (c, law * n)
    a = 1.0 - (1.0 - ZA) ** k
    freq = float((out["accept_len"] > 0).mean())
    assert abs(freq - a) < 5 * math.sqrt(a * (1 - a) / n) + 1e-12
    # acceptance is membership: deterministic, no uniform involved
    toks2 = toks.reshape(n, k)
    first_ok = np.argmax(keep[toks2], axis=1)
    acc = keep[toks2].any(axis=1)
    got = out["accepted_nodes"][:, 0]
    assert np.array_equal(got[acc], first_ok[acc]) and (got[~acc] == -1).all()


@pytest.mark.parametrize("kind", ["min_p", "eta"])
def test_truncation_leaf_bonus_is_p_theta(kind):
    rng = np.random.default_rng(631 if kind == "min_p" else 632)
    V, n = 8, 400_000
    lg, q = rows_from_probs(rng, V, 2, sharp=1.6, draft_noise=0.6)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1], lg, q, n)
    args, _ = _sets(kind, lg[0])
    _, (keep1, p1) = _sets(kind, lg[1])
    out = _run(cu, par, toks, logits, qq, rule="truncation", seed=19, **args)
    sel = out["accept_len"] == 1
    m = int(sel.sum())
    assert m > n // 4
    c = np.bincount(out["out_tokens"][sel, 1], minlength=V)
    pt = np.where(keep1, p1, 0.0)
    pt /= pt.sum()
    assert c[~keep1].sum() == 0
    assert stats.chisquare(c[keep1], pt[keep1] * m).pvalue > 1e-3


def test_truncation_chain_block_efficiency():
    """E[accepted] of a chain = sum_i prod_{j<=i} Z_A(q_j), at least the
    lossless truncated walk's sum_i prod_{j<=i} sum min(p_Theta, q_j)."""
    rng = np.random.default_rng(641)
    V, n, K = 12, 300_000, 3
    parent = np.arange(-1, K - 1, dtype=np.int32)
    lg, q = rows_from_probs(rng, V, K + 1, sharp=1.4, draft_noise=0.9)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    za, al = [], []
    for r in range(K):
        keep, p = min_p_set(lg[r], 1.0, np.float32(0.15))
        qr = q[r].astype(np.float64)
        pt = np.where(keep, p, 0.0) / p[keep].sum()
        za.append(qr[keep].sum())
        al.append(np.minimum(pt, qr).sum())
    e_tr = sum(np.prod(za[: i + 1]) for i in range(K))
    e_ll = sum(np.prod(al[: i + 1]) for i in range(K))
    assert e_tr >= e_ll
    tr = _run(cu, par, toks, logits, qq, rule="truncation", min_p=0.15, seed=23)
    ll = _run(cu, par, toks, logits, qq, min_p=0.15, seed=23)
    sd = float(tr["accept_len"].std()) / math.sqrt(n)
    assert abs(tr["accept_len"].mean() - e_tr) < 5 * sd
    sd = float(ll["accept_len"].std()) / math.sqrt(n)
    assert abs(ll["accept_len"].mean() - e_ll) < 5 * sd


def test_eta_truncation_sd_emits_p_theta():
    rng = np.random.default_rng(651)
    V, n = 8, 600_000
    lg, q = rows_from_probs(rng, V, 4, sharp=1.6, draft_noise=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1, -1, -1], lg, q, n)
    out = _run(cu, par, toks, logits, qq, eta=(0.1, 0.4), seed=29)
    assert (out["flag_kind"] != 2).all()
    keep, p = _sets("eta", lg[0])[1]
    pt = np.where(keep, p, 0.0) / p[keep].sum()
    c = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert c[~keep].sum() == 0
    assert stats.chisquare(c[keep], pt[keep] * n).pvalue > 1e-3


def test_eta_near_tie_flag_and_arguments():
    rng = np.random.default_rng(661)
    lg, q = rows_from_probs(rng, 20, 3, sharp=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1, 0], lg, q, 4)
    # a band wider than every logit difference: some threshold in it changes
    # the first position's outcome of every request
    out = _run(cu, par, toks, logits, qq, eta=(0.1, 0.4), set_tol=1e3)
    assert (out["flag_depth"] == 0).all() and (out["flag_kind"] == 2).all()
    with pytest.raises(ValueError):  # truncation-based verification needs an allowed set
        _run(cu, par, toks, logits, qq, rule="truncation")
    with pytest.raises(ValueError):
        _run(cu, par, toks, logits, qq, eta=(1.5, 0.4))
    with pytest.raises(ValueError):
        _run(cu, par, toks, logits, qq, eta=(0.1, 0.4), min_p=0.2)
    with pytest.raises(ValueError):
        oracle.verify(cu, par, toks, logits, None, temperature=1.0, seed=1, siblings="deterministic",
                      rule="truncation", min_p=0.2)
