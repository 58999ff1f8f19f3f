"""Oracle pins of the lossy accept rules of [LOSSY] section 3.1.

Lenience (appendix A.3): a drafted x is accepted with h = min(1, p/(l q)) and
a rejection resamples from (p - q)+ normalised; the emitted law is
min(q, p/l) + Delta_l (p - min(p, q)) with Delta_l = sum(q - min(q, p/l)) /
sum(q - min(q, p)). Interpolation (CoS; appendix A.1 gives the same form for
DIVERSED): h = min(1, nu/q) with nu = lambda p + (1 - lambda) q, residual
(nu - q)+ normalised, which is (p - q)+ normalised; the emitted law is nu.

Pins: both laws by chi-square on one drafted position at V = 8 (expected laws
computed here in fp64 from the closed forms), the acceptance rates
sum min(q, p/l) and sum min(q, nu), l = 1 and lambda = 1 reproduce the
lossless walk bit for bit, a tiny l or lambda -> 0 accepts (almost) every
draft, and the argument checks.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from sampler_cases import replicated_batch, rows_from_probs, softmax64


def _run(cu, par, toks, logits, q, rule, param, seed=5, T=1.0):
    return oracle.verify(cu, par, toks, logits, q, temperature=T, seed=seed, max_depth=int(np.diff(cu).max()),
                         rule=rule, rule_param=param)


def lenience_law(p, q, ell):
    ceil = np.minimum(q, p / ell)
    delta = (q - ceil).sum() / (q - np.minimum(q, p)).sum()
    return ceil + delta * (p - np.minimum(p, q))


@pytest.mark.parametrize("ell", [0.5, 0.8])
def test_lenience_law_and_acceptance(ell):
    rng = np.random.default_rng(501 if ell < 0.6 else 502)
    V, n = 8, 800_000
    lg, q = rows_from_probs(rng, V, 2, sharp=1.0, draft_noise=1.3)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1], lg, q, n)
    out = _run(cu, par, toks, logits, qq, "lenience", ell, seed=11)
    p, q0 = softmax64(lg[0]), q[0].astype(np.float64)
    law = lenience_law(p, q0, np.float64(np.float32(ell)))
    assert abs(law.sum() - 1.0) < 1e-6  # the closed form is a distribution
    c = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(c, law / law.sum() * n).pvalue > 1e-3, (c, law * n)
    a = float(np.minimum(q0, p / np.float32(ell)).sum())
    freq = out["accept_len"].mean()
    assert abs(freq - a) < 5 * math.sqrt(a * (1 - a) / n)


@pytest.mark.parametrize("lam", [0.3, 0.7])
def test_interpolation_law_and_acceptance(lam):
    rng = np.random.default_rng(511 if lam < 0.5 else 512)
    V, n = 8, 800_000
    lg, q = rows_from_probs(rng, V, 2, sharp=1.0, draft_noise=1.3)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1], lg, q, n)
    out = _run(cu, par, toks, logits, qq, "interpolation", lam, seed=13)
    p, q0 = softmax64(lg[0]), q[0].astype(np.float64)
    lam32 = np.float64(np.float32(lam))
    nu = lam32 * p + (1 - lam32) * q0
    c = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(c, nu / nu.sum() * n).pvalue > 1e-3, (c, nu * n)
    a = float(np.minimum(q0, nu).sum())
    freq = out["accept_len"].mean()
    assert abs(freq - a) < 5 * math.sqrt(a * (1 - a) / n)


@pytest.mark.parametrize("rule", ["lenience", "interpolation"])
def test_param_one_is_lossless(rule):
    rng = np.random.default_rng(521)
    V, n = 50, 3000
    parent = np.array([-1, -1, 0, 0, 1, 2, -1], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.5, draft_noise=0.9)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    a = oracle.verify(cu, par, toks, logits, qq, temperature=1.0, seed=3, max_depth=7)
    b = _run(cu, par, toks, logits, qq, rule, 1.0, seed=3)
    for k in ("accept_len", "accepted_nodes", "out_tokens", "n_rejections"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("rule", ["lenience", "interpolation"])
def test_extreme_relaxation_accepts_drafts(rule):
    """l -> 0 (p/(l q) huge) or lambda -> 0 (nu -> q) accepts every draft with
    p(x) > 0: a chain is accepted to its end."""
    rng = np.random.default_rng(531)
    V, n, K = 30, 2000, 4
    parent = np.arange(-1, K - 1, dtype=np.int32)
    lg, q = rows_from_probs(rng, V, K + 1, sharp=1.0, draft_noise=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    out = _run(cu, par, toks, logits, qq, rule, 1e-9, seed=7)
    assert (out["accept_len"] == K).all()


def test_rule_arguments_checked():
    rng = np.random.default_rng(541)
    lg, q = rows_from_probs(rng, 5, 2)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1], lg, q, 3)
    for rule, param in (("lenience", 0.0), ("interpolation", 1.5)):
        with pytest.raises(ValueError):
            _run(cu, par, toks, logits, qq, rule, param)
    with pytest.raises(ValueError):
        oracle.verify(cu, par, toks, logits, None, temperature=1.0, seed=1, siblings="deterministic",
                      rule="lenience", rule_param=0.5)
    with pytest.raises(ValueError):
        _run(cu, par, toks, logits, qq, "typical", 0.5)
