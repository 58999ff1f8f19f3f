"""Oracle pins: target distribution, residual, inverse CDF and the walk.

Pins come from what the pages fix: the losslessness theorem ([SD] "Proof of
Lossless Distribution Equivalence"), acceptance = sum min(p, q) = 1 - TV
([LOSSY] G.1, F.1), the chain expectation ([SPEED] AL formula, [SD] E[tau]),
the pipeline example ([SD] pipeline figure), draft == target accepting
everything ([LOSSY] 2.1 h(x) = 1), plus brute force on tiny inputs.
"""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from closed_forms import acceptance, chain_expected_emitted, sibling_rejection_chain, tv
from sampler_cases import draw, replicated_batch, rows_from_probs, softmax64


def test_softmax_hand_values():
    p = oracle.target_probs(np.log(np.array([1.0, 2.0, 3.0], np.float32)), 1.0)
    np.testing.assert_allclose(p, [1 / 6, 2 / 6, 3 / 6], rtol=1e-7)
    p2 = oracle.target_probs(np.log(np.array([1.0, 2.0, 3.0], np.float32)), 2.0)
    w = np.sqrt([1.0, 2.0, 3.0])
    np.testing.assert_allclose(p2, w / w.sum(), rtol=1e-7)
    lg = np.array([0.5, -np.inf, 1.5, 3.0], np.float32)
    p3 = oracle.target_probs(lg, 0.5)
    assert p3[1] == 0.0 and abs(p3.sum() - 1.0) < 1e-15
    np.testing.assert_allclose(oracle.target_probs(lg + np.float32(64.0), 0.5), p3, rtol=1e-12)
    with pytest.raises(ValueError):
        oracle.target_probs(np.array([-np.inf, -np.inf], np.float32), 1.0)
    with pytest.raises(ValueError):
        oracle.target_probs(np.array([0.0, np.nan], np.float32), 1.0)
    assert oracle.argmax(np.array([1.0, 3.0, -2.0, 3.0], np.float32)) == 1


def test_residual_values_and_identity():
    r, R = oracle.residual([0.5, 0.3, 0.2], [0.2, 0.5, 0.3])
    assert R == pytest.approx(0.3, abs=1e-15)
    np.testing.assert_allclose(r, [1.0, 0.0, 0.0])
    rng = np.random.default_rng(0)
    for _ in range(50):
        p = rng.dirichlet(np.ones(17))
        q = rng.dirichlet(np.ones(17))
        r, R = oracle.residual(p, q)
        assert R == pytest.approx(np.maximum(q - p, 0).sum(), abs=1e-14)  # sum (p-q)+ = sum (q-p)+
        assert R == pytest.approx(tv(p, q), abs=1e-14)
        assert r.sum() == pytest.approx(1.0, abs=1e-14) and (r >= 0).all()
    same, R0 = oracle.residual(p, p)  # zero mass: kept unchanged
    assert R0 == 0.0 and (same == p).all()


def test_inverse_cdf_brute_force_and_histogram():
    rng = np.random.default_rng(1)
    for _ in range(200):
        V = int(rng.integers(1, 12))
        P = rng.random(V) * (rng.random(V) < 0.7)
        if P.sum() == 0:
            P[rng.integers(0, V)] = 0.3
        u = float(rng.random())
        y, margin = oracle.inverse_cdf(P, u)
        cdf = np.cumsum(P) / P.sum()
        want = int(np.flatnonzero(cdf > u)[0])
        assert y == want and P[y] > 0
        assert margin == pytest.approx(min(u - (cdf[y - 1] if y else 0.0), cdf[y] - u), abs=1e-12)
    # exact boundary: the strict '>' skips the zero-mass token sitting on u*total
    assert oracle.inverse_cdf([0.5, 0.0, 0.5], 0.5)[0] == 2
    assert oracle.inverse_cdf([0.25, 0.25, 0.0, 0.5], 0.5)[0] == 3
    P = np.array([0.1, 0.0, 0.4, 0.25, 0.0, 0.25])
    ys = np.array([oracle.inverse_cdf(P, u)[0] for u in rng.random(40000)])
    counts = np.bincount(ys, minlength=6)
    assert counts[1] == 0 and counts[4] == 0
    nz = P > 0
    assert stats.chisquare(counts[nz], P[nz] * ys.size).pvalue > 1e-3


def _run(cu, par, toks, logits, q, T=1.0, seed=1234, **kw):
    return oracle.verify(cu, par, toks, logits, q, temperature=T, seed=seed, **kw)


@pytest.mark.parametrize("tree", ["chain", "tree3"])
def test_lossless_first_token_chi_square(tree):
    """10^6 seeded trials at vocab 8: the first emitted token ~ p."""
    rng = np.random.default_rng(11 if tree == "chain" else 12)
    V, n = 8, 1_000_000
    parent = np.array([-1, 0], np.int32) if tree == "chain" else np.array([-1, -1, -1], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.0, draft_noise=1.2)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    out = _run(cu, par, toks, logits, qq)
    first = out["out_tokens"][:, 0]
    counts = np.bincount(first, minlength=V)
    p_root = softmax64(lg[0])
    res = stats.chisquare(counts, p_root * n)
    assert res.pvalue > 1e-3, (counts, p_root * n)
    if tree == "chain":
        # second token given node 0 accepted: ~ p at the row after node 0
        sel = out["accept_len"] >= 1
        c2 = np.bincount(out["out_tokens"][sel, 1], minlength=V)
        assert stats.chisquare(c2, softmax64(lg[1]) * sel.sum()).pvalue > 1e-3
    else:
        # given child c accepted, the bonus token ~ p at row(c)
        for c in range(3):
            sel = out["accepted_nodes"][:, 0] == c
            c2 = np.bincount(out["out_tokens"][sel, 1], minlength=V)
            assert stats.chisquare(c2, softmax64(lg[1 + c]) * sel.sum()).pvalue > 1e-3


def test_acceptance_rate_is_one_minus_tv():
    rng = np.random.default_rng(21)
    V, n = 8, 400_000
    lg, q = rows_from_probs(rng, V, 2, sharp=1.0, draft_noise=1.0)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1], lg, q, n)
    out = _run(cu, par, toks, logits, qq, seed=77)
    p = softmax64(lg[0])
    alpha = acceptance(p, q[0].astype(np.float64))
    assert alpha == pytest.approx(1.0 - tv(p, q[0]), abs=1e-7)  # q rounded to fp32
    freq = out["accept_len"].mean()
    sigma = math.sqrt(alpha * (1 - alpha) / n)
    assert abs(freq - alpha) < 5 * sigma


def test_chain_expected_emitted_tokens():
    rng = np.random.default_rng(31)
    V, n, K = 16, 300_000, 4
    lg, q = rows_from_probs(rng, V, K + 1, sharp=1.5, draft_noise=0.6)
    cu, par, toks, logits, qq = replicated_batch(rng, np.arange(-1, K - 1), lg, q, n)
    out = _run(cu, par, toks, logits, qq, seed=99)
    emitted = out["accept_len"] + 1
    alphas = [acceptance(softmax64(lg[i]), q[i]) for i in range(K)]
    want = chain_expected_emitted(alphas)
    assert abs(emitted.mean() - want) < 5 * emitted.std() / math.sqrt(n)
    # per-position conditional acceptance rates
    for i in range(K):
        reached = out["accept_len"] >= i
        acc = out["accept_len"][reached] >= i + 1
        assert abs(acc.mean() - alphas[i]) < 5 * math.sqrt(alphas[i] * (1 - alphas[i]) / reached.sum())


def test_sibling_rejection_probability():
    rng = np.random.default_rng(41)
    V, n, k = 8, 400_000, 3
    lg, q = rows_from_probs(rng, V, k + 1, sharp=1.0, draft_noise=1.5)
    cu, par, toks, logits, qq = replicated_batch(rng, [-1] * k, lg, q, n)
    out = _run(cu, par, toks, logits, qq, seed=5)
    prob_none, _ = sibling_rejection_chain(softmax64(lg[0]), q[0], k)
    none = (out["accept_len"] == 0).mean()
    assert abs(none - prob_none) < 5 * math.sqrt(prob_none * (1 - prob_none) / n)
    assert (out["n_rejections"][out["accept_len"] == 0] == k).all()


def test_draft_equal_target_accepts_everything():
    rng = np.random.default_rng(51)
    V = 300
    for parent in (np.arange(-1, 6), np.array([-1, 0, 0, 1, 2, -1, 5])):
        T = parent.size
        lg = (rng.standard_normal((T + 1, V)) * 3).astype(np.float32)
        q = np.stack([oracle.target_probs(r, 1.0) for r in lg]).astype(np.float32)
        cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, 2000)
        out = _run(cu, par, toks, logits, qq, seed=3)
        _, depth = oracle.ancestors(parent)
        ok = out["flag_depth"] < 0
        assert ok.mean() > 0.99
        # every accept test passes, so the walk reaches a leaf: its depth = accept_len
        for b in np.flatnonzero(ok):
            last = out["accepted_nodes"][b, out["accept_len"][b] - 1]
            assert not (parent == last).any()  # stopped at a leaf
            assert out["accept_len"][b] == depth[last]
            assert out["accepted_nodes"][b, 0] == np.flatnonzero(parent == -1)[0]  # first root child


def test_pipeline_example_accept_three_reject_fourth():
    """[SD] pipeline figure: x1..x3 accepted, x4 rejected and replaced, x5 discarded."""
    V = 10
    rng = np.random.default_rng(61)
    lg = rng.standard_normal((6, V)).astype(np.float32)
    toks = np.array([1, 2, 3, 4, 5], np.int32)
    q = np.full((6, V), 1.0 / V, np.float32)
    for i in range(3):
        lg[i, toks[i]] = 20.0  # p(x_i) ~ 1 >= q(x_i): always accepted
    lg[3, toks[3]] = -np.inf   # p(x4) = 0: always rejected
    cu = np.array([0, 5], np.int32)
    out = _run(cu, np.arange(-1, 4).astype(np.int32), toks, lg, q, seed=8)
    assert out["accept_len"][0] == 3
    assert out["out_tokens"][0, :3].tolist() == [1, 2, 3]
    y = out["out_tokens"][0, 3]
    assert y != 4 and out["out_tokens"][0, 4] == -1
    P = softmax64(lg[3])
    r = np.maximum(P - q[3].astype(np.float64), 0)
    yy, _ = oracle.inverse_cdf(r, oracle.uniform(8, 0, 0, 1, 0))
    assert y == yy


def test_zero_draft_probability_follows_formula():
    V = 5
    lg = np.zeros((2, V), np.float32)
    q = np.array([[0.0, 0.25, 0.25, 0.25, 0.25]] * 2, np.float32)
    out = _run(np.array([0, 1], np.int32), np.array([-1], np.int32), np.array([0], np.int32), lg, q)
    assert out["accept_len"][0] == 1  # p(0) > 0 = q(0): ratio +inf, accepted
    lg[0, 0] = -np.inf
    out = _run(np.array([0, 1], np.int32), np.array([-1], np.int32), np.array([0], np.int32), lg, q)
    assert out["accept_len"][0] == 0  # p(0) = 0 = q(0): rejected


def test_empty_tree_draws_bonus_from_root():
    rng = np.random.default_rng(71)
    V = 50
    lg = rng.standard_normal((3, V)).astype(np.float32)
    q = np.full((3, V), 1.0 / V, np.float32)
    cu = np.array([0, 0, 1], np.int32)  # request 0 empty, request 1 one node
    out = _run(cu, np.array([-1], np.int32), np.array([7], np.int32), lg, q, seed=9, max_depth=1)
    assert out["accept_len"][0] == 0
    y, _ = oracle.inverse_cdf(softmax64(lg[0]), oracle.uniform(9, 0, 0, 1, 0))
    assert out["out_tokens"][0, 0] == y
    assert out["uniforms"][0] == oracle.uniform(9, 1, 0, 0, 0)  # node 0 of request 1
    assert out["uniforms"][1 + 0] == oracle.uniform(9, 0, 0, 1, 0)  # [N + b] final draw of request 0


def _greedy_brute(parent, toks, lg_rows):
    """Enumerate every node; a node is reachable if every node on its path
    carries the argmax token of its parent's row. The accepted path is the
    deepest reachable one, earlier index sequences winning ties."""
    T = len(parent)
    am = [int(np.flatnonzero(r == r.max())[0]) for r in lg_rows]
    best = []
    for j in range(T):
        path = []
        x = j
        while x >= 0:
            path.append(x)
            x = parent[x]
        path = path[::-1]
        if all(toks[n] == am[parent[n] + 1] for n in path):
            # a path is taken only if no earlier sibling also matched at any level
            ok = True
            for n in path:
                sibs = [s for s in range(T) if parent[s] == parent[n] and s < n and toks[s] == toks[n]]
                if sibs:
                    ok = False
            if ok and len(path) > len(best):
                best = path
    last = best[-1] if best else -1
    return best, am[last + 1]


def test_greedy_matches_brute_force():
    rng = np.random.default_rng(81)
    V = 3
    for _ in range(300):
        T = int(rng.integers(0, 7))
        parent = np.array([rng.integers(-1, j) if j else -1 for j in range(T)], np.int32)
        lg = rng.integers(0, 3, size=(T + 1, V)).astype(np.float32)  # many ties
        toks = rng.integers(0, V, size=T).astype(np.int32)
        out = _run(np.array([0, T], np.int32), parent, toks, lg, None, T=0.0, max_depth=6)
        path, bonus = _greedy_brute(list(parent), toks, lg)
        assert out["accept_len"][0] == len(path)
        assert out["accepted_nodes"][0, :len(path)].tolist() == path
        assert out["out_tokens"][0, len(path)] == bonus


def test_invalid_inputs_flag_request():
    lg = np.zeros((5, 6), np.float32)  # N + B = 3 + 2 rows
    q = np.full((5, 6), 1 / 6, np.float32)
    out = _run(np.array([0, 2, 3], np.int32), np.array([-1, 1, -1], np.int32), np.array([0, 1, 2], np.int32),
               lg, q, max_depth=2)
    assert out["status"][0] & 0x01 and out["out_tokens"][0].tolist() == [-1, -1, -1]
    assert out["status"][1] == 0
    out = _run(np.array([0, 1], np.int32), np.array([-1], np.int32), np.array([6], np.int32), lg[:2], q[:2])
    assert out["status"][0] & 0x04
