"""Oracle pins: budgeted super-tree packing ([ECHO] section 3.1, Figure 3 step 3).

The packer keeps the K_max best candidates of the batch's candidate trees by
(smallest score on the path, descending; request; local index) and flattens
them request by request. Pins, none of which restates that rule:
- path scores (cumulative log q, which never rise along a path): the kept
  set is the ancestor-closed set of K_max nodes with the largest total score,
  found by brute force over every such set of a tiny batch;
- arbitrary scores: the kept set equals a best-first expansion of the
  super-tree (a heap over the frontier; a node enters with the smaller of its
  own score and its parent's entry key, ties to the lower candidate index):
  a frontier procedure instead of a global sort;
- invariants on random batches: N = min(K_max, candidates), every kept
  node's parent kept, packed parents in [-1, j-1], original order inside a
  request, tokens and sources consistent; budget 0 and budget >= M; NaN
  scores rank last; invalid requests keep nothing and are flagged.
"""
import heapq
import itertools

import numpy as np
import pytest

import oracle


def _batch(rng, sizes, monotone=True, quant=None):
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    par, tok, sc = [], [], []
    for T in sizes:
        p = np.array([-1] + [int(rng.integers(-1, j)) for j in range(1, T)], np.int32)[:T]
        s = np.zeros(T, np.float32)
        for j in range(T):
            step = np.log(rng.uniform(0.01, 1.0))
            if not monotone:
                step = rng.normal(0, 2)
            if quant:
                step = np.round(step * quant) / quant
            s[j] = np.float32((s[p[j]] if p[j] >= 0 else 0.0) + step)
        par.append(p)
        tok.append(rng.integers(0, 1000, T).astype(np.int32))
        sc.append(s)
    return cu, np.concatenate(par), np.concatenate(tok), np.concatenate(sc)


def _kept(cu, out):
    return set(out["src"].tolist())


def _closed(cu, par, kept):
    for m in kept:
        b = int(np.searchsorted(cu, m, side="right") - 1)
        p = par[m]
        if p >= 0 and cu[b] + p not in kept:
            return False
    return True


def test_brute_force_max_total_score():
    rng = np.random.default_rng(1001)
    for trial in range(40):
        sizes = [int(x) for x in rng.integers(1, 5, size=int(rng.integers(1, 4)))]
        cu, par, tok, sc = _batch(rng, sizes)
        M = int(cu[-1])
        K = int(rng.integers(0, M + 1))
        out = oracle.pack(cu, par, tok, sc, K)
        best, best_set = -np.inf, None
        for sub in itertools.combinations(range(M), K):
            s = set(sub)
            if not _closed(cu, par, s):
                continue
            tot = float(sum(sc[m] for m in s))
            if tot > best + 1e-9:
                best, best_set = tot, s
        assert out["total_nodes"] == K
        assert _kept(cu, out) == best_set, (trial, sizes, K)


def _best_first(cu, par, sc, K):
    """Heap expansion of the super-tree: repeatedly take the frontier node with
    the highest key (ties: lowest candidate index); children join the frontier
    once their parent is taken, keyed by min(own score, parent's key)."""
    B = len(cu) - 1
    kids = {}
    heap = []
    for b in range(B):
        for j in range(cu[b + 1] - cu[b]):
            m = cu[b] + j
            s = -np.inf if np.isnan(sc[m]) else float(sc[m])
            if par[m] < 0:
                heapq.heappush(heap, (-s, m))
            else:
                kids.setdefault(cu[b] + par[m], []).append(m)
    order = []
    while heap and len(order) < K:
        negkey, m = heapq.heappop(heap)
        order.append(m)
        for c in kids.get(m, []):
            s = -np.inf if np.isnan(sc[c]) else float(sc[c])
            heapq.heappush(heap, (-min(s, -negkey), c))
    return order


@pytest.mark.parametrize("monotone", [True, False])
def test_equals_best_first_expansion(monotone):
    rng = np.random.default_rng(1011 if monotone else 1012)
    for _ in range(30):
        sizes = [int(x) for x in rng.integers(0, 65, size=int(rng.integers(1, 12)))]
        cu, par, tok, sc = _batch(rng, sizes, monotone=monotone)
        M = int(cu[-1])
        K = int(rng.integers(0, M + 2))
        out = oracle.pack(cu, par, tok, sc, K)
        assert _kept(cu, out) == set(_best_first(cu, par, sc, K))


def test_invariants_and_edges():
    rng = np.random.default_rng(1021)
    for _ in range(30):
        sizes = [int(x) for x in rng.integers(0, 65, size=int(rng.integers(1, 40)))]
        cu, par, tok, sc = _batch(rng, sizes, monotone=bool(rng.integers(0, 2)), quant=4)
        M = int(cu[-1])
        K = int(rng.integers(0, M + 5))
        out = oracle.pack(cu, par, tok, sc, K)
        N = out["total_nodes"]
        assert N == min(K, M) and out["cu_nodes"][-1] == N and out["status"] == 0
        assert (np.diff(out["cu_nodes"]) >= 0).all() and (np.diff(out["cu_nodes"]) <= np.diff(cu)).all()
        kept = _kept(cu, out)
        assert _closed(cu, par, kept)
        for b in range(len(sizes)):
            s = out["src"][out["cu_nodes"][b]:out["cu_nodes"][b + 1]]
            assert (np.diff(s) > 0).all() and ((s >= cu[b]) & (s < cu[b + 1])).all()
            p = out["parent"][out["cu_nodes"][b]:out["cu_nodes"][b + 1]]
            for j, (m, pj) in enumerate(zip(s, p)):
                assert -1 <= pj < j
                assert (pj < 0) == (par[m] < 0)
                if pj >= 0:
                    assert s[pj] == cu[b] + par[m]
        assert np.array_equal(out["draft_tokens"], tok[out["src"]])
    # budget >= M: the identity packing; budget 0: nothing
    cu, par, tok, sc = _batch(rng, [5, 0, 7])
    full = oracle.pack(cu, par, tok, sc, 100)
    assert np.array_equal(full["cu_nodes"], cu) and np.array_equal(full["parent"], par)
    assert oracle.pack(cu, par, tok, sc, 0)["total_nodes"] == 0


def test_nan_and_invalid_requests():
    rng = np.random.default_rng(1031)
    cu, par, tok, sc = _batch(rng, [4, 4])
    sc = sc.copy()
    sc[1] = np.nan  # counts as -inf: it and its subtree go last
    out = oracle.pack(cu, par, tok, sc, 7)
    missing = set(range(8)) - _kept(cu, out)
    assert len(missing) == 1 and (missing == {1} or par[list(missing)[0]] >= 0)
    bad = par.copy()
    bad[5] = 3  # parent not before the node: request 1 keeps nothing
    out = oracle.pack(cu, bad, tok, sc, 8)
    assert out["status"] & 0x01 and out["cu_nodes"][2] == out["cu_nodes"][1] == 4
    # offsets that go backwards reject the whole batch
    out = oracle.pack(np.array([0, 5, 3, 8], np.int32), np.zeros(8, np.int32) - 1, tok, sc, 8)
    assert out["status"] & 0x02 and out["total_nodes"] == 0
