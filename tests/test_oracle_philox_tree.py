"""Oracle pins: Philox4x32-10 and the tree mask."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from workloads import eagle_tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["out"]]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_uniform_is_word0_mapped_to_open_interval():
    seed = 0x0123456789ABCDEF
    for rid, j, purpose, step in [(0, 0, 0, 0), (7, 3, 1, 9), (2**32 - 1, 63, 0, 2**32 - 1)]:
        w = oracle.philox4x32_10([rid, j, purpose, step], [seed & 0xFFFFFFFF, seed >> 32])
        u = oracle.uniform(seed, rid, j, purpose, step)
        assert u == (float(w[0]) + 0.5) / 2.0**32
        assert 0.0 < u < 1.0


def test_uniforms_are_uniform():
    # 64-bin chi-square of 2^16 variates over the (request, node) counter grid
    us = np.array([oracle.uniform(42, r, j, 0, 5) for r in range(1024) for j in range(64)])
    counts, _ = np.histogram(us, bins=64, range=(0.0, 1.0))
    assert stats.chisquare(counts).pvalue > 1e-3


def _mask(parent):
    anc, _ = oracle.ancestors(parent)
    T = len(parent)
    return np.array([[(int(anc[j]) >> i) & 1 for i in range(T)] for j in range(T)], dtype=np.int64)


def test_tree_mask_worked_example():
    with open(os.path.join(GOLDEN, "tree_mask_worked_example.json")) as f:
        ex = json.load(f)
    assert _mask(ex["parent"]).tolist() == ex["mask"]


def _closure_mask(parent):
    """Independent brute force: reflexive-transitive closure of the child->parent
    relation by repeated boolean matrix products."""
    T = len(parent)
    A = np.eye(T, dtype=bool)
    for j, p in enumerate(parent):
        if p >= 0:
            A[j, p] = True
    while True:
        A2 = (A.astype(np.int64) @ A.astype(np.int64)) > 0
        if (A2 == A).all():
            return A.astype(np.int64)
        A = A2


def test_tree_mask_all_small_trees():
    count = 0
    for T in range(1, 8):
        for parent in itertools.product(*[range(-1, j) for j in range(T)]):
            parent = list(parent)
            m = _mask(parent)
            assert (m == _closure_mask(parent)).all(), parent
            _, depth = oracle.ancestors(parent)
            assert (depth == m.sum(axis=1)).all()
            count += 1
    assert count == sum(__import__("math").factorial(T) for T in range(1, 8))


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 3], [-2]])
def test_tree_rejects_non_topological(bad):
    with pytest.raises(ValueError):
        oracle.ancestors(bad)


def test_eagle60_tree_shape():
    par = eagle_tree()
    assert par.size == 60
    _, depth = oracle.ancestors(par)
    assert depth.max() == 6
    levels = [int((depth == d).sum()) for d in range(1, 7)]
    assert levels == [4, 8, 9, 13, 13, 13]
    branching = [4, 3, 2, 2, 1, 1]
    nchild = np.bincount(par + 1, minlength=61)
    assert nchild[0] == 4
    for j in range(60):
        assert nchild[j + 1] <= (branching[depth[j]] if depth[j] < 6 else 0)
