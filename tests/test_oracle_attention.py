"""Oracle pins: tree-masked GQA attention.

Special cases reduce to textbook attention, checked against CPU torch in
fp64: a single node (plain decode attention), a chain (causal mask over the
draft tail), a star (each node sees the context and itself), and a general
tree against an explicit dense mask built by brute force. Constant keys give
the mean of the visible values.
"""
import numpy as np
import pytest
import torch

import oracle


def _inputs(rng, B, T_list, Hq, Hkv, D, L, Lcap=None):
    N = sum(T_list)
    Lcap = Lcap or (L + max(T_list))
    q = rng.standard_normal((N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, Lcap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Lcap, D)).astype(np.float32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(T_list)
    ctx = np.full(B, L, np.int32)
    return q, k, v, cu, ctx


def _dense_reference(q, k, v, cu, ctx, parent, Hq, Hkv, visible_fn):
    """softmax(q K^T / sqrt(D) + mask) V in fp64 torch, mask from visible_fn(parent_b, j, i)."""
    D = q.shape[2]
    G = Hq // Hkv
    out = np.zeros(q.shape, np.float64)
    for b in range(len(ctx)):
        T = cu[b + 1] - cu[b]
        L = ctx[b]
        par = parent[cu[b]:cu[b + 1]]
        for j in range(T):
            n = cu[b] + j
            keys = list(range(L)) + [L + i for i in range(T) if visible_fn(par, j, i)]
            for h in range(Hq):
                g = h // G
                Q = torch.tensor(q[n, h], dtype=torch.float64)
                K = torch.tensor(k[b, g, keys], dtype=torch.float64)
                Vv = torch.tensor(v[b, g, keys], dtype=torch.float64)
                w = torch.softmax(K @ Q / np.sqrt(D), dim=0)
                out[n, h] = (w @ Vv).numpy()
    return out


def test_single_node_is_decode_attention():
    rng = np.random.default_rng(1)
    q, k, v, cu, ctx = _inputs(rng, 3, [1, 1, 1], 4, 2, 16, 37)
    parent = np.full(3, -1, np.int32)
    got = oracle.attention(q, k, v, ctx, cu, parent, Hq=4, Hkv=2)
    ref = _dense_reference(q, k, v, cu, ctx, parent, 4, 2, lambda par, j, i: i == j)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_chain_is_causal_over_draft_tail():
    rng = np.random.default_rng(2)
    q, k, v, cu, ctx = _inputs(rng, 2, [5, 3], 8, 2, 32, 20)
    parent = np.concatenate([np.arange(-1, 4), np.arange(-1, 2)]).astype(np.int32)
    got = oracle.attention(q, k, v, ctx, cu, parent, Hq=8, Hkv=2)
    ref = _dense_reference(q, k, v, cu, ctx, parent, 8, 2, lambda par, j, i: i <= j)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_star_tree_sees_only_itself():
    rng = np.random.default_rng(3)
    q, k, v, cu, ctx = _inputs(rng, 1, [6], 2, 1, 8, 11)
    parent = np.full(6, -1, np.int32)
    got = oracle.attention(q, k, v, ctx, cu, parent, Hq=2, Hkv=1)
    ref = _dense_reference(q, k, v, cu, ctx, parent, 2, 1, lambda par, j, i: i == j)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _is_ancestor_or_self(par, j, i):
    x = j
    while x >= 0:
        if x == i:
            return True
        x = par[x]
    return False


def test_general_tree_matches_dense_mask_and_gqa_mapping():
    rng = np.random.default_rng(4)
    T_list = [7, 1, 4]
    q, k, v, cu, ctx = _inputs(rng, 3, T_list, 6, 3, 16, 9)
    parent = np.array([-1, 0, 0, 1, -1, 3, 2, -1, -1, 0, 0, 2], np.int32)
    got = oracle.attention(q, k, v, ctx, cu, parent, Hq=6, Hkv=3)
    ref = _dense_reference(q, k, v, cu, ctx, parent, 6, 3, _is_ancestor_or_self)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # a wrong head mapping (h % Hkv instead of h // G) must be visible
    assert np.abs(got[:, 1] - got[:, 0]).max() > 1e-3


def test_constant_keys_average_visible_values():
    rng = np.random.default_rng(5)
    T_list = [6]
    q, k, v, cu, ctx = _inputs(rng, 1, T_list, 2, 1, 8, 13)
    k[:] = 0.25
    parent = np.array([-1, 0, 1, 0, 3, -1], np.int32)
    got = oracle.attention(q, k, v, ctx, cu, parent, Hq=2, Hkv=1)
    anc, depth = oracle.ancestors(parent)
    for j in range(6):
        keys = list(range(13)) + [13 + i for i in range(6) if (int(anc[j]) >> i) & 1]
        want = v[0, 0, keys].astype(np.float64).mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(got[j, h], want, rtol=0, atol=1e-12)


def test_bf16_bits_and_item_subset():
    rng = np.random.default_rng(6)
    q, k, v, cu, ctx = _inputs(rng, 2, [3, 2], 4, 1, 16, 10)
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    bits = [x.view(torch.int16).numpy().view(np.uint16) for x in (tq, tk, tv)]
    parent = np.array([-1, 0, 0, -1, 0], np.int32)
    got = oracle.attention(*bits, ctx, cu, parent, Hq=4, Hkv=1, dtype="bf16")
    ref = oracle.attention(*(x.float().numpy() for x in (tq, tk, tv)), ctx, cu, parent, Hq=4, Hkv=1)
    np.testing.assert_array_equal(got, ref)
    items = np.array([[4, 3], [0, 0], [2, 1]], np.int64)
    sub = oracle.attention(*bits, ctx, cu, parent, Hq=4, Hkv=1, dtype="bf16", items=items)
    for r, (n, h) in enumerate(items):
        np.testing.assert_array_equal(sub[r], got[n, h])


def test_bad_packing_raises():
    rng = np.random.default_rng(7)
    q, k, v, cu, ctx = _inputs(rng, 1, [3], 1, 1, 8, 4)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, ctx, cu, np.array([-1, 2, 0], np.int32), Hq=1, Hkv=1)
