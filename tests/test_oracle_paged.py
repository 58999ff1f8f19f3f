"""Oracle pins: attention over a paged KV cache.

A paged cache only changes where a slot's key and value are stored: slot t of
request b sits in block block_table[b, t // block_size] at row
t % block_size of a pool ([SD] "Tree Attention Mask Mechanics" names
PagedAttention tree variants as the kernels the mask is handed to). The pins:
the same caches scattered into a shuffled pool whose spare blocks hold NaN
give bit for bit the contiguous oracle's result; requests whose first blocks
are shared (a common prompt prefix) equal the contiguous result on caches
holding that shared data; a block id out of range is an error.
"""
import numpy as np
import pytest

import oracle
from workloads import to_paged


def _case(rng, B=3, T_list=(4, 1, 6), Hq=4, Hkv=2, D=64, L=150, bs=64):
    Lcap = ((L + max(T_list) + bs - 1) // bs) * bs
    N = sum(T_list)
    q = rng.standard_normal((N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, Lcap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Lcap, D)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(T_list)]).astype(np.int32)
    ctx = np.array([L, L - 37, L + 1][:B], np.int32)
    parent = np.concatenate([np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, T)], np.int32)
                             for T in T_list])
    return q, k, v, cu, ctx, parent


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_equals_contiguous(bs, dtype):
    rng = np.random.default_rng(801 + bs)
    q, k, v, cu, ctx, parent = _case(rng, bs=bs)
    if dtype == "bf16":  # bf16 bit patterns: the top half of the fp32 words
        q, k, v = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in (q, k, v)]
    ref = oracle.attention(q, k, v, ctx, cu, parent, Hq=4, Hkv=2, dtype=dtype)
    kp, vp, bt = to_paged(k, v, bs, rng)
    got = oracle.attention(q, kp, vp, ctx, cu, parent, Hq=4, Hkv=2, dtype=dtype, block_table=bt)
    assert np.isfinite(got).all()
    assert np.array_equal(got, ref)


def test_paged_shared_prefix():
    rng = np.random.default_rng(811)
    q, k, v, cu, ctx, parent = _case(rng, bs=64)
    kp, vp, bt = to_paged(k, v, 64, rng, share_prefix_blocks=2)
    got = oracle.attention(q, kp, vp, ctx, cu, parent, Hq=4, Hkv=2, block_table=bt)
    k2, v2 = k.copy(), v.copy()
    k2[1:, :, :128] = k[0, :, :128]
    v2[1:, :, :128] = v[0, :, :128]
    ref = oracle.attention(q, k2, v2, ctx, cu, parent, Hq=4, Hkv=2)
    assert np.array_equal(got, ref)
    assert not np.array_equal(got, oracle.attention(q, k, v, ctx, cu, parent, Hq=4, Hkv=2))


def test_paged_block_out_of_range():
    rng = np.random.default_rng(821)
    q, k, v, cu, ctx, parent = _case(rng, bs=64)
    kp, vp, bt = to_paged(k, v, 64, rng)
    bad = bt.copy()
    bad[1, 0] = kp.shape[0]
    with pytest.raises(ValueError):
        oracle.attention(q, kp, vp, ctx, cu, parent, Hq=4, Hkv=2, block_table=bad)
