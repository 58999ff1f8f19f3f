"""GPU parity of the sampler's edge cases against the fp64 oracle, in both
walk layouts (one workgroup per request, and several "slices" per request).

- Greedy ties: integer-valued logits with the row maximum at tokens 4095 and
  4096, the two sides of a 4096-token chunk boundary: the argmax is the
  lowest index ([SD] greedy verification; ties broken by the lowest token).
- q(x) = 0 for a drafted token ([SD] "Heterogeneous Vocabulary Alignment"
  speaks of forcing rejection; the acceptance formula min(1, p/q) gives
  +inf, so the token is accepted iff p(x) > 0, and rejected when p(x) = 0).
- Rows with no distribution: a NaN at index 0, a +inf, all -inf. The walk
  stops there without a token and the status word says why.
- A zero residual: q = 2p (q is used as given, unnormalised), so a
  rejection leaves sum max(0, p - q) = 0; the distribution is kept and the
  status word says so.
- Zero-mass tokens around the inverse-CDF crossing ([SD] "Mathematical
  Rejection Sampling Algorithm": the resample is from the normalised
  residual; zero-mass tokens must never be drawn).
- Empty requests (no draft node: one token drawn from p at the root).

Each case also runs in a batch large enough (over 128 MiB of logits) that
the walk reduces the rows it reaches itself instead of after a statistics
pass over every row.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_16_amd as sv
from gpu_helpers import compare_walk

pytestmark = pytest.mark.gpu

V_EVEN, V_ODD = 3 * 4096 + 100, 3 * 4096 + 99  # four chunks; vector and scalar loads
LAYOUTS = ["single", "sliced"]


def _softmax_rows(lg):
    z = lg.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def _run(cu, parent, tokens, logits, q, T, layout, seed=0xE06E):
    """GPU walk in the given layout and the oracle on the same bytes."""
    md = max(int(np.diff(cu).max()), 1)
    r = sv.sample(torch.from_numpy(cu).cuda(), torch.from_numpy(parent).cuda(), torch.from_numpy(tokens).cuda(),
                  torch.from_numpy(logits).cuda(), None if q is None else torch.from_numpy(q).cuda(),
                  temperature=T, seed=seed, max_nodes=md, uniforms_out=True, residual_passes=True,
                  walk_mode=layout)
    torch.cuda.synchronize()
    ref = oracle.verify(cu, parent, tokens, logits, q if T > 0 else None, temperature=T, seed=seed, max_depth=md)
    assert np.array_equal(r["uniforms"].cpu().numpy(), ref["uniforms"])
    return r, ref


@pytest.mark.parametrize("B", [8, 800])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_ties_across_a_chunk_boundary(layout, T, B):
    # (800 requests: 3200 rows of 12388 logits, over 128 MiB, so the walk
    # reduces the rows it reaches and merges them with one wave)
    rng = np.random.default_rng(1201)
    V = V_EVEN
    parent = np.array([-1, 0, -1], np.int32)  # node 0, its child 1, and a second root child 2
    n_rows = B * (parent.size + 1)
    lg = rng.integers(-4, 4, size=(n_rows, V)).astype(np.float32)
    # the maximum 6 at 4095 and 4096 in every row, and again at 8191 in half of them
    lg[:, 4095] = 6.0
    lg[:, 4096] = 6.0
    lg[::2, 8191] = 6.0
    q = _softmax_rows(lg + rng.standard_normal(lg.shape).astype(np.float32)).astype(np.float32)
    toks = np.empty((B, parent.size), np.int32)
    toks[:, 0] = np.where(np.arange(B) % 2 == 0, 4095, 4096)  # the argmax, or its tie partner
    toks[:, 1] = 4095
    toks[:, 2] = 4095
    cu = (np.arange(B + 1) * parent.size).astype(np.int32)
    r, ref = _run(cu, np.tile(parent, B), toks.reshape(-1), lg, q, T, layout)
    assert int(r["status"].item()) == 0
    compare_walk(r, ref, B, greedy=T == 0, max_flagged=0 if B <= 64 else B // 64)
    if T == 0:
        acc = r["accept_len"].cpu().numpy()
        out = r["out_tokens"].cpu().numpy()
        # requests whose first node carries 4096 accept the second root child (4095)
        assert (acc[1::2] == 1).all() and (out[1::2, 0] == 4095).all()
        assert (acc[0::2] == 2).all() and (out[0::2, 2] == 4095).all()


@pytest.mark.parametrize("B", [6, 800])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_draft_probability_zero(layout, B):
    """q(x) = 0 at a drafted token: accepted iff p(x) > 0. (800 requests:
    3200 rows of 12388 logits, over 128 MiB, so the walk reduces its own
    rows.)"""
    rng = np.random.default_rng(1202)
    V = V_EVEN
    parent = np.array([-1, -1, 0], np.int32)
    lg = (rng.standard_normal((B * 4, V)) * 3).astype(np.float32)
    q = _softmax_rows(lg + rng.standard_normal(lg.shape).astype(np.float32)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, 3)).astype(np.int32)
    for b in range(B):
        root = 4 * b
        q[root, toks[b, 0]] = 0.0  # first root child: q = 0, p > 0: always accepted
        if b % 2:
            lg[root, toks[b, 0]] = -np.inf  # ... unless p = 0 as well: always rejected
        q[root + 1, toks[b, 2]] = 0.0  # node 0's child: q = 0
    cu = (np.arange(B + 1) * 3).astype(np.int32)
    r, ref = _run(cu, np.tile(parent, B), toks.reshape(-1), lg, q, 1.0, layout)
    assert int(r["status"].item()) == 0
    compare_walk(r, ref, B, greedy=False, max_flagged=0 if B <= 64 else B // 64)
    nodes = r["accepted_nodes"].cpu().numpy()
    assert (nodes[0::2, 0] == 0).all() and (nodes[0::2, 1] == 2).all()
    assert (nodes[1::2, 0] != 0).all()


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_rows_without_distribution_reduced_by_the_walk(layout, T):
    """The same four rows without a distribution in a batch of 1000 requests
    (3000 rows of 12388 logits, over 128 MiB), so that the walk reduces the
    rows it reaches itself instead of a statistics pass: its NaN / +inf test
    (a NaN chunk sum, or a per-logit test of a chunk whose maximum is -inf)
    must stop the same walks."""
    rng = np.random.default_rng(1204)
    V, B = V_EVEN, 1000
    parent = np.array([-1, 0], np.int32)
    lg = (rng.standard_normal((B * 3, V)) * 2).astype(np.float32)
    q = _softmax_rows(lg + rng.standard_normal(lg.shape).astype(np.float32)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, 2)).astype(np.int32)
    for b in range(5):
        a = int(np.argmax(lg[3 * b]))
        toks[b] = [a, 17]
        q[3 * b, a] = 0.0
    lg[3 * 0 + 1, 0] = np.nan
    lg[3 * 1 + 1, 5000] = np.inf
    lg[3 * 2 + 1, :] = -np.inf
    lg[3 * 3 + 1, V - 1] = np.nan
    cu = (np.arange(B + 1) * 2).astype(np.int32)
    call = sv.SampleCall(torch.from_numpy(cu).cuda(), torch.from_numpy(np.tile(parent, B)).cuda(),
                         torch.from_numpy(toks.reshape(-1)).cuda(), torch.from_numpy(lg).cuda(),
                         None if T == 0 else torch.from_numpy(q).cuda(), temperature=T, seed=1, max_nodes=2,
                         walk_mode=layout)
    assert call.walk_layout()[1]  # the walk reduces the rows it reaches
    del call
    r, ref = _run(cu, np.tile(parent, B), toks.reshape(-1), lg, q, T, layout)
    st = int(r["status"].item())
    assert st & 0x08 and not (st & ~0x08)
    assert all(ref["status"][b] & 0x08 for b in range(4)) and ref["status"][4] == 0
    compare_walk(r, ref, B, greedy=T == 0, max_flagged=max(2, B // 64))
    acc = r["accept_len"].cpu().numpy()
    out = r["out_tokens"].cpu().numpy()
    assert (acc[:4] == 1).all() and (out[:4, 1] == -1).all()


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_rows_without_distribution(layout, T):
    """Row 1 (after node 0) of request k holds a NaN at index 0, a +inf, only
    -inf, or a NaN in the last chunk; node 0 is always accepted (greedy: it
    is the argmax; sampled: q = 0 at a finite logit), so the walk reaches the
    row and stops there without a token. Request 4 is clean."""
    rng = np.random.default_rng(1203)
    V, B = V_EVEN, 5
    parent = np.array([-1, 0], np.int32)
    lg = (rng.standard_normal((B * 3, V)) * 2).astype(np.float32)
    q = _softmax_rows(lg + rng.standard_normal(lg.shape).astype(np.float32)).astype(np.float32)
    toks = np.zeros((B, 2), np.int32)
    for b in range(B):
        a = int(np.argmax(lg[3 * b]))
        toks[b] = [a, 17]
        q[3 * b, a] = 0.0
    lg[3 * 0 + 1, 0] = np.nan
    lg[3 * 1 + 1, 5000] = np.inf
    lg[3 * 2 + 1, :] = -np.inf
    lg[3 * 3 + 1, V - 1] = np.nan
    cu = (np.arange(B + 1) * 2).astype(np.int32)
    r, ref = _run(cu, np.tile(parent, B), toks.reshape(-1), lg, q, T, layout)
    st = int(r["status"].item())
    assert st & 0x08 and not (st & ~0x08)
    assert all(ref["status"][b] & 0x08 for b in range(4)) and ref["status"][4] == 0
    compare_walk(r, ref, B, greedy=T == 0, max_flagged=0)
    acc = r["accept_len"].cpu().numpy()
    out = r["out_tokens"].cpu().numpy()
    assert (acc[:4] == 1).all() and (out[:4, 1] == -1).all()
    assert out[4, acc[4]] >= 0


@pytest.mark.parametrize("B", [16, 800])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_zero_residual(layout, B):
    """q = 2 p at the root row: a rejection (u > 1/2) leaves no residual mass;
    the distribution stays p and the next sibling is tested against it."""
    rng = np.random.default_rng(1204)
    V = V_EVEN
    parent = np.array([-1, -1, -1], np.int32)
    lg = (rng.standard_normal((B * 4, V)) * 2).astype(np.float32)
    p = _softmax_rows(lg)
    q = _softmax_rows(lg + rng.standard_normal(lg.shape).astype(np.float32)).astype(np.float32)
    for b in range(B):
        q[4 * b] = (2.0 * p[4 * b]).astype(np.float32)
    toks = np.stack([rng.integers(0, V, size=3) for _ in range(B)]).astype(np.int32)
    cu = (np.arange(B + 1) * 3).astype(np.int32)
    r, ref = _run(cu, np.tile(parent, B), toks.reshape(-1), lg, q, 1.0, layout, seed=0x2E50)
    rejected = (ref["n_rejections"] > 0).any()
    assert rejected  # some request rejects a root child
    st = int(r["status"].item())
    assert bool(st & 0x10) == bool((ref["status"] & 0x10).any()) and not (st & ~0x10)
    compare_walk(r, ref, B, greedy=False, max_flagged=0 if B <= 64 else B // 64)
    ok = ref["flag_depth"] < 0
    assert np.array_equal(r["residual_passes"].cpu().numpy()[ok], ref["n_rejections"][ok])


@pytest.mark.parametrize("B", [24, 800])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("V", [V_EVEN, V_ODD])
def test_zero_mass_tokens_in_the_draw(layout, V, B):
    """Rows where most tokens have zero mass (-inf logits), with the finite
    ones scattered over every chunk and zero-mass runs around them; root
    children are rejected often (q far from p), so draws come from residuals
    and from p. No zero-mass token is ever emitted."""
    rng = np.random.default_rng(1205 + V % 2)
    parent = np.array([-1, -1, 0], np.int32)
    lg = np.full((B * 4, V), -np.inf, np.float32)
    for r in range(lg.shape[0]):
        keep = rng.choice(V, size=40, replace=False)
        lg[r, keep] = (rng.standard_normal(40) * 2).astype(np.float32)
    q = _softmax_rows(np.where(np.isfinite(lg), rng.standard_normal(lg.shape) * 3, -np.inf)).astype(np.float32)
    toks = np.empty((B, 3), np.int32)
    for b in range(B):
        fin = np.flatnonzero(np.isfinite(lg[4 * b]))
        toks[b] = rng.choice(fin, size=3)
    cu = (np.arange(B + 1) * 3).astype(np.int32)
    r, ref = _run(cu, np.tile(parent, B), toks.reshape(-1), lg, q, 1.0, layout, seed=0x2E51)
    assert int(r["status"].item()) & ~0x10 == 0
    compare_walk(r, ref, B, greedy=False, max_flagged=1 if B <= 64 else B // 64)
    acc = r["accept_len"].cpu().numpy()
    out = r["out_tokens"].cpu().numpy()
    nodes = r["accepted_nodes"].cpu().numpy()
    for b in range(B):
        pos = 4 * b
        for d in range(acc[b] + 1):
            assert np.isfinite(lg[pos, out[b, d]]), (b, d)
            if d < acc[b]:
                pos = 4 * b + 1 + nodes[b, d]


@pytest.mark.parametrize("reps", [1, 400])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_empty_requests(layout, T, reps):
    """Requests without draft nodes among ones with trees: each emits one
    token from its root row (the argmax when greedy). (400 copies: 2400
    requests, 4400 rows of 12388 logits, so the walk reduces its own rows.)"""
    rng = np.random.default_rng(1206)
    V = V_EVEN
    sizes = np.tile(np.array([0, 3, 0, 0, 2, 0], np.int32), reps)
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    parent = np.concatenate([np.arange(-1, s - 1) for s in sizes]).astype(np.int32)
    rows = int(cu[-1]) + sizes.size
    lg = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    q = _softmax_rows(lg + rng.standard_normal(lg.shape).astype(np.float32)).astype(np.float32)
    toks = rng.integers(0, V, size=int(cu[-1])).astype(np.int32)
    r, ref = _run(cu, parent, toks, lg, q, T, layout)
    assert int(r["status"].item()) == 0
    compare_walk(r, ref, sizes.size, greedy=T == 0, max_flagged=0 if sizes.size <= 64 else sizes.size // 64)
    acc = r["accept_len"].cpu().numpy()
    out = r["out_tokens"].cpu().numpy()
    for b in np.flatnonzero(sizes == 0):
        assert acc[b] == 0 and out[b, 0] >= 0
        if T == 0:
            assert out[b, 0] == int(np.argmax(lg[cu[b] + b]))
