"""GPU parity of budgeted super-tree packing against the oracle (bit for bit:
integer outputs), and a packed batch verified by the sampler."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_16_amd as sv
from gpu_helpers import compare_walk
from sampler_cases import rows_from_probs
from test_oracle_pack import _batch

pytestmark = pytest.mark.gpu


def _check(cu, par, tok, sc, budget):
    ref = oracle.pack(cu, par, tok, sc, budget)
    r = sv.pack(cu, par, tok, torch.from_numpy(np.ascontiguousarray(sc, np.float32)).cuda(), budget=budget)
    torch.cuda.synchronize()
    N = int(r["total_nodes"].item())
    assert N == ref["total_nodes"]
    assert int(r["status"].item()) == ref["status"]
    assert np.array_equal(r["cu_nodes"].cpu().numpy(), ref["cu_nodes"])
    for k in ("parent", "draft_tokens", "src"):
        assert np.array_equal(r[k][:N].cpu().numpy(), ref[k]), k
    return ref


@pytest.mark.parametrize("case", ["monotone", "free", "ties", "c5_shape", "max_batch", "edges"])
def test_pack_matches_oracle(case):
    rng = np.random.default_rng({"monotone": 1, "free": 2, "ties": 3, "c5_shape": 4, "max_batch": 5,
                                 "edges": 6}[case] + 1100)
    print(f"[pack] {case}", flush=True)
    if case == "c5_shape":  # 256 requests, 64 candidates each, cap 2048
        cu, par, tok, sc = _batch(rng, [64] * 256)
        for K in (2048, 1, 16383, 16384, 20000):
            _check(cu, par, tok, sc, K)
        return
    if case == "max_batch":
        cu, par, tok, sc = _batch(rng, [int(x) for x in rng.integers(0, 9, 8192)], monotone=False, quant=2)
        for K in (0, 5000, int(cu[-1])):
            _check(cu, par, tok, sc, K)
        return
    if case == "edges":
        cu, par, tok, sc = _batch(rng, [5, 0, 7, 64, 1])
        sc = sc.copy()
        sc[[2, 9]] = np.nan
        sc[[3, 4]] = [-0.0, 0.0]
        for K in (0, 1, 3, 50, 1000):
            _check(cu, par, tok, sc, K)
        bad = par.copy()
        bad[7] = 5  # request 2: parent not before the node
        assert _check(cu, bad, tok, sc, 40)["status"] & 0x01
        big = np.concatenate([[0], np.cumsum([3, 65, 2])]).astype(np.int32)  # 65 candidates
        p = np.concatenate([np.full(3, -1), np.full(65, -1), np.full(2, -1)]).astype(np.int32)
        t = np.arange(70, dtype=np.int32)
        assert _check(big, p, t, rng.standard_normal(70).astype(np.float32), 10)["status"] & 0x02
        back = np.array([0, 5, 3, 8], np.int32)  # offsets going backwards
        assert _check(back, np.full(8, -1, np.int32), t[:8], np.zeros(8, np.float32), 4)["status"] & 0x02
        return
    for _ in range(20):
        sizes = [int(x) for x in rng.integers(0, 65, size=int(rng.integers(1, 60)))]
        cu, par, tok, sc = _batch(rng, sizes, monotone=case == "monotone", quant=2 if case == "ties" else None)
        M = int(cu[-1])
        _check(cu, par, tok, sc, int(rng.integers(0, M + 3)))


def test_packed_batch_verifies():
    """Candidates packed under a cap, their rows gathered by src, then the
    sampled walk on the packed layout: the GPU walk matches the oracle's on
    the oracle's packing (which the GPU packing equals)."""
    rng = np.random.default_rng(1151)
    V, sizes = 3000, [int(x) for x in rng.integers(1, 40, 24)]
    cu, par, tok, sc = _batch(rng, sizes)
    M = int(cu[-1])
    lg, q = rows_from_probs(rng, V, M + len(sizes), sharp=2.0, draft_noise=0.8)
    # candidate rows: request b's root row, then one per candidate (as the packed layout)
    cand_row = np.array([cu[b] + b + 1 + j for b in range(len(sizes)) for j in range(sizes[b])], np.int64)
    root_row = np.array([cu[b] + b for b in range(len(sizes))], np.int64)
    r = sv.pack(cu, par, tok, torch.from_numpy(sc).cuda(), budget=M // 2)
    torch.cuda.synchronize()
    N = int(r["total_nodes"].item())
    pcu = r["cu_nodes"].cpu().numpy()
    src = r["src"][:N].cpu().numpy()
    rows = []
    for b in range(len(sizes)):
        rows.append(root_row[b])
        rows.extend(cand_row[src[pcu[b]:pcu[b + 1]]].tolist())
    rows = np.array(rows, np.int64)
    logits, qq = lg[rows], q[rows]
    ptok = r["draft_tokens"][:N].contiguous()
    s = sv.sample(r["cu_nodes"], r["parent"][:N].contiguous(), ptok, torch.from_numpy(logits).cuda(),
                  torch.from_numpy(qq).cuda(), temperature=1.0, seed=99, max_nodes=64)
    torch.cuda.synchronize()
    ref = oracle.verify(pcu, r["parent"][:N].cpu().numpy(), ptok.cpu().numpy(), logits, qq, temperature=1.0,
                        seed=99, max_depth=64)
    compare_walk(s, ref, len(sizes), greedy=False)
