"""Helpers of the GPU parity tests: run the HIP library through the binding and
the oracle on host copies of the same input bytes, then compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle

ATTN_TOL = {"bf16": 1e-2, "f32": 1e-5}
PROB_TOL = 1e-5


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def oracle_attention(w, items=None, block_table=None):
    return oracle.attention(host_bits(w["q"]), host_bits(w["k_cache"]), host_bits(w["v_cache"]), w["ctx_len"],
                            w["cu_nodes"], w["parent"], Hq=w["Hq"], Hkv=w["Hkv"], dtype=w["dtype"], items=items,
                            block_table=block_table)


def sample_items(w, n, seed=0):
    rng = np.random.default_rng(seed)
    N, Hq = w["N"], w["Hq"]
    nodes = rng.integers(0, N, size=n)
    heads = rng.integers(0, Hq, size=n)
    # always include the last node of the last request and node 0 (ragged ends)
    nodes[0], heads[0] = N - 1, Hq - 1
    nodes[1], heads[1] = 0, 0
    return np.stack([nodes, heads], axis=1).astype(np.int64)


def compare_walk(gpu: dict, ref: dict, B: int, greedy: bool):
    """Bit-exact comparison, except after a decision the oracle flags as a
    near-tie (sampled mode only): there only the accepted prefix decided before
    it must agree. Returns the number of flagged requests."""
    acc = gpu["accept_len"].cpu().numpy()
    nodes = gpu["accepted_nodes"].cpu().numpy()
    toks = gpu["out_tokens"].cpu().numpy()
    flagged = 0
    for b in range(B):
        fd = int(ref["flag_depth"][b]) if not greedy else -1
        if fd >= 0:
            flagged += 1
            assert (nodes[b, :fd] == ref["accepted_nodes"][b, :fd]).all(), b
            if ref["flag_kind"][b] == 1:
                assert acc[b] == ref["accept_len"][b], b
            continue
        assert acc[b] == ref["accept_len"][b], (b, acc[b], ref["accept_len"][b])
        assert (nodes[b] == ref["accepted_nodes"][b]).all(), (b, nodes[b], ref["accepted_nodes"][b])
        assert (toks[b] == ref["out_tokens"][b]).all(), (b, toks[b], ref["out_tokens"][b])
    return flagged
