"""Seeded input generators (trees, caches, queries, logits, draft distributions).

Recipe (also listed in the design notes):
  * tree structure on the host with numpy.random.default_rng(cfg.seed):
      chain      parent = [-1, 0, 1, ..., K-2] per request;
      eagle60    the 60-node reduction of the 4-3-2-2-1-1 EAGLE-style tree (eagle_tree);
      super      per-request sizes start at 1; the remaining nodes go one at a time to a
                 uniformly chosen request still below max_T; node i of a request gets a
                 parent drawn uniformly from {-1, 0, ..., i-1}.
  * tensors with a torch.Generator seeded with cfg.seed on the target device:
      q, k, v ~ N(0, 1) in fp32, rounded to bf16 (round-to-nearest-even) for bf16 configs;
      target logits ~ N(0, logit_sigma^2) in fp32, rows [N+B, V];
      draft logits = target + N(0, draft_sigma^2); q = softmax(draft / temperature)
        computed in fp64 and stored as fp32 (the drafter's own distribution);
      draft token of node j ~ Categorical(q at its parent's row) (torch.multinomial),
        siblings being independent draws; or, with candidates="topk", the r-th most
        likely token of q at its parent's row, r being j's rank among its siblings
        in node order (deterministic candidates, as an EAGLE-style drafter's top-k).
  * every request has ctx_len = L; the cache holds Lcap = L + max(T_b) slots per head.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import WorkloadConfig


def chain_tree(K: int) -> np.ndarray:
    return np.arange(-1, K - 1, dtype=np.int32)


def eagle_tree(branching=(4, 3, 2, 2, 1, 1), total: int = 60) -> np.ndarray:
    """Static EAGLE-style tree of `total` nodes cut from the full tree with the
    given per-level branching: every node of the full tree gets the score
    sum of its sibling ranks along its path (rank 0 = first child); the
    `total` lowest scores are kept, ties broken by (depth, BFS index), and the
    kept nodes are numbered in (depth, BFS) order, so parents precede children.
    """
    nodes = []  # (depth, bfs index, score, parent bfs index)
    frontier = [(-1, 0)]
    for depth, width in enumerate(branching, start=1):
        nxt = []
        for pidx, pscore in frontier:
            for rank in range(width):
                idx = len(nodes)
                nodes.append((depth, idx, pscore + rank, pidx))
                nxt.append((idx, pscore + rank))
        frontier = nxt
    keep = sorted(nodes, key=lambda n: (n[2], n[0], n[1]))[:total]
    keep.sort(key=lambda n: (n[0], n[1]))
    local = {n[1]: i for i, n in enumerate(keep)}
    parent = np.array([-1 if n[3] < 0 else local[n[3]] for n in keep], dtype=np.int32)
    return parent


def super_tree_sizes(B: int, total: int, max_T: int, rng: np.random.Generator) -> np.ndarray:
    if total < B or total > B * max_T:
        raise ValueError("total nodes must lie in [B, B*max_T]")
    sizes = np.ones(B, dtype=np.int64)
    for _ in range(total - B):
        open_ = np.flatnonzero(sizes < max_T)
        sizes[open_[rng.integers(0, open_.size)]] += 1
    return sizes


def super_tree_parents(T: int, rng: np.random.Generator) -> np.ndarray:
    return np.array([rng.integers(-1, i) if i > 0 else -1 for i in range(T)], dtype=np.int32)


def _tree(cfg: WorkloadConfig, rng: np.random.Generator):
    if cfg.tree == "chain":
        per = [chain_tree(cfg.K) for _ in range(cfg.B)]
    elif cfg.tree == "eagle60":
        t = eagle_tree(total=cfg.K)
        per = [t.copy() for _ in range(cfg.B)]
    elif cfg.tree == "super":
        sizes = super_tree_sizes(cfg.B, cfg.K, cfg.max_T, rng)
        per = [super_tree_parents(int(s), rng) for s in sizes]
    else:
        raise ValueError(cfg.tree)
    sizes = np.array([p.size for p in per], dtype=np.int64)
    cu = np.zeros(cfg.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(sizes)
    parent = np.concatenate(per).astype(np.int32) if per else np.zeros(0, np.int32)
    return cu, parent, sizes


def _randn(shape, g, device, chunk_dim0=None):
    if chunk_dim0 is None or shape[0] <= chunk_dim0:
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    out = torch.empty(shape, device=device, dtype=torch.float32)
    for s in range(0, shape[0], chunk_dim0):
        e = min(shape[0], s + chunk_dim0)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
    return out


def _as_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def poison_unused_slots(k_cache: torch.Tensor, v_cache: torch.Tensor, ctx_len, cu_nodes) -> None:
    """Fill cache slots no node may read (beyond ctx_len[b] + T_b) with NaN."""
    ctx = np.asarray(ctx_len)
    cu = np.asarray(cu_nodes)
    for b in range(ctx.size):
        used = int(ctx[b]) + int(cu[b + 1] - cu[b])
        k_cache[b, :, used:, :] = float("nan")
        v_cache[b, :, used:, :] = float("nan")


def sibling_ranks(cu: np.ndarray, parent: np.ndarray) -> np.ndarray:
    """Rank of every packed node among the children of its parent (node order)."""
    rank = np.zeros(parent.size, np.int64)
    for b in range(cu.size - 1):
        seen = {}
        for j in range(int(cu[b + 1] - cu[b])):
            pj = int(parent[cu[b] + j])
            rank[cu[b] + j] = seen.get(pj, 0)
            seen[pj] = rank[cu[b] + j] + 1
    return rank


def generate(cfg: WorkloadConfig, device="cpu", *, attn: bool = True, sample: bool = True,
             poison: bool = False, row_chunk: int = 128, candidates: str = "sampled") -> dict:
    """Seeded inputs of one verification step for `cfg` on `device`.

    Returns a dict with host-side structure (numpy: cu_nodes, parent, ctx_len,
    sizes) and device tensors (cu_nodes_t, parent_t, ctx_len_t, q, k_cache,
    v_cache, logits, draft_probs, draft_tokens).
    """
    device = torch.device(device)
    rng = np.random.default_rng(cfg.seed)
    cu, parent, sizes = _tree(cfg, rng)
    B, N = cfg.B, int(cu[-1])
    max_T = int(sizes.max()) if B > 0 else 0
    Lcap = cfg.L + max_T
    ctx_len = np.full(B, cfg.L, dtype=np.int32)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    out = {
        "cfg": cfg, "B": B, "N": N, "V": cfg.V, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D, "dtype": cfg.dtype,
        "Lcap": Lcap, "max_T": max_T, "temperature": cfg.temperature, "seed": cfg.lib_seed, "step": 0,
        "cu_nodes": cu, "parent": parent, "ctx_len": ctx_len, "sizes": sizes,
        "cu_nodes_t": torch.from_numpy(cu).to(device), "parent_t": torch.from_numpy(parent).to(device),
        "ctx_len_t": torch.from_numpy(ctx_len).to(device),
    }
    if attn:
        out["q"] = _as_dtype(_randn((N, cfg.Hq, cfg.D), g, device), cfg.dtype).contiguous()
        kv_chunk = max(1, (1 << 28) // max(1, cfg.Hkv * Lcap * cfg.D * 4))
        out["k_cache"] = _as_dtype(_randn((B, cfg.Hkv, Lcap, cfg.D), g, device, kv_chunk), cfg.dtype).contiguous()
        out["v_cache"] = _as_dtype(_randn((B, cfg.Hkv, Lcap, cfg.D), g, device, kv_chunk), cfg.dtype).contiguous()
        if poison:
            poison_unused_slots(out["k_cache"], out["v_cache"], ctx_len, cu)
    if sample:
        R = N + B
        logits = torch.empty((R, cfg.V), device=device, dtype=torch.float32)
        probs = torch.empty((R, cfg.V), device=device, dtype=torch.float32)
        T = cfg.temperature if cfg.temperature > 0 else 1.0
        for s in range(0, R, row_chunk):
            e = min(R, s + row_chunk)
            tl = torch.randn((e - s, cfg.V), generator=g, device=device, dtype=torch.float32) * cfg.logit_sigma
            dl = tl.double() + torch.randn((e - s, cfg.V), generator=g, device=device,
                                           dtype=torch.float32).double() * cfg.draft_sigma
            logits[s:e] = tl
            probs[s:e] = torch.softmax(dl / T, dim=-1).float()
            del tl, dl
        # draft token of node j ~ q at its parent's row
        req = np.repeat(np.arange(B), sizes)
        prow = (cu[:-1][req] + req + parent + 1).astype(np.int64) if N > 0 else np.zeros(0, np.int64)
        prow_t = torch.from_numpy(prow).to(device)
        toks = torch.empty(N, device=device, dtype=torch.int64)
        if candidates == "topk":
            rank_t = torch.from_numpy(sibling_ranks(cu, parent)).to(device)
            k = min(cfg.V, int(rank_t.max().item()) + 1) if N > 0 else 1
            for s in range(0, N, row_chunk):
                e = min(N, s + row_chunk)
                top = torch.topk(probs[prow_t[s:e]], k, dim=1).indices
                toks[s:e] = top.gather(1, rank_t[s:e].clamp(max=k - 1).unsqueeze(1)).squeeze(1)
        else:
            for s in range(0, N, row_chunk):
                e = min(N, s + row_chunk)
                toks[s:e] = torch.multinomial(probs[prow_t[s:e]], 1, generator=g).squeeze(1)
        out["logits"] = logits
        out["draft_probs"] = probs
        out["draft_tokens"] = toks.to(torch.int32)
    return out


def to_paged(k_cache, v_cache, block_size: int, rng: np.random.Generator, spare_blocks: int = 3,
             share_prefix_blocks: int = 0):
    """Lay contiguous caches [B, Hkv, Lcap, D] out as paged pools.

    Each request's Lcap slots are cut into Lcap / block_size blocks that land
    in a shuffled pool of B * max_blocks + spare_blocks blocks; the spare
    blocks are filled with NaN, so that a read through a wrong block id shows.
    share_prefix_blocks > 0 makes every request's first blocks the same pool
    blocks as request 0's (a shared prompt prefix): request b's data in those
    slots is then request 0's. Works on numpy arrays and torch tensors.
    Returns (k_pool, v_pool, block_table int32 [B, max_blocks]).
    """
    B, Hkv, Lcap, D = k_cache.shape
    assert Lcap % block_size == 0
    mb = Lcap // block_size
    nblk = B * mb + spare_blocks
    perm = rng.permutation(nblk)[: B * mb].reshape(B, mb).astype(np.int32)
    if share_prefix_blocks:
        perm[1:, :share_prefix_blocks] = perm[0, :share_prefix_blocks]
    is_torch = isinstance(k_cache, torch.Tensor)

    def pool_of(x):
        if is_torch:
            fill = 0x7F if x.dtype == torch.uint8 else float("nan")  # 0x7F: the fp8 E4M3 NaN
            pool = torch.full((nblk, Hkv, block_size, D), fill, dtype=x.dtype, device=x.device)
            blocks = x.reshape(B, Hkv, mb, block_size, D).permute(0, 2, 1, 3, 4)
            for b in range(B):
                pool[torch.as_tensor(perm[b], device=x.device).long()] = blocks[b]
            if share_prefix_blocks:
                pool[torch.as_tensor(perm[0, :share_prefix_blocks], device=x.device).long()] = \
                    blocks[0, :share_prefix_blocks]
            return pool
        fill = np.uint16(0x7FC0) if x.dtype == np.uint16 else (np.uint8(0x7F) if x.dtype == np.uint8 else np.nan)
        pool = np.full((nblk, Hkv, block_size, D), fill, dtype=x.dtype)
        blocks = x.reshape(B, Hkv, mb, block_size, D).transpose(0, 2, 1, 3, 4)
        for b in range(B):
            pool[perm[b]] = blocks[b]
        if share_prefix_blocks:
            pool[perm[0, :share_prefix_blocks]] = blocks[0, :share_prefix_blocks]
        return pool

    return pool_of(k_cache), pool_of(v_cache), perm


def to_fp8_e4m3(x, scale: float):
    """x / scale rounded to OCP FP8 E4M3 (finite form) by torch, returned as
    uint8 bytes (a caller's fp8 cache holds these; value = byte * scale)."""
    t = torch.as_tensor(x).float() / scale
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
