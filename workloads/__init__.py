"""Seeded synthetic inputs for the verification step.

This package only draws inputs (trees, KV caches, queries, target logits,
draft distributions and draft tokens). It holds none of the verification
arithmetic and is the one piece of code shared by the GPU library's tests and
bench on one side and the oracle on the other.
"""
from .configs import CONFIGS, C4_BUCKETS, WorkloadConfig, get_config, scaled
from .gen import (chain_tree, eagle_tree, generate, super_tree_sizes, super_tree_parents, poison_unused_slots,
                  to_fp8_e4m3, to_paged)

__all__ = ["CONFIGS", "C4_BUCKETS", "WorkloadConfig", "get_config", "scaled", "chain_tree", "eagle_tree",
           "generate", "super_tree_sizes", "super_tree_parents", "poison_unused_slots"]
