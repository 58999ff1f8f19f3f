"""spec_verify_step_noalloc (library-owned scratch, no allocation) against
spec_verify_step with a caller workspace: bitwise the same outputs, on two
calls in a row, the second with a smaller batch, and an oversize request
rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import speculative_decoding_verification_16_amd as sv
from workloads import CONFIGS, generate, scaled

pytestmark = pytest.mark.gpu

KEYS = ("attn_out", "accept_len", "accepted_nodes", "out_tokens", "residual_passes")


def _calls(cfg):
    w = generate(cfg, "cuda")
    a = sv.AttnCall(w["q"], w["k_cache"], w["v_cache"], w["ctx_len_t"], w["cu_nodes_t"], parent=w["parent_t"],
                    max_nodes=w["max_T"])
    s = sv.SampleCall(a.keep["cu"], w["parent_t"], w["draft_tokens"], w["logits"], w["draft_probs"],
                      temperature=cfg.temperature, seed=w["seed"], max_nodes=w["max_T"], residual_passes=True)
    return sv.StepCall(a, s)


def _snapshot(r):
    return {k: r[k].clone() for k in KEYS}


def test_noalloc_matches_step_twice_then_smaller():
    big = scaled(CONFIGS["c3_eagle_tree"], B=6, L=1500, V=20000)       # sliced walk, split-K attention
    # 366 rows of 128256 logits (188 MB): the sliced walk reduces the rows it
    # reaches, its coordination words zeroed by the attention launch
    lazy = scaled(CONFIGS["c3_eagle_tree"], B=6, L=1500)
    small = scaled(CONFIGS["c5_super_tree"], B=10, K=70, L=300, V=9000)  # wide trees, other layout
    for cfg in (big, lazy, small):
        step = _calls(cfg)
        print(f"[noalloc] {cfg.name} B={cfg.B} ws={step.ws_bytes}", flush=True)
        ref = _snapshot(step())
        torch.cuda.synchronize()
        for _ in range(2):
            # poison the outputs so that a stale result cannot pass
            step.attn.out.fill_(float("nan"))
            step.sample.accept_len.fill_(-7)
            step.sample.out_tokens.fill_(-7)
            r = step.noalloc()
            torch.cuda.synchronize()
            assert int(step.sample.status.item()) == 0 and int(step.attn.status.item()) == 0
            for k in KEYS:
                assert torch.equal(r[k], ref[k]), (cfg.name, k)


def test_noalloc_rejects_oversize_arguments():
    lib = sv.load_library()
    fake = ctypes.c_void_p(0x100000)
    a = sv.SvAttnArgs()
    a.B, a.total_nodes, a.max_nodes, a.Hq, a.Hkv, a.D, a.dtype = 64, 64 * 64, 64, 64, 2, 128, sv.SV_BF16
    a.Lcap = 1 << 20
    a.num_splits = 256
    a.q = a.k_cache = a.v_cache = a.out = a.ctx_len = a.cu_nodes = a.parent = fake
    s = sv.SvSampleArgs()
    s.B, s.V, s.total_nodes, s.max_nodes, s.temperature, s.max_depth = 64, 1000, 64 * 64, 64, 1.0, 64
    s.cu_nodes = s.parent = s.draft_tokens = s.target_logits = s.draft_probs = fake
    s.accept_len = s.accepted_nodes = s.out_tokens = fake
    need = lib.spec_verify_workspace_size(ctypes.byref(a), ctypes.byref(s))
    assert need > (64 << 20)
    rc = lib.spec_verify_step_noalloc(ctypes.byref(a), ctypes.byref(s), None)
    assert rc == sv.SV_ERR_UNSUPPORTED and b"64 MiB" in lib.spec_verify_last_error()
