"""One spec_verify_step call with the optional layouts and rules together:
paged fp8 caches for the attention, truncation-based verification over the
eta set for the sampler; each half against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_16_amd as sv
from gpu_helpers import ATTN_TOL, compare_walk, host_bits
from workloads import CONFIGS, generate, scaled, to_fp8_e4m3, to_paged

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c3_small", "c5_small"])
def test_step_paged_fp8_truncation(name):
    cfg = {"c3_small": scaled(CONFIGS["c3_eagle_tree"], B=3, L=300, V=9000),
           "c5_small": scaled(CONFIGS["c5_super_tree"], B=12, K=100, L=250, V=7001)}[name]
    w = generate(cfg, "cuda")
    print(f"[step-compose] {name} B={w['B']} N={w['N']} V={cfg.V}", flush=True)
    k, v = w["k_cache"], w["v_cache"]
    B, Hkv, Lcap, D = k.shape
    Lp = (Lcap + 127) // 128 * 128
    pad = torch.zeros((B, Hkv, Lp - Lcap, D), dtype=k.dtype, device="cuda")
    k8 = to_fp8_e4m3(torch.cat([k, pad], 2), 1 / 64).contiguous()
    v8 = to_fp8_e4m3(torch.cat([v, pad], 2), 1 / 64).contiguous()
    kp, vp, bt = to_paged(k8, v8, 128, np.random.default_rng(1401))
    a = sv.AttnCall(w["q"], kp.contiguous(), vp.contiguous(), w["ctx_len_t"], w["cu_nodes_t"], parent=w["parent_t"],
                    max_nodes=w["max_T"], block_table=torch.from_numpy(bt).cuda(), kv_fp8_scales=(1 / 64, 1 / 64))
    s = sv.SampleCall(a.keep["cu"], w["parent_t"], w["draft_tokens"], w["logits"], w["draft_probs"],
                      temperature=cfg.temperature, seed=w["seed"], max_nodes=w["max_T"], rule="truncation",
                      eta=(0.05, 0.3), residual_passes=True)
    r = sv.StepCall(a, s)()
    torch.cuda.synchronize()
    assert int(r["status"].item()) == 0 and int(a.status.item()) == 0
    ref = oracle.attention(host_bits(w["q"]), kp.cpu().numpy(), vp.cpu().numpy(), w["ctx_len"], w["cu_nodes"],
                           w["parent"], Hq=w["Hq"], Hkv=w["Hkv"], dtype="bf16", block_table=bt,
                           kv_fp8_scales=(1 / 64, 1 / 64))
    assert float(np.abs(r["attn_out"].cpu().numpy() - ref).max()) <= ATTN_TOL["bf16"]
    o = oracle.verify(w["cu_nodes"], w["parent"], w["draft_tokens"].cpu().numpy(), w["logits"].cpu().numpy(),
                      w["draft_probs"].cpu().numpy(), temperature=cfg.temperature, seed=w["seed"],
                      max_depth=r["accepted_nodes"].shape[1], rule="truncation", eta=(0.05, 0.3))
    compare_walk(r, o, w["B"], greedy=False)
