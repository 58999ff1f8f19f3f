"""spec_verify_step captured in a HIP graph: every replay, with the program's
own eager work and synchronizations between replays, gives the eager result
bit for bit (the library launches kernels only: no allocation, copy, memset
or synchronization inside a call). Under SV_OVERLAP_ON the capture forks
into the library's second stream and joins back, and the replays match the
eager in-order schedule."""
import pytest
import torch

import speculative_decoding_verification_16_amd as sv
from workloads import CONFIGS, generate, scaled

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("overlap", ["off", "on"])
@pytest.mark.parametrize("name", ["c2_small", "c3_small", "c5_small", "c3_reached_rows"])
def test_step_graph_replays_match_eager(name, overlap):
    # (c3_reached_rows: 366 rows of 128256 logits, over 128 MiB, so the
    # sliced walk reduces the rows it reaches; in order, the attention launch
    # zeroes the slices' coordination words)
    cfg = {"c2_small": scaled(CONFIGS["c2_llama8b_chain"], B=4, L=700, V=5000),
           "c3_small": scaled(CONFIGS["c3_eagle_tree"], B=3, L=300, V=9000),
           "c5_small": scaled(CONFIGS["c5_super_tree"], B=12, K=100, L=250, V=7001),
           "c3_reached_rows": scaled(CONFIGS["c3_eagle_tree"], B=6, L=1500)}[name]
    w = generate(cfg, "cuda")
    print(f"[graph] {name} overlap={overlap} B={w['B']} N={w['N']}", flush=True)
    a = sv.AttnCall(w["q"], w["k_cache"], w["v_cache"], w["ctx_len_t"], w["cu_nodes_t"], parent=w["parent_t"],
                    max_nodes=w["max_T"])
    s = sv.SampleCall(a.keep["cu"], w["parent_t"], w["draft_tokens"], w["logits"], w["draft_probs"],
                      temperature=cfg.temperature, seed=w["seed"], max_nodes=w["max_T"], residual_passes=True)
    step = sv.StepCall(a, s)
    stream = torch.cuda.Stream()
    # the inputs were generated, and the calls' outputs and workspaces
    # allocated, in the default stream's order; the allocator may have handed
    # out blocks whose earlier default-stream users have not run yet
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        r = step(stream)
    stream.synchronize()
    keys = ("attn_out", "accept_len", "accepted_nodes", "out_tokens", "residual_passes")
    eager = {k: r[k].clone() for k in keys}
    s.args.step_overlap = sv.OVERLAP_MODES[overlap]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(stream)
    for rep in range(4):
        for k in keys:  # clobber the outputs so that each replay must rewrite them
            r[k].fill_(-7)
        torch.cuda.synchronize()
        _ = (w["logits"][:4].sum() + rep).item()  # eager work between replays
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        for k in keys:
            assert torch.equal(r[k], eager[k]), (rep, k)
    assert int(s.status.item()) == 0
