"""Throughput of one speculative-decoding verification step on one MI355X.

A step is one spec_verify_step call over one batch: tree preprocessing,
tree-masked GQA attention of every draft node against its request's KV cache
(one layer), the row-statistics pass over every target-logit row, and the
rejection-sampling tree walk that emits the accepted path plus a bonus token.
All inputs are synthetic, seeded, and resident in HBM before the timed region.
Workloads smaller than 512 MB are held in several copies that consecutive
steps cycle through, so that no step finds its inputs in the last-level cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line: verified draft tokens/s (sum of T_b over the batch per
second) with the mean and the 10th / 50th / 90th percentile step time, the
roofline position of the dominant kernel (algorithmic bytes over its
HIP-event-timed duration, against the 8 TB/s HBM3E peak, with a measured
device-to-device copy rate beside it), per-kernel times, and the fp64 CPU
oracle timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
ROTATE_BYTES = 512 << 20  # inputs cycled per step: at least twice the 256 MB last-level cache
MAX_INPUT_SETS = 8
DEFAULT_WORKLOAD = "c5_super_tree"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "attn_mfma_kernel": "speculative_decoding_verification_16_amd/csrc/sv_attn.hip",
    "attn_mfma32_kernel": "speculative_decoding_verification_16_amd/csrc/sv_attn.hip",
    "row_stats_kernel": "speculative_decoding_verification_16_amd/csrc/sv_sample.hip",
    "walk_kernel": "speculative_decoding_verification_16_amd/csrc/sv_sample.hip",
}


def attention_kernel_name(w, cfg, kv_fp8: bool = False) -> str:
    """Which attention kernel the library's plan launches: fp32 caches take the
    VALU kernel; bf16 queries (over bf16 or fp8 caches) take 16x16 MFMA tiles
    when a KV head carries at most 64 query rows (Hq/Hkv heads x max_T nodes),
    else 32x32 tiles."""
    if w["dtype"] != "bf16":
        return "attn_valu_kernel"
    return "attn_mfma_kernel" if (cfg.Hq // cfg.Hkv) * w["max_T"] <= 64 else "attn_mfma32_kernel"


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence: timing kept, no system-scope fence


class HipEvents:
    """Timing events created and read through the HIP runtime torch has loaded
    (the library records them on its own stream, outside torch's bookkeeping).
    They are created without the system-scope fence a default event performs
    on each record: the timed steps then carry no cache flush per event (the
    timestamps are device-side and need no host visibility of memory)."""

    def __init__(self, n: int):
        import ctypes

        import torch  # noqa: F401  (loads the runtime that libamdhip64.so.7 resolves to)

        self._ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev.append(h.value)

    def record(self, i: int, stream) -> None:
        rc = self.hip.hipEventRecord(self.ev[i], self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a: int, b: int) -> float:
        out = self._ct.c_float()
        rc = self.hip.hipEventElapsedTime(self._ct.byref(out), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)
        self.ev = []


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle's CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-events", action="store_true", help="time without the per-kernel HIP events")
    ap.add_argument("--min-p", type=float, default=0.0,
                    help="verify against the min-p truncated target (0 = plain lossless verification)")
    ap.add_argument("--eta", type=float, nargs=2, default=None, metavar=("EPS", "DELTA"),
                    help="verify against the eta truncated target {p >= min(EPS, DELTA exp(-H))} instead")
    ap.add_argument("--rule", choices=["lossless", "lenience", "interpolation", "truncation"], default="lossless",
                    help="accept test (lenience and interpolation are lossy, [LOSSY] 3.1; truncation accepts "
                         "any allowed token, [LOSSY] 3.2, and needs --min-p or --eta)")
    ap.add_argument("--rule-param", type=float, default=1.0, help="l or lambda of --rule, in (0, 1]")
    ap.add_argument("--siblings", choices=["sampled", "deterministic"], default="sampled",
                    help="sampled: draft tokens are draws from q; deterministic: the top-k of q as fixed "
                         "candidates, verified by the deterministic-candidate rule (q is not read)")
    ap.add_argument("--walk-mode", choices=["auto", "single", "sliced"], default="auto",
                    help="tree-walk layout (auto picks from the batch size and vocabulary)")
    ap.add_argument("--overlap", choices=["off", "on"], default="off",
                    help="step schedule timed: off = attention, row statistics and walk in order on one stream "
                         "(the library's default); on = the sampler on the bench stream while the attention runs "
                         "concurrently on a second stream (SV_OVERLAP_ON). The other schedule is timed after the "
                         "timed region and reported beside it.")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="lay the KV caches out as a shuffled pool of BLOCK-slot blocks read through a block "
                         "table (BLOCK a multiple of 64; 0 = contiguous caches)")
    ap.add_argument("--graph", action="store_true",
                    help="capture each input set's step in a HIP graph once and time graph replays (launch-bound "
                         "small workloads); per-kernel events and the roofline object are then not recorded")
    ap.add_argument("--hash-inputs", action="store_true",
                    help="record the SHA-256 (first 16 hex digits) of every input buffer of the first input set "
                         "in the JSON line (always done for workloads under 512 MB; copies them to the host: "
                         "seconds for the large workloads)")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="quantise the KV caches to OCP FP8 E4M3 bytes with per-tensor scales (bf16 workloads)")
    ap.add_argument("--input-sets", type=int, default=0, metavar="N",
                    help="cycle through N copies of the inputs (0 = as many as keep the per-step working set "
                         "at 512 MB or more, up to 8)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES three times (calibrates the HBM "
                         "byte counters of rocprofv3 against a kernel of known traffic) and exit")
    return ap.parse_args()


def copy_probe(nbytes: int):
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 3
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "copy_GB_s": round(2 * n * 4 / dt / 1e9, 1)}), flush=True)


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Measured device-to-device copy rate (bytes read + written per second,
    GB/s) of a plain torch copy: the practical HBM ceiling reported beside
    the vendor peak."""
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / sec / 1e9


def source_digest(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    kernel and workload, or None when there is none or the kernel's source has
    changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_bytes:
        return None
    if m_src.group(1) != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return float(m_bytes.group(1))


def attention_bytes(w, kv_elem: int = 0) -> float:
    """Algorithmic bytes of one attention launch: every K and V slot a node can
    see (context + draft slots) once, the queries once, the fp32 outputs once.
    kv_elem: bytes per cache element (0: the query element size; 1: fp8)."""
    e = 2 if w["dtype"] == "bf16" else 4
    ekv = kv_elem or e
    kv = 0
    for b in range(w["B"]):
        T = int(w["cu_nodes"][b + 1] - w["cu_nodes"][b])
        if T > 0:
            kv += w["Hkv"] * (int(w["ctx_len"][b]) + T) * w["D"] * 2 * ekv
    return float(kv + w["N"] * w["Hq"] * w["D"] * (e + 4))


def attention_flops(w) -> float:
    """4 D flops per (query row, visible key): QK^T and PV."""
    tot = 0
    for b in range(w["B"]):
        n0, n1 = int(w["cu_nodes"][b]), int(w["cu_nodes"][b + 1])
        par = w["parent"][n0:n1]
        depth = [0] * (n1 - n0)
        for j in range(n1 - n0):
            depth[j] = 1 + (depth[par[j]] if par[j] >= 0 else 0)
        tot += sum(int(w["ctx_len"][b]) + d for d in depth)
    return float(4 * w["D"] * w["Hq"] * tot)


def row_stats_bytes(w) -> float:
    """Algorithmic bytes of the row-statistics pass: each target-logit row once
    (fp32) plus its 16-byte per-chunk statistics."""
    rows = w["N"] + w["B"]
    nch = (w["V"] + 4095) // 4096
    return float(rows * w["V"] * 4 + rows * nch * 16)


def cpu_baseline(w, budget_s: float, min_p: float = 0.0, siblings: str = "sampled", rule: str = "lossless",
                 rule_param: float = 1.0, eta=None):
    """The fp64 oracle (attention of every (node, head) of a request, then the
    verification walk) over whole requests in order until the budget is spent.
    Returns verified draft tokens/s of that sample, the thread count, a
    description, and the oracle's walk outputs per request of the sample."""
    import numpy as np

    import oracle

    def bits(t):
        import torch
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()

    try:
        threads = min(16, len(os.sched_getaffinity(0)))
    except AttributeError:
        threads = min(16, os.cpu_count() or 1)
    cu, par, ctx = w["cu_nodes"], w["parent"], w["ctx_len"]
    nodes_done, req_done, spent = 0, 0, 0.0
    chunk = 4
    ref = {}
    while req_done < w["B"] and spent < budget_s:
        b0, b1 = req_done, min(w["B"], req_done + chunk)
        n0, n1 = int(cu[b0]), int(cu[b1])
        r0, r1 = n0 + b0, n1 + b1
        sub_cu = (cu[b0:b1 + 1] - cu[b0]).astype(np.int32)
        q = bits(w["q"][n0:n1])
        k = bits(w["k_cache"][b0:b1])
        v = bits(w["v_cache"][b0:b1])
        lg = w["logits"][r0:r1].cpu().numpy()
        qq = w["draft_probs"][r0:r1].cpu().numpy()
        toks = w["draft_tokens"][n0:n1].cpu().numpy()
        t0 = time.perf_counter()
        oracle.attention(q, k, v, ctx[b0:b1], sub_cu, par[n0:n1], Hq=w["Hq"], Hkv=w["Hkv"], dtype=w["dtype"],
                         nthreads=threads)
        o = oracle.verify(sub_cu, par[n0:n1], toks, lg, qq, temperature=w["temperature"], seed=w["seed"],
                          request_id=np.arange(b0, b1, dtype=np.uint32), nthreads=threads, min_p=min_p,
                          siblings=siblings, rule=rule, rule_param=rule_param, eta=eta, max_depth=64)
        spent += time.perf_counter() - t0
        for i, b in enumerate(range(b0, b1)):
            ref[b] = {k: o[k][i] for k in ("accept_len", "accepted_nodes", "out_tokens", "flag_depth", "flag_kind",
                                           "draw_mass")}
        nodes_done += n1 - n0
        req_done = b1
    desc = (f"first {req_done} of {w['B']} requests ({nodes_done} draft nodes): fp64 attention of every "
            f"(node, query head) plus the verification walk, {spent:.1f} s")
    return nodes_done / spent, threads, desc, ref


def compare_sample(s, ref: dict) -> dict:
    """The GPU's walk outputs on the requests of the CPU-baseline sample against
    the oracle's: bit for bit, except after a decision the oracle flags as a
    near tie (only the path decided before it must agree). Returns the counts:
    checked, flagged by kind, flagged requests identical in full anyway,
    mismatched (must be 0), and the final-draw near ties expected from the
    1e-6 CDF tolerance (a draw of a token of mass m is one with probability
    min(1, 2e-6 / m))."""
    acc = s.accept_len.cpu().numpy()
    nodes = s.accepted_nodes.cpu().numpy()
    toks = s.out_tokens.cpu().numpy()
    md = nodes.shape[1]
    kinds = {0: "accept_test", 1: "final_draw", 2: "allowed_set_boundary", 3: "remainder"}
    out = {"checked": len(ref), "flagged": 0, "flagged_by_kind": {}, "flagged_identical": 0, "mismatched": 0,
           "final_draw_expected": 0.0}
    for b, o in ref.items():
        fd = int(o["flag_depth"])
        full = acc[b] == o["accept_len"] and (nodes[b] == o["accepted_nodes"][:md]).all() and \
            (toks[b] == o["out_tokens"][:md + 1]).all()
        m = float(o["draw_mass"])
        out["final_draw_expected"] += min(1.0, 2e-6 / m) if m > 0 else 0.0
        if fd >= 0:
            out["flagged"] += 1
            k = kinds.get(int(o["flag_kind"]), str(int(o["flag_kind"])))
            out["flagged_by_kind"][k] = out["flagged_by_kind"].get(k, 0) + 1
            out["flagged_identical"] += int(full)
            same = (nodes[b, :fd] == o["accepted_nodes"][:fd]).all() and (toks[b, :fd] == o["out_tokens"][:fd]).all()
        else:
            same = full
        out["mismatched"] += 0 if same else 1
    out["final_draw_expected"] = round(out["final_draw_expected"], 2)
    return out


def walk_metrics(w, s, K: int, elapsed: float, passes) -> dict:
    """Acceptance statistics of the first input set's batch: the mean accepted
    length, AL = mean emitted tokens per step ([SPEED] section 3.4: accepted
    drafts plus the token the target always adds), the conditional acceptance
    rate per depth AR_d (accepted at depth d among requests that reached
    depth d with at least one candidate there), ECHO's mean accepted tokens
    (MAT, the mean accepted length) and draft utilisation u = accepted length
    over the tree's depth ([ECHO] section 5.1, averaged over requests with a
    tree)."""
    import numpy as np

    acc = s.accept_len.cpu().numpy()
    nodes = s.accepted_nodes.cpu().numpy()
    cu, par = w["cu_nodes"], w["parent"]
    reached, accepted, util = {}, {}, []
    for b in range(w["B"]):
        p = par[cu[b]:cu[b + 1]]
        if p.size == 0:
            continue
        depth = np.zeros(p.size, np.int64)
        for j in range(p.size):
            depth[j] = 1 + (depth[p[j]] if p[j] >= 0 else 0)
        util.append(acc[b] / depth.max())
        pos = -1
        for d in range(p.size):
            if not (p == pos).any():
                break
            reached[d] = reached.get(d, 0) + 1
            if acc[b] > d:
                accepted[d] = accepted.get(d, 0) + 1
                pos = int(nodes[b, d])
            else:
                break
    ar = [round(accepted.get(d, 0) / reached[d], 4) for d in sorted(reached)]
    return {"mean_accept_len": round(float(acc.mean()), 4),
            "AL": round(float(acc.mean()) + 1.0, 4),
            "AR_per_depth": ar,
            "MAT": round(float(acc.mean()), 4),
            "draft_utilisation_u": round(float(np.mean(util)), 4) if util else None,
            "emitted_tokens_per_s": round(float((acc + 1).sum()) * K / elapsed, 1),
            "residual_passes_per_step": int(passes.sum().item()),
            "max_residual_passes_per_request": int(passes.max().item())}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the verification step shards by request "
              "with no inter-GPU traffic, so one GPU's share is what it measures.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch

    import speculative_decoding_verification_16_amd as sv
    from workloads import generate, get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sv.load_library()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    cfg = get_config(args.workload)
    det = args.siblings == "deterministic"
    cand = "topk" if det else "sampled"
    w = generate(cfg, dev, candidates=cand)
    # Small workloads would stay in the 256 MB last-level cache from one step
    # to the next: consecutive steps then cycle through copies of the inputs
    # in separate buffers, at least 512 MB together (at most 8 copies).
    set_bytes = attention_bytes(w) + 8 * w["V"] * (w["N"] + w["B"])
    n_sets = max(1, min(MAX_INPUT_SETS, math.ceil(ROTATE_BYTES / set_bytes)))
    if args.input_sets:
        n_sets = args.input_sets
    sets = [w] + [generate(cfg, dev, candidates=cand) for _ in range(n_sets - 1)]
    if args.kv_fp8:
        from workloads import to_fp8_e4m3
        for x in sets:
            ks = float(x["k_cache"].float().abs().amax()) / 448.0
            vs = float(x["v_cache"].float().abs().amax()) / 448.0
            x["k_cache"], x["v_cache"] = to_fp8_e4m3(x["k_cache"], ks), to_fp8_e4m3(x["v_cache"], vs)
            x["kv_scales"] = (ks, vs)
    if args.paged:
        import numpy as np

        from workloads import to_paged
        bs = args.paged
        for i, x in enumerate(sets):
            k, v = x["k_cache"], x["v_cache"]
            B_, H_, Lc, D_ = k.shape
            Lp = (Lc + bs - 1) // bs * bs
            if Lp != Lc:
                pad = torch.zeros((B_, H_, Lp - Lc, D_), dtype=k.dtype, device=dev)
                k, v = torch.cat([k, pad], dim=2), torch.cat([v, pad], dim=2)
            kp, vp, bt = to_paged(k, v, bs, np.random.default_rng(77 + i), spare_blocks=0)
            x["k_pool"], x["v_pool"], x["block_table"] = kp, vp, torch.from_numpy(bt).to(dev)
            del k, v
    torch.cuda.synchronize()
    input_sha = None
    if args.hash_inputs or set_bytes < ROTATE_BYTES:
        input_sha = {}
        for key in ("q", "k_cache", "v_cache", "ctx_len_t", "cu_nodes_t", "parent_t", "draft_tokens", "logits",
                    "draft_probs", "k_pool", "v_pool", "block_table"):
            t = w.get(key)
            if isinstance(t, torch.Tensor):
                h = hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()[:16]
                input_sha[key] = h

    stream = torch.cuda.Stream()  # default priority
    calls = []
    with torch.cuda.stream(stream):
        for x in sets:
            if args.paged:
                a = sv.AttnCall(x["q"], x["k_pool"], x["v_pool"], x["ctx_len_t"], x["cu_nodes_t"],
                                parent=x["parent_t"], max_nodes=x["max_T"], block_table=x["block_table"],
                                kv_fp8_scales=x.get("kv_scales"))
            else:
                a = sv.AttnCall(x["q"], x["k_cache"], x["v_cache"], x["ctx_len_t"], x["cu_nodes_t"],
                                parent=x["parent_t"], max_nodes=x["max_T"], kv_fp8_scales=x.get("kv_scales"))
            s = sv.SampleCall(a.keep["cu"], x["parent_t"], x["draft_tokens"], x["logits"],
                              None if det else x["draft_probs"], temperature=cfg.temperature, seed=x["seed"],
                              max_nodes=x["max_T"], residual_passes=True, min_p=args.min_p,
                              siblings=args.siblings, rule=args.rule, rule_param=args.rule_param,
                              eta=tuple(args.eta) if args.eta else None, walk_mode=args.walk_mode,
                              step_overlap=args.overlap)
            calls.append((a, s, sv.StepCall(a, s)))
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    use_events = not (args.no_events or args.graph)
    hev = HipEvents(5 * K) if use_events else None  # per step: attn start/stop, sampler start, stats stop, sampler stop

    for i in range(max(W, n_sets)):
        calls[i % n_sets][2](stream)
    stream.synchronize()
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        # the library launches kernels only (no allocation, copy, memset or
        # synchronization), so a step captures as is
        graphs = []
        for _, _, step in calls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(stream)
            graphs.append(g)
        with torch.cuda.stream(stream):
            for i in range(max(W, n_sets)):
                graphs[i % n_sets].replay()
        stream.synchronize()
        torch.cuda.synchronize()

    sev = HipEvents(2 * K)  # around each step, on the bench stream
    t0 = time.perf_counter()
    for i in range(K):
        a, s, step = calls[i % n_sets]
        sev.record(2 * i, stream)
        if graphs is not None:
            with torch.cuda.stream(stream):
                graphs[i % n_sets].replay()
        elif use_events:
            step.timed(stream, *hev.ev[5 * i:5 * i + 5])
        else:
            step(stream)
        sev.record(2 * i + 1, stream)
    stream.synchronize()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(sev.ms(2 * i, 2 * i + 1) for i in range(K))
    sev.close()
    pct = lambda f: step_ms[min(K - 1, int(round(f * (K - 1))))]
    status = 0
    for a, s, _ in calls:
        status |= int(s.status.item()) | int(a.status.item())
    a, s, _ = calls[0]
    if status:
        print(f"device status bits set: {sv.status_names(status)}", file=sys.stderr)
        sys.exit(1)

    # After the timed region: the same K steps without the library's
    # per-kernel events (each event record adds a few microseconds between
    # kernels, which matters only for the small latency workloads). Reported
    # beside the timed figures, not in place of them.
    plain = None
    if use_events:
        pev = HipEvents(2 * K)
        t1 = time.perf_counter()
        for i in range(K):
            pev.record(2 * i, stream)
            calls[i % n_sets][2](stream)
            pev.record(2 * i + 1, stream)
        stream.synchronize()
        torch.cuda.synchronize()
        plain_elapsed = time.perf_counter() - t1
        pms = sorted(pev.ms(2 * i, 2 * i + 1) for i in range(K))
        pev.close()
        ppct = lambda f: pms[min(K - 1, int(round(f * (K - 1))))]
        plain = {"ms_per_step": round(plain_elapsed / K * 1e3, 4),
                 "step_ms_p10_p50_p90": [round(ppct(0.1), 4), round(ppct(0.5), 4), round(ppct(0.9), 4)]}

    # The other step schedule (SV_OVERLAP_ON when the timed region ran OFF, and
    # back), same inputs and step count, step events only; reported beside
    # the timed figures. Results are bitwise the same in both schedules.
    other = "on" if args.overlap == "off" else "off"
    for _, s_, _ in calls:
        s_.args.step_overlap = sv.OVERLAP_MODES[other]
    for i in range(n_sets):
        calls[i][2](stream)
    stream.synchronize()
    oev = HipEvents(2 * K)
    t2 = time.perf_counter()
    for i in range(K):
        oev.record(2 * i, stream)
        calls[i % n_sets][2](stream)
        oev.record(2 * i + 1, stream)
    stream.synchronize()
    torch.cuda.synchronize()
    other_elapsed = time.perf_counter() - t2
    oms = sorted(oev.ms(2 * i, 2 * i + 1) for i in range(K))
    oev.close()
    for _, s_, _ in calls:
        s_.args.step_overlap = sv.OVERLAP_MODES[args.overlap]
    opct = lambda f: oms[min(K - 1, int(round(f * (K - 1))))]
    other_sched = {"ms_per_step": round(other_elapsed / K * 1e3, 4),
                   "step_ms_p10_p50_p90": [round(opct(0.1), 4), round(opct(0.5), 4), round(opct(0.9), 4)],
                   "value": round(w["N"] * K / other_elapsed, 1)}


    ms = elapsed / K * 1e3
    value = w["N"] * K / elapsed
    acc = s.accept_len.double()
    # residual passes per step, averaged over the input sets (each set runs
    # K / n_sets of the timed steps)
    passes_per_set = [float(c[1].passes.double().sum().item()) for c in calls]
    passes_mean = sum(passes_per_set) / len(passes_per_set)
    passes = s.passes.double()

    kernels = {}
    attn_b, attn_f = attention_bytes(w, 1 if args.kv_fp8 else 0), attention_flops(w)
    rs_b = row_stats_bytes(w)
    # sampled siblings: one 8V pass (logits and q) per rejection; deterministic
    # candidates and the truncation rule's membership tests need none. Under
    # min-p or eta truncation a pass reads only the chunks that hold an allowed
    # token, a number the walk does not report: its passes are not counted
    # there, so the sampler's fraction is a lower bound
    truncated = args.min_p > 0 or args.eta is not None
    per_pass = 0 if det or args.rule == "truncation" or truncated else 8 * w["V"]
    # the walk's layout: workgroups per request, and whether it computes the
    # statistics of the rows it reaches itself (reading no other row) or has a
    # statistics pass read every row first
    slices, lazy = s.walk_layout()
    # rows a walk reaches: the root's and one per accepted node (each read
    # whole, for its normaliser or argmax), averaged over the input sets
    visited_mean = sum(float((c[1].accept_len.double() + 1).sum().item()) for c in calls) / len(calls)
    smp_b = visited_mean * 4 * w["V"] + passes_mean * per_pass
    roofline = None
    if use_events:
        attn_ms = sum(hev.ms(5 * i, 5 * i + 1) for i in range(K)) / K
        rs_ms = sum(hev.ms(5 * i + 2, 5 * i + 3) for i in range(K)) / K
        smp_ms = sum(hev.ms(5 * i + 2, 5 * i + 4) for i in range(K)) / K
        hev.close()
        attn_name = attention_kernel_name(w, cfg, args.kv_fp8)
        kernels[attn_name] = {"us": attn_ms * 1e3, "alg_bytes": attn_b, "GB_s": attn_b / attn_ms / 1e6,
                              "TFLOP_s": attn_f / attn_ms / 1e9}
        walk_ms = smp_ms - rs_ms
        if lazy:
            # the row-statistics launch then only clears the sliced walk's
            # coordination words (or does not run); the walk's launch also
            # holds the attention's split-K merge blocks, if any
            kernels["row_stats_kernel"] = {"us": rs_ms * 1e3, "statistics": False}
            kernels["walk_kernel"] = {"us": walk_ms * 1e3, "alg_bytes": smp_b, "GB_s": smp_b / walk_ms / 1e6,
                                      "slices": slices}
        else:
            kernels["row_stats_kernel"] = {"us": rs_ms * 1e3, "alg_bytes": rs_b, "GB_s": rs_b / rs_ms / 1e6}
            kernels["walk_kernel"] = {"us": walk_ms * 1e3, "slices": slices}
        # the whole sampler on its algorithmic bytes: the logit rows the walk
        # reaches, plus the residual passes it made (logits and q of the
        # rejected row); a statistics pass over every row reads more
        kernels["sampler(stats+finalize+walk)"] = {
            "us": smp_ms * 1e3, "alg_bytes": smp_b, "GB_s": smp_b / smp_ms / 1e6,
            "frac": smp_b / smp_ms / 1e6 / HBM_PEAK_GBS, "rows_reached": visited_mean,
            "rows_read": visited_mean if lazy else float(w["N"] + w["B"]),
            "residual_pass_bytes": passes_mean * per_pass if not truncated else None}
        if args.overlap == "off":
            rest_us = ms * 1e3 - attn_ms * 1e3 - smp_ms * 1e3
            kernels["other(prep+combine)"] = {"us": rest_us}
        else:
            # concurrent spans: each kernel's duration includes the time it
            # shared the device with the other stream's kernels
            kernels["schedule"] = {"concurrent": True,
                                   "note": "attention on a second stream, concurrent with the sampler: the spans "
                                           "overlap and each includes time shared with the other stream"}
        dom = max((k for k in (attn_name, "row_stats_kernel", "walk_kernel") if "alg_bytes" in kernels[k]),
                  key=lambda k: kernels[k]["us"])
        dk = kernels[dom]
        # the committed counters were taken with contiguous bf16 caches
        traffic = counter_traffic(dom, cfg.name) if not (args.paged or args.kv_fp8) else None
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dk["GB_s"], 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(dk["GB_s"] / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "measured_copy_GB_s": round(copy_bandwidth(), 1)}

    cpu = None
    parity = None
    if args.cpu_seconds > 0:
        v_cpu, threads, desc, ref = cpu_baseline(w, args.cpu_seconds, args.min_p, args.siblings, args.rule,
                                                 args.rule_param, tuple(args.eta) if args.eta else None)
        cpu = {"value": round(v_cpu, 2), "unit": "verified draft tokens/s", "cores": threads, "kind": "oracle",
               "sample": desc}
        parity = compare_sample(s, ref)

    line = {
        "metric": "verified draft tokens/sec",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 4),
        "step_ms_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
        **({"without_kernel_events": plain} if plain else {}),
        f"step_overlap_{other}": other_sched,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16+fp8+f32" if args.kv_fp8 else "bf16+f32") if w["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded; no dataset, no model weights)",
        "config": {"workload": cfg.name, "B": w["B"], "draft_nodes": w["N"], "max_T": w["max_T"], "L": cfg.L,
                   "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D, "kv_dtype": cfg.dtype, "V": cfg.V,
                   "temperature": cfg.temperature, "input_seed": cfg.seed, "library_seed": cfg.lib_seed,
                   **({"min_p": args.min_p} if args.min_p > 0 else {}),
                   **({"siblings": "deterministic (top-k of q)"} if det else {}),
                   **({"eta": list(args.eta)} if args.eta else {}),
                   **({"walk_mode": args.walk_mode} if args.walk_mode != "auto" else {}),
                   "step_overlap": args.overlap,
                   **({"kv_layout": f"paged, {args.paged}-slot blocks"} if args.paged else {}),
                   **({"kv_dtype": "fp8 e4m3 (scaled)"} if args.kv_fp8 else {}),
                   **({"rule": args.rule, "rule_param": args.rule_param} if args.rule in ("lenience", "interpolation")
                      else {"rule": args.rule} if args.rule == "truncation" else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "near_ties": parity,
        "input_sets": n_sets,
        "walk_layout": {"slices": slices, "reached_rows_only": lazy},
        **({"input_sha256_16": input_sha} if input_sha else {}),
        **({"hip_graph": True} if args.graph else {}),
        "kernels": {k: {kk: (round(vv, 4 if kk == "frac" else 2) if isinstance(vv, float) else vv)
                        for kk, vv in d.items()} for k, d in kernels.items()},
        "walk": walk_metrics(w, s, K, elapsed, passes),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
