"""Python binding of libspecverify.so (speculative-decoding verification on MI355X).

Argument marshalling only: every step of the verification path runs in the
HIP kernels behind the C ABI of include/spec_verify.h. PyTorch provides the
device memory and the stream. If the library has not been built the calls
raise; there is no fallback.

    attn(...)    tree-masked GQA attention          -> spec_verify_attn
    sample(...)  rejection-sampling tree walk       -> spec_verify_sample
    step(...)    both on one stream                 -> spec_verify_step

AttnCall / SampleCall / StepCall prepare the argument block, outputs and
workspace once so that repeated launches only cross the ABI; StepCall.timed
and StepCall.noalloc reach spec_verify_step_timed and
spec_verify_step_noalloc, SampleCall.walk_layout spec_verify_walk_layout,
and pack(...) / PackCall spec_verify_pack.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_TREE, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP = range(6)
SV_F32, SV_BF16 = 0, 1
SIBLINGS = {"sampled": 0, "deterministic": 1}  # sv_siblings
WALK_MODES = {"auto": 0, "single": 1, "sliced": 2}  # sv_sample_args.walk_mode
OVERLAP_MODES = {"off": 0, "on": 1}  # sv_sample_args.step_overlap
RULES = {"lossless": 0, "lenience": 1, "interpolation": 2, "truncation": 3}  # sv_rule
STATUS_BITS = {0x01: "TREE_INVALID", 0x02: "PACKING", 0x04: "TOKEN_RANGE", 0x08: "NONFINITE",
               0x10: "ZERO_RESIDUAL", 0x20: "CTX_RANGE", 0x40: "SYNC", 0x80: "BLOCK_RANGE"}

_P = ctypes.c_void_p
_i32, _i64, _u32, _u64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float


class SvAttnArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("total_nodes", _i32), ("max_nodes", _i32), ("Hq", _i32), ("Hkv", _i32), ("D", _i32),
                ("dtype", _i32), ("q", _P), ("k_cache", _P), ("v_cache", _P), ("Lcap", _i64), ("ctx_len", _P),
                ("cu_nodes", _P), ("parent", _P), ("anc_mask", _P), ("scale", _f32), ("num_splits", _i32),
                ("out", _P), ("status", _P), ("block_table", _P),
                ("block_size", _i32), ("max_blocks", _i32), ("num_blocks", _i64), ("kv_fp8", _i32),
                ("k_scale", _f32), ("v_scale", _f32)]


class SvSampleArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("V", _i32), ("total_nodes", _i32), ("max_nodes", _i32), ("cu_nodes", _P),
                ("parent", _P), ("draft_tokens", _P), ("target_logits", _P), ("draft_probs", _P),
                ("temperature", _f32), ("min_p", _f32), ("eta_eps", _f32), ("eta_delta", _f32), ("siblings", _i32),
                ("rule", _i32), ("rule_param", _f32), ("seed", _u64), ("step", _u32), ("request_id", _P),
                ("max_depth", _i32),
                ("accept_len", _P), ("accepted_nodes", _P), ("out_tokens", _P), ("probs_out", _P),
                ("uniforms_out", _P), ("residual_passes", _P), ("status", _P), ("walk_mode", _i32),
                ("join_ticks", _i32), ("step_overlap", _i32)]


class SvTiming(ctypes.Structure):
    _fields_ = [("attn_start", _P), ("attn_stop", _P), ("sample_start", _P), ("stats_stop", _P),
                ("sample_stop", _P)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspecverify.so (torch first, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    lib.spec_verify_workspace_size.argtypes = [_P, _P]
    lib.spec_verify_workspace_size.restype = ctypes.c_size_t
    lib.spec_verify_pack_workspace_size.argtypes = [_P]
    lib.spec_verify_pack_workspace_size.restype = ctypes.c_size_t
    for name in ("spec_verify_attn", "spec_verify_sample", "spec_verify_pack"):
        getattr(lib, name).argtypes = [_P, _P, ctypes.c_size_t, _P]
        getattr(lib, name).restype = ctypes.c_int
    lib.spec_verify_step.argtypes = [_P, _P, _P, ctypes.c_size_t, _P]
    lib.spec_verify_step.restype = ctypes.c_int
    lib.spec_verify_step_timed.argtypes = [_P, _P, _P, ctypes.c_size_t, _P, _P]
    lib.spec_verify_step_timed.restype = ctypes.c_int
    lib.spec_verify_step_noalloc.argtypes = [_P, _P, _P]
    lib.spec_verify_step_noalloc.restype = ctypes.c_int
    lib.spec_verify_walk_layout.argtypes = [_P, _P, _P]
    lib.spec_verify_walk_layout.restype = ctypes.c_int
    lib.spec_verify_last_error.argtypes = []
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    lib.spec_verify_struct_size.argtypes = [_i32]
    lib.spec_verify_struct_size.restype = ctypes.c_size_t
    if lib.spec_verify_struct_size(0) != ctypes.sizeof(SvAttnArgs) or \
            lib.spec_verify_struct_size(1) != ctypes.sizeof(SvSampleArgs) or \
            lib.spec_verify_struct_size(2) != ctypes.sizeof(SvPackArgs):
        raise RuntimeError("argument struct layout of the binding does not match the library")
    _lib = lib
    return lib


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"spec_verify error {code}: {msg}")
        self.code = code


def _check(code: int):
    if code != SV_OK:
        raise SpecVerifyError(code, load_library().spec_verify_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_i32(x, device):
    if isinstance(x, torch.Tensor):
        assert x.dtype == torch.int32 and x.is_contiguous(), "int32 contiguous tensor expected"
        return x if x.device == device else x.to(device)
    return torch.as_tensor(x, dtype=torch.int32, device=device)


def _stream_handle(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _event_handle(ev):
    """A hipEvent_t: a raw handle (int) or a torch.cuda.Event."""
    if ev is None:
        return None
    if isinstance(ev, int):
        return ctypes.c_void_p(ev)
    return ctypes.c_void_p(int(ev.cuda_event))


def status_names(word: int) -> list:
    return [n for b, n in STATUS_BITS.items() if word & b]


# ---------------------------------------------------------------------------
class AttnCall:
    """Prepared spec_verify_attn call (outputs and workspace allocated once)."""

    def __init__(self, q, k_cache, v_cache, ctx_len, cu_nodes, *, parent=None, anc_mask=None, max_nodes=0,
                 scale=0.0, num_splits=0, out=None, status=None, block_table=None, kv_fp8_scales=None):
        """block_table: int32 [B, max_blocks] for paged caches; k_cache and
        v_cache are then pools [num_blocks, Hkv, block_size, D].
        kv_fp8_scales=(k_scale, v_scale): k_cache / v_cache are uint8 tensors
        of OCP FP8 E4M3 bytes (q bf16)."""
        load_library()
        dev = q.device
        assert q.is_cuda and q.dim() == 3 and k_cache.dim() == 4 and v_cache.shape == k_cache.shape
        if kv_fp8_scales is None:
            assert q.dtype == k_cache.dtype == v_cache.dtype and q.dtype in (torch.float32, torch.bfloat16)
        else:
            assert q.dtype == torch.bfloat16 and k_cache.dtype == v_cache.dtype == torch.uint8
        for t in (q, k_cache, v_cache):
            assert t.is_contiguous()
        N, Hq, D = q.shape
        B, Hkv, Lcap, D2 = k_cache.shape
        assert D == D2
        if block_table is not None:
            block_table = _dev_i32(block_table, dev)
            assert block_table.dim() == 2
            num_blocks, block_size = B, Lcap
            B, max_blocks = block_table.shape
            Lcap = max_blocks * block_size
        self.keep = {"q": q, "k": k_cache, "v": v_cache, "ctx": _dev_i32(ctx_len, dev), "cu": _dev_i32(cu_nodes, dev),
                     "parent": None if parent is None else _dev_i32(parent, dev), "anc": anc_mask,
                     "block_table": block_table}
        if anc_mask is not None:
            assert anc_mask.dtype == torch.int64 and anc_mask.is_contiguous()
        self.out = out if out is not None else torch.empty((N, Hq, D), dtype=torch.float32, device=dev)
        self.status = status if status is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        a = SvAttnArgs()
        a.B, a.total_nodes, a.max_nodes, a.Hq, a.Hkv, a.D = B, N, int(max_nodes), Hq, Hkv, D
        a.dtype = SV_BF16 if q.dtype == torch.bfloat16 else SV_F32
        a.q, a.k_cache, a.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
        a.Lcap = Lcap
        a.ctx_len, a.cu_nodes = _ptr(self.keep["ctx"]), _ptr(self.keep["cu"])
        a.parent = _ptr(self.keep["parent"])
        a.anc_mask = _ptr(anc_mask)
        a.scale, a.num_splits = float(scale), int(num_splits)
        a.out, a.status = _ptr(self.out), _ptr(self.status)
        if block_table is not None:
            a.block_table, a.block_size, a.max_blocks, a.num_blocks = _ptr(block_table), block_size, max_blocks, \
                num_blocks
        if kv_fp8_scales is not None:
            a.kv_fp8, a.k_scale, a.v_scale = 1, float(kv_fp8_scales[0]), float(kv_fp8_scales[1])
        self.args = a
        lib = load_library()
        self.ws_bytes = lib.spec_verify_workspace_size(ctypes.byref(a), None)
        if self.ws_bytes == 0 and lib.spec_verify_last_error():
            _check(SV_ERR_INVALID_ARG)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)

    def __call__(self, stream=None):
        _check(load_library().spec_verify_attn(ctypes.byref(self.args), _ptr(self.ws), self.ws_bytes,
                                               _stream_handle(stream)))
        return self.out


class SampleCall:
    """Prepared spec_verify_sample call."""

    def __init__(self, cu_nodes, parent, draft_tokens, target_logits, draft_probs, *, temperature, seed, step=0,
                 request_id=None, max_nodes=0, max_depth=None, probs_out=False, uniforms_out=False,
                 residual_passes=False, status=None, min_p=0.0, siblings="sampled", rule="lossless",
                 rule_param=1.0, eta=None, walk_mode="auto", join_ticks=0, step_overlap="off"):
        load_library()
        if siblings not in SIBLINGS:
            raise ValueError(f"siblings must be one of {sorted(SIBLINGS)}")
        if rule not in RULES:
            raise ValueError(f"rule must be one of {sorted(RULES)}")
        if walk_mode not in WALK_MODES:
            raise ValueError(f"walk_mode must be one of {sorted(WALK_MODES)}")
        if step_overlap not in OVERLAP_MODES:
            raise ValueError(f"step_overlap must be one of {sorted(OVERLAP_MODES)}")
        dev = target_logits.device
        assert target_logits.is_cuda and target_logits.dtype == torch.float32 and target_logits.is_contiguous()
        cu = _dev_i32(cu_nodes, dev)
        B = cu.numel() - 1
        toks = _dev_i32(draft_tokens, dev)
        N = toks.numel()
        V = target_logits.shape[1]
        assert target_logits.shape[0] == N + B
        if draft_probs is not None:
            assert draft_probs.dtype == torch.float32 and draft_probs.shape == target_logits.shape
            assert draft_probs.is_contiguous()
        md = int(max_depth) if max_depth is not None else (int(max_nodes) or 64)
        self.keep = {"cu": cu, "parent": _dev_i32(parent, dev), "tok": toks, "logits": target_logits,
                     "q": draft_probs,
                     "rid": None if request_id is None else torch.as_tensor(request_id, device=dev).to(torch.int32)}
        self.accept_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.accepted_nodes = torch.empty((B, md), dtype=torch.int32, device=dev)
        self.out_tokens = torch.empty((B, md + 1), dtype=torch.int32, device=dev)
        self.probs = torch.empty_like(target_logits) if probs_out else None
        self.uniforms = torch.empty(N + B, dtype=torch.float64, device=dev) if uniforms_out else None
        self.passes = torch.empty(B, dtype=torch.int32, device=dev) if residual_passes else None
        self.status = status if status is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        s = SvSampleArgs()
        s.B, s.V, s.total_nodes, s.max_nodes = B, V, N, int(max_nodes)
        s.cu_nodes, s.parent, s.draft_tokens = _ptr(cu), _ptr(self.keep["parent"]), _ptr(toks)
        s.target_logits, s.draft_probs = _ptr(target_logits), _ptr(draft_probs)
        s.temperature, s.seed, s.step = float(temperature), int(seed), int(step)
        s.min_p = float(min_p)
        if eta is not None:  # (eps, delta) of the eta allowed set
            s.eta_eps, s.eta_delta = float(eta[0]), float(eta[1])
        s.siblings = SIBLINGS[siblings]
        s.rule, s.rule_param = RULES[rule], float(rule_param)
        s.request_id = _ptr(self.keep["rid"])
        s.max_depth = md
        s.accept_len, s.accepted_nodes, s.out_tokens = _ptr(self.accept_len), _ptr(self.accepted_nodes), \
            _ptr(self.out_tokens)
        s.probs_out, s.uniforms_out, s.residual_passes = _ptr(self.probs), _ptr(self.uniforms), _ptr(self.passes)
        s.status = _ptr(self.status)
        s.walk_mode, s.join_ticks = WALK_MODES[walk_mode], int(join_ticks)
        s.step_overlap = OVERLAP_MODES[step_overlap]
        self.args = s
        lib = load_library()
        self.ws_bytes = lib.spec_verify_workspace_size(None, ctypes.byref(s))
        if self.ws_bytes == 0 and lib.spec_verify_last_error():
            _check(SV_ERR_INVALID_ARG)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)

    def results(self) -> dict:
        r = {"accept_len": self.accept_len, "accepted_nodes": self.accepted_nodes, "out_tokens": self.out_tokens,
             "status": self.status}
        if self.probs is not None:
            r["probs"] = self.probs
        if self.uniforms is not None:
            r["uniforms"] = self.uniforms
        if self.passes is not None:
            r["residual_passes"] = self.passes
        return r

    def walk_layout(self) -> tuple:
        """spec_verify_walk_layout on the current device: (workgroups per
        request, whether the walk reads only the logit rows it reaches)."""
        n, lazy = _i32(0), _i32(0)
        _check(load_library().spec_verify_walk_layout(ctypes.byref(self.args), ctypes.byref(n), ctypes.byref(lazy)))
        return int(n.value), bool(lazy.value)

    def __call__(self, stream=None):
        _check(load_library().spec_verify_sample(ctypes.byref(self.args), _ptr(self.ws), self.ws_bytes,
                                                 _stream_handle(stream)))
        return self.results()


class StepCall:
    """Prepared spec_verify_step call: attention then sampling on one stream."""

    def __init__(self, attn: AttnCall, sample: SampleCall):
        self.attn, self.sample = attn, sample
        assert attn.args.B == sample.args.B and attn.args.total_nodes == sample.args.total_nodes
        # both halves must see the same cu_nodes buffer
        sample.args.cu_nodes = attn.args.cu_nodes
        sample.keep["cu"] = attn.keep["cu"]
        lib = load_library()
        self.ws_bytes = lib.spec_verify_workspace_size(ctypes.byref(attn.args), ctypes.byref(sample.args))
        if self.ws_bytes == 0 and lib.spec_verify_last_error():
            _check(SV_ERR_INVALID_ARG)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=attn.out.device)

    def __call__(self, stream=None):
        _check(load_library().spec_verify_step(ctypes.byref(self.attn.args), ctypes.byref(self.sample.args),
                                               _ptr(self.ws), self.ws_bytes, _stream_handle(stream)))
        return self._results()

    def timed(self, stream, attn_start=None, attn_stop=None, sample_start=None, stats_stop=None, sample_stop=None):
        """spec_verify_step_timed: the same step, recording the given hipEvent_t
        handles (raw ints or torch.cuda.Event) on the stream."""
        t = SvTiming(_event_handle(attn_start), _event_handle(attn_stop), _event_handle(sample_start),
                     _event_handle(stats_stop), _event_handle(sample_stop))
        _check(load_library().spec_verify_step_timed(ctypes.byref(self.attn.args), ctypes.byref(self.sample.args),
                                                     _ptr(self.ws), self.ws_bytes, _stream_handle(stream),
                                                     ctypes.byref(t)))
        return self._results()

    def noalloc(self, stream=None):
        """spec_verify_step_noalloc: the same step on the library's own scratch
        (this call's workspace is not used)."""
        _check(load_library().spec_verify_step_noalloc(ctypes.byref(self.attn.args), ctypes.byref(self.sample.args),
                                                       _stream_handle(stream)))
        return self._results()

    def _results(self):
        r = self.sample.results()
        r["attn_out"] = self.attn.out
        return r


def attn(q, k_cache, v_cache, ctx_len, cu_nodes, **kw):
    """Tree-masked GQA attention; returns the fp32 output [N, Hq, D]."""
    return AttnCall(q, k_cache, v_cache, ctx_len, cu_nodes, **kw)()


def sample(cu_nodes, parent, draft_tokens, target_logits, draft_probs, **kw):
    """Rejection-sampling walk; returns a dict of device tensors."""
    return SampleCall(cu_nodes, parent, draft_tokens, target_logits, draft_probs, **kw)()


def step(q, k_cache, v_cache, ctx_len, cu_nodes, parent, draft_tokens, target_logits, draft_probs, *,
         temperature, seed, max_nodes=0, attn_kw=None, sample_kw=None):
    a = AttnCall(q, k_cache, v_cache, ctx_len, cu_nodes, parent=parent, max_nodes=max_nodes, **(attn_kw or {}))
    s = SampleCall(a.keep["cu"], parent, draft_tokens, target_logits, draft_probs, temperature=temperature,
                   seed=seed, max_nodes=max_nodes, **(sample_kw or {}))
    return StepCall(a, s)()


# ---------------------------------------------------------------------------
class SvPackArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("total_cand", _i32), ("cu_cand", _P), ("cand_parent", _P), ("cand_token", _P),
                ("cand_score", _P), ("budget", _i32), ("cu_nodes", _P), ("parent", _P), ("draft_tokens", _P),
                ("src", _P), ("total_nodes", _P), ("status", _P)]


class PackCall:
    """Prepared spec_verify_pack call: budgeted super-tree packing of the
    batch's candidate trees (outputs sized for min(budget, candidates))."""

    def __init__(self, cu_cand, cand_parent, cand_token, cand_score, *, budget, status=None):
        lib = load_library()
        dev = cand_score.device if torch.is_tensor(cand_score) else torch.device("cuda")
        cu = _dev_i32(cu_cand, dev)
        par = _dev_i32(cand_parent, dev)
        tok = _dev_i32(cand_token, dev)
        sc = torch.as_tensor(cand_score, dtype=torch.float32, device=dev).contiguous()
        B, M = cu.numel() - 1, par.numel()
        cap = max(min(int(budget), M), 1)
        self.keep = {"cu": cu, "par": par, "tok": tok, "score": sc}
        self.cu_nodes = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.parent = torch.empty(cap, dtype=torch.int32, device=dev)
        self.draft_tokens = torch.empty(cap, dtype=torch.int32, device=dev)
        self.src = torch.empty(cap, dtype=torch.int32, device=dev)
        self.total = torch.empty(1, dtype=torch.int32, device=dev)
        self.status = status if status is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        a = SvPackArgs()
        a.B, a.total_cand, a.budget = B, M, int(budget)
        a.cu_cand, a.cand_parent, a.cand_token, a.cand_score = _ptr(cu), _ptr(par), _ptr(tok), _ptr(sc)
        a.cu_nodes, a.parent, a.draft_tokens, a.src = _ptr(self.cu_nodes), _ptr(self.parent), \
            _ptr(self.draft_tokens), _ptr(self.src)
        a.total_nodes, a.status = _ptr(self.total), _ptr(self.status)
        self.args = a
        self.ws_bytes = lib.spec_verify_pack_workspace_size(ctypes.byref(a))
        if self.ws_bytes == 0 and lib.spec_verify_last_error():
            _check(SV_ERR_INVALID_ARG)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)

    def __call__(self, stream=None):
        _check(load_library().spec_verify_pack(ctypes.byref(self.args), _ptr(self.ws), self.ws_bytes,
                                               _stream_handle(stream)))
        return {"cu_nodes": self.cu_nodes, "parent": self.parent, "draft_tokens": self.draft_tokens,
                "src": self.src, "total_nodes": self.total, "status": self.status}


def pack(cu_cand, cand_parent, cand_token, cand_score, *, budget, **kw):
    """Budgeted super-tree packing; returns a dict of device tensors (parent,
    draft_tokens and src hold min(budget, candidates) entries, the first
    total_nodes of them valid)."""
    return PackCall(cu_cand, cand_parent, cand_token, cand_score, budget=budget, **kw)()
