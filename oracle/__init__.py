"""fp64 CPU oracle of the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY. The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it to check and time the GPU library;
the library itself never imports, links or runs anything from here, and the
oracle shares no code with it (the two only consume the same input bytes).

The arithmetic lives in ``oracle.c`` (plain C loops in fp64, built with the
host compiler into ``liboracle.so``); this module marshals numpy arrays.

Functions and the passages they follow:
  philox4x32_10, uniform   Philox4x32-10 (Salmon et al., SC'11); the uniform
                           r_i of [SD] "Mathematical Rejection Sampling Algorithm".
  ancestors                [SD] "Tree Attention Mask Mechanics".
  attention                [SD] "Tree Attention Mask Mechanics" and
                           "Interaction with Advanced Attention Architectures".
  target_probs, argmax     softmax(logits / T); greedy argmax.
  residual                 [SD] R_i(x); [LOSSY] appendix F.1 r(x).
  remove_candidate         [LOSSY] appendix G.3: the target after a deterministic
                           candidate is tried and rejected.
  inverse_cdf              the draw from R_i / p.
  verify                   the whole walk ([SD] acceptance rule; [LOSSY] 2.1 h(x)).
  min_p_theta,             [LOSSY] section 2.3: the min-p allowed set and the
  truncate_min_p, allowed  truncated target p_Theta, membership decided from
                           the definition in fp64; verify(min_p=...) walks
                           against p_Theta ("truncation sampling + SD", G.2/G.3).
  eta_threshold,           [LOSSY] section 2.3: the eta allowed set
  truncate_eta             {p >= min(eps, delta exp(-H))}.
  verify(siblings=...)     "deterministic": the G.3 rule for deterministic
                           candidates (p~_i, candidates removed one by one).
  verify(rule=...)         [LOSSY] 3.1 lossy accept tests: lenience (A.3) and
                           interpolation / CoS (A.1).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ACCEPT_TOL = 1e-5  # |u - P/Q| below this marks an accept test as a near-tie
CDF_TOL = 1e-6     # a CDF boundary this close to u marks the final draw as a near-tie
RULES = {"lossless": 0, "lenience": 1, "interpolation": 2, "truncation": 3}
SET_TOL = 0.0  # allowed-set band: 0 = each set's own error bound (see verify)


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with the host C compiler."""
    from .build_oracle import build_oracle

    return build_oracle(verbose=verbose)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, u32, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double
    lib.orc_philox4x32_10.argtypes = [P, P, P]
    lib.orc_philox4x32_10.restype = None
    lib.orc_uniform.argtypes = [u64, u32, u32, u32, u32]
    lib.orc_uniform.restype = f64
    lib.orc_ancestors.argtypes = [i32, P, P, P]
    lib.orc_ancestors.restype = i32
    lib.orc_attention.argtypes = [i32, i32, i32, i32, i32, P, P, P, i64, P, P, P, f64, i64, P, P, i32]
    lib.orc_attention.restype = i32
    lib.orc_attention_ex.argtypes = [i32, i32, i32, i32, i32, P, P, P, i64, P, P, P, f64, i64, P, P, i32, P, i32,
                                     i32, i64, i32, f64, f64]
    lib.orc_attention_ex.restype = i32
    lib.orc_fp8_e4m3.argtypes = [ctypes.c_uint8]
    lib.orc_fp8_e4m3.restype = f64
    lib.orc_target_probs.argtypes = [i32, P, f64, P]
    lib.orc_target_probs.restype = i32
    lib.orc_argmax.argtypes = [i32, P]
    lib.orc_argmax.restype = i32
    lib.orc_residual.argtypes = [i32, P, P, P]
    lib.orc_residual.restype = f64
    lib.orc_inverse_cdf.argtypes = [i32, P, f64, P]
    lib.orc_inverse_cdf.restype = i32
    lib.orc_verify.argtypes = [i32, i32, P, P, P, P, P, f64, i32, f64, f64, f64, f64, i32, i32, f64, u64,
                               u32, P, i32,
                               P, P, P, P,
                               P, P, P, P, P, P, P, f64, f64, i32]
    lib.orc_verify.restype = i32
    lib.orc_target_rows.argtypes = [i32, P, f64, i64, P, P]
    lib.orc_target_rows.restype = i32
    lib.orc_truncate_min_p.argtypes = [i32, P, f64, P]
    lib.orc_truncate_min_p.restype = None
    lib.orc_min_p_threshold.argtypes = [f64, f64]
    lib.orc_min_p_threshold.restype = f64
    lib.orc_eta_threshold.argtypes = [i32, P, f64, f64, f64, P, P]
    lib.orc_eta_threshold.restype = f64
    lib.orc_allowed.argtypes = [ctypes.c_float, ctypes.c_float, f64]
    lib.orc_allowed.restype = i32
    lib.orc_row_finite.argtypes = [i32, P]
    lib.orc_row_finite.restype = i32
    lib.orc_truncate_eta.argtypes = [i32, P, f64, f64, f64, P, P]
    lib.orc_truncate_eta.restype = f64
    lib.orc_row_entropy.argtypes = [i32, P, f64]
    lib.orc_row_entropy.restype = f64
    lib.orc_pack.argtypes = [i32, P, P, P, P, i64, P, P, P, P, P, P]
    lib.orc_pack.restype = i32
    lib.orc_remove_candidate.argtypes = [i32, P, i32, P]
    lib.orc_remove_candidate.restype = f64
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def philox4x32_10(counter, key) -> np.ndarray:
    ctr = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().orc_philox4x32_10(_ptr(ctr), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, request_id: int, j: int, purpose: int, step: int) -> float:
    return float(_load().orc_uniform(seed, request_id, j, purpose, step))


def ancestors(parent) -> tuple[np.ndarray, np.ndarray]:
    """(anc bitmasks uint64 [T], depth int32 [T]); raises ValueError on a bad tree."""
    par = np.ascontiguousarray(parent, dtype=np.int32)
    T = par.shape[0]
    anc = np.zeros(max(T, 1), dtype=np.uint64)
    depth = np.zeros(max(T, 1), dtype=np.int32)
    rc = _load().orc_ancestors(T, _ptr(par), _ptr(anc), _ptr(depth))
    if rc != 0:
        raise ValueError(f"invalid tree (code {rc})")
    return anc[:T], depth[:T]


def fp8_e4m3(byte: int) -> float:
    """Value of one OCP FP8 E4M3 (finite form) byte."""
    return float(_load().orc_fp8_e4m3(int(byte)))


def attention(q, k, v, ctx_len, cu_nodes, parent, *, Hq, Hkv, scale=None, dtype="f32", items=None,
              nthreads=None, block_table=None, kv_fp8_scales=None) -> np.ndarray:
    """fp64 tree-masked GQA attention.

    q [N,Hq,D], k/v [B,Hkv,Lcap,D] as float32 arrays (dtype='f32') or as uint16
    bf16 bit patterns (dtype='bf16'). items: optional int64 [n,2] of
    (packed node, q head); returns [n, D] then, else [N, Hq, D].
    block_table: int32 [B, max_blocks] for paged caches; k/v are then pools
    [num_blocks, Hkv, block_size, D] and slot t of request b sits in block
    block_table[b, t // block_size] at row t % block_size.
    kv_fp8_scales=(k_scale, v_scale): k/v are uint8 OCP FP8 E4M3 bytes whose
    element values are the decoded bytes times the scale (q keeps dtype).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    code = {"f32": 0, "bf16": 1}[dtype]
    kv_code, ks, vs = code, 1.0, 1.0
    if kv_fp8_scales is not None:
        assert k.dtype == np.uint8 and v.dtype == np.uint8
        kv_code, (ks, vs) = 2, (float(np.float32(kv_fp8_scales[0])), float(np.float32(kv_fp8_scales[1])))
    elif code == 0:
        assert k.dtype == np.float32 and v.dtype == np.float32
    else:
        assert k.dtype == np.uint16 and v.dtype == np.uint16
    assert q.dtype == (np.float32 if code == 0 else np.uint16)
    D = int(k.shape[3])
    if block_table is None:
        B, Lcap = int(k.shape[0]), int(k.shape[2])
        bt, bs, mb, nb = None, 0, 0, 0
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        B, mb = int(bt.shape[0]), int(bt.shape[1])
        bs, nb = int(k.shape[2]), int(k.shape[0])
        Lcap = mb * bs
    N = int(q.shape[0])
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    cu = np.ascontiguousarray(cu_nodes, dtype=np.int32)
    par = np.ascontiguousarray(parent, dtype=np.int32)
    if items is None:
        n_items = N * Hq
        out = np.zeros((N, Hq, D), dtype=np.float64)
        it_ptr = None
    else:
        items = np.ascontiguousarray(items, dtype=np.int64).reshape(-1, 2)
        n_items = items.shape[0]
        out = np.zeros((n_items, D), dtype=np.float64)
        it_ptr = _ptr(items)
    rc = _load().orc_attention_ex(B, Hq, Hkv, D, code, _ptr(q), _ptr(k), _ptr(v), Lcap, _ptr(ctx), _ptr(cu),
                                  _ptr(par), float(scale), n_items, it_ptr, _ptr(out),
                                  nthreads or _default_threads(), _ptr(bt), bs, mb, nb, kv_code, ks, vs)
    if rc != 0:
        raise ValueError("oracle attention: bad packing or tree")
    return out


def target_probs(logits, temperature: float) -> np.ndarray:
    row = np.ascontiguousarray(logits, dtype=np.float32)
    p = np.zeros(row.shape[0], dtype=np.float64)
    if _load().orc_target_probs(row.shape[0], _ptr(row), float(temperature), _ptr(p)):
        raise ValueError("non-finite or all -inf logits")
    return p


def target_rows(logits2d, temperature: float, rows) -> np.ndarray:
    lg = np.ascontiguousarray(logits2d, dtype=np.float32)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((r.shape[0], lg.shape[1]), dtype=np.float64)
    if _load().orc_target_rows(lg.shape[1], _ptr(lg), float(temperature), r.shape[0], _ptr(r), _ptr(out)):
        raise ValueError("non-finite or all -inf logits")
    return out


def argmax(logits) -> int:
    row = np.ascontiguousarray(logits, dtype=np.float32)
    return int(_load().orc_argmax(row.shape[0], _ptr(row)))


def residual(P, Q) -> tuple[np.ndarray, float]:
    P = np.ascontiguousarray(P, dtype=np.float64)
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    out = np.zeros_like(P)
    R = _load().orc_residual(P.shape[0], _ptr(P), _ptr(Q), _ptr(out))
    return out, float(R)


def remove_candidate(P, x: int) -> tuple[np.ndarray, float]:
    """P with token x taken out and renormalised ([LOSSY] G.3), and the mass left."""
    P = np.ascontiguousarray(P, dtype=np.float64)
    out = np.zeros_like(P)
    R = _load().orc_remove_candidate(P.shape[0], _ptr(P), int(x), _ptr(out))
    return out, float(R)


def inverse_cdf(P, u: float) -> tuple[int, float]:
    P = np.ascontiguousarray(P, dtype=np.float64)
    m = np.zeros(1, dtype=np.float64)
    y = _load().orc_inverse_cdf(P.shape[0], _ptr(P), float(u), _ptr(m))
    return int(y), float(m[0])


def min_p_theta(temperature: float, min_p: float) -> float:
    """Threshold on l_x - l_max of the min-p allowed set: T ln p_base in fp64,
    from the fp32 values of T and p_base as a caller passing fp32 arguments
    gets them; -inf (no truncation) unless 0 < min_p < 1 and T > 0."""
    T, pb = float(np.float32(temperature)), float(np.float32(min_p))
    if not (T > 0.0 and 0.0 < pb < 1.0):
        return float("-inf")
    return float(_load().orc_min_p_threshold(T, pb))


def allowed(logit: float, lmax: float, theta: float) -> bool:
    """Membership test of the allowed sets: fp64(l_x) - fp64(l_max) >= theta."""
    return bool(_load().orc_allowed(float(np.float32(logit)), float(np.float32(lmax)), float(theta)))


def truncate_min_p(logits_row, p_row, theta: float) -> np.ndarray:
    """p_row (a normalised target row) truncated to the min-p allowed set."""
    lg = np.ascontiguousarray(logits_row, dtype=np.float32)
    p = np.array(p_row, dtype=np.float64, copy=True)
    _load().orc_truncate_min_p(lg.shape[0], _ptr(lg), float(theta), _ptr(p))
    return p


def eta_threshold(logits_row, temperature: float, eps: float, delta: float) -> tuple[float, float, float]:
    """(threshold on l_x - l_max, G = E_p[-z], Var_p(z)) of the eta allowed set."""
    lg = np.ascontiguousarray(logits_row, dtype=np.float32)
    g = np.zeros(1, np.float64)
    v = np.zeros(1, np.float64)
    th = _load().orc_eta_threshold(lg.shape[0], _ptr(lg), float(temperature), float(eps), float(delta), _ptr(g),
                                   _ptr(v))
    return float(th), float(g[0]), float(v[0])


def row_finite(logits_row) -> bool:
    lg = np.ascontiguousarray(logits_row, dtype=np.float32)
    return bool(_load().orc_row_finite(lg.shape[0], _ptr(lg)))


def truncate_eta(logits_row, p_row, temperature: float, eps: float, delta: float) -> tuple[np.ndarray, float, float]:
    """p_row truncated to the eta allowed set {p >= min(eps, delta e^-H)}; also
    returns the fp64 threshold on l_x - l_max and the smallest distance of a
    token to it (log-probability units)."""
    lg = np.ascontiguousarray(logits_row, dtype=np.float32)
    p = np.array(p_row, dtype=np.float64, copy=True)
    m = np.zeros(1, np.float64)
    th = _load().orc_truncate_eta(lg.shape[0], _ptr(lg), float(temperature), float(eps), float(delta), _ptr(p),
                                  _ptr(m))
    return p, float(th), float(m[0])


def row_entropy(logits_row, temperature: float) -> float:
    lg = np.ascontiguousarray(logits_row, dtype=np.float32)
    return float(_load().orc_row_entropy(lg.shape[0], _ptr(lg), float(temperature)))


def eta_params(eta) -> tuple[float, float]:
    """(eps, delta) of the eta allowed set as fp32 arguments reach the library."""
    eps, delta = eta
    return float(np.float32(eps)), float(np.float32(delta))


def verify(cu_nodes, parent, tokens, logits, q, *, temperature, seed, step=0, request_id=None,
           max_depth=None, accept_tol=ACCEPT_TOL, cdf_tol=CDF_TOL, nthreads=None, min_p=0.0,
           siblings="sampled", rule="lossless", rule_param=1.0, eta=None, set_tol=SET_TOL) -> dict:
    """The verification walk for a packed batch; returns a dict of numpy arrays.

    logits, q: float32 [N+B, V] (q may be None when temperature == 0 or the
    siblings are deterministic).
    min_p > 0 verifies against the min-p truncated target ([LOSSY] 2.3, G.2).
    siblings="deterministic": the children of a node are deterministic
    candidates ([LOSSY] G.3): candidate i is accepted with probability
    p~_i(x^(i)), the target with the candidates tried before it removed and
    renormalised; q is not used.
    rule="lenience" (rule_param = l) or "interpolation" (rule_param = lambda),
    both in (0, 1]: the lossy accept tests of [LOSSY] 3.1 (h = min(1, p/(l q))
    and h = min(1, (lambda p + (1 - lambda) q)/q)), residuals unchanged.
    eta=(eps, delta): verify against the eta truncated target ([LOSSY] 2.3)
    instead of min-p.
    Allowed-set membership is the definition in fp64 (l_x - l_max against the
    fp64 threshold). flag_kind 2 marks a position whose outcome some threshold
    within the set's band would change; set_tol > 0 fixes the band's
    half-width (log-probability units), 0 takes each set's own error bound:
    fp64 rounding of T ln p_base for min-p, the first-order bound of two
    fp64 evaluations of the eta threshold (sums of V fp64 weights in any
    order) for eta.
    rule="truncation": truncation-based verification ([LOSSY] 3.2) over the
    min-p or eta allowed set: accept iff the drafted token is allowed; after
    every child of a position is rejected, draw from q restricted to the set.
    """
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}")
    if siblings not in ("sampled", "deterministic"):
        raise ValueError("siblings must be 'sampled' or 'deterministic'")
    det = 1 if siblings == "deterministic" else 0
    cu = np.ascontiguousarray(cu_nodes, dtype=np.int32)
    B = cu.shape[0] - 1
    N = int(cu[-1]) if B >= 0 else 0
    par = np.ascontiguousarray(parent, dtype=np.int32)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    V = int(lg.shape[1])
    qq = None if q is None else np.ascontiguousarray(q, dtype=np.float32)
    if temperature > 0 and not det:
        assert qq is not None and qq.shape == lg.shape
    rid = None if request_id is None else np.ascontiguousarray(request_id, dtype=np.uint32)
    if max_depth is None:
        Ts = np.diff(cu)
        max_depth = int(Ts.max()) if B > 0 else 0
    out = {
        "accept_len": np.zeros(B, np.int32),
        "accepted_nodes": np.zeros((B, max(max_depth, 0)), np.int32),
        "out_tokens": np.zeros((B, max_depth + 1), np.int32),
        "uniforms": np.zeros(N + B, np.float64),
        "flag_depth": np.zeros(B, np.int32),
        "flag_kind": np.zeros(B, np.int32),
        "n_rejections": np.zeros(B, np.int32),
        "status": np.zeros(B, np.int32),
        "min_accept_margin": np.zeros(B, np.float64),
        "cdf_margin": np.zeros(B, np.float64),
        "draw_mass": np.zeros(B, np.float64),
    }
    theta = min_p_theta(temperature, min_p)
    trunc = 1 if theta > float("-inf") else 0
    p_base = float(np.float32(min_p)) if trunc else 0.0
    eps, delta = 0.0, 0.0
    if eta is not None:
        if trunc:
            raise ValueError("min_p and eta are exclusive")
        eps, delta = eta_params(eta)
        trunc = 2 if temperature > 0 else 0
    rc = _load().orc_verify(B, V, _ptr(cu), _ptr(par), _ptr(tok), _ptr(lg), _ptr(qq), float(temperature),
                            trunc, p_base, eps, delta, float(set_tol), det, RULES[rule],
                            float(np.float32(rule_param)), int(seed), int(step), _ptr(rid), int(max_depth),
                            _ptr(out["accept_len"]),
                            _ptr(out["accepted_nodes"]), _ptr(out["out_tokens"]), _ptr(out["uniforms"]),
                            _ptr(out["flag_depth"]), _ptr(out["flag_kind"]), _ptr(out["n_rejections"]),
                            _ptr(out["status"]), _ptr(out["min_accept_margin"]), _ptr(out["cdf_margin"]),
                            _ptr(out["draw_mass"]), float(accept_tol), float(cdf_tol),
                            nthreads or _default_threads())
    if rc != 0:
        raise ValueError("oracle verify: bad arguments")
    return out


def pack(cu_cand, cand_parent, cand_token, cand_score, budget: int) -> dict:
    """Budgeted super-tree packing ([ECHO] 3.1, Figure 3 step 3): keep the
    `budget` best candidates by (min score on the path, descending; request;
    local index) and pack them request by request; see orc_pack."""
    cu = np.ascontiguousarray(cu_cand, dtype=np.int32)
    B = cu.shape[0] - 1
    par = np.ascontiguousarray(cand_parent, dtype=np.int32)
    tok = np.ascontiguousarray(cand_token, dtype=np.int32)
    sc = np.ascontiguousarray(cand_score, dtype=np.float32)
    M = int(cu[-1]) if B > 0 else 0
    cap = max(min(int(budget), M), 1)
    out = {"cu_nodes": np.zeros(B + 1, np.int32), "parent": np.zeros(cap, np.int32),
           "draft_tokens": np.zeros(cap, np.int32), "src": np.zeros(cap, np.int32)}
    n = np.zeros(1, np.int32)
    st = np.zeros(1, np.int32)
    rc = _load().orc_pack(B, _ptr(cu), _ptr(par), _ptr(tok), _ptr(sc), int(budget), _ptr(out["cu_nodes"]),
                          _ptr(out["parent"]), _ptr(out["draft_tokens"]), _ptr(out["src"]), _ptr(n), _ptr(st))
    if rc != 0:
        raise ValueError("oracle pack: bad arguments")
    N = int(n[0])
    for k in ("parent", "draft_tokens", "src"):
        out[k] = out[k][:N]
    out["total_nodes"] = N
    out["status"] = int(st[0])
    return out
