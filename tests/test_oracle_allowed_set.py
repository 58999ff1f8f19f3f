"""Oracle pins of the allowed sets' boundary and of the near-tie flag there.

[LOSSY] section 2.3 defines the min-p set A = {x : p(x) >= p_base max p} and
the eta set A = {x : p(x) >= min(eps, delta exp(-H(p)))} in exact arithmetic.
The oracle decides membership from that definition in fp64 (the logit
difference against T ln p_base, or against the eta threshold). Pins:

- tokens placed one fp32 step inside and one step outside the min-p cutoff,
  at a p_base whose threshold rounds down in fp32 (so a rule on the fp32
  rounding of the threshold would admit the outside token), decided as the
  definition p(x) / max p = exp((l_x - l_max) / T) >= p_base says;
- the flag of a boundary position (kind 2) is exactly "some threshold within
  the band changes the output": with a fixed band, every unflagged request
  gives the same output for every threshold in the band, and every flagged
  one changes at its flagged depth for some threshold there (thresholds
  moved through p_base, or through delta when every row's eta threshold is
  T (ln delta - G));
- the derived eta band (first-order bound of two fp64 evaluations of the
  threshold) is of the size the analysis gives on the workload rows;
- rows without a distribution (NaN, +inf, all -inf) stop greedy and sampled
  walks alike, without a bonus token.
"""
import math

import numpy as np
import pytest

import oracle
from sampler_cases import replicated_batch, rows_from_probs

P_BASE_ROUNDS_DOWN = 0.05  # fp32(1 * ln 0.05f) < ln 0.05f in fp64


def _boundary_row(V=16):
    """A row with l_max = 0, one token one fp32 step outside the min-p cutoff
    of P_BASE_ROUNDS_DOWN at T = 1 (index 1) and one a step inside (index 2);
    the rest far below."""
    th = oracle.min_p_theta(1.0, P_BASE_ROUNDS_DOWN)
    f = np.float32(th)
    assert float(f) < th  # the fp32 rounding of the threshold lies below it
    out = f if float(f) < th else np.nextafter(f, np.float32(-np.inf))
    inside = np.nextafter(out, np.float32(np.inf))
    assert float(inside) >= th
    row = np.full(V, -20.0, np.float32)
    row[0], row[1], row[2] = 0.0, out, inside
    return row, th


def test_min_p_cutoff_one_step_each_side():
    row, th = _boundary_row()
    pb = float(np.float32(P_BASE_ROUNDS_DOWN))
    # the definition, in fp64 through the exponential: p(x) / max p >= p_base
    ratio = np.exp(row.astype(np.float64) - 0.0)
    assert ratio[1] < pb <= ratio[2]
    assert not oracle.allowed(row[1], 0.0, th) and oracle.allowed(row[2], 0.0, th)
    # a rule on fp32(l_x - l_max) >= fp32(theta) would admit the outside token
    assert np.float32(row[1] - np.float32(0.0)) >= np.float32(th)
    p = oracle.target_probs(row, 1.0)
    pt = oracle.truncate_min_p(row, p, th)
    assert pt[1] == 0.0 and pt[2] > 0.0 and pt[0] > 0.0
    np.testing.assert_allclose(pt[[0, 2]], p[[0, 2]] / (p[0] + p[2]), rtol=1e-15)


@pytest.mark.parametrize("token", [1, 2])
def test_min_p_cutoff_decides_the_walk(token):
    """One drafted token at the cutoff, drawn with tiny q so that any positive
    truncated probability accepts it: the outside token is always rejected
    (and never drawn), the inside one always accepted."""
    row, _ = _boundary_row()
    V = row.size
    q = np.full(V, 1e-6, np.float32)
    q[0] = 1.0 - 1e-6 * (V - 1)
    n = 200
    cu = np.arange(n + 1, dtype=np.int32)
    par = np.full(n, -1, np.int32)
    toks = np.full(n, token, np.int32)
    logits = np.tile(np.stack([row, row]), (n, 1))
    qq = np.tile(np.stack([q, q]), (n, 1))
    out = oracle.verify(cu, par, toks, logits, qq, temperature=1.0, seed=77, max_depth=1, min_p=P_BASE_ROUNDS_DOWN)
    assert (out["flag_depth"] < 0).all()
    if token == 1:
        assert (out["accept_len"] == 0).all() and (out["out_tokens"][:, 0] != 1).all()
    else:
        assert (out["accept_len"] == 1).all()


def _shifted_outputs(run, shifts):
    outs = []
    for s in shifts:
        o = run(s)
        outs.append((o["accept_len"], o["accepted_nodes"], o["out_tokens"]))
    return outs


def _same_request(a, b, req, depth=None):
    acc_a, nodes_a, toks_a = a
    acc_b, nodes_b, toks_b = b
    if depth is None:
        return acc_a[req] == acc_b[req] and (nodes_a[req] == nodes_b[req]).all() and (
            toks_a[req] == toks_b[req]).all()
    return (nodes_a[req, :depth] == nodes_b[req, :depth]).all() and (toks_a[req, :depth] == toks_b[req, :depth]).all()


def _check_band_flags(ref, shifted, band_sets):
    """ref: the oracle's run at the exact thresholds with its flags; shifted:
    outputs with every threshold moved by each of the shifts (all within the
    band). Unflagged requests never change; flagged ones keep their prefix,
    and change at the flagged depth for some shift (band_sets: the shifts that
    realise every distinct set of the flagged rows)."""
    base = (ref["accept_len"], ref["accepted_nodes"], ref["out_tokens"])
    B = ref["accept_len"].size
    n_flag = 0
    for b in range(B):
        fd = int(ref["flag_depth"][b])
        if fd < 0:
            for s in shifted:
                assert _same_request(base, s, b), b
            continue
        assert ref["flag_kind"][b] == 2
        n_flag += 1
        for s in shifted:
            assert _same_request(base, s, b, fd), b
        assert any(not _same_request(base, s, b) for s in band_sets), b
    return n_flag


def test_min_p_band_flag_is_exact():
    rng = np.random.default_rng(911)
    V, n, T, pb = 24, 400, 1.0, 0.2
    parent = np.array([-1, -1, 0, 2, -1], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.3, draft_noise=0.9)
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    tol = 0.08  # band half-width in log-probability units (T = 1)
    run = lambda p_base, st=0.0: oracle.verify(cu, par, toks, logits, qq, temperature=T, seed=31, max_depth=5,
                                               min_p=p_base, set_tol=st)
    ref = run(pb, tol)
    th = oracle.min_p_theta(T, pb)
    # thresholds that realise every set inside the band: midpoints between the
    # band's logit differences, and just inside each end
    d = np.unique(np.concatenate([r.astype(np.float64) - r.max() for r in lg]))
    inb = d[np.abs(d - th) <= tol * T]
    assert inb.size >= 2  # the band holds boundary tokens
    cuts = np.concatenate([[th - tol * T * 0.999, th + tol * T * 0.999], (inb[1:] + inb[:-1]) / 2])
    pbs = [float(np.float32(math.exp(t / T))) for t in cuts]
    pbs = [p for p in pbs if abs(T * math.log(p) - th) <= tol * T]
    shifted = _shifted_outputs(lambda p: run(p), pbs)
    n_flag = _check_band_flags(ref, shifted, shifted)
    assert 0 < n_flag < n  # both kinds of requests occur
    # with the band of fp64 rounding only, nothing here is a near tie
    assert (run(pb)["flag_kind"] != 2).all()


def test_eta_band_flag_is_exact():
    """Every row in the delta branch (eps large): the threshold is
    T (ln delta - G), so moving delta moves every row's threshold alike."""
    rng = np.random.default_rng(912)
    V, n, T, eps, delta = 20, 300, 1.0, 0.9, 0.3
    parent = np.array([-1, 0, -1, 2], np.int32)
    lg, q = rows_from_probs(rng, V, parent.size + 1, sharp=1.2, draft_noise=0.8)
    for r in lg:
        th, G, _ = oracle.eta_threshold(r, T, float(np.float32(eps)), float(np.float32(delta)))
        assert abs(th - T * (math.log(np.float32(delta)) - G)) < 1e-12  # delta branch
    cu, par, toks, logits, qq = replicated_batch(rng, parent, lg, q, n)
    tol = 0.04
    run = lambda dl, st=0.0: oracle.verify(cu, par, toks, logits, qq, temperature=T, seed=37, max_depth=4,
                                           eta=(eps, dl), set_tol=st)
    ref = run(delta, tol)
    ln_d = math.log(float(np.float32(delta)))
    shifts = np.linspace(-0.999 * tol, 0.999 * tol, 41)
    deltas = [float(np.float32(math.exp(ln_d + s))) for s in shifts]
    deltas = [x for x in deltas if abs(math.log(x) - ln_d) <= tol]
    shifted = _shifted_outputs(lambda x: run(x), deltas)
    n_flag = _check_band_flags(ref, shifted, shifted)
    assert 0 < n_flag < n


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_eta_derived_band_size(T):
    """The band of two fp64 evaluations of the eta threshold,
    2^-53 (V + 64) (8 + 8 G + 4 Var + 4 G^2), on N(0, 3^2) rows over a
    128256-token vocabulary (the throughput buckets' rows) lies between 1e-12
    and 1e-7 log-probability units, and no row's band holds a token (at T = 2
    the threshold lies among the bulk of the logits, the densest place)."""
    rng = np.random.default_rng(913 + int(4 * T))
    V, rows, hits = 128256, 6, 0
    for _ in range(rows):
        lg = (rng.standard_normal(V) * 3).astype(np.float32)
        th, G, var = oracle.eta_threshold(lg, T, float(np.float32(0.05)), float(np.float32(0.3)))
        band = math.ldexp((V + 64) * (8 + 8 * G + 4 * var + 4 * G * G), -53)
        assert 1e-12 < band < 1e-7, (G, var, band)
        d = lg.astype(np.float64) - float(lg.max())
        hits += int((np.abs(d - th) <= band * T).any())
    assert hits == 0


def _nonfinite_batch():
    rng = np.random.default_rng(915)
    V = 32
    lg, q = rows_from_probs(rng, V, 3, sharp=1.0)
    parent = np.array([-1, 0], np.int32)
    cases = []
    for kind in ("nan0", "posinf", "all_neginf", "nan_late"):
        l2 = lg.copy()
        if kind == "nan0":
            l2[1, 0] = np.nan
        elif kind == "posinf":
            l2[1, 5] = np.inf
        elif kind == "all_neginf":
            l2[1, :] = -np.inf
        else:
            l2[1, V - 1] = np.nan
        cases.append(l2)
    cu = np.array([0, 2, 4, 6, 8], np.int32)
    par = np.tile(parent, 4)
    # the first drafted token is the root row's argmax, so greedy reaches row 1
    a0 = int(np.argmax(lg[0]))
    toks = np.array([a0, 3] * 4, np.int32)
    logits = np.concatenate(cases).astype(np.float32)
    qq = np.tile(q, (4, 1)).astype(np.float32)
    return cu, par, toks, logits, qq


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_nonfinite_rows_stop_the_walk(T):
    cu, par, toks, logits, qq = _nonfinite_batch()
    out = oracle.verify(cu, par, toks, logits, qq if T > 0 else None, temperature=T, seed=3, max_depth=2)
    for b in range(4):
        assert out["status"][b] & 0x08
        if out["accept_len"][b] == 1:  # reached the bad row: no token there
            assert out["out_tokens"][b, 1] == -1
        else:  # rejected at the root: the draw comes from the (finite) root row
            assert out["out_tokens"][b, 0] >= 0 or T == 0.0
    if T == 0.0:
        assert (out["accept_len"] == 1).all() and (out["out_tokens"][:, 1] == -1).all()
    assert not oracle.row_finite(logits[1]) and oracle.row_finite(logits[0])
    assert oracle.argmax(np.array([np.nan, 1.0, 3.0, 3.0], np.float32)) == 2
