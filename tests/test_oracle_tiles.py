"""Pins for the oracle's tiled edge tensor and its Viterbi decision gaps (CPU only).

The oracle materialises the edge potentials in tiles of segment positions
(EN explainer, "1. Problem Statement", "Edge Tensor Materialization", in
pieces).  Every long-sequence expected value is written by the multi-tile path,
so its seams are pinned here: forcing tiles of 1, 2, K-1, K and K+1 positions
must reproduce the one-tile run to 1e-12 in every output, tile = 1 must match
brute-force enumeration, and off-by-one mistakes planted at the seams (in a
copy of the oracle, on the CPU) must be caught.

The Viterbi decision gaps (the gap of each decision along the decoded path,
and of the final label) are pinned against enumeration of every segmentation.
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle
import oracle.semicrf as osc
import pins


def _case(seed, L, T, K, C, proj=False):
    rng = np.random.default_rng(seed)
    em = rng.standard_normal((T, C)) * 1.3
    trans = rng.normal(0, 0.6, (C, C))
    dur = rng.normal(0, 0.6, (K, C))
    pj = (rng.normal(0, 0.7, (L, C)), rng.normal(0, 0.7, (L, C))) if proj else None
    return em, L, trans, dur, K, pj


def _run(case):
    em, L, trans, dur, K, pj = case
    return oracle.sequence(em, L, trans, dur, K, proj=pj)


def _max_diff(a, b):
    keys = ["mu", "grad_em", "grad_trans", "grad_dur", "dS", "grad_proj_start",
            "grad_proj_end", "boundary"]
    err = max(abs(a["logZ"] - b["logZ"]), abs(a["logZ_backward"] - b["logZ_backward"]))
    for k in keys:
        err = max(err, float(np.abs(a[k] - b[k]).max()))
    va, vb = a["viterbi"], b["viterbi"]
    err = max(err, abs(va["score"] - vb["score"]))
    if not (np.array_equal(va["labels"], vb["labels"])
            and np.array_equal(va["seg_start"], vb["seg_start"])):
        err = max(err, 1.0)
    ga, gb = np.asarray(va["gaps"]), np.asarray(vb["gaps"])
    if ga.shape != gb.shape or not np.array_equal(np.isfinite(ga), np.isfinite(gb)):
        return max(err, 1.0)
    fin = np.isfinite(ga)
    if fin.any():
        err = max(err, float(np.abs(ga[fin] - gb[fin]).max()))
    return err


TILE_CASES = [
    # seed, L, T, K, C, projections
    (101, 90, 95, 20, 3, False),     # 4-5 tiles of K-1 .. K+1 positions
    (102, 67, 67, 21, 4, True),      # with projections, 3-4 tiles
    (103, 100, 104, 25, 3, False),
]


@pytest.mark.parametrize("seed,L,T,K,C,proj", TILE_CASES)
@pytest.mark.parametrize("which", ["1", "2", "K-1", "K", "K+1"])
def test_forced_tiles_match_one_tile(monkeypatch, seed, L, T, K, C, proj, which):
    case = _case(seed, L, T, K, C, proj)
    assert osc._tile(K, C) >= L + 1          # the default run is one tile
    ref = _run(case)
    tile = {"1": 1, "2": 2, "K-1": K - 1, "K": K, "K+1": K + 1}[which]
    monkeypatch.setattr(osc, "_tile", lambda K_, C_: tile)
    got = _run(case)
    assert _max_diff(got, ref) < 1e-12


def test_tile_of_one_matches_brute_force(monkeypatch):
    em, L, trans, dur, K, _ = _case(104, 8, 8, 3, 3)
    monkeypatch.setattr(osc, "_tile", lambda K_, C_: 1)
    r = oracle.sequence(em, L, trans, dur, K)
    bf = pins.brute_force(em, L, trans, dur, K)
    assert abs(r["logZ"] - bf["logZ"]) < 1e-12
    assert abs(r["logZ_backward"] - bf["logZ"]) < 1e-12
    np.testing.assert_allclose(r["mu"], bf["mu"], atol=1e-12)
    np.testing.assert_allclose(r["grad_dur"], bf["grad_dur"], atol=1e-12)
    np.testing.assert_allclose(r["grad_trans"], bf["grad_trans"], atol=1e-12)
    np.testing.assert_allclose(r["dS"], bf["end"] - bf["start"], atol=1e-12)
    assert abs(r["viterbi"]["score"] - bf["best"]) < 1e-12


def _planted(name, old, new):
    """A copy of oracle function `name` with the line `old` replaced by `new`."""
    src = inspect.getsource(getattr(osc, name))
    assert old in src, f"seam line not found in {name}"
    ns = {}
    exec(compile(src.replace(old, new), f"<planted {name}>", "exec"), dict(vars(osc)), ns)
    f = ns[name]
    # globals: the live module, so the forced tile size applies inside the copy too
    return types.FunctionType(f.__code__, vars(osc), name, f.__defaults__)


SEAM_MISTAKES = [
    ("forward", "s_lo = max(0, t0 - K)", "s_lo = max(0, t0 - K + 1)"),
    ("viterbi", "s_lo = max(0, t0 - K)", "s_lo = max(0, t0 - K + 1)"),
    ("forward", "psi = edge_potentials(S, trans, dur, K, L, s_lo, t1 - 1, proj)",
     "psi = edge_potentials(S, trans, dur, K, L, s_lo, t1 - 2, proj)"),
    ("backward", "s_hi = min(L, s_lo + tile)", "s_hi = min(L, s_lo + tile - 1)"),
    ("posteriors", "s_hi = min(L, s_lo + tile)", "s_hi = min(L, s_lo + tile - 1)"),
]


@pytest.mark.parametrize("name,old,new", SEAM_MISTAKES,
                         ids=[f"{m[0]}:{m[2]}" for m in SEAM_MISTAKES])
def test_tile_pins_catch_planted_seam_mistakes(monkeypatch, name, old, new):
    # short K and durations that favour long segments, so the terms at a seam matter
    em, L, trans, dur, K, _ = _case(105, 30, 30, 4, 3)
    dur = dur + 1.5 * np.arange(1, K + 1)[:, None]
    case = (em, L, trans, dur, K, None)
    ref = _run(case)
    monkeypatch.setattr(osc, name, _planted(name, old, new))
    monkeypatch.setattr(osc, "_tile", lambda K_, C_: K)
    try:
        err = _max_diff(_run(case), ref)
    except (IndexError, ValueError):
        err = math.inf                    # the mistake broke the run outright
    assert err > 1e-6, f"tile pin missed the planted seam mistake in {name}"


# --------------------------------------------------------------------------- decision gaps


GAP_CASES = [
    # seed, L, T, K, C
    (111, 6, 6, 3, 3),
    (112, 7, 7, 4, 2),
    (113, 5, 5, 8, 3),
    (114, 6, 6, 1, 3),
    (115, 7, 7, 7, 1),
]


@pytest.mark.parametrize("seed,L,T,K,C", GAP_CASES)
def test_viterbi_decision_gaps_match_enumeration(seed, L, T, K, C):
    em, L, trans, dur, K, _ = _case(seed, L, T, K, C)
    v = oracle.sequence(em, L, trans, dur, K, want_grads=False)["viterbi"]
    segs = pins.all_segmentations(em, L, trans, dur, K)
    path = tuple(tuple(int(x) for x in s) for s in v["segments"])
    best = max(sc for _, sc in segs)
    assert abs(v["score"] - best) < 1e-12
    gaps, final_gap = pins.decision_gaps(segs, path)
    ok = np.isfinite(gaps)
    np.testing.assert_array_equal(np.isfinite(v["gaps"]), ok)
    np.testing.assert_allclose(v["gaps"][ok], gaps[ok], atol=1e-12)
    assert (math.isinf(final_gap) and math.isinf(v["final_gap"])) or \
        abs(v["final_gap"] - final_gap) < 1e-12
    assert abs(v["margin"] - min([final_gap] + list(gaps))) < 1e-12


def test_gaps_are_zero_on_exact_ties():
    """All potentials zero: every choice ties, so every gap is exactly 0."""
    em, L, trans, dur, K = np.zeros((6, 2)), 6, np.zeros((2, 2)), np.zeros((3, 2)), 3
    v = oracle.sequence(em, L, trans, dur, K, want_grads=False)["viterbi"]
    # (the first segment, [0, 1), has no alternative at its end node: gap inf)
    assert v["gaps"][0] == math.inf and np.all(v["gaps"][1:] == 0.0) and v["final_gap"] == 0.0
    # ties go to the lowest (k, c'), and the lowest final label
    assert np.all(v["seg_start"] == 1) and np.all(v["labels"] == 0)
