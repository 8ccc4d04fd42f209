"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: brute-force
enumeration, the textbook linear-chain CRF at K = 1, exact segmentation counts,
the pages' own invariants (marginals sum to one, mass conservation), a
hand-worked centring example and the pages' memory arithmetic, and
finite differences of log Z.  The last test plants plausible mistakes in the
oracle (on the CPU) and checks that the pins catch each of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.semicrf as osc
import pins
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, L, T, K, C, scale=1.0, trans_sd=0.5, dur_sd=0.5):
    rng = np.random.default_rng(seed)
    em = scale * rng.standard_normal((T, C))
    trans = rng.normal(0, trans_sd, (C, C))
    dur = rng.normal(0, dur_sd, (K, C))
    return em, L, trans, dur, K


BF_CASES = [
    # seed, L, T, K, C
    (1, 6, 6, 3, 3),
    (2, 7, 9, 4, 2),     # ragged: padding rows must be ignored
    (3, 5, 5, 8, 3),     # K > L
    (4, 6, 6, 1, 3),     # K = 1
    (5, 7, 7, 7, 1),     # C = 1
    (6, 1, 3, 2, 4),     # L = 1
    (7, 6, 6, 2, 4),
]


# --------------------------------------------------------------------------- centring / memory


def test_centering_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "centering_example.json")))
    nu, S = oracle.centered_prefix(np.array(g["em"]), g["length"])
    np.testing.assert_allclose(nu, g["nu"], atol=1e-15)
    np.testing.assert_allclose(S, g["S"], atol=1e-15)


def test_pages_memory_arithmetic():
    g = json.load(open(os.path.join(GOLDEN, "pages_memory.json")))
    T, K, C, f = g["T"], g["K"], g["C"], g["bytes_per_float"]
    edge = T * K * C * C * f
    prefix = T * C * f
    rings = (K * C + 2 * K * C) * f     # forward K x C and backward 2K x C
    assert abs(edge / 1e9 - g["edge_tensor_GB_about"]) < 0.5
    assert abs(prefix / 1e6 - g["prefix_array_MB_about"]) < 0.5
    # the backward ring alone is 2K*C*4 B = 9.6 KB; with the forward ring 14.4 KB
    assert abs(2 * K * C * f / 1e3 - g["ring_buffers_KB_about"]) < 0.5
    assert rings == 3 * K * C * f


# --------------------------------------------------------------------------- brute force


@pytest.mark.parametrize("seed,L,T,K,C", BF_CASES)
def test_oracle_matches_brute_force(seed, L, T, K, C):
    em, L, trans, dur, K = _case(seed, L, T, K, C)
    bf = pins.brute_force(em, L, trans, dur, K)
    assert bf["n"] == pins.count_segmentations(L, K, C)
    r = oracle.sequence(em, L, trans, dur, K)
    assert abs(r["logZ"] - bf["logZ"]) < 1e-12
    assert abs(r["logZ_backward"] - bf["logZ"]) < 1e-12
    np.testing.assert_allclose(r["mu"], bf["mu"], atol=1e-12)
    np.testing.assert_allclose(r["grad_dur"], bf["grad_dur"], atol=1e-12)
    np.testing.assert_allclose(r["grad_trans"], bf["grad_trans"], atol=1e-12)
    np.testing.assert_allclose(r["dS"], bf["end"] - bf["start"], atol=1e-12)
    v = r["viterbi"]
    assert abs(v["score"] - bf["best"]) < 1e-12
    margin = bf["best"] - bf["second"]
    assert abs(v["margin"] - margin) < 1e-12 or (math.isinf(margin) and math.isinf(v["margin"]))
    if margin > 1e-9:
        np.testing.assert_array_equal(v["labels"], bf["labels"])
        np.testing.assert_array_equal(v["seg_start"], bf["seg_start"])
    # the decoded segmentation scores what it claims, from the definition
    assert abs(oracle.segmentation_score(r["S"], trans, dur, K, v["seg_start"], v["labels"])
               - v["score"]) < 1e-12


def test_tiny_slice_brute_force():
    """The T=8 slice of the tiny configuration (K=8, C=4: 312,500 segmentations)."""
    w = workloads.tiny_slice(8)
    out = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K)
    for b in range(w.B):
        bf = pins.brute_force(w.em[b], 8, w.trans, w.dur, w.K)
        assert bf["n"] == 312_500
        assert abs(out["logZ"][b] - bf["logZ"]) < 1e-12
        np.testing.assert_allclose(out["mu"][b], bf["mu"], atol=1e-12)
        assert abs(out["score"][b] - bf["best"]) < 1e-12
        if bf["best"] - bf["second"] > 1e-9:
            np.testing.assert_array_equal(out["labels"][b], bf["labels"])
    bfs = [pins.brute_force(w.em[b], 8, w.trans, w.dur, w.K) for b in range(w.B)]
    np.testing.assert_allclose(out["grad_dur"], sum(b["grad_dur"] for b in bfs), atol=1e-12)
    np.testing.assert_allclose(out["grad_trans"], sum(b["grad_trans"] for b in bfs), atol=1e-12)


# --------------------------------------------------------------------------- K = 1


@pytest.mark.parametrize("seed,L,C", [(11, 40, 3), (12, 25, 6), (13, 1, 4)])
def test_k1_is_linear_chain(seed, L, C):
    em, L, trans, dur, K = _case(seed, L, L + 3, 1, C)
    x = np.array(pins.centred_emissions(em, L))
    lc = pins.linear_chain(x + dur[0][None, :], trans)
    r = oracle.sequence(em, L, trans, dur, 1)
    assert abs(r["logZ"] - lc["logZ"]) < 1e-11
    np.testing.assert_allclose(r["mu"], lc["node"], atol=1e-12)
    np.testing.assert_allclose(r["grad_trans"], lc["pair"], atol=1e-12)
    np.testing.assert_allclose(r["grad_dur"][0], lc["node"].sum(axis=0), atol=1e-11)
    assert abs(r["viterbi"]["score"] - lc["score"]) < 1e-11
    np.testing.assert_array_equal(r["viterbi"]["labels"], lc["path"])
    # every frame is a boundary at K = 1 (NL explainer, "Resultaten": a linear
    # CRF treats every frame as a boundary)
    post = osc.posteriors(r["S"], trans, dur, 1, L, *_ab(r["S"], trans, dur, 1, L))
    np.testing.assert_allclose(post["start"][:L].sum(axis=1), 1.0, atol=1e-12)
    assert np.all(r["viterbi"]["seg_start"] == 1)


def _ab(S, trans, dur, K, L):
    alpha, logZ = osc.forward(S, trans, dur, K, L)
    beta = osc.backward(S, trans, dur, K, L)
    return alpha, beta, logZ


# --------------------------------------------------------------------------- closed forms


@pytest.mark.parametrize("L,K,C", [(1, 1, 1), (9, 3, 2), (12, 12, 1), (20, 5, 3), (30, 7, 4)])
def test_zero_potentials_count(L, K, C):
    em = np.tile(np.arange(C, dtype=np.float64)[None, :] * 2.0, (L, 1))   # constant per label (exact mean)
    r = oracle.sequence(em, L, np.zeros((C, C)), np.zeros((K, C)), K)
    assert abs(r["logZ"] - math.log(pins.count_segmentations(L, K, C))) < 1e-10
    if C == 1 and K >= L:
        assert abs(r["logZ"] - (L - 1) * math.log(2.0)) < 1e-10
    v = r["viterbi"]
    # every segmentation ties at 0: lowest (k, c') everywhere -> unit segments of label 0
    assert v["score"] == 0.0
    assert np.all(v["labels"] == 0) and np.all(v["seg_start"] == 1)
    assert v["margin"] == 0.0 or (L == 1 and C == 1)


# --------------------------------------------------------------------------- invariants


@pytest.mark.parametrize("seed,L,K,C", [(21, 60, 5, 3), (22, 80, 12, 4), (23, 50, 50, 2)])
def test_invariants(seed, L, K, C):
    em, L, trans, dur, K = _case(seed, L, L, K, C, scale=2.0)
    r = oracle.sequence(em, L, trans, dur, K)
    mu = r["mu"]
    assert abs(r["logZ"] - r["logZ_backward"]) < 1e-10
    np.testing.assert_allclose(mu.sum(axis=1), 1.0, atol=1e-12)        # marginals sum to 1
    assert mu.min() > -1e-12 and mu.max() < 1 + 1e-12
    alpha, beta, logZ = _ab(r["S"], trans, dur, K, L)
    post = osc.posteriors(r["S"], trans, dur, K, L, alpha, beta, logZ)
    assert abs(post["start"][0].sum() - 1.0) < 1e-12                   # a segment starts at 0
    assert abs(post["end"][L].sum() - 1.0) < 1e-12                     # and one ends at L
    # mass conservation: expected covered length = L; transitions = segments - 1
    k = np.arange(1, K + 1)[:, None]
    assert abs((k * r["grad_dur"]).sum() - L) < 1e-9
    assert abs(r["grad_trans"].sum() - (r["grad_dur"].sum() - 1.0)) < 1e-9
    np.testing.assert_allclose(r["grad_em"].sum(axis=0), 0.0, atol=1e-10)
    # centring: adding a per-label constant to the emissions changes nothing
    shift = np.random.default_rng(seed).normal(0, 5, C)
    r2 = oracle.sequence(em + shift[None, :], L, trans, dur, K, want_viterbi=False)
    assert abs(r2["logZ"] - r["logZ"]) < 1e-9
    np.testing.assert_allclose(r2["mu"], mu, atol=1e-11)


def test_batch_padding_and_upstream_gradient():
    w = workloads.make_custom(5, B=3, T=30, C=3, K=6)
    g = np.array([0.5, -2.0, 1.25])
    out = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K, grad_log_z=g)
    for b in range(w.B):
        L = int(w.lengths[b])
        r = oracle.sequence(w.em[b], L, w.trans, w.dur, w.K, g=g[b], want_viterbi=False)
        np.testing.assert_allclose(out["grad_em"][b, :L], r["grad_em"], atol=1e-14)
        assert np.all(out["grad_em"][b, L:] == 0) and np.all(out["mu"][b, L:] == 0)
        assert np.all(out["labels"][b, L:] == -1)
    single = [oracle.sequence(w.em[b], int(w.lengths[b]), w.trans, w.dur, w.K,
                              want_viterbi=False) for b in range(w.B)]
    np.testing.assert_allclose(out["grad_dur"], sum(g[b] * single[b]["grad_dur"] for b in range(3)),
                               atol=1e-12)


# --------------------------------------------------------------------------- finite differences


def _logz(em, L, trans, dur, K, nu=None):
    _, S = osc.centered_prefix(em, L, nu=nu)
    return osc.forward(S, trans, dur, K, L)[1]


def test_finite_differences():
    em, L, trans, dur, K = _case(31, 14, 16, 5, 3, scale=1.5)
    r = oracle.sequence(em, L, trans, dur, K, want_viterbi=False)
    h = 1e-5
    nu0 = em[:L].mean(axis=0)
    fd_em = np.zeros((L, 3))
    fd_mu = np.zeros((L, 3))
    for t in range(L):
        for c in range(3):
            e = np.zeros_like(em)
            e[t, c] = h
            fd_em[t, c] = (_logz(em + e, L, trans, dur, K) - _logz(em - e, L, trans, dur, K)) / (2 * h)
            fd_mu[t, c] = (_logz(em + e, L, trans, dur, K, nu0)
                           - _logz(em - e, L, trans, dur, K, nu0)) / (2 * h)
    np.testing.assert_allclose(r["grad_em"], fd_em, atol=1e-8)
    np.testing.assert_allclose(r["mu"], fd_mu, atol=1e-8)
    fd_tr = np.zeros_like(trans)
    for i in range(3):
        for j in range(3):
            e = np.zeros_like(trans)
            e[i, j] = h
            fd_tr[i, j] = (_logz(em, L, trans + e, dur, K) - _logz(em, L, trans - e, dur, K)) / (2 * h)
    np.testing.assert_allclose(r["grad_trans"], fd_tr, atol=1e-8)
    fd_du = np.zeros_like(dur)
    for i in range(K):
        for j in range(3):
            e = np.zeros_like(dur)
            e[i, j] = h
            fd_du[i, j] = (_logz(em, L, trans, dur + e, K) - _logz(em, L, trans, dur - e, K)) / (2 * h)
    np.testing.assert_allclose(r["grad_dur"], fd_du, atol=1e-8)
    # the pages' weaker criterion: cosine >= 0.9999 (EN explainer, "4. Results and Benchmarks")
    a, b = r["grad_em"].ravel(), fd_em.ravel()
    assert a @ b / (np.linalg.norm(a) * np.linalg.norm(b)) >= 0.9999


# --------------------------------------------------------------------------- gold-segmentation loss


def _gold(seed, L, T, K, C):
    labels, seg = workloads.gold_segmentation(seed, np.array([L]), T, C, K)
    return labels[0, :L], seg[0, :L]


@pytest.mark.parametrize("seed,L,T,K,C", BF_CASES)
def test_nll_matches_brute_force(seed, L, T, K, C):
    em, L, trans, dur, K = _case(seed, L, T, K, C)
    labels, seg = _gold(100 + seed, L, T, K, C)
    r = oracle.nll_sequence(em, L, trans, dur, K, labels, seg)
    ref = pins.brute_force_nll(em, L, trans, dur, K, labels, seg)
    assert abs(r["nll"] - ref) < 1e-10 * max(1.0, abs(ref))
    assert r["nll"] >= -1e-12                      # log Z >= the score of any segmentation
    # the centred emission gradient sums to zero over labels at every position
    assert np.abs(r["grad_em"].sum(axis=1)).max() < 1e-12


def test_nll_finite_differences():
    em, L, trans, dur, K = _case(57, 6, 6, 3, 2, scale=1.2, trans_sd=0.8, dur_sd=0.8)
    labels, seg = _gold(157, L, 6, K, 2)
    g = 0.7
    r = oracle.nll_sequence(em, L, trans, dur, K, labels, seg, g=g)
    f = lambda e, t, d: g * pins.brute_force_nll(e, L, t, d, K, labels, seg)
    h = 1e-5
    for arr, key in ((em, "grad_em"), (trans, "grad_trans"), (dur, "grad_dur")):
        fd = np.zeros(r[key].shape)
        for idx in np.ndindex(*fd.shape):
            e = np.zeros_like(arr)
            e[idx] = h
            args_p = [em, trans, dur]
            args_m = [em, trans, dur]
            pos = 0 if arr is em else (1 if arr is trans else 2)
            args_p[pos] = arr + e
            args_m[pos] = arr - e
            fd[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        np.testing.assert_allclose(r[key], fd, atol=1e-7, err_msg=key)


def _mut_gold_no_trans(labels, seg_start, L, K, C, _orig=osc.gold_features, **kw):
    f = list(_orig(labels, seg_start, L, K, C, **kw))
    f[2] = np.zeros_like(f[2])                     # transitions of y* not counted
    return tuple(f)


def _mut_gold_dur_index(labels, seg_start, L, K, C, _orig=osc.gold_features, **kw):
    f = list(_orig(labels, seg_start, L, K, C, **kw))
    f[1] = np.vstack([f[1][1:], f[1][:1]])         # length k counted as k - 1
    return tuple(f)


def _mut_gold_extent(labels, seg_start, L, K, C, _orig=osc.gold_features, **kw):
    f = list(_orig(labels, seg_start, L, K, C, **kw))
    f[0] = np.roll(f[0], 1, axis=0)                # segment extents off by one position
    return tuple(f)


@pytest.mark.parametrize("name,fn", [
    ("gold transitions dropped", _mut_gold_no_trans),
    ("gold duration index", _mut_gold_dur_index),
    ("gold segment extents", _mut_gold_extent),
])
def test_nll_pins_catch_planted_mistakes(monkeypatch, name, fn):
    em, L, trans, dur, K = _case(59, 6, 6, 3, 2, scale=1.2, trans_sd=0.8, dur_sd=0.8)
    labels, seg = _gold(159, L, 6, K, 2)
    h = 1e-5
    monkeypatch.setattr(osc, "gold_features", fn)
    bad = oracle.nll_sequence(em, L, trans, dur, K, labels, seg)
    f = lambda e, t, d: pins.brute_force_nll(e, L, t, d, K, labels, seg)
    err = 0.0
    for arr, key in ((em, "grad_em"), (trans, "grad_trans"), (dur, "grad_dur")):
        for idx in np.ndindex(*bad[key].shape):
            e = np.zeros_like(arr)
            e[idx] = h
            a = [em, trans, dur]
            b = [em, trans, dur]
            pos = 0 if arr is em else (1 if arr is trans else 2)
            a[pos] = arr + e
            b[pos] = arr - e
            err = max(err, abs(bad[key][idx] - (f(*a) - f(*b)) / (2 * h)))
    assert err > 1e-3, f"pin missed planted mistake: {name}"


# --------------------------------------------------------------------------- planted mistakes


def _mut_transpose(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    return _orig(S, np.asarray(trans).T, dur, K, L, s_lo, s_hi, proj)


def _mut_dur_shift(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    d = np.vstack([np.asarray(dur)[1:], np.zeros((1, np.asarray(dur).shape[1]))])
    return _orig(S, trans, d, K, L, s_lo, s_hi, proj)


def _mut_drop_dur(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    return _orig(S, trans, np.zeros_like(dur), K, L, s_lo, s_hi, proj)


def _mut_sign(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    return _orig(-S, trans, dur, K, L, s_lo, s_hi, proj)


def _mut_start_trans(trans, _orig=osc._trans_with_start):
    t = np.asarray(trans, dtype=np.float64)
    return np.vstack([t, t[:1]])          # first segment wrongly pays trans[0, c]


def _mut_no_centering(em_b, L, nu=None, _orig=osc.centered_prefix):
    return _orig(em_b, L, nu=np.zeros(np.asarray(em_b).shape[1]))


@pytest.mark.parametrize("name,attr,fn", [
    ("transposed trans", "edge_potentials", _mut_transpose),
    ("dur index off by one", "edge_potentials", _mut_dur_shift),
    ("dropped dur", "edge_potentials", _mut_drop_dur),
    ("content sign", "edge_potentials", _mut_sign),
    ("transition into first segment", "_trans_with_start", _mut_start_trans),
    ("no centring", "centered_prefix", _mut_no_centering),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, attr, fn):
    em, L, trans, dur, K = _case(41, 6, 6, 3, 3, scale=1.0, trans_sd=0.7, dur_sd=0.7)
    em = em + np.array([0.9, -0.4, 0.3])[None, :]     # non-zero means, so centring matters
    bf = pins.brute_force(em, L, trans, dur, K)
    good = oracle.sequence(em, L, trans, dur, K)
    assert abs(good["logZ"] - bf["logZ"]) < 1e-12
    monkeypatch.setattr(osc, attr, fn)
    bad = oracle.sequence(em, L, trans, dur, K)
    err = max(abs(bad["logZ"] - bf["logZ"]), np.abs(bad["mu"] - bf["mu"]).max(),
              np.abs(bad["grad_trans"] - bf["grad_trans"]).max())
    assert err > 1e-3, f"pin missed planted mistake: {name}"


# --------------------------------------------------------------------------- boundary projections


def _proj(seed, L, C, sd=0.8):
    rng = np.random.default_rng(seed)
    return rng.normal(0, sd, (L, C)), rng.normal(0, sd, (L, C))


@pytest.mark.parametrize("seed,L,T,K,C", BF_CASES)
def test_projections_match_brute_force(seed, L, T, K, C):
    """Start / end projections (reading 9) against the enumeration, which adds them to
    each segment's score position by position: log Z, every expectation, the start and
    end marginals (the projections' gradients), the boundary probability and Viterbi."""
    em, L, trans, dur, K = _case(seed, L, T, K, C)
    proj = _proj(seed + 500, L, C)
    bf = pins.brute_force(em, L, trans, dur, K, proj=proj)
    r = oracle.sequence(em, L, trans, dur, K, g=1.0, proj=proj)
    assert abs(r["logZ"] - bf["logZ"]) < 1e-12
    assert abs(r["logZ_backward"] - bf["logZ"]) < 1e-12
    np.testing.assert_allclose(r["mu"], bf["mu"], atol=1e-12)
    np.testing.assert_allclose(r["grad_dur"], bf["grad_dur"], atol=1e-12)
    np.testing.assert_allclose(r["grad_trans"], bf["grad_trans"], atol=1e-12)
    np.testing.assert_allclose(r["grad_proj_start"], bf["start"][:L], atol=1e-12)
    np.testing.assert_allclose(r["grad_proj_end"], bf["end"][1:], atol=1e-12)
    np.testing.assert_allclose(r["boundary"], bf["start"][:L].sum(axis=1), atol=1e-12)
    v = r["viterbi"]
    assert abs(v["score"] - bf["best"]) < 1e-12
    if bf["best"] - bf["second"] > 1e-9:
        np.testing.assert_array_equal(v["labels"], bf["labels"])
        np.testing.assert_array_equal(v["seg_start"], bf["seg_start"])
    assert abs(oracle.segmentation_score(r["S"], trans, dur, K, v["seg_start"], v["labels"], proj)
               - v["score"]) < 1e-12


@pytest.mark.parametrize("side", [0, 1])
def test_constant_projection_is_a_duration_shift(side):
    """P_start[t, c] = x_c for every t (or P_end) adds x_c once per segment of label c,
    exactly what adding x_c to dur[k-1, c] for every k does."""
    em, L, trans, dur, K = _case(91, 40, 40, 6, 3)
    x = np.array([0.7, -1.1, 0.4])
    proj = [np.zeros((L, 3)), np.zeros((L, 3))]
    proj[side] = np.tile(x, (L, 1))
    a = oracle.sequence(em, L, trans, dur, K, proj=tuple(proj))
    b = oracle.sequence(em, L, trans, dur + x[None, :], K)
    assert abs(a["logZ"] - b["logZ"]) < 1e-11
    np.testing.assert_allclose(a["mu"], b["mu"], atol=1e-12)
    np.testing.assert_allclose(a["grad_dur"], b["grad_dur"], atol=1e-12)
    np.testing.assert_allclose(a["grad_trans"], b["grad_trans"], atol=1e-12)
    assert abs(a["viterbi"]["score"] - b["viterbi"]["score"]) < 1e-11
    np.testing.assert_array_equal(a["viterbi"]["labels"], b["viterbi"]["labels"])
    # the projection's gradient sums to the expected segment count of each label
    g = a["grad_proj_start" if side == 0 else "grad_proj_end"]
    np.testing.assert_allclose(g.sum(axis=0), a["grad_dur"].sum(axis=0), atol=1e-11)


def test_k1_projections_are_unary_scores():
    """K = 1: every position is a segment, so both projections act as unary scores of
    the textbook linear-chain CRF; every position is a boundary."""
    em, L, trans, dur, K = _case(92, 30, 30, 1, 4)
    ps, pe = _proj(93, L, 4)
    x = np.array(pins.centred_emissions(em, L))
    lc = pins.linear_chain(x + dur[0][None, :] + ps + pe, trans)
    r = oracle.sequence(em, L, trans, dur, 1, proj=(ps, pe))
    assert abs(r["logZ"] - lc["logZ"]) < 1e-11
    np.testing.assert_allclose(r["mu"], lc["node"], atol=1e-12)
    np.testing.assert_allclose(r["grad_proj_start"], lc["node"], atol=1e-12)
    np.testing.assert_allclose(r["grad_proj_end"], lc["node"], atol=1e-12)
    np.testing.assert_allclose(r["boundary"], 1.0, atol=1e-12)
    assert abs(r["viterbi"]["score"] - lc["score"]) < 1e-11
    np.testing.assert_array_equal(r["viterbi"]["labels"], lc["path"])


def test_boundary_probability_invariants():
    """A segment always starts at 0 and one always ends at L - 1; boundary
    probabilities lie in [0, 1] and sum to the expected number of segments."""
    em, L, trans, dur, K = _case(94, 120, 120, 15, 4, scale=1.5)
    ps, pe = _proj(95, L, 4, sd=1.5)
    r = oracle.sequence(em, L, trans, dur, K, proj=(ps, pe))
    bnd = r["boundary"]
    assert abs(bnd[0] - 1.0) < 1e-12
    assert abs(r["grad_proj_end"][L - 1].sum() - 1.0) < 1e-12
    assert bnd.min() > -1e-12 and bnd.max() < 1 + 1e-12
    assert abs(bnd.sum() - r["grad_dur"].sum()) < 1e-9
    assert abs(r["grad_proj_end"].sum() - r["grad_dur"].sum()) < 1e-9
    # a position strictly inside every segment that can cover it is no boundary:
    # forbid starts at t = 5 for every label
    ps2 = ps.copy()
    ps2[5] = -np.inf
    r2 = oracle.sequence(em, L, trans, dur, K, proj=(ps2, pe), want_viterbi=True)
    assert r2["boundary"][5] == 0.0 and r2["viterbi"]["seg_start"][5] == 0


def test_projection_finite_differences():
    em, L, trans, dur, K = _case(96, 9, 9, 4, 3)
    ps, pe = _proj(97, L, 3)
    r = oracle.sequence(em, L, trans, dur, K, g=0.6, proj=(ps, pe), want_viterbi=False)
    h = 1e-5

    def lz(a, b):
        _, S = oracle.centered_prefix(em, L)
        return oracle.forward(S, trans, dur, K, L, (a, b))[1]

    for arr, key, which in ((ps, "grad_proj_start", 0), (pe, "grad_proj_end", 1)):
        for idx in np.ndindex(*arr.shape):
            e = np.zeros_like(arr)
            e[idx] = h
            up = (ps + e, pe) if which == 0 else (ps, pe + e)
            dn = (ps - e, pe) if which == 0 else (ps, pe - e)
            fd = 0.6 * (lz(*up) - lz(*dn)) / (2 * h)
            assert abs(r[key][idx] - fd) < 1e-8, (key, idx)


def test_nll_with_projections_matches_brute_force():
    em, L, trans, dur, K = _case(98, 6, 6, 3, 2)
    proj = _proj(99, L, 2)
    labels, seg = _gold(198, L, 6, K, 2)
    r = oracle.nll_sequence(em, L, trans, dur, K, labels, seg, 0.8, proj)
    assert abs(r["nll"] - pins.brute_force_nll(em, L, trans, dur, K, labels, seg, proj)) < 1e-12
    h = 1e-5
    for which, key in ((0, "grad_proj_start"), (1, "grad_proj_end")):
        for idx in np.ndindex(L, 2):
            e = np.zeros((L, 2))
            e[idx] = h
            up = [proj[0], proj[1]]
            dn = [proj[0], proj[1]]
            up[which] = proj[which] + e
            dn[which] = proj[which] - e
            fd = 0.8 * (pins.brute_force_nll(em, L, trans, dur, K, labels, seg, up)
                        - pins.brute_force_nll(em, L, trans, dur, K, labels, seg, dn)) / (2 * h)
            assert abs(r[key][idx] - fd) < 1e-7, (key, idx)


def _mut_proj_end_shift(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    ps, pe = proj
    return _orig(S, trans, dur, K, L, s_lo, s_hi, (ps, np.roll(pe, -1, axis=0)))   # P_end[s+k]


def _mut_proj_swap(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    return _orig(S, trans, dur, K, L, s_lo, s_hi, (proj[1], proj[0]))


def _mut_proj_drop_start(S, trans, dur, K, L, s_lo, s_hi, proj=None, _orig=osc.edge_potentials):
    return _orig(S, trans, dur, K, L, s_lo, s_hi, (np.zeros_like(proj[0]), proj[1]))


@pytest.mark.parametrize("name,fn", [
    ("end projection off by one", _mut_proj_end_shift),
    ("start and end projections swapped", _mut_proj_swap),
    ("start projection dropped", _mut_proj_drop_start),
])
def test_projection_pins_catch_planted_mistakes(monkeypatch, name, fn):
    em, L, trans, dur, K = _case(101, 6, 6, 3, 3)
    proj = _proj(102, L, 3)
    bf = pins.brute_force(em, L, trans, dur, K, proj=proj)
    monkeypatch.setattr(osc, "edge_potentials", fn)
    bad = oracle.sequence(em, L, trans, dur, K, proj=proj)
    err = max(abs(bad["logZ"] - bf["logZ"]), np.abs(bad["grad_proj_start"] - bf["start"][:L]).max(),
              np.abs(bad["grad_proj_end"] - bf["end"][1:]).max())
    assert err > 1e-3, f"pin missed planted mistake: {name}"
