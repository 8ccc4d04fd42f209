"""Long maximum durations (K up to 8000): parity with stored fp64 oracle values, and the
pages' genome-scale case T = 10^6, K = 2000 by properties that hold at any size.

Tolerances as for the rest of the path (log Z and Viterbi score 1e-5 relative; mu,
grad_em 1e-4 absolute; grad_trans, grad_dur 1e-4 relative).
"""

import os

import numpy as np
import pytest

import decode_check
import oracle
import workloads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FIXTURE = os.path.join(GOLDEN, "oracle_extreme_k.npz")
LOGZ_RTOL = 1e-5
MARG_ATOL = 1e-4
GRAD_RTOL = 1e-4


@pytest.fixture(scope="module")
def crf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import semi_markov_crf_amd
    semi_markov_crf_amd._native.load()
    return semi_markov_crf_amd


def to_dev(*arrays):
    import torch
    d = torch.device("cuda:0")
    return [torch.from_numpy(np.ascontiguousarray(a)).to(d) for a in arrays]


def np_(t):
    return t.detach().cpu().numpy()


def close_rel(gpu, ref, rtol, scale, what):
    err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    bound = rtol * np.maximum(1.0, np.abs(np.asarray(scale, np.float64)))
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}, ratio {(err / bound).max():.2f}"


def close_abs(gpu, ref, atol, what):
    err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    assert err.max() <= atol, f"{what}: max abs err {err.max():.3e} > {atol}"


def _projections(seed, B, T, C, sd):
    """The fixture script's seeded N(0, sd) projections (tests/golden/make_extreme_k_fixture.py)."""
    if sd == 0.0:
        return None, None
    rng = np.random.default_rng(seed)
    return (rng.normal(0, sd, (B, T, C)).astype(np.float32),
            rng.normal(0, sd, (B, T, C)).astype(np.float32))


@pytest.mark.parametrize("name", [f"x{i}" for i in range(1, 11)])
def test_long_durations_against_oracle(crf, name):
    if not os.path.exists(FIXTURE):
        pytest.skip(f"{FIXTURE} not generated")
    f = np.load(FIXTURE, allow_pickle=False)
    if f"{name}_case" not in f.files:
        pytest.skip(f"{name} not in {FIXTURE}")
    seed, B, T, C, K, scale, ragged, sd = f[f"{name}_case"]
    seed, B, T, C, K = int(seed), int(B), int(T), int(C), int(K)
    print(f"\n[long durations {name}: B={B} T={T} C={C} K={K} projections sd={sd}]", flush=True)
    w = workloads.make_custom(seed, B, T, C, K, em_scale=float(scale), ragged=bool(ragged))
    ps, pe = _projections(seed + 1000, B, T, C, float(sd))
    em, lengths, trans, dur = to_dev(w.em, w.lengths, w.trans, w.dur)
    kw = {}
    if ps is not None:
        tps, tpe = to_dev(ps, pe)
        kw = {"proj_start": tps, "proj_end": tpe}
    lz = np_(crf.logz(em, lengths, trans, dur, check_status=True, **kw))
    close_rel(lz, f[f"{name}_logZ"], LOGZ_RTOL, f[f"{name}_logZ"], "logz")
    out = crf.backward(em, lengths, trans, dur, want_boundaries=True, check_status=True, **kw)
    close_abs(np_(out["grad_proj_start"]), f[f"{name}_grad_proj_start"], MARG_ATOL, "grad_proj_start")
    close_abs(np_(out["grad_proj_end"]), f[f"{name}_grad_proj_end"], MARG_ATOL, "grad_proj_end")
    close_abs(np_(out["boundary"]), f[f"{name}_boundary"], MARG_ATOL, "boundary")
    close_rel(np_(out["log_z"]), f[f"{name}_logZ"], LOGZ_RTOL, f[f"{name}_logZ"], "backward log_z")
    close_abs(np_(out["marginals"]), f[f"{name}_mu"], MARG_ATOL, "marginals")
    close_abs(np_(out["grad_em"]), f[f"{name}_grad_em"], MARG_ATOL, "grad_em")
    close_rel(np_(out["grad_trans"]), f[f"{name}_grad_trans"], GRAD_RTOL, f[f"{name}_grad_trans"],
              "grad_trans")
    close_rel(np_(out["grad_dur"]), f[f"{name}_grad_dur"], GRAD_RTOL, f[f"{name}_grad_dur"],
              "grad_dur")
    score, labels, seg = crf.viterbi(em, lengths, trans, dur, check_status=True, **kw)
    close_rel(np_(score), f[f"{name}_score"], LOGZ_RTOL, f[f"{name}_score"], "viterbi score")
    labels, seg = np_(labels), np_(seg)
    for b in range(B):
        L = int(w.lengths[b])
        proj = None if ps is None else (ps[b, :L], pe[b, :L])
        decode_check.check_decode(w.em[b], L, w.trans, w.dur, K, labels[b], seg[b],
                                  float(f[f"{name}_score"][b]),
                                  decode_check.fixture_path(f, b, f"{name}_"), proj)


def test_genome_scale_long_durations(crf):
    """T = 10^6, K = 2000, C = 6 (the pages' genome-scale case, EN explainer, "4. Results
    and Benchmarks"): the forward and backward sweeps agree on log Z, marginals sum to
    one, duration mass is conserved (sum_k k * grad_dur = L), boundary probabilities are
    valid, and the decoded segmentation, rescored by the oracle's O(L) definition, has the
    reported score, which is at most log Z."""
    w = workloads.long_duration()
    L = int(w.lengths[0])
    print(f"\n[genome scale: T={w.T} K={w.K} C={w.C}]", flush=True)
    em, lengths, trans, dur = to_dev(w.em, w.lengths, w.trans, w.dur)
    lz = float(np_(crf.logz(em, lengths, trans, dur, check_status=True))[0])
    out = crf.backward(em, lengths, trans, dur, want_boundaries=True, check_status=True)
    close_rel(np_(out["log_z"])[0], lz, 1e-6, lz, "backward vs forward log Z")
    mu = np_(out["marginals"])[0].astype(np.float64)
    assert np.abs(mu.sum(axis=1) - 1.0).max() < 1e-5
    assert mu.min() > -1e-6
    gd = np_(out["grad_dur"]).astype(np.float64)
    k = np.arange(1, w.K + 1)[:, None]
    assert abs((k * gd).sum() - L) < 1e-4 * L
    bnd = np_(out["boundary"])[0].astype(np.float64)
    assert abs(bnd[0] - 1.0) < 1e-5 and bnd.min() > -1e-6 and bnd.max() < 1 + 1e-5
    assert abs(bnd.sum() - gd.sum()) < 1e-4 * gd.sum()
    score, labels, seg = crf.viterbi(em, lengths, trans, dur, check_status=True)
    s = float(np_(score)[0])
    _, S = oracle.centered_prefix(w.em[0], L)
    got = oracle.segmentation_score(S, w.trans, w.dur, w.K, np_(seg)[0], np_(labels)[0])
    close_rel(got, s, LOGZ_RTOL, s, "rescored Viterbi segmentation")
    assert s <= lz + LOGZ_RTOL * abs(lz)


@pytest.mark.parametrize("case", [(77, 2, 50, 128, 30), (78, 2, 40, 100, 97)],
                         ids=["C128_K30", "C100_K97"])
def test_largest_label_counts_against_oracle(crf, case):
    """The largest label counts (64 < C <= 128: 4 lanes per label, one duration chunk of
    the posterior kernel at a time)."""
    seed, B, T, C, K = case
    print(f"\n[large label count seed={seed} B={B} T={T} C={C} K={K}]", flush=True)
    w = workloads.make_custom(seed, B, T, C, K, ragged=True)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, K)
    em, lengths, trans, dur = to_dev(w.em, w.lengths, w.trans, w.dur)
    close_rel(np_(crf.logz(em, lengths, trans, dur, check_status=True)), ref["logZ"], LOGZ_RTOL,
              ref["logZ"], "logz")
    out = crf.backward(em, lengths, trans, dur, check_status=True)
    close_abs(np_(out["marginals"]), ref["mu"], MARG_ATOL, "marginals")
    close_abs(np_(out["grad_em"]), ref["grad_em"], MARG_ATOL, "grad_em")
    close_rel(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, ref["grad_trans"], "grad_trans")
    close_rel(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, ref["grad_dur"], "grad_dur")
    score, labels, seg = crf.viterbi(em, lengths, trans, dur, check_status=True)
    close_rel(np_(score), ref["score"], LOGZ_RTOL, ref["score"], "viterbi score")
