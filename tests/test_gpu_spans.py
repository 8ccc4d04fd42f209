"""The checkpoint spans swept at once against the in-order sweeps and the oracle.

Every span of delta positions starts a burn-in of 3K positions early from a uniform ring;
a seam check at each checkpoint proves that the two spans' states agree up to a constant
(within seam_tolerance) and the sequence is swept again in order from the first seam that
does not.  A negative seam_tolerance accepts no seam: that is the in-order sweep, used here
as a reference beside the oracle.  Tolerances as in test_gpu_parity.py.
"""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

LOGZ_RTOL, MARG_ATOL, GRAD_RTOL = 1e-5, 1e-4, 1e-4


@pytest.fixture(scope="module")
def crf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import semi_markov_crf_amd
    semi_markov_crf_amd._native.load()
    return semi_markov_crf_amd


def dev(w):
    import torch
    d = torch.device("cuda:0")
    return (torch.from_numpy(w.em).to(d), torch.from_numpy(w.lengths).to(d),
            torch.from_numpy(w.trans).to(d), torch.from_numpy(w.dur).to(d))


def np_(t):
    return t.detach().cpu().numpy()


def close_rel(got, ref, rtol, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() <= rtol, f"{what}: rel err {err.max():.3e}"


def close_abs(got, ref, atol, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert err.max() <= atol, f"{what}: abs err {err.max():.3e}"


CASES = [
    # seed, B, T, C, K, em_scale, delta
    (201, 3, 2000, 6, 20, 1.5, 0),       # many spans, ragged
    (202, 2, 3000, 4, 40, 1.0, 250),     # 64 lanes per label
    (203, 2, 1500, 16, 12, 1.0, 100),    # 16 labels
    (204, 2, 2500, 8, 150, 2.0, 0),      # 32 lanes per label, long burn-in
    (205, 3, 700, 5, 6, 1.0, 7),         # spans shorter than the burn-in
    (206, 2, 1200, 24, 10, 1.0, 90),     # 24 labels: one barrier per position
    (207, 2, 1000, 40, 16, 1.0, 0),      # 40 labels
    (208, 2, 600, 64, 8, 1.5, 50),       # 64 labels, 4 lanes per label
    (209, 1, 6000, 3, 1030, 1.5, 1500),  # long durations: burn-in of 3K from a uniform ring
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_spans_at_once_match_in_order_sweeps_and_oracle(crf, case):
    seed, B, T, C, K, scale, delta = case
    w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=True, min_len=T // 3)
    em, lengths, trans, dur = dev(w)
    print(f"\n[spans seed={seed} B={B} T={T} C={C} K={K} delta={delta}]", flush=True)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, want_viterbi=False)
    lz, bound, rep = crf.logz(em, lengths, trans, dur, delta=delta, want_seams=True,
                              check_status=True)
    close_rel(np_(lz), ref["logZ"], LOGZ_RTOL, "logz")
    assert np.all(np_(rep) == 0), np_(rep)
    lz_seq, _, rep_seq = crf.logz(em, lengths, trans, dur, delta=delta, seam_tolerance=-1.0,
                                  want_seams=True)
    close_rel(np_(lz_seq), ref["logZ"], LOGZ_RTOL, "logz (in order)")
    D = crf.checkpoint_interval(T, K, delta)
    many = np.asarray(w.lengths) > D                    # sequences with a seam
    np.testing.assert_array_equal(np_(rep_seq), many.astype(np.int32))

    out = crf.backward(em, lengths, trans, dur, delta=delta, want_seams=True,
                       want_node_mass=True, check_status=True)
    seq = crf.backward(em, lengths, trans, dur, delta=delta, seam_tolerance=-1.0,
                       want_seams=True)
    assert np.all(np_(out["seam_repairs"]) == 0)
    np.testing.assert_array_equal(np_(seq["seam_repairs"]), 2 * many.astype(np.int32))
    b = np_(out["seam_bound"])
    print(f"seam bound per sequence {b}", flush=True)
    assert np.all(b >= 0) and np.all(b <= 1e-4 * 2 * np.ceil(np.asarray(w.lengths) / D))
    for o, what in ((out, "at once"), (seq, "in order")):
        close_rel(np_(o["log_z"]), ref["logZ"], LOGZ_RTOL, f"backward log_z {what}")
        close_abs(np_(o["marginals"]), ref["mu"], MARG_ATOL, f"marginals {what}")
        close_abs(np_(o["grad_em"]), ref["grad_em"], MARG_ATOL, f"grad_em {what}")
        close_rel(np_(o["grad_trans"]), ref["grad_trans"], GRAD_RTOL, f"grad_trans {what}")
        close_rel(np_(o["grad_dur"]), ref["grad_dur"], GRAD_RTOL, f"grad_dur {what}")
    nm = np_(out["node_mass"])
    for i in range(B):
        L = int(w.lengths[i])
        print(f"node mass deviation {np.abs(nm[i, :L] - 1.0).max():.2e}", flush=True)
        assert np.abs(nm[i, :L] - 1.0).max() <= 1e-4
    # the two agree far closer than the oracle tolerance
    close_abs(np_(out["marginals"]), np_(seq["marginals"]), 1e-5, "at once vs in order")


def test_seams_that_cannot_converge_are_repaired(crf):
    """Only segments of length exactly K: the forward values live on one residue class of
    the position mod K, which a uniform start never reaches, so every seam fails and each
    sequence is swept in order from its first seam; the results still match the oracle."""
    K, C = 5, 3
    w = workloads.make_custom(211, 2, 600, C, K, em_scale=1.0, ragged=False)
    w.dur[:K - 1] = -np.inf
    em, lengths, trans, dur = dev(w)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, want_viterbi=False)
    lz, _, rep = crf.logz(em, lengths, trans, dur, delta=50, want_seams=True, check_status=True)
    close_rel(np_(lz), ref["logZ"], LOGZ_RTOL, "logz")
    assert np.all(np_(rep) == 1)
    out = crf.backward(em, lengths, trans, dur, delta=50, want_seams=True, check_status=True)
    assert np.all(np_(out["seam_repairs"]) == 2)
    close_rel(np_(out["log_z"]), ref["logZ"], LOGZ_RTOL, "backward log_z")
    close_abs(np_(out["marginals"]), ref["mu"], MARG_ATOL, "marginals")
    close_rel(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, "grad_dur")
    close_rel(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, "grad_trans")


VIT_CASES = [
    # seed, B, T, C, K, em_scale
    (221, 3, 3000, 6, 40, 2.0),
    (222, 2, 4000, 4, 100, 1.5),
    (223, 2, 2000, 16, 20, 1.0),
    (224, 2, 1500, 24, 16, 1.5),
    (225, 2, 1000, 64, 8, 1.5),
    (226, 1, 5000, 3, 1030, 2.0),        # long durations
]


@pytest.mark.parametrize("case", VIT_CASES, ids=[f"s{c[0]}" for c in VIT_CASES])
def test_decode_over_spans_matches_oracle_decisions(crf, case):
    """The forward max-plus sweep over spans at once: the score, and every decision of the
    oracle's path whose gap exceeds 1e-4, are those of the in-order sweep and the oracle."""
    import decode_check
    seed, B, T, C, K, scale = case
    w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=True, min_len=T // 2)
    em, lengths, trans, dur = dev(w)
    print(f"\n[decode over spans seed={seed} B={B} T={T} C={C} K={K}]", flush=True)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, want_grads=False)
    score, labels, seg, bound, rep = crf.viterbi(em, lengths, trans, dur, want_seams=True,
                                                 check_status=True)
    s2, l2, g2, _, rep2 = crf.viterbi(em, lengths, trans, dur, seam_tolerance=-1.0,
                                      want_seams=True, check_status=True)
    D = crf.default_interval(crf.OP_VITERBI, B, T, C, K)
    assert np.all(np_(rep) == 0)
    np.testing.assert_array_equal(np_(rep2), (np.asarray(w.lengths) > D).astype(np.int32))
    print(f"seam bound {np_(bound)}", flush=True)
    for sc, lab, sg, what in ((score, labels, seg, "at once"), (s2, l2, g2, "in order")):
        close_rel(np_(sc), ref["score"], LOGZ_RTOL, f"score {what}")
        lab, sg = np_(lab), np_(sg)
        n = 0
        for b in range(B):
            L = int(w.lengths[b])
            n += decode_check.check_decode(w.em[b], L, w.trans, w.dur, K, lab[b], sg[b],
                                           float(ref["score"][b]), ref["paths"][b])
        print(f"{what}: {n} unique decisions compared", flush=True)
        assert n > 0
