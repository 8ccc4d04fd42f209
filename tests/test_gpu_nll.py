"""Parity of the gold-segmentation training loss (semicrf_nll, through the C ABI) with the
fp64 oracle.

Tolerances: nll = log Z - score carries the error of log Z, so
  nll                      |gpu - ref| <= 1e-5 * max(1, |log Z|)
  grad_em                  |gpu - ref| <= 1e-4
  grad_trans, grad_dur     |gpu - ref| <= 1e-4 * max(1, |ref|)
(the gold half of the gradients is integer counts, exact on both sides).
"""

import os

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
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


CASES = [
    # seed, B, T, C, K, em_scale
    (1, 3, 40, 4, 6, 1.0),
    (2, 2, 17, 3, 20, 2.0),      # K > T
    (3, 4, 65, 5, 1, 1.0),       # K = 1: every segment has length 1
    (4, 2, 30, 1, 7, 1.0),       # C = 1
    (6, 2, 300, 6, 40, 3.0),     # several tiles of the segment kernel, ragged tail
    (7, 2, 150, 39, 30, 1.0),    # speech-like label count
    (13, 2, 400, 8, 150, 2.0),   # long segments
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}" for c in CASES])
def test_nll_against_oracle(crf, case):
    import torch
    seed, B, T, C, K, scale = case
    print(f"\n[nll case seed={seed} B={B} T={T} C={C} K={K}]", flush=True)
    w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=True)
    labels, seg = workloads.gold_segmentation(seed + 100, w.lengths, T, C, K)
    g = np.random.default_rng(seed).uniform(0.5, 1.5, B).astype(np.float32)
    ref = oracle.nll_batch(w.em, w.lengths, w.trans, w.dur, K, labels, seg, grad_nll=g)
    em, lengths, trans, dur, lab, st, gd = to_dev(w.em, w.lengths, w.trans, w.dur, labels, seg, g)
    out = crf.nll(em, lengths, trans, dur, lab, st, grad_nll=gd, check_status=True)
    close_rel(np_(out["nll"]), ref["nll"], LOGZ_RTOL, ref["logZ"], "nll")
    assert np.all(np_(out["nll"]) > -LOGZ_RTOL * np.maximum(1, np.abs(ref["logZ"])))
    close_abs(np_(out["grad_em"]), ref["grad_em"], MARG_ATOL, "grad_em")
    close_rel(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, ref["grad_trans"], "grad_trans")
    close_rel(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, ref["grad_dur"], "grad_dur")
    # default upstream gradient: all ones; bitwise reproducible
    a = crf.nll(em, lengths, trans, dur, lab, st)
    b = crf.nll(em, lengths, trans, dur, lab, st, grad_nll=torch.ones_like(gd))
    for k in a:
        np.testing.assert_array_equal(np_(a[k]), np_(b[k]))


def test_nll_of_the_viterbi_segmentation_is_smallest(crf):
    """The best segmentation has the largest score, so the smallest loss of any gold
    segmentation: nll(viterbi) <= nll(random gold), and exp(-nll) <= 1."""
    w = workloads.make_custom(71, 3, 200, 5, 12, em_scale=2.0, ragged=True)
    em, lengths, trans, dur = to_dev(w.em, w.lengths, w.trans, w.dur)
    _, vlab, vseg = crf.viterbi(em, lengths, trans, dur)
    best = np_(crf.nll(em, lengths, trans, dur, vlab.int(), vseg.to(em.device))["nll"])
    labels, seg = workloads.gold_segmentation(72, w.lengths, w.T, w.C, w.K)
    lab, st = to_dev(labels, seg)
    rnd = np_(crf.nll(em, lengths, trans, dur, lab, st)["nll"])
    assert np.all(best >= -1e-4) and np.all(best <= rnd + 1e-4)


def test_invalid_gold_is_flagged(crf):
    """Too long a segment, a label change inside a segment, no start at t = 0 or a
    label out of range: NaN for that sequence, status flag, and its gold counts left out
    of the gradients (which then equal the log Z gradients for it)."""
    import torch
    B, T, C, K = 5, 24, 3, 4
    w = workloads.make_custom(81, B, T, C, K, ragged=False)
    labels, seg = workloads.gold_segmentation(82, w.lengths, T, C, K)
    labels[1, :6] = 2; seg[1, :6] = 0; seg[1, 0] = 1; seg[1, 6] = 1   # segment of 6 > K
    seg[2, 0] = 0                                                       # no start at 0
    labels[3, 5] = C                                                    # label out of range
    seg[4, :3] = (1, 0, 1); labels[4, :2] = (0, 1)                     # change inside
    em, lengths, trans, dur, lab, st = to_dev(w.em, w.lengths, w.trans, w.dur, labels, seg)
    ws = torch.empty(crf.workspace_bytes(crf.OP_BACKWARD, B, T, C, K), dtype=torch.uint8,
                     device=em.device)
    out = crf.nll(em, lengths, trans, dur, lab, st, workspace=ws)
    assert crf.read_status(ws) == 1
    v = np_(out["nll"])
    assert np.isfinite(v[0]) and np.all(np.isnan(v[1:]))
    bw = crf.backward(em, lengths, trans, dur)
    ref0 = oracle.nll_batch(w.em[:1], w.lengths[:1], w.trans, w.dur, K, labels[:1], seg[:1])
    ge = np_(out["grad_em"])
    close_abs(ge[0], ref0["grad_em"][0], MARG_ATOL, "grad_em of the valid sequence")
    np.testing.assert_array_equal(ge[1:], np_(bw["grad_em"])[1:])
    _, _, tc = oracle.gold_features(labels[0], seg[0], T, K, C)
    close_rel(np_(out["grad_trans"]), np_(bw["grad_trans"]).astype(np.float64) - tc, GRAD_RTOL,
              tc + 1, "grad_trans")
    # a valid call on the same workspace clears the flag
    crf.nll(em, lengths, trans, dur, lab[:1].expand(B, T).contiguous(),
            st[:1].expand(B, T).contiguous(), workspace=ws)
    assert crf.read_status(ws) == 0


def _fixture(i):
    path = os.path.join(GOLDEN, f"oracle_cfg{i}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return dict(np.load(path, allow_pickle=False))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_nll_at_config_size(crf, cfg):
    """Full configuration sizes: log Z and the log Z gradients come from the stored oracle
    fixture (the same values the backward pass is checked against), the gold score and
    the gold feature counts from the oracle's O(L) definitions."""
    ref = _fixture(cfg)
    if "win_pos" not in ref:
        pytest.skip("fixture written by an older script")
    w = workloads.make(cfg)
    print(f"\n[nll config {cfg}: {w.name} B={w.B} T={w.T} C={w.C} K={w.K}]", flush=True)
    labels, seg = workloads.gold_segmentation(2000 + cfg, w.lengths, w.T, w.C, w.K)
    em, lengths, trans, dur, lab, st = to_dev(w.em, w.lengths, w.trans, w.dur, labels, seg)
    out = crf.nll(em, lengths, trans, dur, lab, st, check_status=True)
    nll, ge = np_(out["nll"]), np_(out["grad_em"])
    tcount = np.zeros((w.C, w.C))
    dcount = np.zeros((w.K, w.C))
    for b in range(w.B):
        L = int(w.lengths[b])
        _, S = oracle.centered_prefix(w.em[b], L)
        score = oracle.segmentation_score(S, w.trans, w.dur, w.K, seg[b, :L], labels[b, :L])
        close_rel(nll[b], ref["logZ"][b] - score, LOGZ_RTOL, ref["logZ"][b], f"nll[{b}]")
        ind, dc, tc = oracle.gold_features(labels[b, :L], seg[b, :L], L, w.K, w.C)
        tcount += tc
        dcount += dc
        gold = ind - ind.mean(axis=0, keepdims=True)
        full = list(ref["full_seqs"])
        if b in full:
            close_abs(ge[b, :L], ref["grad_em_full"][full.index(b)][:L] - gold, MARG_ATOL,
                      f"grad_em[{b}]")
        else:
            o0, o1 = ref["win_off"][b], ref["win_off"][b + 1]
            pos = ref["win_pos"][o0:o1]
            close_abs(ge[b, pos], ref["grad_em_win"][o0:o1] - gold[pos], MARG_ATOL,
                      f"grad_em[{b}] (seam windows)")
    close_rel(np_(out["grad_trans"]), ref["grad_trans"] - tcount, GRAD_RTOL, ref["grad_trans"],
              "grad_trans")
    close_rel(np_(out["grad_dur"]), ref["grad_dur"] - dcount, GRAD_RTOL, ref["grad_dur"],
              "grad_dur")
