"""Parity of the boundary projections and boundary probabilities (through the C ABI) with
the fp64 oracle.

Tolerances as for the rest of the path:
  log Z, Viterbi score, nll          |gpu - ref| <= 1e-5 * max(1, |log Z|)
  marginals, grad_em, start / end
  marginals, boundary probability    |gpu - ref| <= 1e-4
  grad_trans, grad_dur               |gpu - ref| <= 1e-4 * max(1, |ref|)
"""

import os

import numpy as np
import pytest

import decode_check
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


def projections(seed, B, T, C, sd):
    """Seeded N(0, sd) boundary projections [B, T, C] (start, end), float32."""
    rng = np.random.default_rng(seed)
    return (rng.normal(0, sd, (B, T, C)).astype(np.float32),
            rng.normal(0, sd, (B, T, C)).astype(np.float32))


CASES = [
    # seed, B, T, C, K, em_scale, proj sd
    (1, 3, 40, 4, 6, 1.0, 0.8),
    (2, 2, 17, 3, 20, 2.0, 1.0),      # K > T
    (3, 4, 65, 5, 1, 1.0, 0.8),       # K = 1
    (4, 2, 30, 1, 7, 1.0, 0.8),       # C = 1
    (6, 2, 300, 6, 40, 3.0, 2.0),     # several S chunks, rebases, ragged tail
    (7, 2, 150, 39, 30, 1.0, 0.8),    # label count of the generic (C > 16) kernels
    (8, 2, 70, 64, 64, 1.0, 0.5),     # large label set
    (11, 2, 220, 12, 50, 1.5, 1.0),   # 16 bulk lanes per label
    (13, 2, 400, 8, 150, 2.0, 1.5),   # 32 bulk lanes per label, long segments
    (14, 2, 260, 6, 30, 1.0, 12.0),   # projections large enough to leave the linear range
]


@pytest.mark.parametrize("case", CASES, ids=[f"p{c[0]}" for c in CASES])
def test_projections_against_oracle(crf, case):
    import torch
    seed, B, T, C, K, scale, sd = case
    print(f"\n[projection case seed={seed} B={B} T={T} C={C} K={K} sd={sd}]", flush=True)
    w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=True)
    ps, pe = projections(seed + 300, B, T, C, sd)
    g = np.random.default_rng(seed).uniform(0.5, 1.5, B).astype(np.float32)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, grad_log_z=g, proj_start=ps,
                       proj_end=pe)
    em, lengths, trans, dur, tps, tpe, gd = to_dev(w.em, w.lengths, w.trans, w.dur, ps, pe, g)

    lz = crf.logz(em, lengths, trans, dur, proj_start=tps, proj_end=tpe, check_status=True)
    close_rel(np_(lz), ref["logZ"], LOGZ_RTOL, ref["logZ"], "logz")

    out = crf.backward(em, lengths, trans, dur, proj_start=tps, proj_end=tpe, grad_log_z=gd,
                       check_status=True)
    close_rel(np_(out["log_z"]), ref["logZ"], LOGZ_RTOL, ref["logZ"], "backward log_z")
    close_abs(np_(out["marginals"]), ref["mu"], MARG_ATOL, "marginals")
    close_abs(np_(out["grad_em"]), ref["grad_em"], MARG_ATOL, "grad_em")
    close_rel(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, ref["grad_trans"], "grad_trans")
    close_rel(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, ref["grad_dur"], "grad_dur")
    close_abs(np_(out["grad_proj_start"]), ref["grad_proj_start"], MARG_ATOL, "grad_proj_start")
    close_abs(np_(out["grad_proj_end"]), ref["grad_proj_end"], MARG_ATOL, "grad_proj_end")
    close_abs(np_(out["boundary"]), ref["boundary"], MARG_ATOL, "boundary")

    score, labels, seg = crf.viterbi(em, lengths, trans, dur, proj_start=tps, proj_end=tpe,
                                     check_status=True)
    close_rel(np_(score), ref["score"], LOGZ_RTOL, ref["score"], "viterbi score")
    labels, seg = np_(labels), np_(seg)
    for b in range(B):
        L = int(w.lengths[b])
        decode_check.check_decode(w.em[b], L, w.trans, w.dur, K, labels[b], seg[b],
                                  float(ref["score"][b]), ref["paths"][b],
                                  (ps[b, :L], pe[b, :L]))

    # the training loss with projections
    glab, gseg = workloads.gold_segmentation(seed + 400, w.lengths, T, C, K)
    nref = oracle.nll_batch(w.em, w.lengths, w.trans, w.dur, K, glab, gseg, grad_nll=g,
                            proj_start=ps, proj_end=pe)
    tl, tg = to_dev(glab, gseg)
    n = crf.nll(em, lengths, trans, dur, tl, tg, proj_start=tps, proj_end=tpe, grad_nll=gd,
                check_status=True)
    close_rel(np_(n["nll"]), nref["nll"], LOGZ_RTOL, nref["logZ"], "nll")
    close_abs(np_(n["grad_em"]), nref["grad_em"], MARG_ATOL, "nll grad_em")
    close_rel(np_(n["grad_trans"]), nref["grad_trans"], GRAD_RTOL, ref["grad_trans"],
              "nll grad_trans")
    close_rel(np_(n["grad_dur"]), nref["grad_dur"], GRAD_RTOL, ref["grad_dur"], "nll grad_dur")
    close_abs(np_(n["grad_proj_start"]), nref["grad_proj_start"], MARG_ATOL, "nll grad_proj_start")
    close_abs(np_(n["grad_proj_end"]), nref["grad_proj_end"], MARG_ATOL, "nll grad_proj_end")
    del torch


def test_one_projection_alone_and_zero_projections(crf):
    """Only one of the two arrays given; all-zero arrays give the results of none."""
    import torch
    w = workloads.make_custom(51, 3, 90, 5, 12, em_scale=1.5, ragged=True)
    ps, pe = projections(52, 3, 90, 5, 1.0)
    em, lengths, trans, dur, tps, tpe = to_dev(w.em, w.lengths, w.trans, w.dur, ps, pe)
    for kw, refkw in (({"proj_start": tps}, {"proj_start": ps}),
                      ({"proj_end": tpe}, {"proj_end": pe})):
        ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K, **refkw)
        out = crf.backward(em, lengths, trans, dur, check_status=True, **kw)
        close_rel(np_(out["log_z"]), ref["logZ"], LOGZ_RTOL, ref["logZ"], f"log_z {list(kw)}")
        close_abs(np_(out["marginals"]), ref["mu"], MARG_ATOL, f"marginals {list(kw)}")
        close_abs(np_(out["boundary"]), ref["boundary"], MARG_ATOL, f"boundary {list(kw)}")
        score = np_(crf.viterbi(em, lengths, trans, dur, **kw)[0])
        close_rel(score, ref["score"], LOGZ_RTOL, ref["score"], f"viterbi {list(kw)}")
    z = torch.zeros_like(em)
    a = crf.backward(em, lengths, trans, dur, want_boundaries=True)
    b = crf.backward(em, lengths, trans, dur, proj_start=z, proj_end=z)
    for k in ("log_z", "marginals", "grad_em", "grad_trans", "grad_dur", "boundary",
              "grad_proj_start", "grad_proj_end"):
        np.testing.assert_allclose(np_(b[k]), np_(a[k]), rtol=1e-6, atol=1e-7, err_msg=k)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K)
    close_abs(np_(a["boundary"]), ref["boundary"], MARG_ATOL, "boundary without projections")


def test_autograd_with_projections(crf):
    import torch
    w = workloads.make_custom(53, 2, 50, 5, 10, ragged=True)
    ps, pe = projections(54, 2, 50, 5, 0.7)
    em, lengths, trans, dur, tps, tpe = to_dev(w.em, w.lengths, w.trans, w.dur, ps, pe)
    for t in (em, trans, dur, tps, tpe):
        t.requires_grad_(True)
    lz = crf.log_partition(em, lengths, trans, dur, tps, tpe)
    wts = torch.tensor([0.3, -1.7], device=em.device)
    (lz * wts).sum().backward()
    out = crf.backward(em.detach(), lengths, trans.detach(), dur.detach(), proj_start=tps.detach(),
                       proj_end=tpe.detach(), grad_log_z=wts)
    np.testing.assert_allclose(np_(tps.grad), np_(out["grad_proj_start"]), atol=1e-6)
    np.testing.assert_allclose(np_(tpe.grad), np_(out["grad_proj_end"]), atol=1e-6)
    np.testing.assert_allclose(np_(em.grad), np_(out["grad_em"]), atol=1e-6)


def _fixture(i):
    path = os.path.join(GOLDEN, f"oracle_cfg{i}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return dict(np.load(path, allow_pickle=False))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_boundaries_at_config_size(crf, cfg):
    """Full configuration sizes, properties that hold at any size: without projections
    the boundary probability is the start mass of the stored oracle fixture's duration
    gradient (sum over t of boundary = sum of grad_dur), 1 at t = 0 and in [0, 1]; a
    constant start projection x_c equals the duration shift dur + x_c (log Z and the
    marginals), and its gradient sums to the expected segment count of each label."""
    import torch
    ref = _fixture(cfg)
    w = workloads.make(cfg)
    print(f"\n[boundaries config {cfg}: {w.name} B={w.B} T={w.T} C={w.C} K={w.K}]", flush=True)
    em, lengths, trans, dur = to_dev(w.em, w.lengths, w.trans, w.dur)
    out = crf.backward(em, lengths, trans, dur, want_boundaries=True, check_status=True)
    bnd = np_(out["boundary"]).astype(np.float64)
    total = bnd.sum()
    assert abs(total - ref["grad_dur"].sum()) <= 1e-4 * ref["grad_dur"].sum()
    for b in range(w.B):
        L = int(w.lengths[b])
        assert abs(bnd[b, 0] - 1.0) < 1e-5
        assert bnd[b, :L].min() > -1e-6 and bnd[b, :L].max() < 1 + 1e-5
        assert np.all(bnd[b, L:] == 0)
        gpe = np_(out["grad_proj_end"][b, L - 1]).astype(np.float64)
        assert abs(gpe.sum() - 1.0) < 1e-5
    x = np.random.default_rng(cfg).normal(0, 0.5, w.C).astype(np.float32)
    xs = torch.from_numpy(np.broadcast_to(x, w.em.shape).copy()).to(em.device)
    a = crf.backward(em, lengths, trans, dur, proj_start=xs, check_status=True)
    d2 = torch.from_numpy((w.dur + x[None, :]).astype(np.float32)).to(em.device)
    c = crf.backward(em, lengths, trans, d2, check_status=True)
    la, lc = np_(a["log_z"]), np_(c["log_z"])
    close_rel(la, lc, LOGZ_RTOL, lc, "constant start projection vs duration shift")
    close_abs(np_(a["marginals"]), np_(c["marginals"]), MARG_ATOL, "marginals")
    gsum = np_(a["grad_proj_start"]).astype(np.float64).sum(axis=(0, 1))
    close_rel(gsum, np_(c["grad_dur"]).astype(np.float64).sum(axis=0), GRAD_RTOL,
              np_(c["grad_dur"]).sum(axis=0), "start gradient vs segment counts")
    sa = np_(crf.viterbi(em, lengths, trans, dur, proj_start=xs)[0])
    sc = np_(crf.viterbi(em, lengths, trans, d2)[0])
    close_rel(sa, sc, LOGZ_RTOL, sc, "viterbi with constant start projection")
