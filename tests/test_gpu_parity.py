"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (fixed here, derived in the design doc):
  log Z, Viterbi score     |gpu - ref| <= 1e-5 * max(1, |ref|)
  marginals, grad_em       |gpu - ref| <= 1e-4
  grad_trans, grad_dur     |gpu - ref| <= 1e-4 * max(1, |ref|)   (sums over up to B*T positions)
  Viterbi segmentation     valid, rescored in fp64 by the oracle within 1e-3 of the best,
                           and equal to the oracle's path at every decision whose gap
                           exceeds 1e-4 (decode_check.py)
  node mass                |sum over labels of the unnormalised marginals - 1| <= 1e-4
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


def dev(w):
    import torch
    d = torch.device("cuda:0")
    return (torch.from_numpy(w.em).to(d), torch.from_numpy(w.lengths).to(d),
            torch.from_numpy(w.trans).to(d), torch.from_numpy(w.dur).to(d))


def np_(t):
    return t.detach().cpu().numpy()


def assert_scalar_close(gpu, ref, rtol, what):
    gpu, ref = np.asarray(gpu, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = rtol * np.maximum(1.0, np.abs(ref))
    bad = err > bound
    assert not bad.any(), f"{what}: max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"


def assert_abs_close(gpu, ref, atol, what):
    err = np.abs(np.asarray(gpu, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    assert err.max() <= atol, f"{what}: max abs err {err.max():.3e} > {atol}"


def check_viterbi(w, score, labels, seg, ref, paths=None):
    """Score within 1e-5 relative; every decode valid, its fp64 rescore within 1e-3 of the
    best, and equal to the oracle's path at every decision whose gap exceeds 1e-4."""
    assert_scalar_close(score, ref["score"], LOGZ_RTOL, "viterbi score")
    paths = paths if paths is not None else ref.get("paths")
    checked = 0
    for b in range(w.B):
        L = int(w.lengths[b])
        checked += decode_check.check_decode(w.em[b], L, w.trans, w.dur, w.K, labels[b],
                                             seg[b], float(ref["score"][b]),
                                             None if paths is None else paths[b])
    return checked


SMALL = [
    # seed, B, T, C, K, em_scale, ragged
    (1, 3, 40, 4, 6, 1.0, True),
    (2, 2, 17, 3, 20, 2.0, True),       # K > T
    (3, 4, 65, 5, 1, 1.0, True),        # K = 1: linear chain
    (4, 2, 30, 1, 7, 1.0, True),        # C = 1
    (5, 5, 9, 6, 4, 1.0, True),         # many length-1..9 sequences
    (6, 2, 300, 6, 40, 3.0, True),      # several S chunks, rebases, ragged tail
    (7, 2, 150, 39, 30, 1.0, True),     # speech-like label count (8 lanes per label)
    (8, 2, 70, 64, 64, 1.0, False),     # large label set, NT = 1024
    (9, 1, 1, 3, 5, 1.0, False),        # L = T = 1
    (10, 3, 129, 20, 70, 1.0, True),    # 8 lanes per label, K not a multiple of 8
    (11, 2, 220, 12, 50, 1.5, True),    # 9..16 labels: 16 bulk lanes per label
    (12, 2, 160, 16, 9, 1.0, True),     # 16 labels, one bulk duration (k = 8, 9)
    (13, 2, 400, 8, 150, 2.0, True),    # 32 bulk lanes per label, many ring rescales
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_small_cases_against_oracle(crf, case):
    import torch
    seed, B, T, C, K, scale, ragged = case
    w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=ragged)
    em, lengths, trans, dur = dev(w)
    g = np.random.default_rng(seed).uniform(0.5, 1.5, B).astype(np.float32)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, grad_log_z=g)

    lz = crf.logz(em, lengths, trans, dur, check_status=True)
    assert_scalar_close(np_(lz), ref["logZ"], LOGZ_RTOL, "logz")

    out = crf.backward(em, lengths, trans, dur, grad_log_z=torch.from_numpy(g).cuda(),
                       want_node_mass=True, check_status=True)
    assert_scalar_close(np_(out["log_z"]), ref["logZ"], LOGZ_RTOL, "backward log_z")
    nm = np_(out["node_mass"])
    for b in range(B):
        L = int(w.lengths[b])
        assert np.abs(nm[b, :L] - 1.0).max() <= 1e-4 and np.all(nm[b, L:] == 0)
    assert_abs_close(np_(out["marginals"]), ref["mu"], MARG_ATOL, "marginals")
    assert_abs_close(np_(out["grad_em"]), ref["grad_em"], MARG_ATOL, "grad_em")
    assert_scalar_close(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, "grad_trans")
    assert_scalar_close(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, "grad_dur")

    score, labels, seg = crf.viterbi(em, lengths, trans, dur, check_status=True)
    check_viterbi(w, np_(score), np_(labels), np_(seg), ref)


def test_checkpoint_interval_invariance_and_determinism(crf):
    w = workloads.make_custom(21, 2, 400, 6, 30, em_scale=2.0, ragged=True)
    em, lengths, trans, dur = dev(w)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K, want_viterbi=False)
    lz = np_(crf.logz(em, lengths, trans, dur))
    outs = {}
    for delta in (0, 1, 7, 30, 64, 399, 400):
        o = crf.backward(em, lengths, trans, dur, delta=delta)
        outs[delta] = {k: np_(v) for k, v in o.items()}
        # log Z of the backward call comes from the restored last span: equal to the
        # full sweep's up to rounding
        assert_scalar_close(outs[delta]["log_z"], lz, 1e-6, f"log_z delta={delta}")
        assert_abs_close(outs[delta]["marginals"], ref["mu"], MARG_ATOL, f"marginals delta={delta}")
        assert_abs_close(outs[delta]["grad_em"], ref["grad_em"], MARG_ATOL, f"grad_em delta={delta}")
        assert_scalar_close(outs[delta]["grad_dur"], ref["grad_dur"], GRAD_RTOL, f"dur delta={delta}")
        assert_scalar_close(outs[delta]["grad_trans"], ref["grad_trans"], GRAD_RTOL, f"tr delta={delta}")
    again = crf.backward(em, lengths, trans, dur, delta=30)
    for k in ("grad_em", "grad_trans", "grad_dur", "marginals", "log_z"):
        np.testing.assert_array_equal(np_(again[k]), outs[30][k])     # bitwise reproducible


def test_forbidden_transitions_and_durations(crf):
    """-inf entries: transitions c -> c forbidden, durations above 5 forbidden for label 0."""
    w = workloads.make_custom(31, 2, 60, 4, 8, ragged=True)
    w.trans[np.arange(4), np.arange(4)] = -np.inf
    w.dur[5:, 0] = -np.inf
    em, lengths, trans, dur = dev(w)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K)
    assert_scalar_close(np_(crf.logz(em, lengths, trans, dur)), ref["logZ"], LOGZ_RTOL, "logz")
    out = crf.backward(em, lengths, trans, dur)
    assert_abs_close(np_(out["marginals"]), ref["mu"], MARG_ATOL, "marginals")
    assert_scalar_close(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, "grad_trans")
    assert_scalar_close(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, "grad_dur")
    score, labels, seg = crf.viterbi(em, lengths, trans, dur)
    check_viterbi(w, np_(score), np_(labels), np_(seg), ref)


@pytest.mark.parametrize("big", [False, True], ids=["forbidden", "large_transition"])
def test_wide_label_transitions(crf, big):
    """More than 16 labels (the register-blocked transition step): self-transitions
    forbidden, and with `big` one transition weight of 70 (2^101 in base 2), which makes
    the blocked transition posteriors leave the fp32 range, so the exact per-term sum
    serves those tiles.  The raw node mass is held to 1e-4 without the large weight; with
    it (log Z about 3,000, one transition dominating every path) the streamed fp32 sums
    drift up to 1.6e-4 from 1, the same with the per-term transition step, so it is held to
    5e-4 there; the normalised marginals stay within 1e-11 of the oracle."""
    w = workloads.make_custom(33, 2, 90, 24, 12, ragged=True)
    w.trans[np.arange(24), np.arange(24)] = -np.inf
    if big:
        w.trans[0, 1] = 70.0
    print(f"\n[wide labels: C={w.C} K={w.K} big={big}]", flush=True)
    em, lengths, trans, dur = dev(w)
    ref = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K)
    assert_scalar_close(np_(crf.logz(em, lengths, trans, dur)), ref["logZ"], LOGZ_RTOL, "logz")
    out = crf.backward(em, lengths, trans, dur, want_node_mass=True, check_status=True)
    nm = np_(out["node_mass"])[w.lengths[:, None] > np.arange(w.T)]
    assert np.abs(nm - 1.0).max() <= (5e-4 if big else 1e-4)
    assert_abs_close(np_(out["marginals"]), ref["mu"], MARG_ATOL, "marginals")
    assert_abs_close(np_(out["grad_em"]), ref["grad_em"], MARG_ATOL, "grad_em")
    assert_scalar_close(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, "grad_trans")
    assert_scalar_close(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, "grad_dur")
    score, labels, seg = crf.viterbi(em, lengths, trans, dur)
    check_viterbi(w, np_(score), np_(labels), np_(seg), ref)


def test_invalid_length_is_flagged(crf):
    import torch
    w = workloads.make_custom(41, 3, 20, 3, 4, ragged=False)
    em, lengths, trans, dur = dev(w)
    bad = torch.tensor([20, 0, 21], dtype=torch.int32, device=em.device)
    lz = crf.logz(em, bad, trans, dur)
    ws = torch.empty(crf.workspace_bytes(crf.OP_LOGZ, 3, 20, 3, 4), dtype=torch.uint8,
                     device=em.device)
    lz = crf.logz(em, bad, trans, dur, workspace=ws)
    assert crf.read_status(ws) == 1
    v = np_(lz)
    assert np.isfinite(v[0]) and np.isnan(v[1]) and np.isnan(v[2])
    crf.logz(em, lengths, trans, dur, workspace=ws)
    assert crf.read_status(ws) == 0


def test_autograd_matches_backward(crf):
    import torch
    w = workloads.make_custom(51, 2, 50, 5, 10, ragged=True)
    em, lengths, trans, dur = dev(w)
    em.requires_grad_(True); trans.requires_grad_(True); dur.requires_grad_(True)
    lz = crf.log_partition(em, lengths, trans, dur)
    wts = torch.tensor([0.3, -1.7], device=em.device)
    (lz * wts).sum().backward()
    out = crf.backward(em.detach(), lengths, trans.detach(), dur.detach(), grad_log_z=wts)
    np.testing.assert_allclose(np_(em.grad), np_(out["grad_em"]), atol=1e-6)
    np.testing.assert_allclose(np_(trans.grad), np_(out["grad_trans"]), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(np_(dur.grad), np_(out["grad_dur"]), rtol=1e-6, atol=1e-6)


# --------------------------------------------------------------------------- the five configs


def _fixture(i):
    path = os.path.join(GOLDEN, f"oracle_cfg{i}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return dict(np.load(path, allow_pickle=False))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_config_against_oracle_fixture(crf, cfg):
    ref = _fixture(cfg)
    if "win_pos" not in ref:
        pytest.skip("fixture written by an older script")
    w = workloads.make(cfg)
    em, lengths, trans, dur = dev(w)
    print(f"\n[config {cfg}: {w.name} B={w.B} T={w.T} C={w.C} K={w.K}]", flush=True)
    lz = np_(crf.logz(em, lengths, trans, dur, check_status=True))
    assert_scalar_close(lz, ref["logZ"], LOGZ_RTOL, "logz")
    out = crf.backward(em, lengths, trans, dur, want_node_mass=True, check_status=True)
    assert_scalar_close(np_(out["log_z"]), ref["logZ"], LOGZ_RTOL, "backward log_z")
    mu, ge, nm = np_(out["marginals"]), np_(out["grad_em"]), np_(out["node_mass"])
    # every position of the sequences stored in full
    for i, b in enumerate(ref["full_seqs"]):
        assert_abs_close(mu[b], ref["mu_full"][i], MARG_ATOL, f"marginals of sequence {b}")
        assert_abs_close(ge[b], ref["grad_em_full"][i], MARG_ATOL, f"grad_em of sequence {b}")
    # contiguous windows around every checkpoint seam of both sweep directions and the
    # first and last 2K positions of the other sequences (the seams of the interval the
    # backward above took by default)
    if "seam_interval" in ref:
        assert crf.default_interval(crf.OP_BACKWARD, w.B, w.T, w.C, w.K) == \
            int(ref["seam_interval"]), "the fixture's windows are not on the backward's seams"
    off, pos = ref["win_off"], ref["win_pos"]
    for b in range(w.B):
        p = pos[off[b]:off[b + 1]]
        if len(p):
            assert_abs_close(mu[b, p], ref["mu_win"][off[b]:off[b + 1]], MARG_ATOL,
                             f"marginals, seam windows of sequence {b}")
            assert_abs_close(ge[b, p], ref["grad_em_win"][off[b]:off[b + 1]], MARG_ATOL,
                             f"grad_em, seam windows of sequence {b}")
    assert_scalar_close(np_(out["grad_trans"]), ref["grad_trans"], GRAD_RTOL, "grad_trans")
    assert_scalar_close(np_(out["grad_dur"]), ref["grad_dur"], GRAD_RTOL, "grad_dur")
    # the marginals before normalisation sum to 1 over labels at every position (the
    # pages' self-consistency check, EN explainer "4. Results and Benchmarks"), and mass
    # is conserved
    for b in range(w.B):
        L = int(w.lengths[b])
        assert np.all(nm[b, L:] == 0)
        assert mu[b, :L].min() > -1e-6 and np.all(mu[b, L:] == 0)
        assert np.abs(ge[b, :L].sum(axis=0)).max() < 1e-3 * max(1, L / 1000)
    k = np.arange(1, w.K + 1)[:, None]
    total = float(w.lengths.astype(np.int64).sum())
    assert abs((k * np_(out["grad_dur"]).astype(np.float64)).sum() - total) < 1e-4 * total
    score, labels, seg = crf.viterbi(em, lengths, trans, dur, check_status=True)
    paths = [decode_check.fixture_path(ref, b) for b in range(w.B)]
    n = check_viterbi(w, np_(score), np_(labels), np_(seg), ref, paths)
    print(f"Viterbi: {n} unique decisions of the oracle's paths compared", flush=True)
    drift = [float(np.abs(nm[b, :int(w.lengths[b])].astype(np.float64) - 1.0).max())
             for b in range(w.B)]
    L0 = int(w.lengths[0])
    print("node mass - 1 of sequence 0 at t = 0, L/4, L/2, 3L/4, L-1:",
          [float(nm[0, t]) - 1.0 for t in (0, L0 // 4, L0 // 2, 3 * L0 // 4, L0 - 1)], flush=True)
    print(f"max |node mass - 1| per sequence: {np.array(drift)}", flush=True)
    assert max(drift) <= 1e-4


# label counts 1..8 take the rows-per-lane kernels (odd T: a partial last lane, lengths
# inside the last tile), 39 and 64 the column kernels
SCAN_CUSTOM = {"ragged": (61, 5, 3000, 7), "c1_odd": (62, 3, 2051, 1), "c3_odd": (63, 4, 1027, 3),
               "c8_odd": (64, 2, 4093, 8), "c5_short": (65, 3, 5, 5), "c64": (66, 2, 777, 64)}


@pytest.mark.parametrize("cfg_or_case", ["tiny", "speech", "long"] + list(SCAN_CUSTOM))
def test_prefix_scan_against_oracle(crf, cfg_or_case):
    """Centring + prefix sums (fp64 on both sides): |gpu - ref| <= 1e-9 * max(1, |ref|)."""
    if cfg_or_case in SCAN_CUSTOM:
        seed, B, T, C = SCAN_CUSTOM[cfg_or_case]
        w = workloads.make_custom(seed, B, T, C, 3, em_scale=3.0, ragged=True)
    else:
        w = workloads.make({"tiny": 0, "speech": 1, "long": 3}[cfg_or_case])
    em, lengths, _, _ = dev(w)
    S = np_(crf.prefix(em, lengths, check_status=True))
    assert S.shape == (w.B, w.T + 1, w.C)
    for b in range(w.B):
        L = int(w.lengths[b])
        _, ref = oracle.centered_prefix(w.em[b], L)
        err = np.abs(S[b, :L + 1] - ref) / np.maximum(1.0, np.abs(ref))
        assert err.max() <= 1e-9, (b, err.max())
        flat = np.abs(S[b, L + 1:] - S[b, L]) / np.maximum(1.0, np.abs(S[b, L]))
        assert flat.size == 0 or flat.max() <= 1e-9      # flat beyond the length
        assert np.abs(S[b, L]).max() < 1e-9 * max(1, L)  # centred: S[L] = 0


def test_long_genomic_peak_device_memory(crf):
    """The long genomic configuration (B=1, T=10^6, K=200, C=6) streams: the backward pass
    and the Viterbi decode together allocate well under 1 GB of device memory, where the
    dense edge tensor alone would take T*K*C^2*4 B = 28.8 GB (about 29 GB in the EN
    explainer, "1. Problem Statement")."""
    import torch
    w = workloads.make(3)
    print(f"\n[peak memory: {w.name} B={w.B} T={w.T} C={w.C} K={w.K}]", flush=True)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    em, lengths, trans, dur = dev(w)
    out = crf.backward(em, lengths, trans, dur, check_status=True)
    score, labels, seg = crf.viterbi(em, lengths, trans, dur, check_status=True)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    dense = w.T * w.K * w.C * w.C * 4
    print(f"peak device memory {peak / 2**20:.1f} MiB (inputs, outputs and workspaces); "
          f"dense edge tensor {dense / 1e9:.1f} GB", flush=True)
    assert np.isfinite(np_(out["log_z"])).all() and np.isfinite(np_(score)).all()
    assert peak < 1 << 30
    assert dense > 25 * peak
