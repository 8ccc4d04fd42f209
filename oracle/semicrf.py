"""Plain fp64 semi-Markov CRF: the definition the streaming GPU path must reproduce.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Slow and obvious on
purpose: it builds the dense edge-potential tensor psi[s, k, c', c] in fp64
(tile by tile over segment start positions) and runs the textbook recursions
over it.  Nothing here is blocked, fused, factored or streamed.

What is computed, with the passage each step follows (pages titled
"Streaming Structured Inference with Flash-SemiCRF"):

* A semi-CRF labels whole segments [s, s+k) with one of C labels, 1 <= k <= K,
  and sums over every segmentation (gist.science EN explainer, "1. Problem
  Statement": segments, max duration K, labels C; the edge tensor of size
  O(T*K*C^2)).
* Emissions are centred per sequence and label by their mean nu[c] over the
  valid positions, then prefix-summed: S[0,c] = 0, S[t,c] = sum_{u<t}
  (em[u,c] - nu[c])  (EN explainer, "2. Methodology", "Emission Baseline
  Centering" and "On-the-Fly Edge Computation via Prefix Sums").
* The content score of segment [s, s+k) with label c is S[s+k,c] - S[s,c]
  (same passage).  The edge potential adds the duration score dur[k-1, c] and
  the transition score trans[c', c] from the previous segment's label c'
  (the potential is a sum of separately computed terms, EN explainer,
  "2. Methodology", "Boundary Projections", which adds further terms the same
  way).
* log Z is the log-sum-exp over all segmentations; the gradients of log Z are
  the posterior expectations of the features (exact gradients: EN explainer,
  "4. Results and Benchmarks", correctness checks).

Readings taken where the pages are silent (each is listed in the design doc):

1. No transition score into the first segment and none after the last one.
   The first segment is modelled as coming from a virtual start label whose
   transition row is all zeros; alpha of the start label is 0 at position 0
   and -inf elsewhere.  With K = 1 this is exactly a linear-chain CRF with
   no boundary transitions.
2. dur[k-1, c] scores a segment of length k (k = 1..K).
3. trans[c', c]: row = previous label, column = next label.
4. Two adjacent segments may carry the same label (trans[c, c] applies).
5. The centring mean runs over the valid positions t < L only; emissions at
   t >= L are ignored.
6. The centring is part of the function: grad_em = g * (mu - mean_t mu), where
   mu[t, c] is the posterior probability that position t lies in a segment of
   label c ("marginals"), and g the upstream gradient of log Z.
7. Viterbi ties go to the lexicographically lowest (k, c') at every node and
   to the lowest final label.  The margin is the minimum, over the decisions
   along the decoded path (including the final label), of the gap between
   the chosen value and the runner-up; it equals the score gap between the
   best and the second-best segmentation.
8. The training loss of a gold segmentation is its negative log-probability,
   log Z - score(y*); its gradient is expected minus gold feature counts.
9. Boundary projections (EN explainer, "2. Methodology", "Boundary
   Projections": separate start and end features added to the edge
   potential): P_start[t, c] scores a segment of label c that starts at t,
   P_end[t, c] one whose last position is t, so segment [s, s+k) of label c
   gains P_start[s, c] + P_end[s+k-1, c].  Both are [L, C] per sequence, not
   centred.  Their gradients are the start and end marginals; the boundary
   probability at t (EN explainer, "4. Results and Benchmarks": boundary
   probabilities checked at genome scale) is the probability that some
   segment starts at t, sum_c start[t, c].
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _lse(x: np.ndarray, axis=None) -> np.ndarray:
    """log(sum(exp(x))) along ``axis`` in fp64; -inf when every entry is -inf."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = np.log(np.sum(np.exp(x - m_safe), axis=axis, keepdims=True)) + m_safe
    if axis is None:
        return out.reshape(())
    return np.squeeze(out, axis=axis)


def centered_prefix(em_b: np.ndarray, L: int, nu: np.ndarray | None = None):
    """Centring and prefix sum for one sequence ("Emission Baseline Centering",
    "On-the-Fly Edge Computation via Prefix Sums").

    em_b: [T, C]; only rows t < L are used.  Returns (nu [C], S [L+1, C]) in
    fp64 with S[0] = 0 and S[t] = sum_{u<t} (em[u] - nu).  Passing ``nu``
    freezes the centring mean (used to isolate d logZ / d S)."""
    # Accumulated in extended precision and rounded to fp64: a sequential fp64
    # cumulative sum drifts by up to ~T * 2^-53 * max|S| (about 1e-7 at T = 1e6).
    x = np.asarray(em_b[:L], dtype=np.longdouble)
    nu_l = x.mean(axis=0) if nu is None else np.asarray(nu, dtype=np.longdouble)
    S = np.zeros((L + 1, x.shape[1]), dtype=np.float64)
    S[1:] = np.cumsum(x - nu_l[None, :], axis=0).astype(np.float64)
    return nu_l.astype(np.float64), S


def _trans_with_start(trans: np.ndarray) -> np.ndarray:
    """[C+1, C]: rows 0..C-1 are trans[c', c]; row C is the virtual start label
    with zero transition score (reading 1)."""
    trans = np.asarray(trans, dtype=np.float64)
    return np.vstack([trans, np.zeros((1, trans.shape[1]))])


def edge_potentials(S: np.ndarray, trans: np.ndarray, dur: np.ndarray, K: int, L: int,
                    s_lo: int, s_hi: int, proj=None) -> np.ndarray:
    """Dense edge potentials psi[s - s_lo, k - 1, c', c] for segment starts
    s in [s_lo, s_hi), lengths k = 1..K, previous label c' in 0..C (C = start)
    and label c:

        psi = S[s+k, c] - S[s, c] + dur[k-1, c] + trans_start[c', c]
              (+ P_start[s, c] + P_end[s+k-1, c] with proj = (P_start, P_end))

    and -inf where the segment would end past L.  This is one tile of the
    O(T*K*C^2) tensor the pages say standard implementations materialise
    (EN explainer, "1. Problem Statement", "Edge Tensor Materialization")."""
    C = S.shape[1]
    ts = _trans_with_start(trans)
    dur = np.asarray(dur, dtype=np.float64)[:K]
    s = np.arange(s_lo, s_hi)
    k = np.arange(1, K + 1)
    end = s[:, None] + k[None, :]                      # [n, K]
    valid = end <= L
    content = S[np.minimum(end, L)] - S[s][:, None, :]  # [n, K, C]
    seg = content + dur[None, :, :]                     # [n, K, C]
    if proj is not None:
        ps, pe = (np.asarray(x, dtype=np.float64) for x in proj)
        seg = seg + ps[s][:, None, :] + pe[np.minimum(end, L) - 1]
    psi = seg[:, :, None, :] + ts[None, None, :, :]     # [n, K, C+1, C]
    psi[~valid] = NEG_INF
    return psi


def _tile(K: int, C: int) -> int:
    return int(max(1, min(1024, (1 << 22) // max(1, K * (C + 1) * C))))


def forward(S, trans, dur, K: int, L: int, proj=None):
    """alpha[t, c'] = log-sum over segmentations of [0, t) whose last segment
    has label c' (column C: the virtual start, alive only at t = 0), by

        alpha[t, c] = LSE_{k = 1..min(K, t), c'} (alpha[t-k, c'] + psi[t-k, k, c', c])

    Returns (alpha [L+1, C+1], logZ = LSE_c alpha[L, c])."""
    C = S.shape[1]
    alpha = np.full((L + 1, C + 1), NEG_INF)
    alpha[0, C] = 0.0
    tile = _tile(K, C)
    ks_all = np.arange(1, K + 1)
    for t0 in range(1, L + 1, tile):
        t1 = min(L + 1, t0 + tile)
        s_lo = max(0, t0 - K)
        psi = edge_potentials(S, trans, dur, K, L, s_lo, t1 - 1, proj)
        for t in range(t0, t1):
            ks = ks_all[: min(K, t)]
            edges = psi[t - ks - s_lo, ks - 1]                   # [k, C+1, C]
            scores = alpha[t - ks][:, :, None] + edges          # [k, C+1, C]
            alpha[t, :C] = _lse(scores.reshape(-1, C), axis=0)
    return alpha, float(_lse(alpha[L, :C]))


def backward(S, trans, dur, K: int, L: int, proj=None):
    """beta[s, c'] = log-sum over segmentations of [s, L) given that the
    previous segment (label c') ends at s:

        beta[L, c] = 0,
        beta[s, c'] = LSE_{k = 1..min(K, L-s), c} (psi[s, k, c', c] + beta[s+k, c])

    beta[0, C] (virtual start) equals log Z."""
    C = S.shape[1]
    beta = np.full((L + 1, C + 1), NEG_INF)
    beta[L, :] = 0.0
    tile = _tile(K, C)
    starts = list(range(0, L, tile))
    for s_lo in reversed(starts):
        s_hi = min(L, s_lo + tile)
        psi = edge_potentials(S, trans, dur, K, L, s_lo, s_hi, proj)
        for s in range(s_hi - 1, s_lo - 1, -1):
            kmax = min(K, L - s)
            scores = psi[s - s_lo, :kmax] + beta[s + 1: s + kmax + 1, :C][:, None, :]   # [k, C+1, C]
            beta[s, :] = _lse(scores.transpose(1, 0, 2).reshape(C + 1, -1), axis=1)
    return beta


def posteriors(S, trans, dur, K: int, L: int, alpha, beta, logZ: float, proj=None):
    """Edge marginals p(s, k, c', c) = exp(alpha[s, c'] + psi + beta[s+k, c] - logZ)
    summed into the feature expectations (= gradients of log Z):

    * grad_dur[k-1, c]  = sum_{s, c'} p           (d logZ / d dur)
    * grad_trans[c', c] = sum_{s, k}  p, real c'   (d logZ / d trans)
    * start[s, c] / end[e, c]: probability that a segment of label c starts at s
      / ends at e;  d logZ / d S[t, c] = end[t, c] - start[t, c];
      d logZ / d P_start[s, c] = start[s, c], d logZ / d P_end[t, c] = end[t+1, c]
    * mu[t, c] = P(position t lies in a segment of label c), via a difference
      array over the segment marginals."""
    C = S.shape[1]
    grad_dur = np.zeros((K, C))
    grad_trans = np.zeros((C, C))
    start = np.zeros((L + 1, C))
    end = np.zeros((L + 1, C))
    tile = _tile(K, C)
    for s_lo in range(0, L, tile):
        s_hi = min(L, s_lo + tile)
        psi = edge_potentials(S, trans, dur, K, L, s_lo, s_hi, proj)      # [n, K, C+1, C]
        s = np.arange(s_lo, s_hi)
        e = np.minimum(s[:, None] + np.arange(1, K + 1)[None, :], L)      # [n, K]
        logp = alpha[s_lo:s_hi][:, None, :, None] + psi + beta[e][:, :, None, :C] - logZ
        p = np.exp(logp)                                                   # -inf -> 0
        grad_dur += p.sum(axis=(0, 2))
        grad_trans += p[:, :, :C, :].sum(axis=(0, 1))
        q = p.sum(axis=2)                                                  # [n, K, C]
        start[s_lo:s_hi] += q.sum(axis=1)
        np.add.at(end, e.reshape(-1), q.reshape(-1, C))
    diff = start[:L] - np.vstack([np.zeros((1, C)), end[1:L]])
    mu = np.cumsum(diff, axis=0)                                           # [L, C]
    return {"grad_dur": grad_dur, "grad_trans": grad_trans, "start": start, "end": end,
            "mu": mu, "dS": end - start}


def viterbi(S, trans, dur, K: int, L: int, proj=None):
    """Max-plus version of ``forward`` with backpointers.  Ties go to the
    lexicographically lowest (k, c'), then the lowest final label (reading 7).
    Returns score, labels [L], seg_start [L] (uint8), margin, segments (s, k, c)
    in order, and the decision gaps: ``gaps[i]`` is the gap at the node where
    segment i ends (its label fixed), between the chosen (k, c') and the best
    other choice there; ``final_gap`` the gap of the final label.  Because the
    decoded path continues optimally from every node it visits, a segmentation
    that also has a segment of label c ending where segment i ends, but a
    different length or previous label, scores at most score - gaps[i]; one with
    another final label at most score - final_gap."""
    C = S.shape[1]
    V = np.full((L + 1, C + 1), NEG_INF)
    V[0, C] = 0.0
    bp = np.zeros((L + 1, C), dtype=np.int64)        # flat index k_idx*(C+1) + c'
    gap = np.full((L + 1, C), np.inf)
    tile = _tile(K, C)
    ks_all = np.arange(1, K + 1)
    for t0 in range(1, L + 1, tile):
        t1 = min(L + 1, t0 + tile)
        s_lo = max(0, t0 - K)
        psi = edge_potentials(S, trans, dur, K, L, s_lo, t1 - 1, proj)
        for t in range(t0, t1):
            ks = ks_all[: min(K, t)]
            scores = (V[t - ks][:, :, None] + psi[t - ks - s_lo, ks - 1]).reshape(-1, C)
            idx = np.argmax(scores, axis=0)                       # first maximiser
            best = scores[idx, np.arange(C)]
            V[t, :C] = best
            bp[t] = idx
            if scores.shape[0] > 1:
                rest = scores.copy()
                rest[idx, np.arange(C)] = NEG_INF
                gap[t] = best - rest.max(axis=0)
    final = V[L, :C]
    c = int(np.argmax(final))
    score = float(final[c])
    others = np.delete(final, c)
    margin = float(score - others.max()) if others.size else np.inf
    final_gap = margin
    labels = np.empty(L, dtype=np.int32)
    seg_start = np.zeros(L, dtype=np.uint8)
    segments = []
    gaps = []
    t = L
    while t > 0:
        margin = min(margin, float(gap[t, c]))
        gaps.append(float(gap[t, c]))
        k_idx, cp = divmod(int(bp[t, c]), C + 1)
        k = k_idx + 1
        s = t - k
        labels[s:t] = c
        seg_start[s] = 1
        segments.append((s, k, c))
        t, c = s, cp
    segments.reverse()
    gaps.reverse()
    return {"score": score, "labels": labels, "seg_start": seg_start, "margin": margin,
            "segments": segments, "gaps": np.array(gaps), "final_gap": final_gap}


def segmentation_score(S, trans, dur, K: int, seg_start: np.ndarray, labels: np.ndarray,
                       proj=None) -> float:
    """Score of one segmentation given per-position labels and segment-start
    flags, straight from the definition: sum of content + duration scores of
    its segments (+ the start and end projections of each, reading 9) and the
    transition scores between consecutive segments.  Raises ValueError if the
    segmentation is not valid."""
    L = len(labels)
    starts = [int(i) for i in np.nonzero(seg_start[:L])[0]]
    if not starts or starts[0] != 0:
        raise ValueError("segmentation must start at position 0")
    bounds = starts + [L]
    total = 0.0
    prev = None
    trans = np.asarray(trans, dtype=np.float64)
    dur = np.asarray(dur, dtype=np.float64)
    for s, e in zip(bounds[:-1], bounds[1:]):
        k = e - s
        c = int(labels[s])
        if not (1 <= k <= K) or np.any(labels[s:e] != c) or not (0 <= c < S.shape[1]):
            raise ValueError(f"invalid segment [{s}, {e}) label {c}")
        total += S[e, c] - S[s, c] + dur[k - 1, c]
        if proj is not None:
            total += float(proj[0][s, c]) + float(proj[1][e - 1, c])
        if prev is not None:
            total += trans[prev, c]
        prev = c
    return total


def gold_features(labels, seg_start, L: int, K: int, C: int, *, boundaries=False):
    """Feature counts of one segmentation, from its definition: the per-position
    label indicator [L, C], the number of segments of each length k and label c
    [K, C], and the number of transitions c' -> c between consecutive segments
    [C, C]; with ``boundaries`` also the segment-start and segment-end (last
    position) indicators [L, C] each, the features of the projections.  Raises
    ValueError for an invalid segmentation (same checks as
    ``segmentation_score``)."""
    starts = [int(i) for i in np.nonzero(np.asarray(seg_start)[:L])[0]]
    if not starts or starts[0] != 0:
        raise ValueError("segmentation must start at position 0")
    ind = np.zeros((L, C))
    dcount = np.zeros((K, C))
    tcount = np.zeros((C, C))
    sind = np.zeros((L, C))
    eind = np.zeros((L, C))
    prev = None
    for s, e in zip(starts, starts[1:] + [L]):
        k = e - s
        c = int(labels[s])
        if not (1 <= k <= K) or not (0 <= c < C) or np.any(np.asarray(labels[s:e]) != c):
            raise ValueError(f"invalid segment [{s}, {e}) label {c}")
        ind[s:e, c] = 1.0
        sind[s, c] = 1.0
        eind[e - 1, c] = 1.0
        dcount[k - 1, c] += 1.0
        if prev is not None:
            tcount[prev, c] += 1.0
        prev = c
    if boundaries:
        return ind, dcount, tcount, sind, eind
    return ind, dcount, tcount


def nll_sequence(em_b, L: int, trans, dur, K: int, labels, seg_start, g: float = 1.0,
                 proj=None):
    """Training loss of one gold segmentation y*: nll = log Z - score(y*), minus
    the log-probability the model gives y* (the loss of the pages' training
    convergence check, EN explainer, "4. Results and Benchmarks").  Gradients of
    g * nll: the posterior expectations of the features (the gradients of log Z)
    minus the features of y*, with the centring in the function (reading 6)."""
    r = sequence(em_b, L, trans, dur, K, g=g, want_viterbi=False, proj=proj)
    C = r["S"].shape[1]
    score = segmentation_score(r["S"], trans, dur, K, seg_start, labels, proj)
    ind, dcount, tcount, sind, eind = gold_features(labels, seg_start, L, K, C, boundaries=True)
    grad_em = r["grad_em"] - g * (ind - ind.mean(axis=0, keepdims=True))
    out = {"nll": r["logZ"] - score, "score": score, "logZ": r["logZ"], "grad_em": grad_em,
           "grad_trans": r["grad_trans"] - g * tcount, "grad_dur": r["grad_dur"] - g * dcount}
    if proj is not None:
        out.update(grad_proj_start=r["grad_proj_start"] - g * sind,
                   grad_proj_end=r["grad_proj_end"] - g * eind)
    return out


def _proj_of(proj_start, proj_end, b: int, L: int, C: int):
    """(P_start, P_end) rows t < L of sequence b; a missing array counts as zeros."""
    if proj_start is None and proj_end is None:
        return None
    z = np.zeros((L, C))
    ps = z if proj_start is None else np.asarray(proj_start[b, :L], dtype=np.float64)
    pe = z if proj_end is None else np.asarray(proj_end[b, :L], dtype=np.float64)
    return ps, pe


def nll_batch(em, lengths, trans, dur, K: int, gold_labels, gold_seg_start, grad_nll=None,
              proj_start=None, proj_end=None):
    """``nll_sequence`` for every b, packed with the ABI's conventions (zeros at
    t >= L; grad_trans and grad_dur summed over the batch)."""
    em = np.asarray(em)
    B, T, C = em.shape
    g = np.ones(B) if grad_nll is None else np.asarray(grad_nll, dtype=np.float64)
    out = {"nll": np.zeros(B), "score": np.zeros(B), "logZ": np.zeros(B),
           "grad_em": np.zeros((B, T, C)), "grad_trans": np.zeros((C, C)),
           "grad_dur": np.zeros(np.asarray(dur).shape),
           "grad_proj_start": np.zeros((B, T, C)), "grad_proj_end": np.zeros((B, T, C))}
    for b in range(B):
        L = int(lengths[b])
        proj = _proj_of(proj_start, proj_end, b, L, C)
        r = nll_sequence(em[b], L, trans, dur, K, gold_labels[b, :L], gold_seg_start[b, :L],
                         float(g[b]), proj)
        out["nll"][b], out["score"][b], out["logZ"][b] = r["nll"], r["score"], r["logZ"]
        out["grad_em"][b, :L] = r["grad_em"]
        if proj is not None:
            out["grad_proj_start"][b, :L] = r["grad_proj_start"]
            out["grad_proj_end"][b, :L] = r["grad_proj_end"]
        out["grad_trans"] += r["grad_trans"]
        out["grad_dur"] += r["grad_dur"]
    return out


def sequence(em_b, L: int, trans, dur, K: int, g: float = 1.0, *, want_viterbi=True,
             want_grads=True, proj=None):
    """Everything for one sequence (fp64): log Z, mu, grad_em (with the
    centring in the function, reading 6), grad_trans, grad_dur scaled by the
    upstream gradient g, and the Viterbi decode.  With proj = (P_start [L, C],
    P_end [L, C]) the projections enter every segment (reading 9) and the
    gradients include grad_proj_start / grad_proj_end (g times the start / end
    marginals); ``boundary`` [L] is the probability that a segment starts at t."""
    _, S = centered_prefix(em_b, L)
    alpha, logZ = forward(S, trans, dur, K, L, proj)
    out = {"logZ": logZ, "S": S}
    if want_grads:
        beta = backward(S, trans, dur, K, L, proj)
        post = posteriors(S, trans, dur, K, L, alpha, beta, logZ, proj)
        mu = post["mu"]
        out.update(mu=mu, grad_em=g * (mu - mu.mean(axis=0, keepdims=True)),
                   grad_trans=g * post["grad_trans"], grad_dur=g * post["grad_dur"],
                   dS=post["dS"], logZ_backward=float(beta[0, S.shape[1]]),
                   grad_proj_start=g * post["start"][:L], grad_proj_end=g * post["end"][1:],
                   boundary=post["start"][:L].sum(axis=1))
    if want_viterbi:
        out["viterbi"] = viterbi(S, trans, dur, K, L, proj)
    return out


def _sequence_job(args):
    return sequence(*args[:5], g=args[5], want_viterbi=args[6], want_grads=args[7],
                    proj=args[8])


def batch(em, lengths, trans, dur, K: int, grad_log_z=None, *, want_viterbi=True,
          want_grads=True, workers: int = 1, proj_start=None, proj_end=None):
    """Run ``sequence`` for every b and pack the results into padded arrays
    with the ABI's conventions (zeros / -1 at t >= L).  grad_trans and grad_dur
    are summed over the batch.  proj_start / proj_end: [B, T, C] or None
    (zeros).  With Viterbi, ``paths[b]`` holds the decoded segments [n, 3] as
    (start, length, label) rows with their decision gaps (see ``viterbi``)."""
    em = np.asarray(em)
    B, T, C = em.shape
    g = np.ones(B) if grad_log_z is None else np.asarray(grad_log_z, dtype=np.float64)
    jobs = [(em[b], int(lengths[b]), trans, dur, K, float(g[b]), want_viterbi, want_grads,
             _proj_of(proj_start, proj_end, b, int(lengths[b]), C))
            for b in range(B)]
    if workers > 1 and B > 1:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(min(workers, B)) as pool:
            res = pool.map(_sequence_job, jobs)
    else:
        res = [_sequence_job(j) for j in jobs]
    out = {"logZ": np.array([r["logZ"] for r in res])}
    if want_grads:
        mu = np.zeros((B, T, C))
        ge = np.zeros((B, T, C))
        gps = np.zeros((B, T, C))
        gpe = np.zeros((B, T, C))
        bnd = np.zeros((B, T))
        for b, r in enumerate(res):
            L = int(lengths[b])
            mu[b, :L] = r["mu"]
            ge[b, :L] = r["grad_em"]
            gps[b, :L] = r["grad_proj_start"]
            gpe[b, :L] = r["grad_proj_end"]
            bnd[b, :L] = r["boundary"]
        out.update(mu=mu, grad_em=ge, grad_proj_start=gps, grad_proj_end=gpe, boundary=bnd,
                   grad_trans=sum(r["grad_trans"] for r in res),
                   grad_dur=sum(r["grad_dur"] for r in res),
                   logZ_backward=np.array([r["logZ_backward"] for r in res]))
    if want_viterbi:
        labels = np.full((B, T), -1, dtype=np.int32)
        seg = np.zeros((B, T), dtype=np.uint8)
        for b, r in enumerate(res):
            L = int(lengths[b])
            labels[b, :L] = r["viterbi"]["labels"]
            seg[b, :L] = r["viterbi"]["seg_start"]
        out.update(score=np.array([r["viterbi"]["score"] for r in res]),
                   margin=np.array([r["viterbi"]["margin"] for r in res]),
                   labels=labels, seg_start=seg,
                   paths=[{"segments": np.array(r["viterbi"]["segments"], dtype=np.int64)
                           .reshape(-1, 3), "gaps": r["viterbi"]["gaps"],
                           "final_gap": r["viterbi"]["final_gap"]} for r in res])
    return out
