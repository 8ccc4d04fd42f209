"""Independent reference computations that pin the fp64 oracle.

Nothing here imports ``oracle/`` or the HIP path.  Each routine reaches the
answer by a different route than the oracle's edge-tensor recursions:

* ``brute_force`` enumerates every segmentation of a short sequence and scores
  each one from the definition, with the segment content summed position by
  position from the centred emissions (no prefix-sum differences, no
  recursions).
* ``linear_chain`` is the textbook linear-chain CRF forward-backward and
  Viterbi with unary and pairwise scores, which a semi-CRF must reduce to at
  K = 1 (gist.science EN explainer, "1. Problem Statement": linear-chain
  CRFs are the K = 1 case).
* ``count_segmentations`` is the exact integer count of segmentations with
  parts <= K and C labels, i.e. Z when every potential is zero.
"""

from __future__ import annotations

import itertools
import math

import numpy as np


def _logsumexp_list(vals):
    m = max(vals)
    if m == -math.inf:
        return -math.inf
    return m + math.log(sum(math.exp(v - m) for v in vals))


def compositions(L: int, K: int):
    """All ordered tuples of segment lengths in [1, K] summing to L."""
    if L == 0:
        yield ()
        return
    for k in range(1, min(K, L) + 1):
        for rest in compositions(L - k, K):
            yield (k,) + rest


def count_segmentations(L: int, K: int, C: int) -> int:
    """Exact number of labelled segmentations: sum over compositions of C^parts."""
    n = [0] * (L + 1)
    n[0] = 1
    for t in range(1, L + 1):
        n[t] = C * sum(n[t - k] for k in range(1, min(K, t) + 1))
    return n[L]


def centred_emissions(em_b, L):
    """Per-label mean over the L valid positions subtracted, with plain loops."""
    C = len(em_b[0])
    nu = [sum(float(em_b[t][c]) for t in range(L)) / L for c in range(C)]
    return [[float(em_b[t][c]) - nu[c] for c in range(C)] for t in range(L)]


def _proj_rows(proj, L, C):
    if proj is None:
        z = [[0.0] * C for _ in range(L)]
        return z, z
    return ([[float(v) for v in row] for row in proj[0][:L]],
            [[float(v) for v in row] for row in proj[1][:L]])


def brute_force(em_b, L: int, trans, dur, K: int, proj=None):
    """Enumerate every segmentation of [0, L) (lengths <= K, C labels, no
    transition into the first segment).  Returns log Z, posterior expectations
    (mu, grad_dur, grad_trans, start / end marginals) and the best and
    second-best scores with the best segmentation.  proj = (P_start, P_end):
    a segment [s, s+k) of label c also scores P_start[s][c] + P_end[s+k-1][c]."""
    x = centred_emissions(em_b, L)
    C = len(x[0])
    trans = np.asarray(trans, dtype=np.float64)
    dur = np.asarray(dur, dtype=np.float64)
    ps, pe = _proj_rows(proj, L, C)
    scores_all = []
    records = []
    for comp in compositions(L, K):
        m = len(comp)
        starts = [sum(comp[:i]) for i in range(m)]
        # content of segment i with label c, summed position by position
        cont = np.array([[sum(x[u][c] for u in range(s, s + k)) + ps[s][c] + pe[s + k - 1][c]
                          for c in range(C)] for s, k in zip(starts, comp)])   # [m, C]
        labs = np.array(list(itertools.product(range(C), repeat=m)))     # [C^m, m]
        sc = np.zeros(len(labs))
        for i, k in enumerate(comp):
            sc += cont[i, labs[:, i]] + dur[k - 1, labs[:, i]]
            if i > 0:
                sc += trans[labs[:, i - 1], labs[:, i]]
        scores_all.append(sc)
        records.append((comp, starts, labs))
    flat = np.concatenate(scores_all)
    m = flat.max()
    logZ = float(m + np.log(np.exp(flat - m).sum()))

    mu = np.zeros((L, C))
    grad_dur = np.zeros((K, C))
    grad_trans = np.zeros((C, C))
    start = np.zeros((L + 1, C))
    end = np.zeros((L + 1, C))
    for (comp, starts, labs), sc in zip(records, scores_all):
        w = np.exp(sc - logZ)
        for i, (s, k) in enumerate(zip(starts, comp)):
            for c in range(C):
                wc = w[labs[:, i] == c].sum()
                mu[s:s + k, c] += wc
                grad_dur[k - 1, c] += wc
                start[s, c] += wc
                end[s + k, c] += wc
            if i > 0:
                np.add.at(grad_trans, (labs[:, i - 1], labs[:, i]), w)

    order = np.argsort(-flat, kind="stable")
    best = float(flat[order[0]])
    second = float(flat[order[1]]) if flat.size > 1 else -math.inf
    # decode the best segmentation
    idx = int(order[0])
    for (comp, starts, labs), sc in zip(records, scores_all):
        if idx < len(sc):
            labels = np.empty(L, dtype=np.int32)
            seg = np.zeros(L, dtype=np.uint8)
            for i, (s, k) in enumerate(zip(starts, comp)):
                labels[s:s + k] = labs[idx, i]
                seg[s] = 1
            break
        idx -= len(sc)
    return {"logZ": logZ, "mu": mu, "grad_dur": grad_dur, "grad_trans": grad_trans,
            "start": start, "end": end, "best": best, "second": second,
            "labels": labels, "seg_start": seg, "n": int(flat.size)}


def brute_force_nll(em_b, L: int, trans, dur, K: int, labels, seg_start, proj=None) -> float:
    """-log P(y*) of the segmentation given by (labels, seg_start): every
    segmentation is enumerated and scored position by position (centred emissions
    summed over each segment, no prefix sums, plus the projections of its first and
    last position), and the gold one is picked out by its segments."""
    x = centred_emissions(em_b, L)
    C = len(x[0])
    ps, pe = _proj_rows(proj, L, C)
    trans = np.asarray(trans, dtype=np.float64)
    dur = np.asarray(dur, dtype=np.float64)
    starts = [t for t in range(L) if seg_start[t]]
    gold = tuple((s, e - s, int(labels[s])) for s, e in zip(starts, starts[1:] + [L]))
    scores = []
    gold_score = None
    for comp in compositions(L, K):
        st = [sum(comp[:i]) for i in range(len(comp))]
        for labs in itertools.product(range(C), repeat=len(comp)):
            sc = 0.0
            for i, (s, k) in enumerate(zip(st, comp)):
                sc += sum(x[u][labs[i]] for u in range(s, s + k)) + dur[k - 1, labs[i]]
                sc += ps[s][labs[i]] + pe[s + k - 1][labs[i]]
                if i > 0:
                    sc += trans[labs[i - 1], labs[i]]
            scores.append(sc)
            if tuple(zip(st, comp, labs)) == gold:
                gold_score = sc
    assert gold_score is not None, "gold segmentation not among the enumerated ones"
    return _logsumexp_list(scores) - gold_score


def linear_chain(unary, trans):
    """Textbook linear-chain CRF over L positions and C states with scores
    unary[t][c] and trans[c'][c] (no start / end scores): forward, backward,
    node and pairwise marginals, Viterbi with the lowest index on ties."""
    unary = [[float(v) for v in row] for row in unary]
    trans = [[float(v) for v in row] for row in trans]
    L, C = len(unary), len(unary[0])
    alpha = [unary[0][:]]
    for t in range(1, L):
        alpha.append([unary[t][c] + _logsumexp_list([alpha[t - 1][cp] + trans[cp][c]
                                                     for cp in range(C)]) for c in range(C)])
    logZ = _logsumexp_list(alpha[L - 1])
    beta = [[0.0] * C for _ in range(L)]
    for t in range(L - 2, -1, -1):
        beta[t] = [_logsumexp_list([trans[cp][c] + unary[t + 1][c] + beta[t + 1][c]
                                    for c in range(C)]) for cp in range(C)]
    node = [[math.exp(alpha[t][c] + beta[t][c] - logZ) for c in range(C)] for t in range(L)]
    pair = np.zeros((C, C))
    for t in range(1, L):
        for cp in range(C):
            for c in range(C):
                pair[cp, c] += math.exp(alpha[t - 1][cp] + trans[cp][c] + unary[t][c]
                                        + beta[t][c] - logZ)
    # Viterbi
    V = [unary[0][:]]
    bp = [[0] * C]
    for t in range(1, L):
        row, brow = [], []
        for c in range(C):
            cands = [V[t - 1][cp] + trans[cp][c] for cp in range(C)]
            j = max(range(C), key=lambda i: (cands[i], -i))
            row.append(unary[t][c] + cands[j])
            brow.append(j)
        V.append(row)
        bp.append(brow)
    c = max(range(C), key=lambda i: (V[L - 1][i], -i))
    score = V[L - 1][c]
    path = [c]
    for t in range(L - 1, 0, -1):
        c = bp[t][c]
        path.append(c)
    path.reverse()
    return {"logZ": logZ, "node": np.array(node), "pair": pair, "score": score,
            "path": np.array(path, dtype=np.int32)}


def all_segmentations(em_b, L: int, trans, dur, K: int):
    """Every segmentation of [0, L) as (segments, score), segments a tuple of
    (start, length, label) in order; the score summed position by position from
    the centred emissions (no prefix sums), plus durations and transitions."""
    x = centred_emissions(em_b, L)
    C = len(x[0])
    trans = np.asarray(trans, dtype=np.float64)
    dur = np.asarray(dur, dtype=np.float64)
    out = []
    for comp in compositions(L, K):
        st = [sum(comp[:i]) for i in range(len(comp))]
        for labs in itertools.product(range(C), repeat=len(comp)):
            sc = 0.0
            for i, (s, k) in enumerate(zip(st, comp)):
                sc += sum(x[u][labs[i]] for u in range(s, s + k)) + dur[k - 1, labs[i]]
                if i > 0:
                    sc += trans[labs[i - 1], labs[i]]
            out.append((tuple(zip(st, comp, labs)), sc))
    return out


def decision_gaps(segmentations, path):
    """Gaps of the decisions along ``path`` (a tuple of (start, length, label)),
    from the enumerated segmentations alone.  For segment i of the path, ending at
    e with label c after label c' (or after nothing when it starts at 0): the best
    score minus the best score of any segmentation that also has a segment of label
    c ending at e but a different start or previous label (inf if none).  The
    final gap: the best score minus the best score with another last label."""
    best = max(sc for _, sc in segmentations)
    gaps = []
    for i, (s, k, c) in enumerate(path):
        e = s + k
        prev = path[i - 1][2] if i > 0 else None
        alt = -math.inf
        for segs, sc in segmentations:
            for j, (s2, k2, c2) in enumerate(segs):
                if s2 + k2 == e and c2 == c:
                    p2 = segs[j - 1][2] if j > 0 else None
                    if (s2, p2) != (s, prev):
                        alt = max(alt, sc)
                    break
        gaps.append(best - alt)
    last = path[-1][2]
    alt = max((sc for segs, sc in segmentations if segs[-1][2] != last), default=-math.inf)
    return np.array(gaps), best - alt
