"""Checks of a decoded segmentation against the oracle's Viterbi path (test helper).

The oracle returns its best path as segments (start, length, label) with the gap of
every decision along it: at the node where segment i ends (label c at position e) the
gap between the chosen (start, previous label) and the best other choice there, and the
gap of the final label.  A segmentation that passes through that node with another
choice scores at most best - gap (the oracle's path continues optimally from every node
it visits), so a decode that is optimal to within `tol` must

* end with the oracle's final label when the final gap exceeds `tol`;
* wherever it has a segment of label c ending at e, and the oracle's decision there has a
  gap above `tol`, use the oracle's start and previous label for it;

and its score, recomputed in fp64 from the definition, must be within `atol` of the best.
Where several segmentations tie (gaps of 0, e.g. a run of one label split 2+1 or 1+2),
only the decisions that are unique are compared.
"""

import numpy as np

import oracle


def decode_segments(labels, seg_start, L):
    starts = np.nonzero(np.asarray(seg_start[:L]))[0]
    assert len(starts) and starts[0] == 0, "a decode must start a segment at 0"
    ends = np.append(starts[1:], L)
    return starts, ends, np.asarray(labels)[starts]


def assert_decisions(labels, seg_start, L, path_segs, gaps, final_gap, tol=1e-4):
    """Returns the number of the oracle's decisions that were compared."""
    st, en, lab = decode_segments(labels, seg_start, L)
    node = {int(e): (int(s), int(c), int(lab[i - 1]) if i > 0 else -1)
            for i, (s, e, c) in enumerate(zip(st, en, lab))}
    checked = 0
    path_segs = np.asarray(path_segs)
    if final_gap > tol:
        assert int(lab[-1]) == int(path_segs[-1][2]), "final label differs from the oracle's"
        checked += 1
    for i, (s, k, c) in enumerate(path_segs):
        e = int(s + k)
        if gaps[i] > tol and e in node and node[e][1] == int(c):
            prev = int(path_segs[i - 1][2]) if i > 0 else -1
            assert node[e][0] == int(s) and node[e][2] == prev, \
                (f"decision at the end {e} of label {int(c)}: decode starts at {node[e][0]} "
                 f"after label {node[e][2]}, the oracle at {int(s)} after {prev} "
                 f"(gap {gaps[i]:.3g})")
            checked += 1
    return checked


def check_decode(em_b, L, trans, dur, K, labels_b, seg_b, best, path=None, proj=None,
                 tol=1e-4, atol=1e-3):
    """Validity, fp64 rescore within `atol` of `best`, and the oracle's unique decisions
    (path: dict with segments, gaps, final_gap)."""
    assert np.all(np.asarray(labels_b)[L:] == -1) and np.all(np.asarray(seg_b)[L:] == 0)
    _, S = oracle.centered_prefix(em_b, L)
    got = oracle.segmentation_score(S, trans, dur, K, seg_b[:L], labels_b[:L], proj)
    assert got >= best - atol, f"decode scores {got!r}, the best is {best!r}"
    if path is not None:
        return assert_decisions(labels_b, seg_b, L, path["segments"], path["gaps"],
                                path["final_gap"], tol)
    return 0


def fixture_path(f, b, prefix=""):
    """Path b of a fixture written with path_off / path_segs / path_gaps / final_gap."""
    off = f[prefix + "path_off"]
    return {"segments": f[prefix + "path_segs"][off[b]:off[b + 1]],
            "gaps": f[prefix + "path_gaps"][off[b]:off[b + 1]],
            "final_gap": float(f[prefix + "final_gap"][b])}
