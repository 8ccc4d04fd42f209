"""Write the oracle's expected values for the five synthetic configurations.

Calls only ``oracle/`` (fp64) on inputs from ``workloads.make(i)``; nothing here
touches the HIP path.  Output: ``tests/golden/oracle_cfg{i}.npz`` with

* log Z (forward and backward recursions), the batch-summed gradients of trans and
  dur, the Viterbi score and margin of every sequence;
* the Viterbi path of every sequence with the gap of each decision along it
  (``path_segs`` rows (start, length, label), ``path_gaps``, offsets ``path_off``,
  ``final_gap``), so a decode can be compared decision by decision;
* mu and grad_em (float32) on contiguous windows of positions: [j*D - K, j*D + K]
  around every multiple j*D of the checkpoint interval D counted from either end of the
  sequence (where the span sweeps of the two directions join), plus the first and last
  2K positions (``win_pos`` per sequence with offsets ``win_off``); instead, every
  position for the tiny and speech configurations and for sequence 0 of the genomic one
  (``mu_full`` / ``grad_em_full`` with ``full_seqs``).  D is the interval the library's
  backward takes by default at each shape (``SEAM_INTERVAL``, stored as
  ``seam_interval``; the header ``include/semicrf.h`` states the rule, and the parity
  test checks that the library still picks it).

Usage:  python tests/golden/make_oracle_fixtures.py [cfg ...] [--workers N]
"""

from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle      # noqa: E402
import workloads   # noqa: E402

FULL_SEQS = {0: "all", 1: "all", 2: [0], 3: [], 4: []}
# the backward's default checkpoint interval at the windowed shapes: genomic (56 spans a
# sequence), long genomic (224 spans), large label set (16 spans a sequence)
SEAM_INTERVAL = {2: 1786, 3: 4465, 4: 625}


def window_positions(L: int, T: int, K: int, D: int) -> np.ndarray:
    """Sorted positions in [0, L): windows of half-width K around every multiple of the
    checkpoint interval D from either end, and the first and last 2K positions."""
    keep = np.zeros(L, dtype=bool)
    keep[: min(L, 2 * K)] = True
    keep[max(0, L - 2 * K):] = True
    for j in range(1, (L + D - 1) // D + 1):
        for c in (j * D, L - j * D):
            lo, hi = max(0, c - K), min(L, c + K + 1)
            if lo < hi:
                keep[lo:hi] = True
    return np.nonzero(keep)[0].astype(np.int32)


def make_fixture(index: int, workers: int) -> str:
    w = workloads.make(index)
    t0 = time.time()
    res = oracle.batch(w.em, w.lengths, w.trans, w.dur, w.K, want_viterbi=True,
                       want_grads=True, workers=workers)
    dt = time.time() - t0
    out = {
        "logZ": res["logZ"], "logZ_backward": res["logZ_backward"],
        "grad_trans": res["grad_trans"], "grad_dur": res["grad_dur"],
        "score": res["score"], "margin": res["margin"],
        "oracle_seconds": np.array(dt), "workers": np.array(workers),
    }
    # Viterbi paths with their decision gaps
    segs = [p["segments"] for p in res["paths"]]
    out["path_off"] = np.cumsum([0] + [len(s) for s in segs]).astype(np.int64)
    out["path_segs"] = np.concatenate(segs).astype(np.int32)
    out["path_gaps"] = np.concatenate([p["gaps"] for p in res["paths"]])
    out["final_gap"] = np.array([p["final_gap"] for p in res["paths"]])
    # mu / grad_em windows (none where every position is stored)
    full = list(range(w.B)) if FULL_SEQS[index] == "all" else FULL_SEQS[index]
    D = SEAM_INTERVAL.get(index, w.T)
    out["seam_interval"] = np.array(D, dtype=np.int32)
    pos = [np.zeros(0, dtype=np.int32) if b in full else window_positions(int(L), w.T, w.K, D)
           for b, L in enumerate(w.lengths)]
    out["win_off"] = np.cumsum([0] + [len(p) for p in pos]).astype(np.int64)
    out["win_pos"] = np.concatenate(pos)
    C = w.C
    out["mu_win"] = np.concatenate([res["mu"][b, p].reshape(-1, C)
                                    for b, p in enumerate(pos)]).astype(np.float32)
    out["grad_em_win"] = np.concatenate([res["grad_em"][b, p].reshape(-1, C)
                                         for b, p in enumerate(pos)]).astype(np.float32)
    out["full_seqs"] = np.array(full, dtype=np.int32)
    if full:
        out["mu_full"] = res["mu"][full].astype(np.float32)
        out["grad_em_full"] = res["grad_em"][full].astype(np.float32)
    path = os.path.join(HERE, f"oracle_cfg{index}.npz")
    np.savez_compressed(path, **out)
    print(f"cfg {index} ({w.name}): {dt:.1f} s, logZ {res['logZ']}, margins {res['margin']}, "
          f"{len(out['win_pos'])} window positions, {os.path.getsize(path) / 1e6:.1f} MB",
          flush=True)
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("cfg", nargs="*", type=int, default=[0, 1, 2, 4, 3])
    ap.add_argument("--workers", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args()
    for i in a.cfg:
        make_fixture(i, a.workers)


if __name__ == "__main__":
    main()
