"""Write the oracle's expected values for the five synthetic configurations.

Calls only ``oracle/`` (fp64) on inputs from ``workloads.make(i)``; nothing
here touches the HIP path.  Output: ``tests/golden/oracle_cfg{i}.npz`` with
log Z, the batch-summed gradients of trans and dur, the Viterbi score and
margin for every sequence, and mu / grad_em at a fixed sample of positions
(every position for the tiny configuration).  Full Viterbi labels are stored
when the margin exceeds 1e-4 (otherwise several segmentations are optimal
within the tolerance and only validity and optimality can be checked).

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

SAMPLES_PER_SEQ = {0: None, 1: 48, 2: 96, 3: 384, 4: 32}


def sample_positions(index: int, lengths: np.ndarray) -> np.ndarray:
    """[B, n] positions: the first and last two, then uniform draws (seed 77)."""
    n = SAMPLES_PER_SEQ[index]
    rng = np.random.default_rng(77 + index)
    out = []
    for L in lengths:
        L = int(L)
        fixed = [0, 1, L - 2, L - 1]
        draw = rng.integers(0, L, size=n - len(fixed))
        out.append(np.array(fixed + list(draw), dtype=np.int64))
    return np.stack(out)


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
    if SAMPLES_PER_SEQ[index] is None:
        out["mu"] = res["mu"]
        out["grad_em"] = res["grad_em"]
    else:
        pos = sample_positions(index, w.lengths)
        b = np.arange(w.B)[:, None]
        out["positions"] = pos
        out["mu_sample"] = res["mu"][b, pos].astype(np.float32)
        out["grad_em_sample"] = res["grad_em"][b, pos].astype(np.float32)
    keep = res["margin"] > 1e-4
    out["labels_stored"] = keep
    if keep.any():
        out["labels"] = np.where(keep[:, None], res["labels"], -2).astype(np.int16)
        out["seg_start"] = np.where(keep[:, None], res["seg_start"], 0).astype(np.uint8)
    path = os.path.join(HERE, f"oracle_cfg{index}.npz")
    np.savez_compressed(path, **out)
    print(f"cfg {index} ({w.name}): {dt:.1f} s, logZ {res['logZ']}, margins {res['margin']}",
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
