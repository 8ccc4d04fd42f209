"""Write the oracle's expected values for the long-duration cases (K up to 2049).

Calls only ``oracle/`` (fp64) on inputs from ``workloads.make_custom`` with the seeds and
shapes listed in CASES; nothing here touches the HIP path.  Output:
``tests/golden/oracle_extreme_k.npz`` holding, per case, log Z, mu, grad_em, grad_trans,
grad_dur (upstream gradient 1), the Viterbi score, margin, labels and segment starts.
The oracle needs minutes for these shapes, so the values are stored instead of being
recomputed by the GPU tests.

Usage:  python tests/golden/make_extreme_k_fixture.py [--workers N]
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

# name: (seed, B, T, C, K, em_scale, ragged)
CASES = {
    "x1": (601, 2, 2300, 6, 2000, 2.0, True),    # genomic label count at K = 2000
    "x2": (602, 1, 1300, 7, 1100, 1.5, False),   # 7 labels, 64 lanes each
    "x3": (603, 1, 2100, 4, 2049, 2.0, False),   # the largest K, log-space ring only
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args()
    out = {}
    for name, (seed, B, T, C, K, scale, ragged) in CASES.items():
        w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=ragged)
        t0 = time.time()
        r = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, workers=a.workers)
        print(f"{name}: B={B} T={T} C={C} K={K} {time.time() - t0:.1f} s, logZ {r['logZ']}, "
              f"margin {r['margin']}", flush=True)
        out[f"{name}_case"] = np.array([seed, B, T, C, K, scale, ragged], dtype=np.float64)
        for k in ("logZ", "score", "margin", "grad_trans", "grad_dur"):
            out[f"{name}_{k}"] = np.asarray(r[k], dtype=np.float64)
        for k in ("mu", "grad_em"):
            out[f"{name}_{k}"] = r[k].astype(np.float32)
        out[f"{name}_labels"] = r["labels"].astype(np.int16)
        out[f"{name}_seg_start"] = r["seg_start"].astype(np.uint8)
    np.savez_compressed(os.path.join(HERE, "oracle_extreme_k.npz"), **out)


if __name__ == "__main__":
    main()
