"""Write the oracle's expected values for the long-duration cases (K up to 8000).

Calls only ``oracle/`` (fp64) on inputs from ``workloads.make_custom`` with the seeds and
shapes listed in CASES; nothing here touches the HIP path.  Output:
``tests/golden/oracle_extreme_k.npz`` holding, per case, log Z, mu, grad_em, grad_trans,
grad_dur, the start / end marginals and boundary probabilities (upstream gradient 1), the
Viterbi score, margin, labels and segment starts, and the Viterbi paths with the gap of
every decision along them.  Two cases carry boundary projections.
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

# name: (seed, B, T, C, K, em_scale, ragged, projection sd (0: none))
CASES = {
    "x1": (601, 2, 2300, 6, 2000, 2.0, True, 0.0),    # genomic label count at K = 2000
    "x2": (602, 1, 1300, 7, 1100, 1.5, False, 0.0),   # 7 labels, 64 lanes each
    "x3": (603, 1, 2100, 4, 2049, 2.0, False, 0.0),   # the largest K, log-space ring only
    "x4": (604, 1, 1400, 6, 1200, 1.5, False, 1.0),   # boundary projections, 64 lanes
    "x5": (605, 3, 60, 5, 1500, 1.0, True, 0.5),      # K > T on the 64-lane path
    "x6": (606, 1, 8100, 3, 8000, 2.0, False, 0.0),   # K = 8000: log-semiring rings in global memory
    "x7": (607, 2, 4500, 3, 4000, 1.5, True, 0.5),    # K = 4000 with projections
    "x8": (608, 1, 5000, 6, 4000, 2.0, False, 0.0),   # log rings global, max-plus ring LDS
    "x9": (609, 1, 2600, 12, 2049, 1.5, False, 0.0),  # 12 labels at K = 2049
    "x10": (610, 2, 1200, 24, 500, 1.0, True, 0.0),   # 24 labels at K = 500
}


def projections(seed: int, B: int, T: int, C: int, sd: float):
    """Seeded N(0, sd) start / end projections [B, T, C] float32 (None when sd = 0)."""
    if sd == 0.0:
        return None, None
    rng = np.random.default_rng(seed)
    return (rng.normal(0, sd, (B, T, C)).astype(np.float32),
            rng.normal(0, sd, (B, T, C)).astype(np.float32))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args()
    out = {}
    for name, (seed, B, T, C, K, scale, ragged, sd) in CASES.items():
        w = workloads.make_custom(seed, B, T, C, K, em_scale=scale, ragged=ragged)
        ps, pe = projections(seed + 1000, B, T, C, sd)
        t0 = time.time()
        r = oracle.batch(w.em, w.lengths, w.trans, w.dur, K, workers=a.workers,
                         proj_start=ps, proj_end=pe)
        print(f"{name}: B={B} T={T} C={C} K={K} {time.time() - t0:.1f} s, logZ {r['logZ']}, "
              f"margin {r['margin']}", flush=True)
        out[f"{name}_case"] = np.array([seed, B, T, C, K, scale, ragged, sd], dtype=np.float64)
        for k in ("logZ", "score", "margin", "grad_trans", "grad_dur"):
            out[f"{name}_{k}"] = np.asarray(r[k], dtype=np.float64)
        for k in ("mu", "grad_em", "grad_proj_start", "grad_proj_end", "boundary"):
            out[f"{name}_{k}"] = r[k].astype(np.float32)
        out[f"{name}_labels"] = r["labels"].astype(np.int16)
        out[f"{name}_seg_start"] = r["seg_start"].astype(np.uint8)
        # the Viterbi paths with the gap of every decision along them
        segs = [p["segments"] for p in r["paths"]]
        out[f"{name}_path_off"] = np.cumsum([0] + [len(x) for x in segs]).astype(np.int64)
        out[f"{name}_path_segs"] = np.concatenate(segs).astype(np.int32)
        out[f"{name}_path_gaps"] = np.concatenate([p["gaps"] for p in r["paths"]])
        out[f"{name}_final_gap"] = np.array([p["final_gap"] for p in r["paths"]])
    np.savez_compressed(os.path.join(HERE, "oracle_extreme_k.npz"), **out)


if __name__ == "__main__":
    main()
