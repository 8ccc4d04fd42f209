"""Seeded synthetic workloads for the streaming semi-Markov CRF.

This module only draws random inputs.  It holds none of the method's
arithmetic (no prefix sums, no recursions, no potentials), so that both the
fp64 oracle (``oracle/``) and the HIP path (``semi_markov_crf_amd``) can consume
the same arrays without sharing any code that computes a result.

The five configurations follow the synthetic stand-ins for the workloads the
Flash-SemiCRF pages measure on (gist.science explainer, "4. Results and
Benchmarks": TIMIT speech with K=30, genome-scale sequences of 10^5 to 10^6
positions, K=200, C=6).  TIMIT itself is not used: the speech configuration
only mimics its label count and duration range with random data.

Every generator uses ``numpy.random.default_rng(1000 + index)`` (PCG64) and
draws, in this order: lengths, ground-truth segment durations and labels,
emission noise, transitions, durations.  Emissions are float32 ``[B, T, C]``
(C innermost), lengths int32 ``[B]``, trans float32 ``[C, C]`` (row = previous
label, column = next label), dur float32 ``[K, C]`` (row ``k-1`` scores a
segment of length ``k``).  Positions ``t >= lengths[b]`` hold noise and must be
ignored by every consumer.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "CONFIGS", "make", "make_custom", "tiny_slice"]


@dataclasses.dataclass
class Workload:
    name: str
    em: np.ndarray        # float32 [B, T, C]
    lengths: np.ndarray   # int32 [B]
    trans: np.ndarray     # float32 [C, C]
    dur: np.ndarray       # float32 [K, C]
    K: int
    truth: np.ndarray | None = None   # int32 [B, T] ground-truth labels (-1 on padding), if any

    @property
    def B(self) -> int:
        return int(self.em.shape[0])

    @property
    def T(self) -> int:
        return int(self.em.shape[1])

    @property
    def C(self) -> int:
        return int(self.em.shape[2])

    def positions(self) -> int:
        return int(self.lengths.astype(np.int64).sum())

    def subset(self, b0: int, b1: int, t_max: int | None = None) -> "Workload":
        """Sequences b0..b1-1, optionally cut to the first t_max positions."""
        em = self.em[b0:b1]
        lengths = self.lengths[b0:b1].copy()
        truth = None if self.truth is None else self.truth[b0:b1]
        if t_max is not None:
            em = em[:, :t_max]
            lengths = np.minimum(lengths, t_max).astype(np.int32)
            truth = None if truth is None else truth[:, :t_max]
        return Workload(self.name, np.ascontiguousarray(em), lengths, self.trans, self.dur,
                        self.K, None if truth is None else np.ascontiguousarray(truth))


def _segments(rng: np.random.Generator, L: int, draw_dur, draw_label) -> np.ndarray:
    """Piecewise-constant labels over [0, L): durations and labels are drawn in
    bulk (L of each, enough for the worst case), then laid out until L."""
    durs = draw_dur(L)
    labs = draw_label(L)
    ends = np.cumsum(durs)
    n = int(np.searchsorted(ends, L, side="left")) + 1
    starts = np.concatenate([[0], ends[: n - 1]])
    out = np.empty(L, dtype=np.int32)
    for s, d, c in zip(starts[:n], durs[:n], labs[:n]):
        out[s: min(L, s + d)] = c
    return out


def _assemble(name, rng, B, T, C, K, lengths, draw_dur, draw_label, bump, trans_sd, dur_sd):
    truth = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        truth[b, : lengths[b]] = _segments(rng, int(lengths[b]), draw_dur, draw_label)
    em = rng.standard_normal((B, T, C), dtype=np.float64)
    if bump:
        bb, tt = np.nonzero(truth >= 0)
        em[bb, tt, truth[bb, tt]] += bump
    trans = rng.normal(0.0, trans_sd, size=(C, C))
    dur = rng.normal(0.0, dur_sd, size=(K, C))
    return Workload(name, em.astype(np.float32), lengths.astype(np.int32),
                    trans.astype(np.float32), dur.astype(np.float32), K, truth)


def _tiny(rng):
    B, T, K, C = 2, 64, 8, 4
    lengths = np.full(B, T, dtype=np.int32)
    em = rng.standard_normal((B, T, C), dtype=np.float64)
    trans = rng.normal(0.0, 0.1, size=(C, C))
    dur = rng.normal(0.0, 0.1, size=(K, C))
    return Workload("tiny", em.astype(np.float32), lengths, trans.astype(np.float32),
                    dur.astype(np.float32), K, None)


def _speech(rng):
    B, T, K, C = 32, 800, 30, 39
    lengths = rng.integers(400, 801, size=B).astype(np.int32)
    return _assemble(
        "speech", rng, B, T, C, K, lengths,
        draw_dur=lambda n: np.minimum(rng.geometric(1.0 / 8.0, size=n), K),
        draw_label=lambda n: rng.integers(0, C, size=n),
        bump=2.0, trans_sd=0.5, dur_sd=0.1)


def _genomic_labels(rng, C):
    def draw(n):
        u = rng.random(n)
        alt = rng.integers(1, C, size=n)
        return np.where(u < 0.7, 0, alt)
    return draw


def _genomic(rng, B=4, T=100_000, name="genomic", K=200, mean=50.0):
    C = 6
    lengths = np.full(B, T, dtype=np.int32)
    return _assemble(
        name, rng, B, T, C, K, lengths,
        draw_dur=lambda n: np.minimum(rng.geometric(1.0 / mean, size=n), K),
        draw_label=_genomic_labels(rng, C),
        bump=1.5, trans_sd=0.1, dur_sd=0.1)


def _long(rng):
    return _genomic(rng, B=1, T=1_000_000, name="long")


def _large_c(rng):
    B, T, K, C = 8, 10_000, 64, 64
    lengths = np.full(B, T, dtype=np.int32)
    return _assemble(
        "large_c", rng, B, T, C, K, lengths,
        draw_dur=lambda n: rng.integers(1, 65, size=n),
        draw_label=lambda n: rng.integers(0, C, size=n),
        bump=2.0, trans_sd=0.5, dur_sd=0.1)


CONFIGS = {
    0: ("tiny: B=2 T=64 K=8 C=4", _tiny),
    1: ("speech: B=32 T=400..800 K=30 C=39", _speech),
    2: ("genomic: B=4 T=1e5 K=200 C=6", _genomic),
    3: ("long: B=1 T=1e6 K=200 C=6", _long),
    4: ("large_c: B=8 T=1e4 K=64 C=64", _large_c),
}


def make(index: int) -> Workload:
    """Configuration ``index`` (0..4) drawn with seed 1000 + index."""
    _, fn = CONFIGS[index]
    return fn(np.random.default_rng(1000 + index))


def long_duration(seed: int = 1005, B: int = 1, T: int = 1_000_000, K: int = 2000) -> Workload:
    """The genomic generator (C = 6, one label on 70% of the segments) with a long maximum
    duration: segment lengths geometric with mean K/4, capped at K."""
    return _genomic(np.random.default_rng(seed), B=B, T=T, name=f"long_duration_K{K}", K=K,
                    mean=K / 4.0)


def tiny_slice(T: int = 8) -> Workload:
    """The first T positions of the tiny configuration (all lengths T), small
    enough for brute-force enumeration of every segmentation."""
    w = make(0)
    return w.subset(0, w.B, t_max=T)


def make_custom(seed: int, B: int, T: int, C: int, K: int, *, em_scale: float = 1.0,
                trans_sd: float = 0.5, dur_sd: float = 0.5, ragged: bool = True,
                min_len: int = 1) -> Workload:
    """Plain i.i.d. Gaussian inputs of any shape, for edge cases and tiling tests.
    With ``ragged`` the lengths are uniform in [min_len, T] and the last one is T."""
    rng = np.random.default_rng(seed)
    if ragged:
        lengths = rng.integers(min_len, T + 1, size=B).astype(np.int32)
        lengths[-1] = T
    else:
        lengths = np.full(B, T, dtype=np.int32)
    em = em_scale * rng.standard_normal((B, T, C))
    trans = rng.normal(0.0, trans_sd, size=(C, C))
    dur = rng.normal(0.0, dur_sd, size=(K, C))
    return Workload(f"custom{seed}", em.astype(np.float32), lengths, trans.astype(np.float32),
                    dur.astype(np.float32), K, None)


def gold_segmentation(seed: int, lengths, T: int, C: int, K: int):
    """A random valid segmentation of every sequence, as training targets: segment
    lengths uniform in [1, min(K, rest)], labels uniform in [0, C).  Returns labels
    int32 [B, T] (-1 at t >= L) and seg_start uint8 [B, T] (1 at each segment's first
    position)."""
    rng = np.random.default_rng(seed)
    B = len(lengths)
    labels = np.full((B, T), -1, dtype=np.int32)
    seg = np.zeros((B, T), dtype=np.uint8)
    for b in range(B):
        L = int(lengths[b])
        t = 0
        while t < L:
            k = int(rng.integers(1, min(K, L - t) + 1))
            labels[b, t:t + k] = int(rng.integers(0, C))
            seg[b, t] = 1
            t += k
    return labels, seg
