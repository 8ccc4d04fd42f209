#!/usr/bin/env python3
"""Throughput of the streaming semi-CRF hot path on one MI355X.

One step = one pass of every hot-path stage over one batch of the genomic
workload (B=4, T=100,000, K=200, C=6, synthetic, seeded): semicrf_backward
(centring + prefix scan, forward and backward checkpoint sweeps, span recompute,
segment posteriors, marginals and gradients, log Z) and semicrf_viterbi (prefix
scan, max-plus sweep, backtrace), issued on two streams: the two calls are
independent and their sweeps occupy few compute units, so they run side by side.  Inputs are resident in HBM before the
timed region; W warm-up steps, then K timed steps between two device
synchronisations.  Prints one JSON line.

The roofline object describes the dominant kernel (the checkpoint sweep pair,
timed live with events recorded by the library on the stream it launches on):
algorithmic transcendental operations per launch / its mean duration, against the
chip's exp2/log2 issue rate (256 CUs x 32 lanes/clock x 2.4 GHz: transcendentals
issue at half the 64 lanes/clock of plain fp32 ops on gfx950).  Its HBM traffic comes
from FETCH_SIZE / WRITE_SIZE counter runs calibrated on a plain copy; it is reported
only while the kernel source is the one those counters were taken on.  The centring +
prefix scan is also reported against HBM bandwidth on a shape larger than the
256 MB last-level cache.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CONFIG = 2                       # genomic: B=4, T=1e5, K=200, C=6
PEAK_TRANS_PER_S = 256 * 32 * 2.4e9     # exp2/log2 issue: half of 64 lanes/clock per CU
PEAK_HBM_BPS = 8.0e12
# HBM bytes per checkpoint-sweep launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per
# dispatch, scaled by 2.0 / 1.0, what the counters read for a 1 GiB copy), valid for the
# kernel sources with this SHA-256 (of their concatenation, in this order)
SWEEP_SRCS = [os.path.join(ROOT, "semi_markov_crf_amd", "csrc", f)
              for f in ("sweep_lse_round.h", "sweep_lse_kernel.h", "ring.h", "common.h")]
SWEEP_TRAFFIC = {"sha256": "80e4448cf00fc0a04cf04d3cfa50108d320defcbb64f09c74720172186c70928",
                 "bytes": (19112.97 * 2.0 + 840.0 * 1.0) * 1024}


def hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so.7")       # the runtime torch already loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


class EventSet:
    """n+1 HIP events per step for a staged call (stage i spans events i..i+1)."""

    def __init__(self, hip, steps, nstages):
        self.hip, self.n = hip, nstages + 1
        self.arr = [(ctypes.c_void_p * self.n)() for _ in range(steps)]
        for a in self.arr:
            for i in range(self.n):
                p = ctypes.c_void_p()
                assert hip.hipEventCreate(ctypes.byref(p)) == 0
                a[i] = p.value

    def stage_ms(self):
        out = []
        for a in self.arr:
            row = []
            for i in range(self.n - 1):
                ms = ctypes.c_float()
                assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a[i], a[i + 1]) == 0
                row.append(ms.value)
            out.append(row)
        return out

    def close(self):
        for a in self.arr:
            for i in range(self.n):
                self.hip.hipEventDestroy(a[i])


def cpu_baseline(w, sample_positions):
    """The fp64 oracle (untuned) on one host core: forward, backward, posteriors and
    Viterbi over the first `sample_positions` positions of sequence 0."""
    import oracle
    t0 = time.perf_counter()
    oracle.sequence(w.em[0], sample_positions, w.trans, w.dur, w.K, want_viterbi=True,
                    want_grads=True)
    dt = time.perf_counter() - t0
    return {"value": sample_positions / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"fwd+bwd+posteriors+viterbi over positions [0, {sample_positions}) of "
                      f"sequence 0 of the genomic workload, fp64 NumPy, one process",
            "seconds": dt}


def _time_ms(fn, d, reps):
    """Mean device time of fn() over reps calls after one untimed call (events on the
    current stream, which the binding launches on)."""
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(d)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize(d)
    return e0.elapsed_time(e1) / reps


def extras(crf, w, em, lengths, trans, dur, d):
    """Timings beyond the step: the training loss of gold segmentations and the backward
    pass with boundary projections (both at the genomic shape), and the genome-scale
    long-duration workload (B=1, T=10^6, K=2000, C=6: backward and Viterbi)."""
    import numpy as np
    import torch

    import workloads
    out = {}
    pos = w.positions()
    ws = torch.empty(crf.workspace_bytes(crf.OP_BACKWARD, w.B, w.T, w.C, w.K), dtype=torch.uint8,
                     device=d)
    labels, seg = workloads.gold_segmentation(7, w.lengths, w.T, w.C, w.K)
    gl, gs = torch.from_numpy(labels).to(d), torch.from_numpy(seg).to(d)
    ms = _time_ms(lambda: crf.nll(em, lengths, trans, dur, gl, gs, workspace=ws), d, 3)
    ms0 = _time_ms(lambda: crf.backward(em, lengths, trans, dur, workspace=ws), d, 3)
    out["nll"] = {"ms": ms, "positions_per_s": pos / (ms * 1e-3), "backward_alone_ms": ms0,
                  "what": "semicrf_nll (backward pass + gold-segmentation kernels), genomic shape"}
    # inference alone, and an autograd-style forward then backward as two calls
    ml = _time_ms(lambda: crf.logz(em, lengths, trans, dur, workspace=ws), d, 3)
    mlb = _time_ms(lambda: (crf.logz(em, lengths, trans, dur, workspace=ws),
                            crf.backward(em, lengths, trans, dur, workspace=ws)), d, 3)
    out["logz"] = {"ms": ml, "positions_per_s": pos / (ml * 1e-3),
                   "logz_then_backward_ms": mlb,
                   "what": "semicrf_logz alone (one forward sweep per sequence), and semicrf_logz "
                           "followed by semicrf_backward, genomic shape"}
    g = torch.Generator(device="cpu").manual_seed(11)
    ps = torch.randn(em.shape, generator=g).to(d)
    pe = torch.randn(em.shape, generator=g).to(d)
    ms = _time_ms(lambda: crf.backward(em, lengths, trans, dur, proj_start=ps, proj_end=pe,
                                       workspace=ws), d, 3)
    out["projections"] = {"ms": ms, "positions_per_s": pos / (ms * 1e-3),
                          "what": "semicrf_backward with proj_start / proj_end N(0,1), their "
                                  "gradients and the boundary probabilities, genomic shape"}
    del ws
    x = workloads.long_duration()
    xe, xl, xt, xd = (torch.from_numpy(a).to(d) for a in (x.em, x.lengths, x.trans, x.dur))
    wsb = torch.empty(crf.workspace_bytes(crf.OP_BACKWARD, x.B, x.T, x.C, x.K), dtype=torch.uint8,
                      device=d)
    wsv = torch.empty(crf.workspace_bytes(crf.OP_VITERBI, x.B, x.T, x.C, x.K), dtype=torch.uint8,
                      device=d)
    mb = _time_ms(lambda: crf.backward(xe, xl, xt, xd, workspace=wsb), d, 1)
    mv = _time_ms(lambda: crf.viterbi(xe, xl, xt, xd, workspace=wsv), d, 1)
    lz = crf.backward(xe, xl, xt, xd, workspace=wsb)["log_z"]
    assert np.isfinite(lz.cpu().numpy()).all() and crf.read_status(wsb) == 0
    out["long_duration"] = {"B": x.B, "T": x.T, "K": x.K, "C": x.C, "backward_ms": mb,
                            "viterbi_ms": mv, "fwd_bwd_positions_per_s": x.positions() / (mb * 1e-3),
                            "viterbi_positions_per_s": x.positions() / (mv * 1e-3)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--delta", type=int, default=0, help="checkpoint interval (0: ceil(sqrt(TK)))")
    ap.add_argument("--cpu-sample", type=int, default=40_000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scan-roofline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the timings of the training loss, the projections and the "
                         "long-duration workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import semi_markov_crf_amd as crf
    import workloads
    from semi_markov_crf_amd import _native

    lib = _native.load()
    hip = hip_runtime()
    w = workloads.make(CONFIG)
    d = torch.device("cuda:0")
    em = torch.from_numpy(w.em).to(d)
    lengths = torch.from_numpy(w.lengths).to(d)
    trans = torch.from_numpy(w.trans).to(d)
    dur = torch.from_numpy(w.dur).to(d)
    B, T, C, K = w.B, w.T, w.C, w.K
    delta = crf.checkpoint_interval(T, K, args.delta)
    nb = crf.workspace_bytes(crf.OP_BACKWARD, B, T, C, K, args.delta)
    nv = crf.workspace_bytes(crf.OP_VITERBI, B, T, C, K)
    ws_b = torch.empty(nb, dtype=torch.uint8, device=d)
    ws_v = torch.empty(nv, dtype=torch.uint8, device=d)
    g_em, g_tr, g_du = torch.empty_like(em), torch.empty_like(trans), torch.empty_like(dur)
    mu, lz = torch.empty_like(em), torch.empty(B, dtype=torch.float32, device=d)
    score = torch.empty(B, dtype=torch.float32, device=d)
    labels = torch.empty((B, T), dtype=torch.int32, device=d)
    seg = torch.empty((B, T), dtype=torch.uint8, device=d)
    # semicrf_backward and semicrf_viterbi are independent and each keeps only 2B (resp. B)
    # compute units busy in its sweeps, so they run on two streams (default priority)
    main = torch.cuda.current_stream(d)
    s_b, s_v = torch.cuda.Stream(d), torch.cuda.Stream(d)
    stream_b, stream_v = s_b.cuda_stream, s_v.cuda_stream
    stream = main.cuda_stream

    def _opt(ev):
        if ev is None:
            return None
        return ctypes.byref(_native.options(events=ctypes.cast(ev, ctypes.c_void_p).value))

    def step(ev_b=None, ev_v=None):
        rc = lib.semicrf_backward_ex(em.data_ptr(), lengths.data_ptr(), trans.data_ptr(),
                                     dur.data_ptr(), B, T, C, K, args.delta, stream_b,
                                     ws_b.data_ptr(), nb, None, g_em.data_ptr(), g_tr.data_ptr(),
                                     g_du.data_ptr(), mu.data_ptr(), lz.data_ptr(), _opt(ev_b))
        _native.check("semicrf_backward", rc)
        rc = lib.semicrf_viterbi_ex(em.data_ptr(), lengths.data_ptr(), trans.data_ptr(),
                                    dur.data_ptr(), B, T, C, K, stream_v, ws_v.data_ptr(), nv,
                                    score.data_ptr(), labels.data_ptr(), seg.data_ptr(),
                                    _opt(ev_v))
        _native.check("semicrf_viterbi", rc)

    torch.cuda.synchronize(d)          # inputs are resident before either stream starts
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(d)
    assert crf.read_status(ws_b) == 0 and crf.read_status(ws_v) == 0

    evb = EventSet(hip, args.steps, _native.STAGES["backward"])
    evv = EventSet(hip, args.steps, _native.STAGES["viterbi"])
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(d)
    wall0 = time.perf_counter()
    t_start.record(main)
    s_b.wait_stream(main)
    s_v.wait_stream(main)
    for i in range(args.steps):
        step(evb.arr[i], evv.arr[i])
    main.wait_stream(s_b)
    main.wait_stream(s_v)
    t_end.record(main)
    torch.cuda.synchronize(d)
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    sb = np.array(evb.stage_ms())
    sv = np.array(evv.stage_ms())
    evb.close(); evv.close()
    assert np.isfinite(lz.cpu().numpy()).all()

    positions = w.positions()
    value = positions / (ms_step * 1e-3)
    bwd_ms = float(sb.sum(axis=1).mean())
    vit_ms = float(sv.sum(axis=1).mean())
    # dominant kernel: both checkpoint sweeps in one launch (stage 1), or the span
    # recompute when delta >= T
    nspans = -(-T // delta)
    dom_stage = 1 if nspans > 1 else 2
    dom_ms = float(sb[:, dom_stage].mean())
    trans_per_pos = K * C + C * C + 2 * C          # exp2 of the K*C and C*C terms, 2C log2
    algo = 2 * positions * trans_per_pos           # both directions
    achieved = algo / (dom_ms * 1e-3)
    busy_cus = 2 * B if dom_stage == 1 else min(256, 2 * B * nspans)
    # algorithmic bytes of the sweep pair: S read once per direction, checkpoints written
    nck = sum(max(0, (int(L) - 1) // delta) for L in w.lengths)
    algo_bytes = 2 * B * (T + 1) * C * 8 + 2 * nck * (K * C * 4 + C * 8 + C * 4 + 8)
    digest = hashlib.sha256()
    for src in SWEEP_SRCS:
        with open(src, "rb") as f:
            digest.update(f.read())
    same_src = digest.hexdigest() == SWEEP_TRAFFIC["sha256"]
    traffic = SWEEP_TRAFFIC["bytes"] if (same_src and dom_stage == 1 and delta == 4473) else None

    out = {
        "metric": "fwd+bwd positions/s at T=1e5,K=200,C=6; % of VALU-exp/HBM roofline",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"genomic semi-CRF B={B} T={T} K={K} C={C}, delta={delta} "
                               f"({nspans} checkpoint spans); step = semicrf_backward + "
                               f"semicrf_viterbi",
                   "B": B, "T": T, "K": K, "C": C, "delta": delta, "parallelism": "none (1 GPU)"},
        "roofline": {
            "bound": "alu",
            "kernel": "k_lse_round (checkpoint sweeps: forward and backward of every sequence, "
                      "one workgroup each, one launch)",
            "achieved": achieved / 1e12,
            "peak": PEAK_TRANS_PER_S / 1e12,
            "unit": "Ttrans/s",
            "frac": achieved / PEAK_TRANS_PER_S,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes,
            "algorithmic_per_launch": algo,
            "launch_ms": dom_ms,
            "busy_cus": busy_cus,
            "frac_of_busy_cus": achieved / (PEAK_TRANS_PER_S * busy_cus / 256),
        },
        "stages_ms": {
            "backward": dict(zip(["prefix", "ckpt_sweeps", "span_recompute", "posteriors",
                                  "marginals_grads"], sb.mean(axis=0).round(4).tolist())),
            "viterbi": dict(zip(["prefix", "maxplus_sweep", "backtrace"],
                                sv.mean(axis=0).round(4).tolist())),
        },
        "fwd_bwd_positions_per_s": positions / (bwd_ms * 1e-3),
        "viterbi_positions_per_s": positions / (vit_ms * 1e-3),
        "edges_per_s_nominal": positions * K * C * C / (bwd_ms * 1e-3),
        # recurrence passes over every position in one backward call: the forward and the
        # mirrored checkpoint sweeps, then the span recompute in both directions
        "recurrence_passes": 4,
        "wall_s_timed_region": wall,
    }

    if not args.no_scan_roofline:
        # centring + prefix scan alone on a shape far larger than the last-level cache
        Bs, Ts = 64, 1 << 20
        em_big = torch.randn((Bs, Ts, C), dtype=torch.float32, device=d)
        len_big = torch.full((Bs,), Ts, dtype=torch.int32, device=d)
        S_big = torch.empty((Bs, Ts + 1, C), dtype=torch.float64, device=d)
        nws = crf.workspace_bytes(crf.OP_PREFIX, Bs, Ts, C, 1)
        ws_s = torch.empty(nws, dtype=torch.uint8, device=d)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(4):
            e0.record()
            _native.check("semicrf_prefix", lib.semicrf_prefix(
                em_big.data_ptr(), len_big.data_ptr(), Bs, Ts, C, stream, ws_s.data_ptr(), nws,
                S_big.data_ptr()))
            e1.record()
            torch.cuda.synchronize(d)
            times.append(e0.elapsed_time(e1))
        ms = min(times[1:])
        nbytes = Bs * Ts * C * (4 + 4 + 8)        # em read twice (mean, then scan), S written
        # for scale: a plain device copy of S (read and write 8 B per element)
        S_copy = torch.empty_like(S_big)
        ctimes = []
        for _ in range(4):
            e0.record()
            S_copy.copy_(S_big)
            e1.record()
            torch.cuda.synchronize(d)
            ctimes.append(e0.elapsed_time(e1))
        cms = min(ctimes[1:])
        out["scan_roofline"] = {"bound": "hbm", "shape": f"B={Bs} T={Ts} C={C}",
                                "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": 8000.0,
                                "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / PEAK_HBM_BPS,
                                "ms": ms, "algorithmic_bytes": nbytes,
                                "device_copy_GBps": 2 * S_big.numel() * 8 / (cms * 1e-3) / 1e9}
        del em_big, S_big, S_copy, ws_s

    if not args.no_extras:
        out["extras"] = extras(crf, w, em, lengths, trans, dur, d)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
