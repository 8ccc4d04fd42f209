#!/usr/bin/env python3
"""Throughput of the streaming semi-CRF hot path on one MI355X.

One step = one pass of every hot-path stage over one batch of the genomic workload
(B=4, T=100,000, K=200, C=6, synthetic, seeded, checkpoint interval ceil(sqrt(TK)) =
4,473): semicrf_backward (centring + prefix scan, the checkpoint spans of both directions
swept at once, seam check, segment posteriors, marginals and gradients, log Z) and
semicrf_viterbi (prefix scan, max-plus spans, seam check, backtrace), issued on two
streams: the calls are independent and each keeps part of the chip busy.  Inputs are
resident in HBM before the timed region; W warm-up steps, then K timed steps between two
device synchronisations.  Prints one JSON line.

roofline: the dominant kernel of the fwd+bwd pass is the launch that sweeps every
checkpoint span of both directions (k_lse_round in span mode), timed live with the events
the library records on the stream it launches on.  Its algorithmic work is the factored
recurrence, (K*C + C^2) multiply-adds per position and direction (2 flops each, fp32), over
every position of both directions; the burn-in positions the spans add are reported beside
it.  The peak is the chip's fp32 vector rate (157.3 TFLOP/s: 256 CUs x 2.4 GHz x 256
flop/clock); the plain v_fma_f32 and v_exp_f32 rates measured on the same chip by
libsemicrf_peak.so are reported with it, and the VALU / transcendental instruction counts of
the launch from rocprofv3 counter runs (kept while the kernel sources match the ones the
counters were taken on).  HBM traffic likewise from FETCH_SIZE / WRITE_SIZE runs.
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
PEAK_FP32_FLOPS = 157.3e12       # MI355X fp32 vector: 256 CUs x 2.4 GHz x 256 flop/clock
PEAK_HBM_BPS = 8.0e12
CLOCK_HZ = 2.4e9
N_CU = 256
# Counter runs of the span-sweep launch at the bench shape (rocprofv3 --pmc, summarised in
# profiles/counters_k_lse_round_spans_genomic_B4_T1e5_K200_C6.md): instructions per
# dispatch, and HBM bytes (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, the factors a 1 GiB device
# copy reads), valid for the kernel sources with this SHA-256 (of their concatenation, in
# this order).  Empty until counters are taken on the current sources.
SWEEP_SRCS = [os.path.join(ROOT, "semi_markov_crf_amd", "csrc", f)
              for f in ("sweep_lse_round.h", "sweep_lse_kernel.h", "ring.h", "common.h",
                        "internal.h")]
SWEEP_COUNTERS = {"sha256": "0244f0f5b1363f7def4dadcf5e2c70e3dfd9768ba3dab55edcf571c721abad0d",
                  "delta": 1786, "valu": 191_963_364, "trans": 5_562_640,
                  "hbm_bytes": (24_244 * 2.0 + 47_885 * 1.0) * 1024}


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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


def measured_peaks():
    """Plain v_fma_f32, v_exp_f32 and interleaved rates of this chip (lane operations/s)."""
    path = os.path.join(ROOT, "semi_markov_crf_amd", "libsemicrf_peak.so")
    lib = ctypes.CDLL(path)
    lib.semicrf_peak_rates.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    out = (ctypes.c_double * 3)()
    if lib.semicrf_peak_rates(4096, 3, out) != 0:
        raise RuntimeError("semicrf_peak_rates failed")
    return {"fma_f32_lane_ops_per_s": out[0], "exp_f32_lane_ops_per_s": out[1],
            "exp_plus_fma_lane_ops_per_s": out[2],
            "fma_f32_per_cu_clock": out[0] / (N_CU * CLOCK_HZ),
            "exp_f32_per_cu_clock": out[1] / (N_CU * CLOCK_HZ)}


def _oracle_job(args):
    import oracle
    em_b, n, trans, dur, K = args
    t0 = time.perf_counter()
    oracle.sequence(em_b, n, trans, dur, K, want_viterbi=True, want_grads=True)
    return time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, sample_positions):
    """The fp64 oracle, untuned: forward, backward, posteriors and Viterbi over the first
    `sample_positions` positions of every sequence, one process per sequence."""
    import multiprocessing as mp
    usable = len(os.sched_getaffinity(0))
    workers = max(1, min(w.B, usable))
    jobs = [(w.em[b], sample_positions, w.trans, w.dur, w.K) for b in range(w.B)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        per_seq = pool.map(_oracle_job, jobs)
    wall = time.perf_counter() - t0
    pos = w.B * sample_positions
    return {"value": pos / wall, "unit": "positions/s", "cores": workers, "kind": "oracle",
            "sample": f"fwd+bwd+posteriors+viterbi over positions [0, {sample_positions}) of "
                      f"each of the {w.B} genomic sequences, fp64 NumPy, one process per "
                      f"sequence",
            "seconds": wall, "seconds_per_sequence": per_seq,
            "host": {"cpu_model": cpu_model(), "cpu_count": os.cpu_count(),
                     "usable_cores": usable}}


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


def config_timings(crf, d):
    """The other configurations: backward (log Z and every gradient), Viterbi and log Z
    alone, positions/s and nominal edges/s (B*T*K*C^2 per pass)."""
    import torch

    import workloads
    out = {}
    for i in (1, 3, 4):
        w = workloads.make(i)
        em, lengths, trans, dur = (torch.from_numpy(a).to(d) for a in
                                   (w.em, w.lengths, w.trans, w.dur))
        wsb = torch.empty(crf.workspace_bytes(crf.OP_BACKWARD, w.B, w.T, w.C, w.K),
                          dtype=torch.uint8, device=d)
        wsv = torch.empty(crf.workspace_bytes(crf.OP_VITERBI, w.B, w.T, w.C, w.K),
                          dtype=torch.uint8, device=d)
        wsl = torch.empty(crf.workspace_bytes(crf.OP_LOGZ, w.B, w.T, w.C, w.K),
                          dtype=torch.uint8, device=d)
        reps = 2 if i == 3 else 5
        mb = _time_ms(lambda: crf.backward(em, lengths, trans, dur, workspace=wsb), d, reps)
        mv = _time_ms(lambda: crf.viterbi(em, lengths, trans, dur, workspace=wsv), d, reps)
        ml = _time_ms(lambda: crf.logz(em, lengths, trans, dur, workspace=wsl), d, reps)
        pos = w.positions()
        edges = w.B * w.T * w.K * w.C * w.C
        out[w.name] = {"B": w.B, "T": w.T, "K": w.K, "C": w.C, "positions": pos,
                       "backward_ms": mb, "viterbi_ms": mv, "logz_ms": ml,
                       "fwd_bwd_positions_per_s": pos / (mb * 1e-3),
                       "viterbi_positions_per_s": pos / (mv * 1e-3),
                       "logz_positions_per_s": pos / (ml * 1e-3),
                       "fwd_bwd_edges_per_s_nominal": edges / (mb * 1e-3),
                       "kernel": "round kernel" if w.C <= 16 else "one barrier per position"}
        del wsb, wsv, wsl
    return out


def only_config(crf, d, name, reps, delta=0):
    """One other configuration alone: backward, Viterbi and log Z, each timed over reps
    calls after one untimed call (delta: the checkpoint interval of log Z and the backward,
    0 for the library default)."""
    import torch

    import workloads
    w = workloads.long_duration() if name == "long_duration" else \
        workloads.make({"speech": 1, "long": 3, "large_c": 4}[name])
    em, lengths, trans, dur = (torch.from_numpy(a).to(d) for a in (w.em, w.lengths, w.trans, w.dur))
    ws = {op: torch.empty(crf.workspace_bytes(op, w.B, w.T, w.C, w.K, delta), dtype=torch.uint8,
                          device=d)
          for op in (crf.OP_BACKWARD, crf.OP_VITERBI, crf.OP_LOGZ)}
    mb = _time_ms(lambda: crf.backward(em, lengths, trans, dur, delta=delta,
                                       workspace=ws[crf.OP_BACKWARD]), d, reps)
    mv = _time_ms(lambda: crf.viterbi(em, lengths, trans, dur, workspace=ws[crf.OP_VITERBI]), d,
                  reps)
    ml = _time_ms(lambda: crf.logz(em, lengths, trans, dur, delta=delta,
                                   workspace=ws[crf.OP_LOGZ]), d, reps)
    pos = w.positions()
    return {"config": name, "B": w.B, "T": w.T, "K": w.K, "C": w.C, "positions": pos,
            "reps": reps,
            "delta": delta or crf.default_interval(crf.OP_BACKWARD, w.B, w.T, w.C, w.K),
            "backward_ms": mb, "viterbi_ms": mv, "logz_ms": ml,
            "fwd_bwd_positions_per_s": pos / (mb * 1e-3)}


def extras(crf, w, em, lengths, trans, dur, d):
    """Timings beyond the step: the training loss of gold segmentations, the backward
    pass with boundary projections, log Z alone (all at the genomic shape), and the
    genome-scale long-duration workload (B=1, T=10^6, K=2000, C=6)."""
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
    wsl = torch.empty(crf.workspace_bytes(crf.OP_LOGZ, w.B, w.T, w.C, w.K), dtype=torch.uint8,
                      device=d)
    ml = _time_ms(lambda: crf.logz(em, lengths, trans, dur, workspace=wsl), d, 3)
    mlb = _time_ms(lambda: (crf.logz(em, lengths, trans, dur, workspace=wsl),
                            crf.backward(em, lengths, trans, dur, workspace=ws)), d, 3)
    out["logz"] = {"ms": ml, "positions_per_s": pos / (ml * 1e-3),
                   "logz_then_backward_ms": mlb,
                   "what": "semicrf_logz alone (inference), and semicrf_logz followed by "
                           "semicrf_backward, genomic shape"}
    g = torch.Generator(device="cpu").manual_seed(11)
    ps = torch.randn(em.shape, generator=g).to(d)
    pe = torch.randn(em.shape, generator=g).to(d)
    ms = _time_ms(lambda: crf.backward(em, lengths, trans, dur, proj_start=ps, proj_end=pe,
                                       workspace=ws), d, 3)
    out["projections"] = {"ms": ms, "positions_per_s": pos / (ms * 1e-3),
                          "what": "semicrf_backward with proj_start / proj_end N(0,1), their "
                                  "gradients and the boundary probabilities, genomic shape"}
    del ws, wsl
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


def span_positions(lengths, delta, warm):
    """Positions the span sweeps execute per direction: every span from its burn-in start
    (or 0) to its end."""
    n = 0
    for L in lengths:
        L = int(L)
        for t0 in range(0, L, delta):
            n += min(L, t0 + delta) - max(0, t0 - warm)
    return n


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--delta", type=int, default=0,
                    help="checkpoint interval of the backward (0: the library default)")
    ap.add_argument("--cpu-sample", type=int, default=12_000,
                    help="positions of every sequence the oracle baseline runs over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scan-roofline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configurations, the training loss, the projections "
                         "and the long-duration workload")
    ap.add_argument("--only-config", choices=("speech", "long", "large_c", "long_duration"),
                    help="time one other configuration alone (backward, Viterbi, log Z; for "
                         "profiling it) and print its timings instead of the step")
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
    if args.only_config:
        print(json.dumps(only_config(crf, torch.device("cuda:0"), args.only_config,
                                     max(1, args.steps), args.delta)), flush=True)
        return
    hip = hip_runtime()
    w = workloads.make(CONFIG)
    d = torch.device("cuda:0")
    em = torch.from_numpy(w.em).to(d)
    lengths = torch.from_numpy(w.lengths).to(d)
    trans = torch.from_numpy(w.trans).to(d)
    dur = torch.from_numpy(w.dur).to(d)
    B, T, C, K = w.B, w.T, w.C, w.K
    delta = (crf.checkpoint_interval(T, K, args.delta) if args.delta
             else crf.default_interval(crf.OP_BACKWARD, B, T, C, K))
    vdelta = crf.default_interval(crf.OP_VITERBI, B, T, C, K)
    nb = crf.workspace_bytes(crf.OP_BACKWARD, B, T, C, K, args.delta)
    nv = crf.workspace_bytes(crf.OP_VITERBI, B, T, C, K)
    ws_b = torch.empty(nb, dtype=torch.uint8, device=d)
    ws_v = torch.empty(nv, dtype=torch.uint8, device=d)
    g_em, g_tr, g_du = torch.empty_like(em), torch.empty_like(trans), torch.empty_like(dur)
    mu, lz = torch.empty_like(em), torch.empty(B, dtype=torch.float32, device=d)
    score = torch.empty(B, dtype=torch.float32, device=d)
    labels = torch.empty((B, T), dtype=torch.int32, device=d)
    seg = torch.empty((B, T), dtype=torch.uint8, device=d)
    rep_b = torch.empty(B, dtype=torch.int32, device=d)
    rep_v = torch.empty(B, dtype=torch.int32, device=d)
    bound_b = torch.empty(B, dtype=torch.float32, device=d)
    # semicrf_backward and semicrf_viterbi are independent: two streams (default priority)
    main = torch.cuda.current_stream(d)
    s_b, s_v = torch.cuda.Stream(d), torch.cuda.Stream(d)
    stream_b, stream_v = s_b.cuda_stream, s_v.cuda_stream
    stream = main.cuda_stream

    def _opt(ev, rep, bound=None):
        o = _native.options(seam_repairs=rep.data_ptr(),
                            seam_bound=None if bound is None else bound.data_ptr())
        if ev is not None:
            o.events = ctypes.cast(ev, ctypes.c_void_p).value
        return ctypes.byref(o)

    def step(ev_b=None, ev_v=None):
        rc = lib.semicrf_backward_ex(em.data_ptr(), lengths.data_ptr(), trans.data_ptr(),
                                     dur.data_ptr(), B, T, C, K, args.delta, stream_b,
                                     ws_b.data_ptr(), nb, None, g_em.data_ptr(), g_tr.data_ptr(),
                                     g_du.data_ptr(), mu.data_ptr(), lz.data_ptr(),
                                     _opt(ev_b, rep_b, bound_b))
        _native.check("semicrf_backward", rc)
        rc = lib.semicrf_viterbi_ex(em.data_ptr(), lengths.data_ptr(), trans.data_ptr(),
                                    dur.data_ptr(), B, T, C, K, stream_v, ws_v.data_ptr(), nv,
                                    score.data_ptr(), labels.data_ptr(), seg.data_ptr(),
                                    _opt(ev_v, rep_v))
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
    # dominant kernel of the fwd+bwd pass: the span sweeps of both directions (stage 1, one
    # launch)
    dom_ms = float(sb[:, 1].mean())
    flop_per_pos = 2 * (K * C + C * C)               # multiply-adds of the factored recurrence
    algo = 2 * positions * flop_per_pos              # both directions
    achieved = algo / (dom_ms * 1e-3)
    warm = max(3 * K, 64)
    executed_pos = 2 * span_positions(w.lengths, delta, warm)
    nspans = -(-T // delta)
    workgroups = B * nspans          # both directions of a span share a workgroup
    busy_cus = min(N_CU, workgroups)
    peaks = measured_peaks()
    same_src = sources_sha(SWEEP_SRCS) == SWEEP_COUNTERS.get("sha256")
    counted = None
    traffic = None
    if same_src and delta == SWEEP_COUNTERS.get("delta"):
        c = SWEEP_COUNTERS
        t = dom_ms * 1e-3
        counted = {
            "valu_insts_per_launch": c["valu"], "trans_f32_insts_per_launch": c["trans"],
            "valu_lane_ops_per_s": c["valu"] * 64 / t,
            "trans_lane_ops_per_s": c["trans"] * 64 / t,
            "valu_frac_of_measured_fma_peak": c["valu"] * 64 / t / peaks["fma_f32_lane_ops_per_s"],
            "trans_frac_of_measured_exp_peak": c["trans"] * 64 / t / peaks["exp_f32_lane_ops_per_s"],
            "valu_issue_frac_busy_cus": c["valu"] / t / (busy_cus * CLOCK_HZ *
                                                          peaks["fma_f32_per_cu_clock"] / 64),
            "source": "profiles/counters_k_lse_round_spans_genomic_B4_T1e5_K200_C6.md"}
        traffic = c.get("hbm_bytes")

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
                               f"({nspans} checkpoint spans; decode {vdelta}); step = "
                               f"semicrf_backward + semicrf_viterbi",
                   "B": B, "T": T, "K": K, "C": C, "delta": delta, "viterbi_delta": vdelta,
                   "parallelism": "none (1 GPU)"},
        "roofline": {
            "bound": "alu",
            "kernel": "k_lse_round, span mode: every checkpoint span of both directions of "
                      "every sequence at once, the two directions of a span in one "
                      "workgroup, one launch",
            "achieved": achieved / 1e12,
            "peak": PEAK_FP32_FLOPS / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_FLOPS,
            "traffic": traffic,
            "algorithmic_per_launch": algo,
            "algorithmic_unit": f"fp32 flop: 2 directions x positions x 2 x (K*C + C^2) = "
                                f"2 x {positions} x {flop_per_pos}",
            "executed_positions_per_launch": executed_pos,
            "launch_ms": dom_ms,
            "workgroups": workgroups,
            "busy_cus": busy_cus,
            "frac_of_busy_cus": achieved / (PEAK_FP32_FLOPS * busy_cus / N_CU),
            "measured_peaks": peaks,
            "counted": counted,
        },
        "stages_ms": {
            "backward": dict(zip(["prefix", "span_sweeps", "seam_check_and_repair",
                                  "posteriors", "marginals_grads"],
                                 sb.mean(axis=0).round(4).tolist())),
            "viterbi": dict(zip(["prefix", "maxplus_spans_seam_repair", "backtrace"],
                                sv.mean(axis=0).round(4).tolist())),
        },
        "seam_repairs": {"backward": int(rep_b.sum().item()), "viterbi": int(rep_v.sum().item())},
        "seam_bound_max": float(bound_b.max().item()),
        "fwd_bwd_positions_per_s": positions / (bwd_ms * 1e-3),
        "viterbi_positions_per_s": positions / (vit_ms * 1e-3),
        "edges_per_s_nominal": positions * K * C * C / (bwd_ms * 1e-3),
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
        nbytes = Bs * Ts * C * (4 + 4 + 8)        # em read twice (mean, then scan), S written fp64
        nbytes12 = Bs * Ts * C * 12               # the same with S in fp32
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
                                "frac_on_12C_bytes": nbytes12 / (ms * 1e-3) / PEAK_HBM_BPS,
                                "device_copy_GBps": 2 * S_big.numel() * 8 / (cms * 1e-3) / 1e9}
        del em_big, S_big, S_copy, ws_s

    if not args.no_extras:
        out["configs"] = config_timings(crf, d)
        out["extras"] = extras(crf, w, em, lengths, trans, dur, d)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
