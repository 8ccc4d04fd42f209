"""MI355X (gfx950) streaming semi-Markov CRF: Python binding of the C ABI.

The functions below only marshal arguments: they check devices, dtypes and
shapes, allocate the outputs and the workspace with PyTorch (which supplies
device memory and the current stream) and call ``libsemicrf.so``.  Every step of
the computation runs in the library's HIP kernels.

    logz(em, lengths, trans, dur)            -> log Z  [B]
    backward(em, lengths, trans, dur, ...)   -> gradients, marginals, log Z, boundaries
    viterbi(em, lengths, trans, dur)         -> best score, labels, segment starts
    nll(em, lengths, trans, dur, gold...)    -> training loss of gold segmentations
    log_partition(em, lengths, trans, dur)   -> log Z with autograd support

Shapes: em [B, T, C] float32, lengths [B] int32, trans [C, C] float32 (row =
previous label), dur [K, C] float32 (row k-1 scores length k).  Every call also
takes optional boundary projections proj_start / proj_end [B, T, C] float32: a
segment [s, e) of label c gains proj_start[b, s, c] + proj_end[b, e-1, c].
"""

from __future__ import annotations

import torch

from . import _native
from ._native import OP_BACKWARD, OP_LOGZ, OP_PREFIX, OP_VITERBI, SemiCRFError

__all__ = ["prefix", "logz", "backward", "viterbi", "nll", "log_partition", "workspace_bytes",
           "checkpoint_interval", "default_interval", "read_status", "SemiCRFError",
           "OP_LOGZ", "OP_BACKWARD", "OP_VITERBI", "OP_PREFIX"]


def checkpoint_interval(T: int, K: int, delta: int = 0) -> int:
    return int(_native.load().semicrf_checkpoint_interval(T, K, delta))


def default_interval(op: int, B: int, T: int, C: int, K: int) -> int:
    """Checkpoint interval `op` uses for delta = 0."""
    return int(_native.load().semicrf_default_interval(op, B, T, C, K))


def workspace_bytes(op: int, B: int, T: int, C: int, K: int, delta: int = 0) -> int:
    return int(_native.load().semicrf_workspace_bytes(op, B, T, C, K, delta))


def prefix(em, lengths, *, workspace=None, check_status=False) -> torch.Tensor:
    """Centred prefix sums S [B, T+1, C] float64."""
    if em.dim() != 3 or em.dtype != torch.float32 or lengths.dtype != torch.int32:
        raise TypeError("emissions float32 [B, T, C] and lengths int32 [B] required")
    if em.device.type != "cuda" or lengths.device != em.device:
        raise ValueError("emissions and lengths must be on the same GPU")
    if not (em.is_contiguous() and lengths.is_contiguous()) or lengths.shape != em.shape[:1]:
        raise ValueError("contiguous emissions [B, T, C] and lengths [B] required")
    B, T, C = (int(v) for v in em.shape)
    ws, n = _workspace(OP_PREFIX, B, T, C, 1, 0, em.device, workspace)
    S = torch.empty((B, T + 1, C), dtype=torch.float64, device=em.device)
    rc = _native.load().semicrf_prefix(em.data_ptr(), lengths.data_ptr(), B, T, C,
                                       _stream(em.device), ws.data_ptr(), n, S.data_ptr())
    _native.check("semicrf_prefix", rc)
    _maybe_check(ws, check_status, "semicrf_prefix")
    return S


def _check_inputs(em, lengths, trans, dur):
    for name, t, dt in (("emissions", em, torch.float32), ("lengths", lengths, torch.int32),
                        ("trans", trans, torch.float32), ("dur", dur, torch.float32)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != em.device:
            raise ValueError(f"{name} is on {t.device}, emissions on {em.device}")
    if em.dim() != 3:
        raise ValueError("emissions must be [B, T, C]")
    B, T, C = em.shape
    if lengths.shape != (B,) or trans.shape != (C, C) or dur.dim() != 2 or dur.shape[1] != C:
        raise ValueError("shape mismatch: lengths [B], trans [C, C], dur [K, C] required")
    return int(B), int(T), int(C), int(dur.shape[0])


def _workspace(op, B, T, C, K, delta, device, workspace):
    n = workspace_bytes(op, B, T, C, K, delta)
    if n == 0:
        raise SemiCRFError("semicrf_workspace_bytes", 3)
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    if workspace.numel() < n or workspace.data_ptr() % 256:
        raise ValueError(f"workspace must hold {n} bytes, 256-byte aligned")
    return workspace, n


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def read_status(workspace: torch.Tensor) -> int:
    """Device status flag of the last call that used ``workspace`` (synchronises)."""
    return int(_native.load().semicrf_read_status(workspace.data_ptr(),
                                                  _stream(workspace.device)))


def _maybe_check(workspace, check_status, fn):
    if check_status:
        _native.check(fn, read_status(workspace))


def _proj(em, proj_start, proj_end):
    """Checked projection pointers (None for an absent array) and the tensors to keep."""
    out = []
    for name, x in (("proj_start", proj_start), ("proj_end", proj_end)):
        if x is None:
            out.append(None)
            continue
        if x.shape != em.shape or x.dtype != torch.float32 or x.device != em.device:
            raise ValueError(f"{name} must be a float32 tensor shaped like the emissions, on "
                             f"their device")
        out.append(x.contiguous())
    return out


def _ptr(x):
    return None if x is None else x.data_ptr()


def _options(**fields):
    """Options struct for the *_ex calls (None when every field is NULL)."""
    fields = {k: v for k, v in fields.items() if v is not None}
    return _native.options(**fields) if fields else None


def _seams(B, dev, want):
    if not want:
        return None, None
    return (torch.empty(B, dtype=torch.float32, device=dev),
            torch.empty(B, dtype=torch.int32, device=dev))


def logz(em, lengths, trans, dur, *, proj_start=None, proj_end=None, delta=0, workspace=None,
         seam_tolerance=0.0, want_seams=False, check_status=False):
    """log Z [B].  With want_seams, returns (log Z, seam_bound [B], seam_repairs [B]) (see
    semicrf_options in include/semicrf.h); seam_tolerance < 0 forces the in-order sweep."""
    B, T, C, K = _check_inputs(em, lengths, trans, dur)
    ps, pe = _proj(em, proj_start, proj_end)
    ws, n = _workspace(OP_LOGZ, B, T, C, K, delta, em.device, workspace)
    out = torch.empty(B, dtype=torch.float32, device=em.device)
    sb, sr = _seams(B, em.device, want_seams)
    opt = _options(proj_start=_ptr(ps), proj_end=_ptr(pe), seam_bound=_ptr(sb),
                   seam_repairs=_ptr(sr), seam_tolerance=float(seam_tolerance) or None)
    rc = _native.load().semicrf_logz_ex(em.data_ptr(), lengths.data_ptr(), trans.data_ptr(),
                                        dur.data_ptr(), B, T, C, K, delta, _stream(em.device),
                                        ws.data_ptr(), n, out.data_ptr(), opt)
    _native.check("semicrf_logz", rc)
    _maybe_check(ws, check_status, "semicrf_logz")
    return (out, sb, sr) if want_seams else out


def backward(em, lengths, trans, dur, *, proj_start=None, proj_end=None, grad_log_z=None,
             delta=0, want_marginals=True, want_boundaries=False, want_node_mass=False,
             seam_tolerance=0.0, want_seams=False, workspace=None, check_status=False) -> dict:
    """Gradients of sum_b grad_log_z[b] * log Z_b (all ones when None).  Returns a dict
    with grad_em [B,T,C], grad_trans [C,C], grad_dur [K,C], marginals [B,T,C] (or
    None) and log_z [B]; with want_boundaries (or projections given) also
    grad_proj_start / grad_proj_end [B,T,C] and boundary [B,T], the probability that a
    segment starts at t; with want_node_mass the per-position sum over labels of the
    marginals before normalisation, node_mass [B,T]; with want_seams seam_bound [B] and
    seam_repairs [B] (semicrf_options); seam_tolerance < 0 forces the in-order sweeps."""
    B, T, C, K = _check_inputs(em, lengths, trans, dur)
    dev = em.device
    ps, pe = _proj(em, proj_start, proj_end)
    want_b = want_boundaries or ps is not None or pe is not None
    if grad_log_z is not None:
        if grad_log_z.shape != (B,) or grad_log_z.dtype != torch.float32 or grad_log_z.device != dev:
            raise ValueError("grad_log_z must be a float32 [B] tensor on the emissions' device")
        grad_log_z = grad_log_z.contiguous()
    ws, n = _workspace(OP_BACKWARD, B, T, C, K, delta, dev, workspace)
    grad_em = torch.empty_like(em)
    grad_trans = torch.empty_like(trans)
    grad_dur = torch.empty_like(dur)
    mu = torch.empty_like(em) if want_marginals else None
    lz = torch.empty(B, dtype=torch.float32, device=dev)
    gps = torch.empty_like(em) if want_b else None
    gpe = torch.empty_like(em) if want_b else None
    bnd = torch.empty((B, T), dtype=torch.float32, device=dev) if want_b else None
    nm = torch.empty((B, T), dtype=torch.float32, device=dev) if want_node_mass else None
    sb, sr = _seams(B, dev, want_seams)
    opt = _options(proj_start=_ptr(ps), proj_end=_ptr(pe), grad_proj_start=_ptr(gps),
                   grad_proj_end=_ptr(gpe), boundary=_ptr(bnd), node_mass=_ptr(nm),
                   seam_bound=_ptr(sb), seam_repairs=_ptr(sr),
                   seam_tolerance=float(seam_tolerance) or None)
    rc = _native.load().semicrf_backward_ex(
        em.data_ptr(), lengths.data_ptr(), trans.data_ptr(), dur.data_ptr(), B, T, C, K, delta,
        _stream(dev), ws.data_ptr(), n, _ptr(grad_log_z), grad_em.data_ptr(),
        grad_trans.data_ptr(), grad_dur.data_ptr(), _ptr(mu), lz.data_ptr(), opt)
    _native.check("semicrf_backward", rc)
    _maybe_check(ws, check_status, "semicrf_backward")
    out = {"grad_em": grad_em, "grad_trans": grad_trans, "grad_dur": grad_dur,
           "marginals": mu, "log_z": lz}
    if want_b:
        out.update(grad_proj_start=gps, grad_proj_end=gpe, boundary=bnd)
    if want_node_mass:
        out["node_mass"] = nm
    if want_seams:
        out.update(seam_bound=sb, seam_repairs=sr)
    return out


def nll(em, lengths, trans, dur, gold_labels, gold_seg_start, *, proj_start=None,
        proj_end=None, grad_nll=None, delta=0, workspace=None, check_status=False) -> dict:
    """Training loss of gold segmentations, nll[b] = log Z_b - score_b(y*), and the
    gradients of sum_b grad_nll[b] * nll[b] (all ones when None).  gold_labels int32
    [B,T] and gold_seg_start uint8 [B,T] on the emissions' device.  Returns a dict with
    nll [B], grad_em [B,T,C], grad_trans [C,C], grad_dur [K,C] and, with projections,
    grad_proj_start / grad_proj_end [B,T,C]."""
    B, T, C, K = _check_inputs(em, lengths, trans, dur)
    dev = em.device
    ps, pe = _proj(em, proj_start, proj_end)
    want_p = ps is not None or pe is not None
    for name, x, dt in (("gold_labels", gold_labels, torch.int32),
                        ("gold_seg_start", gold_seg_start, torch.uint8)):
        if x.shape != (B, T) or x.dtype != dt or x.device != dev:
            raise ValueError(f"{name} must be a {dt} [B, T] tensor on the emissions' device")
    if grad_nll is not None:
        if grad_nll.shape != (B,) or grad_nll.dtype != torch.float32 or grad_nll.device != dev:
            raise ValueError("grad_nll must be a float32 [B] tensor on the emissions' device")
        grad_nll = grad_nll.contiguous()
    gold_labels, gold_seg_start = gold_labels.contiguous(), gold_seg_start.contiguous()
    ws, n = _workspace(OP_BACKWARD, B, T, C, K, delta, dev, workspace)
    out = torch.empty(B, dtype=torch.float32, device=dev)
    grad_em = torch.empty_like(em)
    grad_trans = torch.empty_like(trans)
    grad_dur = torch.empty_like(dur)
    gps = torch.empty_like(em) if want_p else None
    gpe = torch.empty_like(em) if want_p else None
    opt = _options(proj_start=_ptr(ps), proj_end=_ptr(pe), grad_proj_start=_ptr(gps),
                   grad_proj_end=_ptr(gpe))
    rc = _native.load().semicrf_nll(
        em.data_ptr(), lengths.data_ptr(), trans.data_ptr(), dur.data_ptr(),
        gold_labels.data_ptr(), gold_seg_start.data_ptr(), B, T, C, K, delta, _stream(dev),
        ws.data_ptr(), n, _ptr(grad_nll), out.data_ptr(), grad_em.data_ptr(),
        grad_trans.data_ptr(), grad_dur.data_ptr(), opt)
    _native.check("semicrf_nll", rc)
    _maybe_check(ws, check_status, "semicrf_nll")
    res = {"nll": out, "grad_em": grad_em, "grad_trans": grad_trans, "grad_dur": grad_dur}
    if want_p:
        res.update(grad_proj_start=gps, grad_proj_end=gpe)
    return res


def viterbi(em, lengths, trans, dur, *, proj_start=None, proj_end=None, workspace=None,
            seam_tolerance=0.0, want_seams=False, check_status=False):
    """Returns (best_score [B] float32, labels [B,T] int32, seg_start [B,T] uint8), and with
    want_seams also seam_bound [B] and seam_repairs [B] (semicrf_options)."""
    B, T, C, K = _check_inputs(em, lengths, trans, dur)
    dev = em.device
    ps, pe = _proj(em, proj_start, proj_end)
    ws, n = _workspace(OP_VITERBI, B, T, C, K, 0, dev, workspace)
    score = torch.empty(B, dtype=torch.float32, device=dev)
    labels = torch.empty((B, T), dtype=torch.int32, device=dev)
    seg = torch.empty((B, T), dtype=torch.uint8, device=dev)
    sb, sr = _seams(B, dev, want_seams)
    opt = _options(proj_start=_ptr(ps), proj_end=_ptr(pe), seam_bound=_ptr(sb),
                   seam_repairs=_ptr(sr), seam_tolerance=float(seam_tolerance) or None)
    rc = _native.load().semicrf_viterbi_ex(em.data_ptr(), lengths.data_ptr(), trans.data_ptr(),
                                           dur.data_ptr(), B, T, C, K, _stream(dev),
                                           ws.data_ptr(), n, score.data_ptr(), labels.data_ptr(),
                                           seg.data_ptr(), opt)
    _native.check("semicrf_viterbi", rc)
    _maybe_check(ws, check_status, "semicrf_viterbi")
    if want_seams:
        return score, labels, seg, sb, sr
    return score, labels, seg


class _LogPartition(torch.autograd.Function):
    @staticmethod
    def forward(ctx, em, lengths, trans, dur, proj_start, proj_end, delta):
        ctx.save_for_backward(em, lengths, trans, dur, proj_start, proj_end)
        ctx.delta = delta
        return logz(em, lengths, trans, dur, proj_start=proj_start, proj_end=proj_end,
                    delta=delta)

    @staticmethod
    def backward(ctx, g):
        em, lengths, trans, dur, ps, pe = ctx.saved_tensors
        out = backward(em, lengths, trans, dur, proj_start=ps, proj_end=pe,
                       grad_log_z=g.contiguous().float(), delta=ctx.delta, want_marginals=False)
        return (out["grad_em"], None, out["grad_trans"], out["grad_dur"],
                out.get("grad_proj_start") if ps is not None else None,
                out.get("grad_proj_end") if pe is not None else None, None)


def log_partition(em, lengths, trans, dur, proj_start=None, proj_end=None,
                  delta: int = 0) -> torch.Tensor:
    """log Z [B] as a differentiable op (a drop-in CRF-layer loss term); the optional
    boundary projections receive gradients too."""
    return _LogPartition.apply(em, lengths, trans, dur, proj_start, proj_end, delta)
