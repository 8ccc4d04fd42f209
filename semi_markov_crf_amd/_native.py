"""ctypes loader for ``libsemicrf.so`` (the C ABI declared in include/semicrf.h).

torch is imported before the library is opened so that both bind to the same
HIP runtime (they share the ``libamdhip64.so.7`` soname).  Loading fails loudly
when the library has not been built: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the dlopen below, see module docstring)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsemicrf.so")

OP_LOGZ, OP_BACKWARD, OP_VITERBI, OP_PREFIX = 0, 1, 2, 3
STATUS_NAMES = {0: "SEMICRF_OK", 1: "SEMICRF_ERR_INVALID", 2: "SEMICRF_ERR_WORKSPACE",
                3: "SEMICRF_ERR_UNSUPPORTED", 4: "SEMICRF_ERR_DEVICE",
                5: "SEMICRF_ERR_UNIMPLEMENTED"}

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


class Options(ctypes.Structure):
    """struct semicrf_options (include/semicrf.h), field for field."""
    _fields_ = [("proj_start", _vp), ("proj_end", _vp), ("grad_proj_start", _vp),
                ("grad_proj_end", _vp), ("boundary", _vp), ("node_mass", _vp),
                ("events", _vp), ("seam_bound", _vp), ("seam_repairs", _vp),
                ("seam_tolerance", ctypes.c_double)]


_opt = ctypes.POINTER(Options)

# the problem statement's argument lists: (emissions, lengths, trans, dur, B, T, C, K, ...)
_LOGZ = [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]
_BACKWARD = [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size,
             _vp, _vp, _vp, _vp, _vp, _vp]
_VITERBI = [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp, _vp, _vp]

# name -> (restype, argtypes); every pointer is passed as an integer address
SIGNATURES = {
    "semicrf_status_string": (ctypes.c_char_p, [_c_int]),
    "semicrf_checkpoint_interval": (_c_int, [_c_int, _c_int, _c_int]),
    "semicrf_default_interval": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "semicrf_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "semicrf_prefix": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "semicrf_logz": (_c_int, _LOGZ),
    "semicrf_backward": (_c_int, _BACKWARD),
    "semicrf_viterbi": (_c_int, _VITERBI),
    "semicrf_logz_ex": (_c_int, _LOGZ + [_opt]),
    "semicrf_backward_ex": (_c_int, _BACKWARD + [_opt]),
    "semicrf_viterbi_ex": (_c_int, _VITERBI + [_opt]),
    "semicrf_nll": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                             _c_int, _vp, _vp, _c_size, _vp, _vp, _vp, _vp, _vp, _opt]),
    "semicrf_read_status": (_c_int, [_vp, _vp]),
    "semicrf_logz_static": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _vp, _vp]),
}
STATIC_SCRATCH_BYTES = 32 << 20
STAGES = {"logz": 2, "backward": 5, "viterbi": 3}


def options(**fields) -> Options:
    """An Options struct; fields not given are NULL (integer addresses or None)."""
    o = Options()
    for k, v in fields.items():
        setattr(o, k, v)
    return o


class SemiCRFError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m "
                              f"semi_markov_crf_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().semicrf_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise SemiCRFError(fn, status)
