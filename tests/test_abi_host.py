"""C ABI checks that need no GPU: the library loads, exports every function that
include/semicrf.h declares, and its host-side logic (status strings, checkpoint
interval, workspace sizing, argument validation) behaves as documented.  No call
here reaches a kernel launch."""

import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "semicrf.h")
LIB = os.path.join(ROOT, "semi_markov_crf_amd", "libsemicrf.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(semicrf_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def native():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (python -m semi_markov_crf_amd.build)")
    from semi_markov_crf_amd import _native
    return _native


def test_header_declares_the_three_calls():
    fns = declared_functions()
    for f in ("semicrf_logz", "semicrf_backward", "semicrf_viterbi", "semicrf_workspace_bytes",
              "semicrf_status_string"):
        assert f in fns


def test_every_declared_symbol_is_exported(native):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (semicrf_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    lib = native.load()
    for f in declared_functions():
        assert getattr(lib, f) is not None
    assert set(native.SIGNATURES) == set(declared_functions())


def test_status_strings(native):
    for s in range(5):
        assert native.status_string(s)
    assert native.status_string(99) == "unknown status"


def test_checkpoint_interval(native):
    lib = native.load()
    f = lib.semicrf_checkpoint_interval
    assert f(100_000, 200, 0) == 4473          # ceil(sqrt(2e7))
    assert f(1_000_000, 200, 0) == 14143       # ceil(sqrt(2e8))
    assert f(800, 30, 0) == 155
    assert f(10_000, 64, 0) == 800
    assert f(64, 8, 0) == math.ceil(math.sqrt(512))
    assert f(10, 200, 0) == 10                 # clamped to T
    assert f(100, 5, 7) == 7
    assert f(100, 5, 1000) == 100
    assert f(0, 5, 0) == 0 and f(10, 0, 0) == 0 and f(10, 5, -1) == 0


def test_workspace_bytes(native):
    lib = native.load()
    ws = lib.semicrf_workspace_bytes
    for op in range(3):
        a = ws(op, 4, 1000, 6, 20, 0)
        assert a > 0 and a % 256 == 0
        assert ws(op, 8, 1000, 6, 20, 0) > a           # grows with B
        assert ws(op, 4, 2000, 6, 20, 0) > a           # and with T
    # backward holds O(B*T*C) per-position values plus checkpoints
    assert ws(1, 1, 10_000, 6, 200, 0) > 5 * 8 * 10_001 * 6
    assert ws(4, 1, 10, 2, 2, 0) == 0                  # unknown op
    assert 0 < ws(3, 1, 10, 2, 2, 0) < ws(0, 1, 10, 2, 2, 0)   # prefix: S goes to the caller
    assert ws(0, 0, 10, 2, 2, 0) == 0 and ws(0, 1, 0, 2, 2, 0) == 0
    assert ws(0, 1, 10, 2000, 2, 0) == 0               # C beyond the supported range
    assert ws(0, 1, 10, 2, 70000, 0) == 0              # K beyond 65535


@pytest.mark.parametrize("C,kmax", [(1, 2049), (4, 2049), (5, 2049), (7, 2049), (8, 1025), (9, 513), (16, 513),
                                    (17, 257), (39, 257), (64, 257), (128, 97)])
def test_supported_duration_range(native, C, kmax):
    """The largest K each label count supports, as the header states it."""
    lib = native.load()
    ws = lib.semicrf_workspace_bytes
    for op in range(3):
        assert ws(op, 2, 1000, C, kmax, 0) > 0, (op, C, kmax)
        assert ws(op, 2, 1000, C, kmax + 1, 0) == 0, (op, C, kmax + 1)
    assert ws(0, 1, 10, 129, 1, 0) == 0


def test_argument_validation_returns_before_any_launch(native):
    lib = native.load()
    p = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
    n = None
    # NULL inputs / outputs (projections NULL: absent)
    assert lib.semicrf_logz(n, p, p, p, n, n, 1, 4, 2, 2, n, p, 1 << 20, p) == 1
    assert lib.semicrf_logz(p, p, p, p, n, n, 1, 4, 2, 2, n, p, 1 << 20, n) == 1
    # bad sizes
    assert lib.semicrf_logz(p, p, p, p, n, n, 0, 4, 2, 2, n, p, 1 << 20, p) == 1
    assert lib.semicrf_logz(p, p, p, p, n, n, 1, 4, 2, 0, n, p, 1 << 20, p) == 1
    # unsupported label count
    assert lib.semicrf_logz(p, p, p, p, n, n, 1, 4, 4096, 2, n, p, 1 << 20, p) == 3
    # workspace missing, too small, misaligned
    need = lib.semicrf_workspace_bytes(0, 1, 4, 2, 2, 0)
    assert lib.semicrf_logz(p, p, p, p, p, p, 1, 4, 2, 2, n, n, need, p) == 2
    assert lib.semicrf_logz(p, p, p, p, p, p, 1, 4, 2, 2, n, p, need - 1, p) == 2
    assert lib.semicrf_logz(p, p, p, p, n, n, 1, 4, 2, 2, n, ctypes.c_void_p(0x1008), need, p) == 2
    # backward: required gradient outputs, negative delta
    need = lib.semicrf_workspace_bytes(1, 1, 4, 2, 2, 0)
    assert lib.semicrf_backward(p, p, p, p, n, n, 1, 4, 2, 2, 0, n, p, need, n, n, p, p, n, n,
                                n, n, n) == 1
    assert lib.semicrf_backward(p, p, p, p, n, n, 1, 4, 2, 2, -1, n, p, need, n, p, p, p, n, n,
                                p, p, p) == 1
    assert lib.semicrf_backward(p, p, p, p, p, p, 1, 4, 2, 2, 0, n, p, 16, n, p, p, p, n, n,
                                n, n, n) == 2
    # training loss: gold segmentation and loss output required
    assert lib.semicrf_nll(p, p, p, p, n, n, n, p, 1, 4, 2, 2, 0, n, p, need, n, p, p, p, p,
                           n, n) == 1
    assert lib.semicrf_nll(p, p, p, p, n, n, p, p, 1, 4, 2, 2, 0, n, p, need, n, n, p, p, p,
                           n, n) == 1
    # viterbi outputs
    need = lib.semicrf_workspace_bytes(2, 1, 4, 2, 2, 0)
    assert lib.semicrf_viterbi(p, p, p, p, n, n, 1, 4, 2, 2, n, p, need, p, n, p) == 1
    assert lib.semicrf_read_status(n, n) == 2
    need = lib.semicrf_workspace_bytes(3, 1, 4, 2, 1, 0)
    assert lib.semicrf_prefix(p, p, 1, 4, 2, n, p, need, n) == 1
    assert lib.semicrf_prefix(p, p, 1, 4, 2, n, p, need - 1, p) == 2
    for f in ("semicrf_logz_staged", "semicrf_viterbi_staged"):
        args = [p, p, p, p, n, n, 1, 4, 2, 2, n, p, 1 << 20, p] + (
            [n] if f == "semicrf_logz_staged" else [p, p, n])
        assert getattr(lib, f)(*args) == 1          # events pointer required
