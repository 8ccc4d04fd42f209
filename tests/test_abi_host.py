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


def prototype(name):
    """Parameter types of `name` in the header, e.g. ['const float*', 'int', ...]."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    out = []
    for p in m.group(1).split(","):
        typ = re.match(r"(.*?)\b\w+\s*$", " ".join(p.split())).group(1)
        out.append(re.sub(r"\s*\*", "*", typ).strip())
    return out


# The problem statement's calls: each takes (emissions[B,T,C], lengths, trans[C,C],
# dur[K,C], K, stream), with B, T, C explicit, a caller workspace and the outputs.
PROBLEM_STATEMENT = {
    "semicrf_workspace_bytes": ["semicrf_op", "int", "int", "int", "int", "int"],
    "semicrf_logz": ["const float*", "const int32_t*", "const float*", "const float*", "int",
                     "int", "int", "int", "int", "hipStream_t", "void*", "size_t", "float*"],
    "semicrf_backward": ["const float*", "const int32_t*", "const float*", "const float*",
                         "int", "int", "int", "int", "int", "hipStream_t", "void*", "size_t",
                         "const float*", "float*", "float*", "float*", "float*", "float*"],
    "semicrf_viterbi": ["const float*", "const int32_t*", "const float*", "const float*", "int",
                        "int", "int", "int", "hipStream_t", "void*", "size_t", "float*",
                        "int32_t*", "uint8_t*"],
    "semicrf_status_string": ["int"],
}


@pytest.mark.parametrize("name", sorted(PROBLEM_STATEMENT))
def test_prototypes_follow_the_problem_statement(name):
    assert prototype(name) == PROBLEM_STATEMENT[name]


def test_status_codes_in_header():
    text = open(HEADER).read()
    for i, n in enumerate(["SEMICRF_OK", "SEMICRF_ERR_INVALID", "SEMICRF_ERR_WORKSPACE",
                           "SEMICRF_ERR_UNSUPPORTED", "SEMICRF_ERR_DEVICE",
                           "SEMICRF_ERR_UNIMPLEMENTED"]):
        assert re.search(rf"\b{n}\s*=\s*{i}\b", text), n
    for i, n in enumerate(["SEMICRF_OP_LOGZ", "SEMICRF_OP_BACKWARD", "SEMICRF_OP_VITERBI"]):
        assert re.search(rf"\b{n}\s*=\s*{i}\b", text), n


def test_options_struct_matches_binding():
    """The ctypes Options struct lists the header's semicrf_options fields in order."""
    from semi_markov_crf_amd import _native
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct semicrf_options \{(.*?)\} semicrf_options;", text, re.S)
    names = re.findall(r"(\w+)\s*;", body.group(1))
    assert names == [f[0] for f in _native.Options._fields_]


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
    for s in range(6):
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


def test_default_interval(native):
    lib = native.load()
    f = lib.semicrf_default_interval
    LZ, BW, VI = native.OP_LOGZ, native.OP_BACKWARD, native.OP_VITERBI
    # round kernels, both directions of a span in one workgroup: 224 workgroups
    assert f(BW, 4, 100_000, 6, 200) == 1786   # 56 spans a sequence
    assert f(LZ, 4, 100_000, 6, 200) == 1786
    assert f(BW, 1, 1_000_000, 6, 200) == 4465
    # 16 labels: two workgroups a span
    assert f(BW, 4, 100_000, 16, 200) == 3572  # 28 spans a sequence
    # other kernels: 256 workgroups, two a span for the backward
    assert f(BW, 32, 800, 39, 30) == 200       # 4 spans a sequence
    assert f(LZ, 32, 800, 39, 30) == 100       # 8
    assert f(BW, 8, 10_000, 64, 64) == 625     # 16
    assert f(LZ, 8, 10_000, 64, 64) == 313     # 32
    assert f(BW, 1, 1_000_000, 6, 2000) == 7813
    # a batch that fills the device: fewer, longer spans
    assert f(BW, 64, 100_000, 6, 200) == 14286
    # short sequences: one span (no burn-in) beats any split
    assert f(BW, 2, 64, 4, 8) == 64
    assert f(BW, 0, 100, 4, 5) == 0 and f(BW, 1, 0, 4, 5) == 0 and f(BW, 1, 10, 4, 0) == 0
    assert f(BW, 1, 100, 200, 5) == 0          # unsupported label count


def test_decode_interval(native):
    lib = native.load()
    f = lib.semicrf_default_interval
    VI = native.OP_VITERBI
    # round kernels: the span launch's model, one workgroup a span, 224 workgroups
    assert f(VI, 4, 100_000, 6, 200) == 1786
    assert f(VI, 1, 1_000_000, 6, 200) == 4465
    assert f(VI, 2, 2000, 16, 20) == 65        # 31 spans a sequence, one burn-in long
    assert f(VI, 1, 1000, 6, 200) == 1000      # one span: no burn-in
    # other kernels: ceil(sqrt(TK)), halved for few long spans
    assert f(VI, 8, 10_000, 64, 64) == 400     # 104 spans of 800 >= 768: halved
    assert f(VI, 32, 800, 39, 30) == 155       # 192 spans: the batch fills the device
    assert f(VI, 1, 5000, 3, 1030) == 2270     # long durations: spans shorter than 12 K kept
    assert f(VI, 0, 100, 4, 5) == 0 and f(VI, 1, 0, 4, 5) == 0 and f(VI, 1, 10, 4, 0) == 0


def test_workspace_bytes(native):
    lib = native.load()
    ws = lib.semicrf_workspace_bytes
    for op in range(3):
        a = ws(op, 4, 1000, 6, 20, 0)
        assert a > 0 and a % 256 == 0
        assert ws(op, 8, 1000, 6, 20, 0) > a           # grows with B
        assert ws(op, 4, 2000, 6, 20, 0) > a           # and with T
    # backward holds O(B*T*C) per-position values (S and the messages of both directions,
    # fp64) plus checkpoints; with more than 16 labels also the values after the transition
    assert ws(1, 1, 10_000, 6, 200, 0) > 3 * 8 * 10_001 * 6
    assert ws(1, 1, 10_000, 6, 200, 0) < 4 * 8 * 10_001 * 6 + (64 << 20)
    assert ws(1, 1, 10_000, 17, 200, 0) > 5 * 8 * 10_001 * 17
    assert ws(4, 1, 10, 2, 2, 0) == 0                  # unknown op
    assert 0 < ws(3, 1, 10, 2, 2, 0) < ws(0, 1, 10, 2, 2, 0)   # prefix: S goes to the caller
    assert ws(0, 0, 10, 2, 2, 0) == 0 and ws(0, 1, 0, 2, 2, 0) == 0
    assert ws(0, 1, 10, 2000, 2, 0) == 0               # C beyond the supported range
    assert ws(0, 1, 10, 2, 70000, 0) == 0              # K beyond 65535


@pytest.mark.parametrize("C,kmax", [(1, 8193), (4, 8193), (6, 8193), (7, 8193), (8, 2049), (9, 2049),
                                    (16, 2049), (17, 513), (39, 513), (64, 513), (128, 97)])
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
    # NULL inputs / outputs
    assert lib.semicrf_logz(n, p, p, p, 1, 4, 2, 2, 0, n, p, 1 << 20, p) == 1
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 2, 2, 0, n, p, 1 << 20, n) == 1
    # bad sizes, negative delta
    assert lib.semicrf_logz(p, p, p, p, 0, 4, 2, 2, 0, n, p, 1 << 20, p) == 1
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 2, 0, 0, n, p, 1 << 20, p) == 1
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 2, 2, -1, n, p, 1 << 20, p) == 1
    # unsupported label count
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 4096, 2, 0, n, p, 1 << 20, p) == 3
    # workspace missing, too small, misaligned
    need = lib.semicrf_workspace_bytes(0, 1, 4, 2, 2, 0)
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 2, 2, 0, n, n, need, p) == 2
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 2, 2, 0, n, p, need - 1, p) == 2
    assert lib.semicrf_logz(p, p, p, p, 1, 4, 2, 2, 0, n, ctypes.c_void_p(0x1008), need, p) == 2
    # backward: required gradient outputs, negative delta
    need = lib.semicrf_workspace_bytes(1, 1, 4, 2, 2, 0)
    assert lib.semicrf_backward(p, p, p, p, 1, 4, 2, 2, 0, n, p, need, n, n, p, p, n, n) == 1
    assert lib.semicrf_backward(p, p, p, p, 1, 4, 2, 2, -1, n, p, need, n, p, p, p, n, n) == 1
    assert lib.semicrf_backward(p, p, p, p, 1, 4, 2, 2, 0, n, p, 16, n, p, p, p, n, n) == 2
    # training loss: gold segmentation and loss output required; no backward-only options
    assert lib.semicrf_nll(p, p, p, p, n, p, 1, 4, 2, 2, 0, n, p, need, n, p, p, p, p, n) == 1
    assert lib.semicrf_nll(p, p, p, p, p, p, 1, 4, 2, 2, 0, n, p, need, n, n, p, p, p, n) == 1
    opt = native.options(boundary=0x1000)
    assert lib.semicrf_nll(p, p, p, p, p, p, 1, 4, 2, 2, 0, n, p, need, n, p, p, p, p,
                           ctypes.byref(opt)) == 1
    # viterbi outputs; backward-only options refused
    need = lib.semicrf_workspace_bytes(2, 1, 4, 2, 2, 0)
    assert lib.semicrf_viterbi(p, p, p, p, 1, 4, 2, 2, n, p, need, p, n, p) == 1
    opt = native.options(node_mass=0x1000)
    assert lib.semicrf_viterbi_ex(p, p, p, p, 1, 4, 2, 2, n, p, need, p, p, p,
                                  ctypes.byref(opt)) == 1
    assert lib.semicrf_read_status(n, n) == 2
    need = lib.semicrf_workspace_bytes(3, 1, 4, 2, 1, 0)
    assert lib.semicrf_prefix(p, p, 1, 4, 2, n, p, need, n) == 1
    assert lib.semicrf_prefix(p, p, 1, 4, 2, n, p, need - 1, p) == 2


def test_static_scratch_limit_is_checked_before_any_launch(native):
    """semicrf_logz_static: shapes whose log Z workspace exceeds the static array are
    refused with SEMICRF_ERR_WORKSPACE, before the device is touched."""
    lib = native.load()
    p, n = ctypes.c_void_p(0x1000), None
    assert lib.semicrf_workspace_bytes(0, 1, 1_000_000, 6, 200, 0) > native.STATIC_SCRATCH_BYTES
    assert lib.semicrf_logz_static(p, p, p, p, 1, 1_000_000, 6, 200, 0, n, p) == 2
    assert lib.semicrf_logz_static(p, p, p, p, 1, 4, 2, 2, 0, n, n) == 1
    assert lib.semicrf_logz_static(n, p, p, p, 1, 4, 2, 2, 0, n, p) == 1
    assert lib.semicrf_logz_static(p, p, p, p, 1, 4, 2, 2, -1, n, p) == 1
    assert lib.semicrf_workspace_bytes(0, 4, 100_000, 6, 200, 0) <= native.STATIC_SCRATCH_BYTES
