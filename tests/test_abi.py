"""The C-ABI library loads and exports every symbol include/tq.h declares.

CPU only: these calls either need no device (version, strings, dispatcher)
or are rejected by host-side argument checks before any HIP call is made.
"""
import ctypes
import os
import re

import pytest

from bit_weight_only_tq_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


F = 16384  # TQ_WORKSPACE_FLAG_BYTES: split arrival counters at the front of a workspace


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("tq_pack", "tq_gemm", "w4a16_gemm", "tq_unpack", "w4a16_pack", "w4a16_unpack",
                     "w4a16_pack_asym", "w4a16_unpack_asym", "w4a16_gemm_asym"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a prototype for {name}"


def test_binding_declares_nothing_extra():
    assert set(_lib.SIGNATURES) == set(_declared_functions())


def test_one_hip_runtime_per_process():
    """Loading the library before anything imports torch still leaves one HIP
    runtime mapped (the binding loads torch's first)."""
    import subprocess
    import sys
    code = ("from bit_weight_only_tq_amd import _lib; _lib.load(); "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    paths = eval(out.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


def test_version_and_status_strings(lib):
    assert lib.tq_abi_version() == 6
    src = open(HEADER).read()
    assert "#define TQ_ABI_VERSION 6" in src
    for code, name in _lib.STATUS_NAMES.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", src), name
        s = lib.tq_status_str(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.tq_status_str(99) == b"unknown status"


def test_dispatcher_by_m():
    sel = _lib.tq_select_path
    for M in (1, 4, 16):
        assert sel("ternary", M, 4096, 4096) == "gemv"
        assert sel("w4a16", M, 4096, 4096) == "gemv"
    for M in (17, 32, 64, 255):
        assert sel("ternary", M, 8192, 8192) == "stream_mfma"
        assert sel("w4a16", M, 8192, 8192) == "gemm"      # W4A16: the GEMM's 64-row tiles
    # W4A16 at 17..32 rows with K < 8192: two passes of the decode kernels
    assert sel("w4a16", 17, 14336, 4096) == sel("w4a16", 32, 14336, 4096) == "gemv"
    assert sel("w4a16", 33, 14336, 4096) == "gemm"
    for M in (256, 2048, 4096, 8192):
        assert sel("ternary", M, 14336, 4096, "bf16") == "gemm"
        assert sel("w4a16", M, 14336, 4096, "bf16") == "gemm"
        assert sel("w4a16", M, 4096, 16384) == "gemm"
        assert sel("w4a16", M, 4096, 16384 + 128) == "gemm"  # past 128 groups: split K (needs a workspace)
    # bf16 follows the same split (its decode kernels match fp16's)
    for M in (1, 4, 5, 16):
        assert sel("ternary", M, 4096, 4096, "bf16") == "gemv"
        assert sel("w4a16", M, 4096, 4096, "bf16") == "gemv"
    assert sel("ternary", 17, 4096, 4096, "bf16") == "stream_mfma"
    # rows that are not whole 256-column chunk-sets: the medium path's tiles
    # from three activation rows, the decode path below that
    for M in (3, 8, 16):
        assert sel("ternary", M, 4096, 4160) == "stream_mfma"
    for M in (1, 2):
        assert sel("ternary", M, 4096, 4160) == "gemv"


def test_workspace_query():
    """Split-K workspace: the arrival counters (F bytes) and S fp32 partials
    of [M, N] for the medium and large-M paths, none for the GEMV path or
    when the output tiles fill the device; the medium path adds the paired
    activations on large shapes.
    Off the GPU the compute-unit count defaults to 256."""
    wb = _lib.tq_gemm_workspace_bytes
    assert wb(1, 4096, 4096) == 0 and wb(4096, 4096, 4096) == 0
    assert wb(16, 4096, 14336, "bf16") == wb(16, 4096, 14336) > 0  # bf16 streaming kernel: same K split as fp16
    assert wb(64, 8192, 8192) == F + 8 * 64 * 8192 * 4  # 32 tiles -> 8 splits
    assert wb(32, 1024, 8192) == F + 16 * 32 * 1024 * 4  # 4 tiles: capped at 16 splits
    assert wb(40, 10240, 8192) == F + 6 * 40 * 10240 * 4  # 40 tiles: 6 splits keep one round on 256 CUs
    assert wb(100, 2000, 1024) == F + 2 * 100 * 2000 * 4  # 4 K-steps of 256: two per split
    assert wb(100, 2000, 4160) == F + 8 * 100 * 2000 * 4  # K % 256 != 0: 64-column kernel, >= 8 K-steps per split
    # N K >= 2e8: the activations are paired once per call, into the
    # workspace after the split partials (256-byte aligned)
    assert wb(64, 57344, 8192) == F + 64 * 8192 * 2  # 224 tiles: no split, pairs only
    assert wb(32, 8192, 28672) == F + 8 * 32 * 8192 * 4 + 32 * 28672 * 2
    assert wb(32, 8192, 28672, path="stream_mfma") == wb(32, 8192, 28672)
    assert wb(64, 8192, 96) == 0                        # K % 64 != 0
    # large M: 256 x 256 tiles, one per compute unit, >= 16 K-steps per split
    assert wb(2048, 4096, 14336) == F + 2 * 2048 * 4096 * 4  # 128 tiles: two splits fill the device
    assert wb(2048, 14336, 4096) == 0                   # 448 tiles: partials cost more than they save
    assert wb(4096, 4096, 14336) == 0 and wb(8192, 4096, 14336) == 0
    assert wb(300, 1000, 4096) == F + 4 * 300 * 1000 * 4  # 8 tiles, 64 K-steps -> 4 splits
    assert wb(300, 1000, 1024) == 0                     # 16 K-steps: nothing to split
    assert wb(64, 8192, 8192, path="gemm") == F + 8 * 64 * 8192 * 4
    assert wb(4, 8192, 8192, path="gemv") == 0
    # decode (M <= 16): the small-M kernel (M <= 2, and M <= 4 with few waves
    # per SIMD) never splits; the streaming kernel may
    assert wb(4, 4096, 14336) == 0 and wb(2, 4096, 14336) == 0
    assert wb(5, 4096, 14336) == F + 7 * 5 * 4096 * 4 and wb(16, 4096, 14336) == F + 7 * 16 * 4096 * 4


V = ctypes.c_void_p
FAKE = V(0x10000)          # never dereferenced: every call below fails a host check first
MIS = V(0x10002)           # 2-byte aligned only


@pytest.mark.parametrize("args, want", [
    ((None, 0, 1, 64, 64, FAKE, FAKE, None, FAKE, None), "TQ_ERR_NULL"),
    ((FAKE, 0, 1, 64, 64, None, FAKE, None, FAKE, None), "TQ_ERR_NULL"),
    ((FAKE, 0, 1, 64, 64, FAKE, None, None, FAKE, None), "TQ_ERR_NULL"),
    ((FAKE, 0, 1, 64, 64, FAKE, FAKE, None, None, None), "TQ_ERR_NULL"),
    ((FAKE, 7, 1, 64, 64, FAKE, FAKE, None, FAKE, None), "TQ_ERR_DTYPE"),
    ((FAKE, 0, 0, 64, 64, FAKE, FAKE, None, FAKE, None), "TQ_ERR_SHAPE"),
    ((FAKE, 0, 1, -5, 64, FAKE, FAKE, None, FAKE, None), "TQ_ERR_SHAPE"),
    ((FAKE, 0, 1, 64, 0, FAKE, FAKE, None, FAKE, None), "TQ_ERR_SHAPE"),
    ((FAKE, 0, 1, 64, 96, FAKE, FAKE, None, FAKE, None), "TQ_ERR_SHAPE"),   # K % 64 != 0
    ((FAKE, 0, 1, 64, (1 << 22) + 64, FAKE, FAKE, None, FAKE, None), "TQ_ERR_SHAPE"),  # K > 2^22
    ((MIS, 0, 1, 64, 64, FAKE, FAKE, None, FAKE, None), "TQ_ERR_ALIGN"),
    ((FAKE, 0, 1, 64, 64, MIS, FAKE, None, FAKE, None), "TQ_ERR_ALIGN"),
    ((FAKE, 0, 1, 64, 64, FAKE, FAKE, None, V(0x10001), None), "TQ_ERR_ALIGN"),
])
def test_tq_gemm_host_checks(lib, args, want):
    assert _lib.STATUS_NAMES[lib.tq_gemm(*args)] == want


def test_tq_gemm_ws_host_checks(lib):
    name = _lib.STATUS_NAMES
    st = lib.tq_gemm_ws(FAKE, 0, 32, 64, 64, FAKE, FAKE, None, FAKE, MIS, 1024, None, 0)
    assert name[st] == "TQ_ERR_ALIGN"
    st = lib.tq_gemm_ws(FAKE, 0, 32, 64, 64, FAKE, FAKE, None, FAKE, None, 0, None, 1)
    assert name[st] == "TQ_ERR_PATH"
    st = lib.tq_gemm_ws(None, 0, 32, 64, 64, FAKE, FAKE, None, FAKE, None, 0, None, 0)
    assert name[st] == "TQ_ERR_NULL"


def test_w4_workspace_query():
    """W4A16 split-K workspace: S fp32 partials of [M, N] when the plan splits
    the K groups (the streaming kernel at 2 <= M <= 16, the matrix-core GEMM
    above); none where the small-M kernel runs (M <= 4 on its shapes) or when
    one pass over K is cheapest.  Off the GPU the compute-unit count
    defaults to 256."""
    wb = _lib.w4a16_gemm_workspace_bytes
    assert wb(16, 4096, 14336) == F + 8 * 16 * 4096 * 4  # 112 groups -> 8 splits of 14
    assert wb(16, 57344, 8192) == F + 4 * 16 * 57344 * 4
    assert wb(16, 28672, 4096) == 0 and wb(16, 4096, 4096) == 0
    assert wb(1, 4096, 14336) == 0                       # M = 1 never splits
    assert wb(2, 4096, 14336) == 0                       # M = 2: the small-M kernel, no split
    assert wb(5, 4096, 14336) == F + 8 * 5 * 4096 * 4  # M = 5 streams: 112 groups -> 8 splits of 14
    assert wb(16, 4096, 14336, "bf16") == wb(16, 4096, 14336)  # bf16 streams like fp16
    assert wb(16, 4096, 14336, group_size=64) == 0
    assert wb(24, 4096, 4096) == 0                        # blocks of 16 rows, no split on these shapes
    assert wb(24, 1024, 4096) == wb(16, 1024, 4096)       # ... the largest block's need
    # the matrix-core GEMM (17 <= M, K >= 8192 or M > 32): split while the
    # 128-column tiles leave compute units idle, at most 16, >= 1 group each
    assert wb(40, 4096, 14336) == F + 8 * 40 * 4096 * 4  # 32 tiles -> 8 splits
    assert wb(64, 57344, 8192) == 0                       # 448 tiles: one pass
    assert wb(256, 4096, 14336) == F + 8 * 256 * 4096 * 4  # 256-row tiles: 32 tiles -> 8 splits
    assert wb(2048, 4096, 14336) == 0 and wb(4096, 14336, 4096) == 0
    assert wb(4096, 4096, 16384 + 128) == F + 2 * 4096 * 4096 * 4  # 129 groups: two splits at least
    assert wb(16, 4096, 200) == 0                         # K % 128 != 0


def test_w4a16_gemm_ws_host_checks(lib):
    name = _lib.STATUS_NAMES
    st = lib.w4a16_gemm_ws(FAKE, 0, 4, 64, 128, FAKE, FAKE, 128, None, FAKE, MIS, 1024, None, 0)
    assert name[st] == "TQ_ERR_ALIGN"
    st = lib.w4a16_gemm_ws(FAKE, 0, 4, 64, 128, FAKE, FAKE, 128, None, FAKE, None, 0, None, 2)
    assert name[st] == "TQ_ERR_PATH"
    st = lib.w4a16_gemm_ws(FAKE, 0, 4, 64, 128, FAKE, FAKE, 64, None, FAKE, None, 0, None, 0)
    assert name[st] == "TQ_ERR_GROUP"


def test_w4a16_asym_workspace_query():
    """After the arrival counters, with a column order the gathered
    activations (M * K * 2 bytes, rounded up to 256) come first, then the
    split partials of the symmetric query."""
    wb = _lib.w4a16_gemm_asym_workspace_bytes
    sym = _lib.w4a16_gemm_workspace_bytes
    assert wb(16, 4096, 14336) == sym(16, 4096, 14336) == F + 8 * 16 * 4096 * 4
    assert wb(16, 4096, 14336, with_perm=True) == F + 16 * 14336 * 2 + 8 * 16 * 4096 * 4
    assert wb(1, 4096, 4096, with_perm=True) == F + 8192 and wb(1, 4096, 4096) == 0
    assert wb(3, 64, 128, "bf16", with_perm=True) == F + 768  # 3 * 128 * 2 = 768
    assert wb(1, 64, 384, with_perm=True) == F + 768  # 768 already a multiple of 256
    assert wb(1, 64, 256, with_perm=True) == F + 512
    assert wb(5, 64, 128, with_perm=True) == F + 1280
    assert wb(1, 64, 200, with_perm=True) == 0 and wb(1, 64, 256, group_size=64, with_perm=True) == 0


def test_w4a16_asym_host_checks(lib):
    name = _lib.STATUS_NAMES
    g = lib.w4a16_gemm_asym
    # act order needs a workspace at least as large as the gathered activations
    assert name[g(FAKE, 0, 4, 64, 128, FAKE, FAKE, FAKE, FAKE, 128, None, FAKE, None, 0, None, 0)] == "TQ_ERR_SHAPE"
    assert name[g(FAKE, 0, 4, 64, 128, FAKE, FAKE, FAKE, FAKE, 128, None, FAKE, FAKE, 1023, None, 0)] == "TQ_ERR_SHAPE"
    assert name[g(FAKE, 0, 4, 64, 128, FAKE, FAKE, None, MIS, 128, None, FAKE, FAKE, 4096, None, 0)] == "TQ_ERR_ALIGN"
    assert name[g(FAKE, 0, 4, 64, 128, FAKE, FAKE, FAKE, None, 64, None, FAKE, None, 0, None, 0)] == "TQ_ERR_GROUP"
    assert name[g(FAKE, 0, 4, 64, 192, FAKE, FAKE, FAKE, None, 128, None, FAKE, None, 0, None, 0)] == "TQ_ERR_SHAPE"
    assert name[g(FAKE, 0, 4, 64, 128, FAKE, FAKE, FAKE, None, 128, None, FAKE, None, 0, None, 2)] == "TQ_ERR_PATH"
    assert name[g(None, 0, 4, 64, 128, FAKE, FAKE, FAKE, None, 128, None, FAKE, None, 0, None, 0)] == "TQ_ERR_NULL"
    p = lib.w4a16_pack_asym
    assert name[p(FAKE, 4, 128, 128, FAKE, FAKE, FAKE, FAKE, None, None)] == "TQ_ERR_NULL"   # g_idx without perm
    assert name[p(FAKE, 4, 128, 128, None, FAKE, FAKE, None, None, None)] == "TQ_ERR_NULL"   # no zeros
    assert name[p(FAKE, 4, 128, 64, None, FAKE, FAKE, FAKE, None, None)] == "TQ_ERR_GROUP"
    assert name[p(FAKE, 4, 100, 128, None, FAKE, FAKE, FAKE, None, None)] == "TQ_ERR_SHAPE"
    assert name[p(MIS, 4, 128, 128, None, FAKE, FAKE, FAKE, None, None)] == "TQ_ERR_ALIGN"
    u = lib.w4a16_unpack_asym
    assert name[u(FAKE, FAKE, None, None, 4, 128, 128, None, None, None)] == "TQ_ERR_NULL"
    assert name[u(FAKE, FAKE, FAKE, None, 4, 128, 64, None, None, None)] == "TQ_ERR_GROUP"
    assert name[u(FAKE, FAKE, FAKE, None, 4, 100, 128, None, None, None)] == "TQ_ERR_SHAPE"
    assert name[u(FAKE, FAKE, FAKE, MIS, 4, 128, 128, None, None, None)] == "TQ_ERR_ALIGN"


def test_tq_gemm_ex_bad_path(lib):
    st = lib.tq_gemm_ex(FAKE, 0, 32, 64, 64, FAKE, FAKE, None, FAKE, None, 1)  # gemv cannot take M=32
    assert _lib.STATUS_NAMES[st] == "TQ_ERR_PATH"
    st = lib.tq_gemm_ex(FAKE, 0, 1, 64, 64, FAKE, FAKE, None, FAKE, None, 9)
    assert _lib.STATUS_NAMES[st] == "TQ_ERR_PATH"


@pytest.mark.parametrize("args, want", [
    ((FAKE, 0, 1, 64, 128, FAKE, FAKE, 64, None, FAKE, None), "TQ_ERR_GROUP"),
    ((FAKE, 0, 1, 64, 192, FAKE, FAKE, 128, None, FAKE, None), "TQ_ERR_SHAPE"),
    ((FAKE, 0, 1, 64, (1 << 22) + 128, FAKE, FAKE, 128, None, FAKE, None), "TQ_ERR_SHAPE"),
    ((None, 0, 1, 64, 128, FAKE, FAKE, 128, None, FAKE, None), "TQ_ERR_NULL"),
    ((FAKE, 2, 1, 64, 128, FAKE, FAKE, 128, None, FAKE, None), "TQ_ERR_DTYPE"),
])
def test_w4a16_gemm_host_checks(lib, args, want):
    assert _lib.STATUS_NAMES[lib.w4a16_gemm(*args)] == want


def test_prepare_host_checks(lib):
    name = _lib.STATUS_NAMES
    assert name[lib.tq_pack(None, 4, 4, FAKE, FAKE, None)] == "TQ_ERR_NULL"
    assert name[lib.tq_pack(FAKE, 0, 4, FAKE, FAKE, None)] == "TQ_ERR_SHAPE"
    assert name[lib.tq_pack(FAKE, 4, 64, MIS, FAKE, None)] == "TQ_ERR_ALIGN"
    assert name[lib.tq_unpack(None, FAKE, 4, 4, None, None, None)] == "TQ_ERR_NULL"
    assert name[lib.tq_unpack(FAKE, FAKE, 4, -1, None, None, None)] == "TQ_ERR_SHAPE"
    assert name[lib.w4a16_pack(FAKE, 4, 128, 32, FAKE, FAKE, None)] == "TQ_ERR_GROUP"
    assert name[lib.w4a16_pack(FAKE, 4, 100, 128, FAKE, FAKE, None)] == "TQ_ERR_SHAPE"
    assert name[lib.w4a16_pack(MIS, 4, 128, 128, FAKE, FAKE, None)] == "TQ_ERR_ALIGN"
    assert name[lib.w4a16_unpack(FAKE, FAKE, 4, 128, 64, None, None, None)] == "TQ_ERR_GROUP"


def test_noalloc_rejects_schedules_beyond_its_scratch(lib):
    """tq_gemm_noalloc: a schedule whose split partials exceed the 16 MiB
    scratch (prefill 2048 x 4096 x 14336: two splits, 64 MiB) returns
    TQ_ERR_SCRATCH from the host check, before any HIP call; argument errors
    come first, as in tq_gemm_ws."""
    assert lib.tq_gemm_noalloc_scratch_bytes() == 16 << 20
    FAKE = 1 << 20
    assert _lib.tq_gemm_workspace_bytes(2048, 4096, 14336) > 16 << 20
    st = lib.tq_gemm_noalloc(FAKE, 0, 2048, 4096, 14336, FAKE, FAKE, None, FAKE, None, 0)
    assert _lib.STATUS_NAMES[st] == "TQ_ERR_SCRATCH"
    st = lib.tq_gemm_noalloc(FAKE, 0, 2048, 4096, 14336, None, FAKE, None, FAKE, None, 0)
    assert _lib.STATUS_NAMES[st] == "TQ_ERR_NULL"
    st = lib.tq_gemm_noalloc(FAKE, 0, 16, 4096, 4160 + 1, FAKE, FAKE, None, FAKE, None, 0)
    assert _lib.STATUS_NAMES[st] == "TQ_ERR_SHAPE"
