"""CPU-only checks of the library: it loads, exports every entry point that
include/moe.h declares, its host-side validation rejects bad arguments
without touching a GPU, and its MXFP8 encode helpers (compiled for the host)
agree bit for bit with the oracle on every bf16 value and scale."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import moe_oracle as O
from synthetic import bf16_to_f64

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
CSRC = os.path.join(ROOT, "mixture_experts_grouped_router_amd", "csrc")


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"\b(moe_\w+|mxfp8_\w+)\s*\(", txt)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_grouped_router_amd as m
    if not os.path.exists(m.lib_path):
        from mixture_experts_grouped_router_amd import build
        build.build()
    return m.load_library()


def test_exports_every_declared_entry_point(lib):
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name],
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    assert set(names) <= exported


def test_host_validation_without_gpu(lib):
    assert lib.moe_route_topk(None, None, 4, 8, 2, 1, None, None, None) == 1
    assert b"null context" in lib.moe_last_error()
    assert lib.moe_status_string(3) == b"workspace too small"
    n = ctypes.c_size_t()
    assert lib.moe_permute_workspace_size(32768, 128, 8, ctypes.byref(n)) == 0
    assert n.value >= 256 * 128 * 4
    assert lib.moe_permute_workspace_size(-1, 8, 2, ctypes.byref(n)) == 1


def test_workspace_queries(lib):
    import mixture_experts_grouped_router_amd as m
    a = m._FwdArgs()
    a.E, a.H, a.F, a.rows, a.precision = 8, 4096, 14336, 16384, 0
    n = ctypes.c_size_t()
    assert lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(a),
                                                  ctypes.byref(n)) == 0
    assert n.value >= 16384 * 14336 * 2          # the A intermediate
    a.H = 100                                    # not a multiple of 64
    assert lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(a),
                                                  ctypes.byref(n)) == 2
    # per-expert loop: h1 and a in the workspace unless saved; bf16 only
    a.H = 4096
    assert lib.moe_expert_loop_mlp_fwd_workspace_size(ctypes.byref(a),
                                                      ctypes.byref(n)) == 0
    assert n.value >= 16384 * 3 * 14336 * 2
    a.precision = 1
    assert lib.moe_expert_loop_mlp_fwd_workspace_size(ctypes.byref(a),
                                                      ctypes.byref(n)) == 2
    # tensor-scaled FP8: weights quantised by the caller leave their codes
    # (E * 3 * H * F bytes) out of the workspace
    a.precision = 2
    assert lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(a),
                                                  ctypes.byref(n)) == 0
    own = n.value
    a.w_gu_q, a.w_dn_q = 4096, 8192   # only their presence counts here
    assert lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(a),
                                                  ctypes.byref(n)) == 0
    assert own - n.value >= 8 * 3 * 4096 * 14336


@pytest.fixture(scope="module")
def codec_tables(tmp_path_factory):
    d = tmp_path_factory.mktemp("codec")
    exe = str(d / "mx_codec_dump")
    src = os.path.join(ROOT, "tests", "native", "mx_codec_dump.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                   check=True)
    f1, f2 = str(d / "codes.bin"), str(d / "scales.bin")
    subprocess.run([exe, f1, f2], check=True)
    codes = np.fromfile(f1, dtype=np.uint8).reshape(255, 65536)
    sc = np.fromfile(f2, dtype=np.int16)
    return codes, sc


def test_library_e4m3_encode_equals_oracle_exhaustive(codec_tables):
    codes, _ = codec_tables
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    v0 = bf16_to_f64(bits[finite])
    for s in range(-127, 128):
        want = O.e4m3_encode(np.ldexp(v0, -s))
        got = codes[s + 127][finite]
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (s, bits[finite][bad[:4]], got[bad[:4]],
                               want[bad[:4]])


def test_library_e8m0_exponent_equals_oracle_exhaustive(codec_tables):
    _, sc = codec_tables
    a = np.arange(32768, dtype=np.uint32).astype(np.uint16)
    finite = ((a >> 7) & 0xFF) != 0xFF
    want = O.e8m0_exponent(bf16_to_f64(a[finite]))
    np.testing.assert_array_equal(sc[finite].astype(np.int64), want)


def test_library_index_helpers(tmp_path):
    """Multiply-shift division and the MXFP8 GEMM scale layout (host build
    of the library's helpers)."""
    exe = str(tmp_path / "layout_check")
    src = os.path.join(ROOT, "tests", "native", "layout_check.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout


def test_work_items_host_build(tmp_path):
    """The ragged-M GEMMs' work items, built for the host: the M-tile
    records decode every tile as the search over the tile prefix does, every
    tile of a random tile table is one whole item or K-range pieces that
    partition its
    K steps, split slots stay inside their XCD and apart, and the persistent
    take protocol hands out every item once and lets every work-group end."""
    exe = str(tmp_path / "work_items_check")
    src = os.path.join(ROOT, "tests", "native", "work_items_check.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout


def test_offsets_guard_host_build(tmp_path):
    """The device-side offsets guard, built for the host: accepts exactly
    the arrays that run non-decreasing from 0 to rows (exhaustive over small
    arrays), and a rejected array yields an empty tile table."""
    exe = str(tmp_path / "offsets_check")
    src = os.path.join(ROOT, "tests", "native", "offsets_check.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout
