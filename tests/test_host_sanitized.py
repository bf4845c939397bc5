"""Host-side checks built with the address and undefined-behaviour sanitizers
(CPU only):

* the C ABI layer (csrc/smla_api.cpp: argument checks, error text, split
  planning, dispatch) against stub launchers, tests/native/abi_host_check.cpp;
* a bounds-checked host build of the slot lookup the kernels use
  (csrc/smla_lookup.h with SMLA_BOUNDS_CHECK, tests/native/lookup_check.cpp):
  every block-table read is checked against the table array's length, and its
  output is compared bit for bit with the oracle's index conversion on random
  and adversarial tables (negative entries, positions past the table, request
  ids out of range, block sizes that are not powers of two, strides other
  than the block size)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import sparse_mla as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mla_attention_top_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _cxx():
    c = shutil.which("g++")
    if c is None:
        pytest.skip("g++ not available")
    return c


def _build(out, sources, extra):
    cmd = [_cxx(), "-std=c++17", "-O1", "-g", *SAN, *extra, "-o", out, *sources]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_abi_layer_under_sanitizers(tmp_path):
    exe = _build(str(tmp_path / "abi_host_check"),
                 [os.path.join(CSRC, "smla_api.cpp"), os.path.join(NATIVE, "stub_launchers.cpp"),
                  os.path.join(NATIVE, "abi_host_check.cpp")],
                 ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include")])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host checks passed" in r.stdout


@pytest.fixture(scope="module")
def lookup_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("lookup")
    return _build(str(d / "lookup_check"), [os.path.join(NATIVE, "lookup_check.cpp")],
                  ["-DSMLA_BOUNDS_CHECK", "-I", CSRC])


def _run_lookup(exe, tmp, table, R, MB, stride, B, BS, req, loc, declared_len=None):
    T, K = loc.shape
    inp, out = str(tmp / "in.bin"), str(tmp / "out.bin")
    with open(inp, "wb") as f:
        np.array([R, MB, stride, B, BS, T, K, table.size], np.int64).tofile(f)
        table.astype(np.int32).tofile(f)
        req.astype(np.int32).tofile(f)
        loc.astype(np.int32).tofile(f)
    args = [exe, inp, out] + ([str(declared_len)] if declared_len is not None else [])
    r = subprocess.run(args, capture_output=True, text=True, env=ENV, timeout=120)
    if r.returncode != 0:
        return None, r
    return np.fromfile(out, np.int64).reshape(T, K), r


CASES = [  # (R, max_blocks, row padding, block size, block stride rows)
    (5, 9, 0, 16, 16), (5, 9, 3, 48, 48), (3, 7, 0, 64, 3 * 64), (1, 1, 0, 1, 1), (4, 33, 5, 100, 101),
]


@pytest.mark.parametrize("R,MB,pad,B,BS", CASES)
def test_bounds_checked_lookup_matches_the_oracle(lookup_exe, tmp_path, R, MB, pad, B, BS):
    rng = np.random.default_rng(R * 1000 + MB + B)
    stride = MB + pad
    # the table holds R rows of `stride` entries, the last one cut after max_blocks
    table = rng.integers(0, R * MB * 2, (R - 1) * stride + MB).astype(np.int32)
    table[rng.random(table.size) < 0.15] = -1
    table[rng.random(table.size) < 0.05] = -7
    T, K = 40, 300
    req = rng.integers(0, R, T).astype(np.int32)
    bad_req = [3, 11, 29]
    req[bad_req] = [-1, R, R + 9]                            # requests outside the table: rows of -1
    loc = rng.integers(-3, MB * B + 2 * B, (T, K)).astype(np.int32)
    loc[0, :4] = [np.iinfo(np.int32).max, np.iinfo(np.int32).min, MB * B - 1, MB * B]
    got, r = _run_lookup(lookup_exe, tmp_path, table, R, MB, stride, B, BS, req, loc)
    assert got is not None, r.stderr
    good = np.setdiff1d(np.arange(T), bad_req)
    padded = np.full((R, stride), -1, np.int64)
    padded.reshape(-1)[:table.size] = table                 # the oracle takes a [R, max_blocks] table
    want, _ = O.convert_indices(req[good], padded[:, :MB], loc[good], B, BS)
    g = got[good]
    assert ((g >= 0) == (want >= 0)).all()
    assert (g[g >= 0].astype(np.int32) == want[want >= 0]).all()
    assert (got[bad_req] == -1).all()


def test_bounds_check_reports_a_read_past_the_table(lookup_exe, tmp_path):
    """The check of the check: told the table is one row shorter than the
    reads need, the bounds-checked build must stop with a report."""
    R, MB, B = 3, 4, 16
    table = np.arange(R * MB, dtype=np.int32)
    req = np.array([R - 1], np.int32)
    loc = np.array([[MB * B - 1]], np.int32)                # reads the last entry of the last row
    got, r = _run_lookup(lookup_exe, tmp_path, table, R, MB, MB, B, B, req, loc, declared_len=(R - 1) * MB)
    assert got is None and "bounds: block table read at" in r.stderr
