"""Sanitizer builds of the host-side code, on the CPU.

* The fp64 oracle (`oracle/mta_oracle.cpp`) built with AddressSanitizer and
  UndefinedBehaviorSanitizer; the oracle pins (`tests/test_oracle_pins.py`) run against it in a
  child process with the sanitizer runtime preloaded (Python itself is not instrumented). A
  copy with a planted out-of-bounds read shows that the sanitizer is live in that setup.
* The C ABI's host code: argument validation, the key-split plan and the dispatch
  (`mta_api.hip`, `mta_split.hip`, `mta_fused.hip`, `mta_materialized.hip`,
  `mta_backward.hip`, `mta_bwd_fused.hip`) built with the sanitizers on the host side only (device code is built as
  usual and never runs here); the per-shape kernel instantiation units are replaced by stubs.
  The C-ABI tests (`tests/test_abi.py`) run against that library.

A sanitizer report ends the child process with a non-zero status, which fails the test (the
child runs pytest without output capture, so that the report reaches its stderr).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"}


def _runtime(cmd):
    try:
        path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if path and os.path.isfile(path) else None


def _child(code, preload, timeout=600):
    env = dict(os.environ, **SAN_ENV)
    # the sanitizer runtime must come first; any library already preloaded stays after it
    env["LD_PRELOAD"] = preload + ((":" + os.environ["LD_PRELOAD"]) if os.environ.get("LD_PRELOAD") else "")
    return subprocess.run([sys.executable, "-c", code, ROOT], capture_output=True, text=True, env=env,
                          timeout=timeout)


# ---- oracle ------------------------------------------------------------------------------------
_ORACLE_DRIVER = (
    "import sys; sys.path.insert(0, sys.argv[1]);"
    "from oracle import oracle; oracle._LIB = {lib!r}; oracle._lib = None;"
    "import pytest;"
    "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', {kfilter}"
    " sys.argv[1] + '/tests/test_oracle_pins.py']))"
)


def _build_oracle(src_text, out):
    cpp = out + ".cpp"
    with open(cpp, "w") as f:
        f.write(src_text)
    subprocess.run(["g++", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fopenmp",
                    "-std=c++17", "-shared", "-fPIC", "-o", out, cpp], check=True)
    return out


@pytest.fixture(scope="module")
def gcc_asan():
    path = _runtime(["g++", "-print-file-name=libasan.so"])
    if path is None:
        pytest.skip("g++ has no AddressSanitizer runtime")
    return path


def test_oracle_pins_under_asan_and_ubsan(tmp_path, gcc_asan):
    src = open(os.path.join(ROOT, "oracle", "mta_oracle.cpp")).read()
    lib = _build_oracle(src, str(tmp_path / "libmta_oracle_san.so"))
    r = _child(_ORACLE_DRIVER.format(lib=lib, kfilter=""), gcc_asan)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr, r.stderr[-3000:]


def test_planted_out_of_bounds_read_is_reported(tmp_path, gcc_asan):
    # values read from row j + 1: one row past the end of v for the last key
    src = open(os.path.join(ROOT, "oracle", "mta_oracle.cpp")).read()
    old = "o[c] += a_u[j] * p.v[idx4(p, b, j, m, c)];"
    assert src.count(old) == 1
    lib = _build_oracle(src.replace(old, "o[c] += a_u[j] * p.v[idx4(p, b, j + 1, m, c)];"),
                        str(tmp_path / "libmta_oracle_oob.so"))
    r = _child(_ORACLE_DRIVER.format(lib=lib, kfilter="'-k', 'sdpa',"), gcc_asan)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stdout[-2000:] + r.stderr[-2000:]


# ---- C ABI host code ---------------------------------------------------------------------------
_STUB = """// Stand-ins for the per-shape kernel instantiation units: the host-side checks under test
// never reach them (no device is present), and a launch through them reports an error.
#include <hip/hip_runtime.h>
#include "mta_internal.h"
#include "mta_bwd_tile.h"
namespace mta {{
{decls}
}}
"""


def _stub_source():
    names = []
    for fn in sorted(os.listdir(CSRC)):
        if fn.startswith("mta_fused_") and fn.endswith(".hip"):
            names.append("launch_" + fn[len("mta_"):-len(".hip")])
    decls = "\n".join(f"hipError_t {n}(const Problem&, hipStream_t) {{ return hipErrorInvalidValue; }}"
                      for n in names)
    tiles = [fn[len("mta_bwd_tile_"):-len(".hip")] for fn in sorted(os.listdir(CSRC))
             if fn.startswith("mta_bwd_tile_d") and fn.endswith(".hip")]
    decls += "\n" + "\n".join(
        f"hipError_t launch_bwd_tiles_{n}(const bwt::BwArgs&, int, int, int, size_t, unsigned, hipStream_t) "
        "{ return hipErrorInvalidValue; }" for n in tiles)
    return _STUB.format(decls=decls)


@pytest.fixture(scope="module")
def abi_san_lib(tmp_path_factory):
    rt = _runtime([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"])
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("no hipcc with a host AddressSanitizer runtime")
    work = tmp_path_factory.mktemp("abi_san")
    stub = work / "stubs.hip"
    stub.write_text(_stub_source())
    srcs = [os.path.join(CSRC, n) for n in ("mta_api.hip", "mta_split.hip", "mta_fused.hip", "mta_materialized.hip",
                                            "mta_backward.hip", "mta_bwd_fused.hip")] + [str(stub)]
    # sanitizers on the host side only: each -fsanitize follows -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for s in srcs:
        o = str(work / (os.path.basename(s) + ".o"))
        subprocess.run([HIPCC] + flags + host_san + ["-c", s, "-o", o], check=True, capture_output=True)
        objs.append(o)
    lib = str(work / "libmta_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + host_san + ["-o", lib] + objs, check=True,
                   capture_output=True)
    return lib, rt


_ABI_DRIVER = (
    "import sys; sys.path.insert(0, sys.argv[1]);"
    "from token_attention_amd import mta; mta._LIB_PATH = {lib!r}; mta._lib = None;"
    "import pytest;"
    "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', sys.argv[1] + '/tests/test_abi.py']))"
)


def test_abi_host_code_under_asan_and_ubsan(abi_san_lib):
    lib, rt = abi_san_lib
    r = _child(_ABI_DRIVER.format(lib=lib), rt)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr, r.stderr[-3000:]
