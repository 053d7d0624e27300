"""The host code of the library (planner, plan check, ABI validation) built
with AddressSanitizer and UndefinedBehaviorSanitizer, and the CPU test suite
of those parts run against that build: any out-of-bounds access, use after
free, signed overflow or other undefined behaviour aborts the run.  The
device launchers are replaced by stand-ins (tests/sanitize_stubs.cpp) that
report TRI_ERR_HIP, so the build needs no GPU toolchain."""
import os
import shutil
import subprocess
import sys

import pytest

from static_triangle_sparse_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SUITE = ["test_planner.py", "test_abi.py", "test_check_plan.py", "test_layer_policy.py"]


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    if not shutil.which("g++") or not _runtime("libasan.so"):
        pytest.skip("g++ with AddressSanitizer not available")
    out = tmp_path_factory.mktemp("san")
    lib = str(out / "libtriattn_host_san.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", B.INCLUDE, "-I", B.CSRC,
           os.path.join(B.CSRC, "plan.cpp"), os.path.join(B.CSRC, "api.cpp"),
           os.path.join(HERE, "sanitize_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    return lib


def test_cpu_suite_under_address_and_ub_sanitizers(san_lib, tmp_path):
    env = dict(os.environ)
    env["TRI_ATTN_LIB"] = san_lib
    env["LD_PRELOAD"] = _runtime("libasan.so")
    # the interpreter's own allocations are not this library's: leaks and
    # allocator-pairing reports are off; a memory error or UB ends the run
    # with its report in the log files (pytest's capture would swallow it)
    log = str(tmp_path / "san")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:alloc_dealloc_mismatch=0:new_delete_type_mismatch=0:log_path={log}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:log_path={log}"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(HERE, f) for f in SUITE]]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       cwd=os.path.dirname(HERE), timeout=1200)
    reports = "".join(open(os.path.join(tmp_path, f)).read()[:3000] for f in sorted(os.listdir(tmp_path))
                      if f.startswith("san"))
    tail = r.stdout[-3000:]
    assert not reports, reports
    assert r.returncode == 0, tail
    assert " passed" in tail


def test_the_sanitized_build_is_the_one_loaded(san_lib):
    # the suite above runs against the sanitized build, not the in-tree one
    env = dict(os.environ, TRI_ATTN_LIB=san_lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0")
    code = ("import static_triangle_sparse_amd as t, static_triangle_sparse_amd._abi as a; t.load(); "
            "print(a.LIB_PATH); print(open('/proc/self/maps').read().count('libtriattn_host_san'))")
    r = subprocess.run([sys.executable, "-c", code], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, env=env, cwd=os.path.dirname(HERE), timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
    lines = r.stdout.strip().splitlines()
    assert lines[-2] == san_lib and int(lines[-1]) > 0
