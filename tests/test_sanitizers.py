"""Host AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU, no GPU).

The oracle is built with gcc's sanitizers and run by a driver that calls
every entry point on small seeded inputs and edge cases.  The library's host
code (the C ABI's checks, workspace layouts, dispatch) is built with the
sanitizers on the host side only -- the device code is compiled as usual --
and driven through size queries and calls that the host checks reject
before any HIP call.  Leak detection is on for the oracle; for the library
it is off, since the HIP runtime keeps allocations until exit."""
import os
import shutil
import subprocess

import pytest

from query_aware_kv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _run(exe, asan_options):
    env = dict(os.environ, ASAN_OPTIONS=asan_options,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           os.path.join(ROOT, "oracle", "tb_oracle.c"),
                           os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    assert "oracle driver done" in _run(exe, "detect_leaks=1")


def test_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    cc = B.hipcc()
    clangxx = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/llvm/bin/clang++"
    # host-side sanitizers only: every -fsanitize= is preceded by -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-O3", "-Wall")]
    procs, objs = [], []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([cc, *flags, "-O1", "-g", *host_san, "-c",
                                       os.path.join(B.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out.decode(errors="replace")[-3000:]
    exe = str(tmp_path / "abi_san")
    subprocess.check_call([clangxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                           os.path.join(SAN, "abi_driver.cpp"), *objs, "-L/opt/rocm/lib",
                           "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert "abi driver done" in _run(exe, "detect_leaks=0")
