"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU (no GPU needed):

* the C oracle (oracle/oracle.c) with tests/sanitize/oracle_driver.c: every
  entry point on small cases (a permute round trip with an empty shard and
  uneven heads checked against the index map, masked attention with a row
  that sees no key, row subsets, a merge with -inf partials);
* the library's host half (argument validation, offsets, masks, split plans,
  pointer tables: every csrc/*.hip built with the sanitizers on its host
  side only) with tests/sanitize/abi_driver.cpp: every entry point, valid
  and invalid, with host arrays allocated at exactly their documented
  lengths.  Calls that pass validation reach a launch, which fails without a
  GPU.
A read or write past an allocation, a use after free, an overflow or other
undefined behaviour ends the driver with a report and fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.slow
def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-fopenmp", "-ffp-contract=off", "-std=c11", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=120)
    assert "oracle host checks ok" in r.stdout


@pytest.mark.slow
def test_library_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    from concurrent.futures import ThreadPoolExecutor
    from sequence_attention_dits_amd import build
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        # the sanitizers apply to the host side only; device code as in the library
        _run([HIPCC, "--offload-arch=gfx950", "-O3", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
              "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", '-DUAA_BUILD_ID="sanitize"',
              "-c", os.path.join(build.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([CLANG, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=dict(ENV, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES=""), timeout=120)
    assert "abi host checks ok" in r.stdout
