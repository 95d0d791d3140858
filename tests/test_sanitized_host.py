"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):

* the CPU oracle (oracle/fp8_oracle.c through oracle/sanitize_check.c), every
  function on small ragged inputs in exactly-sized buffers, built with gcc;
* the library's host-side argument validation (the C ABI in csrc/api.hip and
  the launchers' host code), built by hipcc with the sanitizers on its host
  pass only, and driven by
  tests/sanitize_host_driver.c through calls that never reach a launch.

Any out-of-bounds access, use after free or undefined behaviour aborts the
program with a report and fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...: rc {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SAN, "-I", os.path.join(ROOT, "oracle"),
          "-o", exe, os.path.join(ROOT, "oracle", "sanitize_check.c"), "-lm"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"}, timeout=600)
    assert "ok" in r.stdout


def test_library_host_validation_under_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    csrc = os.path.join(ROOT, "block_scaled_fp8_02_amd", "csrc")
    objs = []
    procs = []
    for f in sorted(os.listdir(csrc)):
        if not f.endswith(".hip"):
            continue
        o = str(tmp_path / (f + ".o"))
        objs.append(o)
        # sanitizers on the host pass only (each flag after -Xarch_host); the
        # device code is compiled as usual and never runs here
        host_san = [a for flag in SAN for a in ("-Xarch_host", flag)]
        procs.append(subprocess.Popen(
            [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
             "-c", os.path.join(csrc, f), "-o", o], stdout=subprocess.PIPE, stderr=subprocess.PIPE))
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err.decode()[-3000:]
    lib = str(tmp_path / "libfp8blk_san.so")
    _run([hipcc, "-shared", "-fPIC", "-fsanitize=address,undefined", "-o", lib, *objs])
    exe = str(tmp_path / "drv")
    _run([clang, *SAN, "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize_host_driver.c"),
          "-L", str(tmp_path), "-lfp8blk_san", f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib",
          "-L/opt/rocm/lib", "-lamdhip64", "-o", exe])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"}, timeout=120)
    assert "ok" in r.stdout
