"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU oracle and of the
library's host code, each driven through its edge cases on the CPU (no GPU):

- oracle/k3moe_oracle.c with tests/sanitize/oracle_driver.c (gcc);
- every library source, its host side instrumented (the kernels are never
  launched), with tests/sanitize/host_driver.cpp: argument validation of every
  entry point, workspace sizes, status strings, the residency pool's slot layout
  and LRU planning against a reference.

Any sanitizer report aborts the driver (halt_on_error / -fno-sanitize-recover)."""
import concurrent.futures
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "mxfp4_routed_expert_k3moe_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "k3moe_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    # device code as in the product build; the sanitizers instrument the host side only
    flags = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [str(tmp_path / (os.path.basename(src) + ".o")) for src in srcs]
    with concurrent.futures.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda so: _run([HIPCC] + flags + ["-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    # the driver and the link through the same clang (one sanitizer runtime)
    exe = str(tmp_path / "host_asan")
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + san +
         ["-I", os.path.join(ROOT, "include"), os.path.join(HERE, "host_driver.cpp")] + objs +
         ["-o", exe, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    r = _run([exe], env=ENV)
    assert "all checks passed" in r.stdout
