"""Host-only AddressSanitizer + UndefinedBehaviorSanitizer builds (no GPU involved).

- The fp64 oracle (oracle/oracle.c), driven by tests/sanitize/oracle_checks.c: routing, expert FFNs and
  whole layers in every gating and activation mode, fp32 and bf16, and its argument checks.
- libmoe's C ABI with its host code sanitized (device code compiled as usual, never launched), driven by
  tests/sanitize/abi_checks.c: every argument check of every entry point returns its error status before
  any HIP call.
Any memory error or undefined behaviour aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# sanitizer flags for the host half of a HIP compile only (each one behind -Xarch_host)
HOST_SAN = [f for x in ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer"] for f in ("-Xarch_host", x)]


def run(cmd, **kw):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert p.returncode == 0, "%s\n%s" % (" ".join(cmd), p.stdout[-4000:])
    return p.stdout


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="moe_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp):
    exe = os.path.join(tmp, "oracle_checks")
    run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off"] + SAN +
        [os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), os.path.join(ROOT, "oracle", "oracle.c"),
         "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4")
    assert "oracle checks ok" in run([exe], env=env)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_argument_checks_under_asan_ubsan(tmp):
    csrc = os.path.join(ROOT, "fine_grained_shared_amd", "csrc")
    objs, procs = [], []
    for f in ("api", "router", "dispatch", "ffn", "combine"):
        o = os.path.join(tmp, f + ".o")
        objs.append(o)
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC"] + HOST_SAN + \
              ["-c", os.path.join(csrc, f + ".hip"), "-o", o]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for cmd, p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, "%s\n%s" % (" ".join(cmd), out[-4000:])
    drv = os.path.join(tmp, "drv.o")
    run([CLANG, "-O1", "-g"] + SAN + ["-c", os.path.join(ROOT, "tests", "sanitize", "abi_checks.c"), "-o", drv])
    exe = os.path.join(tmp, "abi_checks")
    # link: the sanitizer runtimes for the host code; -fno-gpu-sanitize keeps the device code as built
    run([HIPCC, "--offload-arch=gfx950", "-fno-gpu-sanitize"] + SAN[:1] + objs + [drv, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    assert "abi checks ok" in run([exe], env=env)
