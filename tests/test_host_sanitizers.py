"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two programs are built with plain g++/gcc (no GPU code: the kernel source is left out and its
host-side launchers are stubs) and run:
  - tests/sanitize/host_checks.cpp: the task-graph builder, validator, simulator and the C ABI's
    host paths (host-only contexts for the workload shapes, batched graphs, every corruption kind,
    refused configurations and arguments);
  - tests/sanitize/oracle_checks.c: the oracle (both its fp64 and fp32 builds) decoding a small
    model through its cache and without one, its cache accessors and argument checks.
A memory error, a leak or undefined behaviour makes the program exit non-zero with the sanitizer's
report, and the test fails with it.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


@pytest.fixture(scope="module")
def outdir():
    d = tempfile.mkdtemp(prefix="mk_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"), reason="needs g++ and HIP headers")
def test_host_runtime_and_graph_under_sanitizers(outdir):
    exe = os.path.join(outdir, "host_checks")
    csrc = os.path.join(ROOT, "persistent_megakernel_03_amd", "csrc")
    run(["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                        os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
                                        os.path.join(csrc, "mk_api.cpp"), os.path.join(csrc, "mk_graph.cpp"),
                                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = run([exe], env=ENV, timeout=600)
    assert "0 failures" in r.stdout


@pytest.mark.parametrize("precision", ["f64", "f32"])
def test_oracle_under_sanitizers(outdir, precision):
    exe = os.path.join(outdir, "oracle_checks_" + precision)
    extra = ["-DORC_FP32"] if precision == "f32" else []
    run(["gcc", "-std=c11"] + SAN + ["-fopenmp", "-ffp-contract=off"] + extra +
        [os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(ROOT, "seeded_inputs", "gen.c"), "-lm", "-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout
