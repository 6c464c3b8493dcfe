"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds a copy of libsgmv whose host code (the C-ABI's argument validation, the host segment
builder, the grouping cache's host path, the no-alloc entry point's checks) is instrumented
with -fsanitize=address,undefined; device code is compiled as usual and never runs. A child
process with the sanitizer runtime preloaded then drives that copy through its C-ABI
(tests/sanitize_driver.py): host builds compared with the oracle, bad ids, the cache, and
every argument error that returns before a launch. Any report aborts the child, so the test
passes only on a clean run.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segmented_gather_gemv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not (os.path.exists(_hipcc()) and os.path.exists(CLANG)):
        pytest.skip("ROCm toolchain not found")
    out = tmp_path_factory.mktemp("san")
    # the sanitizers apply to the host compilation only (each flag behind -Xarch_host)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC]
    cmds, objs = [], []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip"):
            o = str(out / (f + ".o"))
            cmds.append([_hipcc(), "--offload-arch=gfx950", "-Xclang", "-target-feature",
                         "-Xclang", "-packed-fp32-ops", *host_san, *common, "-c",
                         os.path.join(CSRC, f), "-o", o])
            objs.append(o)
        elif f.endswith(".cpp"):
            o = str(out / (f + ".o"))
            cmds.append([CLANG, "-fsanitize=address,undefined",
                         "-fno-sanitize-recover=undefined", *common, "-c",
                         os.path.join(CSRC, f), "-o", o])
            objs.append(o)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(_run, cmds))
    lib = str(out / "libsgmv_san.so")
    _run([CLANG, "-shared", "-fsanitize=address,undefined", "-shared-libasan", "-o", lib, *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    assert os.path.exists(rt), rt
    return lib, rt


def _driver(lib, rt, *extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # leaks of the interpreter itself are not this library's; every other report aborts
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # nothing here may reach a GPU
    return subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize_driver.py"),
                           lib, *extra], capture_output=True, text=True, env=env, timeout=600)


def test_instrumented_build_reports_a_planted_overflow(sanitized_lib):
    """The build is really instrumented: a host array one entry short is reported."""
    lib, rt = sanitized_lib
    r = _driver(lib, rt, "--plant-overflow")
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
    assert "planted overflow was not reported" not in r.stdout


def test_host_code_is_clean_under_asan_and_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    r = _driver(lib, rt)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "sanitize driver ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
