"""Host-side guards that need no GPU:

* every GEMM launch the library makes for the model shapes reads its packed
  weights inside their bounds (tests/plan_bounds.cpp evaluates the kernels'
  address arithmetic over each launch grid on the host), and every attention
  key split the library picks is a whole number of 64-key tiles in range,
  with long-context sessions fitting a full-capacity launch in one round of
  workgroups;
* the runtime's host code built with AddressSanitizer and
  UndefinedBehaviorSanitizer passes the host-only C-ABI tests (argument
  validation, model and session sizing, the mode choice by concurrency) and
  the launch-plan checks above (including the attention's compacted-grid
  tables)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "self_speculative_lm_amd")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs the HIP compiler")


def _lib():
    from self_speculative_lm_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from self_speculative_lm_amd.build import build
        build()
    return _lib.LIB_PATH


def test_launch_plans_stay_inside_their_bounds(tmp_path):
    from self_speculative_lm_amd.build import hipcc
    lib = _lib()
    exe = str(tmp_path / "plan_bounds")
    cmd = [hipcc(), "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
           os.path.join(ROOT, "tests", "plan_bounds.cpp"), "-o", exe, "-L" + os.path.dirname(lib), "-ltrimode",
           "-Wl,-rpath," + os.path.dirname(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from self_speculative_lm_amd.build import build, sanitizer_runtime
    out = str(tmp_path / "libtrimode_san.so")
    build(sanitize=True, out=out)
    rt = sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    tests = [os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_host_policy.py")]
    code = ("import sys, pytest; sys.path.insert(0, %r); import self_speculative_lm_amd._lib as L; L.LIB_PATH = %r; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider'] + %r))" % (ROOT, out, tests))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    # the launch-plan checks (GEMM plans and reaches, attention splits and
    # compacted-grid tables) against the sanitized host code as well
    from self_speculative_lm_amd.build import hipcc
    exe = str(tmp_path / "plan_bounds_san")
    cmd = [hipcc(), "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
           os.path.join(ROOT, "tests", "plan_bounds.cpp"), "-o", exe, "-L" + os.path.dirname(out),
           "-l:" + os.path.basename(out), "-Wl,-rpath," + os.path.dirname(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    print(r.stdout[-1000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
