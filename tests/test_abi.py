"""Host-side checks of the C ABI (tests/abi_checks.py), run in child
processes so that no GPU is ever touched by them:

* against the built libwanattn.so with HIP_VISIBLE_DEVICES and
  ROCR_VISIBLE_DEVICES hiding every GPU from the child before it starts: the
  checks pass fake device addresses, and should a host check regress, the
  call would reach a launch that fails for want of a device instead of
  dereferencing them;
* against a host-only build of the ABI layer (wan_api.cpp compiled by g++
  under AddressSanitizer and UndefinedBehaviorSanitizer, the kernel launchers
  replaced by tests/hostcheck/launch_stubs.cpp, which launch nothing and
  return an error): every rejection path runs under the sanitizers.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKS = os.path.join(ROOT, "tests", "abi_checks.py")
HOSTCHECK_DIR = os.path.join(ROOT, "_build", "hostcheck")
HOSTCHECK_LIB = os.path.join(HOSTCHECK_DIR, "libwanattn_hostcheck.so")
NO_GPU = {"HIP_VISIBLE_DEVICES": "-1", "ROCR_VISIBLE_DEVICES": "-1"}


def _child(env_extra, *args):
    env = dict(os.environ, PYTHONPATH=ROOT, **NO_GPU, **env_extra)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", CHECKS,
                           *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_abi_checks_without_a_visible_gpu():
    from attention_wan_qk_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from attention_wan_qk_amd.build import build
        build(verbose=False)
    r = _child({})
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]


def _sanitizer_runtime():
    try:
        path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_under_address_and_ub_sanitizers():
    asan = _sanitizer_runtime()
    if asan is None:
        pytest.skip("g++ with AddressSanitizer is not available")
    os.makedirs(HOSTCHECK_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "attention_wan_qk_amd", "csrc", "wan_api.cpp"),
           os.path.join(ROOT, "tests", "hostcheck", "launch_stubs.cpp"), "-o", HOSTCHECK_LIB]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    r = _child({"WANATTN_TEST_LIB": HOSTCHECK_LIB, "LD_PRELOAD": asan,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"},
               "-k", "rejections or exports or status")
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-5000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-5000:]
