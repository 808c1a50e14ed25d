"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): build the host-sanitized library (moe_layer_amd/build_sanitized.py:
device code as usual, the argument checks, workspace sizing, launch set-up and
switch policy instrumented), then run the C-ABI and switch-policy tests
against it in a child process with the sanitizer runtime preloaded.  Any
report aborts the child, so the suite must pass as a whole."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_switch_policy_under_host_sanitizers():
    from moe_layer_amd import build_sanitized as S
    lib = S.build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms   # the host code really is instrumented
    env = dict(os.environ, MOE_LAYER_AMD_LIB=lib, LD_PRELOAD=S.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_switch_policy.py"),
                        os.path.join(ROOT, "tests", "test_sanitized_host.py") + "::test_library_is_the_sanitized_one"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "failed" not in r.stdout


def test_library_is_the_sanitized_one():
    """Inside the child: the binding loaded the library named by the environment."""
    import moe_layer_amd
    want = os.environ.get("MOE_LAYER_AMD_LIB")
    moe_layer_amd.lib()
    from moe_layer_amd import _lib
    if want:
        assert _lib.LIB_PATH == want
        maps = open("/proc/self/maps").read()
        assert want in maps
