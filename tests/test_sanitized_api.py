"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

The library is rebuilt with both sanitizers on the host code (build.py --sanitize: every -fsanitize
after -Xarch_host, the GPU code as in the normal build), and tests/test_api.py -- the export list,
the status strings and every validation path of every entry point, including the stride and extent
arithmetic -- runs against it in a subprocess with the clang ASan runtime preloaded. Any sanitizer
report ends that process with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

from tiled_online_softmax_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(lib, runtime):
    env = dict(os.environ)
    env["FA_LIBRARY"] = lib
    pre = env.get("LD_PRELOAD")
    env["LD_PRELOAD"] = runtime + (":" + pre if pre else "")  # the runtime first, anything already preloaded kept
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    return env


def test_c_abi_validation_under_asan_and_ubsan(tmp_path):
    try:
        build.hipcc()
        runtime = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build(out=str(tmp_path / "libfa_san.so"), sanitize=True)
    env = _env(lib, runtime)
    # the sanitised build is the library the binding loads, inside a process running the ASan runtime
    probe = ("import ctypes, sys; from tiled_online_softmax_amd import fa; fa.lib(); "
             "assert fa.LIB_PATH == sys.argv[1], fa.LIB_PATH; ctypes.CDLL(None)['__asan_init']; print('ok')")
    r = subprocess.run([sys.executable, "-c", probe, lib], env=env, capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_api.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
