"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; the device code is unchanged).

`python -m audio_encoder_tower_amd.build --sanitize` builds a copy of
libaenc.so whose host pass is instrumented; this test (re)builds it when a
source is newer, then runs tests/test_abi_host.py against it in a child
process with the sanitizer runtime preloaded: geometry validation, the
closed forms (parameter count, output shape, workspace and scratch sizes),
the NULL-argument and bad-size paths of every entry point, the front-end
configuration checks and, without a device, the failure path of create.
Any sanitizer report fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


def _asan_runtime():
    for clang in (shutil.which("clang"), "/opt/rocm/llvm/bin/clang"):
        if clang and os.path.exists(clang):
            out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                 text=True).stdout.strip()
            if out and os.path.isabs(out) and os.path.exists(out):
                return out
    return None


@pytest.fixture(scope="module")
def sanitized_lib():
    if not _hipcc():
        pytest.skip("hipcc is not installed")
    rt = _asan_runtime()
    if not rt:
        pytest.skip("no AddressSanitizer runtime next to the ROCm clang")
    from audio_encoder_tower_amd import build as b
    srcs = glob.glob(os.path.join(b.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h")) + [b.__file__]
    newest = max(os.path.getmtime(f) for f in srcs)
    if not os.path.exists(b.SANITIZE_LIB) or os.path.getmtime(b.SANITIZE_LIB) < newest:
        b.build(jobs=8, sanitize=True)
    return b.SANITIZE_LIB, rt


def _env(lib, rt):
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, AENC_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("PYTEST_XDIST_WORKER", None)
    return env


def test_sanitized_library_is_the_one_loaded(sanitized_lib):
    lib, rt = sanitized_lib
    code = ("import audio_encoder_tower_amd as a; a.lib(); "
            "maps = open('/proc/self/maps').read(); "
            f"assert {lib!r} in maps, 'sanitized library not mapped'; "
            "assert 'libclang_rt.asan' in maps, 'sanitizer runtime not mapped'; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib, rt), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_host_abi_under_asan_and_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-p", "no:xdist",
                        "tests/test_abi_host.py"], cwd=ROOT, env=_env(lib, rt), capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
