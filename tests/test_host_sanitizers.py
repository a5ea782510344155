"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the library's host code.

The library is built a second time, with the host half of every source instrumented
(``-Xarch_host -fsanitize=address`` and ``-Xarch_host -fsanitize=undefined``, UB made
fatal); the GPU code objects are the ordinary ones and nothing is launched.  The ABI and
binding tests then run against that build in a child process with the sanitizer runtime
preloaded: argument validation, the overlap checks of every entry point, the scope table,
the FLOP counts and the status strings all execute under the sanitizers, and any report
fails this test.  No GPU is involved.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

from skiparse_sparse_attention_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")


def _asan_runtime():
    res = subprocess.run([CLANGXX, "-print-resource-dir"], capture_output=True, text=True)
    if res.returncode != 0:
        return None
    for sub in ("lib/linux/libclang_rt.asan-x86_64.so", "lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"):
        path = os.path.join(res.stdout.strip(), sub)
        if os.path.exists(path):
            return path
    return None


ASAN_RT = _asan_runtime() if os.path.exists(CLANGXX) else None

pytestmark = pytest.mark.skipif(ASAN_RT is None or not os.path.exists(libbuild.hipcc()),
                                reason="hipcc or the clang sanitizer runtime is not installed")

HOST_SANITIZE = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src, obj):
    flags = [f for f in libbuild.HIPCC_FLAGS if f != "-shared"]
    cmd = [libbuild.hipcc(), *flags, *HOST_SANITIZE, "-c", "-o", obj, os.path.join(libbuild.CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return src, res.returncode, res.stdout + res.stderr


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("hostsan")
    objs = [str(out / (src + ".o")) for src in libbuild.SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(objs))) as pool:
        for src, rc, log in pool.map(_compile, libbuild.SOURCES, objs):
            assert rc == 0, f"sanitizer build of {src} failed:\n{log}"
    lib = str(out / "libskiparse_amd_hostsan.so")
    link = [CLANGXX, "-shared", "-fsanitize=address,undefined", "-shared-libsan", "-o", lib, *objs,
            "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return lib, out


def test_abi_and_binding_tests_are_clean_under_host_sanitizers(sanitized_lib):
    lib, out = sanitized_lib
    log = str(out / "sanitizer")
    env = dict(os.environ)
    env.update({
        "SKIPARSE_AMD_LIB": lib,
        "LD_PRELOAD": ASAN_RT,
        # the interpreter itself is not instrumented: leaks at exit are its own
        "ASAN_OPTIONS": f"detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:log_path={log}",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={log}",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_binding.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(p for p in os.listdir(out) if p.startswith("sanitizer"))
    text = "".join(open(os.path.join(out, p)).read() for p in reports)
    assert not reports, f"sanitizer reports:\n{text[:4000]}"
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert " passed" in res.stdout and "failed" not in res.stdout
    # a child with the same environment really opens the instrumented build
    probe = subprocess.run([sys.executable, "-c", "import skiparse_sparse_attention_amd as sk; "
                            "print(sk.lib()._name); print(sk.version())"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0, probe.stderr
    assert probe.stdout.splitlines()[0] == lib
    shutil.rmtree(out, ignore_errors=True)
