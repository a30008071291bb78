"""The library's host code under AddressSanitizer, on the CPU.

The C ABI's host side (argument validation, pool bookkeeping, chunk and segment
planning, the error paths) is built with AddressSanitizer on the host pass only
(every -fsanitize= after -Xarch_host; the gfx950 device code is built as usual), and
the CPU tests of the ABI run against that build in a child process with the
sanitizer runtime preloaded.  Any invalid host memory access there aborts the child
with a sanitizer report.  No GPU is used: the error paths return before any launch.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_code_is_clean_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the sanitizer runtime is not available")
    sys.path.insert(0, ROOT)
    from pool_score_top_amd import build as B
    csrc = os.path.join(ROOT, "pool_score_top_amd", "csrc")
    flags = [f for f in B.FLAGS if f != "-shared"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    procs = []
    for s in B.SOURCES:
        obj = str(tmp_path / s.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, *B.FILE_FLAGS.get(s, []), *san, "-c",
                                       os.path.join(csrc, s), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    lib = str(tmp_path / "libkpool_asan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import pool_score_top_amd.kpool as K\n"
            "K.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main([%r, %r, '-q', '-m', 'not gpu', '-p', 'no:cacheprovider']))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi_cpu.py"),
               os.path.join(ROOT, "tests", "test_zz_no_alloc.py")))
    # (reports go to files: the child's pytest captures its stderr, and a sanitizer abort
    # ends the child before that capture is printed)
    log = str(tmp_path / "asan")
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    reports = "".join(open(f).read() for f in glob.glob(log + "*"))
    assert not reports, reports[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
