"""Host code under AddressSanitizer (no GPU needed).

The C ABI's argument checks, slot arithmetic and launch planners (the host part
of libwmk.so) and the oracle's C core are rebuilt with AddressSanitizer in a
temporary directory, and the CPU tests that drive them -- the boundary tests in
dry-run mode and the oracle pins -- run against those builds in a child process
that aborts on the first report.  GPU code is never built with a sanitizer:
every sanitizer flag on a hipcc line is passed with -Xarch_host, and the HIP
sources are compiled as usual.  Takes about half a minute (one library build).
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from kv_cache_attention_02_amd import build as wmk_build  # noqa: E402

ASAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1"}
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run_child(script, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **ASAN_ENV)
    return subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def test_libwmk_host_code_under_asan(tmp_path):
    runtime = _clang_asan_runtime()
    if runtime is None or shutil.which(wmk_build.HIPCC) is None and not os.path.exists(wmk_build.HIPCC):
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    flags = [f for f in wmk_build.FLAGS if f != "-shared"]
    procs, objs = [], []
    for src in wmk_build.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = HOST_ASAN + ["-g"] if src.endswith(".cpp") else []
        cmd = [wmk_build.HIPCC] + flags + extra + lang + ["-c", os.path.join(wmk_build.CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for cmd, p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{' '.join(cmd)}\n{err[-2000:]}"
    lib = str(tmp_path / "libwmk_asan.so")
    link = [wmk_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_ASAN[:2] + \
        ["-Xarch_host", "-shared-libasan"] + objs + ["-o", lib]
    r = subprocess.run(link, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    script = ("import sys, pytest\n"
              f"sys.path.insert(0, {ROOT!r})\n"
              "import kv_cache_attention_02_amd as w\n"
              f"w.LIB_PATH = {lib!r}\n"
              "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', "
              f"{os.path.join(ROOT, 'tests', 'test_boundary.py')!r}]))\n")
    r = _run_child(script, runtime)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr


def test_oracle_core_under_asan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    runtime = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle.so")
    cmd = [gcc, "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-march=x86-64-v3", "-fopenmp",
           "-fPIC", "-shared", os.path.join(ROOT, "oracle", "attend.c"), "-o", lib, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    script = ("import sys, pytest\n"
              f"sys.path.insert(0, {ROOT!r})\n"
              "import oracle\n"
              f"oracle._DIR = {str(tmp_path)!r}\n"
              "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', "
              f"{os.path.join(ROOT, 'tests', 'test_oracle.py')!r}]))\n")
    r = _run_child(script, runtime)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr
