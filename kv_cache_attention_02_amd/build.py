"""Build libwmk.so (the C-ABI library of include/wmk.h) for gfx950 with hipcc, in place."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["wmk_api.cpp", "attn_bf16.hip", "attn_f32.hip", "cache_append.hip", "quant_fp8.hip", "attn_bwd.hip",
           "noalloc.hip"]
LIB = os.path.join(PKG, "libwmk.so")
# measurement-only kernels (reference rates of the benchmark), kept out of libwmk.so
RATES_SOURCE = "rates.hip"
RATES_LIB = os.path.join(PKG, "libwmk_rates.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# the attention kernel with per-step phase timestamps (bench.py --step-profile), kept out of libwmk.so
STEPPROF_LIB = os.path.join(PKG, "libwmk_stepprof.so")


def build(verbose=False, extra_flags=()):
    """Compile every source of both libraries (in parallel), link them, and build the
    reference-rate library; returns the path of libwmk.so."""
    jobs = [(LIB, src, tuple(extra_flags)) for src in SOURCES]
    jobs += [(STEPPROF_LIB, src, tuple(extra_flags) + ("-DWMK_STEP_PROFILE",)) for src in SOURCES]
    jobs.append((RATES_LIB, RATES_SOURCE, tuple(extra_flags)))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j, verbose=verbose), jobs))
    for out in (LIB, STEPPROF_LIB):
        _link(out, [o for (lib, _, _), o in zip(jobs, objs) if lib == out])
    _link(RATES_LIB, [objs[-1]])
    return LIB


def _compile(out, src, extra_flags, verbose=False):
    path = os.path.join(CSRC, src)
    obj = out + "." + src + ".o"
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + list(extra_flags) + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(r.stderr.replace("'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)\n", ""))
    return obj


def _link(out, objs):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    for o in objs:
        os.remove(o)


if __name__ == "__main__":
    print(build(verbose=True))
