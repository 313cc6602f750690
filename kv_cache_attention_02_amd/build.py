"""Build libwmk.so (the C-ABI library of include/wmk.h) for gfx950 with hipcc, in place."""
import os
import subprocess

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


def build(verbose=False, extra_flags=()):
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + FLAGS[:-0 or None] + list(extra_flags) + lang + ["-c", path, "-o", obj]
        cmd = [c for c in cmd if c != "-shared"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(r.stderr.replace("'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)\n", ""))
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    for o in objs:
        os.remove(o)
    cmd = [HIPCC] + FLAGS + list(extra_flags) + ["-x", "hip", os.path.join(CSRC, RATES_SOURCE), "-o",
                                                  RATES_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(RATES_LIB + ".tmp", RATES_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
