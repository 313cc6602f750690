"""Seeded synthetic inputs shared by the oracle-side tests and the GPU tests.

This module only draws numbers; it holds none of the attention or cache
arithmetic.  Every value comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
SC'11) under a counter built from the element index and a key built from the
seed, turned into an approximately N(0,1) value by the Irwin-Hall sum of twelve
uniform bytes: ``x = (sum - 1530) / 256`` (exact in fp32), rounded to bf16 with
round-to-nearest-even for bf16 tensors.

Three implementations must agree bit for bit:

* :func:`philox4x32_10_np` / :func:`normal_np` -- NumPy, written from the
  published definition, for small arrays and known-answer checks;
* ``philox.c`` (``libsynth_cpu.so``) -- the same in C with OpenMP, for large
  host arrays;
* ``gen.hip`` (``libsynth_gpu.so``) -- the GPU twin, for large device tensors.

The stream key of an element is (seed, chunk, layer, step, kind); ``kind``
names the tensor role so that Q, K, V and the finalized K/V of one step are
independent draws.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))

# Tensor roles (the low byte of the fourth counter word).
Q, K, V, KFIN, VFIN, KENV, VENV, KLOC, VLOC = range(9)

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10_np(ctr, key):
    """Philox4x32-10 on arrays: ``ctr`` is a (4, n) uint32-valued array, ``key`` a pair."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in ctr]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return [x.astype(np.uint32) for x in c]


def _tag(kind, step, layer):
    return (kind & 0xFF) | ((step & 0xFF) << 8) | (layer << 16)


def normal_np(n, *, seed=0, chunk=0, layer=0, step=0, kind=Q, start=0):
    """fp32 values of elements ``start .. start+n-1`` (NumPy version, for small n)."""
    idx = np.arange(start, start + n, dtype=np.uint64)
    ctr = [idx & _MASK32, idx >> np.uint64(32),
           np.full(n, chunk, dtype=np.uint64), np.full(n, _tag(kind, step, layer), dtype=np.uint64)]
    o = philox4x32_10_np(ctr, (seed & 0xFFFFFFFF, seed >> 32))
    s = np.zeros(n, dtype=np.int64)
    for w in o[:3]:
        w = w.astype(np.int64)
        for b in range(4):
            s += (w >> (8 * b)) & 0xFF
    return ((s - 1530).astype(np.float32) / np.float32(256.0)).astype(np.float32)


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (nearest-even) and return the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_cpu = None
_gpu = None


def _load_cpu():
    global _cpu
    if _cpu is None:
        path = os.path.join(_DIR, "libsynth_cpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        for name, ptr_t in (("synth_fill_f32", ctypes.c_void_p), ("synth_fill_bf16", ctypes.c_void_p)):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [ptr_t, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                          ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        lib.synth_philox4x32_10.restype = None
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _cpu = lib
    return _cpu


def philox4x32_10_c(ctr, key):
    """One Philox4x32-10 block through the C implementation (for cross-checks)."""
    lib = _load_cpu()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    o = np.zeros(4, dtype=np.uint32)
    lib.synth_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return o


def normal(n, *, dtype="bf16", seed=0, chunk=0, layer=0, step=0, kind=Q, start=0):
    """Host array of n draws: uint16 bf16 bit patterns (dtype='bf16') or float32 (dtype='f32')."""
    lib = _load_cpu()
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.synth_fill_bf16(out.ctypes.data, start, n, seed, chunk, layer, step, kind)
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.synth_fill_f32(out.ctypes.data, start, n, seed, chunk, layer, step, kind)
    else:
        raise ValueError(dtype)
    return out


def _load_gpu():
    global _gpu
    if _gpu is None:
        path = os.path.join(_DIR, "libsynth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (bind to torch's HIP runtime, which owns the memory and streams passed in)
        lib = ctypes.CDLL(path)
        lib.synth_gpu_fill.restype = ctypes.c_int
        lib.synth_gpu_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                       ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_void_p]
        _gpu = lib
    return _gpu


def gpu_fill(ptr, n, *, dtype="bf16", seed=0, chunk=0, layer=0, step=0, kind=Q, start=0, stream=0):
    """Fill n elements at device address ``ptr`` on ``stream`` (a raw hipStream_t value)."""
    lib = _load_gpu()
    rc = lib.synth_gpu_fill(ctypes.c_void_p(ptr), start, n, 1 if dtype == "bf16" else 0, seed, chunk, layer,
                            step, kind, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill failed with HIP error {rc}")


def build(verbose=False):
    """Compile libsynth_cpu.so (gcc) and libsynth_gpu.so (hipcc, gfx950) in place."""
    import subprocess
    cmds = [
        ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", os.path.join(_DIR, "philox.c"),
         "-o", os.path.join(_DIR, "libsynth_cpu.so")],
        ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         os.path.join(_DIR, "gen.hip"), "-o", os.path.join(_DIR, "libsynth_gpu.so")],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(c)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr:
            print(r.stderr)
