"""Shared helpers of the GPU tests: seeded inputs on host and device, and the
parity comparison.  Inputs for the oracle are always drawn on the host by the
seeded generator; the device gets the same bits by upload, or by the
generator's GPU twin where a test says so (checked bit-identical separately)."""
import sys

import numpy as np

import synth

# bf16 path: bounds on the sampled rows of an fp32 oracle comparison
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
# fp32 path: online softmax in fp32 against the fp64 oracle; errors are a few
# ulps of fp32 accumulated over at most a few thousand keys
F32_MAX_ABS = 1e-5
F32_REL_L2 = 1e-5
# log-sum-exp of the bf16 training forward (natural log): the kernel's row sum is the
# sum of the weights rounded to bf16 (the weights it multiplies V with), each within a
# relative 2^-8 (8-bit significand), so the sum is within a factor 1 +- 2^-8 of the exact
# one and the log-sum-exp within ln(1 + 2^-8) = 3.90e-3 (reached on rows of a few
# dominant keys; fp32 sums, exponentials and the log add ~1e-6)
LSE_ATOL = 4e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(shape, dtype="bf16", **key):
    """Seeded host array: uint16 bf16 bit patterns or float32."""
    n = int(np.prod(shape))
    return synth.normal(n, dtype=dtype, **key).reshape(shape)


def to_dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def from_dev(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def as_f32(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def dev_fill(shape, dtype="bf16", **key):
    """Device tensor drawn by the generator's GPU twin."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = torch.empty(shape, dtype=tdt, device="cuda")
    synth.gpu_fill(t.data_ptr(), t.numel(), dtype=dtype, stream=torch.cuda.current_stream().cuda_stream, **key)
    return t


def compare(got, ref, max_abs, rel_l2, what=""):
    """got: GPU rows (any float dtype, or bf16 bits); ref: oracle rows (fp64)."""
    g = as_f32(np.asarray(got)).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    ma = float(err.max()) if err.size else 0.0
    rl = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    say(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e} (bounds {max_abs:g}, {rel_l2:g})")
    assert ma <= max_abs, f"{what}: max-abs error {ma} > {max_abs}"
    assert rl <= rel_l2, f"{what}: relative L2 error {rl} > {rel_l2}"
    return ma, rl


def sample_rows(n, rng, k=32, tile=128):
    """Rows to check: first and last rows, every tile boundary region near the
    start and the end (ragged tail included) and random rows."""
    rows = set(range(min(n, 8))) | set(range(max(0, n - 8), n))
    for b in (tile, 2 * tile, (n // tile) * tile):
        rows |= {x for x in (b - 1, b, b + 1) if 0 <= x < n}
    rows |= set(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
    return np.array(sorted(rows))
