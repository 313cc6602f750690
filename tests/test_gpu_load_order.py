"""The library loaded before the caller's first torch tensor still works: the binding
imports torch (and its HIP runtime) before libwmk.so, so the library binds to the
runtime that owns the caller's memory and streams.  Runs in a child process, since this
one has torch loaded already."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import kv_cache_attention_02_amd as wmk
wmk.load()
import torch
c = wmk.Cache(num_layers=1, num_heads=1, head_dim=64, tokens_per_frame=4, sink_frames=1, window_frames=2,
              chunk_frames=1)
k = torch.arange(4 * 64, dtype=torch.float32, device="cuda").reshape(4, 1, 64).to(torch.bfloat16)
c.append_evict(0, k, -k, 1)
torch.cuda.synchronize()
assert torch.equal(c.k[0, 0].view(torch.int16), k.view(torch.int16))
assert torch.equal(c.v[0, 0].view(torch.int16), (-k).view(torch.int16))
print("load order ok", flush=True)
"""


def test_library_loaded_before_torch_tensors():
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "load order ok" in r.stdout
