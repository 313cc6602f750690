"""The chunk-attention calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the library allocates, frees, synchronizes and clears nothing inside a call, so a serving
loop can capture its steady-state step.  On a full ring the key spans are fixed and only
the slots' contents change, so each replay, after an eager append of a new chunk, must
equal the eager call on the same state bit for bit.  Both the workspace entry point
(split tail plus merge kernel) and the no-allocation one are captured."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import dev_fill, from_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_chunk_attention_graph_replays_equal_eager(wmk, entry):
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128   # 288 units of 256 rows: the split tail runs
    nq = cf * tpf
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    fin = [(dev_fill((nq, H, D), seed=5, chunk=c, step=4, kind=synth.KFIN),
            dev_fill((nq, H, D), seed=5, chunk=c, step=4, kind=synth.VFIN)) for c in range(8)]
    for c in range(4):                      # 16 frames appended: the ring is full (14 resident)
        cache.append_evict(0, *fin[c], cf)
    q, k, v = (dev_fill((nq, H, D), seed=6, kind=t) for t in (synth.Q, synth.K, synth.V))
    out_g = torch.empty_like(q)

    def call(out):
        if entry == "workspace":
            return wmk.chunk_attention(cache, 0, q, [(k, v)], out=out)
        return wmk.chunk_attention_noalloc(cache, 0, q, out, [(k, v)])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(out_g)                          # workspace / library scratch set up before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out_g)
    torch.cuda.synchronize()
    for r in range(3):
        cache.append_evict(0, *fin[4 + r], cf)   # eager: the ring turns, the resident set keeps its size
        ref = torch.empty_like(q)
        call(ref)
        torch.cuda.synchronize()
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph {entry} replay {r}")
        assert np.array_equal(from_dev(out_g), from_dev(ref)), f"replay {r}"
        assert not np.array_equal(from_dev(ref), from_dev(torch.zeros_like(ref)))
    cache.close()
