"""GPU: wmk_chunk_attention_noalloc (the split tail's scratch held by the library,
no allocation) against wmk_chunk_attention with a caller workspace, through the C
ABI: two calls in a row on the 832x464 18-slot step, the second with a smaller
input (5500 queries and a 2-frame current chunk: 8 units split in 32 pieces
instead of 32 units in 8 reuse the array), then a call of short key walks (no
cache, a 512-token environment and a 512-token local prompt: the 4-wave kernel
shape, whose 128-row pieces reuse the array again).  Every plan matches the
workspace entry point's, so the outputs are bit-identical; each call is also
checked against the oracle on sampled rows.  Named to run last: it leaves the
library's per-device array in use."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import BF16_MAX_ABS, BF16_REL_L2, compare, from_dev, host, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


def test_noalloc_matches_workspace_entry_two_calls(wmk):
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for c in range(4):
        k = host((cf * tpf, H, D), seed=80, chunk=c, step=4, kind=synth.KFIN)
        v = host((cf * tpf, H, D), seed=80, chunk=c, step=4, kind=synth.VFIN)
        cache.append_evict(0, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
    for call, (nq, nk) in enumerate(((cf * tpf, cf * tpf), (5500, 2 * tpf))):
        q = host((nq, H, D), seed=81 + call, kind=synth.Q)
        k = host((nk, H, D), seed=81 + call, kind=synth.K)
        v = host((nk, H, D), seed=81 + call, kind=synth.V)
        tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
        say(f"noalloc call {call}: q {nq}, current keys {nk}")
        ref = wmk.chunk_attention(cache, 0, tq, [(tk, tv)], use_workspace=True)
        out = torch.full_like(tq, float("nan"))
        wmk.chunk_attention_noalloc(cache, 0, tq, out, [(tk, tv)])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {call}: outputs differ"
        rows = sample_rows(nq, np.random.default_rng(call), k=12, tile=256)
        compare(from_dev(out)[rows], oracle.chunk_attention(cm, q, [(k, v)], 1 / math.sqrt(D), rows=rows),
                BF16_MAX_ABS, BF16_REL_L2, f"call {call}: {len(rows)} rows vs oracle")
    # short walks: 12288 queries x 12 heads over 512 + 512 keys -> 96 q-tiles of 128 rows x 12 heads = 1152
    # units, two full rounds of 512 workgroups and 128 units split in two
    nq = 12288
    q = host((nq, H, D), seed=90, kind=synth.Q)
    segs = [(host((512, H, D), seed=90, kind=synth.KENV), host((512, H, D), seed=90, kind=synth.VENV)),
            (host((512, H, D), seed=90, chunk=1, kind=synth.KLOC), host((512, H, D), seed=90, chunk=1, kind=synth.VLOC))]
    tq = to_dev(q)
    tsegs = [(to_dev(k), to_dev(v)) for k, v in segs]
    say("noalloc call 2: no cache, q 12288, 512 + 512 keys")
    ref = wmk.chunk_attention(None, 0, tq, tsegs, use_workspace=True)
    out = torch.full_like(tq, float("nan"))
    wmk.chunk_attention_noalloc(None, 0, tq, out, tsegs)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "call 2: outputs differ"
    rows = sample_rows(nq, np.random.default_rng(2), k=12, tile=128)
    compare(from_dev(out)[rows], oracle.chunk_attention(oracle.CacheModel(S, W, tpf, H, D), q, segs, 1 / math.sqrt(D),
                                                        rows=rows),
            BF16_MAX_ABS, BF16_REL_L2, f"call 2: {len(rows)} rows vs oracle")
    cache.close()
