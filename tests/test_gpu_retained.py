"""GPU parity of chunk attention with variable retention (a per-call subset of
the resident frames, plus auxiliary KV blocks passed as segments) through the C
ABI: all rows against the oracle on small ragged shapes -- few and many runs of
adjacent slots, bf16 and fp32 -- sampled rows at the 832x464 shape, and bit
equality with plain chunk attention over the same keys gathered by hand."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_REL_L2, compare, dev_fill, from_dev,
                               host, sample_rows, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


def _filled(wmk, S, W, cf, tpf, H, D, n_chunks, dtype, seed):
    """A one-layer cache and its oracle model after n_chunks seeded appends."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf, dtype=tdt)
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for c in range(n_chunks):
        k = host((cf * tpf, H, D), dtype, seed=seed, chunk=c, step=4, kind=synth.KFIN)
        v = host((cf * tpf, H, D), dtype, seed=seed, chunk=c, step=4, kind=synth.VFIN)
        cache.append_evict(0, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
    return cache, cm


@pytest.mark.parametrize("S,W,cf,tpf,H,D,n_chunks,pick,dtype", [
    (2, 4, 2, 37, 2, 128, 5, "random", "bf16"),       # ragged frames, a few runs
    (0, 12, 3, 29, 2, 64, 6, "alternate", "bf16"),    # 6 runs of one slot: the many-span kernel
    (6, 8, 4, 21, 1, 128, 5, "anchors_last2", "bf16"),
    (3, 1, 1, 50, 2, 128, 4, "none", "bf16"),         # nothing retained: segments only
    (2, 4, 2, 13, 2, 64, 5, "alternate", "f32"),
])
def test_retained_small_all_rows(wmk, S, W, cf, tpf, H, D, n_chunks, pick, dtype):
    import torch
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, n_chunks, dtype, seed=31)
    res = cm.resident()
    rng = np.random.default_rng(4)
    if pick == "random":
        keep = [f for f in res if rng.random() < 0.5] or res[:1]
    elif pick == "alternate":
        keep = [f for f in res if oracle.slot_of_frame(f, S, W) % 2 == 0]
    elif pick == "anchors_last2":
        keep = [f for f in res if f < S] + [f for f in res if f >= S][-2:]
    else:
        keep = []
    keep = [int(f) for f in rng.permutation(keep)]       # any order
    nq = cf * tpf
    q, k, v = (host((nq, H, D), dtype, seed=32, kind=t) for t in (synth.Q, synth.K, synth.V))
    ka, va = host((70, H, D), dtype, seed=33, kind=synth.KLOC), host((70, H, D), dtype, seed=33, kind=synth.VLOC)
    say(f"retained S={S} W={W} tpf={tpf} H={H} D={D} {dtype} keep={sorted(keep)}")
    out = wmk.chunk_attention(cache, 0, to_dev(q), [(to_dev(k), to_dev(v)), (to_dev(ka), to_dev(va))],
                              keep_frames=keep)
    torch.cuda.synchronize()
    ref = oracle.chunk_attention(cm, q, [(k, v), (ka, va)], 1 / math.sqrt(D), keep_frames=keep)
    if dtype == "bf16":
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, "all rows")
    else:
        compare(from_dev(out), ref, F32_MAX_ABS, F32_REL_L2, "all rows")
    cache.close()


@pytest.mark.parametrize("pick", ["alternate", "anchors_last4"])
def test_retained_equals_hand_gathered_keys(wmk, pick):
    """The kept frames' rows gathered into one segment, in slot order, give the same
    keys at the same positions: the outputs agree bit for bit (832x464 layer)."""
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    for c in range(5):
        cache.append_evict(0, dev_fill((cf * tpf, H, D), seed=34, chunk=c, step=4, kind=synth.KFIN),
                           dev_fill((cf * tpf, H, D), seed=34, chunk=c, step=4, kind=synth.VFIN), cf)
    slots, F = cache.slots(0)
    if pick == "alternate":
        keep_slots = [s for s in range(S + W) if s % 2 == 1]
    else:
        recent = sorted((f, s) for s, f in enumerate(slots) if f >= S)[-4:]
        keep_slots = sorted(list(range(S)) + [s for _, s in recent])
    keep = [slots[s] for s in keep_slots]
    q, k, v = (dev_fill((cf * tpf, H, D), seed=35, kind=t) for t in (synth.Q, synth.K, synth.V))
    say(f"retained vs gathered 832x464 keep slots {keep_slots}")
    out = wmk.chunk_attention(cache, 0, q, [(k, v)], keep_frames=keep)
    kg = cache.k[0, keep_slots].reshape(-1, H, D).contiguous()
    vg = cache.v[0, keep_slots].reshape(-1, H, D).contiguous()
    ref = wmk.chunk_attention(None, 0, q, [(kg, vg), (k, v)])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    cache.close()


def test_retained_832x464_sampled_rows(wmk):
    """Steady-state 832x464 cache (14 resident frames), anchors plus the 4 latest
    recent frames retained, one 1508-token auxiliary block: sampled rows."""
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, 5, "bf16", seed=36)
    res = cm.resident()
    keep = [f for f in res if f < S] + [f for f in res if f >= S][-4:]
    nq = cf * tpf
    q, k, v = (host((nq, H, D), seed=37, kind=t) for t in (synth.Q, synth.K, synth.V))
    ka, va = host((tpf, H, D), seed=37, kind=synth.KLOC), host((tpf, H, D), seed=37, kind=synth.VLOC)
    say(f"retained 832x464 keep={keep} + auxiliary block")
    out = wmk.chunk_attention(cache, 0, to_dev(q), [(to_dev(k), to_dev(v)), (to_dev(ka), to_dev(va))],
                              keep_frames=keep)
    torch.cuda.synchronize()
    rows = sample_rows(nq, np.random.default_rng(8), k=24, tile=256)
    ref = oracle.chunk_attention(cm, q, [(k, v), (ka, va)], 1 / math.sqrt(D), rows=rows, keep_frames=keep)
    compare(from_dev(out)[rows], ref, BF16_MAX_ABS, BF16_REL_L2, f"{len(rows)} sampled rows")
    cache.close()


@pytest.mark.parametrize("seed", range(8))
def test_retained_random_shapes_all_rows(wmk, seed):
    """Every row of seeded random retained calls against the oracle: random cache shape,
    head_dim 64 or 128, a random subset of the resident frames listed in random order,
    with or without an auxiliary block, with and without the split-tail workspace."""
    import torch
    rng = np.random.default_rng(500 + seed)
    S, W, cf = int(rng.integers(0, 6)), int(rng.integers(1, 10)), int(rng.integers(1, 5))
    tpf, H, D = int(rng.integers(20, 201)), int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    n_chunks = int(rng.integers(2, 10))
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, n_chunks, "bf16", seed=600 + seed)
    res = cm.resident()
    p = rng.uniform(0.2, 0.9)
    keep = [int(f) for f in rng.permutation([f for f in res if rng.random() < p])]
    nq = cf * tpf
    q, k, v = (host((nq, H, D), seed=700 + seed, kind=t) for t in (synth.Q, synth.K, synth.V))
    segs = [(k, v)]
    n_aux = int(rng.integers(0, 151))
    if n_aux:
        segs.append((host((n_aux, H, D), seed=800 + seed, kind=synth.KLOC),
                     host((n_aux, H, D), seed=800 + seed, kind=synth.VLOC)))
    say(f"retained random seed {seed}: S={S} W={W} cf={cf} tpf={tpf} H={H} D={D} chunks={n_chunks} "
        f"keep={sorted(keep)} aux={n_aux}")
    ref = oracle.chunk_attention(cm, q, segs, 1 / math.sqrt(D), keep_frames=keep)
    for use_ws in (False, True):
        out = wmk.chunk_attention(cache, 0, to_dev(q), [(to_dev(a), to_dev(b)) for a, b in segs],
                                  keep_frames=keep, use_workspace=use_ws)
        torch.cuda.synchronize()
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"seed {seed} all rows ws={use_ws}")
    cache.close()
