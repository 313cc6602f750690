"""GPU parity: the HIP path through the C ABI against the oracle, on the same
seeded inputs.  Cache slot maps and contents are compared bit for bit;
attention rows within max-abs 2e-2 and relative L2 1e-2 (bf16) of the fp64
oracle, or 1e-5 (fp32)."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_REL_L2, as_f32, compare, dev_fill,
                               from_dev, host, sample_rows, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


# ----------------------------------------------------------------------------------------------
# input generator: GPU twin == host
# ----------------------------------------------------------------------------------------------

def test_generator_gpu_twin_is_bit_identical(wmk):
    import torch
    for kind in range(9):
        for dt in ("bf16", "f32"):
            key = dict(seed=7, chunk=kind + 3, layer=29, step=kind % 5, kind=kind, start=(1 << 32) - 500_000)
            say(f"generator kind={kind} dtype={dt}")
            g = from_dev(dev_fill((1_000_000,), dt, **key))
            h = host((1_000_000,), dt, **key)
            assert np.array_equal(g.view(np.uint32) if dt == "f32" else g, h.view(np.uint32) if dt == "f32" else h)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------------------------
# tiny rollout, fp32: 1 head, head_dim 64, 16 tokens per frame, chunks of 2 frames,
# 1 sink + window 2, six chunks with append/evict after each
# ----------------------------------------------------------------------------------------------

def _dense_rollout_ref(q, k, v, S, W, cf, tpf, scale):
    n = q.shape[0]
    fr = np.arange(n) // tpf
    cq, ck = fr[:, None] // cf, fr[None, :] // cf
    Fq = cq * cf
    mask = (ck == cq) | ((fr[None, :] < Fq) & ((fr[None, :] < S) | (fr[None, :] >= Fq - W)))
    ivs = [[(int(a), int(b)) for a, b in _runs(mask[i])] for i in range(n)]
    return oracle.attend(q, k, v, ivs, scale)


def _runs(row):
    idx = np.flatnonzero(row)
    if idx.size == 0:
        return []
    cuts = np.flatnonzero(np.diff(idx) > 1)
    starts = np.concatenate([[idx[0]], idx[cuts + 1]])
    ends = np.concatenate([idx[cuts] + 1, [idx[-1] + 1]])
    return list(zip(starts, ends))


def test_tiny_rollout_fp32(wmk):
    import torch
    S, W, cf, tpf, H, D, n_chunks = 1, 2, 2, 16, 1, 64, 6
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf, dtype=torch.float32)
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    qs, ks, vs, outs = [], [], [], []
    for c in range(n_chunks):
        say(f"tiny rollout chunk {c}")
        q, k, v = (host((cf * tpf, H, D), "f32", seed=0, chunk=c, kind=t) for t in (synth.Q, synth.K, synth.V))
        out = wmk.chunk_attention(cache, 0, to_dev(q), [(to_dev(k), to_dev(v))])
        ref = oracle.chunk_attention(cm, q, [(k, v)], 1.0 / math.sqrt(D))
        got = from_dev(out)
        compare(got, ref, F32_MAX_ABS, F32_REL_L2, f"chunk {c}")
        cache.append_evict(0, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
        slots, F = cache.slots(0)
        assert slots == cm.slot_map().tolist() and F == cm.F
        kb, vb = cm.slot_buffers()
        valid = oracle.valid_slots(cm.F, S, W)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(cache.k[0, :valid]).view(np.uint32), kb[:valid].view(np.uint32))
        assert np.array_equal(from_dev(cache.v[0, :valid]).view(np.uint32), vb[:valid].view(np.uint32))
        qs.append(q), ks.append(k), vs.append(v), outs.append(got)
    # the whole rollout as one dense masked softmax over the 12-frame sequence
    ref = _dense_rollout_ref(np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), S, W, cf, tpf,
                             1.0 / math.sqrt(D))
    compare(np.concatenate(outs), ref, F32_MAX_ABS, F32_REL_L2, "dense rollout")
    cache.close()


# ----------------------------------------------------------------------------------------------
# cache append / evict, bit-exact
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("S,W,cf,tpf,H,D,n_app,dt", [
    (6, 8, 4, 1508, 12, 128, 7, "bf16"),   # the 832x464 cache
    (2, 3, 5, 7, 3, 64, 5, "bf16"),        # chunk longer than the window
    (0, 4, 3, 5, 2, 128, 6, "f32"),        # no sinks, ring wraps mid-chunk
    (3, 1, 2, 4, 1, 64, 5, "bf16"),        # window of one frame
])
def test_append_evict_bit_exact(wmk, S, W, cf, tpf, H, D, n_app, dt):
    import torch
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    cache = wmk.Cache(num_layers=3, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf, dtype=tdt)
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.uint16 if dt == "bf16" else np.float32)
    for a in range(n_app):
        say(f"append S={S} W={W} cf={cf} tpf={tpf} H={H} D={D} #{a}")
        k = host((cf * tpf, H, D), dt, seed=1, chunk=a, layer=2, step=4, kind=synth.KFIN)
        v = host((cf * tpf, H, D), dt, seed=1, chunk=a, layer=2, step=4, kind=synth.VFIN)
        cache.append_evict(2, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
        torch.cuda.synchronize()
        slots, F = cache.slots(2)
        assert slots == cm.slot_map().tolist() and F == cm.F
        kb, vb = cm.slot_buffers()
        valid = oracle.valid_slots(cm.F, S, W)
        gk, gv = from_dev(cache.k[2, :valid]), from_dev(cache.v[2, :valid])
        assert np.array_equal(gk.view(np.uint16), kb[:valid].view(np.uint16))
        assert np.array_equal(gv.view(np.uint16), vb[:valid].view(np.uint16))
    assert cache.slots(0) == ([-1] * (S + W), 0)
    cache.close()


@pytest.mark.parametrize("seed", range(6))
def test_append_evict_random_sequences_bit_exact(wmk, seed):
    """Seeded random append sequences over a multi-layer cache: random geometry and dtype,
    each append to a random layer with a random frame count (from one frame to more than
    the whole cache holds); after every append the slot maps and the resident slots of
    every layer equal the oracle's bit for bit (layers not appended to stay unchanged)."""
    import torch
    rng = np.random.default_rng(1500 + seed)
    S, W, cf = int(rng.integers(0, 7)), int(rng.integers(1, 11)), int(rng.integers(1, 6))
    tpf, H, D = int(rng.integers(1, 201)), int(rng.integers(1, 5)), int(rng.choice([64, 128]))
    dt = "bf16" if rng.random() < 0.7 else "f32"
    L = int(rng.integers(1, 4))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    cache = wmk.Cache(num_layers=L, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf, dtype=tdt)
    cms = [oracle.CacheModel(S, W, tpf, H, D, dtype=np.uint16 if dt == "bf16" else np.float32) for _ in range(L)]
    view = np.uint16 if dt == "bf16" else np.uint32
    for a in range(8):
        layer, n = int(rng.integers(0, L)), int(rng.integers(1, S + 2 * W + 3))
        say(f"append random seed {seed}: S={S} W={W} tpf={tpf} H={H} D={D} {dt} L={L} #{a} layer {layer} "
            f"frames {n}")
        k = host((n * tpf, H, D), dt, seed=1600 + seed, chunk=a, layer=layer, step=4, kind=synth.KFIN)
        v = host((n * tpf, H, D), dt, seed=1600 + seed, chunk=a, layer=layer, step=4, kind=synth.VFIN)
        cache.append_evict(layer, to_dev(k), to_dev(v), n)
        cms[layer].append(k, v, n)
        torch.cuda.synchronize()
        for l, cm in enumerate(cms):
            slots, F = cache.slots(l)
            assert slots == cm.slot_map().tolist() and F == cm.F, (l, slots, cm.slot_map().tolist())
            valid = oracle.valid_slots(cm.F, S, W)
            if valid:
                kb, vb = cm.slot_buffers()
                assert np.array_equal(from_dev(cache.k[l, :valid]).view(view), kb[:valid].view(view))
                assert np.array_equal(from_dev(cache.v[l, :valid]).view(view), vb[:valid].view(view))
    cache.close()


@pytest.mark.parametrize("S,W,cf,tpf,H,D,L,first,n_layers,dt", [
    (6, 8, 4, 1508, 12, 128, 3, 0, 3, "bf16"),   # the 832x464 geometry, every layer in one call
    (2, 3, 5, 7, 3, 64, 4, 1, 2, "bf16"),        # chunk longer than the window, a middle run of layers
    (0, 4, 3, 5, 2, 128, 3, 0, 2, "f32"),        # no sinks, ring wraps mid-chunk
    (3, 1, 2, 33, 1, 64, 2, 1, 1, "bf16"),       # a run of one layer, window of one frame
])
def test_append_evict_layers_bit_exact(wmk, S, W, cf, tpf, H, D, L, first, n_layers, dt):
    """Multi-layer appends: after every call the slot maps and resident slots of each layer
    of the run equal the oracle's bit for bit, and the layers outside the run stay empty."""
    import torch
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    view = np.uint16 if dt == "bf16" else np.uint32
    cache = wmk.Cache(num_layers=L, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf, dtype=tdt)
    cms = [oracle.CacheModel(S, W, tpf, H, D, dtype=np.uint16 if dt == "bf16" else np.float32) for _ in range(L)]
    for a in range(5):
        say(f"append_layers S={S} W={W} cf={cf} tpf={tpf} H={H} D={D} {dt} layers [{first}, {first + n_layers}) "
            f"of {L} #{a}")
        k = host((n_layers, cf * tpf, H, D), dt, seed=1700, chunk=a, step=4, kind=synth.KFIN)
        v = host((n_layers, cf * tpf, H, D), dt, seed=1700, chunk=a, step=4, kind=synth.VFIN)
        cache.append_evict_layers(first, to_dev(k), to_dev(v), cf)
        for i in range(n_layers):
            cms[first + i].append(k[i], v[i], cf)
        torch.cuda.synchronize()
        for l, cm in enumerate(cms):
            slots, F = cache.slots(l)
            assert slots == cm.slot_map().tolist() and F == cm.F, (l, slots)
            valid = oracle.valid_slots(cm.F, S, W)
            if valid:
                kb, vb = cm.slot_buffers()
                assert np.array_equal(from_dev(cache.k[l, :valid]).view(view), kb[:valid].view(view))
                assert np.array_equal(from_dev(cache.v[l, :valid]).view(view), vb[:valid].view(view))
    cache.close()


@pytest.mark.parametrize("seed", range(4))
def test_append_evict_layers_random_runs_bit_exact(wmk, seed):
    """Seeded random mixes of multi-layer and single-layer appends on a multi-layer cache:
    single-layer appends put layers out of step; a multi-layer run over layers holding
    different frame counts is refused (WMK_ERR_RANGE, nothing changes); every accepted
    call leaves every layer's slot map and slots equal to the oracle's bit for bit."""
    import torch
    rng = np.random.default_rng(1800 + seed)
    S, W, cf = int(rng.integers(0, 5)), int(rng.integers(1, 7)), int(rng.integers(1, 4))
    tpf, H, D, L = int(rng.integers(1, 120)), int(rng.integers(1, 4)), int(rng.choice([64, 128])), int(rng.integers(2, 6))
    cache = wmk.Cache(num_layers=L, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cms = [oracle.CacheModel(S, W, tpf, H, D) for _ in range(L)]
    refused = 0
    for a in range(12):
        first = 0 if rng.random() < 0.4 else int(rng.integers(0, L))
        n_layers = L - first if rng.random() < 0.5 else int(rng.integers(1, L - first + 1))
        n = int(rng.integers(1, S + 2 * W + 3))
        k = host((n_layers, n * tpf, H, D), seed=1900 + seed, chunk=a, step=4, kind=synth.KFIN)
        v = host((n_layers, n * tpf, H, D), seed=1900 + seed, chunk=a, step=4, kind=synth.VFIN)
        in_step = len({cms[first + i].F for i in range(n_layers)}) == 1
        say(f"append_layers random seed {seed}: S={S} W={W} tpf={tpf} H={H} D={D} L={L} #{a} layers "
            f"[{first}, {first + n_layers}) frames {n} in step {in_step}")
        if rng.random() < 0.2:    # a single-layer append instead: puts that layer out of step
            cache.append_evict(first, to_dev(k[0]), to_dev(v[0]), n)
            cms[first].append(k[0], v[0], n)
        elif in_step:
            cache.append_evict_layers(first, to_dev(k), to_dev(v), n)
            for i in range(n_layers):
                cms[first + i].append(k[i], v[i], n)
        else:
            with pytest.raises(wmk.WmkError) as e:
                cache.append_evict_layers(first, to_dev(k), to_dev(v), n)
            assert e.value.status == wmk.WMK_ERR_RANGE
            refused += 1
        torch.cuda.synchronize()
        for l, cm in enumerate(cms):
            slots, F = cache.slots(l)
            assert slots == cm.slot_map().tolist() and F == cm.F, (l, slots)
            valid = oracle.valid_slots(cm.F, S, W)
            if valid:
                kb, vb = cm.slot_buffers()
                assert np.array_equal(from_dev(cache.k[l, :valid]).view(np.uint16), kb[:valid].view(np.uint16))
                assert np.array_equal(from_dev(cache.v[l, :valid]).view(np.uint16), vb[:valid].view(np.uint16))
    say(f"refused runs: {refused}")
    cache.close()


# ----------------------------------------------------------------------------------------------
# chunk attention, small shapes: every row
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", [
    dict(S=2, W=3, cf=2, tpf=37, H=3, D=128, warm=4, nq=None, extra=0),   # ragged q and kv tiles
    dict(S=1, W=2, cf=1, tpf=300, H=2, D=64, warm=3, nq=None, extra=0),   # head_dim 64
    dict(S=0, W=2, cf=1, tpf=50, H=2, D=128, warm=0, nq=1, extra=0),      # empty cache, one query
    dict(S=3, W=4, cf=2, tpf=64, H=1, D=128, warm=6, nq=130, extra=3),    # 4 segments (chunk + 3 extra)
    dict(S=1, W=1, cf=1, tpf=129, H=4, D=128, warm=2, nq=257, extra=1),
    # more than 32 key tiles (2757 keys): the 8-wave kernel shape; the cases above walk at
    # most 32 tiles and run the 4-wave shape (128-row q-tiles, two workgroups per CU)
    dict(S=2, W=5, cf=2, tpf=300, H=2, D=128, warm=6, nq=None, extra=1),
])
def test_chunk_attention_small_all_rows(wmk, case):
    import torch
    S, W, cf, tpf, H, D = (case[x] for x in ("S", "W", "cf", "tpf", "H", "D"))
    nq = case["nq"] or cf * tpf
    cache = wmk.Cache(num_layers=2, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for a in range(case["warm"]):
        k = host((cf * tpf, H, D), seed=2, chunk=a, layer=1, kind=synth.KFIN)
        v = host((cf * tpf, H, D), seed=2, chunk=a, layer=1, kind=synth.VFIN)
        cache.append_evict(1, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
    q = host((nq, H, D), seed=3, kind=synth.Q)
    segs = []
    for e in range(1 + case["extra"]):
        n = nq if e == 0 else 17 + 40 * e
        segs.append((host((n, H, D), seed=3, chunk=e, kind=synth.K), host((n, H, D), seed=3, chunk=e, kind=synth.V)))
    say(f"chunk attention small {case}")
    for use_ws in (False, True):
        out = wmk.chunk_attention(cache, 1, to_dev(q), [(to_dev(k), to_dev(v)) for k, v in segs],
                                  use_workspace=use_ws)
        torch.cuda.synchronize()
        ref = oracle.chunk_attention(cm, q, segs, 1.0 / math.sqrt(D))
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"all rows ws={use_ws}")
    cache.close()


def _random_case(seed):
    """A seeded random chunk-attention case: cache geometry, warm-up, query count and extra
    segments drawn so that calls land on both kernel shapes (up to and beyond 32 key tiles),
    with ragged query and key tiles, empty and partly filled caches, 64- and 128-dim heads."""
    r = np.random.default_rng(1000 + seed)
    D = int(r.choice([64, 128], p=[0.25, 0.75]))
    S, W, cf = int(r.integers(0, 4)), int(r.integers(1, 6)), int(r.integers(1, 4))
    tpf = int(r.integers(17, 400))
    H = int(r.integers(1, 4))
    warm = int(r.integers(0, 8))
    nq = int(r.integers(1, 700))
    extra = [int(r.integers(1, 300)) for _ in range(int(r.integers(0, 4)))]
    return dict(S=S, W=W, cf=cf, tpf=tpf, H=H, D=D, warm=warm, nq=nq, extra=extra, seed=seed)


@pytest.mark.parametrize("seed", range(12))
def test_chunk_attention_random_shapes_all_rows(wmk, seed):
    """Every row of a dozen seeded random calls (see _random_case) against the oracle, with
    and without the split-tail workspace."""
    import torch
    case = _random_case(seed)
    S, W, cf, tpf, H, D = (case[x] for x in ("S", "W", "cf", "tpf", "H", "D"))
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for a in range(case["warm"]):
        k = host((cf * tpf, H, D), seed=seed, chunk=a, layer=3, kind=synth.KFIN)
        v = host((cf * tpf, H, D), seed=seed, chunk=a, layer=3, kind=synth.VFIN)
        cache.append_evict(0, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
    nq = case["nq"]
    q = host((nq, H, D), seed=seed, layer=4, kind=synth.Q)
    segs = [(host((nq, H, D), seed=seed, layer=4, kind=synth.K), host((nq, H, D), seed=seed, layer=4, kind=synth.V))]
    for e, n in enumerate(case["extra"]):
        segs.append((host((n, H, D), seed=seed, chunk=e + 1, layer=5, kind=synth.KLOC),
                     host((n, H, D), seed=seed, chunk=e + 1, layer=5, kind=synth.VLOC)))
    keys = oracle.valid_slots(cm.F, S, W) * tpf + sum(k.shape[0] for k, _ in segs)
    say(f"random case {case}: {keys} keys")
    ref = oracle.chunk_attention(cm, q, segs, 1.0 / math.sqrt(D))
    for use_ws in (False, True):
        out = wmk.chunk_attention(cache, 0, to_dev(q), [(to_dev(k), to_dev(v)) for k, v in segs],
                                  use_workspace=use_ws)
        torch.cuda.synchronize()
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"seed {seed} all rows ws={use_ws}")
    cache.close()


def test_chunk_attention_no_keys_gives_zeros(wmk):
    import torch
    cache = wmk.Cache(num_layers=1, num_heads=2, head_dim=128, tokens_per_frame=8, sink_frames=1, window_frames=1,
                      chunk_frames=1)
    q = to_dev(host((200, 2, 128), seed=4))
    out = torch.full_like(q, 7.0)
    wmk.chunk_attention(cache, 0, q, [], out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    cache.close()


def test_scale_and_sharp_softmax(wmk):
    """q x 8 sharpens the softmax so that max-abs errors are informative."""
    import torch
    H, D, n, nk = 2, 128, 300, 1000
    q = as_f32(host((n, H, D), seed=5)) * 8
    qb = synth.f32_to_bf16_bits(q).reshape(n, H, D)
    k, v = host((nk, H, D), seed=5, kind=synth.K), host((nk, H, D), seed=5, kind=synth.V)
    for scale in (1 / math.sqrt(D), 0.5 / math.sqrt(D)):
        out = wmk.chunk_attention(None, 0, to_dev(qb), [(to_dev(k), to_dev(v))], scale=scale)
        torch.cuda.synchronize()
        ref = oracle.chunk_attention(None, qb, [(k, v)], scale)
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"sharp scale={scale:.4f}")


# ----------------------------------------------------------------------------------------------
# the 18-slot 832x464 step: Q 6032, KV 27144, 12 heads x 128, bf16
# ----------------------------------------------------------------------------------------------

def _warm_cache(wmk, cm, cache, layer, n_appends, cf, tpf, H, D, seed):
    for a in range(n_appends):
        k = host((cf * tpf, H, D), seed=seed, chunk=a, layer=layer, step=4, kind=synth.KFIN)
        v = host((cf * tpf, H, D), seed=seed, chunk=a, layer=layer, step=4, kind=synth.VFIN)
        cache.append_evict(layer, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)


def test_chunk_attention_832x464_18_slots(wmk):
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    say("832x464: warming the cache with 4 chunks")
    _warm_cache(wmk, cm, cache, 0, 4, cf, tpf, H, D, seed=0)
    slots, F = cache.slots(0)
    assert F == 16 and sum(s >= 0 for s in slots) == 14
    q = host((cf * tpf, H, D), seed=0, chunk=4, kind=synth.Q)
    k = host((cf * tpf, H, D), seed=0, chunk=4, kind=synth.K)
    v = host((cf * tpf, H, D), seed=0, chunk=4, kind=synth.V)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    rows = sample_rows(cf * tpf, np.random.default_rng(0), k=40)
    say(f"832x464: oracle on {len(rows)} rows")
    ref = oracle.chunk_attention(cm, q, [(k, v)], 1 / math.sqrt(D), rows=rows)
    outs = {}
    for use_ws in (False, True):
        say(f"832x464: chunk_attention workspace={use_ws}")
        out = wmk.chunk_attention(cache, 0, qd, [(kd, vd)], use_workspace=use_ws)
        torch.cuda.synchronize()
        outs[use_ws] = from_dev(out)
        compare(outs[use_ws][rows], ref, BF16_MAX_ABS, BF16_REL_L2, f"sampled rows ws={use_ws}")
    # split and unsplit schedules agree everywhere (different summation order only)
    compare(outs[True], as_f32(outs[False]), 4e-3, 2e-3, "split vs unsplit, all rows")
    # every row of two heads against the oracle: head 0 (whole units only) and head 11, whose
    # 256-row units run as the split tail (pieces plus the merge kernel) when the workspace is on
    heads = [0, 11]
    kc, vc = cm.logical_kv()
    ka = np.ascontiguousarray(np.concatenate([kc, k])[:, heads])
    va = np.ascontiguousarray(np.concatenate([vc, v])[:, heads])
    nq, nk = cf * tpf, ka.shape[0]
    assert nk == 18 * tpf
    say(f"832x464: oracle on all {nq} rows of heads {heads}")
    ref_h = oracle.attend(np.ascontiguousarray(q[:, heads]), ka, va, [[(0, nk)]] * nq, 1 / math.sqrt(D))
    for use_ws in (False, True):
        compare(outs[use_ws][:, heads], ref_h, BF16_MAX_ABS, BF16_REL_L2, f"all rows of heads {heads} ws={use_ws}")
    cache.close()


# ----------------------------------------------------------------------------------------------
# MoBA
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("tpf,frames,cf,H,D,bidir", [
    (4, 6, 2, 2, 128, 1),      # many chunks inside one 128-row tile
    (40, 7, 3, 2, 128, 1),     # last chunk of each part shorter
    (70, 5, 2, 1, 64, 0),      # no bidirectional block, head_dim 64
    (130, 6, 3, 3, 128, 1),    # chunk boundaries inside tiles
])
def test_moba_small_all_rows(wmk, tpf, frames, cf, H, D, bidir):
    import torch
    n = (2 + bidir) * frames * tpf
    q, k, v = (host((n, H, D), seed=8, kind=t) for t in (synth.Q, synth.K, synth.V))
    say(f"moba small tpf={tpf} frames={frames} cf={cf} H={H} D={D} bidir={bidir}")
    out = wmk.moba_attention(to_dev(q), to_dev(k), to_dev(v), tokens_per_frame=tpf, frames=frames, chunk_frames=cf,
                             bidir_block=bidir)
    torch.cuda.synchronize()
    ref = oracle.moba_attention(q, k, v, tpf, frames, cf, bidir, 1 / math.sqrt(D))
    compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, "all rows")


@pytest.mark.parametrize("seed", range(8))
def test_moba_random_shapes_all_rows(wmk, seed):
    """Every row of seeded random MoBA forward calls against the oracle: tokens per frame,
    frame and chunk counts (a partial last chunk included), the bidirectional block on or
    off, heads, head_dim 64 or 128, bf16 or fp32."""
    import torch
    r = np.random.default_rng(2100 + seed)
    tpf, frames = int(r.integers(3, 151)), int(r.integers(1, 9))
    cf, bidir, H = int(r.integers(1, frames + 1)), int(r.integers(0, 2)), int(r.integers(1, 4))
    D, dt = int(r.choice([64, 128])), ("bf16" if r.random() < 0.75 else "f32")
    n = (2 + bidir) * frames * tpf
    q, k, v = (host((n, H, D), dt, seed=2200 + seed, kind=t) for t in (synth.Q, synth.K, synth.V))
    say(f"moba random seed {seed}: tpf={tpf} frames={frames} cf={cf} bidir={bidir} H={H} D={D} {dt} n={n}")
    out = wmk.moba_attention(to_dev(q), to_dev(k), to_dev(v), tokens_per_frame=tpf, frames=frames, chunk_frames=cf,
                             bidir_block=bidir)
    torch.cuda.synchronize()
    ref = oracle.moba_attention(q, k, v, tpf, frames, cf, bidir, 1 / math.sqrt(D))
    if dt == "bf16":
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"seed {seed} all rows")
    else:
        compare(from_dev(out), ref, F32_MAX_ABS, F32_REL_L2, f"seed {seed} fp32 all rows")


def test_moba_fp32_small(wmk):
    import torch
    tpf, frames, cf, H, D = 6, 4, 2, 2, 64
    n = 3 * frames * tpf
    q, k, v = (host((n, H, D), "f32", seed=9, kind=t) for t in (synth.Q, synth.K, synth.V))
    out = wmk.moba_attention(to_dev(q), to_dev(k), to_dev(v), tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
    torch.cuda.synchronize()
    ref = oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 1 / math.sqrt(D))
    compare(from_dev(out), ref, F32_MAX_ABS, F32_REL_L2, "fp32 all rows")


def test_moba_noisy_rows_match_chunk_attention(wmk):
    """The two kernels cross-check: noisy chunk i of MoBA = chunk attention over a cache
    holding the clean chunks < i (no eviction) with noisy chunk i as the current chunk."""
    import torch
    tpf, frames, cf, H, D = 100, 6, 2, 2, 128
    L, cl = frames * tpf, cf * tpf
    n = 3 * L
    q, k, v = (host((n, H, D), seed=10, kind=t) for t in (synth.Q, synth.K, synth.V))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    moba = wmk.moba_attention(qd, kd, vd, tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
    for c in range(frames // cf):
        cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=0,
                          window_frames=frames, chunk_frames=cf)
        if c > 0:
            cache.append_evict(0, kd[:c * cl], vd[:c * cl], c * cf)
        rows = slice(L + c * cl, L + (c + 1) * cl)
        out = wmk.chunk_attention(cache, 0, qd[rows], [(kd[rows], vd[rows])])
        torch.cuda.synchronize()
        compare(from_dev(out), as_f32(from_dev(moba[rows])), 8e-3, 4e-3, f"noisy chunk {c}")
        cache.close()


def test_moba_training_sequence_full_size(wmk):
    """21 clean + 21 noisy + 21 bidirectional frames of 1560 tokens, chunks of 3, 12 x 128."""
    import torch
    tpf, frames, cf, H, D = 1560, 21, 3, 12, 128
    L, cl = frames * tpf, cf * tpf
    n = 3 * L
    say("moba full size: drawing inputs")
    q, k, v = (host((n, H, D), seed=0, kind=t) for t in (synth.Q, synth.K, synth.V))
    say("moba full size: kernel")
    out = wmk.moba_attention(to_dev(q), to_dev(k), to_dev(v), tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
    torch.cuda.synchronize()
    got = from_dev(out)
    rng = np.random.default_rng(1)
    rows = {0, L - 1, L, 2 * L - 1, 2 * L, n - 1}
    for part in range(3):
        for kk in (1, 3, 6):
            b = part * L + kk * cl
            rows |= {b - 1, b, b + 1}
    for b in (L, 2 * L):              # q-tiles straddling the part boundaries
        rows |= {((b // 128) * 128) + 3, b + 5}
    rows |= set(int(x) for x in rng.choice(n, 12, replace=False))
    rows = np.array(sorted(rows))
    say(f"moba full size: oracle on {len(rows)} rows")
    ref = oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 1 / math.sqrt(D), rows=rows)
    compare(got[rows], ref, BF16_MAX_ABS, BF16_REL_L2, "sampled rows")
    # every row of one head (rows in runs of equal mask intervals, dense BLAS blocks)
    say("moba full size: oracle on every row of head 5")
    ref5 = oracle.attention_by_runs(q, k, v, lambda i: oracle.moba_row_intervals(i, tpf, frames, cf), 1 / math.sqrt(D),
                                    heads=[5])
    compare(got[:, [5]], ref5, BF16_MAX_ABS, BF16_REL_L2, "every row of head 5")


# ----------------------------------------------------------------------------------------------
# 720p step: 3600 tokens per frame, 24 heads, 18 slots; chunk-causal cross-attention
# ----------------------------------------------------------------------------------------------

def test_720p_self_and_cross_attention(wmk):
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 3600, 24, 128
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    say("720p: warming the cache")
    _warm_cache(wmk, cm, cache, 0, 4, cf, tpf, H, D, seed=1)
    nq = cf * tpf
    q = host((nq, H, D), seed=1, chunk=4, kind=synth.Q)
    k = host((nq, H, D), seed=1, chunk=4, kind=synth.K)
    v = host((nq, H, D), seed=1, chunk=4, kind=synth.V)
    qd = to_dev(q)
    say("720p: self-attention")
    out = wmk.chunk_attention(cache, 0, qd, [(to_dev(k), to_dev(v))])
    torch.cuda.synchronize()
    rows = sample_rows(nq, np.random.default_rng(2), k=8)
    say(f"720p: oracle on {len(rows)} rows")
    ref = oracle.chunk_attention(cm, q, [(k, v)], 1 / math.sqrt(D), rows=rows)
    compare(from_dev(out)[rows], ref, BF16_MAX_ABS, BF16_REL_L2, "self, sampled rows")
    # every row of head 13 over all 64 800 keys (the head's units include split-tail pieces)
    say("720p: oracle on every row of head 13")
    kc, vc = cm.logical_kv()
    kall, vall = np.concatenate([kc, k]), np.concatenate([vc, v])
    ref13 = oracle.attention_by_runs(q, kall, vall, lambda i: [(0, kall.shape[0])], 1 / math.sqrt(D), heads=[13])
    compare(from_dev(out)[:, [13]], ref13, BF16_MAX_ABS, BF16_REL_L2, "self, every row of head 13")
    cache.close()

    # cross-attention: chunk 2 reads the shared environment prompt and its own local prompt
    ke, ve = host((512, H, D), seed=1, kind=synth.KENV), host((512, H, D), seed=1, kind=synth.VENV)
    kl = [host((512, H, D), seed=1, chunk=j, kind=synth.KLOC) for j in range(4)]
    vl = [host((512, H, D), seed=1, chunk=j, kind=synth.VLOC) for j in range(4)]
    say("720p: cross-attention")
    out = wmk.chunk_attention(None, 0, qd, [(to_dev(ke), to_dev(ve)), (to_dev(kl[2]), to_dev(vl[2]))])
    torch.cuda.synchronize()
    rows = sample_rows(nq, np.random.default_rng(3), k=64)
    ref = oracle.cross_attention(q, 2, ke, ve, kl, vl, 1 / math.sqrt(D), rows=rows)
    compare(from_dev(out)[rows], ref, BF16_MAX_ABS, BF16_REL_L2, "cross, sampled rows")
    kx, vx = np.concatenate([ke] + kl), np.concatenate([ve] + vl)
    ivx = oracle.cross_row_intervals(2, 512, 512)
    refx = oracle.attention_by_runs(q, kx, vx, lambda i: ivx, 1 / math.sqrt(D), heads=[0, 23])
    compare(from_dev(out)[:, [0, 23]], refx, BF16_MAX_ABS, BF16_REL_L2, "cross, every row of heads 0 and 23")


# ----------------------------------------------------------------------------------------------
# per-key softmax weights: with V[j] = e_(j - base) the output row is the weight vector over
# keys base .. base+127, so every allowed and every masked key is checked on its own
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("tpf,frames,cf", [(40, 7, 3), (43, 6, 2)])
def test_moba_per_key_weights(wmk, tpf, frames, cf):
    import torch
    H, D = 1, 128
    n = 3 * frames * tpf
    q, k = (host((n, H, D), seed=8, kind=t) for t in (synth.Q, synth.K))
    rows = np.arange(n)
    for base in range(0, n, 128):
        v = np.zeros((n, H, D), np.float32)
        for j in range(base, min(n, base + 128)):
            v[j, 0, j - base] = 1.0
        vb = synth.f32_to_bf16_bits(v).reshape(n, H, D)
        out = wmk.moba_attention(to_dev(q), to_dev(k), to_dev(vb), tokens_per_frame=tpf, frames=frames,
                                 chunk_frames=cf)
        torch.cuda.synchronize()
        got = as_f32(from_dev(out))[:, 0, :]
        ivs = [oracle.moba_row_intervals(int(i), tpf, frames, cf) for i in rows]
        _, p = oracle.attend(q, k, k, ivs, 1 / math.sqrt(D), want_probs=True)
        ref = np.zeros((n, 128))
        w = min(n, base + 128) - base
        ref[:, :w] = p[:, 0, base:base + w]
        err = np.abs(got - ref)
        # bf16 output of a weight w: |error| <= 2^-8 w + a few ulps of fp32 accumulation
        bad = np.argwhere(err > 8e-3 * np.maximum(ref, 1e-3) + 2e-4)
        say(f"  keys {base}..{base + w - 1}: max weight error {err.max():.2e}, {len(bad)} bad (row, key) pairs")
        assert len(bad) == 0, f"first bad (row, key): {[(int(r), int(c) + base) for r, c in bad[:5]]}"


# ----------------------------------------------------------------------------------------------
# the binding's scratch is per (device, stream): two streams running split-tail calls at once
# ----------------------------------------------------------------------------------------------

def test_two_streams_split_tail_concurrently(wmk):
    """Chunk attention with the split tail on two streams at once (different queries, one
    cache): each stream gets its own scratch from the binding, so both outputs equal the
    same calls made one after the other."""
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    for c in range(4):
        cache.append_evict(0, dev_fill((cf * tpf, H, D), seed=90, chunk=c, kind=synth.KFIN),
                           dev_fill((cf * tpf, H, D), seed=90, chunk=c, kind=synth.VFIN), cf)
    qs = [dev_fill((cf * tpf, H, D), seed=91 + i, kind=synth.Q) for i in range(2)]
    k, v = dev_fill((cf * tpf, H, D), seed=93, kind=synth.K), dev_fill((cf * tpf, H, D), seed=93, kind=synth.V)
    torch.cuda.synchronize()
    say("two streams: serial references")
    refs = [wmk.chunk_attention(cache, 0, q, [(k, v)]).clone() for q in qs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(qs[0]) for _ in range(2)]
    say("two streams: concurrent calls")
    for rep in range(3):
        for i in range(2):
            streams[i].wait_stream(torch.cuda.current_stream())
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                wmk.chunk_attention(cache, 0, qs[i], [(k, v)], out=outs[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i].view(torch.int16), refs[i].view(torch.int16)), (rep, i)
    cache.close()
