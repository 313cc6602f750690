"""GPU parity of chunk attention with the FP8-quantized QK^T through the C ABI:
the e4m3 codes and block scales of Q and K (read back from the workspace)
bit for bit against the oracle's quantizer, the outputs against the oracle's
quantized attention (bf16 bounds) on small ragged shapes and sampled rows at
832x464 and 720p, the quantization error against the exact attention (the looser
bound of the quantized path), and bit-identical outputs from two caches that hold
the same frames with their rings wrapped at different slots."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import BF16_MAX_ABS, BF16_REL_L2, compare, dev_fill, from_dev, host, sample_rows, say, to_dev
from tests.test_oracle import QK8_MAX_ABS_VS_EXACT, QK8_REL_L2_VS_EXACT

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


def _a256(x):
    return (x + 255) // 256 * 256


def _regions(ws, H, nq, nk):
    """Split a workspace read back to the host into its four regions (include/wmk.h)."""
    kt, qb = -(-nk // 64), -(-nq // 32)
    b = from_dev(ws).view(np.uint8)
    o = 0
    k8 = b[o:o + kt * H * 8192].reshape(kt, H, 64, 128)
    o += _a256(kt * H * 8192)
    ks = b[o:o + kt * H * 4].view(np.float32).reshape(kt, H)
    o += _a256(kt * H * 4)
    q8 = b[o:o + qb * H * 4096].reshape(qb, H, 32, 128)
    o += _a256(qb * H * 4096)
    qs = b[o:o + qb * H * 4].view(np.float32).reshape(qb, H)
    # undo the chunk permutation of the key tiles: chunk c of row r sits at c ^ ((r // 2) % 8)
    chunks = k8.reshape(kt, H, 64, 8, 16)
    logical = np.empty_like(chunks)
    for r in range(64):
        for c in range(8):
            logical[:, :, r, c] = chunks[:, :, r, c ^ ((r // 2) % 8)]
    return logical.reshape(kt, H, 64, 128), ks, q8, qs


def _filled(wmk, S, W, cf, tpf, H, D, n_chunks, seed):
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for c in range(n_chunks):
        k = host((cf * tpf, H, D), seed=seed, chunk=c, step=4, kind=synth.KFIN)
        v = host((cf * tpf, H, D), seed=seed, chunk=c, step=4, kind=synth.VFIN)
        cache.append_evict(0, to_dev(k), to_dev(v), cf)
        cm.append(k, v, cf)
    return cache, cm


def _check_codes(ws, cm, q, segments, H):
    k_seq, _ = oracle.qk8_key_sequence(cm, segments)
    k8, ks, q8, qs = _regions(ws, H, q.shape[0], k_seq.shape[0])
    kc, kss = oracle.quantize_e4m3_blocks(k_seq, 64)
    qc, qss = oracle.quantize_e4m3_blocks(q, 32)
    np.testing.assert_array_equal(ks.view(np.uint32), kss.view(np.uint32))
    np.testing.assert_array_equal(qs.view(np.uint32), qss.view(np.uint32))
    np.testing.assert_array_equal(k8, kc)
    np.testing.assert_array_equal(q8, qc)


@pytest.mark.parametrize("S,W,cf,tpf,n_chunks,nseg", [
    (2, 3, 2, 37, 5, 1),     # ring wrapped, ragged frames: key tiles straddle slots and the segment
    (1, 2, 1, 100, 3, 2),    # two segments after the cache
    (0, 1, 1, 50, 0, 3),     # no cache frames yet: segments only
])
def test_qk8_small_codes_and_all_rows(wmk, S, W, cf, tpf, n_chunks, nseg):
    import torch
    H, D = 2, 128
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, n_chunks, seed=41)
    nq = cf * tpf + 7
    q = host((nq, H, D), seed=42, kind=synth.Q)
    segs = [(host((33 + 40 * i, H, D), seed=43 + i, kind=synth.K), host((33 + 40 * i, H, D), seed=43 + i, kind=synth.V))
            for i in range(nseg)]
    nk = oracle.valid_slots(cm.F, S, W) * tpf + sum(k.shape[0] for k, _ in segs)
    ws = torch.zeros(wmk.qk8_workspace_bytes(H, nq, nk), dtype=torch.uint8, device="cuda")
    say(f"qk8 small S={S} W={W} tpf={tpf} chunks={n_chunks} segments={nseg} nq={nq} nk={nk}")
    out = wmk.chunk_attention_qk8(cache, 0, to_dev(q), [(to_dev(k), to_dev(v)) for k, v in segs], ws=ws)
    torch.cuda.synchronize()
    _check_codes(ws, cm, q, segs, H)
    ref = oracle.chunk_attention_qk8(cm, q, segs, 1 / math.sqrt(D))
    compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, "all rows")
    cache.close()


@pytest.mark.parametrize("seed", range(6))
def test_qk8_random_shapes_codes_and_all_rows(wmk, seed):
    """Seeded random FP8 calls: random ring state, frame size, query count and 1-3
    segments of random length; the quantized codes and scales bit for bit, every row
    against the quantized oracle."""
    import torch
    rng = np.random.default_rng(1100 + seed)
    S, W, cf = int(rng.integers(0, 5)), int(rng.integers(1, 7)), int(rng.integers(1, 4))
    tpf, n_chunks, nseg = int(rng.integers(8, 201)), int(rng.integers(0, 10)), int(rng.integers(1, 4))
    H, D = int(rng.integers(1, 4)), 128
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, n_chunks, seed=1200 + seed)
    nq = int(rng.integers(1, 1001))
    q = host((nq, H, D), seed=1300 + seed, kind=synth.Q)
    lens = [int(x) for x in rng.integers(1, 151, size=nseg)]
    segs = [(host((n, H, D), seed=1400 + 10 * seed + i, kind=synth.K),
             host((n, H, D), seed=1400 + 10 * seed + i, kind=synth.V)) for i, n in enumerate(lens)]
    nk = oracle.valid_slots(cm.F, S, W) * tpf + sum(lens)
    ws = torch.zeros(wmk.qk8_workspace_bytes(H, nq, nk), dtype=torch.uint8, device="cuda")
    say(f"qk8 random seed {seed}: S={S} W={W} cf={cf} tpf={tpf} chunks={n_chunks} H={H} nq={nq} "
        f"segments={lens} nk={nk}")
    out = wmk.chunk_attention_qk8(cache, 0, to_dev(q), [(to_dev(k), to_dev(v)) for k, v in segs], ws=ws)
    torch.cuda.synchronize()
    _check_codes(ws, cm, q, segs, H)
    ref = oracle.chunk_attention_qk8(cm, q, segs, 1 / math.sqrt(D))
    compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"seed {seed} all rows")
    cache.close()


def test_qk8_832x464(wmk):
    """Warm 832x464 cache (14 resident frames) + the 6032-token chunk, split tail on:
    codes of every block bit for bit, sampled rows against the quantized oracle and
    against the exact attention."""
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, 5, seed=44)
    nq = cf * tpf
    q, k, v = (host((nq, H, D), seed=45, kind=t) for t in (synth.Q, synth.K, synth.V))
    nk = 14 * tpf + nq
    ws = torch.zeros(wmk.qk8_workspace_bytes(H, nq, nk), dtype=torch.uint8, device="cuda")
    say("qk8 832x464")
    out = wmk.chunk_attention_qk8(cache, 0, to_dev(q), [(to_dev(k), to_dev(v))], ws=ws)
    torch.cuda.synchronize()
    _check_codes(ws, cm, q, [(k, v)], H)
    rows = sample_rows(nq, np.random.default_rng(9), k=24, tile=256)
    got = from_dev(out)[rows]
    compare(got, oracle.chunk_attention_qk8(cm, q, [(k, v)], 1 / math.sqrt(D), rows=rows), BF16_MAX_ABS,
            BF16_REL_L2, f"{len(rows)} rows vs quantized oracle")
    compare(got, oracle.chunk_attention(cm, q, [(k, v)], 1 / math.sqrt(D), rows=rows), QK8_MAX_ABS_VS_EXACT,
            QK8_REL_L2_VS_EXACT, f"{len(rows)} rows vs exact attention")
    cache.close()


def test_qk8_720p_sampled_heads(wmk):
    """The 720p step (tpf 3600, 24 heads, 14 resident frames + the 14 400-token chunk:
    64 800 keys) through the FP8 path.  Quantization and attention are per head, so the
    oracle works on three heads: their codes and scales bit for bit, and sampled rows
    against the quantized oracle and the exact attention."""
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 3600, 24, 128
    heads = [0, 13, 23]
    cache, cm = _filled(wmk, S, W, cf, tpf, H, D, 5, seed=46)
    nq = cf * tpf
    q, k, v = (host((nq, H, D), seed=47, kind=t) for t in (synth.Q, synth.K, synth.V))
    nk = 14 * tpf + nq
    ws = torch.zeros(wmk.qk8_workspace_bytes(H, nq, nk), dtype=torch.uint8, device="cuda")
    say("qk8 720p")
    out = wmk.chunk_attention_qk8(cache, 0, to_dev(q), [(to_dev(k), to_dev(v))], ws=ws)
    torch.cuda.synchronize()
    k_seq, v_seq = oracle.qk8_key_sequence(cm, [(k, v)])
    assert k_seq.shape[0] == nk
    k8, ks, q8, qs = _regions(ws, H, nq, nk)
    q32 = oracle.widen(q)[:, heads]
    kc, kss = oracle.quantize_e4m3_blocks(k_seq[:, heads], 64)
    qc, qss = oracle.quantize_e4m3_blocks(q32, 32)
    np.testing.assert_array_equal(ks[:, heads].view(np.uint32), kss.view(np.uint32))
    np.testing.assert_array_equal(qs[:, heads].view(np.uint32), qss.view(np.uint32))
    np.testing.assert_array_equal(k8[:, heads], kc)
    np.testing.assert_array_equal(q8[:, heads], qc)
    rows = sample_rows(nq, np.random.default_rng(10), k=12, tile=256)
    got = from_dev(out)[rows][:, heads]
    qd = oracle.dequantize_e4m3_blocks(qc, qss, nq)[rows]
    kd = oracle.dequantize_e4m3_blocks(kc, kss, nk)
    scale = 1 / math.sqrt(D)
    compare(got, oracle.attend_dense_f64(qd, kd, v_seq[:, heads], scale), BF16_MAX_ABS, BF16_REL_L2,
            f"{len(rows)} rows x {len(heads)} heads vs quantized oracle")
    exact = oracle.attend_dense_f64(q32[rows], k_seq[:, heads], v_seq[:, heads], scale)
    compare(got, exact, QK8_MAX_ABS_VS_EXACT, QK8_REL_L2_VS_EXACT, f"{len(rows)} rows vs exact attention")
    cache.close()


def test_qk8_default_workspace_repeats_bit_exactly(wmk):
    """Two calls with the binding's shared workspace (quantized operands rewritten each
    call) give identical outputs, and a call on other inputs in between does not leak."""
    import torch
    H, D, tpf = 12, 128, 1508
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=6, window_frames=8,
                      chunk_frames=4)
    for c in range(3):
        cache.append_evict(0, dev_fill((4 * tpf, H, D), seed=46, chunk=c, kind=synth.KFIN),
                           dev_fill((4 * tpf, H, D), seed=46, chunk=c, kind=synth.VFIN), 4)
    q, k, v = (dev_fill((4 * tpf, H, D), seed=47, kind=t) for t in (synth.Q, synth.K, synth.V))
    say("qk8 repeat")
    a = wmk.chunk_attention_qk8(cache, 0, q, [(k, v)]).clone()
    wmk.chunk_attention_qk8(None, 0, q[:1000], [(k[:500] * 2, v[:500])])
    b = wmk.chunk_attention_qk8(cache, 0, q, [(k, v)])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    cache.close()


def test_qk8_same_frames_at_two_ring_phases_bit_identical(wmk):
    """The 832x464 cache filled two ways so that it holds the same frame contents -- sinks
    from chunks 0 and 1, the window from chunks 3 and 4 -- with the ring wrapped at different
    slots (20 frames appended against 24): the FP8 scale blocks follow the time-ordered key
    sequence, so the two calls quantize the same blocks and give bit-identical outputs,
    which also equal the quantized oracle within the bf16 bounds."""
    import torch
    S, W, cf, tpf, H, D = 6, 8, 4, 1508, 12, 128
    fin = [(host((cf * tpf, H, D), seed=48, chunk=c, step=4, kind=synth.KFIN),
            host((cf * tpf, H, D), seed=48, chunk=c, step=4, kind=synth.VFIN)) for c in range(5)]
    caches, models = [], []
    for order in ((0, 1, 2, 3, 4), (0, 1, 2, 2, 3, 4)):
        c = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=cf)
        cm = oracle.CacheModel(S, W, tpf, H, D)
        for i in order:
            c.append_evict(0, to_dev(fin[i][0]), to_dev(fin[i][1]), cf)
            cm.append(fin[i][0], fin[i][1], cf)
        caches.append(c)
        models.append(cm)
    assert caches[0].slots(0)[0] != caches[1].slots(0)[0]
    ka, _ = models[0].logical_kv()
    kb, _ = models[1].logical_kv()
    assert np.array_equal(ka, kb)
    nq = cf * tpf
    q, k, v = (host((nq, H, D), seed=49, kind=t) for t in (synth.Q, synth.K, synth.V))
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    say("qk8 two ring phases")
    a = wmk.chunk_attention_qk8(caches[0], 0, tq, [(tk, tv)]).clone()
    b = wmk.chunk_attention_qk8(caches[1], 0, tq, [(tk, tv)])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rows = sample_rows(nq, np.random.default_rng(11), k=8, tile=256)
    compare(from_dev(a)[rows], oracle.chunk_attention_qk8(models[0], q, [(k, v)], 1 / math.sqrt(D), rows=rows),
            BF16_MAX_ABS, BF16_REL_L2, f"{len(rows)} rows vs quantized oracle")
    for c in caches:
        c.close()
