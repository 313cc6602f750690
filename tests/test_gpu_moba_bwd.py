"""GPU parity of the MoBA training forward (log-sum-exp) and backward (dq, dk,
dv) through the C ABI against the oracle: every element on small sequences
(ragged frames, partial last chunk, with and without the bidirectional block),
and at the full 98 280-token sequence sampled dq rows, the dk/dv of whole
self-contained blocks (noisy chunk 0), sampled dk/dv key rows of clean chunks 0
and 3 (the longest walks of the dK/dV kernel) against the oracle's per-key
backward, and the column sums that softmax fixes; every element of a
12 600-token sequence with the same structure."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import LSE_ATOL, as_f32, from_dev, host, say, to_dev

pytestmark = pytest.mark.gpu

# gradients are rounded to bf16 on output; bounds relative to the largest entry
GRAD_MAX_ABS_REL = 2e-2
GRAD_REL_L2 = 1e-2


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


def compare_grad(got, ref, what):
    g = as_f32(np.asarray(got)).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape and np.all(np.isfinite(g)), what
    scale = max(np.abs(r).max(), 1e-30)
    ma = np.abs(g - r).max() / scale
    rl = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    say(f"  {what}: max_abs/max={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= GRAD_MAX_ABS_REL, (what, ma)
    assert rl <= GRAD_REL_L2, (what, rl)


def _inputs(n, H, D, seed):
    q, k, v = (host((n, H, D), seed=seed, kind=t) for t in (synth.Q, synth.K, synth.V))
    do = host((n, H, D), seed=seed, kind=synth.KLOC)       # the upstream gradient: one more seeded draw
    return q, k, v, do


@pytest.mark.parametrize("tpf,frames,cf,bidir,H", [
    (40, 5, 2, 1, 2),     # 600 tokens: q-tiles and key tiles straddle chunks and parts
    (37, 4, 3, 0, 2),     # ragged frames, partial last chunk, no bidirectional block
    (64, 3, 1, 1, 1),     # tile-aligned frames
])
def test_moba_backward_small_all_elements(wmk, tpf, frames, cf, bidir, H):
    import torch
    D = 128
    n = (2 + bidir) * frames * tpf
    q, k, v, do = _inputs(n, H, D, seed=70)
    say(f"moba bwd small tpf={tpf} frames={frames} cf={cf} bidir={bidir} n={n}")
    dq_, dk_, dv_, do_ = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    out, lse = wmk.moba_attention_train(dq_, dk_, dv_, tokens_per_frame=tpf, frames=frames, chunk_frames=cf,
                                        bidir_block=bidir)
    gq, gk, gv = wmk.moba_attention_backward(dq_, dk_, dv_, out, do_, lse, tokens_per_frame=tpf, frames=frames,
                                             chunk_frames=cf, bidir_block=bidir)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    mask = oracle.moba_mask(tpf, frames, cf, bidir)
    ref_lse = oracle.attention_lse(q, k, mask, scale)
    np.testing.assert_allclose(from_dev(lse), ref_lse, rtol=0, atol=LSE_ATOL)
    rq, rk, rv = oracle.moba_attention_backward(q, k, v, do, tpf, frames, cf, bidir, scale)
    compare_grad(from_dev(gq), rq, "dq")
    compare_grad(from_dev(gk), rk, "dk")
    compare_grad(from_dev(gv), rv, "dv")


@pytest.mark.parametrize("seed", range(6))
def test_moba_train_and_backward_random_shapes(wmk, seed):
    """Seeded random MoBA sequences (tokens per frame, frame and chunk counts, with and without
    the bidirectional block): the forward's output and log-sum-exp and every element of dq,
    dk and dv against the oracle.  The shapes put chunk and part boundaries anywhere inside
    the 64- and 256-row tiles, and give the backward's longest-first launch order from a
    few to many runs of equal walk length."""
    import torch
    r = np.random.default_rng(2000 + seed)
    tpf, frames = int(r.integers(5, 91)), int(r.integers(2, 8))
    cf, bidir, H, D = int(r.integers(1, frames + 1)), int(r.integers(0, 2)), int(r.integers(1, 3)), 128
    n = (2 + bidir) * frames * tpf
    q, k, v, do = _inputs(n, H, D, seed=300 + seed)
    say(f"moba random seed={seed}: tpf={tpf} frames={frames} cf={cf} bidir={bidir} H={H} n={n}")
    dq_, dk_, dv_, do_ = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    out, lse = wmk.moba_attention_train(dq_, dk_, dv_, tokens_per_frame=tpf, frames=frames, chunk_frames=cf,
                                        bidir_block=bidir)
    gq, gk, gv = wmk.moba_attention_backward(dq_, dk_, dv_, out, do_, lse, tokens_per_frame=tpf, frames=frames,
                                             chunk_frames=cf, bidir_block=bidir)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    ref_out = oracle.moba_attention(q, k, v, tpf, frames, cf, bidir, scale)
    compare_grad(from_dev(out), ref_out, "out")
    mask = oracle.moba_mask(tpf, frames, cf, bidir)
    np.testing.assert_allclose(from_dev(lse), oracle.attention_lse(q, k, mask, scale), rtol=0, atol=LSE_ATOL)
    rq, rk, rv = oracle.moba_attention_backward(q, k, v, do, tpf, frames, cf, bidir, scale)
    compare_grad(from_dev(gq), rq, "dq")
    compare_grad(from_dev(gk), rk, "dk")
    compare_grad(from_dev(gv), rv, "dv")


def test_moba_backward_mid_size_all_elements(wmk):
    """21 + 21 + 21 frames of 200 tokens in chunks of 3 (12 600 tokens, 2 heads): every
    element of dq, dk and dv against the oracle.  A clean key of chunk 0 is read by the
    clean rows of all 7 chunks and the noisy rows of chunks 1-6 (8 400 rows, 132 query
    tiles), so the dK/dV kernel's long walks over query tiles are all compared."""
    import torch
    tpf, frames, cf, H, D = 200, 21, 3, 2, 128
    n = 3 * frames * tpf
    q, k, v, do = _inputs(n, H, D, seed=72)
    say(f"moba bwd mid size n={n}")
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    out, lse = wmk.moba_attention_train(tq, tk, tv, tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
    gq, gk, gv = wmk.moba_attention_backward(tq, tk, tv, out, tdo, lse, tokens_per_frame=tpf, frames=frames,
                                             chunk_frames=cf)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    say("  oracle backward")
    rq, rk, rv = oracle.moba_attention_backward(q, k, v, do, tpf, frames, cf, 1, scale)
    compare_grad(from_dev(gq), rq, "dq")
    compare_grad(from_dev(gk), rk, "dk")
    compare_grad(from_dev(gv), rv, "dv")
    # the keys with the longest walks on their own: clean chunk 0
    cl = cf * tpf
    compare_grad(from_dev(gk)[:cl], rk[:cl], "dk of clean chunk 0")
    compare_grad(from_dev(gv)[:cl], rv[:cl], "dv of clean chunk 0")


def test_moba_backward_full_sequence(wmk):
    """21 + 21 + 21 frames of 1560 tokens, chunks of 3, 12 heads."""
    import torch
    tpf, frames, cf, H, D = 1560, 21, 3, 12, 128
    L, cl = frames * tpf, cf * tpf
    n = 3 * L
    q, k, v, do = _inputs(n, H, D, seed=71)
    say("moba bwd full sequence")
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    out, lse = wmk.moba_attention_train(tq, tk, tv, tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
    gq, gk, gv = wmk.moba_attention_backward(tq, tk, tv, out, tdo, lse, tokens_per_frame=tpf, frames=frames,
                                             chunk_frames=cf)
    torch.cuda.synchronize()
    gq, gk, gv = from_dev(gq), from_dev(gk), from_dev(gv)
    scale = 1 / math.sqrt(D)
    heads = [0, 7]
    # (a) sampled dq rows: each row against its allowed keys
    rng = np.random.default_rng(12)
    rows = sorted(set(rng.choice(n, 6, replace=False).tolist()) | {0, cl - 1, L, L + cl, 2 * L, n - 1})
    for i in rows:
        keys = np.concatenate([np.arange(a, b) for a, b in oracle.moba_row_intervals(i, tpf, frames, cf)])
        sub = lambda x: x[:, heads]
        rq, _, _ = oracle.attention_backward(sub(q[i:i + 1]), sub(k[keys]), sub(v[keys]), sub(do[i:i + 1]),
                                             np.ones((1, keys.size), bool), scale)
        compare_grad(gq[i:i + 1][:, heads], rq, f"dq row {i}")
    # (b) noisy chunk 0: its rows see only its own keys and its keys are seen only by its rows
    blk = slice(L, L + cl)
    sub = lambda x: x[blk][:, heads]
    rq, rk, rv = oracle.attention_backward(sub(q), sub(k), sub(v), sub(do), np.ones((cl, cl), bool), scale)
    compare_grad(gk[blk][:, heads], rk, "dk of noisy chunk 0")
    compare_grad(gv[blk][:, heads], rv, "dv of noisy chunk 0")
    compare_grad(gq[blk][:, heads], rq, "dq of noisy chunk 0")
    # (c) sampled key rows with the longest walks: clean chunk 0 (read by the clean rows of all
    # 7 chunks and the noisy rows of chunks 1-6: 60 840 rows, ~950 query tiles), clean chunk 3,
    # and a noisy key -- exact dk, dv from the oracle's per-key backward (each attending row's
    # softmax over its own allowed keys)
    keys = np.array([0, 1, 2345, cl - 1, 3 * cl, 3 * cl + 2000, L + 2 * cl + 17])
    say("  oracle per-key backward")
    sub = lambda x: np.ascontiguousarray(x[:, heads])
    rk, rv = oracle.attention_key_gradients(sub(q), sub(k), sub(v), sub(do),
                                            lambda i: oracle.moba_row_intervals(i, tpf, frames, cf), keys, scale)
    compare_grad(gk[keys][:, heads], rk, "dk of sampled keys (clean chunks 0 and 3, noisy chunk 2)")
    compare_grad(gv[keys][:, heads], rv, "dv of sampled keys (clean chunks 0 and 3, noisy chunk 2)")
    # (d) softmax invariants over the whole sequence: sum_j dk_j = 0, sum_j dv_j = sum_i dout_i
    dk64, dv64 = as_f32(gk).astype(np.float64), as_f32(gv).astype(np.float64)
    do64 = as_f32(do).astype(np.float64)
    assert np.abs(dk64.sum(axis=0)).max() <= 1e-2 * np.abs(dk64).sum(axis=0).max()
    err = np.abs(dv64.sum(axis=0) - do64.sum(axis=0)).max()
    assert err <= 1e-2 * np.abs(do64).sum(axis=0).max(), err
