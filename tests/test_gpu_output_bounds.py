"""Every entry point writes exactly its outputs: each output is placed between two
guard regions holding a fixed bit pattern, and after the call the guards are
unchanged, every element of the output was written (none still holds the
pattern, a value far outside any attention output or gradient), and the output
equals, bit for bit, the same call writing into a plain tensor.  The shapes run
both kernel shapes (8 and 4 waves) with and without the split tail, ragged last
query tiles, head_dim 64 and 128, and every mask mode."""
import ctypes
import math

import pytest

import synth
from tests.gpu_helpers import dev_fill, say

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements on each side (16-byte aligned for every dtype here)
PAT16 = 0x5A5A        # bf16 ~ 1.5e16
PAT32 = 0x5A5A5A5A    # fp32 ~ 1.5e16


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


def guarded(shape, dtype):
    """(buffer, view): a contiguous view of `shape` between two guard regions."""
    import torch
    n = math.prod(shape)
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    _bits(buf).fill_(PAT16 if dtype == torch.bfloat16 else PAT32)
    return buf, buf[GUARD:GUARD + n].view(shape)


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check(buf, view, plain, what):
    import torch
    torch.cuda.synchronize()
    pat = PAT16 if buf.dtype == torch.bfloat16 else PAT32
    b = _bits(buf)
    n = view.numel()
    assert bool((b[:GUARD] == pat).all()), f"{what}: written before the output"
    assert bool((b[GUARD + n:] == pat).all()), f"{what}: written after the output"
    assert not bool((_bits(view) == pat).any()), f"{what}: elements left unwritten"
    assert torch.equal(_bits(view), _bits(plain)), f"{what}: differs from the same call into a plain tensor"
    say(f"  {what}: {n} elements, guards intact")


@pytest.mark.parametrize("q_tokens,heads,head_dim,keys,what", [
    (2000, 40, 128, 4096, "8 waves, split tail, ragged tile"),
    (3000, 30, 128, 1024, "4 waves, split tail, ragged tile"),
    (700, 5, 64, 900, "head_dim 64, ragged keys"),
    (129, 3, 128, 64, "one full tile and one row"),
])
def test_chunk_attention_writes_only_its_output(wmk, q_tokens, heads, head_dim, keys, what):
    import torch
    say(f"chunk attention {q_tokens}x{heads}x{head_dim} over {keys} keys ({what})")
    q = dev_fill((q_tokens, heads, head_dim), kind=synth.Q, seed=11)
    k = dev_fill((keys, heads, head_dim), kind=synth.K, seed=11)
    v = dev_fill((keys, heads, head_dim), kind=synth.V, seed=11)
    plain = wmk.chunk_attention(None, 0, q, [(k, v)])
    buf, out = guarded(q.shape, torch.bfloat16)
    wmk.chunk_attention(None, 0, q, [(k, v)], out=out)
    check(buf, out, plain, what)


def test_cache_calls_write_only_their_outputs(wmk):
    import torch
    H, D, tpf = 4, 128, 100
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=tpf, sink_frames=2,
                      window_frames=3, chunk_frames=2)
    for c in range(4):
        cache.append_evict(0, dev_fill((2 * tpf, H, D), kind=synth.KFIN, chunk=c, seed=12),
                           dev_fill((2 * tpf, H, D), kind=synth.VFIN, chunk=c, seed=12), 2)
    q = dev_fill((2 * tpf + 37, H, D), kind=synth.Q, seed=12)
    k = dev_fill((2 * tpf + 37, H, D), kind=synth.K, seed=12)
    v = dev_fill((2 * tpf + 37, H, D), kind=synth.V, seed=12)
    calls = [
        ("chunk attention over the cache", lambda out: wmk.chunk_attention(cache, 0, q, [(k, v)], out=out)),
        ("retained frames", lambda out: wmk.chunk_attention(cache, 0, q, [(k, v)], out=out, keep_frames=[0, 1, 7])),
        ("FP8 QK^T", lambda out: wmk.chunk_attention_qk8(cache, 0, q, [(k, v)], out=out)),
        ("no-allocation entry point", lambda out: wmk.chunk_attention_noalloc(cache, 0, q, out, [(k, v)])),
    ]
    for what, call in calls:
        plain = torch.empty_like(q)
        call(plain)
        buf, out = guarded(q.shape, torch.bfloat16)
        call(out)
        check(buf, out, plain, what)
    cache.close()


def test_cross_attention_train_writes_only_its_output(wmk):
    import torch
    cq, nc, ne, nl, H, D = 1000, 3, 300, 200, 6, 128
    q = dev_fill((cq * nc, H, D), kind=synth.Q, seed=13)
    kx = dev_fill((ne + nc * nl, H, D), kind=synth.KLOC, seed=13)
    vx = dev_fill((ne + nc * nl, H, D), kind=synth.VLOC, seed=13)
    plain = wmk.cross_attention_train(q, kx, vx, chunk_q_tokens=cq, env_tokens=ne, local_tokens=nl)
    buf, out = guarded(q.shape, torch.bfloat16)
    wmk.cross_attention_train(q, kx, vx, chunk_q_tokens=cq, env_tokens=ne, local_tokens=nl, out=out)
    check(buf, out, plain, "cross-attention training mask")


def test_moba_forward_and_backward_write_only_their_outputs(wmk):
    import torch
    tpf, frames, cf, H, D = 50, 5, 2, 4, 128
    n = 3 * frames * tpf
    q, k, v, do = (dev_fill((n, H, D), kind=t, seed=14) for t in (synth.Q, synth.K, synth.V, synth.KLOC))
    mk = dict(tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
    o_plain, lse_plain = wmk.moba_attention_train(q, k, v, **mk)
    obuf, o = guarded(q.shape, torch.bfloat16)
    lbuf, lse = guarded((H, n), torch.float32)
    wmk.moba_attention_train(q, k, v, out=o, lse=lse, **mk)
    check(obuf, o, o_plain, "MoBA training forward, output")
    check(lbuf, lse, lse_plain, "MoBA training forward, log-sum-exp")
    o2 = torch.empty_like(q)
    wmk.moba_attention(q, k, v, out=o2, **mk)
    obuf2, o3 = guarded(q.shape, torch.bfloat16)
    wmk.moba_attention(q, k, v, out=o3, **mk)
    check(obuf2, o3, o2, "MoBA forward")

    dq_p, dk_p, dv_p = wmk.moba_attention_backward(q, k, v, o_plain, do, lse_plain, **mk)
    grads = [guarded(q.shape, torch.bfloat16) for _ in range(3)]
    hd = wmk.wmk_head_desc(H, D, wmk.WMK_BF16)
    md = wmk.wmk_moba_desc(tpf, frames, cf, 1)
    wsb = wmk.wmk_moba_backward_workspace_bytes(ctypes.byref(md), ctypes.byref(hd))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert wmk.wmk_moba_attention_backward(
        ctypes.byref(md), ctypes.byref(hd), q.data_ptr(), k.data_ptr(), v.data_ptr(), o_plain.data_ptr(),
        do.data_ptr(), lse_plain.data_ptr(), grads[0][1].data_ptr(), grads[1][1].data_ptr(),
        grads[2][1].data_ptr(), 1.0 / math.sqrt(D), ws.data_ptr(), wsb, st) == 0
    for (buf, g), ref, what in zip(grads, (dq_p, dk_p, dv_p), ("dq", "dk", "dv")):
        check(buf, g, ref, f"MoBA backward, {what}")
