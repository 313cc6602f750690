"""GPU parity of the chunk-causal cross-attention over a multi-chunk sequence
(query chunk i reads the environment prompt and its own local prompt only)
through the C ABI, against the oracle on the same seeded inputs: all rows on
small shapes (ragged chunks and prompts, an empty environment or local
prompt, head_dim 64, fp32), sampled rows at the 720p shape, and the isolation
of every chunk from the other chunks' prompts."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_REL_L2, compare, from_dev, host,
                               sample_rows, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wmk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_attention_02_amd as m
    m.load()
    return m


def _inputs(cq, nc, ne, nl, H, D, seed, dtype="bf16"):
    q = host((cq * nc, H, D), dtype=dtype, seed=seed, kind=synth.Q)
    k = host((ne + nc * nl, H, D), dtype=dtype, seed=seed, kind=synth.KLOC)
    v = host((ne + nc * nl, H, D), dtype=dtype, seed=seed, kind=synth.VLOC)
    return q, k, v


@pytest.mark.parametrize("cq,nc,ne,nl,H,D", [
    (5, 4, 3, 7, 2, 128),        # several chunks inside one query tile
    (300, 3, 70, 130, 2, 128),   # chunk and prompt boundaries inside tiles
    (257, 2, 0, 65, 1, 64),      # no environment prompt, head_dim 64
    (100, 5, 200, 0, 2, 128),    # no local prompts: every chunk reads the environment only
])
def test_cross_train_small_all_rows(wmk, cq, nc, ne, nl, H, D):
    import torch
    q, k, v = _inputs(cq, nc, ne, nl, H, D, seed=21)
    say(f"cross train small cq={cq} chunks={nc} env={ne} local={nl} H={H} D={D}")
    out = wmk.cross_attention_train(to_dev(q), to_dev(k), to_dev(v), chunk_q_tokens=cq, env_tokens=ne,
                                    local_tokens=nl)
    torch.cuda.synchronize()
    ref = oracle.cross_attention_train(q, k, v, cq, ne, nl, 1 / math.sqrt(D))
    compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, "all rows")


def test_cross_train_fp32_small(wmk):
    import torch
    cq, nc, ne, nl, H, D = 7, 3, 5, 9, 2, 64
    q, k, v = _inputs(cq, nc, ne, nl, H, D, seed=22, dtype="f32")
    say(f"cross train fp32 cq={cq} chunks={nc} env={ne} local={nl}")
    out = wmk.cross_attention_train(to_dev(q), to_dev(k), to_dev(v), chunk_q_tokens=cq, env_tokens=ne,
                                    local_tokens=nl)
    torch.cuda.synchronize()
    ref = oracle.cross_attention_train(q, k, v, cq, ne, nl, 1 / math.sqrt(D))
    compare(from_dev(out), ref, F32_MAX_ABS, F32_REL_L2, "all rows")


def test_cross_train_chunks_ignore_other_prompts(wmk):
    """Altering local prompt j leaves every other chunk's rows bit for bit unchanged."""
    import torch
    cq, nc, ne, nl, H, D = 700, 4, 256, 300, 2, 128
    q, k, v = _inputs(cq, nc, ne, nl, H, D, seed=23)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    say(f"cross train isolation cq={cq} chunks={nc} env={ne} local={nl}")
    base = from_dev(wmk.cross_attention_train(dq, dk, dv, chunk_q_tokens=cq, env_tokens=ne, local_tokens=nl))
    j = 2
    dk2, dv2 = dk.clone(), dv.clone()
    dk2[ne + j * nl: ne + (j + 1) * nl] *= -1
    dv2[ne + j * nl: ne + (j + 1) * nl] += 1
    alt = from_dev(wmk.cross_attention_train(dq, dk2, dv2, chunk_q_tokens=cq, env_tokens=ne, local_tokens=nl))
    torch.cuda.synchronize()
    for c in range(nc):
        rows = slice(c * cq, (c + 1) * cq)
        if c == j:
            assert not np.array_equal(base[rows], alt[rows])
        else:
            np.testing.assert_array_equal(base[rows], alt[rows])


@pytest.mark.parametrize("seed", range(8))
def test_cross_train_random_shapes_all_rows(wmk, seed):
    """Every row of seeded random multi-chunk sequences against the oracle: chunk lengths,
    chunk count, environment and local prompt lengths (either may be empty, not both),
    heads and head_dim drawn at random, with and without the split-tail workspace."""
    import torch
    rng = np.random.default_rng(900 + seed)
    cq, nc = int(rng.integers(1, 1201)), int(rng.integers(1, 7))
    ne, nl = int(rng.integers(0, 601)), int(rng.integers(0, 401))
    if ne + nl == 0:
        nl = 1
    H, D = int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    q, k, v = _inputs(cq, nc, ne, nl, H, D, seed=1000 + seed)
    say(f"cross train random seed {seed}: cq={cq} chunks={nc} env={ne} local={nl} H={H} D={D}")
    ref = oracle.cross_attention_train(q, k, v, cq, ne, nl, 1 / math.sqrt(D))
    for use_ws in (False, True):
        out = wmk.cross_attention_train(to_dev(q), to_dev(k), to_dev(v), chunk_q_tokens=cq, env_tokens=ne,
                                        local_tokens=nl, use_workspace=use_ws)
        torch.cuda.synchronize()
        compare(from_dev(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"seed {seed} all rows ws={use_ws}")


def test_cross_train_720p(wmk):
    """720p chunks (4 frames x 3600 tokens, 24 heads) of a 3-chunk sequence with
    512-token environment and local prompts, split tail on: sampled rows."""
    import torch
    cq, nc, ne, nl, H, D = 4 * 3600, 3, 512, 512, 24, 128
    q, k, v = _inputs(cq, nc, ne, nl, H, D, seed=24)
    say(f"cross train 720p cq={cq} chunks={nc} env={ne} local={nl} H={H}")
    out = wmk.cross_attention_train(to_dev(q), to_dev(k), to_dev(v), chunk_q_tokens=cq, env_tokens=ne,
                                    local_tokens=nl, use_workspace=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sample_rows(cq * nc, rng, k=24, tile=256)
    rows = np.unique(np.concatenate([rows, [cq - 1, cq, 2 * cq - 1, 2 * cq]]))
    ref = oracle.cross_attention_train(q, k, v, cq, ne, nl, 1 / math.sqrt(D), rows=rows)
    compare(from_dev(out)[rows], ref, BF16_MAX_ABS, BF16_REL_L2, f"{len(rows)} sampled rows")
