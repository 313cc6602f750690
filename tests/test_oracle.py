"""Pins of the oracle: brute force, invariants, closed forms, layout and traces.

Every check here compares the oracle with something other than itself: a
dense NumPy fp64 masked softmax built from a per-pair mask predicate, a list
simulation of the pages' generation loop, a mathematical identity, or a count
derived by hand from the pages (fixtures under tests/golden/).
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="session", autouse=True)
def _built():
    if not os.path.exists(os.path.join(os.path.dirname(oracle.__file__), "liboracle.so")):
        oracle.build()
    if not os.path.exists(os.path.join(os.path.dirname(synth.__file__), "libsynth_cpu.so")):
        synth.build()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def dense_masked_softmax(q, k, v, mask, scale):
    """Brute force: scores for every pair, -inf where masked, softmax, times V (fp64)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = np.einsum("ihd,jhd->hij", q, k) * scale            # [H][nq][nk]
    s = np.where(mask[None, :, :], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    den = p.sum(-1, keepdims=True)
    p = np.divide(p, den, out=np.zeros_like(p), where=den > 0)
    return np.einsum("hij,jhd->ihd", p, v), p


def mask_from_intervals(ivs, nk):
    m = np.zeros((len(ivs), nk), dtype=bool)
    for i, row in enumerate(ivs):
        for a, b in row:
            m[i, a:b] = True
    return m


# ---------------------------------------------------------------------------------------------
# attention core vs brute force
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nk,H,D", [(5, 11, 3, 7), (17, 40, 2, 64), (1, 1, 1, 1), (9, 33, 4, 128)])
def test_attend_matches_dense_brute_force(nq, nk, H, D):
    rng = np.random.default_rng(nq * 1000 + nk)
    q, k, v = _rand((nq, H, D), 1), _rand((nk, H, D), 2), _rand((nk, H, D), 3)
    ivs = []
    for i in range(nq):
        cuts = np.sort(rng.choice(nk + 1, size=4, replace=True))
        ivs.append([(int(cuts[0]), int(cuts[1])), (int(cuts[2]), int(cuts[3]))])
    ivs[0] = [(0, nk)]
    scale = 0.37
    out, probs = oracle.attend(q, k, v, ivs, scale, want_probs=True)
    ref, pref = dense_masked_softmax(q, k, v, mask_from_intervals(ivs, nk), scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(probs, pref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_probabilities_sum_to_one():
    """I1: every softmax row with at least one allowed key sums to one."""
    q, k, v = _rand((12, 2, 16), 4), _rand((30, 2, 16), 5), _rand((30, 2, 16), 6)
    ivs = [[(0, 3 + i)] if i % 3 else [(2, 9), (20, 30)] for i in range(12)]
    _, p = oracle.attend(q, k, v, ivs, 0.25, want_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)


def test_empty_row_outputs_zero():
    q, k, v = _rand((3, 1, 8), 7), _rand((5, 1, 8), 8), _rand((5, 1, 8), 9)
    out = oracle.attend(q, k, v, [[], [(0, 5)], []], 1.0)
    assert np.all(out[0] == 0) and np.all(out[2] == 0) and np.any(out[1] != 0)


def test_bf16_inputs_widen_exactly():
    x = np.array([1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    w = oracle.widen(b)
    assert w.dtype == np.float32
    np.testing.assert_array_equal(w[:3], x[:3])
    assert abs(w[3] - 1e-3) < 1e-5


# ---------------------------------------------------------------------------------------------
# closed forms (C1-C4)
# ---------------------------------------------------------------------------------------------

def test_zero_query_gives_mean_of_allowed_values():
    """C1: q = 0 makes every allowed score equal, so the output is the mean of the allowed v."""
    k, v = _rand((20, 2, 8), 10), _rand((20, 2, 8), 11)
    q = np.zeros((2, 2, 8), np.float32)
    ivs = [[(3, 9), (15, 20)], [(0, 20)]]
    out = oracle.attend(q, k, v, ivs, 0.5)
    np.testing.assert_allclose(out[0], np.concatenate([v[3:9], v[15:20]]).astype(np.float64).mean(0), atol=1e-12)
    np.testing.assert_allclose(out[1], v.astype(np.float64).mean(0), atol=1e-12)


def test_equal_keys_give_mean_of_values():
    """C2: identical keys make the weights uniform whatever q is."""
    q, v = _rand((4, 1, 16), 12), _rand((10, 1, 16), 13)
    k = np.repeat(_rand((1, 1, 16), 14), 10, axis=0)
    out = oracle.attend(q, k, v, [[(0, 10)]] * 4, 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(v.astype(np.float64).mean(0), out.shape), atol=1e-12)


def test_dominant_logit_selects_its_value():
    """C3: a key whose logit exceeds all others by 40 takes weight 1 - O(e^-40)."""
    D = 4
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((9, 1, D), np.float32)
    k[5, 0, 0] = 40.0
    v = _rand((9, 1, D), 15)
    out = oracle.attend(q, k, v, [[(0, 9)]], 1.0)
    np.testing.assert_allclose(out[0, 0], v[5, 0], atol=1e-6)


def test_constant_values_pass_through():
    """C4: when every allowed v is the same vector, so is the output."""
    q, k = _rand((6, 3, 8), 16), _rand((25, 3, 8), 17)
    c = _rand((1, 3, 8), 18)
    v = np.repeat(c, 25, axis=0)
    out = oracle.attend(q, k, v, [[(i, 25)] for i in range(6)], 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(c.astype(np.float64), out.shape), atol=1e-12)


def test_linear_in_values():
    """I6: for fixed q and k the output is linear in V."""
    q, k = _rand((5, 2, 8), 19), _rand((13, 2, 8), 20)
    v1, v2 = _rand((13, 2, 8), 21), _rand((13, 2, 8), 22)
    ivs = [[(0, 13)], [(2, 7)], [(0, 1), (5, 13)], [(12, 13)], [(0, 13)]]
    a, b = 0.75, -1.5
    lhs = oracle.attend(q, k, (a * v1 + b * v2).astype(np.float32), ivs, 0.4)
    rhs = a * oracle.attend(q, k, v1, ivs, 0.4) + b * oracle.attend(q, k, v2, ivs, 0.4)
    np.testing.assert_allclose(lhs, rhs, atol=1e-6)


# ---------------------------------------------------------------------------------------------
# cache policy: loop simulation, layout, traces
# ---------------------------------------------------------------------------------------------

def loop_simulation(S, W, n_frames_total, per_append):
    """The repo-explainer loop at frame granularity: the state list keeps the anchor
    frames and, after each append, drops the oldest non-anchor frames beyond W."""
    state, anchors, history = [], [], []
    f = 0
    while f < n_frames_total:
        for _ in range(min(per_append, n_frames_total - f)):
            state.append(f)
            if len(anchors) < S:
                anchors.append(f)
            f += 1
        while len([x for x in state if x not in anchors]) > W:
            oldest = min(x for x in state if x not in anchors)
            state.remove(oldest)
        history.append((f, list(state)))
    return history


@pytest.mark.parametrize("S,W,cf", [(6, 8, 4), (1, 2, 2), (0, 3, 1), (2, 5, 3), (3, 1, 2), (4, 4, 4)])
def test_resident_set_matches_loop_simulation(S, W, cf):
    """I4: after every append the sinks are frames 0..S-1 and the rest are the last W frames."""
    for F, state in loop_simulation(S, W, 40, cf):
        assert oracle.resident_frames(F, S, W) == sorted(state)
        assert oracle.valid_slots(F, S, W) == len(state)


@pytest.mark.parametrize("S,W,cf", [(6, 8, 4), (1, 2, 2), (0, 3, 1), (2, 5, 3), (3, 1, 2), (5, 3, 7)])
def test_resident_frames_fill_slot_prefix(S, W, cf):
    """I5: resident frames always occupy slots 0..valid-1, one frame per slot."""
    for F in range(0, 60):
        slots = sorted(oracle.slot_of_frame(f, S, W) for f in oracle.resident_frames(F, S, W))
        assert slots == list(range(oracle.valid_slots(F, S, W)))


@settings(max_examples=300, deadline=None)
@given(S=st.integers(0, 6), W=st.integers(1, 8), lens=st.lists(st.integers(1, 20), min_size=1, max_size=12))
def test_cache_model_matches_the_loop_for_any_append_lengths(S, W, lens):
    """I4/I5 for appends of any lengths: after each append the cache model holds exactly the
    frames the frame-level loop keeps (append, then drop the oldest non-anchor frames beyond
    W), each in its own slot of the prefix, with its own K and V."""
    cm = oracle.CacheModel(S, W, 1, 1, 1, dtype=np.float32)
    state, anchors, f = [], [], 0
    for n in lens:
        ids = np.arange(f, f + n, dtype=np.float32).reshape(n, 1, 1)
        cm.append(ids, -ids - 1, n)
        for _ in range(n):
            state.append(f)
            if len(anchors) < S:
                anchors.append(f)
            f += 1
        while len([x for x in state if x not in anchors]) > W:
            state.remove(min(x for x in state if x not in anchors))
        assert cm.resident() == sorted(state)
        assert sorted(oracle.slot_of_frame(x, S, W) for x in state) == list(range(len(state)))
        kb, vb = cm.slot_buffers()
        for x in state:
            slot = oracle.slot_of_frame(x, S, W)
            assert kb[slot, 0, 0, 0] == x and vb[slot, 0, 0, 0] == -x - 1


def test_long_append_keeps_last_window_frames():
    """An append longer than the window leaves the same resident set as appending its
    frames one by one; the skipped frames are exactly the ones the loop would evict."""
    S, W, tpf, H, D = 2, 3, 2, 1, 4
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    rows = _rand((9 * tpf, H, D), 23)
    cm.append(rows, -rows, 9)
    assert cm.resident() == [0, 1, 6, 7, 8]
    assert oracle.frames_kept_by_append(0, 9, S, W) == [0, 1, 6, 7, 8]
    kb, vb = cm.slot_buffers()
    for f in cm.resident():
        s = oracle.slot_of_frame(f, S, W)
        np.testing.assert_array_equal(kb[s], rows[f * tpf:(f + 1) * tpf])
        np.testing.assert_array_equal(vb[s], -rows[f * tpf:(f + 1) * tpf])


def test_traces_match_hand_derivation():
    g = _golden("cache_traces.json")
    t = g["tiny_rollout"]
    S, W, cf = t["sink_frames"], t["window_frames"], t["chunk_frames"]
    cm = oracle.CacheModel(S, W, 1, 1, 1, dtype=np.float32)
    for c, want in enumerate(t["resident_before_chunk"]):
        assert cm.resident() == want
        cm.append(np.zeros((cf, 1, 1), np.float32), np.zeros((cf, 1, 1), np.float32), cf)
    assert cm.slot_map().tolist() == t["slot_map_after_6_chunks"]

    t = g["rolling_832x464"]
    S, W, cf = t["sink_frames"], t["window_frames"], t["chunk_frames"]
    cm = oracle.CacheModel(S, W, 1, 1, 1, dtype=np.float32)
    z = np.zeros((cf, 1, 1), np.float32)
    for c in range(8):
        if c < len(t["valid_slots_before_chunk"]):
            assert oracle.valid_slots(cm.F, S, W) == t["valid_slots_before_chunk"][c]
        if c == 4:
            assert cm.slot_map().tolist() == t["slot_map_before_chunk_4"]
        if c == 5:
            assert cm.slot_map().tolist() == t["slot_map_before_chunk_5"]
        cm.append(z, z, cf)
    assert cm.F == 32
    assert cm.slot_map().tolist() == t["slot_map_after_32_frames"]


def test_eighteen_slot_layout():
    """6 anchors + 8 recent + 4 current frames once the 832x464 session is past chunk 3."""
    g = _golden("layout_18slot.json")
    S, W, cf, tpf = g["anchor_frames"], g["recent_frames"], g["current_frames"], g["tokens_per_frame"]
    for F in range(16, 16 + 4 * 50, 4):
        res = oracle.resident_frames(F, S, W)
        assert len([f for f in res if f < S]) == S
        assert len([f for f in res if f >= S]) == W
        assert len(res) + cf == g["total_slots"]
        assert len(res) * tpf == g["cache_tokens"]
        assert (len(res) + cf) * tpf == g["kv_tokens"]
        assert cf * tpf == g["q_tokens"]


def test_cache_model_contents_by_slot():
    """P4: a slot holds exactly the rows of the append call that carried its frame."""
    S, W, cf, tpf, H, D = 2, 3, 2, 3, 2, 4
    cm = oracle.CacheModel(S, W, tpf, H, D)
    sent = {}
    for c in range(7):
        kb = synth.normal(cf * tpf * H * D, seed=5, chunk=c, kind=synth.KFIN).reshape(cf * tpf, H, D)
        vb = synth.normal(cf * tpf * H * D, seed=5, chunk=c, kind=synth.VFIN).reshape(cf * tpf, H, D)
        for j in range(cf):
            sent[c * cf + j] = (kb[j * tpf:(j + 1) * tpf], vb[j * tpf:(j + 1) * tpf])
        cm.append(kb, vb, cf)
        kbuf, vbuf = cm.slot_buffers()
        for s, f in enumerate(cm.slot_map()):
            if f >= 0:
                np.testing.assert_array_equal(kbuf[s], sent[f][0])
                np.testing.assert_array_equal(vbuf[s], sent[f][1])
            else:
                assert s >= oracle.valid_slots(cm.F, S, W)


# ---------------------------------------------------------------------------------------------
# rollout: incremental cache attention vs one dense masked softmax (tiny workload, fp32)
# ---------------------------------------------------------------------------------------------

def rollout_allowed(fq, fk, S, W, cf):
    """Frame-level mask of the whole tiny rollout: a query frame sees its own chunk
    (both directions) and, among earlier chunks' frames, the sinks and the last W."""
    cq, ck = fq // cf, fk // cf
    Fq = cq * cf
    return (ck == cq) or (fk < Fq and (fk < S or fk >= Fq - W))


def _tiny_rollout(S, W, cf, tpf, H, D, n_chunks, seed):
    """Run the oracle chunk by chunk (current chunk's K/V as the segment, then append it)
    and return (all q, all k, all v, outputs), each stacked over the whole sequence."""
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    n = cf * tpf * H * D
    qs, ks, vs, outs = [], [], [], []
    for c in range(n_chunks):
        q = synth.normal(n, dtype="f32", seed=seed, chunk=c, kind=synth.Q).reshape(cf * tpf, H, D)
        k = synth.normal(n, dtype="f32", seed=seed, chunk=c, kind=synth.K).reshape(cf * tpf, H, D)
        v = synth.normal(n, dtype="f32", seed=seed, chunk=c, kind=synth.V).reshape(cf * tpf, H, D)
        outs.append(oracle.chunk_attention(cm, q, [(k, v)], 1.0 / np.sqrt(D)))
        cm.append(k, v, cf)
        qs.append(q), ks.append(k), vs.append(v)
    return np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), np.concatenate(outs)


def _dense_rollout_mask(S, W, cf, tpf, n_frames):
    fr = np.arange(n_frames * tpf) // tpf
    return np.array([[rollout_allowed(a, b, S, W, cf) for b in fr] for a in fr])


def test_tiny_rollout_matches_dense_masked_softmax():
    """The tiny fp32 workload verbatim: 1 head, head_dim 64, 16 tokens per frame,
    chunks of 2 frames, 1 sink + window 2, 6 chunks, checked against one dense mask."""
    S, W, cf, tpf, H, D, n = 1, 2, 2, 16, 1, 64, 6
    q, k, v, out = _tiny_rollout(S, W, cf, tpf, H, D, n, seed=0)
    ref, _ = dense_masked_softmax(q, k, v, _dense_rollout_mask(S, W, cf, tpf, n * cf), 1.0 / np.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,W,cf", [(1, 10, 2), (0, 12, 3), (4, 8, 4)])
def test_full_window_rollout_is_block_causal(S, W, cf):
    """I2: when S + W covers all history, the rollout equals full-sequence block-causal attention."""
    tpf, H, D, n = 3, 2, 8, 4
    assert S + W >= cf * (n - 1)          # every earlier chunk stays resident
    q, k, v, out = _tiny_rollout(S, W, cf, tpf, H, D, n, seed=1)
    fr = np.arange(n * cf * tpf) // (cf * tpf)
    mask = fr[None, :] <= fr[:, None]
    ref, _ = dense_masked_softmax(q, k, v, mask, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_permuting_current_chunk_permutes_outputs():
    """I3: permuting the current chunk's tokens (q rows with their k/v rows) permutes outputs."""
    S, W, cf, tpf, H, D = 2, 3, 2, 5, 2, 16
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    for c in range(3):
        cm.append(_rand((cf * tpf, H, D), 30 + c), _rand((cf * tpf, H, D), 40 + c), cf)
    q, k, v = _rand((cf * tpf, H, D), 50), _rand((cf * tpf, H, D), 51), _rand((cf * tpf, H, D), 52)
    perm = np.random.default_rng(3).permutation(cf * tpf)
    a = oracle.chunk_attention(cm, q, [(k, v)], 0.3)
    b = oracle.chunk_attention(cm, q[perm], [(k[perm], v[perm])], 0.3)
    np.testing.assert_allclose(b, a[perm], atol=1e-12)


def test_chunk_attention_rows_subset():
    S, W, cf, tpf, H, D = 1, 2, 2, 4, 3, 8
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    cm.append(_rand((cf * tpf, H, D), 60), _rand((cf * tpf, H, D), 61), cf)
    q, k, v = _rand((cf * tpf, H, D), 62), _rand((cf * tpf, H, D), 63), _rand((cf * tpf, H, D), 64)
    full = oracle.chunk_attention(cm, q, [(k, v)], 0.5)
    rows = [7, 0, 3]
    np.testing.assert_array_equal(oracle.chunk_attention(cm, q, [(k, v)], 0.5, rows=rows), full[rows])


# ---------------------------------------------------------------------------------------------
# variable retention: a call attends a chosen subset of the resident frames
# ---------------------------------------------------------------------------------------------

def _retained_rollout(S, W, cf, tpf, H, D, n_chunks, seed, pick):
    """Rollout where chunk c attends only pick(c, resident) of the resident frames."""
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    n = cf * tpf * H * D
    qs, ks, vs, outs, kept = [], [], [], [], []
    for c in range(n_chunks):
        q = synth.normal(n, dtype="f32", seed=seed, chunk=c, kind=synth.Q).reshape(cf * tpf, H, D)
        k = synth.normal(n, dtype="f32", seed=seed, chunk=c, kind=synth.K).reshape(cf * tpf, H, D)
        v = synth.normal(n, dtype="f32", seed=seed, chunk=c, kind=synth.V).reshape(cf * tpf, H, D)
        keep = pick(c, cm.resident())
        kept.append(set(keep))
        outs.append(oracle.chunk_attention(cm, q, [(k, v)], 1.0 / np.sqrt(D), keep_frames=keep))
        cm.append(k, v, cf)
        qs.append(q), ks.append(k), vs.append(v)
    return np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), np.concatenate(outs), kept


@pytest.mark.parametrize("S,W,cf,policy", [(2, 4, 2, "random"), (1, 6, 3, "anchors_and_last"), (3, 3, 1, "random")])
def test_retained_rollout_matches_dense_frame_mask(S, W, cf, policy):
    """Retention stated pairwise: a query frame of chunk c sees its own chunk and exactly the
    frames kept for chunk c, which must be a subset of the sinks and the last W frames."""
    tpf, H, D, n = 3, 2, 8, 6
    rng = np.random.default_rng(11)

    def pick(c, resident):
        if policy == "random":
            return [f for f in resident if rng.random() < 0.6]
        return [f for f in resident if f < S] + [f for f in resident if f >= S][-2:]   # anchors + 2 latest

    q, k, v, out, kept = _retained_rollout(S, W, cf, tpf, H, D, n, seed=4, pick=pick)
    fr = np.arange(n * cf * tpf) // tpf
    mask = np.zeros((fr.size, fr.size), dtype=bool)
    for a in range(fr.size):
        c = fr[a] // cf
        for b in range(fr.size):
            mask[a, b] = (fr[b] // cf == c) or (fr[b] in kept[c] and rollout_allowed(fr[a], fr[b], S, W, cf))
    ref, _ = dense_masked_softmax(q, k, v, mask, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_retention_of_every_resident_frame_is_plain_chunk_attention():
    S, W, cf, tpf, H, D = 2, 3, 2, 4, 2, 8
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    for c in range(4):
        cm.append(_rand((cf * tpf, H, D), 70 + c), _rand((cf * tpf, H, D), 80 + c), cf)
    q, k, v = _rand((cf * tpf, H, D), 90), _rand((cf * tpf, H, D), 91), _rand((cf * tpf, H, D), 92)
    full = oracle.chunk_attention(cm, q, [(k, v)], 0.4)
    shuffled = list(np.random.default_rng(2).permutation(cm.resident()))
    np.testing.assert_array_equal(oracle.chunk_attention(cm, q, [(k, v)], 0.4, keep_frames=shuffled), full)


def test_dropped_frames_do_not_matter_and_empty_keep_is_segment_attention():
    S, W, cf, tpf, H, D = 2, 4, 2, 3, 2, 8
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    for c in range(4):
        cm.append(_rand((cf * tpf, H, D), 100 + c), _rand((cf * tpf, H, D), 110 + c), cf)
    q, k, v = _rand((cf * tpf, H, D), 120), _rand((cf * tpf, H, D), 121), _rand((cf * tpf, H, D), 122)
    res = cm.resident()
    keep = [res[0], res[-1], res[3]]
    a = oracle.chunk_attention(cm, q, [(k, v)], 0.7, keep_frames=keep)
    for f in set(res) - set(keep):            # scramble every dropped frame
        cm.frames[f] = (cm.frames[f][0] * -3 + 1, cm.frames[f][1] + 5)
    np.testing.assert_array_equal(oracle.chunk_attention(cm, q, [(k, v)], 0.7, keep_frames=keep), a)
    # nothing retained: plain softmax over the segment alone
    m = np.ones((cf * tpf, cf * tpf), dtype=bool)
    ref, _ = dense_masked_softmax(q, k, v, m, 0.7)
    np.testing.assert_allclose(oracle.chunk_attention(cm, q, [(k, v)], 0.7, keep_frames=[]), ref, atol=1e-12)
    # one kept frame whose values are one constant row per head, no segment: the output is that row
    f = res[2]
    const = _rand((1, H, D), 123)
    cm.frames[f] = (cm.frames[f][0], np.repeat(const, tpf, axis=0))
    np.testing.assert_allclose(oracle.chunk_attention(cm, q, [], 0.7, keep_frames=[f]),
                               np.repeat(const, cf * tpf, axis=0), atol=1e-6)


def test_retention_rejects_non_resident_and_repeated_frames():
    cm = oracle.CacheModel(1, 2, 2, 1, 4, dtype=np.float32)
    for c in range(3):
        cm.append(_rand((4, 1, 4), c), _rand((4, 1, 4), 10 + c), 2)
    q = _rand((2, 1, 4), 5)
    assert cm.resident() == [0, 4, 5]
    for bad in ([1], [6], [-1], [0, 0]):
        with pytest.raises(ValueError):
            oracle.chunk_attention(cm, q, [], 1.0, keep_frames=bad)


# ---------------------------------------------------------------------------------------------
# MoBA mask
# ---------------------------------------------------------------------------------------------

def moba_pair_allowed(i, j, tpf, frames, cf):
    """M1-M4 stated pairwise: clean->clean if key chunk <= query chunk; noisy->clean if
    key chunk < query chunk; noisy->noisy if same chunk; block->block always."""
    L = frames * tpf
    pi, pj = i // L, j // L
    ki, kj = ((i % L) // tpf) // cf, ((j % L) // tpf) // cf
    if pi == 0 and pj == 0:
        return kj <= ki
    if pi == 1 and pj == 0:
        return kj < ki
    if pi == 1 and pj == 1:
        return kj == ki
    if pi == 2 and pj == 2:
        return True
    return False


@settings(max_examples=150, deadline=None)
@given(tpf=st.integers(1, 5), frames=st.integers(1, 9), bidir=st.integers(0, 1), data=st.data())
def test_moba_intervals_match_pairwise_mask_any_shape(tpf, frames, bidir, data):
    """The row intervals equal M1-M4 stated pairwise for any frame size, frame and chunk
    count (a partial last chunk included), with and without the bidirectional block."""
    cf = data.draw(st.integers(1, frames))
    n = (2 + bidir) * frames * tpf
    want = np.array([[moba_pair_allowed(i, j, tpf, frames, cf) for j in range(n)] for i in range(n)])
    ivs = [oracle.moba_row_intervals(i, tpf, frames, cf, bidir) for i in range(n)]
    np.testing.assert_array_equal(mask_from_intervals(ivs, n), want)


@pytest.mark.parametrize("tpf,frames,cf", [(4, 6, 2), (3, 7, 3), (2, 5, 1), (5, 4, 4), (1, 9, 2)])
def test_moba_intervals_match_pairwise_mask(tpf, frames, cf):
    n = 3 * frames * tpf
    want = np.array([[moba_pair_allowed(i, j, tpf, frames, cf) for j in range(n)] for i in range(n)])
    ivs = [oracle.moba_row_intervals(i, tpf, frames, cf) for i in range(n)]
    np.testing.assert_array_equal(mask_from_intervals(ivs, n), want)


def test_moba_tiny_matches_dense_brute_force():
    tpf, frames, cf, H, D = 4, 6, 2, 2, 16
    n = 3 * frames * tpf
    q, k, v = _rand((n, H, D), 70), _rand((n, H, D), 71), _rand((n, H, D), 72)
    mask = np.array([[moba_pair_allowed(i, j, tpf, frames, cf) for j in range(n)] for i in range(n)])
    ref, _ = dense_masked_softmax(q, k, v, mask, 0.25)
    out = oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 0.25)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_moba_allowed_pair_count_at_full_size():
    """945 of 3969 frame pairs (23.8 %) for 21+21+21 frames in chunks of 3, at 1560 tokens per frame."""
    g = _golden("moba_pairs.json")
    tpf, frames, cf = 1560, g["frames"], g["chunk_frames"]
    total = 0
    for i in range(0, 3 * frames * tpf, tpf):       # one row per frame: every row of a frame has the same mask
        total += sum(b - a for a, b in oracle.moba_row_intervals(i, tpf, frames, cf)) * tpf
    assert total == g["allowed_frame_pairs"] * tpf * tpf
    assert g["clean_clean"] + g["noisy_clean"] + g["noisy_noisy"] + g["block_block"] == g["allowed_frame_pairs"]
    assert (3 * frames) ** 2 == g["total_frame_pairs"]


def test_moba_noisy_rows_equal_teacher_forced_chunk_attention():
    """I7: noisy chunk i = chunk attention over a cache holding clean chunks < i (no
    eviction) with noisy chunk i as the current chunk."""
    tpf, frames, cf, H, D = 3, 6, 2, 2, 8
    L = frames * tpf
    n = 3 * L
    q, k, v = _rand((n, H, D), 80), _rand((n, H, D), 81), _rand((n, H, D), 82)
    moba = oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 0.3)
    cl = cf * tpf
    for c in range(frames // cf):
        cm = oracle.CacheModel(0, frames, tpf, H, D, dtype=np.float32)
        if c > 0:
            cm.append(k[:c * cl], v[:c * cl], c * cf)
        rows = slice(L + c * cl, L + (c + 1) * cl)
        got = oracle.chunk_attention(cm, q[rows], [(k[rows], v[rows])], 0.3)
        np.testing.assert_allclose(moba[rows], got, atol=1e-12)


def test_moba_clean_rows_equal_block_causal_chunk_attention():
    """Clean chunk i = chunk attention over a cache of clean chunks < i plus clean chunk i."""
    tpf, frames, cf, H, D = 2, 6, 3, 1, 8
    L = frames * tpf
    q, k, v = _rand((3 * L, H, D), 83), _rand((3 * L, H, D), 84), _rand((3 * L, H, D), 85)
    moba = oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 0.6)
    cl = cf * tpf
    for c in range(frames // cf):
        cm = oracle.CacheModel(0, frames, tpf, H, D, dtype=np.float32)
        if c > 0:
            cm.append(k[:c * cl], v[:c * cl], c * cf)
        rows = slice(c * cl, (c + 1) * cl)
        np.testing.assert_allclose(moba[rows], oracle.chunk_attention(cm, q[rows], [(k[rows], v[rows])], 0.6),
                                   atol=1e-12)


def test_moba_block_rows_equal_plain_bidirectional_attention():
    """I8: rows of the appended block equal dense attention over the block alone."""
    tpf, frames, cf, H, D = 3, 5, 2, 2, 8
    L = frames * tpf
    q, k, v = _rand((3 * L, H, D), 86), _rand((3 * L, H, D), 87), _rand((3 * L, H, D), 88)
    moba = oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 0.45)
    B = slice(2 * L, 3 * L)
    ref, _ = dense_masked_softmax(q[B], k[B], v[B], np.ones((L, L), bool), 0.45)
    np.testing.assert_allclose(moba[B], ref, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# chunk-wise causal cross-attention
# ---------------------------------------------------------------------------------------------

def test_cross_attention_ignores_other_chunks_prompts():
    """I9: chunk i's output does not change when another chunk's local prompt changes."""
    H, D, ne, nl, nc = 2, 16, 7, 5, 4
    q = _rand((6, H, D), 90)
    ke, ve = _rand((ne, H, D), 91), _rand((ne, H, D), 92)
    kl = [_rand((nl, H, D), 100 + j) for j in range(nc)]
    vl = [_rand((nl, H, D), 200 + j) for j in range(nc)]
    a = oracle.cross_attention(q, 2, ke, ve, kl, vl, 0.25)
    kl2 = [x if j == 2 else x * 3 + 1 for j, x in enumerate(kl)]
    vl2 = [x if j == 2 else -x for j, x in enumerate(vl)]
    b = oracle.cross_attention(q, 2, ke, ve, kl2, vl2, 0.25)
    np.testing.assert_array_equal(a, b)
    c = oracle.chunk_attention(None, q, [(ke, ve), (kl[2], vl[2])], 0.25)
    np.testing.assert_allclose(a, c, atol=1e-12)
    allk = np.concatenate([ke] + kl)
    allv = np.concatenate([ve] + vl)
    m = np.zeros((6, allk.shape[0]), bool)
    m[:, :ne] = True
    m[:, ne + 2 * nl: ne + 3 * nl] = True
    ref, _ = dense_masked_softmax(q, allk, allv, m, 0.25)
    np.testing.assert_allclose(a, ref, atol=1e-12)


@settings(max_examples=150, deadline=None)
@given(cq=st.integers(1, 6), nc=st.integers(1, 6), ne=st.integers(0, 7), nl=st.integers(0, 7))
def test_cross_train_intervals_match_pairwise_rule(cq, nc, ne, nl):
    """X1 stated pairwise: row i (chunk c = i // cq) reads key j iff j is in the environment
    prompt or in chunk c's own local prompt; the generator's row intervals say the same."""
    n_k = ne + nc * nl
    want = np.array([[j < ne or ne + (i // cq) * nl <= j < ne + (i // cq + 1) * nl for j in range(n_k)]
                     for i in range(cq * nc)]).reshape(cq * nc, n_k)
    ivs = [oracle.cross_train_row_intervals(i, cq, ne, nl) for i in range(cq * nc)]
    np.testing.assert_array_equal(mask_from_intervals(ivs, n_k), want)


def _xtrain_case(seed, cq=3, nc=4, ne=2, nl=3, H=2, D=16):
    q = _rand((cq * nc, H, D), seed)
    k = _rand((ne + nc * nl, H, D), seed + 1)
    v = _rand((ne + nc * nl, H, D), seed + 2)
    return q, k, v


def test_cross_train_zero_query_gives_mean_of_env_and_own_prompt():
    """Closed form (C1) per chunk: q = 0 gives the plain mean of the values of
    the environment prompt and of the chunk's own local prompt."""
    cq, nc, ne, nl = 3, 4, 2, 3
    _, k, v = _xtrain_case(300, cq, nc, ne, nl)
    q = np.zeros((cq * nc,) + k.shape[1:], np.float32)
    out = oracle.cross_attention_train(q, k, v, cq, ne, nl, 0.3)
    for c in range(nc):
        allowed = np.concatenate([v[:ne], v[ne + c * nl: ne + (c + 1) * nl]]).astype(np.float64)
        for r in range(c * cq, (c + 1) * cq):
            np.testing.assert_allclose(out[r], allowed.mean(axis=0), atol=1e-12)


def test_cross_train_without_env_is_plain_attention_per_chunk():
    """No environment prompt: chunk c is textbook softmax attention of its
    queries over its own local prompt alone."""
    cq, nc, ne, nl, H, D = 3, 4, 0, 5, 2, 16
    q, k, v = _xtrain_case(310, cq, nc, ne, nl, H, D)
    out = oracle.cross_attention_train(q, k, v, cq, ne, nl, 0.25)
    for c in range(nc):
        for h in range(H):
            qc = q[c * cq:(c + 1) * cq, h].astype(np.float64)
            kc = k[c * nl:(c + 1) * nl, h].astype(np.float64)
            vc = v[c * nl:(c + 1) * nl, h].astype(np.float64)
            logits = 0.25 * qc @ kc.T
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(out[c * cq:(c + 1) * cq, h], p @ vc, atol=1e-12)


def test_cross_train_one_chunk_is_full_attention():
    """A single chunk reads every key: plain dense attention."""
    cq, ne, nl = 5, 4, 3
    q, k, v = _xtrain_case(320, cq, 1, ne, nl)
    out = oracle.cross_attention_train(q, k, v, cq, ne, nl, 0.3)
    ref, _ = dense_masked_softmax(q, k, v, np.ones((cq, ne + nl), bool), 0.3)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_cross_train_chunks_ignore_other_prompts_and_match_inference_form():
    """I9 in the training form: altering local prompt j changes only chunk j's
    rows; chunk c's rows equal the inference call of chunk c."""
    cq, nc, ne, nl, H, D = 3, 4, 2, 3, 2, 16
    q, k, v = _xtrain_case(330, cq, nc, ne, nl, H, D)
    a = oracle.cross_attention_train(q, k, v, cq, ne, nl, 0.25)
    for j in range(nc):
        k2, v2 = k.copy(), v.copy()
        k2[ne + j * nl: ne + (j + 1) * nl] *= -2
        v2[ne + j * nl: ne + (j + 1) * nl] += 1
        b = oracle.cross_attention_train(q, k2, v2, cq, ne, nl, 0.25)
        for c in range(nc):
            rows = slice(c * cq, (c + 1) * cq)
            if c == j:
                assert np.abs(a[rows] - b[rows]).max() > 1e-3
            else:
                np.testing.assert_array_equal(a[rows], b[rows])
    kl = [k[ne + c * nl: ne + (c + 1) * nl] for c in range(nc)]
    vl = [v[ne + c * nl: ne + (c + 1) * nl] for c in range(nc)]
    for c in range(nc):
        inf = oracle.cross_attention(q[c * cq:(c + 1) * cq], c, k[:ne], v[:ne], kl, vl, 0.25)
        np.testing.assert_allclose(a[c * cq:(c + 1) * cq], inf, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# input generator
# ---------------------------------------------------------------------------------------------

def test_generator_known_answers():
    """Philox4x32-10 known-answer vectors of the Random123 distribution."""
    kats = [((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
            ((0xffffffff,) * 4, (0xffffffff, 0xffffffff), (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
            ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
             (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1))]
    for ctr, key, want in kats:
        got = synth.philox4x32_10_np([np.array([c]) for c in ctr], key)
        assert [int(x[0]) for x in got] == list(want)
        assert synth.philox4x32_10_c(ctr, key).tolist() == list(want)


def test_generator_c_matches_numpy_and_moments():
    for kind in range(9):
        a = synth.normal_np(20000, seed=11, chunk=3, layer=7, step=2, kind=kind, start=1 << 33)
        b = synth.normal(20000, dtype="f32", seed=11, chunk=3, layer=7, step=2, kind=kind, start=1 << 33)
        np.testing.assert_array_equal(a, b)
        bb = synth.normal(20000, dtype="bf16", seed=11, chunk=3, layer=7, step=2, kind=kind, start=1 << 33)
        np.testing.assert_array_equal(bb, synth.f32_to_bf16_bits(a))
    x = synth.normal(1 << 20, dtype="f32", seed=0)
    assert abs(x.mean()) < 5e-3 and abs(x.var() - 65535 / 65536) < 5e-3
    assert x.min() >= -1530 / 256 and x.max() <= 1530 / 256


# ---------------------------------------------------------------------------------------------
# FP8 e4m3 quantization of QK^T
# ---------------------------------------------------------------------------------------------

def _e4m3_by_search(x):
    """Nearest finite e4m3 value by exhaustive search over the 126 positive magnitudes and
    zero; a tie goes to the even code."""
    mags = [(oracle.e4m3_value(np.uint8(c)).item(), c) for c in range(0x7F)]
    out = []
    for v in np.asarray(x, np.float32):
        a = abs(float(v))
        best = min(abs(a - m) for m, _ in mags)
        cands = [c for m, c in mags if abs(a - m) == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out.append(c | (0x80 if np.signbit(v) else 0))
    return np.array(out, np.uint8)


def test_e4m3_spec_values():
    """OCP FP8 e4m3 facts: 1.0 = 0x38, largest finite 448 = 0x7e, smallest normal 2^-6 =
    0x08, smallest subnormal 2^-9 = 0x01, 0x7f is NaN, the sign is the top bit."""
    v = oracle.e4m3_value(np.array([0x38, 0x7E, 0x08, 0x01, 0x7F, 0xB8, 0x00, 0x80], np.uint8))
    assert v[0] == 1.0 and v[1] == 448.0 and v[2] == 2.0 ** -6 and v[3] == 2.0 ** -9
    assert np.isnan(v[4]) and v[5] == -1.0 and v[6] == 0.0 and v[7] == 0.0 and np.signbit(v[7])
    finite = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.sum(np.isfinite(finite)) == 254
    pos = np.sort(finite[:0x7F])
    assert np.all(np.diff(pos) > 0)                    # 127 distinct non-negative values


def test_e4m3_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_round(oracle.e4m3_value(codes).astype(np.float32)), codes)


def test_e4m3_round_matches_nearest_value_search():
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    pos = np.sort(vals)
    mids = (pos[:-1] + pos[1:]) / 2                  # every tie, exactly representable in fp32
    rng = np.random.default_rng(0)
    x = np.concatenate([mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(1)),
                        np.nextafter(mids.astype(np.float32), np.float32(-1)),
                        rng.uniform(-448, 448, 2000), rng.standard_normal(2000) * 0.01,
                        rng.standard_normal(2000) * 2.0 ** -8, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_round(x), _e4m3_by_search(x))
    with pytest.raises(ValueError):
        oracle.e4m3_round(np.array([448.5], np.float32))


def test_quantize_blocks_scale_and_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((150, 3, 64)) * np.array([1.0, 1e-3, 300.0])[None, :, None]).astype(np.float32)
    x[64:128, 1] = 0.0                                  # an all-zero block
    codes, scales = oracle.quantize_e4m3_blocks(x, 64)
    assert codes.shape == (3, 3, 64, 64) and scales.shape == (3, 3)
    assert scales[1, 1] == 0 and not codes[1, 1].any()
    xd = oracle.dequantize_e4m3_blocks(codes, scales, 150)
    for b in range(3):
        for hh in range(3):
            blk = x[b * 64:(b + 1) * 64, hh]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert scales[b, hh] == np.float32(amax) / np.float32(448)
            assert np.abs(oracle.e4m3_value(codes[b, hh])).max() == 448.0    # the largest entry hits the top
            err = np.abs(xd[b * 64:(b + 1) * 64, hh] - blk)
            # half a quantum: 2^-4 relative in the normal range, 2^-10 * scale below it
            bound = np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * scales[b, hh]) * (1 + 1e-6)
            assert np.all(err <= bound)


def _lossless(shape, rows, seed):
    """Values that FP8 block quantization reproduces exactly: random e4m3 grid values with
    one entry per (block, head) at +-448, times a power of two per block."""
    rng = np.random.default_rng(seed)
    n, H, D = shape
    codes = rng.integers(0, 0x7E, size=shape).astype(np.uint8) | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    x = oracle.e4m3_value(codes)
    for b in range(-(-n // rows)):
        for hh in range(H):
            x[b * rows, hh, 0] = 448.0
            x[b * rows:(b + 1) * rows, hh] *= 2.0 ** int(rng.integers(-12, -4))
    return x.astype(np.float32)


def test_qk8_is_exact_on_losslessly_quantizable_inputs():
    """Per-block power-of-two scales make quantization exact, so the quantized path equals the
    plain attention; a wrong block partition (of Q rows, or of the time-ordered key sequence)
    would mix two blocks' scales and lose bits."""
    S, W, cf, tpf, H, D = 2, 3, 2, 24, 2, 64
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    for c in range(5):                                   # ring wrapped: slot order != time order
        cm.append(_rand((cf * tpf, H, D), 200 + c), _rand((cf * tpf, H, D), 210 + c), cf)
    assert list(cm.slot_map()) != sorted(cm.slot_map())
    nk = len(cm.resident()) * tpf
    kl = _lossless((nk + 40, H, D), 64, 3)               # the keys in time order, then a segment
    for i, f in enumerate(cm.resident()):
        cm.frames[f] = (kl[i * tpf:(i + 1) * tpf], cm.frames[f][1])
    seg_k, seg_v = kl[nk:], _rand((40, H, D), 220)
    q = _lossless((70, H, D), 32, 4)
    a = oracle.chunk_attention_qk8(cm, q, [(seg_k, seg_v)], 0.05)
    b = oracle.chunk_attention(cm, q, [(seg_k, seg_v)], 0.05)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # one extra key ahead of the segment shifts its rows against the 64-key blocks: lossy
    extra = [(np.full((1, H, D), 0.5, np.float32), seg_v[:1]), (seg_k, seg_v)]
    c = oracle.chunk_attention_qk8(cm, q, extra, 0.05)
    assert np.abs(c - oracle.chunk_attention(cm, q, extra, 0.05)).max() > 1e-9
    cm2_frames = dict(cm.frames)
    f0 = cm.resident()[0]
    kk = cm.frames[f0][0].copy()
    kk[0, :, 0] *= 3.0                                   # one key 3x larger: its block's scale moves
    cm.frames[f0] = (kk, cm.frames[f0][1])
    d = oracle.chunk_attention_qk8(cm, q, [(seg_k, seg_v)], 0.05)
    e = oracle.chunk_attention(cm, q, [(seg_k, seg_v)], 0.05)
    assert np.abs(d - e).max() > 1e-9
    cm.frames = cm2_frames
    # the same lossless keys laid out in slot order instead (what a block cut along the
    # ring's physical order would see) straddle the scale blocks differently: lossy
    valid = oracle.valid_slots(cm.F, S, W)
    for s_, f in enumerate(cm.slot_map()[:valid]):
        cm.frames[f] = (kl[s_ * tpf:(s_ + 1) * tpf], cm.frames[f][1])
    g = oracle.chunk_attention_qk8(cm, q, [(seg_k, seg_v)], 0.05)
    assert np.abs(g - oracle.chunk_attention(cm, q, [(seg_k, seg_v)], 0.05)).max() > 1e-9


def test_qk8_key_sequence_is_time_order():
    """The FP8 key sequence lists the resident frames oldest first (sinks, then the window),
    then the segments -- whatever slots the ring put them in."""
    S, W, cf, tpf, H, D = 2, 3, 2, 5, 1, 8
    cm = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    frames = {}
    for c in range(5):
        k, v = _rand((cf * tpf, H, D), 300 + c), _rand((cf * tpf, H, D), 310 + c)
        for j in range(cf):
            frames[c * cf + j] = (k[j * tpf:(j + 1) * tpf], v[j * tpf:(j + 1) * tpf])
        cm.append(k, v, cf)
    k, v = oracle.qk8_key_sequence(cm, [(np.ones((3, H, D), np.float32), np.zeros((3, H, D), np.float32))])
    # F = 10, S = 2, W = 3: sinks 0, 1 and the window 7, 8, 9 (slots 2 + (f - 2) % 3: 4, 2, 3)
    want = [0, 1, 7, 8, 9]
    assert [int(x) for x in cm.slot_map()] == [0, 1, 8, 9, 7]
    assert k.shape[0] == len(want) * tpf + 3
    for i, f in enumerate(want):
        np.testing.assert_array_equal(k[i * tpf:(i + 1) * tpf], frames[f][0])
        np.testing.assert_array_equal(v[i * tpf:(i + 1) * tpf], frames[f][1])
    np.testing.assert_array_equal(k[-3:], 1.0)


def test_qk8_depends_on_resident_frames_not_ring_phase():
    """Two caches holding the same frame contents, appended so that their rings wrap at
    different slots, give bit-identical quantized attention."""
    S, W, cf, tpf, H, D = 2, 4, 2, 40, 2, 64
    chunks = [(_rand((cf * tpf, H, D), 500 + c), _rand((cf * tpf, H, D), 520 + c)) for c in range(5)]
    a = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    b = oracle.CacheModel(S, W, tpf, H, D, dtype=np.float32)
    for c in (0, 1, 2, 3):        # F = 8: sinks from chunk 0, window = chunks 2, 3
        a.append(*chunks[c], cf)
    for c in (0, 4, 4, 2, 3):     # F = 10: the same sinks and window, ring shifted by 2
        b.append(*chunks[c], cf)
    assert list(a.slot_map()) != list(b.slot_map())
    ka, va = a.logical_kv()
    kb, vb = b.logical_kv()
    np.testing.assert_array_equal(ka, kb)
    np.testing.assert_array_equal(va, vb)
    q = _rand((50, H, D), 540)
    seg = (_rand((30, H, D), 541), _rand((30, H, D), 542))
    np.testing.assert_array_equal(oracle.chunk_attention_qk8(a, q, [seg], 0.1),
                                  oracle.chunk_attention_qk8(b, q, [seg], 0.1))


def test_dense_f64_attention_matches_c_core():
    q, k, v = _rand((9, 3, 32), 400), _rand((50, 3, 32), 401), _rand((50, 3, 32), 402)
    a = oracle.attend_dense_f64(q, k, v, 0.3)
    b = oracle.attend(q, k, v, [[(0, 50)]] * 9, 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_qk8_error_against_exact_attention_is_small():
    """The quantization error itself, at N(0,1) inputs with a 832x464-like key count per
    head (cache + current chunk, 2 heads): the looser bound of the quantized path."""
    S, W, cf, tpf, H, D = 6, 8, 4, 48, 2, 128
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for c in range(5):
        cm.append(synth.normal(cf * tpf * H * D, seed=9, chunk=c, kind=synth.KFIN).reshape(cf * tpf, H, D),
                  synth.normal(cf * tpf * H * D, seed=9, chunk=c, kind=synth.VFIN).reshape(cf * tpf, H, D), cf)
    q, k, v = (synth.normal(cf * tpf * H * D, seed=10, kind=t).reshape(cf * tpf, H, D)
               for t in (synth.Q, synth.K, synth.V))
    a = oracle.chunk_attention_qk8(cm, q, [(k, v)], 1 / np.sqrt(D))
    b = oracle.chunk_attention(cm, q, [(k, v)], 1 / np.sqrt(D))
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel < QK8_REL_L2_VS_EXACT, rel
    assert np.abs(a - b).max() < QK8_MAX_ABS_VS_EXACT


# bounds of the quantized path against exact attention (N(0,1) inputs, D = 128): e4m3 keeps
# 3 mantissa bits, so each score carries an error of a few percent of its magnitude
QK8_REL_L2_VS_EXACT = 0.1
QK8_MAX_ABS_VS_EXACT = 0.05


# ---------------------------------------------------------------------------------------------
# MoBA backward: gradients against central finite differences of the forward (C fp64 core)
# ---------------------------------------------------------------------------------------------

def _grid(shape, seed):
    """Values on a 2^-10 grid in (-4, 4): q +- 2^-12 stays exact in fp32."""
    rng = np.random.default_rng(seed)
    return (np.round(rng.standard_normal(shape) * 1024) / 1024).clip(-3.9, 3.9).astype(np.float32)


@pytest.mark.parametrize("tpf,frames,cf,bidir", [(2, 3, 1, 1), (1, 4, 2, 0), (3, 2, 1, 1)])
def test_moba_backward_matches_finite_differences(tpf, frames, cf, bidir):
    H, D, scale, h = 2, 8, 0.35, 2.0 ** -12
    n = (2 + bidir) * frames * tpf
    q, k, v = _grid((n, H, D), 1), _grid((n, H, D), 2), _grid((n, H, D), 3)
    do = _rand((n, H, D), 4).astype(np.float64)
    ivs = [oracle.moba_row_intervals(i, tpf, frames, cf, bidir) for i in range(n)]

    def loss(qq, kk, vv):
        return float((oracle.attend(qq, kk, vv, ivs, scale) * do).sum())

    dq, dk, dv = oracle.moba_attention_backward(q, k, v, do.astype(np.float32), tpf, frames, cf, bidir, scale)
    do = do.astype(np.float32).astype(np.float64)       # the gradients were taken for the fp32 dO
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros(x.shape)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=2e-6 * max(1.0, np.abs(fd).max()), err_msg=name)


def test_backward_identities_and_empty_rows():
    """Softmax is invariant to a shift of all of a row's keys (sum_j dK_j = 0) and its rows sum
    to one (sum_j dV_j = sum of dO over rows that have keys); a row with no key gets dq = 0."""
    n, H, D = 12, 2, 16
    q, k, v, do = (_rand((n, H, D), 50 + i) for i in range(4))
    mask = np.tril(np.ones((n, n), bool))
    mask[5] = False                                       # row 5 sees nothing
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask, 0.25)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    has = mask.any(axis=1)
    np.testing.assert_allclose(dv.sum(axis=0), do[has].astype(np.float64).sum(axis=0), atol=1e-12)
    assert not dq[5].any()


def test_lse_matches_c_probabilities():
    n, H, D = 10, 2, 16
    q, k = _rand((n, H, D), 60), _rand((n, H, D), 61)
    ivs = [oracle.moba_row_intervals(i, 2, 5, 2, 0) for i in range(n)]
    mask = oracle.mask_from_row_intervals(ivs, n)
    lse = oracle.attention_lse(q, k, mask, 0.3)
    _, probs = oracle.attend(q, k, np.zeros_like(k), ivs, 0.3, want_probs=True)   # [nq][H][nk]
    s = np.einsum("ihd,jhd->hij", q.astype(np.float64), k.astype(np.float64)) * 0.3
    p = np.where(mask[None], np.exp(s - lse[:, :, None]), 0.0)
    np.testing.assert_allclose(p.transpose(1, 0, 2), probs, atol=1e-14)



@pytest.mark.parametrize("tpf,frames,cf,bidir", [(4, 6, 2, 1), (7, 5, 3, 0), (5, 4, 1, 1)])
def test_key_gradients_match_the_dense_backward(tpf, frames, cf, bidir):
    """The streamed per-key gradients (each row's softmax over its own allowed keys, rows in
    runs of equal intervals) equal the dense masked backward's dk and dv rows."""
    n = (2 + bidir) * frames * tpf
    H, D = 2, 16
    q, k, v, do = (_rand((n, H, D), 600 + i) for i in range(4))
    rq, rk, rv = oracle.attention_backward(q, k, v, do, oracle.moba_mask(tpf, frames, cf, bidir), 0.3)
    rng = np.random.default_rng(7)
    keys = np.array(sorted(rng.choice(n, size=min(n, 17), replace=False)))
    ivs = lambda i: oracle.moba_row_intervals(i, tpf, frames, cf, bidir)
    gk, gv = oracle.attention_key_gradients(q, k, v, do, ivs, keys, 0.3, block=5)
    np.testing.assert_allclose(gk, rk[keys], rtol=0, atol=1e-12 * max(1.0, np.abs(rk).max()))
    np.testing.assert_allclose(gv, rv[keys], rtol=0, atol=1e-12 * max(1.0, np.abs(rv).max()))
    # every key at once, in a shuffled order
    allk = rng.permutation(n)
    gk, gv = oracle.attention_key_gradients(q, k, v, do, ivs, allk, 0.3, block=64)
    np.testing.assert_allclose(gk, rk[allk], rtol=0, atol=1e-12 * max(1.0, np.abs(rk).max()))
    np.testing.assert_allclose(gv, rv[allk], rtol=0, atol=1e-12 * max(1.0, np.abs(rv).max()))



@pytest.mark.parametrize("tpf,frames,cf,bidir", [(4, 6, 2, 1), (7, 5, 3, 0)])
def test_attention_by_runs_matches_the_c_core(tpf, frames, cf, bidir):
    """The BLAS-blocked, run-by-run masked attention equals the C core row by row: MoBA
    masks, the cross-attention training mask, and an unmasked call with a ragged block."""
    n = (2 + bidir) * frames * tpf
    H, D = 3, 16
    q, k, v = (_rand((n, H, D), 700 + i) for i in range(3))
    ivs = lambda i: oracle.moba_row_intervals(i, tpf, frames, cf, bidir)
    a = oracle.attention_by_runs(q, k, v, ivs, 0.4, block=7)
    b = oracle.attend(q, k, v, [ivs(i) for i in range(n)], 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    a = oracle.attention_by_runs(q, k, v, ivs, 0.4, heads=[2, 0], block=64)
    np.testing.assert_allclose(a, b[:, [2, 0]], rtol=0, atol=1e-12)
    xi = lambda i: oracle.cross_train_row_intervals(i, 9, 5, 4)
    kx, vx = _rand((5 + 4 * (n // 9 + 1), H, D), 710), _rand((5 + 4 * (n // 9 + 1), H, D), 711)
    a = oracle.attention_by_runs(q[:9 * (n // 9)], kx, vx, xi, 0.4, block=4)
    b = oracle.attend(q[:9 * (n // 9)], kx, vx, [xi(i) for i in range(9 * (n // 9))], 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    a = oracle.attention_by_runs(q, k, v, lambda i: [(0, n)], 0.4, block=13)
    np.testing.assert_allclose(a, oracle.attend(q, k, v, [[(0, n)]] * n, 0.4), rtol=0, atol=1e-12)
