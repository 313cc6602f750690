"""The C ABI on the host, without a GPU: exported symbols, argument checks and
status codes, no state change on error, and the host-side bookkeeping and
launch planning (through the WMK_DRY_RUN hook, which plans every call and logs
each launch instead of enqueueing it)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import kv_cache_attention_02_amd as wmk
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wmk.h")

# fake, 16-byte aligned "device" addresses: only ever checked, never dereferenced on these paths
KBUF, VBUF, QBUF, OBUF, SBUF = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(wmk.LIB_PATH):
        from kv_cache_attention_02_amd import build
        build.build()
    return wmk.load()


@pytest.fixture
def dry(tmp_path, monkeypatch):
    path = tmp_path / "launches.log"
    monkeypatch.setenv("WMK_DRY_RUN", str(path))
    return path


def _desc(L=1, H=12, D=128, tpf=1508, S=6, W=8, cf=4, dtype=wmk.WMK_BF16):
    return wmk.wmk_cache_desc(L, H, D, tpf, S, W, cf, dtype)


def _init(lib, d, k=KBUF, v=VBUF, cap=None):
    h = ctypes.c_void_p()
    cap = lib.wmk_cache_bytes(ctypes.byref(d)) if cap is None else cap
    st = lib.wmk_cache_init(ctypes.byref(d), k, v, cap, ctypes.byref(h))
    return st, h


def _slots(lib, h, layer, n):
    arr = (ctypes.c_int64 * n)()
    F = ctypes.c_int64()
    assert lib.wmk_cache_slots(h, layer, arr, ctypes.byref(F)) == wmk.WMK_OK
    return list(arr), F.value


def test_library_exports_every_header_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^[A-Za-z_][\w \*]*?\b(wmk_\w+)\s*\(", text, flags=re.M))
    assert declared == set(wmk.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_cache_bytes(lib):
    d = _desc(L=30)
    assert lib.wmk_cache_bytes(ctypes.byref(d)) == 30 * 14 * 1508 * 12 * 128 * 2
    d = _desc(L=1, H=1, D=64, tpf=16, S=1, W=2, cf=2, dtype=wmk.WMK_F32)
    assert lib.wmk_cache_bytes(ctypes.byref(d)) == 3 * 16 * 64 * 4
    for bad in (_desc(D=96), _desc(W=0), _desc(S=-1), _desc(L=0), _desc(dtype=7), _desc(tpf=0)):
        assert lib.wmk_cache_bytes(ctypes.byref(bad)) == 0
    assert lib.wmk_cache_bytes(None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), wmk.WMK_ERR_SHAPE), (dict(W=0), wmk.WMK_ERR_SHAPE), (dict(H=0), wmk.WMK_ERR_SHAPE),
    (dict(H=4097), wmk.WMK_ERR_SHAPE),
    (dict(dtype=5), wmk.WMK_ERR_DTYPE), (dict(S=-2), wmk.WMK_ERR_SHAPE), (dict(cf=0), wmk.WMK_ERR_SHAPE),
])
def test_init_rejects_bad_descriptor(lib, kw, status):
    d = _desc(**kw)
    h = ctypes.c_void_p(0x1234)
    st = lib.wmk_cache_init(ctypes.byref(d), KBUF, VBUF, 1 << 40, ctypes.byref(h))
    assert st == status
    assert h.value == 0x1234          # untouched
    assert lib.wmk_last_error()


def test_init_pointer_checks(lib):
    d = _desc()
    assert _init(lib, d, k=0)[0] == wmk.WMK_ERR_NULL
    assert _init(lib, d, k=KBUF + 8)[0] == wmk.WMK_ERR_ALIGN
    assert _init(lib, d, cap=lib.wmk_cache_bytes(ctypes.byref(d)) - 1)[0] == wmk.WMK_ERR_CAPACITY
    assert lib.wmk_cache_init(None, KBUF, VBUF, 1 << 40, None) == wmk.WMK_ERR_NULL
    st, h = _init(lib, d)
    assert st == wmk.WMK_OK and lib.wmk_last_error() == b""
    assert _slots(lib, h, 0, 14) == ([-1] * 14, 0)
    lib.wmk_cache_destroy(h)
    lib.wmk_cache_destroy(None)


def test_append_argument_errors_leave_state(lib, dry):
    d = _desc(L=2)
    _, h = _init(lib, d)
    assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 4, None) == wmk.WMK_OK
    before = _slots(lib, h, 0, 14)
    cases = [((None, 0, QBUF, SBUF, 4), wmk.WMK_ERR_NULL), ((h, 2, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE),
             ((h, -1, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE), ((h, 0, QBUF, SBUF, 0), wmk.WMK_ERR_SHAPE),
             ((h, 0, QBUF + 4, SBUF, 4), wmk.WMK_ERR_ALIGN), ((h, 0, None, SBUF, 4), wmk.WMK_ERR_NULL)]
    for args, status in cases:
        assert lib.wmk_cache_append_evict(*args, None) == status
        assert lib.wmk_last_error()
    assert _slots(lib, h, 0, 14) == before
    assert _slots(lib, h, 1, 14) == ([-1] * 14, 0)
    lib.wmk_cache_destroy(h)


def test_refused_launch_does_not_advance_state(lib, monkeypatch):
    monkeypatch.setenv("WMK_FAULT_INJECT", "1")
    d = _desc()
    _, h = _init(lib, d)
    assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 4, None) == wmk.WMK_ERR_HIP
    assert _slots(lib, h, 0, 14) == ([-1] * 14, 0)
    assert lib.wmk_cache_append_evict_layers(h, 0, 1, QBUF, SBUF, 4, None) == wmk.WMK_ERR_HIP
    assert _slots(lib, h, 0, 14) == ([-1] * 14, 0)
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    seg = (wmk.wmk_kv_segment * 1)(wmk.wmk_kv_segment(QBUF, SBUF, 6032))
    assert lib.wmk_chunk_attention(h, 0, ctypes.byref(hd), QBUF, 6032, seg, 1, OBUF, 0.088, None, 0,
                                   None) == wmk.WMK_ERR_HIP
    lib.wmk_cache_destroy(h)


@pytest.mark.parametrize("S,W,cf,n_appends", [(6, 8, 4, 20), (1, 2, 2, 8), (0, 3, 1, 10), (2, 5, 3, 9),
                                              (3, 1, 2, 6), (4, 4, 4, 7), (2, 3, 5, 5), (0, 1, 3, 4)])
def test_append_plan_matches_oracle_policy(lib, dry, S, W, cf, n_appends):
    """Every planned copy writes exactly the frames the oracle keeps, into the
    oracle's slots, in at most three contiguous ranges; the host slot map
    equals the oracle's after every append."""
    tpf, H, D = 3, 2, 64
    fb = tpf * H * D * 2
    d = _desc(L=2, H=H, D=D, tpf=tpf, S=S, W=W, cf=cf)
    _, h = _init(lib, d)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    layer_bytes = (S + W) * fb
    held = {}
    for a in range(n_appends):
        F = cm.F
        assert lib.wmk_cache_append_evict(h, 1, QBUF, SBUF, cf, None) == wmk.WMK_OK
        line = dry.read_text().strip().splitlines()[-1]
        head, *ranges = line.split(" ")[0:1] + line.split(" ")[5:]
        assert line.startswith(f"append layer=1 F={F} n={cf} ranges={len(ranges)}")
        assert 1 <= len(ranges) <= 3
        written = {}
        for r in ranges:
            src, dst, nb = (int(x) for x in r.split(":"))
            assert src % fb == 0 and (dst - layer_bytes) % fb == 0 and nb % fb == 0
            for i in range(nb // fb):
                written[(dst - layer_bytes) // fb + i] = F + src // fb + i
        assert sorted(written.values()) == oracle.frames_kept_by_append(F, cf, S, W)
        for slot, frame in written.items():
            assert slot == oracle.slot_of_frame(frame, S, W)
        held.update(written)
        cm.append(np.zeros((cf * tpf, H, D), np.uint16), np.zeros((cf * tpf, H, D), np.uint16), cf)
        slots, Fh = _slots(lib, h, 1, S + W)
        assert Fh == cm.F
        assert slots == cm.slot_map().tolist()
        assert all(held[s] == f for s, f in enumerate(slots) if f >= 0)
    assert _slots(lib, h, 0, S + W) == ([-1] * (S + W), 0)
    lib.wmk_cache_destroy(h)


@pytest.mark.parametrize("S,W,cf,n_appends", [(6, 8, 4, 8), (0, 3, 1, 7), (2, 3, 5, 4), (3, 1, 2, 5)])
def test_append_layers_plan_equals_per_layer_appends(lib, dry, S, W, cf, n_appends):
    """One multi-layer append plans the same ranges as wmk_cache_append_evict on its first
    layer, with sources one [n_frames * tpf] block and destinations one layer apart, and
    leaves every layer of the run with the oracle's slot map; layers outside the run are
    untouched."""
    tpf, H, D = 3, 2, 64
    fb = tpf * H * D * 2
    d = _desc(L=5, H=H, D=D, tpf=tpf, S=S, W=W, cf=cf)
    _, h = _init(lib, d)
    _, h1 = _init(lib, d)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for a in range(n_appends):
        F = cm.F
        assert lib.wmk_cache_append_evict(h1, 1, QBUF, SBUF, cf, None) == wmk.WMK_OK
        single = dry.read_text().strip().splitlines()[-1].split(" ")
        assert lib.wmk_cache_append_evict_layers(h, 1, 3, QBUF, SBUF, cf, None) == wmk.WMK_OK
        multi = dry.read_text().strip().splitlines()[-1].split(" ")
        assert multi[:8] == ["append_layers", "first=1", "layers=3", f"F={F}", f"n={cf}", single[4],
                             f"src_stride={cf * fb}", f"dst_stride={(S + W) * fb}"]
        assert multi[8:] == single[5:]
        cm.append(np.zeros((cf * tpf, H, D), np.uint16), np.zeros((cf * tpf, H, D), np.uint16), cf)
        for layer in (1, 2, 3):
            assert _slots(lib, h, layer, S + W) == (cm.slot_map().tolist(), cm.F)
        for layer in (0, 4):
            assert _slots(lib, h, layer, S + W) == ([-1] * (S + W), 0)
    lib.wmk_cache_destroy(h)
    lib.wmk_cache_destroy(h1)


def test_append_layers_argument_errors_leave_state(lib, dry):
    d = _desc(L=4)
    _, h = _init(lib, d)
    assert lib.wmk_cache_append_evict_layers(h, 0, 4, QBUF, SBUF, 4, None) == wmk.WMK_OK
    assert lib.wmk_cache_append_evict(h, 3, QBUF, SBUF, 4, None) == wmk.WMK_OK   # layer 3 now one chunk ahead
    before = [_slots(lib, h, layer, 14) for layer in range(4)]
    cases = [((None, 0, 2, QBUF, SBUF, 4), wmk.WMK_ERR_NULL), ((h, 0, 2, None, SBUF, 4), wmk.WMK_ERR_NULL),
             ((h, 0, 0, QBUF, SBUF, 4), wmk.WMK_ERR_SHAPE), ((h, 0, 2, QBUF, SBUF, 0), wmk.WMK_ERR_SHAPE),
             ((h, -1, 2, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE), ((h, 3, 2, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE),
             ((h, 4, 1, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE), ((h, 2, 2, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE),
             ((h, 0, 4, QBUF, SBUF, 4), wmk.WMK_ERR_RANGE), ((h, 0, 2, QBUF + 4, SBUF, 4), wmk.WMK_ERR_ALIGN)]
    n_before = len(dry.read_text().splitlines())
    for args, status in cases:
        assert lib.wmk_cache_append_evict_layers(*args, None) == status, args
        assert lib.wmk_last_error()
    assert len(dry.read_text().splitlines()) == n_before   # nothing planned or launched
    assert [_slots(lib, h, layer, 14) for layer in range(4)] == before
    assert lib.wmk_cache_append_evict_layers(h, 0, 3, QBUF, SBUF, 4, None) == wmk.WMK_OK   # layers in step
    assert [_slots(lib, h, layer, 14)[1] for layer in range(4)] == [8, 8, 8, 8]
    lib.wmk_cache_destroy(h)


def test_append_longer_than_window_skips_overwritten_frames(lib, dry):
    S, W, tpf, H, D = 2, 3, 1, 1, 64
    d = _desc(H=H, D=D, tpf=tpf, S=S, W=W, cf=9)
    _, h = _init(lib, d)
    assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 9, None) == wmk.WMK_OK
    slots, F = _slots(lib, h, 0, S + W)
    assert F == 9
    cm = oracle.CacheModel(S, W, tpf, H, D)
    cm.append(np.zeros((9, H, D), np.uint16), np.zeros((9, H, D), np.uint16), 9)
    # frames 2..5 are skipped; 6, 7, 8 land in window slots 3, 4, 2
    assert slots == cm.slot_map().tolist() == [0, 1, 8, 6, 7]
    line = dry.read_text().strip().splitlines()[-1]
    assert line.startswith("append layer=0 F=0 n=9 ranges=3")


def _attn(lib, h, layer, hd, nq, segs, scale=0.088, q=QBUF, out=OBUF, ws=None, wsb=0):
    arr = (wmk.wmk_kv_segment * max(1, len(segs)))(*[wmk.wmk_kv_segment(k, v, t) for k, v, t in segs])
    return lib.wmk_chunk_attention(h, layer, ctypes.byref(hd) if hd is not None else None, q, nq, arr, len(segs),
                                   out, scale, ws, wsb, None)


def test_chunk_attention_argument_errors(lib, dry):
    d = _desc()
    _, h = _init(lib, d)
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    cur = [(QBUF, SBUF, 6032)]
    assert _attn(lib, h, 0, hd, 6032, cur) == wmk.WMK_OK
    bad = [
        (dict(hd=None), wmk.WMK_ERR_NULL),
        (dict(hd=wmk.wmk_head_desc(12, 96, wmk.WMK_BF16)), wmk.WMK_ERR_SHAPE),
        (dict(hd=wmk.wmk_head_desc(8, 128, wmk.WMK_BF16)), wmk.WMK_ERR_SHAPE),
        (dict(hd=wmk.wmk_head_desc(12, 128, wmk.WMK_F32)), wmk.WMK_ERR_DTYPE),
        (dict(hd=wmk.wmk_head_desc(12, 128, 9)), wmk.WMK_ERR_DTYPE),
        (dict(nq=0), wmk.WMK_ERR_SHAPE),
        (dict(segs=[(QBUF, SBUF, 0)]), wmk.WMK_ERR_SHAPE),
        (dict(segs=[(QBUF, SBUF, 8)] * 5), wmk.WMK_ERR_SHAPE),
        (dict(segs=[(0, SBUF, 8)]), wmk.WMK_ERR_NULL),
        (dict(segs=[(QBUF + 2, SBUF, 8)]), wmk.WMK_ERR_ALIGN),
        (dict(scale=0.0), wmk.WMK_ERR_RANGE), (dict(scale=-1.0), wmk.WMK_ERR_RANGE),
        (dict(scale=math.inf), wmk.WMK_ERR_RANGE), (dict(scale=math.nan), wmk.WMK_ERR_RANGE),
        (dict(layer=1), wmk.WMK_ERR_RANGE), (dict(layer=-1), wmk.WMK_ERR_RANGE),
        (dict(q=QBUF + 8), wmk.WMK_ERR_ALIGN), (dict(out=0), wmk.WMK_ERR_NULL),
    ]
    for kw, status in bad:
        args = dict(layer=0, hd=hd, nq=6032, segs=cur)
        args.update(kw)
        n_before = len(dry.read_text().splitlines())
        st = _attn(lib, h, args.pop("layer"), args.pop("hd"), args.pop("nq"), args.pop("segs"), **args)
        assert st == status, (kw, st)
        assert len(dry.read_text().splitlines()) == n_before   # nothing planned or launched
    lib.wmk_cache_destroy(h)


def _last_attn(dry):
    lines = [x for x in dry.read_text().splitlines() if x.startswith("attn")]
    return dict(kv.split("=") for kv in lines[-1].split(" ")[1:])


def test_plan_of_the_18_slot_step(lib, dry):
    """832x464 step with a warm cache: 14 resident frames + the 4-frame chunk = 27144 keys;
    q-tiles of the kernel's block size x 12 heads; with workspace, the units past the last full
    round of 256 CUs (one workgroup each in the dry-run device model) are split over the GPU."""
    d = _desc()
    _, h = _init(lib, d)
    for _ in range(4):
        assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 4, None) == wmk.WMK_OK
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    assert _attn(lib, h, 0, hd, 6032, [(QBUF, SBUF, 6032)]) == wmk.WMK_OK
    p = _last_attn(dry)
    bq = int(p["bq"])
    qtiles = (6032 + bq - 1) // bq
    assert (p["kv"], p["units"], p["qtiles"], p["split_units"]) == ("27144", str(12 * qtiles), str(qtiles), "0")
    wsb = lib.wmk_attention_workspace_bytes(ctypes.byref(hd), 6032)
    assert wsb > 0
    assert _attn(lib, h, 0, hd, 6032, [(QBUF, SBUF, 6032)], ws=0x60000000, wsb=wsb) == wmk.WMK_OK
    p = _last_attn(dry)
    tail = (12 * qtiles) % 256
    assert int(p["split_units"]) == tail
    assert int(p["splits"]) == min(256 // tail, (27144 + 63) // 64 // 8)
    # too little workspace: no split
    assert _attn(lib, h, 0, hd, 6032, [(QBUF, SBUF, 6032)], ws=0x60000000, wsb=wsb // 4) == wmk.WMK_OK
    assert _last_attn(dry)["split_units"] == "0"
    # empty cache and no segment: planned, zero keys
    _, h2 = _init(lib, d)
    assert _attn(lib, h2, 0, hd, 100, []) == wmk.WMK_OK
    assert _last_attn(dry)["kv"] == "0"
    lib.wmk_cache_destroy(h)
    lib.wmk_cache_destroy(h2)


def test_short_units_plan_the_four_wave_kernel(lib, dry):
    """Calls whose units walk at most 32 key tiles (bf16, head_dim 128, no MoBA mask) are
    planned for the 4-wave kernel (128-row q-tiles, two workgroups per CU); longer walks,
    head_dim 64 and the MoBA mask keep the 8-wave kernel (256-row q-tiles). The workspace
    query covers both shapes."""
    hd = wmk.wmk_head_desc(24, 128, wmk.WMK_BF16)
    # 720p cross-attention: 14400 queries over a 512-token environment + a 512-token local prompt
    segs = [(KBUF, VBUF, 512), (QBUF, SBUF, 512)]
    assert _attn(lib, None, 0, hd, 14400, segs) == wmk.WMK_OK
    p = _last_attn(dry)
    assert (p["bq"], p["qtiles"], p["units"]) == ("128", str(-(-14400 // 128)), str(24 * -(-14400 // 128)))
    # 32 tiles (2048 keys): still short; 33 tiles: long
    assert _attn(lib, None, 0, hd, 14400, [(KBUF, VBUF, 2048)]) == wmk.WMK_OK
    assert _last_attn(dry)["bq"] == "128"
    assert _attn(lib, None, 0, hd, 14400, [(KBUF, VBUF, 2049)]) == wmk.WMK_OK
    assert _last_attn(dry)["bq"] == "256"
    # head_dim 64 keeps the 8-wave kernel
    hd64 = wmk.wmk_head_desc(24, 64, wmk.WMK_BF16)
    assert _attn(lib, None, 0, hd64, 14400, segs) == wmk.WMK_OK
    assert _last_attn(dry)["bq"] == "256"
    # the cross-attention training mask: 512 + 512 keys per row
    xd = wmk.wmk_xattn_desc(4680, 7, 512, 512)
    hd12 = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd12), QBUF, KBUF, VBUF, OBUF, 0.088, None,
                                         0, None) == wmk.WMK_OK
    assert _last_attn(dry)["bq"] == "128"
    # MoBA keeps the 8-wave kernel whatever its tile counts
    md = wmk.wmk_moba_desc(40, 3, 1, 1)
    assert lib.wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd12), QBUF, KBUF, VBUF, OBUF, 0.088, None) == \
        wmk.WMK_OK
    assert _last_attn(dry)["bq"] == "256"
    # one workspace size serves both shapes: with it the short call splits its tail
    wsb = lib.wmk_attention_workspace_bytes(ctypes.byref(hd), 14400)
    assert _attn(lib, None, 0, hd, 14400, segs, ws=0x60000000, wsb=wsb) == wmk.WMK_OK
    p = _last_attn(dry)
    units = 24 * -(-14400 // 128)  # 2712 units over 512 slots (two 4-wave workgroups per CU): 152 left over
    assert p["bq"] == "128" and int(p["split_units"]) == units % 512 and int(p["splits"]) == min(512 // 152, 16 // 8)


def _oracle_qtile_cost(qt, tpf, frames, cf, bq, bk=64):
    n = 3 * frames * tpf
    tiles = set()
    for i in range(qt * bq, min((qt + 1) * bq, n)):
        for a, b in oracle.moba_row_intervals(i, tpf, frames, cf):
            tiles.update(range(a // bk, (b + bk - 1) // bk))
    return len(tiles)


@pytest.mark.parametrize("tpf,frames,cf", [(1560, 21, 3), (40, 7, 3), (200, 5, 2)])
def test_moba_launch_order_is_longest_first(lib, dry, tpf, frames, cf):
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    md = wmk.wmk_moba_desc(tpf, frames, cf, 1)
    assert lib.wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.088,
                                  None) == wmk.WMK_OK
    n = 3 * frames * tpf
    p = _last_attn(dry)
    bq = int(p["bq"])
    nqt = (n + bq - 1) // bq
    assert int(p["q"]) == n and int(p["qtiles"]) == nqt and int(p["groups"]) > 0
    groups = [tuple(int(x) for x in ln.split()[1:]) for ln in dry.read_text().splitlines() if ln.startswith("group")]
    groups = groups[-int(p["groups"]):]
    order = [s + i for s, c in groups for i in range(c)]
    assert sorted(order) == list(range(nqt))
    step = 1 if nqt < 200 else 7
    sample = order[::step]
    costs = [_oracle_qtile_cost(qt, tpf, frames, cf, bq) for qt in sample]
    assert all(a >= b for a, b in zip(costs, costs[1:]))


def test_moba_argument_errors(lib, dry):
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    for md, status in [(wmk.wmk_moba_desc(0, 21, 3, 1), wmk.WMK_ERR_SHAPE),
                       (wmk.wmk_moba_desc(1560, 21, 3, 2), wmk.WMK_ERR_SHAPE),
                       (wmk.wmk_moba_desc(1560, 0, 3, 1), wmk.WMK_ERR_SHAPE),
                       (wmk.wmk_moba_desc(1 << 20, 1 << 12, 3, 1), wmk.WMK_ERR_SHAPE)]:
        assert lib.wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.088,
                                      None) == status
    md = wmk.wmk_moba_desc(1560, 21, 3, 1)
    assert lib.wmk_moba_attention(None, ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.1, None) == \
        wmk.WMK_ERR_NULL
    assert lib.wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd), QBUF, 0, VBUF, OBUF, 0.1, None) == \
        wmk.WMK_ERR_NULL
    assert lib.wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.0, None) \
        == wmk.WMK_ERR_RANGE


def test_cross_train_argument_errors_and_plan(lib, dry):
    """Chunk-causal cross-attention over a multi-chunk sequence: bad descriptors are
    refused before anything is planned; a valid call plans the cross mask over
    q = chunks * chunk_q_tokens rows and env + chunks * local keys, and splits the
    last round when workspace is given (every q-tile visits the same key tiles)."""
    hd = wmk.wmk_head_desc(24, 128, wmk.WMK_BF16)
    bad = [(wmk.wmk_xattn_desc(0, 4, 512, 512), wmk.WMK_ERR_SHAPE),
           (wmk.wmk_xattn_desc(14400, 0, 512, 512), wmk.WMK_ERR_SHAPE),
           (wmk.wmk_xattn_desc(14400, 4, -1, 512), wmk.WMK_ERR_SHAPE),
           (wmk.wmk_xattn_desc(14400, 4, 512, -1), wmk.WMK_ERR_SHAPE),
           (wmk.wmk_xattn_desc(14400, 4, 0, 0), wmk.WMK_ERR_SHAPE),
           (wmk.wmk_xattn_desc(1 << 20, 1 << 12, 512, 512), wmk.WMK_ERR_SHAPE)]
    for xd, status in bad:
        n_before = len(dry.read_text().splitlines()) if dry.exists() else 0
        assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.088,
                                             None, 0, None) == status
        assert (len(dry.read_text().splitlines()) if dry.exists() else 0) == n_before
    xd = wmk.wmk_xattn_desc(14400, 4, 512, 512)
    assert lib.wmk_cross_attention_train(None, ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.1, None, 0, None) == \
        wmk.WMK_ERR_NULL
    assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF, KBUF, 0, OBUF, 0.1, None, 0,
                                         None) == wmk.WMK_ERR_NULL
    assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF + 4, KBUF, VBUF, OBUF, 0.1, None,
                                         0, None) == wmk.WMK_ERR_ALIGN
    assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, -1.0, None, 0,
                                         None) == wmk.WMK_ERR_RANGE
    assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.088, None, 0,
                                         None) == wmk.WMK_OK
    p = _last_attn(dry)
    bq = int(p["bq"])
    qtiles = (4 * 14400 + bq - 1) // bq
    assert (p["mask"], p["q"], p["kv"], p["qtiles"], p["units"], p["split_units"]) == \
        ("2", str(4 * 14400), str(512 + 4 * 512), str(qtiles), str(24 * qtiles), "0")
    wsb = lib.wmk_attention_workspace_bytes(ctypes.byref(hd), 4 * 14400)
    assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.088,
                                         0x60000000, wsb, None) == wmk.WMK_OK
    p = _last_attn(dry)
    slots = 256 * (2 if bq == 128 else 1)  # dry-run device: one 8-wave or two 4-wave workgroups per CU
    tail = (24 * qtiles) % slots
    # 8 + 8 key tiles per q-tile: exactly two pieces of the minimum size
    assert int(p["split_units"]) == tail and int(p["splits"]) == min(slots // tail, 16 // 8)


def _attn_keep(lib, h, layer, keep, hd, nq, segs, scale=0.088, keep_null=False):
    arr = (wmk.wmk_kv_segment * max(1, len(segs)))(*[wmk.wmk_kv_segment(k, v, t) for k, v, t in segs])
    ka = None if keep_null else (ctypes.c_int64 * max(1, len(keep)))(*keep)
    return lib.wmk_chunk_attention_retained(h, layer, ka, len(keep), ctypes.byref(hd), QBUF, nq, arr, len(segs),
                                            OBUF, scale, None, 0, None)


def _spans(dry):
    lines = dry.read_text().splitlines()
    last = max(i for i, x in enumerate(lines) if x.startswith("attn"))
    out = []
    for x in lines[last + 1:]:
        if x.startswith("span"):
            _, _, end, k, v = x.split()
            out.append((int(end), int(k, 16), int(v, 16)))
    return out


@pytest.mark.parametrize("S,W,cf,n_chunks,seed", [(6, 8, 4, 5, 0), (6, 8, 4, 3, 1), (2, 5, 3, 6, 2), (0, 7, 2, 9, 3)])
def test_retained_spans_follow_slot_policy(lib, dry, S, W, cf, n_chunks, seed):
    """Variable retention: the kept frames become one key span per run of adjacent
    slots, at the slots the oracle's policy gives those frames, in slot order,
    followed by the segments."""
    tpf, H, D, L = 16, 2, 64, 3
    d = _desc(L=L, H=H, D=D, tpf=tpf, S=S, W=W, cf=cf)
    _, h = _init(lib, d)
    cm = oracle.CacheModel(S, W, tpf, H, D)
    for _ in range(n_chunks):
        assert lib.wmk_cache_append_evict(h, 1, QBUF, SBUF, cf, None) == wmk.WMK_OK
        cm.append(np.zeros((cf * tpf, H, D), np.uint16), np.zeros((cf * tpf, H, D), np.uint16), cf)
    frame_b = tpf * H * D * 2
    layer_b = (S + W) * frame_b
    hd = wmk.wmk_head_desc(H, D, wmk.WMK_BF16)
    rng = np.random.default_rng(seed)
    res = cm.resident()
    for trial in range(6):
        keep = [int(f) for f in rng.permutation(res) if rng.random() < 0.5]
        assert _attn_keep(lib, h, 1, keep, hd, 40, [(QBUF, SBUF, 40)]) == wmk.WMK_OK
        slots = sorted(oracle.slot_of_frame(f, S, W) for f in keep)
        runs = []
        for s in slots:
            if runs and runs[-1][1] == s:
                runs[-1][1] = s + 1
            else:
                runs.append([s, s + 1])
        want, end = [], 0
        for a, b in runs:
            end += (b - a) * tpf
            want.append((end, KBUF + layer_b + a * frame_b, VBUF + layer_b + a * frame_b))
        want.append((end + 40, QBUF, SBUF))
        assert _spans(dry) == want, (keep, runs)
        assert _last_attn(dry)["kv"] == str(end + 40)
    # every resident frame: the same plan as plain chunk attention
    assert _attn_keep(lib, h, 1, res, hd, 40, [(QBUF, SBUF, 40)]) == wmk.WMK_OK
    a = _spans(dry)
    assert _attn(lib, h, 1, hd, 40, [(QBUF, SBUF, 40)]) == wmk.WMK_OK
    assert _spans(dry) == a
    lib.wmk_cache_destroy(h)


def test_retained_argument_errors(lib, dry):
    S, W, tpf, H, D = 0, 40, 16, 2, 64
    d = _desc(H=H, D=D, tpf=tpf, S=S, W=W, cf=40)
    _, h = _init(lib, d)
    assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 40, None) == wmk.WMK_OK   # frames 0..39 resident
    hd = wmk.wmk_head_desc(H, D, wmk.WMK_BF16)
    seg = [(QBUF, SBUF, 40)]
    every_other = list(range(0, 40, 2))                      # 20 runs of one slot
    bad = [
        (dict(keep=[40]), wmk.WMK_ERR_RANGE), (dict(keep=[-1]), wmk.WMK_ERR_RANGE),
        (dict(keep=[3, 3]), wmk.WMK_ERR_RANGE),
        (dict(keep=[1], keep_null=True), wmk.WMK_ERR_NULL),
        (dict(keep=every_other), wmk.WMK_ERR_CAPACITY),
        (dict(keep=every_other[:13], segs=seg * 4), wmk.WMK_ERR_CAPACITY),
        (dict(keep=[1], segs=seg * 5), wmk.WMK_ERR_SHAPE),
        (dict(keep=[1], layer=1), wmk.WMK_ERR_RANGE),
        (dict(keep=[1], scale=0.0), wmk.WMK_ERR_RANGE),
    ]
    for kw, status in bad:
        args = dict(layer=0, keep=[], segs=seg, keep_null=False, scale=0.088)
        args.update(kw)
        n_before = len(dry.read_text().splitlines())
        st = _attn_keep(lib, h, args["layer"], args["keep"], hd, 40, args["segs"], scale=args["scale"],
                        keep_null=args["keep_null"])
        assert st == status, (kw, st)
        assert len(dry.read_text().splitlines()) == n_before
    # a NULL cache is refused; 12 runs + 4 segments = 16 spans is the limit
    arr = (wmk.wmk_kv_segment * 1)(wmk.wmk_kv_segment(QBUF, SBUF, 40))
    assert lib.wmk_chunk_attention_retained(None, 0, None, 0, ctypes.byref(hd), QBUF, 40, arr, 1, OBUF, 0.1, None,
                                            0, None) == wmk.WMK_ERR_NULL
    assert _attn_keep(lib, h, 0, every_other[:12], hd, 40, seg * 4) == wmk.WMK_OK
    assert len(_spans(dry)) == 16
    assert _attn_keep(lib, h, 0, [], hd, 40, seg) == wmk.WMK_OK      # segments only
    assert _spans(dry) == [(40, QBUF, SBUF)]
    lib.wmk_cache_destroy(h)


def _qk8(lib, h, hd, nq, segs, ws, wsb, layer=0, scale=0.088):
    arr = (wmk.wmk_kv_segment * max(1, len(segs)))(*[wmk.wmk_kv_segment(k, v, t) for k, v, t in segs])
    return lib.wmk_chunk_attention_qk8(h, layer, ctypes.byref(hd), QBUF, nq, arr, len(segs), OBUF, scale, ws, wsb,
                                       None)


def _qk8_layout(H, nq, nk):
    a = lambda x: (x + 255) // 256 * 256
    kt, qb = -(-nk // 64), -(-nq // 32)
    return a(kt * H * 8192) + a(kt * H * 4) + a(qb * H * 4096) + a(qb * H * 4)


def test_qk8_workspace_errors_and_plan(lib, dry):
    """FP8 QK^T: the workspace holds the quantized operands (sized from the key count) and
    is required; the rest of it serves the split tail as for the plain call."""
    d = _desc()
    _, h = _init(lib, d)
    for _ in range(4):
        assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 4, None) == wmk.WMK_OK
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    nk = 14 * 1508 + 6032
    need = _qk8_layout(12, 6032, nk)
    full = lib.wmk_attention_qk8_workspace_bytes(ctypes.byref(hd), 6032, nk)
    assert full == need + lib.wmk_attention_workspace_bytes(ctypes.byref(hd), 6032)
    for bad_hd in (wmk.wmk_head_desc(12, 64, wmk.WMK_BF16), wmk.wmk_head_desc(12, 128, wmk.WMK_F32)):
        assert lib.wmk_attention_qk8_workspace_bytes(ctypes.byref(bad_hd), 6032, nk) == 0
    cur = [(QBUF, SBUF, 6032)]
    WS = 0x60000000
    bad = [
        (dict(ws=None, wsb=0), wmk.WMK_ERR_CAPACITY),
        (dict(ws=WS, wsb=need - 1), wmk.WMK_ERR_CAPACITY),
        (dict(ws=WS + 16, wsb=need), wmk.WMK_ERR_ALIGN),
        (dict(hd=wmk.wmk_head_desc(12, 128, wmk.WMK_F32)), wmk.WMK_ERR_DTYPE),
        (dict(segs=[(QBUF, SBUF, 8)] * 5), wmk.WMK_ERR_SHAPE),
        (dict(layer=3), wmk.WMK_ERR_RANGE),
        (dict(scale=0.0), wmk.WMK_ERR_RANGE),
    ]
    for kw, status in bad:
        args = dict(hd=hd, segs=cur, ws=WS, wsb=need, layer=0, scale=0.088)
        args.update(kw)
        n_before = len(dry.read_text().splitlines()) if dry.exists() else 0
        st = _qk8(lib, h, args["hd"], 6032, args["segs"], args["ws"], args["wsb"], layer=args["layer"],
                  scale=args["scale"])
        assert st == status, (kw, st)
        assert (len(dry.read_text().splitlines()) if dry.exists() else 0) == n_before
    # head_dim 64 is refused (a cache-less call with a 64-dim descriptor)
    hd64 = wmk.wmk_head_desc(12, 64, wmk.WMK_BF16)
    assert _qk8(lib, None, hd64, 100, [(QBUF, SBUF, 100)], WS, need) == wmk.WMK_ERR_SHAPE
    # exactly the operand regions: planned as FP8, no split; the full size: split as the plain call
    assert _qk8(lib, h, hd, 6032, cur, WS, need) == wmk.WMK_OK
    p = _last_attn(dry)
    assert (p["qk8"], p["kv"], p["split_units"]) == ("1", str(nk), "0")
    assert _qk8(lib, h, hd, 6032, cur, WS, full) == wmk.WMK_OK
    p = _last_attn(dry)
    assert _attn(lib, h, 0, hd, 6032, cur, ws=WS, wsb=full - need) == wmk.WMK_OK
    q = _last_attn(dry)
    assert q["qk8"] == "0" and (p["split_units"], p["splits"]) == (q["split_units"], q["splits"])
    assert int(p["split_units"]) > 0
    lib.wmk_cache_destroy(h)


@pytest.mark.parametrize("S,W,cf,n_chunks", [(6, 8, 4, 5), (6, 8, 4, 6), (6, 8, 4, 3), (2, 5, 3, 6), (0, 7, 2, 9)])
def test_qk8_spans_follow_time_order(lib, dry, S, W, cf, n_chunks):
    """The FP8 call lists the resident frames oldest first (sinks, then the window), one
    span per run of frames in adjacent slots, then the segments: the key sequence its
    scale blocks are cut along.  The plain call on the same cache keeps slot order."""
    tpf, H, D, L = 16, 2, 128, 2
    d = _desc(L=L, H=H, D=D, tpf=tpf, S=S, W=W, cf=cf)
    _, h = _init(lib, d)
    for _ in range(n_chunks):
        assert lib.wmk_cache_append_evict(h, 1, QBUF, SBUF, cf, None) == wmk.WMK_OK
    F = n_chunks * cf
    frame_b = tpf * H * D * 2
    layer_b = (S + W) * frame_b
    hd = wmk.wmk_head_desc(H, D, wmk.WMK_BF16)
    slots = [oracle.slot_of_frame(f, S, W) for f in oracle.resident_frames(F, S, W)]
    runs = []
    for s_ in slots:
        if runs and runs[-1][1] == s_:
            runs[-1][1] = s_ + 1
        else:
            runs.append([s_, s_ + 1])
    want, end = [], 0
    for a, b in runs:
        end += (b - a) * tpf
        want.append((end, KBUF + layer_b + a * frame_b, VBUF + layer_b + a * frame_b))
    want.append((end + 40, QBUF, SBUF))
    assert _qk8(lib, h, hd, 40, [(QBUF, SBUF, 40)], 0x60000000, 1 << 30, layer=1) == wmk.WMK_OK
    assert _spans(dry) == want
    assert len(runs) <= 3 and (len(runs) == 1) == (slots == sorted(slots))
    valid = oracle.valid_slots(F, S, W)
    assert _attn(lib, h, 1, hd, 40, [(QBUF, SBUF, 40)]) == wmk.WMK_OK
    assert _spans(dry) == [(valid * tpf, KBUF + layer_b, VBUF + layer_b), (valid * tpf + 40, QBUF, SBUF)]
    lib.wmk_cache_destroy(h)


def test_moba_train_and_backward_argument_errors(lib, dry):
    """Training forward (with log-sum-exp) and backward: argument checks before anything is
    planned; a valid backward logs its plan."""
    md = wmk.wmk_moba_desc(1560, 21, 3, 1)
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    LSE, DO, DQ, DK, DV, WS = 0x61000000, 0x62000000, 0x63000000, 0x64000000, 0x65000000, 0x66000000
    n = 3 * 21 * 1560
    need = lib.wmk_moba_backward_workspace_bytes(ctypes.byref(md), ctypes.byref(hd))
    assert need == (n * 12 * 4 + 255) // 256 * 256
    assert lib.wmk_moba_backward_workspace_bytes(None, ctypes.byref(hd)) == 0
    fwd = lambda **kw: lib.wmk_moba_attention_train(
        ctypes.byref(kw.get("md", md)), ctypes.byref(kw.get("hd", hd)), QBUF, KBUF, VBUF, OBUF, kw.get("lse", LSE),
        kw.get("scale", 0.088), None)
    bwd = lambda **kw: lib.wmk_moba_attention_backward(
        ctypes.byref(kw.get("md", md)), ctypes.byref(kw.get("hd", hd)), QBUF, KBUF, VBUF, OBUF, kw.get("dout", DO),
        kw.get("lse", LSE), kw.get("dq", DQ), DK, DV, kw.get("scale", 0.088), kw.get("ws", WS),
        kw.get("wsb", need), None)
    bad = [
        (fwd, dict(lse=0), wmk.WMK_ERR_NULL), (fwd, dict(lse=LSE + 4), wmk.WMK_ERR_ALIGN),
        (fwd, dict(hd=wmk.wmk_head_desc(12, 128, wmk.WMK_F32)), wmk.WMK_ERR_DTYPE),
        (fwd, dict(scale=-1.0), wmk.WMK_ERR_RANGE),
        (bwd, dict(dout=0), wmk.WMK_ERR_NULL), (bwd, dict(dq=0), wmk.WMK_ERR_NULL),
        (bwd, dict(dq=DQ + 2), wmk.WMK_ERR_ALIGN),
        (bwd, dict(hd=wmk.wmk_head_desc(12, 64, wmk.WMK_BF16)), wmk.WMK_ERR_SHAPE),
        (bwd, dict(hd=wmk.wmk_head_desc(12, 128, wmk.WMK_F32)), wmk.WMK_ERR_DTYPE),
        (bwd, dict(ws=0), wmk.WMK_ERR_CAPACITY), (bwd, dict(wsb=need - 4), wmk.WMK_ERR_CAPACITY),
        (bwd, dict(md=wmk.wmk_moba_desc(1560, 21, 3, 2)), wmk.WMK_ERR_SHAPE),
    ]
    for fn, kw, status in bad:
        n_before = len(dry.read_text().splitlines()) if dry.exists() else 0
        assert fn(**kw) == status, (kw, status)
        assert (len(dry.read_text().splitlines()) if dry.exists() else 0) == n_before
    assert fwd() == wmk.WMK_OK
    assert _last_attn(dry)["mask"] == "1"
    assert bwd() == wmk.WMK_OK
    last = [x for x in dry.read_text().strip().splitlines() if x.startswith("moba_bwd")][-1]
    assert last.startswith(f"moba_bwd n={n} heads=12 part={21 * 1560} chunk={3 * 1560} parts=3 ")


def _bwd_order(dry, which):
    lines = dry.read_text().splitlines()
    last = max(i for i, x in enumerate(lines) if x.startswith("moba_bwd"))
    runs = [tuple(int(v) for v in x.split()[2:]) for x in lines[last + 1:] if x.startswith(f"bgroup {which} ")]
    return [s + i for s, c in runs for i in range(c)]


@pytest.mark.parametrize("tpf,frames,cf", [(40, 7, 3), (64, 6, 2), (1560, 21, 3)])
def test_moba_backward_launch_order_is_longest_first(lib, dry, tpf, frames, cf):
    """Both backward kernels launch their 256-row (dQ) and 256-key (dK/dV) tiles longest walk first:
    each order is a permutation of the tiles, and the number of 64-wide tiles each one walks --
    counted here from the oracle's per-row intervals (rows for dQ; for dK/dV the query tiles
    holding some row that allows a key of the block) -- never increases along it."""
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    md = wmk.wmk_moba_desc(tpf, frames, cf, 1)
    need = lib.wmk_moba_backward_workspace_bytes(ctypes.byref(md), ctypes.byref(hd))
    assert lib.wmk_moba_attention_backward(ctypes.byref(md), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, SBUF,
                                           0x70000000, 0x71000000, 0x72000000, 0x73000000, 0.088, 0x60000000, need,
                                           None) == wmk.WMK_OK
    n = 3 * frames * tpf
    nt = (n + 255) // 256
    oq, ok = _bwd_order(dry, "q"), _bwd_order(dry, "k")
    assert sorted(oq) == list(range(nt)) and sorted(ok) == list(range(nt))
    step = 1 if nt < 100 else 5
    iv = [oracle.moba_row_intervals(i, tpf, frames, cf) for i in range(n)]

    def q_cost(t):
        tiles = set()
        for i in range(t * 256, min(t * 256 + 256, n)):
            for a, b in iv[i]:
                tiles.update(range(a // 64, (b + 63) // 64))
        return len(tiles)

    def k_cost(t):
        # a row tile is walked when some row of it allows a key of [c0, c1): rows of one chunk share
        # their intervals, so test one row per (64-row tile, chunk boundary) piece
        c0, c1 = t * 256, min(t * 256 + 256, n)
        walked = set()
        for i in range(n):
            if i // 64 in walked:
                continue
            if any(a < c1 and c0 < b for a, b in iv[i]):
                walked.add(i // 64)
        return len(walked)

    for order, cost in ((oq, q_cost), (ok, k_cost)):
        costs = [cost(t) for t in order[::step]]
        assert all(a >= b for a, b in zip(costs, costs[1:])), costs


# ---- the Python binding's own argument checks (raised before any library call)

def test_binding_rejects_mismatched_tensors():
    import torch
    bf = torch.bfloat16
    q = torch.zeros(64, 2, 128, dtype=bf)
    k = torch.zeros(100, 2, 128, dtype=bf)
    bad = [
        (lambda: wmk.chunk_attention(None, 0, q[:, :, :64]), "contiguous"),
        (lambda: wmk.chunk_attention(None, 0, q, [(k, k[:99])]), "shape"),
        (lambda: wmk.chunk_attention(None, 0, q, [(k.float(), k.float())]), "dtype"),
        (lambda: wmk.chunk_attention(None, 0, q, [(k[:, :1].contiguous(), k[:, :1].contiguous())]), "shape"),
        (lambda: wmk.chunk_attention(None, 0, q, out=torch.zeros(63, 2, 128, dtype=bf)), "shape"),
        (lambda: wmk.chunk_attention(None, 0, q.view(64, 256)), "dimensions"),
        (lambda: wmk.chunk_attention(None, 0, q, [(k, k)]), "device tensor"),
        (lambda: wmk.moba_attention(q, q, q, tokens_per_frame=10, frames=2, chunk_frames=1), "MoBA sequence"),
        (lambda: wmk.moba_attention(torch.zeros(60, 2, 128, dtype=bf), k, k, tokens_per_frame=10, frames=2,
                                    chunk_frames=1), "shape"),
        (lambda: wmk.moba_attention_train(torch.zeros(60, 2, 128, dtype=bf), torch.zeros(60, 2, 128, dtype=bf),
                                          torch.zeros(60, 2, 128, dtype=bf), tokens_per_frame=10, frames=2,
                                          chunk_frames=1, lse=torch.zeros(2, 59)), "shape"),
        (lambda: wmk.cross_attention_train(q, k, k, chunk_q_tokens=32, env_tokens=10, local_tokens=40), "shape"),
        (lambda: wmk.cross_attention_train(q, k, k, chunk_q_tokens=30, env_tokens=20, local_tokens=40), "chunks"),
    ]
    for fn, what in bad:
        with pytest.raises(ValueError, match=what):
            fn()


def test_binding_scratch_is_per_stream(monkeypatch):
    """The binding keeps one scratch buffer per (device, stream): two streams never share one."""
    import torch
    made = []

    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

    class FakeCtx:
        def __init__(self, s):
            pass

        def __enter__(self):
            return self

        def __exit__(self, *a):
            return False

    real_empty = torch.empty

    def fake_empty(n, dtype, device):
        made.append(n)
        return real_empty(n, dtype=dtype)

    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda idx=None: FakeStream(11))
    monkeypatch.setattr(torch.cuda, "stream", FakeCtx)
    monkeypatch.setattr(torch, "empty", fake_empty)
    monkeypatch.setattr(wmk, "_workspaces", {})
    a = wmk.workspace("cuda:0", 100)
    b = wmk.workspace("cuda:0", 100, FakeStream(22))
    c = wmk.workspace("cuda:0", 50, FakeStream(11))
    d = wmk.workspace("cuda:0", 200, FakeStream(22))
    assert a is c and a is not b and d is not b and made == [100, 100, 200]


def test_noalloc_plans_like_the_workspace_entry(lib, dry):
    """wmk_chunk_attention_noalloc plans exactly as wmk_chunk_attention with an ample
    workspace (same split units and pieces), its scratch at the library's own address,
    and refuses bad arguments before planning anything."""
    d = _desc()
    _, h = _init(lib, d)
    for _ in range(4):
        assert lib.wmk_cache_append_evict(h, 0, QBUF, SBUF, 4, None) == wmk.WMK_OK
    hd = wmk.wmk_head_desc(12, 128, wmk.WMK_BF16)
    for nq, nk in ((6032, 6032), (5500, 3016), (700, 100)):
        seg = (wmk.wmk_kv_segment * 1)(wmk.wmk_kv_segment(QBUF, SBUF, nk))
        assert lib.wmk_chunk_attention_noalloc(h, 0, ctypes.byref(hd), QBUF, nq, seg, 1, OBUF, 0.088,
                                               None) == wmk.WMK_OK
        a = _last_attn(dry)
        assert _attn(lib, h, 0, hd, nq, [(QBUF, SBUF, nk)], ws=0x60000000, wsb=1 << 30) == wmk.WMK_OK
        b = _last_attn(dry)
        assert a == b, (nq, a, b)
    assert (a["split_units"], a["splits"]) == ("0", "1")
    seg = (wmk.wmk_kv_segment * 1)(wmk.wmk_kv_segment(QBUF, SBUF, 6032))
    n_before = len(dry.read_text().splitlines())
    for args, status in [((h, 0, ctypes.byref(hd), QBUF, 6032, seg, 1, OBUF, 0.0), wmk.WMK_ERR_RANGE),
                         ((h, 1, ctypes.byref(hd), QBUF, 6032, seg, 1, OBUF, 0.088), wmk.WMK_ERR_RANGE),
                         ((h, 0, None, QBUF, 6032, seg, 1, OBUF, 0.088), wmk.WMK_ERR_NULL),
                         ((h, 0, ctypes.byref(hd), QBUF + 4, 6032, seg, 1, OBUF, 0.088), wmk.WMK_ERR_ALIGN)]:
        assert lib.wmk_chunk_attention_noalloc(*args, None) == status
    assert len(dry.read_text().splitlines()) == n_before
    lib.wmk_cache_destroy(h)


_FASTDIV_CHECK = r"""
#include "fastdiv.h"
#include <cstdio>
#include <random>
int main() {
    using namespace wmk;
    std::mt19937_64 g(7);
    long bad = 0, n_checked = 0;
    auto check = [&](uint32_t n, uint32_t d, FastDiv f) {
        ++n_checked;
        if (fastdiv(n, f) != n / d) { if (bad < 5) printf("wrong: %u / %u\n", n, d); ++bad; }
    };
    // every divisor up to 70000: around the first 64 multiples, near 2^31 and at random
    for (uint32_t d = 1; d <= 70000; ++d) {
        const FastDiv f = make_fastdiv(d);
        for (uint64_t k = 0; k < 64; ++k)
            for (int e = -1; e <= 1; ++e) { const int64_t n = (int64_t)(k * d) + e; if (n >= 0) check((uint32_t)n, d, f); }
        const int64_t top = (int64_t)(((1ull << 31) - 1) / d * d);
        for (int e = -1; e <= 1; ++e) if (top + e < (1ll << 31)) check((uint32_t)(top + e), d, f);
        for (int r = 0; r < 32; ++r) check((uint32_t)(g() & 0x7fffffffu), d, f);
    }
    // random divisors below 2^31, at random dividends, 2^31 - 1 and multiples +- 1
    for (int r = 0; r < 1000000; ++r) {
        const uint32_t d = 1 + (uint32_t)(g() % 0x7ffffffeu);
        const FastDiv f = make_fastdiv(d);
        check((uint32_t)(g() & 0x7fffffffu), d, f);
        check(0x7fffffffu, d, f);
        const uint32_t q = (uint32_t)(g() % (0x80000000ull / d));
        check(q * d, d, f);
        if (q * d) check(q * d - 1, d, f);
    }
    // the divisors of the workloads (tokens per frame, chunk and part lengths, heads), every n < 2^24
    for (uint32_t d : {1u, 3u, 12u, 24u, 64u, 1508u, 1560u, 3600u, 4680u, 32760u})
        { const FastDiv f = make_fastdiv(d); for (uint32_t n = 0; n < (1u << 24); ++n) check(n, d, f); }
    printf("%ld %ld\n", n_checked, bad);
    return bad != 0;
}
"""


def test_fast_division_is_exact(tmp_path):
    """The kernels' multiply-shift division (csrc/fastdiv.h, Granlund-Montgomery) equals
    integer division for every dividend below 2^31: checked on the host, with the same
    constexpr code the kernels compile, over all divisors to 70000 at the multiples'
    edges, a million random divisors, and every dividend below 2^24 for the workloads'
    divisors."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(_FASTDIV_CHECK)
    exe = tmp_path / "fastdiv_check"
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "kv_cache_attention_02_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    checked, wrong = map(int, r.stdout.split()[-2:])
    assert wrong == 0 and checked > 100_000_000


def _logged_tiles(dry, n_before):
    """The tile lines the last planned attention call logged: {(r0, r1): set of tiles}, plus bq."""
    lines = dry.read_text().splitlines()[n_before:]
    out = {}
    for ln in lines:
        if ln.startswith("tiles "):
            r0, r1, b0, e0, b1, e1, b2, e2, b3, e3, total = (int(x) for x in ln.split()[1:])
            tiles = set(range(b0, e0)) | set(range(b1, e1)) | set(range(b2, e2)) | set(range(b3, e3))
            assert total == (e0 - b0) + (e1 - b1) + (e2 - b2) + (e3 - b3) == len(tiles)   # disjoint ranges
            out[(r0, r1)] = tiles
    return out


def _oracle_tiles(row_intervals, r0, r1):
    """Tiles of 64 keys that any row in [r0, r1) may read, from the oracle's row intervals."""
    tiles = set()
    for i in range(r0, r1):
        for lo, hi in row_intervals(i):
            if hi > lo:
                tiles |= set(range(lo // 64, (hi - 1) // 64 + 1))
    return tiles


def test_planned_key_tiles_equal_the_oracles_row_intervals(lib, dry):
    """The key tiles every q-tile's workgroup walks (the kernels' own planner, run on the host
    in dry-run mode) are exactly the 64-key tiles its rows' oracle intervals touch: for seeded
    random MoBA sequences (with and without the bidirectional block), cross-attention
    training sequences and plain calls."""
    rng = np.random.default_rng(77)
    hd = wmk.wmk_head_desc(2, 128, wmk.WMK_BF16)
    checked = 0
    for case in range(40):
        n_before = len(dry.read_text().splitlines()) if dry.exists() else 0
        kind = case % 3
        if kind == 0:
            tpf, frames = int(rng.integers(1, 200)), int(rng.integers(1, 9))
            cf, bidir = int(rng.integers(1, frames + 1)), int(rng.integers(0, 2))
            md = wmk.wmk_moba_desc(tpf, frames, cf, bidir)
            assert lib.wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.1,
                                          None) == wmk.WMK_OK
            n = (2 + bidir) * frames * tpf
            rows = lambda i: oracle.moba_row_intervals(i, tpf, frames, cf, bidir)  # noqa: E731
        elif kind == 1:
            cq, nc = int(rng.integers(1, 700)), int(rng.integers(1, 8))
            ne, nl = int(rng.integers(0, 600)), int(rng.integers(0, 400))
            if ne + nl == 0:
                nl = 1
            xd = wmk.wmk_xattn_desc(cq, nc, ne, nl)
            assert lib.wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, 0.1,
                                                 None, 0, None) == wmk.WMK_OK
            n = cq * nc
            rows = lambda i: oracle.cross_train_row_intervals(i, cq, ne, nl)  # noqa: E731
        else:
            n, nk = int(rng.integers(1, 2000)), int(rng.integers(1, 5000))
            assert _attn(lib, None, 0, hd, n, [(KBUF, VBUF, nk)]) == wmk.WMK_OK
            rows = lambda i: [(0, nk)]  # noqa: E731
        logged = _logged_tiles(dry, n_before)
        assert sum(r1 - r0 for r0, r1 in logged) == n and min(r0 for r0, _ in logged) == 0
        for (r0, r1), tiles in logged.items():
            assert tiles == _oracle_tiles(rows, r0, r1), (case, r0, r1)
            checked += 1
    assert checked > 100


def test_planned_backward_query_tiles_equal_the_oracles_mask(lib, dry):
    """The query tiles every 256-key block's dK/dV workgroup walks (the kernel's own column
    planner, run on the host in dry-run mode) are exactly the 64-row tiles holding some row
    that the oracle's MoBA mask lets see a key of the block, for seeded random sequences with
    and without the bidirectional block."""
    rng = np.random.default_rng(78)
    hd = wmk.wmk_head_desc(2, 128, wmk.WMK_BF16)
    checked = 0
    for case in range(16):
        tpf, frames = int(rng.integers(1, 120)), int(rng.integers(1, 8))
        cf, bidir = int(rng.integers(1, frames + 1)), int(rng.integers(0, 2))
        md = wmk.wmk_moba_desc(tpf, frames, cf, bidir)
        need = lib.wmk_moba_backward_workspace_bytes(ctypes.byref(md), ctypes.byref(hd))
        n_before = len(dry.read_text().splitlines()) if dry.exists() else 0
        assert lib.wmk_moba_attention_backward(ctypes.byref(md), ctypes.byref(hd), QBUF, KBUF, VBUF, OBUF, SBUF,
                                               0x70000000, 0x71000000, 0x72000000, 0x73000000, 0.088, 0x60000000,
                                               need, None) == wmk.WMK_OK
        n = (2 + bidir) * frames * tpf
        mask = oracle.moba_mask(tpf, frames, cf, bidir)          # [row][key]
        blocks = 0
        for ln in dry.read_text().splitlines()[n_before:]:
            if not ln.startswith("ktiles "):
                continue
            c0, c1, b0, e0, b1, e1, b2, e2, b3, e3, total = (int(x) for x in ln.split()[1:])
            tiles = set(range(b0, e0)) | set(range(b1, e1)) | set(range(b2, e2)) | set(range(b3, e3))
            assert total == (e0 - b0) + (e1 - b1) + (e2 - b2) + (e3 - b3) == len(tiles)
            rows = np.flatnonzero(mask[:, c0:c1].any(axis=1))
            assert tiles == set((rows // 64).tolist()), (case, c0, c1)
            blocks += 1
            checked += 1
        assert blocks == (n + 255) // 256
    assert checked >= 40
