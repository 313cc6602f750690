"""wmk -- sink + window KV-cache chunk attention for MI355X (gfx950).

Python binding of the C ABI in ``include/wmk.h`` (``libwmk.so``, built in place
by :func:`kv_cache_attention_02_amd.build.build`).  The functions named
``wmk_*`` are the C entry points themselves, loaded with ctypes; the helpers
below them (:class:`Cache`, :func:`chunk_attention`, :func:`moba_attention`)
only marshal torch tensors into pointers, sizes and the current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback path: if ``libwmk.so`` is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libwmk.so")

WMK_OK, WMK_ERR_NULL, WMK_ERR_SHAPE, WMK_ERR_DTYPE, WMK_ERR_RANGE, WMK_ERR_ALIGN, WMK_ERR_CAPACITY, WMK_ERR_HIP = \
    range(8)
STATUS_NAMES = {0: "WMK_OK", 1: "WMK_ERR_NULL", 2: "WMK_ERR_SHAPE", 3: "WMK_ERR_DTYPE", 4: "WMK_ERR_RANGE",
                5: "WMK_ERR_ALIGN", 6: "WMK_ERR_CAPACITY", 7: "WMK_ERR_HIP"}
WMK_F32, WMK_BF16 = 0, 1
MAX_SEGMENTS = 4


class wmk_cache_desc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("sink_frames", ctypes.c_int32),
                ("window_frames", ctypes.c_int32), ("chunk_frames", ctypes.c_int32), ("dtype", ctypes.c_int)]


class wmk_head_desc(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int)]


class wmk_kv_segment(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("tokens", ctypes.c_int32)]


class wmk_moba_desc(ctypes.Structure):
    _fields_ = [("tokens_per_frame", ctypes.c_int32), ("frames", ctypes.c_int32), ("chunk_frames", ctypes.c_int32),
                ("bidir_block", ctypes.c_int32)]


class wmk_xattn_desc(ctypes.Structure):
    _fields_ = [("chunk_q_tokens", ctypes.c_int32), ("chunks", ctypes.c_int32), ("env_tokens", ctypes.c_int32),
                ("local_tokens", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "wmk_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(wmk_cache_desc)]),
    "wmk_cache_init": (ctypes.c_int, [ctypes.POINTER(wmk_cache_desc), _P, _P, ctypes.c_size_t, ctypes.POINTER(_P)]),
    "wmk_cache_destroy": (None, [_P]),
    "wmk_cache_append_evict": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, ctypes.c_int32, _P]),
    "wmk_cache_append_evict_layers": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32, _P]),
    "wmk_cache_slots": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64)]),
    "wmk_attention_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(wmk_head_desc), ctypes.c_int32]),
    "wmk_chunk_attention": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(wmk_head_desc), _P, ctypes.c_int32,
                                           ctypes.POINTER(wmk_kv_segment), ctypes.c_int32, _P, ctypes.c_float, _P,
                                           ctypes.c_size_t, _P]),
    "wmk_chunk_attention_noalloc": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(wmk_head_desc), _P,
                                                   ctypes.c_int32, ctypes.POINTER(wmk_kv_segment), ctypes.c_int32,
                                                   _P, ctypes.c_float, _P]),
    "wmk_attention_qk8_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(wmk_head_desc), ctypes.c_int32,
                                                            ctypes.c_int64]),
    "wmk_chunk_attention_qk8": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(wmk_head_desc), _P, ctypes.c_int32,
                                               ctypes.POINTER(wmk_kv_segment), ctypes.c_int32, _P, ctypes.c_float,
                                               _P, ctypes.c_size_t, _P]),
    "wmk_chunk_attention_retained": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                                    ctypes.c_int32, ctypes.POINTER(wmk_head_desc), _P, ctypes.c_int32,
                                                    ctypes.POINTER(wmk_kv_segment), ctypes.c_int32, _P,
                                                    ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "wmk_moba_attention": (ctypes.c_int, [ctypes.POINTER(wmk_moba_desc), ctypes.POINTER(wmk_head_desc), _P, _P, _P,
                                          _P, ctypes.c_float, _P]),
    "wmk_moba_attention_train": (ctypes.c_int, [ctypes.POINTER(wmk_moba_desc), ctypes.POINTER(wmk_head_desc), _P,
                                                _P, _P, _P, _P, ctypes.c_float, _P]),
    "wmk_moba_backward_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(wmk_moba_desc),
                                                            ctypes.POINTER(wmk_head_desc)]),
    "wmk_moba_attention_backward": (ctypes.c_int, [ctypes.POINTER(wmk_moba_desc), ctypes.POINTER(wmk_head_desc), _P,
                                                   _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                                   ctypes.c_size_t, _P]),
    "wmk_cross_attention_train": (ctypes.c_int, [ctypes.POINTER(wmk_xattn_desc), ctypes.POINTER(wmk_head_desc), _P,
                                                 _P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "wmk_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGNATURES)

_lib = None


def load():
    """Load libwmk.so (raises if it is not built) and return the ctypes handle.

    torch is imported first: it brings its own HIP runtime, and libwmk.so must bind to
    that same runtime (already loaded, it satisfies the library's dependency), so that
    the device memory and streams torch hands over are valid in the library's calls.
    Loaded the other way round, the process would hold two runtimes and the library's
    launches would fail."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(there is no fallback implementation)")
        import torch  # noqa: F401  (its HIP runtime before the library's dependency)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def __getattr__(name):  # wmk_* entry points resolve to the loaded C functions
    if name in _SIGNATURES:
        return getattr(load(), name)
    raise AttributeError(name)


class WmkError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def _check(status):
    if status != WMK_OK:
        raise WmkError(status, load().wmk_last_error().decode())


# ----------------------------------------------------------------------------------------------
# torch marshalling helpers
# ----------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t == torch.bfloat16:
        return WMK_BF16
    if t == torch.float32:
        return WMK_F32
    raise TypeError(f"unsupported dtype {t} (bfloat16 or float32)")


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


_workspaces = {}


def workspace(device, nbytes, stream=None):
    """A scratch buffer of at least nbytes for calls on `stream` (default: the
    current stream of `device`), grown on demand and kept for reuse.  One buffer
    per (device, stream): calls on different streams never share scratch, and a
    buffer is allocated on the stream that uses it, so when it is replaced the
    caching allocator reuses its memory only behind that stream's queued work."""
    torch = _torch()
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    s = torch.cuda.current_stream(idx) if stream is None else stream
    key = (idx, s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=torch.device("cuda", idx))
        _workspaces[key] = ws
    return ws


def _check_tensor(name, t, *, dtype=None, device=None, rows=None, heads=None, head_dim=None, ndim=3):
    """Raise ValueError unless t is a contiguous tensor of the given dtype, device and
    shape [rows][heads][head_dim] (None: any)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    want = (rows, heads, head_dim)
    for i, w in enumerate(want[:ndim]):
        if w is not None and t.shape[i] != w:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                             f"{tuple(x if x is not None else '*' for x in want[:ndim])}")


def _on_device(**tensors):
    """Raise ValueError unless every tensor is device memory (checked after the shapes)."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor (is on {t.device})")


def _check_like(name, t, ref, rows=None):
    _check_tensor(name, t, dtype=ref.dtype, device=ref.device, rows=ref.shape[0] if rows is None else rows,
                  heads=ref.shape[1], head_dim=ref.shape[2])


class Cache:
    """A per-layer sink + window KV cache over torch-allocated K/V buffers.

    Buffers are [num_layers][S + W][tokens_per_frame][heads][head_dim] each,
    allocated here through torch (the library itself never allocates).
    """

    def __init__(self, *, num_layers, num_heads, head_dim, tokens_per_frame, sink_frames, window_frames,
                 chunk_frames, dtype=None, device="cuda"):
        torch = _torch()
        dtype = torch.bfloat16 if dtype is None else dtype
        self.desc = wmk_cache_desc(num_layers, num_heads, head_dim, tokens_per_frame, sink_frames, window_frames,
                                   chunk_frames, _dtype_code(dtype))
        nbytes = load().wmk_cache_bytes(ctypes.byref(self.desc))
        if nbytes == 0:
            raise WmkError(WMK_ERR_SHAPE, "invalid cache descriptor: " + load().wmk_last_error().decode())
        shape = (num_layers, sink_frames + window_frames, tokens_per_frame, num_heads, head_dim)
        self.k = torch.empty(shape, dtype=dtype, device=device)
        self.v = torch.empty(shape, dtype=dtype, device=device)
        self.dtype = dtype
        self._h = ctypes.c_void_p()
        _check(load().wmk_cache_init(ctypes.byref(self.desc), _ptr(self.k), _ptr(self.v), nbytes,
                                     ctypes.byref(self._h)))

    @property
    def handle(self):
        return self._h

    def append_evict(self, layer, k_new, v_new, n_frames=None, stream=None):
        """Append the finalized frames k_new/v_new ([n_frames * tokens_per_frame][H][D]) to `layer`."""
        tpf = self.desc.tokens_per_frame
        _check_tensor("k_new", k_new, dtype=self.dtype, device=self.k.device, heads=self.desc.num_heads,
                      head_dim=self.desc.head_dim)
        if n_frames is None:
            if k_new.shape[0] % tpf:
                raise ValueError(f"k_new has {k_new.shape[0]} rows, not a whole number of {tpf}-token frames")
            n_frames = k_new.shape[0] // tpf
        if k_new.shape[0] != n_frames * tpf:
            raise ValueError(f"k_new has {k_new.shape[0]} rows, {n_frames} frames need {n_frames * tpf}")
        _check_like("v_new", v_new, k_new)
        _on_device(k_new=k_new)
        _check(load().wmk_cache_append_evict(self._h, layer, _ptr(k_new), _ptr(v_new), n_frames,
                                             _stream_ptr(stream)))

    def append_evict_layers(self, first_layer, k_new, v_new, n_frames=None, stream=None):
        """Append one finalized chunk to layers [first_layer, first_layer + len(k_new)) in one
        launch: k_new/v_new are [n_layers][n_frames * tokens_per_frame][H][D]."""
        torch = _torch()
        tpf, H, D = self.desc.tokens_per_frame, self.desc.num_heads, self.desc.head_dim
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if not isinstance(t, torch.Tensor) or t.dim() != 4:
                raise ValueError(f"{name} must be a 4-d tensor [n_layers][n_frames * tokens_per_frame][H][D]")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if t.dtype != self.dtype or t.device != self.k.device:
                raise ValueError(f"{name} is {t.dtype} on {t.device}, expected {self.dtype} on {self.k.device}")
            if tuple(t.shape[2:]) != (H, D) or t.shape != k_new.shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [*][*][{H}][{D}] like k_new")
        n_layers, rows = k_new.shape[0], k_new.shape[1]
        if n_frames is None:
            if rows % tpf:
                raise ValueError(f"k_new has {rows} rows per layer, not a whole number of {tpf}-token frames")
            n_frames = rows // tpf
        if rows != n_frames * tpf:
            raise ValueError(f"k_new has {rows} rows per layer, {n_frames} frames need {n_frames * tpf}")
        _on_device(k_new=k_new)
        _check(load().wmk_cache_append_evict_layers(self._h, first_layer, n_layers, _ptr(k_new), _ptr(v_new),
                                                    n_frames, _stream_ptr(stream)))

    def slots(self, layer):
        n = self.desc.sink_frames + self.desc.window_frames
        arr = (ctypes.c_int64 * n)()
        F = ctypes.c_int64()
        _check(load().wmk_cache_slots(self._h, layer, arr, ctypes.byref(F)))
        return list(arr), F.value

    def close(self):
        if self._h:
            load().wmk_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _check_cache(cache, q):
    if cache is None:
        return
    if q.dtype != cache.dtype or q.device != cache.k.device or q.shape[1:] != cache.k.shape[3:]:
        raise ValueError(f"q ({q.dtype}, {q.device}, heads x dim {tuple(q.shape[1:])}) does not match the cache "
                         f"({cache.dtype}, {cache.k.device}, {tuple(cache.k.shape[3:])})")


def _segments(segments, q):
    """ctypes array of the (k, v) segments; each [n][H][D] like q."""
    segs = (wmk_kv_segment * max(1, len(segments)))()
    for i, (k, v) in enumerate(segments):
        _check_tensor(f"segment {i} k", k, dtype=q.dtype, device=q.device, heads=q.shape[1], head_dim=q.shape[2])
        _check_like(f"segment {i} v", v, k)
        segs[i] = wmk_kv_segment(k.data_ptr(), v.data_ptr(), k.shape[0])
    return segs


def chunk_attention(cache, layer, q, segments=(), out=None, scale=None, use_workspace=True, stream=None,
                    keep_frames=None):
    """out[q_tokens][H][D] = attention of q over the resident frames of `layer` in `cache`
    (None for none) and every token of `segments` (a list of (k, v) tensors).
    keep_frames: attend only these resident frames (global frame indices);
    None attends all of them."""
    torch = _torch()
    _check_tensor("q", q)
    nq, H, D = q.shape
    _check_cache(cache, q)
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    segs = _segments(segments, q)
    _on_device(q=q)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ws, wsb = ctypes.c_void_p(0), 0
    if use_workspace:
        wsb = load().wmk_attention_workspace_bytes(ctypes.byref(hd), nq)
        if wsb:
            w = workspace(q.device, wsb, stream)
            ws, wsb = _ptr(w), w.numel()
    if keep_frames is None:
        _check(load().wmk_chunk_attention(cache.handle if cache is not None else None, layer, ctypes.byref(hd),
                                          _ptr(q), nq, segs, len(segments), _ptr(out), scale, ws, wsb,
                                          _stream_ptr(stream)))
    else:
        keep = [int(f) for f in keep_frames]
        arr = (ctypes.c_int64 * max(1, len(keep)))(*keep)
        _check(load().wmk_chunk_attention_retained(cache.handle if cache is not None else None, layer, arr,
                                                   len(keep), ctypes.byref(hd), _ptr(q), nq, segs, len(segments),
                                                   _ptr(out), scale, ws, wsb, _stream_ptr(stream)))
    return out


def chunk_attention_noalloc(cache, layer, q, out, segments=(), scale=None, stream=None):
    """chunk_attention through wmk_chunk_attention_noalloc: the split tail's scratch is the
    library's own device array, so nothing is allocated (``out`` is required)."""
    _check_tensor("q", q)
    nq, H, D = q.shape
    _check_cache(cache, q)
    _check_like("out", out, q)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    segs = _segments(segments, q)
    _on_device(q=q)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(load().wmk_chunk_attention_noalloc(cache.handle if cache is not None else None, layer, ctypes.byref(hd),
                                              _ptr(q), nq, segs, len(segments), _ptr(out), scale,
                                              _stream_ptr(stream)))
    return out


def qk8_workspace_bytes(num_heads, q_tokens, kv_tokens, head_dim=128):
    """Bytes of workspace chunk_attention_qk8 needs (quantized operands + split scratch)."""
    hd = wmk_head_desc(num_heads, head_dim, WMK_BF16)
    return load().wmk_attention_qk8_workspace_bytes(ctypes.byref(hd), q_tokens, kv_tokens)


def chunk_attention_qk8(cache, layer, q, segments=(), out=None, scale=None, stream=None, ws=None):
    """chunk_attention with the FP8-quantized QK^T.  ``ws``: a uint8 device tensor to use as
    the workspace (its head then holds the quantized operands, see include/wmk.h); by
    default a cached one sized for every resident frame plus the segments."""
    torch = _torch()
    _check_tensor("q", q)
    nq, H, D = q.shape
    _check_cache(cache, q)
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    segs = _segments(segments, q)
    kv = sum(k.shape[0] for k, _ in segments)
    _on_device(q=q)
    if cache is not None:
        kv += (cache.desc.sink_frames + cache.desc.window_frames) * cache.desc.tokens_per_frame
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if ws is None:
        wsb = load().wmk_attention_qk8_workspace_bytes(ctypes.byref(hd), nq, kv)
        ws = workspace(q.device, wsb, stream) if wsb else None
    elif not (isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8 and ws.dim() == 1 and ws.is_contiguous()
              and ws.device == q.device):
        raise ValueError("ws must be a contiguous 1-d uint8 tensor on the device of q")
    wsp, wsb = (_ptr(ws), ws.numel()) if ws is not None else (ctypes.c_void_p(0), 0)
    _check(load().wmk_chunk_attention_qk8(cache.handle if cache is not None else None, layer, ctypes.byref(hd),
                                          _ptr(q), nq, segs, len(segments), _ptr(out), scale, wsp, wsb,
                                          _stream_ptr(stream)))
    return out


def moba_attention(q, k, v, *, tokens_per_frame, frames, chunk_frames, bidir_block=1, out=None, scale=None,
                   stream=None):
    """MoBA-masked attention forward over [clean | noisy | block]."""
    torch = _torch()
    _check_moba(q, k, v, tokens_per_frame, frames, bidir_block)
    n, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q)
    _on_device(q=q)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    md = wmk_moba_desc(tokens_per_frame, frames, chunk_frames, bidir_block)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(load().wmk_moba_attention(ctypes.byref(md), ctypes.byref(hd), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     scale, _stream_ptr(stream)))
    return out


def _check_moba(q, k, v, tokens_per_frame, frames, bidir_block):
    """q, k, v: [(2 + bidir_block) * frames * tokens_per_frame][H][D], alike."""
    _check_tensor("q", q)
    n = (2 + bidir_block) * frames * tokens_per_frame
    if q.shape[0] != n:
        raise ValueError(f"q has {q.shape[0]} rows; the MoBA sequence has (2 + {bidir_block}) * {frames} * "
                         f"{tokens_per_frame} = {n}")
    _check_like("k", k, q)
    _check_like("v", v, q)


def moba_attention_train(q, k, v, *, tokens_per_frame, frames, chunk_frames, bidir_block=1, out=None, lse=None,
                         scale=None, stream=None):
    """MoBA forward for training: returns (out, lse) with lse [H][n] fp32 (natural log)."""
    torch = _torch()
    _check_moba(q, k, v, tokens_per_frame, frames, bidir_block)
    n, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q)
    if lse is None:
        lse = torch.empty((H, n), dtype=torch.float32, device=q.device)
    _check_tensor("lse", lse, dtype=torch.float32, device=q.device, rows=H, heads=n, ndim=2)
    _on_device(q=q)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    md = wmk_moba_desc(tokens_per_frame, frames, chunk_frames, bidir_block)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(load().wmk_moba_attention_train(ctypes.byref(md), ctypes.byref(hd), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                           _ptr(lse), scale, _stream_ptr(stream)))
    return out, lse


def moba_attention_backward(q, k, v, out, dout, lse, *, tokens_per_frame, frames, chunk_frames, bidir_block=1,
                            scale=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for the MoBA-masked attention."""
    torch = _torch()
    _check_moba(q, k, v, tokens_per_frame, frames, bidir_block)
    n, H, D = q.shape
    _check_like("out", out, q)
    _check_like("dout", dout, q)
    _check_tensor("lse", lse, dtype=torch.float32, device=q.device, rows=H, heads=n, ndim=2)
    _on_device(q=q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    md = wmk_moba_desc(tokens_per_frame, frames, chunk_frames, bidir_block)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    wsb = load().wmk_moba_backward_workspace_bytes(ctypes.byref(md), ctypes.byref(hd))
    ws = workspace(q.device, wsb, stream)
    _check(load().wmk_moba_attention_backward(ctypes.byref(md), ctypes.byref(hd), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), scale,
                                              _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return dq, dk, dv


def cross_attention_train(q, k, v, *, chunk_q_tokens, env_tokens, local_tokens, out=None, scale=None,
                          use_workspace=True, stream=None):
    """Chunk-causal cross-attention over a multi-chunk sequence: query chunk i
    (rows [i * chunk_q_tokens, (i + 1) * chunk_q_tokens)) reads keys
    [0, env_tokens) and its own local prompt [env_tokens + i * local_tokens, +local_tokens)."""
    torch = _torch()
    _check_tensor("q", q)
    nq, H, D = q.shape
    if chunk_q_tokens <= 0 or nq % chunk_q_tokens:
        raise ValueError(f"{nq} query tokens are not a whole number of chunks of {chunk_q_tokens}")
    chunks = nq // chunk_q_tokens
    nk = env_tokens + chunks * local_tokens
    _check_tensor("k", k, dtype=q.dtype, device=q.device, rows=nk, heads=H, head_dim=D)
    _check_like("v", v, k)
    _on_device(q=q)
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q)
    hd = wmk_head_desc(H, D, _dtype_code(q.dtype))
    xd = wmk_xattn_desc(chunk_q_tokens, chunks, env_tokens, local_tokens)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ws, wsb = ctypes.c_void_p(0), 0
    if use_workspace:
        wsb = load().wmk_attention_workspace_bytes(ctypes.byref(hd), nq)
        if wsb:
            w = workspace(q.device, wsb, stream)
            ws, wsb = _ptr(w), w.numel()
    _check(load().wmk_cross_attention_train(ctypes.byref(xd), ctypes.byref(hd), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(out), scale, ws, wsb, _stream_ptr(stream)))
    return out
