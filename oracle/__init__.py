"""ORACLE -- test infrastructure only.

A plain, slow CPU statement of what the sink + window KV-cache chunk attention
computes.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark import it; the product library never does, and this package imports
nothing from the product package.  It shares no code with the GPU path.

Sources (cited by page title and section):

* "LingBot-World-Infinity: The Open-Source World Model That Refuses to Forget"
  (repo-explainer page), sections "The trick: treat video like a causal
  stream" (the simplified loop: keep the anchor tokens, evict old tokens, step,
  append) and "How the cache keeps the world alive" (a sliding KV cache with
  sink tokens kept at the front, old tokens discarded once the window is full).
* "Westlake AGI Lab's 'World in World' Steers Frozen Video Models", second
  paragraph: the native block holds 18 latent-frame slots -- six anchors, eight
  recent finalized states and four states of the current chunk.
* "Infinite Worlds with Versatile Interactions", paragraph on causal
  pretraining: each frame state depends only on past observations; the
  teacher-forcing mask; MoBA appends a fully bidirectional block to it; a
  causal cross-attention mask keeps chunk-wise prompts from leaking future
  semantics.
* "Mix Forcing: Causal Pre-Training via Mixture Attention for Interactive
  World Models", Overview, "Mix the training modes" and "Condition each chunk":
  chunks are generated from current inputs and cached history; MoBA mixes
  teacher forcing with bidirectional training; each chunk's cross-attention
  reads the shared environment prompt and its own local prompt only (at
  inference one chunk at a time; in training every chunk of a sequence at
  once, under the causal cross-attention mask).

* "Infinite Worlds with Versatile Interactions", deployment paragraph: a
  dynamic KV-cache scheduler adapts the retained history to the current
  control signal (here: a call attends a chosen subset of the resident
  frames).
* LingBot-World 2.0 speed-up page (kaarelkaarelson.com/lingbot), step table
  ("Attention" row: FlashAttention-2 replaced by SageAttention 2.2, a
  quantized-QK^T kernel) and roofline table ("SageAttention" row): the
  precision variant of the attention step.

Readings where the pages are silent (all stated once more in the design notes):
sinks and window are counted in latent frames; the window excludes the current
chunk; append and evict happen in one call after a chunk is finalized; an
append longer than the window keeps only its last W non-sink frames; the
current chunk attends itself bidirectionally; MoBA clean chunks are
block-causal among themselves; the MoBA bidirectional block attends only
itself and nothing else attends it; a row with no allowed key outputs zero.

Numerics: the attention arithmetic is in ``attend.c`` (fp64, two-pass
softmax).  Integer parts (slot arithmetic, resident sets, masks as key
intervals) are here, in Python.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_lib = None


# --------------------------------------------------------------------------------------------
# Build / load of the fp64 attention core
# --------------------------------------------------------------------------------------------

def build(verbose=False):
    """Compile ``liboracle.so`` from ``attend.c`` with gcc (OpenMP, no BLAS)."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           os.path.join(_DIR, "attend.c"), "-o", os.path.join(_DIR, "liboracle.so"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr:
        print(r.stderr)


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_DIR, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.oracle_attend.restype = ctypes.c_int
        lib.oracle_attend.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                      ctypes.c_void_p]
        _lib = lib
    return _lib


def widen(x):
    """float32 view of an input: bf16 bit patterns (uint16) are widened exactly, float32 passes."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if x.dtype == np.float32:
        return x
    raise TypeError(f"unsupported input dtype {x.dtype}")


def attend(q, k, v, intervals, scale, want_probs=False):
    """Masked softmax attention in fp64 (``attend.c``).

    q: [nq][H][D]; k, v: [nk][H][D] (float32 or bf16 bits as uint16).
    intervals: list (one entry per query row) of lists of disjoint half-open
    key ranges (lo, hi) into k/v.  Returns out [nq][H][D] float64, and the
    dense probabilities [nq][H][nk] when ``want_probs``.
    """
    q = np.ascontiguousarray(widen(q))
    k = np.ascontiguousarray(widen(k))
    v = np.ascontiguousarray(widen(v))
    nq, H, D = q.shape
    nk = k.shape[0]
    if k.shape != (nk, H, D) or v.shape != (nk, H, D):
        raise ValueError("k/v shape mismatch")
    if len(intervals) != nq:
        raise ValueError("one interval list per query row is required")
    ptr = np.zeros(nq + 1, dtype=np.int64)
    los, his = [], []
    for i, ivs in enumerate(intervals):
        ivs = sorted((int(a), int(b)) for a, b in ivs if b > a)
        for (a0, b0), (a1, _) in zip(ivs, ivs[1:]):
            if a1 < b0:
                raise ValueError(f"row {i}: overlapping key intervals")
        for a, b in ivs:
            los.append(a)
            his.append(b)
        ptr[i + 1] = ptr[i] + len(ivs)
    lo = np.asarray(los, dtype=np.int64) if los else np.zeros(1, dtype=np.int64)
    hi = np.asarray(his, dtype=np.int64) if his else np.zeros(1, dtype=np.int64)
    out = np.empty((nq, H, D), dtype=np.float64)
    probs = np.empty((nq, H, nk), dtype=np.float64) if want_probs else None
    rc = _load().oracle_attend(q.ctypes.data, nq, k.ctypes.data, v.ctypes.data, nk, H, D, ptr.ctypes.data,
                               lo.ctypes.data, hi.ctypes.data, float(scale), out.ctypes.data,
                               probs.ctypes.data if probs is not None else None)
    if rc != 0:
        raise RuntimeError(f"oracle_attend failed ({rc})")
    return (out, probs) if want_probs else out


# --------------------------------------------------------------------------------------------
# Cache policy: sinks + sliding window, counted in latent frames
# ("How the cache keeps the world alive"; 18-slot layout of "World in World")
# --------------------------------------------------------------------------------------------

def slot_of_frame(f, S, W):
    """Slot of frame f: the first S frames own slots 0..S-1 for good; later frames
    share the W window slots in turn, so frame f overwrites frame f-W."""
    return f if f < S else S + (f - S) % W


def resident_frames(F, S, W):
    """Frames held after F frames were appended, in time order: the sinks
    (the first min(F, S) frames) and the last W non-sink frames."""
    return list(range(min(F, S))) + list(range(max(S, F - W), F))


def valid_slots(F, S, W):
    """Number of filled slots after F appended frames."""
    return min(F, S) + min(max(F - S, 0), W)


def frames_kept_by_append(F, n, S, W):
    """Frames of an append of n frames (frames F..F+n-1) that are still resident
    after it: sinks, and the last W non-sink frames.  The others would be
    evicted by the same call and are never written."""
    return [f for f in range(F, F + n) if f < S or f >= F + n - W]


class CacheModel:
    """One layer of the KV cache, kept as a map frame -> its K/V rows.

    ``append`` follows the loop of the repo-explainer page (evict old non-sink
    frames, keep the anchors, append the finalized frames); here the eviction
    and the append are one call made after a chunk is finalized.
    """

    def __init__(self, S, W, tokens_per_frame, H, D, dtype=np.uint16):
        if S < 0 or W < 1 or tokens_per_frame < 1:
            raise ValueError("need S >= 0, W >= 1, tokens_per_frame >= 1")
        self.S, self.W, self.tpf, self.H, self.D, self.dtype = S, W, tokens_per_frame, H, D, dtype
        self.F = 0
        self.frames = {}  # frame index -> (k rows [tpf][H][D], v rows [tpf][H][D])

    def append(self, k_new, v_new, n_frames):
        k_new = np.asarray(k_new).reshape(n_frames * self.tpf, self.H, self.D)
        v_new = np.asarray(v_new).reshape(n_frames * self.tpf, self.H, self.D)
        for f in frames_kept_by_append(self.F, n_frames, self.S, self.W):
            j = f - self.F
            rows = slice(j * self.tpf, (j + 1) * self.tpf)
            self.frames[f] = (k_new[rows].copy(), v_new[rows].copy())
        self.F += n_frames
        keep = set(resident_frames(self.F, self.S, self.W))
        self.frames = {f: kv for f, kv in self.frames.items() if f in keep}

    def resident(self):
        return resident_frames(self.F, self.S, self.W)

    def slot_map(self):
        """frame held by each of the S+W slots, -1 where empty."""
        m = np.full(self.S + self.W, -1, dtype=np.int64)
        for f in self.resident():
            m[slot_of_frame(f, self.S, self.W)] = f
        return m

    def slot_buffers(self):
        """K and V laid out by slot, [S+W][tpf][H][D]; empty slots are zero."""
        shape = (self.S + self.W, self.tpf, self.H, self.D)
        kb = np.zeros(shape, dtype=self.dtype)
        vb = np.zeros(shape, dtype=self.dtype)
        for f in self.resident():
            s = slot_of_frame(f, self.S, self.W)
            kb[s], vb[s] = self.frames[f]
        return kb, vb

    def logical_kv(self, frames=None):
        """Resident K and V concatenated in time order, [n_resident*tpf][H][D].
        ``frames``: only these resident frames (variable retention)."""
        fs = self.resident()
        if frames is not None:
            frames = [int(f) for f in frames]
            if len(set(frames)) != len(frames):
                raise ValueError("a retained frame is listed twice")
            missing = set(frames) - set(fs)
            if missing:
                raise ValueError(f"frames {sorted(missing)} are not resident")
            fs = sorted(frames)
        if not fs:
            e = np.zeros((0, self.H, self.D), dtype=self.dtype)
            return e, e.copy()
        return (np.concatenate([self.frames[f][0] for f in fs]),
                np.concatenate([self.frames[f][1] for f in fs]))


# --------------------------------------------------------------------------------------------
# Chunk attention at inference ("Mix Forcing" Overview: chunks from current inputs and
# cached history; "World in World": anchors + recent + current chunk slots)
# --------------------------------------------------------------------------------------------

def chunk_attention(cache, q, segments, scale, rows=None, keep_frames=None):
    """Queries of the current chunk attend every resident cache frame and every
    token of the passed segments (the current chunk's own K/V, bidirectionally,
    or prompt K/V for cross-attention).  ``cache`` may be None.

    q: [nq][H][D]; segments: list of (k, v), each [n][H][D].  ``rows`` selects
    the query rows to evaluate (default: all).  Returns fp64 [len(rows)][H][D].

    ``keep_frames``: variable retention ("LingBot-World-Infinity" overview,
    deployment: a dynamic KV-cache scheduler adapts the retained history) --
    only these resident frames are attended; the rest stay cached but unseen.
    Temporary auxiliary KV blocks ("World in World", second paragraph) are
    simply further segments.
    """
    ks, vs = [], []
    if cache is not None:
        kc, vc = cache.logical_kv(keep_frames)
        ks.append(kc)
        vs.append(vc)
    elif keep_frames:
        raise ValueError("retained frames need a cache")
    for k, v in segments:
        ks.append(np.asarray(k))
        vs.append(np.asarray(v))
    k_all = np.concatenate([widen(x) for x in ks]) if ks else np.zeros((0,) + q.shape[1:], np.float32)
    v_all = np.concatenate([widen(x) for x in vs]) if vs else np.zeros((0,) + q.shape[1:], np.float32)
    q = np.asarray(q)
    if rows is not None:
        q = q[np.asarray(rows)]
    nk = k_all.shape[0]
    return attend(q, k_all, v_all, [[(0, nk)]] * q.shape[0], scale)


# --------------------------------------------------------------------------------------------
# MoBA training mask ("Infinite Worlds with Versatile Interactions", causal pretraining
# paragraph; "Mix Forcing", "Mix the training modes")
# --------------------------------------------------------------------------------------------

def moba_row_intervals(i, tokens_per_frame, frames, chunk_frames, bidir_block=1):
    """Allowed key ranges of token i in the sequence [clean | noisy | bidirectional].

    Each part holds ``frames`` latent frames; a token's frame g inside its part
    lies in chunk k = g // chunk_frames.  Clean tokens see clean keys of chunks
    <= k (block-causal); noisy tokens see clean keys of chunks < k and noisy
    keys of chunk k (teacher forcing); tokens of the bidirectional block see
    the whole block and nothing else.
    """
    L = frames * tokens_per_frame
    cl = chunk_frames * tokens_per_frame
    part, r = divmod(i, L)
    k = (r // tokens_per_frame) // chunk_frames
    if part == 0:
        return [(0, min((k + 1) * cl, L))]
    if part == 1:
        out = [(0, min(k * cl, L))] if k > 0 else []
        out.append((L + k * cl, L + min((k + 1) * cl, L)))
        return out
    if part == 2 and bidir_block:
        return [(2 * L, 3 * L)]
    raise ValueError("token index outside the sequence")


def moba_attention(q, k, v, tokens_per_frame, frames, chunk_frames, bidir_block, scale, rows=None):
    """MoBA-masked attention over the whole training sequence; fp64 rows."""
    q = np.asarray(q)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    ivs = [moba_row_intervals(int(i), tokens_per_frame, frames, chunk_frames, bidir_block) for i in rows]
    return attend(q[rows], k, v, ivs, scale)


# --------------------------------------------------------------------------------------------
# Chunk-wise causal cross-attention ("Mix Forcing", "Condition each chunk")
# --------------------------------------------------------------------------------------------

def cross_row_intervals(chunk, env_tokens, local_tokens):
    """Over keys [env | local_0 | local_1 | ...]: chunk i reads env and local_i only."""
    a = env_tokens + chunk * local_tokens
    return [(0, env_tokens), (a, a + local_tokens)]


def cross_attention(q, chunk, k_env, v_env, k_locals, v_locals, scale, rows=None):
    """Queries of chunk ``chunk`` attend the environment prompt and their own local prompt."""
    k_all = np.concatenate([widen(k_env)] + [widen(x) for x in k_locals])
    v_all = np.concatenate([widen(v_env)] + [widen(x) for x in v_locals])
    q = np.asarray(q)
    if rows is not None:
        q = q[np.asarray(rows)]
    iv = cross_row_intervals(chunk, k_env.shape[0], k_locals[0].shape[0])
    return attend(q, k_all, v_all, [iv] * q.shape[0], scale)


def cross_train_row_intervals(i, chunk_q_tokens, env_tokens, local_tokens):
    """Training form over a multi-chunk sequence: query row i belongs to chunk
    i // chunk_q_tokens and reads the environment prompt and that chunk's local
    prompt only, over keys [env | local_0 | local_1 | ...]."""
    return cross_row_intervals(i // chunk_q_tokens, env_tokens, local_tokens)


def cross_attention_train(q, k, v, chunk_q_tokens, env_tokens, local_tokens, scale, rows=None):
    """Chunk-causal cross-attention of every query chunk at once; fp64 rows."""
    q = np.asarray(q)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    ivs = [cross_train_row_intervals(int(i), chunk_q_tokens, env_tokens, local_tokens) for i in rows]
    return attend(q[rows], k, v, ivs, scale)


# --------------------------------------------------------------------------------------------
# Quantized QK^T: FP8 e4m3 codes with one fp32 scale per block (the precision variant of the
# attention step; LingBot-World 2.0 speed-up page, step table "Attention" row: SageAttention 2.2,
# a quantized-QK^T kernel, replaces FlashAttention-2; roofline table "SageAttention" row).  The
# pages fix no format or block shape; the readings here: OCP e4m3 (largest finite 448), round to
# nearest even, symmetric absmax scaling per (block of rows, head) -- 32 query rows, 64 keys --
# with no smoothing; K blocks are 64 consecutive keys of the key sequence in time order (the
# resident frames oldest first -- sinks, then the recent window -- then the segments), so which
# keys share a scale depends only on the resident frames, never on where the ring buffer wraps;
# P and V stay bf16/fp32 as in the plain path.
# --------------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code):
    """Real value of e4m3 codes (uint8): sign, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2^-6); 0x7f / 0xff are NaN."""
    c = np.asarray(code).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e4m3_round(x):
    """Nearest e4m3 code of float32 values with |x| <= 448 (ties to the even mantissa).
    The quantum is 2^(e-3) for a value in [2^e, 2^(e+1)), e >= -6, and 2^-9 below 2^-6."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_round takes finite values with |x| <= 448")
    _, ex = np.frexp(a)                     # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.exp2(e - 3.0)
    n = np.rint(a / quantum)                # exact division by a power of two; rint ties to even
    # n lies in [8, 16] for normals (16: carried into the next binade), [0, 8] below 2^-6
    carry = n >= 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, n / 2, n)
    normal = n >= 8
    field = np.where(normal, e + 7, 0)
    mant = np.where(normal, n - 8, n)
    code = (field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_e4m3_blocks(x, rows):
    """Per-block FP8 quantization of x [n][H][D] (float32 or bf16 bits): blocks of ``rows``
    consecutive rows per head (the last one zero-padded).  In fp32: scale = amax / 448,
    inv = 448 / amax, code = e4m3(clamp(x * inv, -448, 448)); an all-zero block has scale 0
    and zero codes.  Returns codes [nb][H][rows][D] (uint8) and scales [nb][H] (float32)."""
    x = widen(x)
    n, H, D = x.shape
    nb = -(-n // rows)
    xp = np.zeros((nb * rows, H, D), np.float32)
    xp[:n] = x
    xb = xp.reshape(nb, rows, H, D).transpose(0, 2, 1, 3)            # [nb][H][rows][D]
    amax = np.max(np.abs(xb), axis=(2, 3)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / amax, np.float32(0)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    y = np.clip(xb * inv[:, :, None, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_round(y), scale


def dequantize_e4m3_blocks(codes, scales, n):
    """Inverse layout of ``quantize_e4m3_blocks``: fp64 [n][H][D] = value(code) * scale."""
    nb, H, rows, D = codes.shape
    v = e4m3_value(codes) * scales.astype(np.float64)[:, :, None, None]
    return v.transpose(0, 2, 1, 3).reshape(nb * rows, H, D)[:n]


def attend_dense_f64(q, k, v, scale):
    """Unmasked softmax attention of fp64 q [nq][H][D] over k, v [nk][H][D], in numpy fp64
    (two passes: row max, then exponentials, sum and weighted values)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    out = np.zeros(q.shape, np.float64)
    if k.shape[0] == 0:
        return out
    for hh in range(q.shape[1]):
        s = (q[:, hh, :] @ k[:, hh, :].T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, hh, :] = (p @ v[:, hh, :]) / p.sum(axis=1, keepdims=True)
    return out


def qk8_key_sequence(cache, segments):
    """Keys and values in the order the 64-key scale blocks are cut along: the resident
    frames in time order (the sinks, then the recent window, oldest first), then each
    segment."""
    ks, vs = [], []
    if cache is not None:
        kc, vc = cache.logical_kv()
        ks.append(kc)
        vs.append(vc)
    for k, v in segments:
        ks.append(np.asarray(k))
        vs.append(np.asarray(v))
    return np.concatenate([widen(x) for x in ks]), np.concatenate([widen(x) for x in vs])


def chunk_attention_qk8(cache, q, segments, scale, rows=None):
    """Chunk attention with the FP8-quantized QK^T: Q quantized in blocks of 32 rows, K in
    blocks of 64 keys of the time-ordered key sequence, softmax and P V exact (fp64) on the
    dequantized scores.  ``rows`` selects query rows (default: all).  Returns fp64."""
    k_all, v_all = qk8_key_sequence(cache, segments)
    q32 = widen(q)
    qc, qs = quantize_e4m3_blocks(q32, 32)
    kc, ks = quantize_e4m3_blocks(k_all, 64)
    qd = dequantize_e4m3_blocks(qc, qs, q32.shape[0])
    kd = dequantize_e4m3_blocks(kc, ks, k_all.shape[0])
    if rows is not None:
        qd = qd[np.asarray(rows)]
    return attend_dense_f64(qd, kd, v_all, scale)


# --------------------------------------------------------------------------------------------
# MoBA backward: gradients of the masked attention w.r.t. q, k, v (the training use of the MoBA
# mask, "Infinite Worlds with Versatile Interactions", causal pretraining paragraph).  The pages
# state no backward; this is the derivative of the forward above, written out per head:
#   S = scale Q K^T (masked entries -inf),  P = softmax_rows(S) (an empty row is 0),  O = P V,
#   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P * (dP - D),
#   dQ = scale dS K,  dK = scale dS^T Q.
# The forward for training also returns lse_i = log sum_j exp(S_ij) (natural log; -inf for a
# row with no key).
# --------------------------------------------------------------------------------------------

def mask_from_row_intervals(intervals, nk):
    """Dense boolean mask [nq][nk] from per-row lists of half-open key ranges."""
    m = np.zeros((len(intervals), nk), dtype=bool)
    for i, ivs in enumerate(intervals):
        for a, b in ivs:
            m[i, a:b] = True
    return m


def attention_lse(q, k, mask, scale):
    """lse [H][nq] (fp64) of the masked scores: log sum_j exp(scale q_i . k_j) over allowed j."""
    q = widen(q).astype(np.float64)
    k = widen(k).astype(np.float64)
    out = np.empty((q.shape[1], q.shape[0]), np.float64)
    for hh in range(q.shape[1]):
        s = np.where(mask, (q[:, hh, :] @ k[:, hh, :].T) * scale, -np.inf)
        mx = s.max(axis=1)
        safe = np.where(np.isfinite(mx), mx, 0.0)
        out[hh] = safe + np.log(np.exp(s - safe[:, None]).sum(axis=1))
    return out


def attention_backward(q, k, v, dout, mask, scale):
    """(dq, dk, dv), each fp64 with the shape of its input, of L = sum(dout * O) for the
    masked attention O = softmax(scale q k^T) v, dense per head."""
    q, k, v, do = (widen(x).astype(np.float64) for x in (q, k, v, dout))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for hh in range(q.shape[1]):
        Q, K, V, dO = q[:, hh, :], k[:, hh, :], v[:, hh, :], do[:, hh, :]
        s = np.where(mask, (Q @ K.T) * scale, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
        den = e.sum(axis=1, keepdims=True)
        p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
        o = p @ V
        dv[:, hh, :] = p.T @ dO
        dp = dO @ V.T
        dsum = (dO * o).sum(axis=1, keepdims=True)
        ds = p * (dp - dsum)
        dq[:, hh, :] = scale * (ds @ K)
        dk[:, hh, :] = scale * (ds.T @ Q)
    return dq, dk, dv


def attention_by_runs(q, k, v, row_intervals, scale, heads=None, block=1024):
    """Masked softmax attention in fp64 with dense BLAS products, for checks of every row of
    long sequences: rows are taken in runs that share their allowed key ranges
    ``row_intervals(i)`` (a MoBA chunk, a chunk of queries over the whole cache), and each
    block of a run attends its allowed keys as one dense, unmasked softmax (two passes: row
    max, then exponentials, sums and weighted values).  A row with no key gets 0.
    q: [nq][H][D], k, v: [nk][H][D] (float32 or bf16 bits); ``heads`` selects heads.
    Returns fp64 [nq][len(heads)][D]."""
    q, k, v = (widen(x) for x in (q, k, v))
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    nq, D = q.shape[0], q.shape[2]
    out = np.zeros((nq, len(heads), D), np.float64)
    runs = []
    for i in range(nq):
        ivs = tuple((int(a), int(b)) for a, b in row_intervals(i) if b > a)
        if runs and runs[-1][2] == ivs:
            runs[-1][1] = i + 1
        else:
            runs.append([i, i + 1, ivs])
    for r0, r1, ivs in runs:
        if not ivs:
            continue
        allowed = np.concatenate([np.arange(a, b) for a, b in ivs])
        for x, hh in enumerate(heads):
            K = k[allowed, hh].astype(np.float64)
            V = v[allowed, hh].astype(np.float64)
            for b0 in range(r0, r1, block):
                b1 = min(b0 + block, r1)
                s = (q[b0:b1, hh].astype(np.float64) @ K.T) * scale
                e = np.exp(s - s.max(axis=1, keepdims=True))
                out[b0:b1, x] = (e @ V) / e.sum(axis=1, keepdims=True)
    return out


def attention_key_gradients(q, k, v, dout, row_intervals, keys, scale, block=1024):
    """Exact (fp64) dk and dv at the key rows ``keys`` only, for the masked attention in
    which query row i may attend the half-open key ranges ``row_intervals(i)`` -- the same
    derivative as ``attention_backward``, without a dense mask: for the query rows that
    attend a listed key, each row's softmax (its log-sum-exp, its output O and
    D = dO . O) is formed over its own allowed keys, and then
    dv_j = sum_i P_ij dO_i,  dk_j = scale sum_i P_ij (dO_i . v_j - D_i) q_i.
    Rows are taken in runs that share their intervals (a MoBA chunk, for instance).
    q, k, v, dout: [n][H][D] (float32 or bf16 bits).  Returns (dk, dv), each
    [len(keys)][H][D] fp64, in the order of ``keys``."""
    q, k, v, do = (widen(x) for x in (q, k, v, dout))
    n, H, D = q.shape
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((keys.size, H, D), np.float64)
    dv = np.zeros((keys.size, H, D), np.float64)
    runs = []
    for i in range(n):
        ivs = tuple((int(a), int(b)) for a, b in row_intervals(i) if b > a)
        if runs and runs[-1][2] == ivs:
            runs[-1][1] = i + 1
        else:
            runs.append([i, i + 1, ivs])
    for r0, r1, ivs in runs:
        if not ivs:
            continue
        allowed = np.concatenate([np.arange(a, b) for a, b in ivs])
        hit = np.isin(keys, allowed)
        if not hit.any():
            continue
        jpos = np.searchsorted(allowed, keys[hit])
        for hh in range(H):
            K = k[allowed, hh].astype(np.float64)
            V = v[allowed, hh].astype(np.float64)
            VJ = V[jpos]
            for b0 in range(r0, r1, block):
                b1 = min(b0 + block, r1)
                Q = q[b0:b1, hh].astype(np.float64)
                dO = do[b0:b1, hh].astype(np.float64)
                s = (Q @ K.T) * scale
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                O = (e @ V) / l
                Dsum = (dO * O).sum(axis=1, keepdims=True)
                P = e[:, jpos] / l
                dS = P * (dO @ VJ.T - Dsum)
                dv[hit, hh] += P.T @ dO
                dk[hit, hh] += scale * (dS.T @ Q)
    return dk, dv


def moba_mask(tokens_per_frame, frames, chunk_frames, bidir_block=1):
    n = (2 + bidir_block) * frames * tokens_per_frame
    ivs = [moba_row_intervals(i, tokens_per_frame, frames, chunk_frames, bidir_block) for i in range(n)]
    return mask_from_row_intervals(ivs, n)


def moba_attention_backward(q, k, v, dout, tokens_per_frame, frames, chunk_frames, bidir_block, scale):
    """Gradients of the MoBA-masked attention (dense; for sequences the oracle holds whole)."""
    return attention_backward(q, k, v, dout, moba_mask(tokens_per_frame, frames, chunk_frames, bidir_block), scale)
