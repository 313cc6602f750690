"""Benchmark of the sink + window KV-cache chunk step on one MI355X.

Workload (the 18-slot 832x464 step): 1508 tokens per latent frame (52x29),
12 heads x 128, bf16; 6 sink + 8 window frames resident, current chunk of 4
frames -> Q 6032 tokens attending 27144 keys.  One step = append/evict of a
finalized 4-frame chunk (the ring advances; 14 frames stay resident) followed
by the chunk attention of the next chunk's queries.  Inputs are seeded
synthetic ~N(0,1) draws, resident in HBM before timing.

Printed: one JSON line with the headline throughput (TFLOP/s of allowed
(q, k) pairs, 4 * head_dim flops each), ms per chunk-step, the attention
kernel's roofline fraction measured with HIP events on the launch stream, the
append kernel's HBM bandwidth, the other workloads (MoBA training sequence,
720p self- and cross-attention) and the CPU oracle's rate on a bounded sample.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
CLOCK_WARMUP_S = 0.15       # untimed work before each measurement (see clock_warmup)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_bf16_832x464_hbm_counters.txt")
# the attention kernel's sources: a change to any of them voids the committed counter figures
ATTN_SOURCES = [os.path.join(ROOT, "kv_cache_attention_02_amd", "csrc", f)
                for f in ("attn_bf16.hip", "attn_tiles.h", "fastdiv.h", "wmk_internal.h")]


def kernel_sources_hash():
    """sha256[:16] of the attention kernel's source files, concatenated in ATTN_SOURCES order."""
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]

S, W, CF, TPF, H, D = 6, 8, 4, 1508, 12, 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-extra", action="store_true", help="skip the other workloads (same as --extra none)")
    ap.add_argument("--extra", default="all",
                    help="other workloads to run, comma separated: moba, moba_bwd, 720p, qk8, retained, rolling, "
                         "cross_train "
                         "(or all, none)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="query rows of the CPU oracle run (0: the whole call, all 6032 rows)")
    ap.add_argument("--occupancy-scan", action="store_true",
                    help="also time the attention kernel at 32, 256 and 2048 workgroups (12 heads' shape, "
                         "27136 keys): per-step time against occupancy (pair with a GRBM_GUI_ACTIVE counter pass "
                         "to read the shader clock)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--append-only", action="store_true",
                    help="run only the rolling-session append/evict loop (30 layers, distinct sources and slots; "
                         "for counter runs) and print its timing")
    ap.add_argument("--append-workload", default="rolling", choices=["rolling", "720p", "layers30"],
                    help="append timed by --append-only: the 832x464 rolling session (74 MB per append), the "
                         "720p step's append (354 MB: 4 distinct finalized chunks in turn), or the rolling "
                         "session's 30 appends of one chunk as one multi-layer call (2.2 GB)")
    ap.add_argument("--step-profile", action="store_true",
                    help="run the 832x464 call on the step-profile build of the library (libwmk_stepprof.so: "
                         "per-wave shader cycles of each phase of a 64-key step) and print the per-step budget")
    ap.add_argument("--profile-workload", default="832x464", choices=["832x464", "720p_cross", "832x464_qk8"],
                    help="call profiled by --step-profile: the 832x464 step, the 720p chunk's cross-attention "
                         "(14400 queries x 24 heads over a 512-token environment and a 512-token local prompt), "
                         "or the 832x464 step with the FP8 QK^T (the whole call's time includes its two "
                         "quantization passes)")
    ap.add_argument("--skip-rates", action="store_true",
                    help="skip the reference rates (MFMA microbenchmark, device-to-device copy)")
    ap.add_argument("--rates-only", action="store_true",
                    help="run only the reference rates (MFMA stream, device-to-device copy, fp32 atomic adds) "
                         "and print them")
    return ap.parse_args()


def events_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def clock_warmup(fn, torch, seconds=CLOCK_WARMUP_S):
    """Call fn(i) for i = 0, 1, ... until `seconds` of wall time have passed with the
    GPU kept busy (a few calls stay queued; the host waits every 4 calls) and return
    the number of calls.  The shader clock ramps up over the first ~10-20 ms of
    sustained load; without this the first timed calls run slower."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def pmc_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    src_hash = kernel_sources_hash()
    vals = {}
    for line in open(PMC_SUMMARY):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def rolling_appends(wmk, synth, torch, fill, stream, reps=4):
    """Append/evict as the rolling session runs it: a 30-layer 832x464 cache (3.9 GB of
    K and V) warmed to 14 resident frames, then one 4-frame append per layer from that
    layer's own finalized chunk (30 distinct 37 MB sources, 1.1 GB), back to back.  The
    working set (sources plus the slots written) is far above the 256 MB Infinity Cache,
    so the bytes really move to and from HBM.  Returns microseconds per append."""
    layers = 30
    nq = CF * TPF
    cache = wmk.Cache(num_layers=layers, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S,
                      window_frames=W, chunk_frames=CF)
    src = [(fill((nq, H, D), layer=l, step=4, kind=synth.KFIN), fill((nq, H, D), layer=l, step=4, kind=synth.VFIN))
           for l in range(layers)]

    def sweep():
        for l in range(layers):
            cache.append_evict(l, src[l][0], src[l][1], CF)

    for _ in range(4):  # 16 frames appended: 14 resident, the ring has wrapped
        sweep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        sweep()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * layers)
    del cache, src
    torch.cuda.empty_cache()
    return us, layers * reps


def appends_720p(wmk, synth, torch, fill, stream, reps=4):
    """The 720p step's append/evict (4 frames of 3600 tokens x 24 heads x 128: 177 MB read +
    177 MB written), from 4 distinct finalized chunks in turn (708 MB of sources) into the
    alternating halves of the window: a working set far beyond the 256 MB Infinity Cache.
    4 warm-up appends, then 4 * reps back to back between two events.  Returns microseconds
    per append, the number timed and the bytes per append."""
    tpf, heads = 3600, 24
    nq = CF * tpf
    cache = wmk.Cache(num_layers=1, num_heads=heads, head_dim=D, tokens_per_frame=tpf, sink_frames=S,
                      window_frames=W, chunk_frames=CF)
    fin = [(fill((nq, heads, D), chunk=i, step=4, kind=synth.KFIN), fill((nq, heads, D), chunk=i, step=4,
                                                                          kind=synth.VFIN)) for i in range(4)]
    for kf, vf in fin:
        cache.append_evict(0, kf, vf, CF)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(4 * reps):
        cache.append_evict(0, *fin[i % 4], CF)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (4 * reps)
    del cache, fin
    torch.cuda.empty_cache()
    return us, 4 * reps, 2.0 * 2 * nq * heads * D * 2


def appends_30_layers_one_call(wmk, synth, torch, fill, stream, reps=4):
    """The rolling session's appends of one finalized chunk to all 30 layers of the 832x464
    cache as one wmk_cache_append_evict_layers call (copy_layers_kernel): 30 distinct 37 MB
    sources (1.1 GB, one [30][6032][12][128] tensor each for K and V) into a 3.9 GB cache,
    2.2 GB moved per call, far beyond the 256 MB Infinity Cache.  4 warm-up calls, then
    `reps` back to back between two events.  Returns microseconds per call and the bytes
    per call."""
    layers = 30
    nq = CF * TPF
    cache = wmk.Cache(num_layers=layers, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S,
                      window_frames=W, chunk_frames=CF)
    ks, vs = (torch.empty((layers, nq, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    for l in range(layers):  # generated in place (no copy kernels beside the calibration copies)
        fill(None, out=ks[l], layer=l, step=4, kind=synth.KFIN)
        fill(None, out=vs[l], layer=l, step=4, kind=synth.VFIN)
    for _ in range(4):  # 16 frames appended: 14 resident, the ring has wrapped
        cache.append_evict_layers(0, ks, vs, CF)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        cache.append_evict_layers(0, ks, vs, CF)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del cache, ks, vs
    torch.cuda.empty_cache()
    return us, 2.0 * 2 * layers * nq * H * D * 2


def step_profile(wmk, synth, torch, np, fill, stream, flops, workload="832x464"):
    """A call on the step-profile build: per wave, the shader cycles of each phase of its
    64-key steps -- [A] (S^T of the next tile on the matrix core beside this tile's
    second-half weights), [B] (P V beside the next tile's row max and first-half weights),
    the wait for the step's own direct loads, the barrier, and the issue code before [A] --
    averaged per step, over the full units and over the split tail's pieces; waves 0-3 and
    4-7 (the two waves of each SIMD of an 8-wave workgroup) separately (a call of short key
    walks runs the 4-wave shape, whose records 4-7 stay empty); the unit's fill (entry to the first step);
    and the shader clock from the same span on the 100 MHz real-time counter.
    workload: the 832x464 step, or the 720p chunk's cross-attention."""
    import ctypes
    if workload == "720p_cross":
        tpf, heads = 3600, 24
        nq = CF * tpf
        q = fill((nq, heads, D), chunk=4, kind=synth.Q)
        segs = [(fill((512, heads, D), kind=synth.KENV), fill((512, heads, D), kind=synth.VENV)),
                (fill((512, heads, D), chunk=2, kind=synth.KLOC), fill((512, heads, D), chunk=2, kind=synth.VLOC))]
        cache = None
        flops = 4.0 * D * heads * nq * 1024
    else:
        nq = CF * TPF
        cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S,
                          window_frames=W, chunk_frames=CF)
        for c in range(4):
            cache.append_evict(0, fill((nq, H, D), chunk=c, step=4, kind=synth.KFIN),
                               fill((nq, H, D), chunk=c, step=4, kind=synth.VFIN), CF)
        q, k, v = (fill((nq, H, D), chunk=4, kind=t) for t in (synth.Q, synth.K, synth.V))
        segs = [(k, v)]
    out = torch.empty_like(q)
    if workload == "832x464_qk8":
        call = lambda: wmk.chunk_attention_qk8(cache, 0, q, segs, out=out)  # noqa: E731
    else:
        call = lambda: wmk.chunk_attention(cache, 0, q, segs, out=out)  # noqa: E731
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    call()
    e1.record(stream)
    torch.cuda.synchronize()
    lib = wmk.load()
    lib.wmk_step_profile_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    buf = np.zeros((4096 * 8, 16), np.uint64)
    assert lib.wmk_step_profile_read(buf.ctypes.data, buf.nbytes) == 0
    wg = buf.astype(np.float64).reshape(4096, 8, 16)
    used = wg[:, :, 5].sum(axis=1) > 0
    piece = (buf.reshape(4096, 8, 16)[:, 0, 7] & np.uint64(255)) != np.uint64(255)
    names = ["A_qk_next_and_weights", "B_pv_and_next_max_weights", "wait_own_loads", "barrier", "issue_before_A"]
    res = {"library": "libwmk_stepprof.so", "workload": workload, "call_ms": round(e0.elapsed_time(e1), 4),
           "call_tflops": round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)}
    for label, sel in (("full_units", used & ~piece), ("split_pieces", used & piece)):
        if not sel.any():
            continue
        x = wg[sel]
        part = {"workgroups": int(sel.sum())}
        for waves, tag in ((slice(0, 8), "all_waves"), (slice(0, 4), "waves_0_3"), (slice(4, 8), "waves_4_7")):
            y = x[:, waves].reshape(-1, 16)
            y = y[y[:, 5] > 0]
            if not len(y):  # a 4-wave kernel (short units) fills records 0-3 of each workgroup only
                continue
            per = {nm: round(float(np.mean(y[:, i] / y[:, 5])), 1) for i, nm in enumerate(names)}
            per["phases_sum"] = round(sum(per.values()), 1)
            per["cycles_per_step_span"] = round(float(np.mean(y[:, 6] / y[:, 5])), 1)
            if tag == "all_waves":
                per["steps_per_wave"] = round(float(np.mean(y[:, 5])), 1)
                per["fill_cycles_entry_to_first_step"] = round(float(np.mean(y[:, 9])), 1)
                per["fill_parts"] = {nm: round(float(np.mean(y[:, 10 + i])), 1) for i, nm in enumerate(
                    ["setup_and_q_loads_issued", "first_tiles_issued_and_waited", "barrier_1", "first_scores_and_weights",
                     "barrier_2", "of_setup_until_the_unit_is_known"])}
                per["shader_clock_GHz"] = round(float(np.mean(y[:, 6] / (y[:, 8] * 10.0))), 3)
            part[tag] = per
        res[label] = part
    del cache
    return res


def copy_calibration(torch, dev):
    """Three plain device copies of 256 MiB (torch copy_ of contiguous bytes): a kernel of
    known traffic (256 MiB read and 256 MiB written per launch) whose HBM byte counters
    scale the counters of the kernels measured in the same run."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return 2 * n


def reference_rates(torch, stream, append_bytes):
    """Measured ceilings to read the roofline fractions against: the bf16 matrix-core rate
    of a long stream of independent 32x32x16 MFMAs (clock under sustained load included),
    and the device-to-device copy rate of hipMemcpyAsync (torch's copy_ of contiguous
    bytes) on the append's pattern -- 30 layers x (K + V) of 18.5 MB each, all distinct,
    beyond the Infinity Cache."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_attention_02_amd", "libwmk_rates.so"))
    lib.wmk_rate_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.wmk_rate_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.wmk_rate_mfma_bf16_flops.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus * 8, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    assert lib.wmk_rate_mfma_bf16(blocks, iters, sink.data_ptr(), sp) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        lib.wmk_rate_mfma_bf16(blocks, iters, sink.data_ptr(), sp)
    e1.record(stream)
    torch.cuda.synchronize()
    mfma_tflops = 3 * lib.wmk_rate_mfma_bf16_flops(blocks, iters) / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del sink
    layers, each = 30, int(append_bytes // 4)
    src = torch.empty(layers * 2 * each, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)

    def copies():
        for l in range(2 * layers):
            dst[l * each:(l + 1) * each].copy_(src[l * each:(l + 1) * each])

    copies()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(3):
        copies()
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 3 * 2 * 2 * layers * each / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    # fp32 atomic adds (no return) in the dQ-accumulation pattern of a fused backward:
    # 32 KiB blocks (64 rows x 128 dims, row stride 12 heads) at random 64-row tiles
    lib.wmk_rate_atomic_add_f32.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p]
    n_tiles, heads, ablocks, rounds = 1536, 12, 4608, 32
    acc = torch.zeros(n_tiles * 64 * heads * 128, dtype=torch.float32, device="cuda")
    assert lib.wmk_rate_atomic_add_f32(acc.data_ptr(), n_tiles, heads, ablocks, rounds, sp) == 0
    torch.cuda.synchronize()
    e0.record(stream)
    lib.wmk_rate_atomic_add_f32(acc.data_ptr(), n_tiles, heads, ablocks, rounds, sp)
    e1.record(stream)
    torch.cuda.synchronize()
    atomic_gbps = ablocks * rounds * 64 * 128 * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del acc
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma_tflops, 1),
            "mfma_kernel": f"wmk_rate_mfma_bf16: {blocks} workgroups x 4 waves x {iters} x 4 independent "
                           "v_mfma_f32_32x32x16_bf16",
            "d2d_copy_GBps": round(copy_gbps, 1),
            "d2d_copy": f"hipMemcpyAsync (torch copy_) of {2 * layers} distinct {each / 1e6:.1f} MB ranges",
            "atomic_add_f32_GBps": round(atomic_gbps, 1),
            "atomic_add": f"wmk_rate_atomic_add_f32: {ablocks} x {rounds} blocks of 64 x 128 fp32 added at random "
                          f"64-row tiles of a [{n_tiles * 64}][{heads}][128] buffer"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by heads with no "
              "exchange inside it, so one GPU's share is what is measured.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_attention_02_amd as wmk
    import synth

    if args.step_profile:
        wmk.LIB_PATH = os.path.join(ROOT, "kv_cache_attention_02_amd", "libwmk_stepprof.so")

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def fill(shape, out=None, **key):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev) if out is None else out
        synth.gpu_fill(t.data_ptr(), t.numel(), seed=args.seed, stream=sptr, **key)
        return t

    nq = CF * TPF
    kv_tokens = (S + W + CF) * TPF
    flops = 4.0 * D * H * nq * kv_tokens                 # allowed pairs x 4 * head_dim
    append_bytes = 2.0 * 2 * nq * H * D * 2              # K + V chunk, read + write

    if args.step_profile:
        print(json.dumps(step_profile(wmk, synth, torch, np, fill, stream, flops, args.profile_workload)))
        return

    if args.rates_only:
        rates = reference_rates(torch, stream, append_bytes)
        rates["rates_source_sha256_16"] = hashlib.sha256(
            open(os.path.join(ROOT, "kv_cache_attention_02_amd", "csrc", "rates.hip"), "rb").read()).hexdigest()[:16]
        print(json.dumps(rates))
        return

    if args.append_only:
        if args.append_workload == "720p":
            us, n, nbytes = appends_720p(wmk, synth, torch, fill, stream, reps=args.steps)
            res = {"append_evict_720p_us": round(us, 2), "appends": n, "bytes_per_append": nbytes,
                   "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                   "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        elif args.append_workload == "layers30":
            us, nbytes = appends_30_layers_one_call(wmk, synth, torch, fill, stream, reps=args.steps)
            res = {"append_evict_30_layers_one_call_us": round(us, 2), "calls": args.steps,
                   "bytes_per_call": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                   "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        else:
            us, n = rolling_appends(wmk, synth, torch, fill, stream, reps=args.steps)
            res = {"append_evict_rolling_us": round(us, 2), "appends": n,
                   "GBps": round(append_bytes / (us * 1e-6) / 1e9, 1),
                   "frac_hbm": round(append_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        if args.copy_calibration:
            res["copy_calibration_bytes"] = copy_calibration(torch, dev)
        print(json.dumps(res))
        return

    # ---- resident inputs: a cache warmed to 14 frames plus a pool of finalized chunks
    cache = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S,
                      window_frames=W, chunk_frames=CF)
    pool = 4
    kfin = [fill((nq, H, D), chunk=c, step=4, kind=synth.KFIN) for c in range(pool)]
    vfin = [fill((nq, H, D), chunk=c, step=4, kind=synth.VFIN) for c in range(pool)]
    for c in range(4):
        cache.append_evict(0, kfin[c], vfin[c], CF)
    q = [fill((nq, H, D), chunk=4 + i, kind=synth.Q) for i in range(2)]
    k = [fill((nq, H, D), chunk=4 + i, kind=synth.K) for i in range(2)]
    v = [fill((nq, H, D), chunk=4 + i, kind=synth.V) for i in range(2)]
    out = torch.empty((nq, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        cache.append_evict(0, kfin[i % pool], vfin[i % pool], CF)
        if ev is not None:
            ev[1].record(stream)
        wmk.chunk_attention(cache, 0, q[i % 2], [(k[i % 2], v[i % 2])], out=out)
        if ev is not None:
            ev[2].record(stream)

    # clock warm-up: the shader clock climbs to its loaded level over the first ~10-20 ms of
    # sustained work (measured: 0.94 ms per attention call after 5 steps, 0.89 after 100), so
    # the same step runs for CLOCK_WARMUP_S before the counted warm-up steps; it is reported
    # in the JSON line as clock_warmup
    n_clock = clock_warmup(step, torch)
    for i in range(args.warmup):
        step(n_clock + i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(n_clock + args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    append_ms = np.array(events_ms([(e[0], e[1]) for e in evs]))
    attn_ms = np.array(events_ms([(e[1], e[2]) for e in evs]))
    attn_avg = float(attn_ms.mean())
    slots, F = cache.slots(0)
    assert sum(s >= 0 for s in slots) == S + W, slots

    # append/evict kernel throughput in the rolling session's pattern (30 layers,
    # distinct sources and destinations: real HBM traffic), and back to back on
    # this one-layer cache (4 pooled sources: a working set that fits in the
    # Infinity Cache) for comparison
    roll_us, roll_n = rolling_appends(wmk, synth, torch, fill, stream)
    layers_us, layers_bytes = appends_30_layers_one_call(wmk, synth, torch, fill, stream)
    n_app = 50
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for i in range(n_app):
        cache.append_evict(0, kfin[i % pool], vfin[i % pool], CF)
    eb.record(stream)
    torch.cuda.synchronize()
    append_b2b_us = ea.elapsed_time(eb) * 1e3 / n_app

    result = {
        "metric": "ms/chunk-step + TFLOP/s of sink+window KV-cache attention; % bf16 MFMA peak",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "clock_warmup": {"steps": n_clock, "seconds": CLOCK_WARMUP_S,
                         "why": "untimed steps before the counted warm-up, so that the timed steps run at the "
                                "loaded steady-state shader clock rather than during its ramp"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "832x464 chunk step, 18 slots (6 anchor + 8 recent + 4 current frames), "
                               "append/evict + chunk attention",
                   "tokens_per_frame": TPF, "heads": H, "head_dim": D, "q_tokens": nq, "kv_tokens": kv_tokens,
                   "sink_frames": S, "window_frames": W, "chunk_frames": CF},
        "roofline": {
            "bound": "mfma",
            "achieved": round(flops / (attn_avg * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / (attn_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": pmc_traffic(),
            "kernel": "attn_bf16_kernel<128> + attn_merge_kernel<128> (one call: the split tail's merge runs "
                      "as a second short kernel; both are in the event bracket)",
            "launch_ms_avg": round(attn_avg, 4),
            "launch_ms_median": round(float(np.median(attn_ms)), 4),
            "launch_ms_min": round(float(attn_ms.min()), 4),
            "flops_per_launch": flops,
        },
        "append_evict": {
            "kernel": "copy_ranges_kernel",
            "bytes_per_launch": append_bytes,
            "workload": f"rolling session: {roll_n} appends over 30 layers of a 3.9 GB cache, each from its own "
                        "37 MB source (working set beyond the Infinity Cache)",
            "us_avg": round(roll_us, 2),
            "GBps": round(append_bytes / (roll_us * 1e-6) / 1e9, 1),
            "frac_hbm": round(append_bytes / (roll_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "us_one_layer_4_sources_in_cache": round(append_b2b_us, 2),
            "all_30_layers_one_call": {
                "kernel": "copy_layers_kernel (wmk_cache_append_evict_layers)",
                "bytes_per_call": layers_bytes,
                "us_per_call": round(layers_us, 2),
                "GBps": round(layers_bytes / (layers_us * 1e-6) / 1e9, 1),
                "frac_hbm": round(layers_bytes / (layers_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            },
            "us_in_step_avg": round(float(append_ms.mean()) * 1e3, 2),
            "us_in_step_median": round(float(np.median(append_ms)) * 1e3, 2),
        },
        "ms_per_chunk_step_attention_only": round(attn_avg, 4),
    }

    if not args.skip_rates:
        rates = reference_rates(torch, stream, append_bytes)
        rates["attention_frac_of_mfma_rate"] = round(result["roofline"]["achieved"] / rates["mfma_bf16_tflops"], 4)
        rates["append_frac_of_d2d_copy"] = round(result["append_evict"]["GBps"] / rates["d2d_copy_GBps"], 4)
        result["reference_rates"] = rates

    if args.copy_calibration:
        result["copy_calibration_bytes"] = copy_calibration(torch, dev)

    if args.occupancy_scan:
        result["occupancy_scan"] = occupancy_scan(wmk, synth, torch, fill)

    extra = set() if args.skip_extra or args.extra == "none" else (
        {"moba", "moba_bwd", "720p", "qk8", "retained", "rolling", "cross_train"} if args.extra == "all" else set(args.extra.split(",")))
    if extra:
        result["other_workloads"] = other_workloads(wmk, synth, torch, np, fill, dev, stream, reps=5, which=extra)

    del cache, kfin, vfin, q, k, v, out
    torch.cuda.empty_cache()
    if not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline(args, flops, nq, kv_tokens)
    print(json.dumps(result))


def occupancy_scan(wmk, synth, torch, fill):
    """Chunk attention over 27136 keys (424 tiles, no cache, no split tail) at grid sizes
    32 (one head, 32 q-tiles: 32 CUs busy), 256 (8 heads x 32 q-tiles: every CU once) and
    2048 (8 rounds): time per 64-key step of a workgroup."""
    nkv, res = 27136, {}
    for heads, nq in ((1, 8192), (8, 8192), (8, 65536)):
        q = fill((nq, heads, D), kind=synth.Q)
        k, v = fill((nkv, heads, D), kind=synth.K), fill((nkv, heads, D), kind=synth.V)
        o = torch.empty_like(q)
        for _ in range(2):
            wmk.chunk_attention(None, 0, q, [(k, v)], out=o, use_workspace=False)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            wmk.chunk_attention(None, 0, q, [(k, v)], out=o, use_workspace=False)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        wgs = heads * nq // 256
        rounds = -(-wgs // 256)
        res[f"{wgs}_workgroups"] = {"ms": round(ms, 4), "us_per_step": round(ms * 1e3 / (rounds * nkv // 64), 3),
                                    "tflops": round(4.0 * D * heads * nq * nkv / ms / 1e9, 1)}
        del q, k, v, o
    return res


def other_workloads(wmk, synth, torch, np, fill, dev, stream, reps, which):
    res = {}

    def timed(fn):
        """Mean and min of the calls issued back to back, each between two events on
        the stream: one call is enqueued ahead, so the host's launch work for the next
        call overlaps the running one and the events see GPU time only (a wait for the
        host between calls would add ~20-30 us to each sub-millisecond call).  The same
        call first runs for CLOCK_WARMUP_S (the clock ramps up under sustained load), and
        short calls are repeated until ~20 ms are timed (at least `reps`, at most 100)."""
        n_warm = clock_warmup(lambda i: fn(), torch)
        per_call = CLOCK_WARMUP_S / max(n_warm, 1)
        reps_t = max(reps, min(100, int(0.02 / per_call)))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps_t + 1)]
        fn()
        evs[0].record(stream)
        for i in range(reps_t):
            fn()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(reps_t)]
        return float(np.mean(ms)), float(np.min(ms))

    if "moba" in which:
        # MoBA training sequence: 21 clean + 21 noisy + 21 block frames of 1560 tokens, chunks of 3
        tpf, frames, cf = 1560, 21, 3
        n = 3 * frames * tpf
        mq, mk, mv = (fill((n, H, D), kind=t) for t in (synth.Q, synth.K, synth.V))
        mo = torch.empty_like(mq)
        pairs = 945 * tpf * tpf
        mflops = 4.0 * D * H * pairs
        avg, mn = timed(lambda: wmk.moba_attention(mq, mk, mv, tokens_per_frame=tpf, frames=frames, chunk_frames=cf,
                                                   out=mo))
        res["moba_98280"] = {"ms_avg": round(avg, 3), "ms_min": round(mn, 3), "tflops": round(mflops / avg / 1e9, 1),
                             "frac_peak": round(mflops / avg / 1e9 / PEAK_BF16_TFLOPS, 4),
                             "allowed_pairs_per_head": pairs, "dense_fraction": round(945 / 3969, 4)}
        del mq, mk, mv, mo

    if "moba_bwd" in which:
        # MoBA training step on the same sequence: forward with log-sum-exp, then the
        # backward (dq, dk, dv); FLOPs of the backward counted as 2.5x the forward's
        # (five products per allowed pair instead of two)
        tpf, frames, cf = 1560, 21, 3
        n = 3 * frames * tpf
        bq, bk, bv, bdo = (fill((n, H, D), kind=t) for t in (synth.Q, synth.K, synth.V, synth.KLOC))
        bo, blse = wmk.moba_attention_train(bq, bk, bv, tokens_per_frame=tpf, frames=frames, chunk_frames=cf)
        fwd_flops = 4.0 * D * H * 945 * tpf * tpf
        avg_f, mn_f = timed(lambda: wmk.moba_attention_train(bq, bk, bv, tokens_per_frame=tpf, frames=frames,
                                                             chunk_frames=cf, out=bo, lse=blse))
        avg_b, mn_b = timed(lambda: wmk.moba_attention_backward(bq, bk, bv, bo, bdo, blse, tokens_per_frame=tpf,
                                                                frames=frames, chunk_frames=cf))
        res["moba_98280_train"] = {
            "fwd_ms_avg": round(avg_f, 3), "bwd_ms_avg": round(avg_b, 3), "bwd_ms_min": round(mn_b, 3),
            "fwd_tflops": round(fwd_flops / avg_f / 1e9, 1),
            "bwd_tflops": round(2.5 * fwd_flops / avg_b / 1e9, 1),
            "bwd_frac_peak": round(2.5 * fwd_flops / avg_b / 1e9 / PEAK_BF16_TFLOPS, 4),
            "bwd_flops": 2.5 * fwd_flops}
        del bq, bk, bv, bdo, bo, blse
        torch.cuda.empty_cache()

    if "720p" in which:
        # 720p step: 3600 tokens per frame, 24 heads, 18 slots; chunk-causal cross-attention
        tpf, heads = 3600, 24
        c = wmk.Cache(num_layers=1, num_heads=heads, head_dim=D, tokens_per_frame=tpf, sink_frames=S, window_frames=W,
                      chunk_frames=CF)
        nq = CF * tpf
        fin = [(fill((nq, heads, D), chunk=i, step=4, kind=synth.KFIN),
                fill((nq, heads, D), chunk=i, step=4, kind=synth.VFIN)) for i in range(4)]
        for kf, vf in fin:
            c.append_evict(0, kf, vf, CF)
        q, k, v = (fill((nq, heads, D), chunk=4, kind=t) for t in (synth.Q, synth.K, synth.V))
        o = torch.empty_like(q)
        kv = (S + W + CF) * tpf
        sflops = 4.0 * D * heads * nq * kv
        avg, mn = timed(lambda: wmk.chunk_attention(c, 0, q, [(k, v)], out=o))
        res["720p_self"] = {"ms_avg": round(avg, 3), "ms_min": round(mn, 3), "tflops": round(sflops / avg / 1e9, 1),
                            "frac_peak": round(sflops / avg / 1e9 / PEAK_BF16_TFLOPS, 4), "q_tokens": nq,
                            "kv_tokens": kv}
        ab = 2.0 * 2 * nq * heads * D * 2
        # the four finalized chunks in turn (708 MB of sources, 354 MB of window slots
        # written): a working set beyond the 256 MB Infinity Cache
        turn = iter(range(1 << 30))
        avg_a, mn_a = timed(lambda: c.append_evict(0, *fin[next(turn) % 4], CF))
        res["720p_append_evict"] = {"us_avg": round(avg_a * 1e3, 1), "GBps": round(ab / avg_a / 1e6, 1),
                                    "frac_hbm": round(ab / avg_a / 1e6 / PEAK_HBM_GBPS, 4),
                                    "workload": "4 distinct 177 MB sources in turn into alternating window halves"}
        ke, ve = fill((512, heads, D), kind=synth.KENV), fill((512, heads, D), kind=synth.VENV)
        kl, vl = fill((512, heads, D), chunk=2, kind=synth.KLOC), fill((512, heads, D), chunk=2, kind=synth.VLOC)
        cflops = 4.0 * D * heads * nq * 1024
        avg, mn = timed(lambda: wmk.chunk_attention(None, 0, q, [(ke, ve), (kl, vl)], out=o))
        res["720p_cross"] = {"ms_avg": round(avg, 4), "ms_min": round(mn, 4), "tflops": round(cflops / avg / 1e9, 1),
                             "frac_peak": round(cflops / avg / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del c, q, k, v, o, fin
        torch.cuda.empty_cache()

    if "qk8" in which:
        # FP8-quantized QK^T at 832x464: warm cache + the current chunk; one call =
        # quantization of Q and of the key sequence, then the attention kernel
        c8 = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S, window_frames=W,
                       chunk_frames=CF)
        nq8 = CF * TPF
        for i in range(4):
            c8.append_evict(0, fill((nq8, H, D), chunk=i, step=4, kind=synth.KFIN),
                            fill((nq8, H, D), chunk=i, step=4, kind=synth.VFIN), CF)
        q8, k8, v8 = (fill((nq8, H, D), chunk=4, kind=t) for t in (synth.Q, synth.K, synth.V))
        o8 = torch.empty_like(q8)
        f8 = 4.0 * D * H * nq8 * (S + W + CF) * TPF
        avg, mn = timed(lambda: wmk.chunk_attention_qk8(c8, 0, q8, [(k8, v8)], out=o8))
        res["832x464_qk8"] = {"ms_avg": round(avg, 4), "ms_min": round(mn, 4), "tflops": round(f8 / avg / 1e9, 1),
                              "frac_peak_bf16": round(f8 / avg / 1e9 / PEAK_BF16_TFLOPS, 4),
                              "note": "QK^T in fp8 e4m3 (per-block scales, quantization passes included), P V in bf16"}
        del c8, q8, k8, v8, o8
        torch.cuda.empty_cache()

    if "retained" in which:
        # variable retention at 832x464: of the 14 resident frames keep the 6 anchors and
        # the 4 most recent (in 3 runs of adjacent slots after the ring wrapped) + the chunk
        cr = wmk.Cache(num_layers=1, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S, window_frames=W,
                       chunk_frames=CF)
        nqr = CF * TPF
        for i in range(5):
            cr.append_evict(0, fill((nqr, H, D), chunk=i, step=4, kind=synth.KFIN),
                            fill((nqr, H, D), chunk=i, step=4, kind=synth.VFIN), CF)
        slots_r, _ = cr.slots(0)
        keep = sorted(f for f in slots_r if f >= 0)
        keep = keep[:S] + keep[-4:]
        qr, kr, vr = (fill((nqr, H, D), chunk=5, kind=t) for t in (synth.Q, synth.K, synth.V))
        orr = torch.empty_like(qr)
        fr = 4.0 * D * H * nqr * (len(keep) * TPF + nqr)
        avg, mn = timed(lambda: wmk.chunk_attention(cr, 0, qr, [(kr, vr)], out=orr, keep_frames=keep))
        res["832x464_retained_10_of_14"] = {"ms_avg": round(avg, 4), "ms_min": round(mn, 4),
                                            "tflops": round(fr / avg / 1e9, 1),
                                            "frac_peak": round(fr / avg / 1e9 / PEAK_BF16_TFLOPS, 4),
                                            "kv_tokens": len(keep) * TPF + nqr, "kept_frames": keep}
        del cr, qr, kr, vr, orr
        torch.cuda.empty_cache()

    if "rolling" in which:
        # rolling session at 832x464: 30 layers x 4 denoising steps per chunk over a
        # full 18-slot cache, then the finalized chunk appended to every layer
        layers, steps = 30, 4
        nq = CF * TPF
        rc = wmk.Cache(num_layers=layers, num_heads=H, head_dim=D, tokens_per_frame=TPF, sink_frames=S,
                       window_frames=W, chunk_frames=CF)
        pool = [tuple(fill((nq, H, D), chunk=i, kind=t) for t in (synth.Q, synth.K, synth.V)) for i in range(2)]
        # each layer appends its own finalized chunk (30 distinct sources, as in a real session),
        # all 30 in one wmk_cache_append_evict_layers call after the chunk's last step
        fk, fv = (torch.empty((layers, nq, H, D), dtype=torch.bfloat16, device=dev) for _ in range(2))
        for l in range(layers):
            fill(None, out=fk[l], layer=l, step=4, kind=synth.KFIN)
            fill(None, out=fv[l], layer=l, step=4, kind=synth.VFIN)
        ro = torch.empty((nq, H, D), dtype=torch.bfloat16, device=dev)

        app_ev = []

        def chunk(ci, ev=False):
            for st in range(steps):
                for l in range(layers):
                    rq, rk, rv = pool[(st + l) % 2]
                    wmk.chunk_attention(rc, l, rq, [(rk, rv)], out=ro)
            if ev:
                app_ev.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                app_ev[-1][0].record(stream)
            rc.append_evict_layers(0, fk, fv, CF)
            if ev:
                app_ev[-1][1].record(stream)

        for ci in range(4):  # warm the cache to 14 resident frames
            rc.append_evict_layers(0, fk, fv, CF)
        chunk(4)
        torch.cuda.synchronize()
        n_chunks = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for ci in range(n_chunks):
            chunk(5 + ci, ev=True)
        e1.record(stream)
        torch.cuda.synchronize()
        per_chunk = e0.elapsed_time(e1) / n_chunks
        app_us = float(np.mean([a.elapsed_time(b) for a, b in app_ev])) * 1e3
        chunk_flops = layers * steps * 4.0 * D * H * nq * (S + W + CF) * TPF
        res["rolling_832x464_steady_chunk"] = {
            "ms_per_chunk": round(per_chunk, 2), "calls_per_chunk": layers * steps,
            "appends_per_chunk": f"{layers} layers in one wmk_cache_append_evict_layers call",
            "tflops": round(chunk_flops / per_chunk / 1e9, 1),
            "ms_per_chunk_attention": round(per_chunk - app_us * 1e-3, 2),
            "us_append_all_layers": round(app_us, 2),
            "append_frac_hbm": round(layers * 4.0 * nq * H * D * 2 / (app_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "ms_per_60_chunk_session_at_steady_rate": round(60 * per_chunk, 1)}
        del rc, pool, fk, fv, ro
        torch.cuda.empty_cache()

    if "cross_train" in which:
        # chunk-causal cross-attention over a training sequence: the MoBA shape's 7
        # chunks of 3 frames x 1560 tokens, each reading a 512-token environment
        # prompt and its own 512-token local prompt (12 heads)
        tpf, heads, cq, nc, ne, nl = 1560, 12, 3 * 1560, 7, 512, 512
        q = fill((cq * nc, heads, D), kind=synth.Q)
        kx = fill((ne + nc * nl, heads, D), kind=synth.KLOC)
        vx = fill((ne + nc * nl, heads, D), kind=synth.VLOC)
        o = torch.empty_like(q)
        xflops = 4.0 * D * heads * cq * nc * (ne + nl)
        avg, mn = timed(lambda: wmk.cross_attention_train(q, kx, vx, chunk_q_tokens=cq, env_tokens=ne, local_tokens=nl,
                                                          out=o))
        res["cross_train_32760"] = {"ms_avg": round(avg, 4), "ms_min": round(mn, 4),
                                    "tflops": round(xflops / avg / 1e9, 1),
                                    "frac_peak": round(xflops / avg / 1e9 / PEAK_BF16_TFLOPS, 4),
                                    "q_tokens": cq * nc, "kv_tokens": ne + nc * nl}

    return res


def cpu_baseline(args, flops, nq, kv_tokens):
    """The oracle (fp64 C, OpenMP, as it stands) on the same workload: one whole 832x464
    chunk-attention call -- all 6032 query rows x 12 heads against all 27144 keys -- on
    every host thread OpenMP is given, plus a one-thread run of a row sample for context."""
    import ctypes

    import numpy as np

    import oracle
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    cm = oracle.CacheModel(S, W, TPF, H, D)
    for c in range(4):
        kf = synth.normal(nq * H * D, seed=args.seed, chunk=c, step=4, kind=synth.KFIN).reshape(nq, H, D)
        vf = synth.normal(nq * H * D, seed=args.seed, chunk=c, step=4, kind=synth.VFIN).reshape(nq, H, D)
        cm.append(kf, vf, CF)
    qh = synth.normal(nq * H * D, seed=args.seed, chunk=4, kind=synth.Q).reshape(nq, H, D)
    kh = synth.normal(nq * H * D, seed=args.seed, chunk=4, kind=synth.K).reshape(nq, H, D)
    vh = synth.normal(nq * H * D, seed=args.seed, chunk=4, kind=synth.V).reshape(nq, H, D)
    scale = 1 / math.sqrt(D)
    rows = np.arange(nq) if args.cpu_rows <= 0 else np.linspace(0, nq - 1, args.cpu_rows).astype(np.int64)
    t0 = time.perf_counter()
    oracle.chunk_attention(cm, qh, [(kh, vh)], scale, rows=rows)
    dt = time.perf_counter() - t0
    res = {"value": round(flops * len(rows) / nq / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": (f"one whole 832x464 call: all {nq} query rows x {H} heads against all {kv_tokens} keys "
                      if len(rows) == nq else f"{len(rows)} of {nq} query rows x {H} heads against all {kv_tokens} "
                                              "keys of the 832x464 call ") + f"({dt:.1f} s, fp64, {threads} threads)",
           "ms_per_chunk_step": round(dt * 1e3 * nq / len(rows), 1),
           "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}
    # one thread, on a row sample (the whole call would take minutes)
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        sample = np.linspace(0, nq - 1, 48).astype(np.int64)
        t0 = time.perf_counter()
        oracle.chunk_attention(cm, qh, [(kh, vh)], scale, rows=sample)
        dt1 = time.perf_counter() - t0
        gomp.omp_set_num_threads(threads)
        res["one_thread"] = {"value": round(flops * len(sample) / nq / dt1 / 1e12, 6), "unit": "TFLOP/s",
                             "sample": f"{len(sample)} of {nq} query rows ({dt1:.1f} s)",
                             "ms_per_chunk_step_extrapolated": round(dt1 * 1e3 * nq / len(sample), 1)}
    except OSError:
        pass
    # the same oracle on row samples of the other workloads (all threads), extrapolated to a
    # whole call by allowed (query, key) pairs, and the rolling session by calls
    res["other_workloads_extrapolated"] = cpu_other_workloads(args, res["value"])
    return res


def cpu_other_workloads(args, step_tflops):
    """Oracle rates on row samples of the MoBA training sequence and the 720p step, with the
    whole call's time extrapolated from the sample's allowed pairs; the rolling session's
    steady chunk (120 calls of the 832x464 step) from the whole-call rate above."""
    import numpy as np

    import oracle
    import synth

    out = {}
    # MoBA: 21 + 21 + 21 frames of 1560 tokens, chunks of 3, 12 heads
    tpf, frames, cf = 1560, 21, 3
    n = 3 * frames * tpf
    q, k, v = (synth.normal(n * H * D, seed=args.seed, kind=t).reshape(n, H, D) for t in (synth.Q, synth.K, synth.V))
    rows = np.linspace(0, n - 1, 480).astype(np.int64)
    pairs = sum(b - a for i in rows for a, b in oracle.moba_row_intervals(int(i), tpf, frames, cf))
    t0 = time.perf_counter()
    oracle.moba_attention(q, k, v, tpf, frames, cf, 1, 1 / math.sqrt(D), rows=rows)
    dt = time.perf_counter() - t0
    rate = 4.0 * D * H * pairs / dt / 1e12
    total = 4.0 * D * H * 945 * tpf * tpf
    out["moba_98280"] = {"tflops": round(rate, 5), "sample": f"{len(rows)} of {n} rows ({dt:.1f} s)",
                         "s_per_call_extrapolated": round(total / rate / 1e12, 1)}
    del q, k, v
    # 720p: 14 resident frames + the 14400-token chunk (64800 keys), 24 heads
    tpf, heads = 3600, 24
    nq, nk = CF * tpf, (S + W + CF) * tpf
    q = synth.normal(nq * heads * D, seed=args.seed, kind=synth.Q).reshape(nq, heads, D)
    k = synth.normal(nk * heads * D, seed=args.seed, kind=synth.K).reshape(nk, heads, D)
    v = synth.normal(nk * heads * D, seed=args.seed, kind=synth.V).reshape(nk, heads, D)
    rows = np.linspace(0, nq - 1, 160).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attend(q[rows], k, v, [[(0, nk)]] * len(rows), 1 / math.sqrt(D))
    dt = time.perf_counter() - t0
    rate = 4.0 * D * heads * len(rows) * nk / dt / 1e12
    out["720p_self"] = {"tflops": round(rate, 5), "sample": f"{len(rows)} of {nq} rows x {heads} heads against "
                                                             f"all {nk} keys ({dt:.1f} s)",
                        "s_per_call_extrapolated": round(4.0 * D * heads * nq * nk / rate / 1e12, 1)}
    del q, k, v
    call = 4.0 * D * H * CF * TPF * (S + W + CF) * TPF
    out["rolling_832x464_steady_chunk"] = {"s_per_chunk_extrapolated": round(120 * call / step_tflops / 1e12, 1),
                                           "from": "120 calls at the whole-call rate of the 832x464 step"}
    return out


def _cpu_model():
    """The host CPU: model name plus family / model / stepping numbers from /proc/cpuinfo."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "vendor_id", "cpu family", "model", "stepping") and k not in info:
                    info[k] = v
            if not line.strip() and info:
                break
    except OSError:
        return "unknown"
    return (f"{info.get('model name', 'unknown')} ({info.get('vendor_id', '?')}, family {info.get('cpu family', '?')}"
            f" model {info.get('model', '?')} stepping {info.get('stepping', '?')})")


if __name__ == "__main__":
    main()
