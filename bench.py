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
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_bf16_832x464_hbm_counters.txt")
ATTN_SOURCE = os.path.join(ROOT, "kv_cache_attention_02_amd", "csrc", "attn_bf16.hip")

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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--occupancy-scan", action="store_true",
                    help="also time the attention kernel at 32, 256 and 2048 workgroups (12 heads' shape, "
                         "27136 keys): per-step time against occupancy (pair with a GRBM_GUI_ACTIVE counter pass "
                         "to read the shader clock)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def events_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def pmc_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    src_hash = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()[:16]
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

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def fill(shape, **key):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        synth.gpu_fill(t.data_ptr(), t.numel(), seed=args.seed, stream=sptr, **key)
        return t

    nq = CF * TPF
    kv_tokens = (S + W + CF) * TPF
    flops = 4.0 * D * H * nq * kv_tokens                 # allowed pairs x 4 * head_dim
    append_bytes = 2.0 * 2 * nq * H * D * 2              # K + V chunk, read + write

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

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    append_ms = np.array(events_ms([(e[0], e[1]) for e in evs]))
    attn_ms = np.array(events_ms([(e[1], e[2]) for e in evs]))
    attn_avg = float(attn_ms.mean())
    slots, F = cache.slots(0)
    assert sum(s >= 0 for s in slots) == S + W, slots

    # append/evict kernel throughput: back-to-back launches between one event
    # pair (the per-step brackets above also hold the dispatch gap)
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
            "us_back_to_back": round(append_b2b_us, 2),
            "GBps": round(append_bytes / (append_b2b_us * 1e-6) / 1e9, 1),
            "frac_hbm": round(append_bytes / (append_b2b_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "us_in_step_avg": round(float(append_ms.mean()) * 1e3, 2),
            "us_in_step_median": round(float(np.median(append_ms)) * 1e3, 2),
        },
        "ms_per_chunk_step_attention_only": round(attn_avg, 4),
    }

    if args.copy_calibration:
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 2 * n

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
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
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
        for i in range(4):
            kf = fill((nq, heads, D), chunk=i, step=4, kind=synth.KFIN)
            vf = fill((nq, heads, D), chunk=i, step=4, kind=synth.VFIN)
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
        avg_a, mn_a = timed(lambda: c.append_evict(0, kf, vf, CF))
        res["720p_append_evict"] = {"us_avg": round(avg_a * 1e3, 1), "GBps": round(ab / avg_a / 1e6, 1),
                                    "frac_hbm": round(ab / avg_a / 1e6 / PEAK_HBM_GBPS, 4)}
        ke, ve = fill((512, heads, D), kind=synth.KENV), fill((512, heads, D), kind=synth.VENV)
        kl, vl = fill((512, heads, D), chunk=2, kind=synth.KLOC), fill((512, heads, D), chunk=2, kind=synth.VLOC)
        cflops = 4.0 * D * heads * nq * 1024
        avg, mn = timed(lambda: wmk.chunk_attention(None, 0, q, [(ke, ve), (kl, vl)], out=o))
        res["720p_cross"] = {"ms_avg": round(avg, 4), "ms_min": round(mn, 4), "tflops": round(cflops / avg / 1e9, 1),
                             "frac_peak": round(cflops / avg / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del c, q, k, v, o
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
        fin = [tuple(fill((nq, H, D), chunk=i, step=4, kind=t) for t in (synth.KFIN, synth.VFIN)) for i in range(2)]
        ro = torch.empty((nq, H, D), dtype=torch.bfloat16, device=dev)

        def chunk(ci):
            for st in range(steps):
                for l in range(layers):
                    rq, rk, rv = pool[(st + l) % 2]
                    wmk.chunk_attention(rc, l, rq, [(rk, rv)], out=ro)
            for l in range(layers):
                rc.append_evict(l, fin[ci % 2][0], fin[ci % 2][1], CF)

        for ci in range(4):  # warm the cache to 14 resident frames
            for l in range(layers):
                rc.append_evict(l, fin[ci % 2][0], fin[ci % 2][1], CF)
        chunk(4)
        torch.cuda.synchronize()
        n_chunks = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for ci in range(n_chunks):
            chunk(5 + ci)
        e1.record(stream)
        torch.cuda.synchronize()
        per_chunk = e0.elapsed_time(e1) / n_chunks
        chunk_flops = layers * steps * 4.0 * D * H * nq * (S + W + CF) * TPF
        res["rolling_832x464_steady_chunk"] = {
            "ms_per_chunk": round(per_chunk, 2), "calls_per_chunk": layers * steps, "appends_per_chunk": layers,
            "tflops": round(chunk_flops / per_chunk / 1e9, 1),
            "ms_per_60_chunk_session_at_steady_rate": round(60 * per_chunk, 1)}
        del rc, pool, fin, ro
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
    """The oracle (fp64 C, OpenMP, as it stands) on a bounded sample of the same
    workload: a few query rows of the 832x464 step against all 27144 keys."""
    import numpy as np

    import oracle
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    cm = oracle.CacheModel(S, W, TPF, H, D)
    for c in range(4):
        kf = synth.normal(nq * H * D, seed=args.seed, chunk=c, step=4, kind=synth.KFIN).reshape(nq, H, D)
        vf = synth.normal(nq * H * D, seed=args.seed, chunk=c, step=4, kind=synth.VFIN).reshape(nq, H, D)
        cm.append(kf, vf, CF)
    qh = synth.normal(nq * H * D, seed=args.seed, chunk=4, kind=synth.Q).reshape(nq, H, D)
    kh = synth.normal(nq * H * D, seed=args.seed, chunk=4, kind=synth.K).reshape(nq, H, D)
    vh = synth.normal(nq * H * D, seed=args.seed, chunk=4, kind=synth.V).reshape(nq, H, D)
    oracle.chunk_attention(cm, qh, [(kh, vh)], 1 / math.sqrt(D), rows=np.arange(8))   # warm-up
    rows = np.arange(64)
    t0 = time.perf_counter()
    oracle.chunk_attention(cm, qh, [(kh, vh)], 1 / math.sqrt(D), rows=rows)
    dt = time.perf_counter() - t0
    n = int(min(nq, max(64, 64 * args.cpu_seconds / max(dt, 1e-3))))
    rows = np.linspace(0, nq - 1, n).astype(np.int64)
    t0 = time.perf_counter()
    oracle.chunk_attention(cm, qh, [(kh, vh)], 1 / math.sqrt(D), rows=rows)
    dt = time.perf_counter() - t0
    sample_flops = flops * n / nq
    return {"value": round(sample_flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {nq} query rows x {H} heads of the 832x464 step against all {kv_tokens} keys "
                      f"({dt:.1f} s, fp64)",
            "ms_per_chunk_step_extrapolated": round(dt * 1e3 * nq / n, 1),
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
