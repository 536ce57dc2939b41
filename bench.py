"""Benchmark: 2-bit decode-attention step over a KIVI-style low-bit KV cache, 1 GPU.

A step is one pass of the whole hot path: append one token per sequence (FP16
window write, and a group quantize + pack whenever a group leaves the window),
then decode attention over every cached token (split kernel + combine kernel),
issued as one library call (kvq_decode_step; the window write happens inside the
decode launch). The same step as two calls (append, then decode) is reported too.

Workload (default): GQA layer, batch 1, 32 query / 8 KV heads, head_dim 128,
context 131072, 2-bit, G = 32, R = 128. Several independent caches are built and
stepped round-robin so that consecutive steps never find their cache in the
256 MB last-level cache: the reported bandwidth is HBM bandwidth.

Prints one JSON line. `value` is the effective bandwidth of a whole step:
algorithmic bytes (packed codes + fp16 scales/zero-points + fp16 window) divided
by the step time, measured over the timed steps with one pair of HIP events
bracketing them (no per-step records: each event record costs microseconds of
GPU time here). `roofline` reports the dominant kernel (the decode split kernel),
timed in a second pass of decode calls on the same caches with HIP events that the
library records around that kernel on its own stream.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kvq_workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (timed on any stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p(0)
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        f = ctypes.c_float(0)
        if self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


PREFILL_CHUNK = 131072


def build_caches(torch, kvq, w, copies, max_tokens, dev, gps, ev=None, stream=None, page_groups=0):
    """Build `copies` caches holding the workload's prefill (appends of up to
    PREFILL_CHUNK tokens per sequence: one append for contexts up to 128K).
    With `ev`, each copy's appends are timed (inputs drawn beforehand) and the
    per-copy prefill times in ms are returned as well. With `page_groups`, each cache
    is paged and every sequence gets its pages in a seeded random order."""
    params = wl.torch_key_params(torch, w, dev)
    caches, times = [], []
    lens = w.context_lengths()
    chunk = PREFILL_CHUNK
    for c in range(copies):
        paged = {}
        if page_groups:
            max_pages = -(-((max_tokens + w.group - 1) // w.group) // page_groups)
            paged = dict(page_groups=page_groups, pool_pages=w.batch * max_pages)
        cache = kvq.KVCache(w.batch, w.num_q_heads, w.num_kv_heads, bits=w.bits, group=w.group,
                            residual=w.residual, rotate=w.rotate, max_tokens=max_tokens, device=dev,
                            sink=w.sink, rope=w.rope, **paged)
        if page_groups:
            perm = np.random.default_rng(w.seed + c).permutation(w.batch * max_pages)
            for b in range(w.batch):
                cache.set_pages(b, perm[b * max_pages:(b + 1) * max_pages].tolist())
        if gps:
            cache.set_decode_split(gps)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed * 1000 + c)
        done = np.zeros(w.batch, dtype=np.int64)
        chunks = []
        while np.any(done < lens):
            n = np.minimum(lens - done, chunk)
            k, v = wl.torch_kv(torch, w, params, int(n.max()), gen, dev)
            chunks.append((k, v, n.tolist()))
            done += n
        if ev is not None:
            a, b = ev.create(1)[0], ev.create(1)[0]
            torch.cuda.synchronize()
            ev.record(a, stream)
        for k, v, n in chunks:
            cache.append(k, v, n)
        if ev is not None:
            ev.record(b, stream)
            torch.cuda.synchronize()
            times.append(ev.elapsed_ms(a, b))
            ev.destroy([a, b])
        del chunks
        caches.append(cache)
    torch.cuda.synchronize()
    if ev is not None:
        return caches, params, times
    return caches, params


def step_bytes(cache, w):
    total = 0
    for b in range(w.batch):
        T, Q = cache.seq_len(b)
        total += w.num_kv_heads * wl.algorithmic_bytes(T, Q, w.bits, w.group, w.head_dim)
    return total


def cpu_baseline(w, heads=4, steps=20):
    """Time the CPU oracle (single BLAS thread) on `heads` KV heads of sequence 0 at
    the workload's full context: per step, append one token and attend."""
    from threadpoolctl import threadpool_limits
    from oracle import OracleHead
    ratio = w.num_q_heads // w.num_kv_heads
    T0 = int(w.context_lengths()[0])
    with threadpool_limits(1):
        hs = []
        for h in range(heads):
            oh = OracleHead(w.bits, w.residual, w.rotate, sink=w.sink, rope=w.rope)
            oh.append(wl.keys(w, 0, h, 0, T0), wl.values(w, 0, h, 0, T0))
            hs.append(oh)
        nbytes = 0
        t0 = time.perf_counter()
        for s in range(steps):
            q = wl.queries(w, s)[0]
            for h, oh in enumerate(hs):
                oh.append(wl.keys(w, 0, h, oh.T, oh.T + 1), wl.values(w, 0, h, oh.T, oh.T + 1))
                oh.attend(q[h * ratio:(h + 1) * ratio])
                nbytes += wl.algorithmic_bytes(oh.T, oh.Q, w.bits, w.group, w.head_dim)
        dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"sequence 0, kv-heads 0..{heads - 1} (each with its {ratio} query heads) of "
                      f"{w.name} at full context {T0}, {steps} steps of append-1 + attend; "
                      f"{dt:.1f} s timed, numpy with one BLAS thread"}


def measure_comparisons(torch, kvq, w, ev, stream, dev, iters=20):
    """Achievable HBM read bandwidth (streaming-read probe over 2 GiB) and the FP16-
    cache decode on the workload's shapes (same tokens per sequence, two caches
    round-robin), each timed with one pair of HIP events around `iters` calls."""
    res = {}
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    fold = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        kvq.stream_read(buf, fold)
    torch.cuda.synchronize()
    a, b = ev.create(1)[0], ev.create(1)[0]
    ev.record(a, stream)
    for _ in range(iters):
        kvq.stream_read(buf, fold)
    ev.record(b, stream)
    torch.cuda.synchronize()
    res["hbm_stream_read_gbps"] = round(buf.numel() * iters / (ev.elapsed_ms(a, b) * 1e-3) / 1e9, 1)
    del buf

    lens = w.context_lengths() + 1
    t_cap = int(lens.max())
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 31)
    shape = (w.batch, w.num_kv_heads, t_cap, w.head_dim)
    caches = []
    for _ in range(2):
        k = torch.randn(shape, generator=gen, device=dev).to(torch.float16)
        v = torch.randn(shape, generator=gen, device=dev).to(torch.float16)
        caches.append((k, v))
    lens_dev = torch.tensor(lens.astype(np.int32), device=dev)
    q = torch.randn((w.batch, w.num_q_heads, w.head_dim), generator=gen, device=dev).to(torch.float16)
    op = kvq.Fp16Decode(w.batch, w.num_q_heads, w.num_kv_heads, t_cap, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    for i in range(4):
        op(*caches[i % 2], lens_dev, t_cap, q, out)
    torch.cuda.synchronize()
    ev.record(a, stream)
    for i in range(iters):
        op(*caches[i % 2], lens_dev, t_cap, q, out)
    ev.record(b, stream)
    torch.cuda.synchronize()
    us = ev.elapsed_ms(a, b) / iters * 1e3
    fp16_bytes = int(lens.sum()) * w.num_kv_heads * 2 * 2 * w.head_dim
    res.update({"fp16_decode_us": round(us, 2), "fp16_cache_bytes": fp16_bytes,
                "fp16_decode_gbps": round(fp16_bytes / (us * 1e-6) / 1e9, 1),
                "fp16_outputs_finite": bool(torch.isfinite(out).all())})
    ev.destroy([a, b])
    del caches
    torch.cuda.synchronize()
    return res


COPY_BYTES = 1 << 30
KERNEL_SOURCE = os.path.join(ROOT, "bit_asymmetric_kv_amd", "csrc", "decode.hip")


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES bytes, repeated 5 times: run under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to learn how those counters scale."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}))


def _counter_per_dispatch(path, kernel_substr, counter):
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels matching {kernel_substr!r} under {path}")
    return sum(vals.values()) / len(vals), len(vals)


def summarize_traffic(dec_fetch, dec_write, copy_fetch, copy_write, workload, out_path):
    """HBM bytes per decode split launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    each scaled by the same counter's reading for the calibration copy."""
    f_dec, n1 = _counter_per_dispatch(dec_fetch, "decode_split_kernel", "FETCH_SIZE")
    w_dec, n2 = _counter_per_dispatch(dec_write, "decode_split_kernel", "WRITE_SIZE")
    f_cp, _ = _counter_per_dispatch(copy_fetch, "copy", "FETCH_SIZE")
    w_cp, _ = _counter_per_dispatch(copy_write, "copy", "WRITE_SIZE")
    f_scale = COPY_BYTES / (f_cp * 1024.0)
    w_scale = COPY_BYTES / (w_cp * 1024.0)
    res = {"workload": workload,
           "bytes_per_launch": int(f_dec * 1024 * f_scale + w_dec * 1024 * w_scale),
           "fetch_kib_per_dispatch": f_dec, "write_kib_per_dispatch": w_dec,
           "copy_fetch_kib": f_cp, "copy_write_kib": w_cp, "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale, "dispatches": [n1, n2],
           "kernel_source_sha256": kernel_source_hash()}
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--calibrate-copy":
        calibrate_copy()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-traffic":
        summarize_traffic(*sys.argv[2:8])
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 256 steps over 8 caches: each cache takes 32 appends, so every cache moves one
    # group out of its FP16 window (one flush) inside the timed region, as in steady state.
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--kernel-iters", type=int, default=200,
                    help="decode calls timed with events around the split kernel (roofline)")
    ap.add_argument("--workload", default="gqa_128k_2bit", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--copies", type=int, default=8, help="independent caches stepped round-robin")
    ap.add_argument("--groups-per-split", type=int, default=0)
    ap.add_argument("--page-groups", type=int, default=0,
                    help="paged caches with this many groups per page (pages in random order)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparisons", action="store_true",
                    help="skip the streaming-read probe and the FP16-cache decode")
    ap.add_argument("--warm-iters", type=int, default=30,
                    help="extra decode calls on one cache to report a last-level-cache-resident time (0: skip)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters, if present")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are per-GPU and "
              f"the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_asymmetric_kv_amd as kvq
    kvq.load()
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[args.workload]
    total_steps = args.warmup + args.steps
    max_tokens = int(w.context_lengths().max()) + total_steps + 64 + 1
    print(f"[bench] building {args.copies} caches of {w.name}", file=sys.stderr, flush=True)
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    caches, params, prefill_ms = build_caches(torch, kvq, w, args.copies, max_tokens, dev, args.groups_per_split,
                                              ev, stream, args.page_groups)
    # Prefill-side quantization throughput: every copy's prefill appends, timed.
    lens = w.context_lengths()
    pf_tokens = int(lens.sum())
    pf_in_bytes = pf_tokens * w.num_kv_heads * 2 * 2 * w.head_dim
    pf_out_per_head = sum(wl.algorithmic_bytes(int(t), int(q), w.bits, w.group, w.head_dim)
                    for t, q in ((t, caches[0].seq_len(b)[1]) for b, t in enumerate(lens)))
    pf_med = float(np.median(prefill_ms[1:] if len(prefill_ms) > 1 else prefill_ms))
    prefill = {"tokens_per_sequence_max": int(lens.max()), "kv_heads": w.num_kv_heads,
               "us": round(pf_med * 1e3, 1),
               "tokens_per_s": round(pf_tokens / (pf_med * 1e-3), 1),
               "input_fp16_gbps": round(pf_in_bytes / (pf_med * 1e-3) / 1e9, 1),
               "in_plus_out_gbps": round((pf_in_bytes + pf_out_per_head * w.num_kv_heads) / (pf_med * 1e-3) / 1e9, 1),
               "append_tokens_max": PREFILL_CHUNK, "copies_timed": len(prefill_ms)}

    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 7919)
    knew, vnew = wl.torch_kv(torch, w, params, total_steps + 64, gen, dev)   # [B, steps, Hkv, D]
    knew = knew.transpose(0, 1).contiguous().view(total_steps + 64, w.batch, 1, w.num_kv_heads, w.head_dim)
    vnew = vnew.transpose(0, 1).contiguous().view(total_steps + 64, w.batch, 1, w.num_kv_heads, w.head_dim)
    knew2, vnew2 = knew[total_steps:], vnew[total_steps:]
    q = torch.randn((total_steps, w.batch, w.num_q_heads, w.head_dim), generator=gen, device=dev).to(torch.float16)
    outs = [torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev) for _ in caches]
    torch.cuda.synchronize()

    # Timed region: warmup steps, then exactly `steps` steps with only the two
    # bracketing events (per-step event records cost several microseconds each here).
    print(f"[bench] {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    nbytes = []
    t_start, t_end = ev.create(1)[0], ev.create(1)[0]
    for s in range(args.warmup):
        c = caches[s % len(caches)]
        c.step(knew[s], vnew[s], q[s], out=outs[s % len(caches)])
    torch.cuda.synchronize()
    ev.record(t_start, stream)
    host_t0 = time.perf_counter()
    for s in range(args.warmup, total_steps):
        c = caches[s % len(caches)]
        c.step(knew[s], vnew[s], q[s], out=outs[s % len(caches)])
        nbytes.append(step_bytes(c, w))
    host_enqueue_s = time.perf_counter() - host_t0
    ev.record(t_end, stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(t_start, t_end)

    # The same step as two library calls (append, then decode), for reference.
    n2 = min(args.steps, 64)
    torch.cuda.synchronize()
    ev.record(t_start, stream)
    for i in range(n2):
        s = total_steps + i
        c = caches[s % len(caches)]
        c.append(knew2[i], vnew2[i])
        c.decode(q[i], outs[s % len(caches)])
    ev.record(t_end, stream)
    torch.cuda.synchronize()
    two_call_us = ev.elapsed_ms(t_start, t_end) / n2 * 1e3
    bytes_avg = float(np.mean(nbytes))
    ms_per_step = total_ms / args.steps
    value = bytes_avg / (ms_per_step * 1e-3) / 1e9
    out_ok = all(bool(torch.isfinite(o).all()) for o in outs)

    # Kernel timing: decode calls on the same caches (round-robin, no appends), with
    # HIP events recorded around the split kernel on its stream by the library.
    nk = args.kernel_iters
    ks, ke = ev.create(nk), ev.create(nk)
    kbytes = []
    torch.cuda.synchronize()
    for i in range(nk):
        c = caches[i % len(caches)]
        c.set_profile_events(ks[i], ke[i])
        c.decode(q[i % total_steps], outs[i % len(caches)])
        kbytes.append(step_bytes(c, w))
    torch.cuda.synchronize()
    for c in caches:
        c.set_profile_events(0, 0)
    kern_ms = np.array([ev.elapsed_ms(ks[i], ke[i]) for i in range(nk)])
    kern_avg_ms = float(np.mean(kern_ms))
    achieved = float(np.mean(kbytes)) / (kern_avg_ms * 1e-3) / 1e9

    # warm (last-level-cache resident) decode of one cache, for reference only
    c = caches[0]
    qw = q[0].contiguous()
    nw = max(0, args.warm_iters)
    wst, wen = ev.create(nw), ev.create(nw)
    for i in range(nw):
        ev.record(wst[i], stream)
        c.decode(qw, outs[0])
        ev.record(wen[i], stream)
    torch.cuda.synchronize()
    warm = [ev.elapsed_ms(wst[i], wen[i]) for i in range(nw // 3, nw)] or [float("nan")]
    for e in (ks, ke, wst, wen, [t_start, t_end]):
        ev.destroy(e)

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                t = json.load(f)
            # counters taken on another build of the kernel no longer describe it
            if t.get("workload") == w.name and t.get("kernel_source_sha256") == kernel_source_hash():
                traffic = t.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    comp = None
    if not args.no_comparisons:
        print("[bench] streaming-read probe and FP16-cache decode", file=sys.stderr, flush=True)
        for c in caches:
            c.close()
        del caches
        torch.cuda.empty_cache()
        comp = measure_comparisons(torch, kvq, w, ev, stream, dev)
        comp["quantized_decode_speedup_vs_fp16"] = round(comp["fp16_decode_us"] / (kern_avg_ms * 1e3), 2)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)

    result = {
        "metric": "2-bit decode-attention µs/step + effective HBM GB/s (% of MI355X peak), 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "context": int(w.context_lengths().max()), "bits": w.bits,
                   "group": w.group, "residual": w.residual, "rotate": w.rotate, "sink": w.sink,
                   "pre_rope": w.rope, "page_groups": args.page_groups,
                   "caches_round_robin": args.copies, "parallelism": "single GPU"},
        "step": {"algorithmic_bytes": int(bytes_avg), "frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
                 "two_call_us_per_step": round(two_call_us, 2),
                 "decode_split_kernel_us": round(kern_avg_ms * 1e3, 2),
                 "decode_split_kernel_p10_p50_p90_us": [round(float(np.percentile(kern_ms, p)) * 1e3, 2)
                                                        for p in (10, 50, 90)],
                 "kernel_timing_calls": nk,
                 "warm_decode_attention_us": round(float(np.median(warm)) * 1e3, 2),
                 "host_enqueue_us_per_step": round(host_enqueue_s / args.steps * 1e6, 2),
                 "outputs_finite": out_ok},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": f"decode_split_kernel<{w.bits},{w.num_q_heads // w.num_kv_heads}>",
                     "frac_of_measured_stream_read": (round(achieved / comp["hbm_stream_read_gbps"], 4)
                                                      if comp else None)},
        "comparison": comp,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
