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
bracketing them (no per-step records). `roofline` reports the dominant kernel (the
decode split kernel), timed in a second pass of decode calls on the same caches
with HIP events that the library attaches to that kernel's launch
(hipExtLaunchKernelGGL): they carry the kernel's own start and end timestamps, as a
kernel trace reports them. Every event is created without the system-scope fence
(hipEventDisableSystemFence): a default event record writes back and invalidates the
caches, which costs several microseconds per record and lengthens the kernel it
brackets.

Steady state: cache c is prefilled with a few extra tokens (under 32) so that, when
the timed steps start, it sits 31 - 32 c / copies appends past its last group flush;
the timed steps then contain about steps / 32 group flushes, spread over the caches,
whatever the number of steps. A separate pass times single steps and reports the
steps with a group flush apart from the others.
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
EVENT_NO_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (timed on any stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p(0)
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), EVENT_NO_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
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


def steady_offsets(w, copies, warmup):
    """Extra prefill tokens per cache copy (0..31): copy c then starts the timed steps
    31 - 32 c / copies appends past its last group flush, judged on sequence 0 (all
    sequences of an equal-length workload share it; ragged ones have their own)."""
    o = 1 if w.sink else 0
    T0 = int(w.context_lengths()[0])
    out = []
    for c in range(copies):
        appends = len(range(c, warmup, copies))   # warmup steps that reach copy c
        phase = 31 - (32 * c) // copies
        out.append((phase - (T0 + appends - o - w.residual)) % 32)
    return out


def will_flush(T, w):
    """Whether appending one token to a sequence holding T tokens moves a group out
    of its FP16 window (the residual rule, as the library applies it)."""
    o = 1 if w.sink else 0
    q = lambda t: 32 * (max(0, t - o - w.residual) // 32)
    return q(T + 1) != q(T)


def build_caches(torch, kvq, w, copies, max_tokens, dev, gps, ev=None, stream=None, page_groups=0, extra=None):
    """Build `copies` caches holding the workload's prefill (appends of up to
    PREFILL_CHUNK tokens per sequence: one append for contexts up to 128K), copy c
    with extra[c] more tokens per sequence if given.
    With `ev`, each copy's appends are timed (inputs drawn beforehand) and the
    per-copy prefill times in ms are returned as well. With `page_groups`, each cache
    is paged and every sequence gets its pages in a seeded random order."""
    params = wl.torch_key_params(torch, w, dev)
    caches, times = [], []
    chunk = PREFILL_CHUNK
    for c in range(copies):
        lens = w.context_lengths() + (extra[c] if extra else 0)
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, heads=4, steps=12):
    """Time the CPU oracle on `heads` KV heads of sequence 0 at the workload's full
    context, twice: with numpy / BLAS at their default thread count and pinned to one
    thread. Per run: the prefill (quantize the whole prompt), then `steps` steps of
    append-1 + attend. The throughput `value` is the algorithmic bytes of the attended
    steps over their time at the default thread count."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import OracleHead
    ratio = w.num_q_heads // w.num_kv_heads
    T0 = int(w.context_lengths()[0])
    inputs = [(wl.keys(w, 0, h, 0, T0 + steps), wl.values(w, 0, h, 0, T0 + steps)) for h in range(heads)]
    qs = [wl.queries(w, s)[0] for s in range(steps)]

    def run():
        t0 = time.perf_counter()
        hs = []
        for h in range(heads):
            oh = OracleHead(w.bits, w.residual, w.rotate, sink=w.sink, rope=w.rope)
            oh.append(inputs[h][0][:T0], inputs[h][1][:T0])
            hs.append(oh)
        t1 = time.perf_counter()
        nbytes = 0
        for s in range(steps):
            for h, oh in enumerate(hs):
                oh.append(inputs[h][0][oh.T:oh.T + 1], inputs[h][1][oh.T:oh.T + 1])
                oh.attend(qs[s][h * ratio:(h + 1) * ratio])
                nbytes += wl.algorithmic_bytes(oh.T, oh.Q, w.bits, w.group, w.head_dim)
        t2 = time.perf_counter()
        return {"prefill_s_per_head": round((t1 - t0) / heads, 3),
                "step_s_per_head": round((t2 - t1) / (steps * heads), 3),
                "total_s": round(t2 - t0, 2), "gbps": nbytes / (t2 - t1) / 1e9}

    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    default = run()
    with threadpool_limits(1):
        single = run()
    return {"value": default["gbps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"sequence 0, kv-heads 0..{heads - 1} (each with its {ratio} query heads) of {w.name} at "
                      f"full context {T0}: prefill, then {steps} steps of append-1 + attend, run once with "
                      f"numpy/BLAS at {threads} threads and once at 1 thread",
            "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "default_threads": default, "one_thread": single}


def time_calls(ev, stream, torch, fn, iters):
    """Average µs of `iters` calls of fn(i), bracketed by one pair of events."""
    a, b = ev.create(1)[0], ev.create(1)[0]
    torch.cuda.synchronize()
    ev.record(a, stream)
    for i in range(iters):
        fn(i)
    ev.record(b, stream)
    torch.cuda.synchronize()
    us = ev.elapsed_ms(a, b) / iters * 1e3
    ev.destroy([a, b])
    return us


def measure_comparisons(torch, kvq, w, ev, stream, dev, nbytes, iters=20):
    """Achievable HBM read bandwidth (streaming-read probe: over 2 GiB, and over
    buffers of the decode's own byte count, round-robin so that none is cache
    resident) and the FP16-cache decode on the workload's shapes (same tokens per
    sequence, two caches round-robin), each timed with one pair of HIP events around
    `iters` calls."""
    res = {}
    # two workgroups of 256 threads per compute unit: the fastest grid in a sweep of
    # 1 to 64 per unit (101 MB to 2 GiB)
    fold = torch.zeros(2 * torch.cuda.get_device_properties(dev).multi_processor_count, dtype=torch.int32,
                       device=dev)
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    for _ in range(2):
        kvq.stream_read(buf, fold)
    us = time_calls(ev, stream, torch, lambda i: kvq.stream_read(buf, fold), iters)
    res["hbm_stream_read_gbps"] = round(buf.numel() / (us * 1e-6) / 1e9, 1)
    del buf
    nb = (int(nbytes) + 15) // 16 * 16
    copies = max(2, min(8, (1 << 30) // nb))
    bufs = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(copies)]
    for b_ in bufs:
        kvq.stream_read(b_, fold)
    us = time_calls(ev, stream, torch, lambda i: kvq.stream_read(bufs[i % copies], fold), 4 * iters)
    res["stream_read_same_bytes_us"] = round(us, 2)
    res["stream_read_same_bytes_gbps"] = round(nb / (us * 1e-6) / 1e9, 1)
    del bufs
    torch.cuda.empty_cache()

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
    us = time_calls(ev, stream, torch, lambda i: op(*caches[i % 2], lens_dev, t_cap, q, out), iters)
    fp16_bytes = int(lens.sum()) * w.num_kv_heads * 2 * 2 * w.head_dim
    res.update({"fp16_decode_call_us": round(us, 2), "fp16_cache_bytes": fp16_bytes,
                "fp16_decode_gbps": round(fp16_bytes / (us * 1e-6) / 1e9, 1),
                "fp16_outputs_finite": bool(torch.isfinite(out).all())})
    del caches
    torch.cuda.synchronize()
    return res


COPY_BYTES = 1 << 30
# The decode kernel's sources: its own file and the header whose device helpers (the
# group store, the sequence records) it compiles in.
KERNEL_SOURCES = [os.path.join(ROOT, "bit_asymmetric_kv_amd", "csrc", "decode.hip"),
                  os.path.join(ROOT, "bit_asymmetric_kv_amd", "csrc", "kvq_internal.h")]


def kernel_source_hash():
    """sha256 over the decode kernel's sources, in order (counter summaries carry it,
    so that they are used only for the device code they were measured on)."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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
    each scaled by the same counter's reading for the calibration copy. The result is
    merged into out_path under workloads[workload]; the copy's readings are stored
    once under "calibration" ("-" for copy_fetch and copy_write reuses them)."""
    data = {"calibration": None, "workloads": {}}
    if os.path.exists(out_path):
        with open(out_path) as f:
            old = json.load(f)
        if "workloads" in old:
            data = old
    if copy_fetch == "-" or copy_write == "-":
        cal = data["calibration"]
        if cal is None:
            raise SystemExit(f"{out_path} holds no calibration copy readings")
    else:
        f_cp, _ = _counter_per_dispatch(copy_fetch, "copy", "FETCH_SIZE")
        w_cp, _ = _counter_per_dispatch(copy_write, "copy", "WRITE_SIZE")
        cal = {"copy_bytes": COPY_BYTES, "copy_fetch_kib": f_cp, "copy_write_kib": w_cp,
               "fetch_scale": COPY_BYTES / (f_cp * 1024.0), "write_scale": COPY_BYTES / (w_cp * 1024.0)}
        data["calibration"] = cal
    f_dec, n1 = _counter_per_dispatch(dec_fetch, "decode_split_kernel", "FETCH_SIZE")
    w_dec, n2 = _counter_per_dispatch(dec_write, "decode_split_kernel", "WRITE_SIZE")
    res = {"bytes_per_launch": int(f_dec * 1024 * cal["fetch_scale"] + w_dec * 1024 * cal["write_scale"]),
           "fetch_kib_per_dispatch": f_dec, "write_kib_per_dispatch": w_dec, "dispatches": [n1, n2],
           "kernel_source_sha256": kernel_source_hash()}
    data["workloads"][workload] = res
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: res}))


def summarize_trace(trace_dir, workload, out_path):
    """Average duration of the decode split kernel in a rocprofv3 --kernel-trace --stats
    run (its kernel_stats.csv), stored in out_path under workloads[workload]["trace"]
    with the kernel source hash, so that the bench line can give the kernel's own
    time beside the event timing."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    calls = total_ns = 0
    for f in files:
        for r in csv.DictReader(open(f)):
            if "decode_split_kernel" in r["Name"]:
                calls += int(r["Calls"])
                total_ns += float(r["TotalDurationNs"])
    if not calls:
        raise SystemExit(f"no decode_split_kernel rows in the kernel stats under {trace_dir}")
    data = {"calibration": None, "workloads": {}}
    if os.path.exists(out_path):
        with open(out_path) as f:
            old = json.load(f)
        if "workloads" in old:
            data = old
    res = {"avg_us": round(total_ns / calls / 1e3, 3), "dispatches": calls, "kernel_source_sha256": kernel_source_hash()}
    data["workloads"].setdefault(workload, {})["trace"] = res
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: res}))


def _counters_per_dispatch(path, kernel_substr):
    """Every counter of the kernels matching kernel_substr under a rocprofv3 --pmc
    output folder, summed over its samples (shader engines, dies) per dispatch and
    averaged over the dispatches."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if kernel_substr in r["Kernel_Name"]:
                k = (r["Counter_Name"], r["Dispatch_Id"])
                vals[k] = vals.get(k, 0.0) + float(r["Counter_Value"])
    per = {}
    for (c, _), v in vals.items():
        per.setdefault(c, []).append(v)
    if not per:
        raise SystemExit(f"no counter samples for kernels matching {kernel_substr!r} under {path}")
    return {c: sum(v) / len(v) for c, v in per.items()}


def summarize_issue(sq1, sq2, workload, groups, waves_per_simd, out_path):
    """Instruction-issue figures of the decode split kernel from two rocprofv3 --pmc
    runs of SQ counters (the two passes of the counter summaries in profiles/):
    instructions per 32-token group and wave, and the share of the SIMDs' cycles that
    issue vector ALU work (per-wave fraction of SQ_WAVE_CYCLES times the waves that
    share a SIMD; one vector ALU per SIMD, so at most 1), and the same sum for
    instructions of any kind in progress (units overlap, so it can pass 1). Merged
    into out_path under workloads[workload]."""
    groups, waves_per_simd = int(groups), int(waves_per_simd)
    c = _counters_per_dispatch(sq1, "decode_split_kernel")
    c.update(_counters_per_dispatch(sq2, "decode_split_kernel"))
    need = ("SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY",
            "SQ_WAIT_INST_ANY")
    missing = [k for k in need if k not in c]
    if missing:
        raise SystemExit(f"counters missing from the runs: {missing}")
    wc = c["SQ_WAVE_CYCLES"]
    res = {"valu_instructions_per_group": round(c["SQ_INSTS_VALU"] / groups, 1),
           "mfma_per_group": round(c["SQ_INSTS_MFMA"] / groups, 2),
           "lds_per_group": round(c["SQ_INSTS_LDS"] / groups, 1) if "SQ_INSTS_LDS" in c else None,
           "vmem_reads_per_group": round(c["SQ_INSTS_VMEM_RD"] / groups, 2) if "SQ_INSTS_VMEM_RD" in c else None,
           "valu_active_per_wave_cycle": round(c["SQ_ACTIVE_INST_VALU"] / wc, 4),
           "any_issue_per_wave_cycle": round(c["SQ_ACTIVE_INST_ANY"] / wc, 4),
           "wait_per_wave_cycle": round(c["SQ_WAIT_INST_ANY"] / wc, 4),
           "waves_per_simd": waves_per_simd,
           "simd_valu_busy_frac": round(waves_per_simd * c["SQ_ACTIVE_INST_VALU"] / wc, 3),
           "simd_any_active_per_cycle": round(waves_per_simd * c["SQ_ACTIVE_INST_ANY"] / wc, 3),
           "groups_per_launch": groups,
           "kernel_source_sha256": kernel_source_hash()}
    data = {"workloads": {}}
    if os.path.exists(out_path):
        with open(out_path) as f:
            old = json.load(f)
        if "workloads" in old:
            data = old
    data["workloads"][workload] = res
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: res}))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-issue":
        summarize_issue(*sys.argv[2:8])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--calibrate-copy":
        calibrate_copy()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-traffic":
        summarize_traffic(*sys.argv[2:8])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        summarize_trace(*sys.argv[2:5])
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--kernel-iters", type=int, default=200,
                    help="decode calls timed with events around the split kernel (roofline)")
    ap.add_argument("--workload", default="gqa_128k_2bit", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--copies", type=int, default=8, help="independent caches stepped round-robin")
    ap.add_argument("--groups-per-split", type=int, default=0)
    ap.add_argument("--page-groups", type=int, default=0,
                    help="paged caches with this many groups per page (pages in random order)")
    ap.add_argument("--flush-split-steps", type=int, default=96,
                    help="single steps timed one by one, steps with a group flush reported apart (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparisons", action="store_true",
                    help="skip the streaming-read probe and the FP16-cache decode")
    ap.add_argument("--warm-iters", type=int, default=30,
                    help="extra decode calls on one cache to report a last-level-cache-resident time (0: skip)")
    ap.add_argument("--issue-json", default=os.path.join(ROOT, "profiles", "issue.json"),
                    help="instruction-issue figures from rocprofv3 SQ counters (--summarize-issue)")
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
    copies = args.copies
    extra = steady_offsets(w, copies, args.warmup)
    n_split = max(0, args.flush_split_steps)
    n2 = min(args.steps, 64)
    total_steps = args.warmup + args.steps + n_split + n2
    max_tokens = int(w.context_lengths().max()) + 32 + total_steps + 1
    print(f"[bench] building {copies} caches of {w.name}", file=sys.stderr, flush=True)
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    caches, params, prefill_ms = build_caches(torch, kvq, w, copies, max_tokens, dev, args.groups_per_split,
                                              ev, stream, args.page_groups, extra)
    # Prefill-side quantization throughput: every copy's prefill appends, timed.
    lens0 = w.context_lengths()
    rates = []
    for c in range(copies):
        lens_c = lens0 + extra[c]
        out_b = sum(wl.algorithmic_bytes(int(t), 32 * (max(0, int(t) - (1 if w.sink else 0) - w.residual) // 32),
                                         w.bits, w.group, w.head_dim) for t in lens_c) * w.num_kv_heads
        rates.append((int(lens_c.sum()), out_b, prefill_ms[c]))
    sel = rates[1:] if copies > 1 else rates   # the first copy's appends also warm the kernels up
    pf_tokens, pf_out, pf_ms = sorted(sel, key=lambda r: r[2])[len(sel) // 2]
    pf_in_bytes = pf_tokens * w.num_kv_heads * 2 * 2 * w.head_dim
    prefill = {"tokens_per_sequence_max": int(lens0.max()), "kv_heads": w.num_kv_heads,
               "us": round(pf_ms * 1e3, 1),
               "tokens_per_s": round(pf_tokens / (pf_ms * 1e-3), 1),
               "input_fp16_gbps": round(pf_in_bytes / (pf_ms * 1e-3) / 1e9, 1),
               "in_plus_out_gbps": round((pf_in_bytes + pf_out) / (pf_ms * 1e-3) / 1e9, 1),
               "append_tokens_max": PREFILL_CHUNK, "copies_timed": len(prefill_ms)}

    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 7919)
    knew, vnew = wl.torch_kv(torch, w, params, total_steps, gen, dev)   # [B, steps, Hkv, D]
    knew = knew.transpose(0, 1).contiguous().view(total_steps, w.batch, 1, w.num_kv_heads, w.head_dim)
    vnew = vnew.transpose(0, 1).contiguous().view(total_steps, w.batch, 1, w.num_kv_heads, w.head_dim)
    q = torch.randn((total_steps, w.batch, w.num_q_heads, w.head_dim), generator=gen, device=dev).to(torch.float16)
    outs = [torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev) for _ in caches]
    torch.cuda.synchronize()

    # Host mirror of every copy's lengths: per-step algorithmic bytes and whether the
    # step moves a group out of some sequence's window, known before any step runs.
    T = [lens0.astype(np.int64) + extra[c] for c in range(copies)]
    o = 1 if w.sink else 0
    step_info = []
    for s in range(total_steps):
        c = s % copies
        flush = any(will_flush(int(t), w) for t in T[c])
        T[c] = T[c] + 1
        nb = sum(wl.algorithmic_bytes(int(t), 32 * (max(0, int(t) - o - w.residual) // 32), w.bits, w.group,
                                      w.head_dim) for t in T[c]) * w.num_kv_heads
        step_info.append((c, flush, nb))

    # Timed region: warmup steps, then exactly `steps` steps with only the two
    # bracketing events.
    print(f"[bench] {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    t_start, t_end = ev.create(1)[0], ev.create(1)[0]
    for s in range(args.warmup):
        c = caches[s % copies]
        c.step(knew[s], vnew[s], q[s], out=outs[s % copies])
    torch.cuda.synchronize()
    ev.record(t_start, stream)
    host_t0 = time.perf_counter()
    for s in range(args.warmup, args.warmup + args.steps):
        c = caches[s % copies]
        c.step(knew[s], vnew[s], q[s], out=outs[s % copies])
    host_enqueue_s = time.perf_counter() - host_t0
    ev.record(t_end, stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(t_start, t_end)
    timed = step_info[args.warmup:args.warmup + args.steps]
    bytes_avg = float(np.mean([x[2] for x in timed]))
    flushes_timed = sum(1 for x in timed if x[1])
    ms_per_step = total_ms / args.steps
    value = bytes_avg / (ms_per_step * 1e-3) / 1e9

    # Single steps, each between its own pair of events: steps with a group flush
    # (a quantize + pack launch before the decode) apart from the others.
    flush_split = None
    s0 = args.warmup + args.steps
    if n_split:
        es, ee = ev.create(n_split), ev.create(n_split)
        for i in range(n_split):
            s = s0 + i
            c = caches[s % copies]
            ev.record(es[i], stream)
            c.step(knew[s], vnew[s], q[s], out=outs[s % copies])
            ev.record(ee[i], stream)
        torch.cuda.synchronize()
        us = np.array([ev.elapsed_ms(es[i], ee[i]) * 1e3 for i in range(n_split)])
        fl = np.array([step_info[s0 + i][1] for i in range(n_split)])
        flush_split = {"steps": n_split, "flush_steps": int(fl.sum()),
                       "no_flush_us_p50": round(float(np.median(us[~fl])), 2) if (~fl).any() else None,
                       "flush_us_p50": round(float(np.median(us[fl])), 2) if fl.any() else None,
                       "all_us_p50": round(float(np.median(us)), 2)}
        ev.destroy(es)
        ev.destroy(ee)
    s0 += n_split

    # The same step as two library calls (append, then decode), for reference.
    torch.cuda.synchronize()
    ev.record(t_start, stream)
    for i in range(n2):
        s = s0 + i
        c = caches[s % copies]
        c.append(knew[s], vnew[s])
        c.decode(q[s], outs[s % copies])
    ev.record(t_end, stream)
    torch.cuda.synchronize()
    two_call_us = ev.elapsed_ms(t_start, t_end) / n2 * 1e3
    out_ok = all(bool(torch.isfinite(o_).all()) for o_ in outs)

    # Kernel timing: decode calls on the same caches (round-robin, no appends), with
    # HIP events that the library attaches to the split kernel's launch.
    nk = args.kernel_iters
    ks, ke = ev.create(nk), ev.create(nk)
    kbytes = [step_bytes(caches[i % copies], w) for i in range(copies)]
    torch.cuda.synchronize()
    for i in range(nk):
        c = caches[i % copies]
        c.set_profile_events(ks[i], ke[i])
        c.decode(q[i % total_steps], outs[i % copies])
    torch.cuda.synchronize()
    for c in caches:
        c.set_profile_events(0, 0)
    kern_ms = np.array([ev.elapsed_ms(ks[i], ke[i]) for i in range(nk)])
    kern_avg_ms = float(np.mean(kern_ms))
    kbytes_avg = float(np.mean([kbytes[i % copies] for i in range(nk)]))
    achieved = kbytes_avg / (kern_avg_ms * 1e-3) / 1e9
    # The whole decode call (split kernel + combine kernel), the scope the FP16-cache
    # decode is compared at.
    decode_call_us = time_calls(ev, stream, torch, lambda i: caches[i % copies].decode(q[i % total_steps],
                                                                                      outs[i % copies]), nk)

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

    traffic = traced_us = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                t = json.load(f)
            # counters taken on another build of the kernel no longer describe it
            t = t.get("workloads", {}).get(w.name, {})
            if t.get("kernel_source_sha256") == kernel_source_hash():
                traffic = t.get("bytes_per_launch")
            tr = t.get("trace") or {}
            if tr.get("kernel_source_sha256") == kernel_source_hash():
                traced_us = tr.get("avg_us")
        except (OSError, ValueError):
            traffic = traced_us = None

    issue = None
    if os.path.exists(args.issue_json):
        try:
            with open(args.issue_json) as f:
                t = json.load(f).get("workloads", {}).get(w.name, {})
            if t.get("kernel_source_sha256") == kernel_source_hash():
                issue = {k: t[k] for k in ("simd_valu_busy_frac", "simd_any_active_per_cycle", "valu_instructions_per_group",
                                           "mfma_per_group", "waves_per_simd")}
                issue["source"] = "rocprofv3 SQ counters of this kernel source (profiles/issue.json)"
        except (OSError, ValueError, KeyError):
            issue = None

    comp = None
    if not args.no_comparisons:
        print("[bench] streaming-read probe and FP16-cache decode", file=sys.stderr, flush=True)
        for c in caches:
            c.close()
        del caches
        torch.cuda.empty_cache()
        comp = measure_comparisons(torch, kvq, w, ev, stream, dev, kbytes_avg)
        comp["quantized_decode_call_us"] = round(decode_call_us, 2)
        comp["quantized_vs_fp16_decode_call_speedup"] = round(comp["fp16_decode_call_us"] / decode_call_us, 2)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)
        # the whole workload's step on the CPU, estimated from the sampled heads
        cpu_step_s = cpu["default_threads"]["step_s_per_head"] * w.batch * w.num_kv_heads
        cpu["workload_step_s_estimate"] = round(cpu_step_s, 2)
        cpu["gpu_step_speedup"] = round(cpu_step_s / (ms_per_step * 1e-3), 1)

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
                   "caches_round_robin": copies, "extra_prefill_tokens": extra, "parallelism": "single GPU"},
        "step": {"algorithmic_bytes": int(bytes_avg), "frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
                 "group_flushes_timed": flushes_timed,
                 "flush_split": flush_split,
                 "two_call_us_per_step": round(two_call_us, 2),
                 "decode_call_us": round(decode_call_us, 2),
                 "decode_split_kernel_us": round(kern_avg_ms * 1e3, 2),
                 "decode_split_kernel_p10_p50_p90_us": [round(float(np.percentile(kern_ms, p)) * 1e3, 2)
                                                        for p in (10, 50, 90)],
                 "kernel_timing_calls": nk,
                 "warm_decode_attention_us": round(float(np.median(warm)) * 1e3, 2),
                 "host_enqueue_us_per_step": round(host_enqueue_s / args.steps * 1e6, 2),
                 "outputs_finite": out_ok},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": (f"decode_split_kernel<{w.bits},{w.num_q_heads // w.num_kv_heads},"
                                f"{'true' if w.rope else 'false'}>"),
                     "limiter": "vector instruction issue and latency (rocprofv3 SQ counters), below the HBM "
                                "ceiling",
                     "issue": issue,
                     # the kernel's own average duration in a rocprofv3 kernel trace of this
                     # workload and kernel source (profiles/traffic.json), and the fraction that
                     # this run's algorithmic bytes per launch give over it
                     "traced_kernel_us": traced_us,
                     "frac_traced": (round(kbytes_avg / (traced_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                                     if traced_us else None),
                     "frac_of_stream_read_2gib": (round(achieved / comp["hbm_stream_read_gbps"], 4)
                                                  if comp else None),
                     "frac_of_stream_read_same_bytes": (round(achieved / comp["stream_read_same_bytes_gbps"], 4)
                                                        if comp else None)},
        "comparison": comp,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
