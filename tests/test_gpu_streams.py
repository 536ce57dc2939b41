"""GPU parity with the library driven from a side stream. The cache is created,
prefilled and stepped while a non-default stream (default priority) is torch's
current stream; outputs and cache state are read on the default stream only after
it waits for the side stream, with no device-wide synchronization in between. Every
library call enqueues its work on the stream it is given, so the results equal the
oracle's: outputs within 2e-3, packed groups and FP16 window bit for bit."""
import numpy as np
import pytest

import kvq_workloads as wl
from parity_helpers import OUT_TOL, Pair, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("one_call", [True, False])
def test_side_stream_prefill_and_steps(dev, one_call):
    w = wl.WORKLOADS["gqa_128k_2bit"]  # 32 query / 8 KV heads, 2-bit, R 128
    B = w.batch
    ctx = 2000
    steps = 40  # crosses a group flush (2000 - 128 tokens quantized, one more every 32 steps)
    print(f"case side stream {w.name} ctx={ctx} steps={steps} one_call={one_call}", flush=True)
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        p = Pair(w, ctx + steps + 8, dev, torch)
        p.append([ctx] * B)
    ones = np.ones(B, dtype=np.int64)
    worst = 0.0
    for s in range(steps):
        k, v = wl.kv_batch(w, p.T, 1, ones)
        q = wl.queries(w, s)
        with torch.cuda.stream(side):
            kd, vd, qd = to_dev(k, torch, dev), to_dev(v, torch, dev), to_dev(q, torch, dev)
            if one_call:
                out = p.gpu.step(kd, vd, qd, n_tokens=ones.tolist())
            else:
                p.gpu.append(kd, vd, ones.tolist())
                out = p.gpu.decode(qd)
        p.ref.append(k, v, ones)
        p.T += ones
        main.wait_stream(side)
        got = out.cpu().numpy().astype(np.float64)  # copy on the default stream
        exp = p.ref.decode(q)
        err = float(np.abs(got - exp).max())
        assert np.all(np.isfinite(got)) and err <= OUT_TOL, f"step {s}: max |gpu - oracle| = {err:.3e}"
        worst = max(worst, err)
    main.wait_stream(side)
    p.check_state()
    p.gpu.close()
    print(f"worst {worst:.3e}", flush=True)


def test_two_caches_on_two_streams_interleaved(dev):
    """Two caches of different shapes and widths (2-bit 32/8 heads, 4-bit 8/8 heads
    with sink and pre-RoPE keys) stepped in turn on two side streams, with no
    synchronization between their launches: each matches its own oracle, so the
    library keeps no state shared between caches that their calls could race on."""
    base = wl.WORKLOADS["gqa_128k_2bit"]
    other = wl.Workload("mha_4bit_sink_rope", 2, 8, 8, 0, 0, 4, 32, 64, False, 2, 8.0, 2.0, 4242,
                        sink=True, rope=True)
    ctx, steps = 1200, 36
    print(f"case two caches on two streams ctx={ctx} steps={steps}", flush=True)
    main = torch.cuda.current_stream(dev)
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    pairs = []
    for w, st in zip((base, other), streams):
        with torch.cuda.stream(st):
            p = Pair(w, ctx + steps + 8, dev, torch)
            p.append([ctx] * w.batch)
        pairs.append(p)
    for s in range(steps):
        outs = []
        for p, st in zip(pairs, streams):
            w = p.w
            ones = np.ones(w.batch, dtype=np.int64)
            k, v = wl.kv_batch(w, p.T, 1, ones)
            q = wl.queries(w, s)
            with torch.cuda.stream(st):
                out = p.gpu.step(to_dev(k, torch, dev), to_dev(v, torch, dev), to_dev(q, torch, dev),
                                 n_tokens=ones.tolist())
            p.ref.append(k, v, ones)
            p.T += ones
            outs.append((p, out, q))
        for st in streams:
            main.wait_stream(st)
        for p, out, q in outs:
            got = out.cpu().numpy().astype(np.float64)
            err = float(np.abs(got - p.ref.decode(q)).max())
            assert np.all(np.isfinite(got)) and err <= OUT_TOL, f"{p.w.name} step {s}: max |gpu - oracle| = {err:.3e}"
    for st in streams:
        main.wait_stream(st)
    for p in pairs:
        p.check_state()
        p.gpu.close()
