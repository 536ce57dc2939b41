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
