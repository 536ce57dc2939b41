"""GPU parity with an attention sink: token 0 of every sequence stays FP16 in its
own ring slot and the groups start at token 1. Packed groups and the FP16 window
(sink included) bit for bit, outputs within 2e-3 of the float64 oracle, through
both the two-call path (append, decode) and the one-call decode step."""
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


def _two_call(w, contexts, steps, dev, check_every=1):
    contexts = np.asarray(contexts, dtype=np.int64)
    p = Pair(w, int(contexts.max()) + steps + 1, dev, torch)
    print(f"case sink {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} bits={w.bits} "
          f"R={w.residual} rot={w.rotate} ctx={contexts.tolist()[:8]} steps={steps}", flush=True)
    p.append(contexts)
    p.check_state()
    p.check_decode()
    for s in range(steps):
        p.append(np.ones(w.batch, dtype=np.int64))
        if (s + 1) % check_every == 0 or s == steps - 1:
            p.check_state()
            p.check_decode()


@pytest.mark.parametrize("R", [0, 32])
@pytest.mark.parametrize("T", [1, 2, 32, 33, 34, 64, 65, 66, 97, 98])
def test_sink_edge_lengths(dev, R, T):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=1, residual=R, sink=True, name=f"sink_R{R}")
    _two_call(w, [T], 2, dev)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sink_llama_shape(dev, bits):
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=2, bits=bits, sink=True, name="sink_llama")
    _two_call(w, [1000, 1001], 40, dev, check_every=8)


def test_sink_ragged_rotated(dev):
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=5, sink=True, name="sink_rot")
    ctx = np.random.default_rng(41).integers(1, 500, size=5)
    _two_call(w, ctx, 35, dev, check_every=7)


def test_sink_many_splits(dev):
    w = wl.WORKLOADS["million_1m"].scaled(sink=True, name="sink_1m")
    p = Pair(w, 9000, dev, torch, groups_per_split=8)
    print("case sink million_1m reduced T=8193", flush=True)
    p.append([8193])
    p.check_state()
    p.check_decode()


def test_sink_first_appends_one_token_at_a_time(dev):
    # the sink arrives alone, then the window fills and flushes token by token
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=3, residual=32, sink=True, name="sink_tok")
    p = Pair(w, 400, dev, torch)
    print("case sink one token at a time", flush=True)
    for s in range(140):
        p.append([1, 1 if s % 2 else 0, 2])
        if s % 10 == 9:
            p.check_state()
            p.check_decode()


def _step(p, n_tokens):
    w = p.w
    n_tokens = np.asarray(n_tokens, dtype=np.int64)
    k, v = wl.kv_batch(w, p.T, max(int(n_tokens.max()), 1), n_tokens)
    q = wl.queries(w, p.step)
    p.step += 1
    out = p.gpu.step(to_dev(k, torch, p.dev), to_dev(v, torch, p.dev), to_dev(q, torch, p.dev),
                     n_tokens=n_tokens.tolist())
    p.ref.append(k, v, n_tokens)
    p.T += n_tokens
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    err = float(np.abs(got - p.ref.decode(q)).max())
    assert np.all(np.isfinite(got)) and err <= OUT_TOL, f"step {p.step}: max |gpu - oracle| = {err:.3e}"


@pytest.mark.parametrize("rotate", [False, True])
def test_sink_decode_step_from_empty(dev, rotate):
    # the first one-call step appends the sink itself (folded into the decode launch
    # without rotation, through the separate window write with it)
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=4, num_q_heads=8, num_kv_heads=4, residual=32,
                                                   rotate=rotate, sink=True, name="sink_step")
    p = Pair(w, 1200, dev, torch)
    print(f"case sink step rotate={rotate}", flush=True)
    rng = np.random.default_rng(61)
    _step(p, [1, 5, 40, 100])
    for s in range(30):
        _step(p, rng.integers(0, 30, size=4) if s % 4 == 3 else [1, 1, 1, 1])
        if s % 6 == 5:
            p.check_state()
    p.check_state()


def test_sink_changes_output_only_by_what_the_oracle_says(dev):
    # with and without the sink the caches differ (token 0 exact vs quantized with
    # its group); each matches its own oracle and the two outputs are not identical
    outs = []
    for sink in (False, True):
        w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=1, residual=32, sink=sink, name=f"sink{int(sink)}")
        p = Pair(w, 600, dev, torch)
        p.append([500])
        got, exp = p.decode()
        assert float(np.abs(got - exp).max()) <= OUT_TOL
        outs.append(got)
    assert not np.array_equal(outs[0], outs[1])
