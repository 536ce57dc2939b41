"""GPU parity with pre-RoPE keys: keys are stored and quantized as given and the
decode kernel rotates every key (dequantized groups and the FP16 window) at its
position before the scores. Packed groups and the window bit for bit (they hold
the unrotated keys), outputs within 2e-3 of the float64 oracle, which applies the
rotary embedding in float64 after dequantization."""
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


def _two_call(w, contexts, steps, dev, check_every=1, gps=0):
    contexts = np.asarray(contexts, dtype=np.int64)
    p = Pair(w, int(contexts.max()) + steps + 1, dev, torch, groups_per_split=gps)
    print(f"case rope {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} bits={w.bits} "
          f"R={w.residual} sink={w.sink} ctx={contexts.tolist()[:8]} steps={steps}", flush=True)
    p.append(contexts)
    p.check_state()
    p.check_decode()
    for s in range(steps):
        p.append(np.ones(w.batch, dtype=np.int64))
        if (s + 1) % check_every == 0 or s == steps - 1:
            p.check_state()
            p.check_decode()


@pytest.mark.parametrize("R", [0, 32])
@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 64, 65, 97, 130])
def test_rope_edge_lengths(dev, R, T):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=1, residual=R, rope=True, name=f"rope_R{R}")
    _two_call(w, [T], 2, dev)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("ratio", [1, 2, 4, 8])
def test_rope_gqa_ratios(dev, bits, ratio):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(num_q_heads=2 * ratio, num_kv_heads=2, bits=bits, residual=32,
                                              rope=True, name=f"rope_ratio{ratio}")
    _two_call(w, [900], 3, dev)


@pytest.mark.parametrize("sink", [False, True])
def test_rope_llama_shape_steps(dev, sink):
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=2, rope=True, sink=sink, name="rope_llama")
    _two_call(w, [1500, 1501], 40, dev, check_every=8)


def test_rope_long_positions_many_splits(dev):
    # positions up to 20000 (angles far beyond 2 pi at the low frequencies)
    w = wl.WORKLOADS["million_1m"].scaled(rope=True, name="rope_long")
    _two_call(w, [20000], 1, dev, gps=8)


def test_rope_other_base(dev):
    import bit_asymmetric_kv_amd as kvq
    from oracle import OracleHead
    rng = np.random.default_rng(12)
    T = 700
    k = (rng.standard_normal((T, 128)) * 3).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    print("case rope base 500", flush=True)
    cache = kvq.KVCache(1, 4, 1, bits=2, residual=64, max_tokens=T + 1, device=dev, rope=True, rope_base=500.0)
    cache.append(to_dev(k[None, :, None], torch, dev), to_dev(v[None, :, None], torch, dev))
    ref = OracleHead(2, 64, rope=True, rope_base=500.0)
    ref.append(k, v)
    out = cache.decode(to_dev(q, torch, dev))
    torch.cuda.synchronize()
    err = float(np.abs(out.cpu().numpy()[0].astype(np.float64) - ref.attend(q[0])).max())
    assert err <= OUT_TOL, f"max |gpu - oracle| = {err:.3e}"


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


def test_rope_decode_step_folded_window(dev):
    # the one-call step writes the new tokens to the window inside the decode launch
    # and rotates them there
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=3, num_q_heads=8, num_kv_heads=4, residual=32,
                                                   rope=True, sink=True, name="rope_step")
    p = Pair(w, 1500, dev, torch)
    print("case rope step", flush=True)
    rng = np.random.default_rng(71)
    _step(p, [1, 60, 300])
    for s in range(40):
        _step(p, rng.integers(0, 20, size=3) if s % 5 == 4 else [1, 1, 1])
        if s % 8 == 7:
            p.check_state()
    p.check_state()
