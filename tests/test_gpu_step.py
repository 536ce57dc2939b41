"""GPU parity of the one-call decode step (kvq_decode_step): append + decode with
the window write folded into the decode launch. Checked against the CPU oracle
(blocks and window bit for bit, outputs within 2e-3) and against the two-call path
(append, then decode) bit for bit."""
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


def _step(p: Pair, n_tokens):
    w = p.w
    n_tokens = np.asarray(n_tokens, dtype=np.int64)
    n_max = max(int(n_tokens.max()), 1)
    k, v = wl.kv_batch(w, p.T, n_max, n_tokens)
    q = wl.queries(w, p.step)
    p.step += 1
    out = p.gpu.step(to_dev(k, torch, p.dev), to_dev(v, torch, p.dev), to_dev(q, torch, p.dev),
                     n_tokens=n_tokens.tolist())
    p.ref.append(k, v, n_tokens)
    p.T += n_tokens
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    exp = p.ref.decode(q)
    err = float(np.abs(got - exp).max())
    assert np.all(np.isfinite(got)) and err <= OUT_TOL, f"step {p.step}: max |gpu - oracle| = {err:.3e}"
    return err


def _run(w, contexts, n_fn, steps, dev, check_every=1):
    contexts = np.asarray(contexts, dtype=np.int64)
    p = Pair(w, int(contexts.max()) + 64 * steps + 1, dev, torch)
    print(f"case step {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} bits={w.bits} R={w.residual} "
          f"rot={w.rotate} ctx={contexts.tolist()[:6]} steps={steps}", flush=True)
    if contexts.max() > 0:
        p.append(contexts)
    worst = 0.0
    for s in range(steps):
        worst = max(worst, _step(p, n_fn(s)))
        if (s + 1) % check_every == 0 or s == steps - 1:
            p.check_state()
    return worst


def test_step_single_token_crossing_flushes(dev):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(residual=32, name="step_gqa")
    _run(w, [100], lambda s: [1], 70, dev, check_every=7)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_step_ragged_multi_token_and_empty(dev, bits):
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=5, num_q_heads=8, num_kv_heads=4, residual=64, bits=bits,
                                                   name="step_ragged")
    rng = np.random.default_rng(21 + bits)
    _run(w, [0, 1, 77, 300, 64], lambda s: rng.integers(0, 40, size=5) if s % 3 else [1, 1, 1, 1, 1], 18, dev,
         check_every=3)


def test_step_batch_above_inline_records(dev):
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=72, num_q_heads=8, num_kv_heads=2, rotate=False, residual=32,
                                              name="step_b72")
    ctx = np.random.default_rng(31).integers(1, 200, size=72)
    _run(w, ctx, lambda s: np.ones(72, dtype=np.int64), 40, dev, check_every=10)


def test_step_rotated_cache(dev):
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=3, name="step_rot")
    _run(w, [40, 500, 90], lambda s: [1, 2, 1], 40, dev, check_every=8)


def test_step_matches_append_then_decode_bitwise(dev):
    import bit_asymmetric_kv_amd as kvq
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=3, residual=64, name="step_eq")
    caches = [kvq.KVCache(w.batch, w.num_q_heads, w.num_kv_heads, bits=w.bits, residual=w.residual,
                          max_tokens=3000, device=dev) for _ in range(2)]
    T = np.zeros(3, dtype=np.int64)
    rng = np.random.default_rng(5)
    for s in range(60):
        n = np.array([1, 1, 1]) if s else np.array([700, 1500, 33])
        if s % 10 == 5:
            n = rng.integers(0, 50, size=3)
        k, v = wl.kv_batch(w, T, max(int(n.max()), 1), n)
        q = to_dev(wl.queries(w, s), torch, dev)
        kd, vd = to_dev(k, torch, dev), to_dev(v, torch, dev)
        o1 = caches[0].step(kd, vd, q, n_tokens=n.tolist())
        caches[1].append(kd, vd, n.tolist())
        o2 = caches[1].decode(q)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"step {s}: one-call and two-call outputs differ"
        T += n
    for b in range(3):
        assert caches[0].seq_len(b) == caches[1].seq_len(b)
        for h in range(w.num_kv_heads):
            _, Q = caches[0].seq_len(b)
            assert np.array_equal(caches[0].read_groups(b, h, 0, Q // 32), caches[1].read_groups(b, h, 0, Q // 32))
            for which in ("k", "v"):
                assert np.array_equal(caches[0].read_ring(b, h, which), caches[1].read_ring(b, h, which))


def test_step_on_empty_sequence_fails_and_changes_nothing(dev):
    import bit_asymmetric_kv_amd as kvq
    cache = kvq.KVCache(2, 4, 2, bits=2, residual=32, max_tokens=100, device=dev)
    k = torch.zeros(2, 3, 2, 128, dtype=torch.float16, device=dev)
    q = torch.zeros(2, 4, 128, dtype=torch.float16, device=dev)
    with pytest.raises(kvq.KVQError) as e:
        cache.step(k, k, q, n_tokens=[3, 0])
    assert e.value.status == -6
    assert cache.seq_len(0) == (0, 0) and cache.seq_len(1) == (0, 0)
    out = cache.step(k, k, q)
    torch.cuda.synchronize()
    assert cache.seq_len(0) == (3, 0) and bool(torch.isfinite(out).all())


def test_library_allocated_cache_matches_caller_memory(dev):
    """kvq_create with dev_mem NULL: the library allocates the cache itself (and
    frees it in kvq_destroy). Driven through the C ABI directly, it gives the same
    outputs bit for bit as a cache in caller-provided memory fed the same inputs."""
    import ctypes
    import bit_asymmetric_kv_amd as kvq
    from bit_asymmetric_kv_amd import _lib
    lib = _lib.load()
    w = wl.WORKLOADS["gqa_128k_2bit"]
    B, ctx = w.batch, 1000
    print(f"case library-allocated cache {w.name} ctx={ctx}", flush=True)
    cfg = kvq.make_config(B, w.num_q_heads, w.num_kv_heads, residual=w.residual, max_tokens=ctx + 64)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    h = ctypes.c_void_p(0)
    _lib.check(lib.kvq_create(ctypes.byref(cfg), None, 0, stream, ctypes.byref(h)))
    assert h.value
    ref = kvq.KVCache(B, w.num_q_heads, w.num_kv_heads, residual=w.residual, max_tokens=ctx + 64, device=dev)
    try:
        T = np.zeros(B, dtype=np.int64)
        k, v = wl.kv_batch(w, T, ctx, np.full(B, ctx, dtype=np.int64))
        kd, vd = to_dev(k, torch, dev), to_dev(v, torch, dev)
        _lib.check(lib.kvq_append(h, kd.data_ptr(), vd.data_ptr(), None, ctx, stream))
        ref.append(kd, vd)
        T += ctx
        for s in range(40):  # one token per step: crosses a group flush
            k1, v1 = wl.kv_batch(w, T, 1, np.ones(B, dtype=np.int64))
            k1d, v1d = to_dev(k1, torch, dev), to_dev(v1, torch, dev)
            _lib.check(lib.kvq_append(h, k1d.data_ptr(), v1d.data_ptr(), None, 1, stream))
            ref.append(k1d, v1d)
            T += 1
            qd = to_dev(wl.queries(w, s), torch, dev)
            out = torch.empty(B, w.num_q_heads, 128, dtype=torch.float32, device=dev)
            _lib.check(lib.kvq_decode_attention(h, qd.data_ptr(), out.data_ptr(), stream))
            exp = ref.decode(qd)
            torch.cuda.synchronize()
            assert torch.equal(out, exp), f"step {s}: max diff {float((out - exp).abs().max()):.3e}"
        tl, ql = ctypes.c_int64(0), ctypes.c_int64(0)
        _lib.check(lib.kvq_seq_len(h, 0, ctypes.byref(tl), ctypes.byref(ql)))
        assert (tl.value, ql.value) == ref.seq_len(0)
    finally:
        lib.kvq_destroy(h)
        ref.close()
