"""GPU parity: HIP library vs the CPU oracle on reduced-size workloads.

Every case checks packed codes, scales and zero-points and the FP16 window bit for
bit, and decode outputs within max-abs 2e-3 of the float64 oracle.
"""
import numpy as np
import pytest

import kvq_workloads as wl
from parity_helpers import Pair

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _run(w, contexts, steps, dev, max_tokens=None, gps=0, check_every=1):
    contexts = np.asarray(contexts, dtype=np.int64)
    mt = max_tokens or int(contexts.max()) + steps + 1
    p = Pair(w, mt, dev, torch, groups_per_split=gps)
    print(f"case {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} bits={w.bits} R={w.residual} "
          f"rot={w.rotate} ctx={contexts.tolist()[:8]} steps={steps}", flush=True)
    p.append(contexts)
    p.check_state()
    errs = [p.check_decode()]
    for s in range(steps):
        p.append(np.ones(w.batch, dtype=np.int64))
        if (s + 1) % check_every == 0 or s == steps - 1:
            p.check_state()
            errs.append(p.check_decode())
    return max(errs)


def test_tiny_mha_full_size(dev):
    w = wl.WORKLOADS["tiny_mha_4k"]
    _run(w, [w.context], w.steps, dev)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_llama_shape_reduced(dev, bits):
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=2, bits=bits)
    _run(w, [1000, 1000], 40, dev, check_every=8)


@pytest.mark.parametrize("name", ["gqa_128k_2bit", "gqa_128k_4bit"])
def test_gqa_reduced(dev, name):
    w = wl.WORKLOADS[name]
    _run(w, [3000], 2, dev)


def test_million_shape_reduced_many_splits(dev):
    w = wl.WORKLOADS["million_1m"]
    _run(w, [8192], 1, dev, gps=8)


def test_ragged_rotated_reduced(dev):
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=6)
    ctx = np.random.default_rng(5).integers(40, 700, size=6)
    _run(w, ctx, 36, dev, check_every=6)


def test_batch_above_inline_records(dev):
    # more sequences than fit in the kernels' by-value records: the per-sequence
    # records go through the pinned upload path; ragged lengths, flushes interleaved
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=72, num_q_heads=8, num_kv_heads=2, rotate=False, residual=32)
    ctx = np.random.default_rng(9).integers(1, 260, size=72)
    _run(w, ctx, 40, dev, check_every=10)


@pytest.mark.parametrize("ratio", [1, 2, 4, 8])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_gqa_ratios(dev, ratio, bits):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(num_q_heads=2 * ratio, num_kv_heads=2, bits=bits, residual=32,
                                              name=f"ratio{ratio}")
    _run(w, [777], 3, dev)


@pytest.mark.parametrize("R", [0, 32])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 63, 64, 65, 95, 96, 97])
def test_edge_lengths(dev, R, T):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=1, residual=R, name=f"edge_R{R}")
    _run(w, [T], 2, dev)


@pytest.mark.parametrize("T", [1, 32, 33, 64, 65, 97])
def test_edge_lengths_3bit(dev, T):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=1, residual=0, bits=3, name="edge3")
    _run(w, [T], 2, dev)


def test_ragged_interleaved_flushes_and_empty_appends(dev):
    w = wl.WORKLOADS["llama2_7b_b8_32k"].scaled(batch=4, num_q_heads=8, num_kv_heads=4, residual=64, name="ragged")
    p = Pair(w, 2000, dev, torch)
    p.append([5, 130, 0, 64])
    p.append([0, 0, 1, 0])
    p.check_state()
    p.check_decode()
    rng = np.random.default_rng(3)
    for _ in range(6):
        p.append(rng.integers(0, 40, size=4))
        p.check_state()
        p.check_decode()


def test_prefill_in_chunks_matches_single_prefill(dev):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(residual=128, name="chunks")
    a = Pair(w, 3000, dev, torch)
    a.append([2500])
    b = Pair(w, 3000, dev, torch)
    for n in (1, 31, 500, 1000, 968):
        b.append([n])
    T, Q = a.gpu.seq_len(0)
    assert (T, Q) == b.gpu.seq_len(0)
    for h in range(w.num_kv_heads):
        assert np.array_equal(a.gpu.read_groups(0, h, 0, Q // 32), b.gpu.read_groups(0, h, 0, Q // 32))
    b.check_state()


def test_deterministic_and_split_invariant(dev):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(name="det")
    p = Pair(w, 5000, dev, torch)
    p.append([4800])
    q = torch.from_numpy(wl.queries(w, 0)).to(dev)
    o1 = p.gpu.decode(q).clone()
    o2 = p.gpu.decode(q).clone()
    assert torch.equal(o1, o2)
    p.gpu.set_decode_split(4)
    o3 = p.gpu.decode(q).clone()
    p.gpu.set_decode_split(1000)
    o4 = p.gpu.decode(q).clone()
    assert float((o3 - o1).abs().max()) < 1e-5 and float((o4 - o1).abs().max()) < 1e-5


def _adversarial_groups():
    rng = np.random.default_rng(17)
    k = rng.standard_normal((160, 128)).astype(np.float16)
    v = rng.standard_normal((160, 128)).astype(np.float16)
    k[0:32] = np.float16(7.25)                       # constant key group
    v[0:32, 0:32] = np.float16(-3.0)                 # constant value channel groups
    k[32:64] = np.float16(0.0)
    k[40, 5] = np.float16(1000.0)                    # one large outlier in one channel
    ties = np.array([0, 3, 0.5, 1.5, 2.5, 1, 2, 0.25], dtype=np.float16)
    k[64:96, 7] = np.resize(ties, 32)                # exact half-step ties
    v[70, 0:32] = np.resize(ties, 32)
    tiny = np.float16(2.0 ** -24)
    k[96:128, 9] = np.resize(np.array([0, tiny, 2 * tiny], dtype=np.float16), 32)  # subnormal ranges
    v[100, 32:64] = np.resize(np.array([0, tiny], dtype=np.float16), 32)
    k[128:160, 11] = np.resize(np.array([-65504, 65504], dtype=np.float16), 32)    # full fp16 range
    v[130, 64:96] = np.resize(np.array([-65504, 65504], dtype=np.float16), 32)
    # subnormal ranges whose fp16 scale rounds below (max - min) / (2^b - 1), so the
    # top code only stays in range through the clamp to 2^b - 1 (hand-worked in
    # tests/golden/quantizer_cases.json): multiples n * 2^-24 of the smallest subnormal
    for c, ns in zip(range(13, 19), ([0, 4, 3, 2, 1], [0, 7], [0, 10, 9, 8], [0, 15],
                                     [0, 20, 17, 16, 15], [0, 31])):
        grp = np.array(ns, dtype=np.float64) * 2.0 ** -24
        k[96:128, c] = np.resize(grp.astype(np.float16), 32)
        v[101 + c - 13, 32:64] = np.resize(grp.astype(np.float16), 32)
    return k, v


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_adversarial_groups_bit_exact(dev, bits):
    import bit_asymmetric_kv_amd as kvq
    from oracle import OracleHead
    k, v = _adversarial_groups()
    cache = kvq.KVCache(1, 1, 1, bits=bits, residual=0, max_tokens=200, device=dev)
    cache.append(torch.from_numpy(k[None, :, None]).to(dev), torch.from_numpy(v[None, :, None]).to(dev))
    ref = OracleHead(bits, 0)
    ref.append(k, v)
    got = cache.read_groups(0, 0, 0, 5)
    for g in range(5):
        assert np.array_equal(got[g], ref.block(g)), f"group {g}"
    # outputs stay finite; the oracle is matched in relative terms where values reach 65504
    q = torch.from_numpy(np.random.default_rng(1).standard_normal((1, 1, 128)).astype(np.float16) * 0.01).to(dev)
    out = cache.decode(q).cpu().numpy()[0, 0]
    exp = ref.attend(q.cpu().numpy()[0])[0]
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - exp)) <= 2e-3 * max(1.0, np.abs(exp).max())
    # channels that no +-65504 value feeds meet the plain bar
    plain = np.r_[0:64, 96:128]
    assert np.max(np.abs(out[plain] - exp[plain])) <= 2e-3


def test_errors_leave_state_unchanged(dev):
    import bit_asymmetric_kv_amd as kvq
    cache = kvq.KVCache(2, 4, 2, bits=2, residual=32, max_tokens=100, device=dev)
    with pytest.raises(kvq.KVQError) as e:
        cache.decode(torch.zeros(2, 4, 128, dtype=torch.float16, device=dev))
    assert e.value.status == -6
    k = torch.zeros(2, 60, 2, 128, dtype=torch.float16, device=dev)
    cache.append(k, k)
    with pytest.raises(kvq.KVQError) as e:
        cache.append(k, k)            # 120 > max_tokens
    assert e.value.status == -2
    assert cache.seq_len(0) == (60, 0) and cache.seq_len(1) == (60, 0)
    with pytest.raises(kvq.KVQError):
        cache.append(k, k, n_tokens=[61, 0])
    assert cache.seq_len(0) == (60, 0)


@pytest.mark.parametrize("scale", [0.3, 0.02])
def test_explicit_softmax_scale(dev, scale):
    import bit_asymmetric_kv_amd as kvq
    from oracle import OracleCache
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=2, num_q_heads=8, num_kv_heads=2, residual=32, name="scale")
    print(f"case softmax_scale {scale}", flush=True)
    cache = kvq.KVCache(w.batch, w.num_q_heads, w.num_kv_heads, bits=w.bits, residual=w.residual,
                        max_tokens=1200, softmax_scale=scale, device=dev)
    ref = OracleCache(w.batch, w.num_q_heads, w.num_kv_heads, w.bits, w.residual, softmax_scale=scale)
    k, v = wl.kv_batch(w, [0, 0], 1100, np.array([1100, 700]))
    cache.append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), n_tokens=[1100, 700])
    ref.append(k, v, [1100, 700])
    q = wl.queries(w, 0)
    out = cache.decode(torch.from_numpy(q).to(dev)).cpu().numpy().astype(np.float64)
    err = float(np.abs(out - ref.decode(q)).max())
    assert err <= 2e-3, f"max |gpu - oracle| = {err:.3e}"


@pytest.mark.parametrize("R,T", [(1024, 1055), (1024, 1057), (1024, 3000), (4096, 4127), (4096, 6000)])
def test_large_residual_window(dev, R, T):
    # windows of R .. R + 31 tokens spread over many FP16-window workgroups
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=1, residual=R, name=f"bigR{R}")
    _run(w, [T], 2, dev)
