"""GPU checks of the comparison kernels measured beside the quantized path: the
streaming-read probe (its xor fold equals the host fold of the same words) and the
FP16-cache decode (parity with the float64 oracle attention on the same fp16 keys
and values, max-abs 2e-3)."""
import numpy as np
import pytest

import kvq_workloads as wl
from oracle import attention_fp64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("words,workgroups", [(4, 1), (4, 7), (4 * 1000 + 4, 33), (4 * (1 << 20) + 12, 2048)])
def test_stream_read_fold(dev, words, workgroups):
    import bit_asymmetric_kv_amd as kvq
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    # every word of the fold array is written (the poison must not survive)
    fold = torch.full((workgroups,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    print(f"case stream_read words={words} workgroups={workgroups}", flush=True)
    kvq.stream_read(buf, fold)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(fold.cpu().numpy().view(np.uint32)))
    assert got == int(np.bitwise_xor.reduce(host))


def _fp16_case(dev, B, Hq, Hkv, lens, t_cap, seed, scale=0.0):
    import bit_asymmetric_kv_amd as kvq
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, seed=seed)
    print(f"case fp16_decode B={B} Hq={Hq} Hkv={Hkv} lens={list(lens)} t_cap={t_cap}", flush=True)
    k = np.zeros((B, Hkv, t_cap, 128), dtype=np.float16)
    v = np.zeros((B, Hkv, t_cap, 128), dtype=np.float16)
    for b in range(B):
        for h in range(Hkv):
            k[b, h, :lens[b]] = wl.keys(w, b, h, 0, lens[b])
            v[b, h, :lens[b]] = wl.values(w, b, h, 0, lens[b])
    q = wl.queries(w, 0)
    op = kvq.Fp16Decode(B, Hq, Hkv, t_cap, softmax_scale=scale, device=dev)
    lens_dev = torch.tensor(np.asarray(lens, dtype=np.int32), device=dev)
    out = op(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), lens_dev, int(max(lens)),
             torch.from_numpy(q).to(dev))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    sc = scale if scale > 0 else 1.0 / np.sqrt(128.0)
    ratio = Hq // Hkv
    err = 0.0
    for b in range(B):
        for h in range(Hkv):
            exp = attention_fp64(q[b, h * ratio:(h + 1) * ratio], k[b, h, :lens[b]], v[b, h, :lens[b]], sc)
            err = max(err, float(np.abs(got[b, h * ratio:(h + 1) * ratio] - exp).max()))
    assert np.all(np.isfinite(got))
    assert err <= 2e-3, f"max |gpu - oracle| = {err:.3e}"
    return err


def test_fp16_decode_gqa4_ragged(dev):
    _fp16_case(dev, 3, 8, 2, [1, 33, 1000], 1024, 11)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1)])
def test_fp16_decode_head_ratios(dev, Hq, Hkv):
    _fp16_case(dev, 2, Hq, Hkv, [517, 96], 600, 12 + Hq + Hkv)


def test_fp16_decode_long_many_splits(dev):
    # 40,000 tokens in one (b, h): many splits, chunks of a ragged tail, explicit scale
    _fp16_case(dev, 1, 4, 1, [40000], 40000, 13, scale=0.1)


def test_fp16_decode_many_rows(dev):
    # 64 sequences x 8 query heads = 512 (sequence, head) rows: the one-wave-per-row merge
    rng = np.random.default_rng(14)
    lens = rng.integers(1, 400, size=64).tolist()
    _fp16_case(dev, 64, 8, 2, lens, 400, 14)
