"""GPU check of kvq_fp16_decode_attention_noalloc, the FP16-cache decode whose split
partials live in the library's static per-GPU scratch instead of a caller workspace.

Through the C ABI (the binding only marshals arguments): two calls in a row, the
second with a smaller input, each compared with kvq_fp16_decode_attention on the
same inputs (same split plan, so the outputs agree bit for bit) and with the float64
oracle attention (max-abs 2e-3); a shape whose partials exceed the scratch is
refused before any launch.
"""
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


def _inputs(B, Hq, Hkv, lens, t_cap, seed):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, seed=seed)
    k = np.zeros((B, Hkv, t_cap, 128), dtype=np.float16)
    v = np.zeros((B, Hkv, t_cap, 128), dtype=np.float16)
    for b in range(B):
        for h in range(Hkv):
            k[b, h, :lens[b]] = wl.keys(w, b, h, 0, lens[b])
            v[b, h, :lens[b]] = wl.values(w, b, h, 0, lens[b])
    return k, v, wl.queries(w, 0)


def _compare(dev, B, Hq, Hkv, lens, t_cap, seed):
    import bit_asymmetric_kv_amd as kvq
    print(f"case fp16 no-alloc B={B} Hq={Hq} Hkv={Hkv} lens={list(lens)} t_cap={t_cap}", flush=True)
    k, v, q = _inputs(B, Hq, Hkv, lens, t_cap, seed)
    kd, vd, qd = (torch.from_numpy(x).to(dev) for x in (k, v, q))
    lens_dev = torch.tensor(np.asarray(lens, dtype=np.int32), device=dev)
    with_ws = kvq.Fp16Decode(B, Hq, Hkv, t_cap, device=dev)
    no_alloc = kvq.Fp16Decode(B, Hq, Hkv, t_cap, device=dev, static_scratch=True)
    assert no_alloc.workspace is None
    expect = with_ws(kd, vd, lens_dev, int(max(lens)), qd).clone()
    got = no_alloc(kd, vd, lens_dev, int(max(lens)), qd)
    torch.cuda.synchronize()
    assert torch.equal(got, expect), float((got - expect).abs().max())
    out = got.cpu().numpy().astype(np.float64)
    ratio = Hq // Hkv
    err = 0.0
    for b in range(B):
        for h in range(Hkv):
            ref = attention_fp64(q[b, h * ratio:(h + 1) * ratio], k[b, h, :lens[b]], v[b, h, :lens[b]],
                                 1.0 / np.sqrt(128.0))
            err = max(err, float(np.abs(out[b, h * ratio:(h + 1) * ratio] - ref).max()))
    assert err <= 2e-3, f"max |gpu - oracle| = {err:.3e}"


def test_noalloc_matches_workspace_entry_point_twice(dev):
    # first a larger call, then a smaller one over the scratch the first left behind
    _compare(dev, 2, 8, 2, [3000, 1500], 3000, 31)
    _compare(dev, 1, 4, 1, [700], 800, 32)


def test_noalloc_refuses_partials_beyond_the_scratch(dev):
    import bit_asymmetric_kv_amd as kvq
    from bit_asymmetric_kv_amd import _lib
    # 8192 sequences x 8 query heads, one split each: 8192 * 8 * 520 bytes > 4 MiB
    B, Hq, Hkv, t_cap = 8192, 8, 8, 32
    op = kvq.Fp16Decode(B, Hq, Hkv, t_cap, device=dev, static_scratch=True)
    k = torch.zeros((B, Hkv, t_cap, 128), dtype=torch.float16, device=dev)
    q = torch.zeros((B, Hq, 128), dtype=torch.float16, device=dev)
    lens = torch.full((B,), 32, dtype=torch.int32, device=dev)
    with pytest.raises(kvq.KVQError) as e:
        op(k, k, lens, 32, q)
    assert e.value.status == _lib.KVQ_ERR_CAPACITY
