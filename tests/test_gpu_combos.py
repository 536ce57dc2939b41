"""GPU parity of the cache options together: 2/3/4-bit codes, attention sink,
pre-RoPE keys and paged groups in combination, through both the two-call path and
the one-call step, including a batch above the kernels' by-value sequence records."""
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


def _pair(w, max_tokens, dev, paged, seed=0):
    kw = {}
    if paged:
        P = 4
        max_pages = -(-((max_tokens + 31) // 32) // P)
        kw = dict(page_groups=P, pool_pages=w.batch * max_pages + 3)
    p = Pair(w, max_tokens, dev, torch, **kw)
    if paged:
        perm = np.random.default_rng(seed).permutation(w.batch * max_pages + 3)
        for b in range(w.batch):
            p.gpu.set_pages(b, perm[b * max_pages:(b + 1) * max_pages].tolist())
    return p


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
    err = float(np.abs(out.cpu().numpy().astype(np.float64) - p.ref.decode(q)).max())
    assert err <= OUT_TOL, f"step {p.step}: max |gpu - oracle| = {err:.3e}"


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("sink,rope,paged", [(True, True, True), (False, True, True), (True, False, True),
                                             (True, True, False)])
def test_options_together(dev, bits, sink, rope, paged):
    w = wl.WORKLOADS["gqa_128k_2bit"].scaled(batch=3, num_q_heads=8, num_kv_heads=2, residual=32, bits=bits,
                                              sink=sink, rope=rope, name="combo")
    print(f"case combo bits={bits} sink={sink} rope={rope} paged={paged}", flush=True)
    p = _pair(w, 1500, dev, paged, seed=bits)
    p.append([333, 700, 1])
    p.check_state()
    p.check_decode()
    rng = np.random.default_rng(bits)
    for s in range(24):
        _step(p, rng.integers(0, 40, size=3) if s % 6 == 5 else [1, 1, 1])
    p.check_state()
    p.check_decode()


def test_large_batch_paged_sink_rope(dev):
    # 70 sequences: the per-sequence records take the uploaded path
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=70, num_q_heads=8, num_kv_heads=2, rotate=False, residual=32,
                                              sink=True, rope=True, name="combo_b70")
    print("case combo B=70 paged sink rope", flush=True)
    p = _pair(w, 400, dev, True, seed=7)
    ctx = np.random.default_rng(9).integers(1, 300, size=70)
    p.append(ctx)
    p.check_state()
    p.check_decode()
    for s in range(12):
        _step(p, np.ones(70, dtype=np.int64))
    p.check_state()


def test_large_batch_sliced_combine(dev):
    # 70 sequences with 2 query heads: 140 (sequence, query head) rows, below the
    # row-merge threshold, so the sliced combine runs with sequence indices past the
    # inline records (the plan's uniform split count)
    w = wl.WORKLOADS["ragged_b64_wht"].scaled(batch=70, num_q_heads=2, num_kv_heads=2, rotate=False, residual=32,
                                              name="combo_b70_sliced")
    print("case combo B=70 Hq=2 sliced combine", flush=True)
    p = _pair(w, 600, dev, False, seed=11)
    ctx = np.random.default_rng(13).integers(1, 500, size=70)
    p.append(ctx)
    p.check_state()
    p.check_decode()
    for s in range(6):
        _step(p, np.ones(70, dtype=np.int64))
    p.check_decode()
