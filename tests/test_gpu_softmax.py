"""GPU parity of the online softmax under score patterns that move the running
maximum: scores that rise token after token (every group raises the maximum), one
rising spike per group at a random position (the maximum sits in a different lane
and column copy each time, and the earlier weights fall by up to 2^-89), and
scores that only fall after the first group. Every query-head grouping (1, 2, 4, 8
query heads per KV head) is run, since the kernel splits a group's softmax weights
among 16 / (2 * heads) copies of each MFMA column. Outputs within 2e-3 of the
float64 oracle."""
import numpy as np
import pytest

from oracle import OracleCache
from parity_helpers import OUT_TOL, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inputs(pattern, B, Hq, Hkv, T, seed):
    rng = np.random.default_rng(seed)
    D = 128
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    k = rng.standard_normal((B, T, Hkv, D)) * 0.5
    v = rng.standard_normal((B, T, Hkv, D))
    hg = Hq // Hkv
    t = np.arange(T)
    for b in range(B):
        for h in range(Hkv):
            # direction shared by the kv-head's query heads: q . dir ~ |q| for each
            d = q[b, h * hg:(h + 1) * hg].astype(np.float64).sum(axis=0)
            d /= np.linalg.norm(d)
            if pattern == "ramp":
                c = 0.03 * t                       # scores rise by ~0.03 * |q| / sqrt(128) per token
            elif pattern == "falling":
                c = 40.0 - 0.03 * t
            else:                                  # one spike per 32-token group, rising
                c = np.zeros(T)
                for g0 in range(0, T, 32):
                    c[g0 + rng.integers(0, min(32, T - g0))] = 1.2 * (g0 // 32)
            k[b, :, h, :] += c[:, None] * d[None, :]
    return q, k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("pattern", ["ramp", "spikes", "falling"])
@pytest.mark.parametrize("ratio", [1, 2, 4, 8])
def test_running_max_patterns(dev, pattern, ratio):
    import bit_asymmetric_kv_amd as kvq
    B, Hkv, T, R = 2, 2, 1500, 32
    Hq = Hkv * ratio
    q, k, v = _inputs(pattern, B, Hq, Hkv, T, seed=700 + ratio + 10 * len(pattern))
    assert np.all(np.isfinite(k.astype(np.float32)))
    print(f"case softmax {pattern} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
    cache = kvq.KVCache(B, Hq, Hkv, bits=2, residual=R, max_tokens=T + 8, device=dev)
    ref = OracleCache(B, Hq, Hkv, 2, R, False)
    cache.append(to_dev(k, torch, dev), to_dev(v, torch, dev))
    ref.append(k, v)
    got = cache.decode(to_dev(q, torch, dev)).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    exp = ref.decode(q)
    err = float(np.abs(got - exp).max())
    assert np.all(np.isfinite(got)) and err <= OUT_TOL, f"max |gpu - oracle| = {err:.3e}"
    # the same with the smallest splits (4 groups, one per wave: every wave starts
    # its own running maximum)
    cache.set_decode_split(4)
    got2 = cache.decode(to_dev(q, torch, dev)).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    err2 = float(np.abs(got2 - exp).max())
    assert np.all(np.isfinite(got2)) and err2 <= OUT_TOL, f"4-group splits: max |gpu - oracle| = {err2:.3e}"
    cache.close()
