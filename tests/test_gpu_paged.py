"""GPU parity of paged caches: the packed groups live in a pool of pages (P groups
of one sequence for all its kv-heads per page) named by a per-sequence page table
that the caller fills. Groups (read back through the table) and the FP16 window bit
for bit, outputs within 2e-3 of the oracle, and identical to a contiguous cache fed
the same inputs; capacity, reset and validation behaviour on the host side."""
import numpy as np
import pytest

import kvq_workloads as wl
from oracle import OracleHead
from parity_helpers import OUT_TOL, Pair, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _w(**kw):
    base = dict(batch=3, num_q_heads=8, num_kv_heads=4, residual=64, name="paged")
    base.update(kw)
    return wl.WORKLOADS["llama2_7b_b8_32k"].scaled(**base)


def test_paged_random_pages_parity(dev):
    w = _w()
    P, max_tokens = 4, 2000
    max_pages = -(-((max_tokens + 31) // 32) // P)
    pool = w.batch * max_pages + 7
    p = Pair(w, max_tokens, dev, torch, page_groups=P, pool_pages=pool)
    perm = np.random.default_rng(1).permutation(pool)
    for b in range(w.batch):
        p.gpu.set_pages(b, perm[b * max_pages:(b + 1) * max_pages].tolist())
    print(f"case paged P={P} pool={pool}", flush=True)
    p.append([700, 1100, 33])
    p.check_state()
    p.check_decode()
    for s in range(30):
        p.append(np.ones(w.batch, dtype=np.int64))
        if s % 10 == 9:
            p.check_state()
            p.check_decode()


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_paged_matches_contiguous_bitwise(dev, bits):
    w = _w(bits=bits, batch=2)
    P, max_tokens = 2, 1500
    max_pages = -(-((max_tokens + 31) // 32) // P)
    a = Pair(w, max_tokens, dev, torch, page_groups=P, pool_pages=2 * max_pages)
    b = Pair(w, max_tokens, dev, torch)
    for s in range(2):
        a.gpu.set_pages(s, list(range(s, 2 * max_pages, 2)))   # interleaved pages
    print(f"case paged vs contiguous bits={bits}", flush=True)
    for n in ([900, 1200], [1, 1], [40, 0], [1, 1]):
        a.append(n)
        b.append(n)
        q = torch.from_numpy(wl.queries(w, a.step)).to(dev)
        oa, ob = a.gpu.decode(q).clone(), b.gpu.decode(q).clone()
        torch.cuda.synchronize()
        assert torch.equal(oa, ob)
    for s in range(2):
        T, Q = a.gpu.seq_len(s)
        for h in range(w.num_kv_heads):
            assert np.array_equal(a.gpu.read_groups(s, h, 0, Q // 32), b.gpu.read_groups(s, h, 0, Q // 32))
    a.check_state()


def test_paged_pages_on_demand(dev):
    import bit_asymmetric_kv_amd as kvq
    w = _w(batch=2)
    P = 2
    p = Pair(w, 4000, dev, torch, page_groups=P, pool_pages=200)
    print("case paged on demand", flush=True)
    free = list(range(199, -1, -1))
    owned = {0: [], 1: []}

    def grow(b, groups):
        need = -(-groups // P)
        while len(owned[b]) < need:
            owned[b].append(free.pop())
        p.gpu.set_pages(b, owned[b])

    # no pages yet: an append that quantizes groups fails and changes nothing
    with pytest.raises(kvq.KVQError) as e:
        p.gpu.append(*[to_dev(x, torch, dev) for x in wl.kv_batch(w, p.T, 200, np.array([200, 10]))],
                     n_tokens=[200, 10])
    assert e.value.status == kvq.KVQ_ERR_CAPACITY
    assert p.gpu.seq_len(0) == (0, 0) and p.gpu.seq_len(1) == (0, 0)
    rng = np.random.default_rng(2)
    for it in range(25):
        n = rng.integers(1, 150, size=2)
        for b in range(2):
            groups = max(0, (int(p.T[b] + n[b]) - w.residual) // 32)
            grow(b, groups)
        p.append(n)
        if it % 5 == 4:
            p.check_state()
            p.check_decode()


def test_paged_reset_and_reuse(dev):
    w = _w(batch=2)
    P = 2
    max_pages = -(-((2000 + 31) // 32) // P)
    p = Pair(w, 2000, dev, torch, page_groups=P, pool_pages=2 * max_pages)
    pages = list(range(2 * max_pages))
    p.gpu.set_pages(0, pages[:max_pages])
    p.gpu.set_pages(1, pages[max_pages:])
    print("case paged reset", flush=True)
    p.append([900, 500])
    p.check_state()
    p.check_decode()
    # sequence 0 starts over; its old pages go to it again in reverse order
    p.gpu.reset_sequence(0)
    p.gpu.set_pages(0, pages[:max_pages][::-1])
    p.ref.heads[0] = [OracleHead(w.bits, w.residual, w.rotate) for _ in range(w.num_kv_heads)]
    p.T[0] = 0
    assert p.gpu.seq_len(0) == (0, 0)
    p.append([300, 1])
    for _ in range(10):
        p.append([1, 1])
    p.check_state()
    p.check_decode()


def test_paged_one_call_step(dev):
    w = _w(batch=3, residual=32)
    P = 4
    max_pages = -(-((1200 + 31) // 32) // P)
    p = Pair(w, 1200, dev, torch, page_groups=P, pool_pages=3 * max_pages)
    perm = np.random.default_rng(3).permutation(3 * max_pages)
    for b in range(3):
        p.gpu.set_pages(b, perm[b::3].tolist())
    print("case paged step", flush=True)
    p.append([100, 400, 40])
    for s in range(40):
        n = np.ones(3, dtype=np.int64)
        k, v = wl.kv_batch(w, p.T, 1, n)
        q = wl.queries(w, p.step)
        p.step += 1
        out = p.gpu.step(to_dev(k, torch, dev), to_dev(v, torch, dev), to_dev(q, torch, dev))
        p.ref.append(k, v, n)
        p.T += n
        torch.cuda.synchronize()
        err = float(np.abs(out.cpu().numpy().astype(np.float64) - p.ref.decode(q)).max())
        assert err <= OUT_TOL
    p.check_state()


def test_paged_validation(dev):
    import bit_asymmetric_kv_amd as kvq
    plain = kvq.KVCache(1, 4, 1, bits=2, residual=32, max_tokens=500, device=dev)
    with pytest.raises(kvq.KVQError):
        plain.set_pages(0, [0])                       # not a paged cache
    with pytest.raises(kvq.KVQError):                 # page_groups must be a power of two
        kvq.KVCache(1, 4, 1, bits=2, residual=32, max_tokens=500, device=dev, page_groups=3, pool_pages=4)
    c = kvq.KVCache(2, 4, 1, bits=2, residual=32, max_tokens=500, device=dev, page_groups=2, pool_pages=10)
    for bad in ([10], [-1], [1, 1], list(range(9))):  # range, range, duplicate, more than max_pages (8)
        with pytest.raises(kvq.KVQError) as e:
            c.set_pages(0, bad)
        assert e.value.status == kvq.KVQ_ERR_INVALID_ARG
    c.set_pages(0, [0, 1, 2])
    with pytest.raises(kvq.KVQError):
        c.set_pages(1, [2])                           # page 2 belongs to sequence 0
    k = torch.zeros(2, 100, 1, 128, dtype=torch.float16, device=dev)
    c.set_pages(1, [3])
    c.append(k, k, n_tokens=[100, 60])                # 2 groups for sequence 0, 0 for 1
    assert c.seq_len(0) == (100, 64)
    with pytest.raises(kvq.KVQError):
        c.set_pages(0, [4, 1, 2])                     # page 0 holds groups: cannot move
    c.set_pages(0, [0])                               # dropping pages past the used one is fine
    c.set_pages(1, [3, 2])                            # page 2 was freed
    with pytest.raises(kvq.KVQError) as e:
        c.append(k, k, n_tokens=[100, 0])             # sequence 0 would need 3 pages
    assert e.value.status == kvq.KVQ_ERR_CAPACITY
    assert c.seq_len(0) == (100, 64)
