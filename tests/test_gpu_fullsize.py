"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times (automatic split), on sampled (sequence, kv-head) pairs.

The GPU cache holds every head, filled from torch's seeded generator on the device
(kvq_workloads.torch_kv); the rows of the sampled heads are copied back and fed to
the CPU oracle, which checks those heads one by one: packed group blocks and FP16
window bit for bit, decode outputs of their query heads within max-abs 2e-3.
"""
import numpy as np
import pytest

import kvq_workloads as wl
from oracle import OracleHead
from parity_helpers import OUT_TOL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CHUNK = 131072  # prefill append size, as bench.py appends


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _check_blocks(cache, oh, b, h, group_sample):
    ng = oh.Q // 32
    if ng == 0:
        return
    gs = sorted(set(g for g in group_sample(ng) if 0 <= g < ng))
    # read contiguous runs to keep the number of copies small
    got = cache.read_groups(b, h, 0, ng) if ng <= 8192 else None
    for g in gs:
        blk = got[g] if got is not None else cache.read_groups(b, h, g, 1)[0]
        exp = oh.block(g)
        assert np.array_equal(blk, exp), f"group block (b={b}, h={h}, g={g}) differs"
    W = cache.cfg.residual + cache.cfg.group
    rk, rv = cache.read_ring(b, h, "k"), cache.read_ring(b, h, "v")
    # window tokens [o + Q, T) in slot t % W; an attention sink (token 0) in slot W
    slots = [(t, t % W) for t in range(oh.o + oh.Q, oh.T)] + ([(0, W)] if oh.sink and oh.T else [])
    for t, slot in slots:
        assert np.array_equal(rk[slot].view(np.uint16), oh.k16[t].view(np.uint16)), f"ring key t={t}"
        assert np.array_equal(rv[slot].view(np.uint16), oh.v16[t].view(np.uint16)), f"ring value t={t}"


def _run_full(w, dev, sample, steps, check_steps, group_sample=lambda ng: range(ng), one_call=False, page_groups=0):
    """one_call: each step is one kvq_decode_step (append + decode in one call, the
    window write folded into the decode launch), as the bench times it. page_groups:
    a paged cache, every sequence's pages in a seeded random order (as bench.py
    --page-groups lays them out)."""
    import bit_asymmetric_kv_amd as kvq
    lens = w.context_lengths()
    max_tokens = int(lens.max()) + steps + 1
    paged = {}
    if page_groups:
        max_pages = -(-((max_tokens + w.group - 1) // w.group) // page_groups)
        paged = dict(page_groups=page_groups, pool_pages=w.batch * max_pages)
    cache = kvq.KVCache(w.batch, w.num_q_heads, w.num_kv_heads, bits=w.bits, group=w.group,
                        residual=w.residual, rotate=w.rotate, max_tokens=max_tokens, device=dev,
                        sink=w.sink, rope=w.rope, **paged)
    if page_groups:
        perm = np.random.default_rng(w.seed + 5).permutation(w.batch * max_pages)
        for b in range(w.batch):
            cache.set_pages(b, perm[b * max_pages:(b + 1) * max_pages].tolist())
    oracles = {bh: OracleHead(w.bits, w.residual, w.rotate, sink=w.sink, rope=w.rope) for bh in sample}
    params = wl.torch_key_params(torch, w, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 101 + 7)
    print(f"case full-size {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} bits={w.bits} "
          f"R={w.residual} rot={w.rotate} context max {int(lens.max())} steps={steps} sample={sample} "
          f"one_call={one_call} page_groups={page_groups}", flush=True)
    done = np.zeros(w.batch, dtype=np.int64)
    while np.any(done < lens):
        n = np.minimum(lens - done, CHUNK)
        k, v = wl.torch_kv(torch, w, params, int(n.max()), gen, dev)
        cache.append(k, v, n.tolist())
        for (b, h), oh in oracles.items():
            if n[b]:
                oh.append(k[b, :n[b], h].cpu().numpy(), v[b, :n[b], h].cpu().numpy())
        done += n
    torch.cuda.synchronize()
    print(f"  prefill done", flush=True)
    ratio = w.num_q_heads // w.num_kv_heads
    worst = 0.0
    for s in range(steps):
        k, v = wl.torch_kv(torch, w, params, 1, gen, dev)
        for (b, h), oh in oracles.items():
            oh.append(k[b, :1, h].cpu().numpy(), v[b, :1, h].cpu().numpy())
        q = torch.randn((w.batch, w.num_q_heads, w.head_dim), generator=gen, device=dev).to(torch.float16)
        if one_call:
            out = cache.step(k, v, q)
        else:
            cache.append(k, v)
            out = cache.decode(q)
        if s in check_steps:
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            qh = q.cpu().numpy()
            for (b, h), oh in oracles.items():
                T, Q = cache.seq_len(b)
                assert (T, Q) == (oh.T, oh.Q)
                exp = oh.attend(qh[b, h * ratio:(h + 1) * ratio])
                err = float(np.abs(got[b, h * ratio:(h + 1) * ratio] - exp).max())
                assert np.all(np.isfinite(got[b])), "non-finite output"
                assert err <= OUT_TOL, f"step {s} (b={b}, h={h}) T={T}: max |gpu - oracle| = {err:.3e}"
                worst = max(worst, err)
            print(f"  step {s}: outputs of sampled heads within {worst:.2e}", flush=True)
    for (b, h), oh in oracles.items():
        _check_blocks(cache, oh, b, h, group_sample)
    print(f"  blocks and window of sampled heads bit-exact; worst output error {worst:.2e}", flush=True)
    cache.close()
    return worst


def test_full_llama2_7b_b8_32k(dev):
    # flushes at T = 32800 (step 31) and T = 32832 (step 63)
    _run_full(wl.WORKLOADS["llama2_7b_b8_32k"], dev, [(0, 0), (3, 17), (7, 31)], 64, {0, 31, 32, 63})


@pytest.mark.parametrize("name", ["gqa_128k_2bit", "gqa_128k_3bit", "gqa_128k_4bit"])
def test_full_gqa_128k(dev, name):
    _run_full(wl.WORKLOADS[name], dev, [(0, 0), (0, 5)], 1, {0})


def test_full_gqa_128k_one_call_steps(dev):
    # the bench's step: kvq_decode_step with the automatic (weighted) split plan over
    # 40 steps, so one group leaves the window (T - R crosses 131072 + 32 at step 31)
    _run_full(wl.WORKLOADS["gqa_128k_2bit"], dev, [(0, 0), (0, 3), (0, 6)], 40, {0, 30, 31, 39}, one_call=True)


def test_full_gqa_128k_paged_one_call_steps(dev):
    # the paged headline as the bench times it: 16-group pages in random order, one-call
    # steps across a group flush
    _run_full(wl.WORKLOADS["gqa_128k_2bit"], dev, [(0, 1), (0, 7)], 36, {0, 34, 35}, one_call=True,
              page_groups=16)


def test_full_llama2_7b_b8_32k_one_call_steps(dev):
    # batch 8: the folded window write with inline sequence records, flush at step 31
    _run_full(wl.WORKLOADS["llama2_7b_b8_32k"], dev, [(0, 0), (5, 20)], 33, {0, 31, 32}, one_call=True)


def test_full_gqa_128k_hg8(dev):
    # 8 query heads per KV head: a column kind per head and part, no copies
    _run_full(wl.WORKLOADS["gqa_128k_2bit_hg8"], dev, [(0, 2), (0, 7)], 1, {0})


def test_full_million_1m(dev):
    sample = lambda ng: list(range(0, ng, 97)) + list(range(ng - 40, ng))
    _run_full(wl.WORKLOADS["million_1m"], dev, [(0, 3)], 1, {0}, group_sample=sample)


def test_full_gqa_128k_rope_sink(dev):
    # pre-RoPE keys (rotated after dequantization) with an attention sink, two steps
    _run_full(wl.WORKLOADS["gqa_128k_2bit_rope"], dev, [(0, 1), (0, 6)], 2, {0, 1})


def test_full_ragged_b64_wht(dev):
    _run_full(wl.WORKLOADS["ragged_b64_wht"], dev, [(0, 0), (17, 5), (63, 7)], 32, {0, 15, 31})
