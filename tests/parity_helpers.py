"""Shared driver for GPU-vs-oracle parity checks.

Feeds the same seeded fp16 inputs to the HIP library (through its C ABI binding)
and to the CPU oracle, then compares packed group blocks and FP16-window contents
bit for bit and decode outputs within the output tolerance.
"""
from __future__ import annotations

import numpy as np

import kvq_workloads as wl
from oracle import OracleCache, OracleHead

OUT_TOL = 2e-3  # max-abs output error against the float64 oracle (fp32 accumulation)


def to_dev(x, torch, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


class Pair:
    """A GPU cache and its oracle twin fed with identical inputs."""

    def __init__(self, w: wl.Workload, max_tokens: int, device, torch, groups_per_split=0, **cache_kw):
        import bit_asymmetric_kv_amd as kvq
        self.w = w
        self.torch = torch
        self.dev = device
        self.gpu = kvq.KVCache(w.batch, w.num_q_heads, w.num_kv_heads, bits=w.bits, group=w.group,
                               residual=w.residual, rotate=w.rotate, max_tokens=max_tokens, device=device,
                               sink=w.sink, rope=w.rope, **cache_kw)
        if groups_per_split:
            self.gpu.set_decode_split(groups_per_split)
        self.ref = OracleCache(w.batch, w.num_q_heads, w.num_kv_heads, w.bits, w.residual, w.rotate, sink=w.sink,
                               rope=w.rope)
        self.T = np.zeros(w.batch, dtype=np.int64)
        self.step = 0

    def append(self, n_tokens):
        n_tokens = np.asarray(n_tokens, dtype=np.int64)
        n_max = int(n_tokens.max()) if len(n_tokens) else 0
        k, v = wl.kv_batch(self.w, self.T, max(n_max, 1), n_tokens)
        self.gpu.append(to_dev(k, self.torch, self.dev), to_dev(v, self.torch, self.dev), n_tokens.tolist())
        self.ref.append(k, v, n_tokens)
        self.T += n_tokens

    def check_state(self, heads=None):
        """Packed groups and FP16 window of (b, h) pairs: bit-exact."""
        w = self.w
        pairs = heads or [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
        for b, h in pairs:
            T, Q = self.gpu.seq_len(b)
            oh: OracleHead = self.ref.heads[b][h]
            assert (T, Q) == (oh.T, oh.Q), f"lengths of seq {b}: gpu {(T, Q)} oracle {(oh.T, oh.Q)}"
            ng = Q // w.group
            if ng:
                got = self.gpu.read_groups(b, h, 0, ng)
                for g in range(ng):
                    exp = oh.block(g)
                    if not np.array_equal(got[g], exp):
                        bad = np.nonzero(got[g] != exp)[0]
                        raise AssertionError(f"group block (b={b}, h={h}, g={g}) differs at {len(bad)} bytes, "
                                             f"first byte {bad[0]}")
            W = w.residual + w.group
            rk = self.gpu.read_ring(b, h, "k")
            rv = self.gpu.read_ring(b, h, "v")
            o = 1 if w.sink else 0
            # window tokens [o + Q, T) in slot t % W; an attention sink (token 0) in slot W
            slots = [(t, t % W) for t in range(o + Q, T)] + ([(0, W)] if w.sink and T > 0 else [])
            for t, slot in slots:
                gk, ok_ = rk[slot], oh.k16[t]
                if not np.array_equal(gk.view(np.uint16), ok_.view(np.uint16)):
                    bad = np.nonzero(gk.view(np.uint16) != ok_.view(np.uint16))[0]
                    raise AssertionError(
                        f"ring key (b={b}, h={h}, t={t}, slot {slot}, T={T}, Q={Q}) differs in {len(bad)} "
                        f"channels {bad[:6].tolist()}: gpu {gk[bad[:4]].tolist()} oracle {ok_[bad[:4]].tolist()}")
                assert np.array_equal(rv[slot].view(np.uint16), oh.v16[t].view(np.uint16)), \
                    f"ring value (b={b}, h={h}, t={t}, slot {slot})"

    def decode(self):
        q = wl.queries(self.w, self.step)
        self.step += 1
        out = self.gpu.decode(to_dev(q, self.torch, self.dev))
        self.torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        exp = self.ref.decode(q)
        return got, exp

    def check_decode(self, tol=OUT_TOL):
        got, exp = self.decode()
        err = float(np.abs(got - exp).max())
        assert np.all(np.isfinite(got)), "non-finite output"
        assert err <= tol, f"max |gpu - oracle| = {err:.3e} > {tol}"
        return err
