"""Seeded synthetic inputs for the decode-attention workloads.

This module only draws random numbers and rounds them to fp16; it holds none of
the quantization or attention arithmetic. Both the oracle-side tests and the GPU
path are fed from it, so both see identical bits.

The pages measure on real models (LLaMA / Mistral layers); no dataset or weights
are used here. Each workload draws keys, values and queries with the shapes and
the key outlier structure the pages describe: keys carry a few fixed
large-magnitude channels, values show no channel structure ("KV cache
quantization: putting the bits in the cached vectors", full-text-skim notes).

Every tensor is generated per (tensor id, sequence, kv-head, 1,024-token chunk)
from numpy's PCG64 seeded by SeedSequence([seed, tensor id, b, h, chunk]), so any
token range of any head can be regenerated without materialising the rest.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from functools import lru_cache

import numpy as np

CHUNK = 1024
HEAD_DIM = 128

_TID_K, _TID_V, _TID_Q, _TID_OUTLIER, _TID_OFFSET, _TID_LENS = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    context: int                 # prefill tokens per sequence (uniform case)
    steps: int                   # decode steps, each appending one token per sequence
    bits: int
    group: int
    residual: int
    rotate: bool
    n_outliers: int              # key outlier channels per kv-head
    outlier_mult: float          # their multiplier
    offset_sigma: float          # per-channel key offset ~ N(0, sigma); 0 = none
    seed: int
    ragged: tuple = field(default=())   # (lo, hi) inclusive per-sequence context range
    head_dim: int = HEAD_DIM
    sink: bool = False           # token 0 kept FP16 as an attention sink
    rope: bool = False           # keys pre-RoPE, rotated after dequantization

    def context_lengths(self) -> np.ndarray:
        """Prefill length of every sequence."""
        if not self.ragged:
            return np.full(self.batch, self.context, dtype=np.int64)
        lo, hi = self.ragged
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, _TID_LENS])))
        return rng.integers(lo, hi + 1, size=self.batch, dtype=np.int64)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads: the five configurations (the 128K one at 2, 3 and 4 bits) and two
# variants of the 128K shape; shapes, bit widths, window sizes and key distributions.
WORKLOADS = {
    "tiny_mha_4k": Workload("tiny_mha_4k", 1, 8, 8, 4096, 1, 2, 32, 32, False, 4, 10.0, 0.0, 1001),
    "llama2_7b_b8_32k": Workload("llama2_7b_b8_32k", 8, 32, 32, 32768, 64, 2, 32, 128, False, 8, 8.0, 0.0, 1002),
    "gqa_128k_2bit": Workload("gqa_128k_2bit", 1, 32, 8, 131072, 1, 2, 32, 128, False, 4, 10.0, 3.0, 1003),
    "gqa_128k_3bit": Workload("gqa_128k_3bit", 1, 32, 8, 131072, 1, 3, 32, 128, False, 4, 10.0, 3.0, 1003),
    "gqa_128k_4bit": Workload("gqa_128k_4bit", 1, 32, 8, 131072, 1, 4, 32, 128, False, 4, 10.0, 3.0, 1003),
    "million_1m": Workload("million_1m", 1, 32, 8, 1048576, 1, 2, 32, 128, False, 8, 8.0, 0.0, 1004),
    "ragged_b64_wht": Workload("ragged_b64_wht", 64, 32, 8, 0, 32, 2, 32, 64, True, 8, 8.0, 0.0, 1005,
                               ragged=(2048, 32768)),
    # the headline shape with pre-RoPE keys and an attention sink
    "gqa_128k_2bit_rope": Workload("gqa_128k_2bit_rope", 1, 32, 8, 131072, 1, 2, 32, 128, False, 4, 10.0, 3.0,
                                   1006, sink=True, rope=True),
    # the headline context with 8 query heads per KV head (64 / 8, a 70B-class layer)
    "gqa_128k_2bit_hg8": Workload("gqa_128k_2bit_hg8", 1, 64, 8, 131072, 1, 2, 32, 128, False, 4, 10.0, 3.0, 1007),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def key_channel_params(w: Workload, h: int):
    """(multiplier [D] fp32, offset [D] fp32) of kv-head h's keys."""
    mult = np.ones(w.head_dim, dtype=np.float32)
    if w.n_outliers:
        ch = _rng(w.seed, _TID_OUTLIER, h).choice(w.head_dim, size=w.n_outliers, replace=False)
        mult[ch] = np.float32(w.outlier_mult)
    off = np.zeros(w.head_dim, dtype=np.float32)
    if w.offset_sigma:
        off = (_rng(w.seed, _TID_OFFSET, h).standard_normal(w.head_dim) * w.offset_sigma).astype(np.float32)
    return mult, off


@lru_cache(maxsize=2048)
def _chunk_normals(w: Workload, tid: int, b: int, h: int, c: int) -> np.ndarray:
    x = _rng(w.seed, tid, b, h, c).standard_normal((CHUNK, w.head_dim), dtype=np.float32)
    x.flags.writeable = False
    return x


def _token_range(w: Workload, tid: int, b: int, h: int, t0: int, t1: int) -> np.ndarray:
    out = np.empty((t1 - t0, w.head_dim), dtype=np.float32)
    pos = t0
    while pos < t1:
        c = pos // CHUNK
        lo = pos - c * CHUNK
        hi = min(CHUNK, t1 - c * CHUNK)
        out[pos - t0:pos - t0 + hi - lo] = _chunk_normals(w, tid, b, h, c)[lo:hi]
        pos = c * CHUNK + hi
    return out


def keys(w: Workload, b: int, h: int, t0: int, t1: int) -> np.ndarray:
    """Keys of tokens [t0, t1) of sequence b, kv-head h: fp16 [t1 - t0, D].

    k = m_d * (N(0, 1) + mu_d): m_d is the outlier multiplier (1 elsewhere), mu_d a
    fixed per-channel offset (0 unless the workload has one)."""
    mult, off = key_channel_params(w, h)
    x = _token_range(w, _TID_K, b, h, t0, t1)
    return (mult * (x + off)).astype(np.float16)


def values(w: Workload, b: int, h: int, t0: int, t1: int) -> np.ndarray:
    """Values of tokens [t0, t1): fp16 N(0, 1), [t1 - t0, D]."""
    return _token_range(w, _TID_V, b, h, t0, t1).astype(np.float16)


def kv_batch(w: Workload, t0s, n_max: int, n_tokens=None):
    """Stacked [B, n_max, Hkv, D] fp16 keys and values for an append call.

    Sequence b contributes tokens [t0s[b], t0s[b] + n_b); padding rows are zero."""
    B, H, D = w.batch, w.num_kv_heads, w.head_dim
    k = np.zeros((B, n_max, H, D), dtype=np.float16)
    v = np.zeros((B, n_max, H, D), dtype=np.float16)
    for b in range(B):
        n = n_max if n_tokens is None else int(n_tokens[b])
        if n == 0:
            continue
        for h in range(H):
            k[b, :n, h] = keys(w, b, h, int(t0s[b]), int(t0s[b]) + n)
            v[b, :n, h] = values(w, b, h, int(t0s[b]), int(t0s[b]) + n)
    return k, v


def queries(w: Workload, step: int) -> np.ndarray:
    """Query of decode step `step`: fp16 N(0, 1), [B, Hq, D]."""
    q = np.empty((w.batch, w.num_q_heads, w.head_dim), dtype=np.float16)
    for b in range(w.batch):
        q[b] = _rng(w.seed, _TID_Q, b, step).standard_normal((w.num_q_heads, w.head_dim)).astype(np.float16)
    return q


def algorithmic_bytes(T: int, Q: int, bits: int, group: int = 32, head_dim: int = HEAD_DIM) -> int:
    """Bytes one decode step must read for one (sequence, kv-head): packed codes,
    fp16 scales and zero-points of the Q quantized tokens, and the fp16 keys and
    values of the T - Q residual tokens."""
    n_groups = Q // group
    per_group = 2 * group * head_dim * bits // 8 + 2 * (2 * head_dim) + 2 * (2 * group * head_dim // group)
    return n_groups * per_group + (T - Q) * 2 * 2 * head_dim


def torch_key_params(torch, w: Workload, device):
    """(multiplier, offset) of every kv-head's keys as device tensors [Hkv, D]."""
    mult = np.stack([key_channel_params(w, h)[0] for h in range(w.num_kv_heads)])
    off = np.stack([key_channel_params(w, h)[1] for h in range(w.num_kv_heads)])
    return torch.tensor(mult, device=device), torch.tensor(off, device=device)


def torch_kv(torch, w: Workload, params, n: int, gen, device):
    """Seeded fp16 keys / values [B, n, Hkv, D] drawn on the device with the
    workload's distribution (same rule as keys() / values(): k = m_d * (N(0,1) + mu_d),
    v = N(0,1)), from torch's generator `gen`. For runs too large to draw on the
    host; callers that check against the oracle copy the rows they check back."""
    mult, off = params
    shape = (w.batch, n, w.num_kv_heads, w.head_dim)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k = (mult * (k + off)).to(torch.float16)
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.float16)
    return k.contiguous(), v.contiguous()
