"""Plain CPU oracle: KIVI-style asymmetric low-bit KV cache + decode attention.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path. Written in numpy from the
pages' description; it shares no code, header, table or constant with the HIP
library.

What it computes, in the pages' order:

* Rotation (optional): a normalized Walsh-Hadamard transform applied to q and k,
  which keeps q.k unchanged because the transform is orthogonal
  ("The Asymmetric Key-Value Cache Compression Framework", Method and In practice;
  "Read What Matters", the Dual-QK abstract on the same orthogonal transform being
  applied to queries).
* Keys are quantized per channel over a group of G tokens, values per token over a
  group of G channels ("The Asymmetric Key-Value Cache Compression Framework",
  Summary and Method; "KV cache quantization: putting the bits in the cached
  vectors", full-text-skim notes on the fixed outlier channels of keys and the
  per-token confinement of values).
* Asymmetric uniform quantizer: 2^b levels between the group's min and max, with
  a scale and a zero-point ("KVQuant" review, Problem: 8 levels at 3 bits, 4 at
  2 bits); b = 2, 3 or 4.
* The most recent tokens stay in FP16 ("The Asymmetric Key-Value Cache Compression
  Framework", In practice); quantized groups are appended along the token
  dimension and combined with the FP16 residual inside attention
  ("KV cache quantization ...", full-text-skim notes on KIVI's grouped/residual split).
* Decode attention: standard scaled dot-product softmax attention over every cached
  token, computed here in float64 on the dequantized cache.
* Pre-RoPE keys (optional): keys are quantized before the rotary position
  embedding and the rotation is applied after dequantization, at each key's
  position ("KVQuant" review, Method and Key idea: quantize keys per channel
  before RoPE, apply RoPE after dequantization; Prior limitations: RoPE rotates
  and mixes channel pairs, smearing the outlier channels).

Readings where the pages are silent (each is listed with its reason in the design
notes of the repository):

* quantizer: s32 = (max - min) / (2^b - 1) in fp32; s and z stored as fp16 (RNE),
  z = min; codes = clamp(rint_even(fp32(x - z) * fp32(1 / s16)), 0, 2^b - 1);
  a group whose fp16 scale is 0 gets all-zero codes;
* residual rule: Q = G * floor(max(0, T - R) / G) tokens are quantized; the rest
  (between R and R + G - 1 of them once T >= R) stay FP16;
* key groups are token ranges [gG, gG + G) aligned to token 0; value groups are
  channel ranges [jG, jG + G); one G serves both;
* rotation: Sylvester (natural) order butterflies in fp32, then one multiply by
  fp32(1/sqrt(128)); rotated k rounded to fp16 before it is stored or quantized;
  rotated q kept in fp32; v is not rotated;
* softmax scale 1/sqrt(head_dim) unless given; query head hq reads KV head
  hq // (Hq // Hkv);
* RoPE (the pages do not define it; the standard rotary embedding is taken): the
  channel pairs (f, f + 64), f = 0..63, of a key at position t (its 0-based index
  in the sequence) are rotated by the angle t * theta_f, theta_f = base^(-f / 64),
  base 10000 unless given: (a, b) -> (a cos - b sin, b cos + a sin); the query is
  passed already rotated at its own position, so attention reads q . RoPE_t(k).

The packed layout of one group block is this library's own storage format (the
pages only ask for a fixed per-token bit count); it is restated here from its
definition, independently of the GPU code, so that packed words can be compared
bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128
GROUP = 32

_F32 = np.float32
_F16 = np.float16


# ---------------------------------------------------------------------------
# Rotation
# ---------------------------------------------------------------------------
def wht128_fp32(x: np.ndarray) -> np.ndarray:
    """Normalized Walsh-Hadamard transform over the last axis (length 128), fp32.

    Butterfly stages with half-width h = 1, 2, 4, ..., 64 in natural (Sylvester)
    order: for each block of 2h entries, (a, b) -> (a + b, a - b), each a single
    fp32 rounding; then one fp32 multiply by fp32(1/sqrt(128)).
    Result equals hadamard(128) @ x / sqrt(128) up to fp32 rounding.
    """
    y = np.array(x, dtype=_F32, copy=True)
    n = y.shape[-1]
    if n != HEAD_DIM:
        raise ValueError("rotation is defined for head_dim 128")
    lead = y.shape[:-1]
    h = 1
    while h < n:
        v = y.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = (a + b).astype(_F32)
        v[..., 1, :] = (a - b).astype(_F32)
        y = v.reshape(lead + (n,))
        h *= 2
    return (y * _F32(1.0 / math.sqrt(128.0))).astype(_F32)


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------
def quantize_uniform(x: np.ndarray, bits: int, axis: int):
    """Asymmetric uniform b-bit quantization of fp16 data along `axis`.

    Each slice along `axis` is one quantization group. Returns (codes uint8,
    s16, z16), where s16/z16 have `axis` removed. Every step is an explicit fp32
    (or fp16 storage) rounding as stated in the module docstring.
    """
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    x16 = np.asarray(x, dtype=_F16)
    x32 = x16.astype(_F32)
    levels = _F32(2 ** bits - 1)
    mn = x32.min(axis=axis)
    mx = x32.max(axis=axis)
    rng = (mx - mn).astype(_F32)
    s32 = (rng / levels).astype(_F32)
    s16 = s32.astype(_F16)
    z16 = mn.astype(_F16)
    s16_32 = s16.astype(_F32)
    zero_scale = s16_32 == _F32(0)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = (_F32(1.0) / np.where(zero_scale, _F32(1.0), s16_32)).astype(_F32)
    inv_b = np.expand_dims(inv, axis)
    z_b = np.expand_dims(z16.astype(_F32), axis)
    diff = (x32 - z_b).astype(_F32)
    prod = (diff * inv_b).astype(_F32)
    r = np.rint(prod).astype(_F32)  # numpy rint rounds half to even
    r = np.clip(r, _F32(0), levels)
    codes = r.astype(np.uint8)
    codes = np.where(np.expand_dims(zero_scale, axis), np.uint8(0), codes).astype(np.uint8)
    return codes, s16, z16


def quantize_key_group(k_group: np.ndarray, bits: int):
    """Keys of one token group, shape [G, D] fp16: per-channel quantization.

    Returns codes [G, D] uint8, s16 [D], z16 [D].
    """
    return quantize_uniform(k_group, bits, axis=0)


def quantize_value_group(v_group: np.ndarray, bits: int, group: int = GROUP):
    """Values of one token group, shape [G, D] fp16: per-token quantization over
    channel groups of `group` channels.

    Returns codes [G, D] uint8, s16 [G, D // group], z16 [G, D // group].
    """
    g, d = v_group.shape
    v = np.asarray(v_group, dtype=_F16).reshape(g, d // group, group)
    codes, s16, z16 = quantize_uniform(v, bits, axis=2)
    return codes.reshape(g, d), s16, z16


# ---------------------------------------------------------------------------
# Group block storage format (head_dim 128, G 32)
# ---------------------------------------------------------------------------
def group_block_bytes(bits: int) -> int:
    """Bytes of one (sequence, kv-head, 32-token group) block."""
    code_bytes = GROUP * HEAD_DIM * bits // 8
    return 2 * code_bytes + 512 + 512


def _code_position(o, lane, slot, bits):
    """Byte offset of the 32-bit word and bit offset inside it for a code (2 and
    4 bits: one field per code).

    Codes of one section (keys or values) are addressed by (operand o in [0, 8),
    lane in [0, 64), slot in [0, 8)).
      2-bit: word at byte 16*lane + 4*(o // 2);
             bit 8*(slot // 2) + 4*(slot % 2) + 2*(o % 2).
      4-bit: word at byte 1024*(o // 4) + 16*lane + 4*(o % 4);
             bit 8*(slot % 4) + 4*(slot // 4).
    """
    o = np.asarray(o)
    lane = np.asarray(lane)
    slot = np.asarray(slot)
    if bits == 2:
        word = 16 * lane + 4 * (o // 2)
        bit = 8 * (slot // 2) + 4 * (slot % 2) + 2 * (o % 2)
    else:
        word = 1024 * (o // 4) + 16 * lane + 4 * (o % 4)
        bit = 8 * (slot % 4) + 4 * (slot // 4)
    return word, bit


def _code_fields(o, lane, slot, bits):
    """Fields (word byte offset, bit offset, width, code bit) holding one code.

    2 and 4 bits: one field of the code's full width (see _code_position).
    3 bits: the two low bits in a 1024-byte plane, word at byte 16*lane + 4*(o//2),
    bit 8*(slot % 4) + 4*(slot // 4) + 2*(o % 2); the high bit in a 512-byte plane
    after it, word at byte 1024 + 8*lane + 4*(o // 4), bit 8*(slot % 4) +
    4*(slot // 4) + (o % 4). (With both fields in place a lane's code nibbles line
    up as in the 4-bit layout.)
    """
    if bits != 3:
        word, bit = _code_position(o, lane, slot, bits)
        return [(word, bit, bits, 0)]
    o = np.asarray(o)
    lane = np.asarray(lane)
    slot = np.asarray(slot)
    base_bit = 8 * (slot % 4) + 4 * (slot // 4)
    lo = (16 * lane + 4 * (o // 2), base_bit + 2 * (o % 2), 2, 0)
    hi = (1024 + 8 * lane + 4 * (o // 4), base_bit + (o % 4), 1, 2)
    return [lo, hi]


def _key_code_coords(i, d):
    """(operand, lane, slot) of key token i (0..31), channel d (0..127)."""
    o = 2 * (d // 32) + i // 16
    lane = i % 16 + 16 * ((d % 32) // 8)
    slot = d % 8
    return o, lane, slot


def _value_code_coords(i, d):
    """(operand, lane, slot) of value token i (0..31), channel d (0..127)."""
    o = d // 16
    lane = d % 16 + 16 * ((i % 16) // 4)
    slot = 4 * (i // 16) + i % 4
    return o, lane, slot


def _value_scale_index(i, j):
    """f16 index of the value scale (or zero) of token i, channel group j."""
    kb = (i % 16) // 4
    slot = 4 * (i // 16) + i % 4
    return (kb * 4 + j) * 8 + slot


def _section_positions(coords_fn, bits):
    """For every code (i, d) of a section, per field: 32-bit word index, bit
    offset, width and the code bit the field starts at."""
    ii, dd = np.meshgrid(np.arange(GROUP), np.arange(HEAD_DIM), indexing="ij")
    o, lane, slot = coords_fn(ii, dd)
    return [((word // 4).astype(np.int64), np.asarray(bit).astype(np.uint32), width, shift)
            for word, bit, width, shift in _code_fields(o, lane, slot, bits)]


_POS_CACHE = {}


def _positions(coords_fn, bits):
    key = (coords_fn.__name__, bits)
    if key not in _POS_CACHE:
        _POS_CACHE[key] = _section_positions(coords_fn, bits)
    return _POS_CACHE[key]


def _pack_section(codes, coords_fn, bits, nbytes):
    words = np.zeros(nbytes // 4, dtype=np.uint32)
    c = codes.astype(np.uint32)
    for widx, bit, width, shift in _positions(coords_fn, bits):
        field = (c >> np.uint32(shift)) & np.uint32(2 ** width - 1)
        np.bitwise_or.at(words, widx.ravel(), (field << bit).ravel())
    return words


def _unpack_section(words, coords_fn, bits):
    out = np.zeros((GROUP, HEAD_DIM), dtype=np.uint32)
    for widx, bit, width, shift in _positions(coords_fn, bits):
        out |= ((words[widx] >> bit) & np.uint32(2 ** width - 1)) << np.uint32(shift)
    return out.astype(np.uint8)


def _value_scale_indices():
    ii, jj = np.meshgrid(np.arange(GROUP), np.arange(HEAD_DIM // GROUP), indexing="ij")
    return _value_scale_index(ii, jj)


def pack_group_block(kc, ks, kz, vc, vs, vz, bits):
    """Pack one group's codes, scales and zero-points into its byte block.

    kc, vc: [32, 128] codes; ks, kz: [128] fp16; vs, vz: [32, 4] fp16.
    Block = [key codes | value codes | key s[128] | key z[128] |
             value s (256 B) | value z (256 B)], little-endian.
    """
    cb = GROUP * HEAD_DIM * bits // 8
    kw = _pack_section(kc, _key_code_coords, bits, cb)
    vw = _pack_section(vc, _value_code_coords, bits, cb)
    idx = _value_scale_indices()
    vs_arr = np.zeros(128, dtype=_F16)
    vz_arr = np.zeros(128, dtype=_F16)
    vs_arr[idx] = vs
    vz_arr[idx] = vz
    out = b"".join([
        kw.astype("<u4").tobytes(),
        vw.astype("<u4").tobytes(),
        np.asarray(ks, dtype="<f2").tobytes(),
        np.asarray(kz, dtype="<f2").tobytes(),
        vs_arr.astype("<f2").tobytes(),
        vz_arr.astype("<f2").tobytes(),
    ])
    assert len(out) == group_block_bytes(bits)
    return np.frombuffer(out, dtype=np.uint8).copy()


def unpack_group_block(block, bits):
    """Inverse of pack_group_block: returns (kc, ks, kz, vc, vs, vz)."""
    block = np.asarray(block, dtype=np.uint8)
    cb = GROUP * HEAD_DIM * bits // 8
    kw = block[:cb].view("<u4")
    vw = block[cb:2 * cb].view("<u4")
    ks = block[2 * cb:2 * cb + 256].view("<f2").astype(_F16)
    kz = block[2 * cb + 256:2 * cb + 512].view("<f2").astype(_F16)
    vs_arr = block[2 * cb + 512:2 * cb + 768].view("<f2")
    vz_arr = block[2 * cb + 768:2 * cb + 1024].view("<f2")
    kc = _unpack_section(kw, _key_code_coords, bits)
    vc = _unpack_section(vw, _value_code_coords, bits)
    idx = _value_scale_indices()
    vs = vs_arr[idx].astype(_F16)
    vz = vz_arr[idx].astype(_F16)
    return kc, ks, kz, vc, vs, vz


def dequantize_block(kc, ks, kz, vc, vs, vz):
    """x_hat = z + s * c, exact in float64. Returns (k_hat [32,128], v_hat [32,128])."""
    k_hat = kz.astype(np.float64)[None, :] + ks.astype(np.float64)[None, :] * kc.astype(np.float64)
    vs_full = np.repeat(vs.astype(np.float64), GROUP, axis=1)
    vz_full = np.repeat(vz.astype(np.float64), GROUP, axis=1)
    v_hat = vz_full + vs_full * vc.astype(np.float64)
    return k_hat, v_hat


# ---------------------------------------------------------------------------
# Streaming rule and attention
# ---------------------------------------------------------------------------
def quantized_count(T: int, R: int, G: int = GROUP, sink: bool = False) -> int:
    """Number of tokens held quantized: G * floor(max(0, T - o - R) / G), o = 1 with
    an attention sink (token 0 stays FP16 and groups start at token 1), else 0.
    The quantized tokens are [o, o + count)."""
    o = 1 if sink else 0
    return G * (max(0, T - o - R) // G)


ROPE_BASE = 10000.0


def rope_fp64(x: np.ndarray, positions, base: float = ROPE_BASE) -> np.ndarray:
    """Rotary position embedding of rows x [n, 128] at integer positions [n], in
    float64: channel f and channel f + 64 form a pair rotated by position * theta_f
    with theta_f = base^(-f / 64) (the standard rotary embedding, pairs taken as the
    two halves of the head; see the module notes)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    theta = float(base) ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=1)


def attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of query rows q [H, D] over keys/values [T, D], float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


class OracleHead:
    """One (sequence, kv-head) stream: FP16 residual + quantized token groups.

    With `sink`, token 0 is an attention sink: it stays FP16 for good and the
    groups cover tokens [1 + g G, 1 + (g + 1) G) ("KV cache quantization: putting
    the bits in the cached vectors", full-text-skim notes: keeping the first token
    in fp16 helps, most at 2 bits).

    With `rope`, the appended keys are pre-RoPE: they are stored and quantized as
    given, and attention rotates every key, dequantized or FP16, at its position
    ("KVQuant" review, Method and Key idea)."""

    def __init__(self, bits: int, residual: int, rotate: bool = False,
                 head_dim: int = HEAD_DIM, group: int = GROUP, sink: bool = False,
                 rope: bool = False, rope_base: float = ROPE_BASE):
        if head_dim != HEAD_DIM or group != GROUP:
            raise ValueError("oracle block format is defined for head_dim 128, G 32")
        if rope and rotate:
            raise ValueError("pre-RoPE keys and the Walsh-Hadamard rotation are exclusive")
        if residual < 0 or residual % group:
            raise ValueError("residual must be a non-negative multiple of G")
        self.bits = bits
        self.R = residual
        self.G = group
        self.rotate = bool(rotate)
        self.sink = bool(sink)
        self.o = 1 if sink else 0   # first token of group 0
        self.rope = bool(rope)
        self.rope_base = float(rope_base)
        self.k16 = np.zeros((0, head_dim), dtype=_F16)   # every appended key (rotated if asked)
        self.v16 = np.zeros((0, head_dim), dtype=_F16)
        nv = head_dim // group
        # quantized groups, oldest first
        self.kc = np.zeros((0, group, head_dim), dtype=np.uint8)
        self.ks = np.zeros((0, head_dim), dtype=_F16)
        self.kz = np.zeros((0, head_dim), dtype=_F16)
        self.vc = np.zeros((0, group, head_dim), dtype=np.uint8)
        self.vs = np.zeros((0, group, nv), dtype=_F16)
        self.vz = np.zeros((0, group, nv), dtype=_F16)

    @property
    def T(self) -> int:
        return self.k16.shape[0]

    @property
    def Q(self) -> int:
        return self.kc.shape[0] * self.G

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        """Append n tokens (k, v: [n, D] fp16), then quantize every group that the
        residual rule moves out of the FP16 window, oldest first. Groups are
        independent, so the due groups are quantized together."""
        k = np.asarray(k, dtype=_F16)
        v = np.asarray(v, dtype=_F16)
        if self.rotate and k.shape[0]:
            k = wht128_fp32(k.astype(_F32)).astype(_F16)
        self.k16 = np.concatenate([self.k16, k], axis=0)
        self.v16 = np.concatenate([self.v16, v], axis=0)
        target = quantized_count(self.T, self.R, self.G, self.sink)
        if self.Q >= target:
            return
        t0, t1 = self.o + self.Q, self.o + target
        n = (t1 - t0) // self.G
        kg = self.k16[t0:t1].reshape(n, self.G, HEAD_DIM)
        vg = self.v16[t0:t1].reshape(n, self.G, HEAD_DIM // self.G, self.G)
        kc, ks, kz = quantize_uniform(kg, self.bits, axis=1)      # per channel, over G tokens
        vc, vs, vz = quantize_uniform(vg, self.bits, axis=3)      # per token, over G channels
        self.kc = np.concatenate([self.kc, kc], axis=0)
        self.ks = np.concatenate([self.ks, ks], axis=0)
        self.kz = np.concatenate([self.kz, kz], axis=0)
        self.vc = np.concatenate([self.vc, vc.reshape(n, self.G, HEAD_DIM)], axis=0)
        self.vs = np.concatenate([self.vs, vs], axis=0)
        self.vz = np.concatenate([self.vz, vz], axis=0)

    def group(self, g: int):
        """(kc, ks, kz, vc, vs, vz) of quantized group g."""
        return self.kc[g], self.ks[g], self.kz[g], self.vc[g], self.vs[g], self.vz[g]

    def block(self, g: int) -> np.ndarray:
        """Packed byte block of quantized group g."""
        return pack_group_block(*self.group(g), self.bits)

    def cache_values(self):
        """Keys and values as attention sees them: dequantized (float64) for the
        quantized tokens [o, o + Q), the stored fp16 values for the rest (the window
        [o + Q, T) and, with a sink, token 0). Attention does not depend on the
        order of the tokens, so the sink comes last here."""
        ng = self.kc.shape[0]
        k_hat = (self.kz.astype(np.float64)[:, None, :]
                 + self.ks.astype(np.float64)[:, None, :] * self.kc.astype(np.float64))
        vs_full = np.repeat(self.vs.astype(np.float64), self.G, axis=2)
        vz_full = np.repeat(self.vz.astype(np.float64), self.G, axis=2)
        v_hat = vz_full + vs_full * self.vc.astype(np.float64)
        k_tail = self.k16[self.o + self.Q:].astype(np.float64)
        v_tail = self.v16[self.o + self.Q:].astype(np.float64)
        pos = np.arange(self.o, self.T)          # quantized tokens, then the window
        if self.sink and self.T > 0:
            k_tail = np.concatenate([k_tail, self.k16[:1].astype(np.float64)], axis=0)
            v_tail = np.concatenate([v_tail, self.v16[:1].astype(np.float64)], axis=0)
            pos = np.concatenate([pos, [0]])
        k_all = np.concatenate([k_hat.reshape(ng * self.G, HEAD_DIM), k_tail], axis=0)
        v_all = np.concatenate([v_hat.reshape(ng * self.G, HEAD_DIM), v_tail], axis=0)
        if self.rope:
            k_all = rope_fp64(k_all, pos, self.rope_base)
        return k_all, v_all

    def prepare_query(self, q: np.ndarray) -> np.ndarray:
        """fp16 query rows [H, D] -> the values attention uses (rotated in fp32 if asked)."""
        q = np.asarray(q, dtype=_F16)
        if self.rotate:
            return wht128_fp32(q.astype(_F32)).astype(np.float64)
        return q.astype(np.float64)

    def attend(self, q: np.ndarray, scale: float | None = None) -> np.ndarray:
        """Decode attention of fp16 query rows q [H, D] over all T cached tokens."""
        if self.T == 0:
            raise ValueError("attention over an empty sequence")
        if scale is None:
            scale = 1.0 / math.sqrt(HEAD_DIM)
        k_all, v_all = self.cache_values()
        return attention_fp64(self.prepare_query(q), k_all, v_all, scale)


class OracleCache:
    """Batch of sequences x kv-heads, mirroring the library's cache object."""

    def __init__(self, batch, num_q_heads, num_kv_heads, bits, residual,
                 rotate=False, softmax_scale=None, head_dim=HEAD_DIM, group=GROUP, sink=False,
                 rope=False, rope_base=ROPE_BASE):
        if num_q_heads % num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        self.B = batch
        self.Hq = num_q_heads
        self.Hkv = num_kv_heads
        self.scale = softmax_scale if softmax_scale else 1.0 / math.sqrt(head_dim)
        self.heads = [[OracleHead(bits, residual, rotate, head_dim, group, sink, rope, rope_base)
                       for _ in range(num_kv_heads)] for _ in range(batch)]

    def append(self, k, v, n_tokens=None):
        """k, v: [B, n_max, Hkv, D] fp16; n_tokens: per-sequence count or None (all)."""
        n_max = k.shape[1]
        for b in range(self.B):
            n = n_max if n_tokens is None else int(n_tokens[b])
            for h in range(self.Hkv):
                self.heads[b][h].append(k[b, :n, h, :], v[b, :n, h, :])

    def seq_len(self, b):
        return self.heads[b][0].T, self.heads[b][0].Q

    def decode(self, q):
        """q: [B, Hq, D] fp16 -> out [B, Hq, D] float64."""
        ratio = self.Hq // self.Hkv
        out = np.zeros((self.B, self.Hq, q.shape[-1]), dtype=np.float64)
        for b in range(self.B):
            for h in range(self.Hkv):
                rows = slice(h * ratio, (h + 1) * ratio)
                out[b, rows] = self.heads[b][h].attend(q[b, rows], self.scale)
        return out
