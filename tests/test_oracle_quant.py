"""Pins for the oracle's asymmetric uniform quantizer and group packing.

Quantization axes: keys per channel over a token group, values per token over a
channel group ("The Asymmetric Key-Value Cache Compression Framework", Summary;
"KV cache quantization: putting the bits in the cached vectors", full-text-skim
notes: per-channel keys confine error to a channel, per-token values confine it
to a token). Levels: 2^b between min and max ("KVQuant" review, Problem).
"""
import json
import os

import numpy as np
import pytest

from oracle import (dequantize_block, group_block_bytes, pack_group_block, quantize_key_group,
                    quantize_uniform, quantize_value_group, unpack_group_block)
from oracle.kvq_oracle import _key_code_coords, _value_code_coords, _code_position, _code_fields, _value_scale_index

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("quantizer_cases.json")["cases"], ids=lambda c: str(c["x"])[:30])
def test_hand_worked_cases(case):
    x = np.array(case["x"], dtype=np.float16)
    assert np.array_equal(x.astype(np.float64), np.array(case["x"], dtype=np.float64)), "fixture not fp16-exact"
    codes, s16, z16 = quantize_uniform(x, case["bits"], axis=0)
    assert codes.tolist() == case["codes"]
    assert float(s16) == case["s16"]
    assert float(z16) == case["z16"]


def test_clamp_cases_bind():
    # The clamp_binds fixtures must really need the clamp: with the stored scale the
    # rounded product of the group maximum lies above the top level (checked here in
    # exact double arithmetic: every value is a small multiple of 2^-24).
    cases = [c for c in _load("quantizer_cases.json")["cases"] if c.get("clamp_binds")]
    assert {c["bits"] for c in cases} == {2, 3, 4}
    for c in cases:
        top = max(c["x"]) - c["z16"]
        assert round(top / c["s16"]) > 2 ** c["bits"] - 1 or top / c["s16"] == 2 ** c["bits"] - 0.5
        assert max(c["codes"]) == 2 ** c["bits"] - 1


def test_dequantize_block_hand_computed():
    # Per-channel key scales and per-(token, channel group) value scales that all
    # differ, so a transposed or tiled scale array reads a different entry.
    # Keys: ks[d] = d / 8, kz[d] = -d, kc[t, d] = (t + d) % 4.
    # Values: vs[t, j] = (t + 1) / 4 + j, vz[t, j] = j - t, vc[t, d] = (3 t + d) % 4,
    # channel d in group j = d // 32.
    d = np.arange(128)
    t = np.arange(32)[:, None]
    ks = (d / 8).astype(np.float16)
    kz = (-d).astype(np.float16)
    kc = ((t + d[None, :]) % 4).astype(np.uint8)
    j = np.arange(4)[None, :]
    vs = ((t + 1) / 4 + j).astype(np.float16)
    vz = (j - t).astype(np.float16)
    vc = ((3 * t + d[None, :]) % 4).astype(np.uint8)
    kh, vh = dequantize_block(kc, ks, kz, vc, vs, vz)
    assert kh.shape == vh.shape == (32, 128)
    # k[5, 70]: kc = 75 % 4 = 3, so -70 + (70 / 8) * 3 = -70 + 26.25 = -43.75
    assert kh[5, 70] == -43.75
    # k[31, 1]: kc = 32 % 4 = 0, so the zero-point -1 alone
    assert kh[31, 1] == -1.0
    # v[9, 100]: group 3, vs = 10 / 4 + 3 = 5.5, vz = 3 - 9 = -6, vc = 127 % 4 = 3:
    # -6 + 16.5 = 10.5 (channel 100 % 4 = 0 would read group 0: -9 + 2.5 * 3 = -1.5)
    assert vh[9, 100] == 10.5
    # v[0, 33]: group 1, vs = 1.25, vz = 1, vc = 33 % 4 = 1: 2.25
    assert vh[0, 33] == 2.25
    # v[20, 31]: group 0, vs = 5.25, vz = -20, vc = 91 % 4 = 3: -20 + 15.75 = -4.25
    assert vh[20, 31] == -4.25


def _rand_groups(rng, n, bits):
    scale = rng.choice([1e-3, 1.0, 30.0, 1000.0], size=(n, 1))
    off = rng.standard_normal((n, 1)) * scale * 3
    x = (rng.standard_normal((n, 32)) * scale + off).astype(np.float16)
    return x


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_invariants_random(bits):
    rng = np.random.default_rng(10 + bits)
    x = _rand_groups(rng, 4000, bits)
    codes, s16, z16 = quantize_uniform(x, bits, axis=1)
    L = 2 ** bits - 1
    assert codes.max() <= L and codes.min() >= 0
    x64 = x.astype(np.float64)
    mn = x64.min(axis=1)
    mx = x64.max(axis=1)
    # z is the group minimum (exact in fp16) and the minimum maps to code 0
    assert np.array_equal(z16.astype(np.float64), mn)
    assert np.all(codes[np.arange(len(x)), x64.argmin(axis=1)] == 0)
    # the maximum maps to the top level whenever the scale is nonzero
    nz = s16 != 0
    assert np.all(codes[np.arange(len(x)), x64.argmax(axis=1)][nz] == L)
    # reconstruction error within half a step (plus the fp16 rounding of the scale)
    s = s16.astype(np.float64)
    s32 = (mx - mn) / L
    xh = z16.astype(np.float64)[:, None] + s[:, None] * codes
    err = np.abs(xh - x64)
    bound = s / 2 * (1 + 1e-6) + L * np.abs(s32 - s) + 1e-12
    assert np.all(err <= bound[:, None])


def test_constant_group_exact():
    for val in [0.0, 7.25, -65504.0, 3.0e-6]:
        x = np.full((32, 128), val, dtype=np.float16)
        kc, ks, kz = quantize_key_group(x, 2)
        vc, vs, vz = quantize_value_group(x, 2)
        kh, vh = dequantize_block(kc, ks, kz, vc, vs, vz)
        assert np.array_equal(kh, x.astype(np.float64))
        assert np.array_equal(vh, x.astype(np.float64))


def test_key_error_confined_to_channel():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((32, 128)).astype(np.float16)
    kc, ks, kz = quantize_key_group(k, 2)
    k2 = k.copy()
    k2[7, 40] = np.float16(50.0)   # an outlier in one channel of one token
    kc2, ks2, kz2 = quantize_key_group(k2, 2)
    changed = np.any(kc != kc2, axis=0) | (ks != ks2) | (kz != kz2)
    assert changed[40] and changed.sum() == 1


def test_value_error_confined_to_token():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((32, 128)).astype(np.float16)
    vc, vs, vz = quantize_value_group(v, 2)
    v2 = v.copy()
    v2[9, 70] = np.float16(-40.0)
    vc2, vs2, vz2 = quantize_value_group(v2, 2)
    changed_tokens = np.any(vc != vc2, axis=1) | np.any(vs != vs2, axis=1) | np.any(vz != vz2, axis=1)
    assert changed_tokens[9] and changed_tokens.sum() == 1
    # and within that token, only the 32-channel group holding channel 70
    assert np.array_equal(vs[9] != vs2[9], np.array([False, False, True, False]))


def test_axes_key_per_channel_value_per_token():
    # Keys: channel d of token t holds d + t/4, so every channel spans 7.75 over the
    # group and has minimum d: one scale and one zero per channel.
    t = np.arange(32, dtype=np.float64)[:, None] / 4
    d = np.arange(128, dtype=np.float64)[None, :]
    k = (d + t).astype(np.float16)
    kc, ks, kz = quantize_key_group(k, 2)
    assert ks.shape == (128,) and np.all(ks == np.float16(np.float32(7.75) / np.float32(3)))
    assert np.array_equal(kz, np.arange(128).astype(np.float16))
    assert np.array_equal(kc[:, 0], kc[:, 77])
    # Values: token t holds t + d/32 over its channels: each token has its own
    # zero-point, each 32-channel group its own minimum.
    v = (t * 4 + d / 32).astype(np.float16)
    vc, vs, vz = quantize_value_group(v, 2)
    assert vs.shape == (32, 4)
    assert np.array_equal(vz, (np.arange(32)[:, None] + np.arange(4)[None, :]).astype(np.float16))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_unpack_roundtrip(bits):
    rng = np.random.default_rng(7 + bits)
    L = 2 ** bits - 1
    kc = rng.integers(0, L + 1, size=(32, 128)).astype(np.uint8)
    vc = rng.integers(0, L + 1, size=(32, 128)).astype(np.uint8)
    ks = rng.standard_normal(128).astype(np.float16)
    kz = rng.standard_normal(128).astype(np.float16)
    vs = rng.standard_normal((32, 4)).astype(np.float16)
    vz = rng.standard_normal((32, 4)).astype(np.float16)
    blk = pack_group_block(kc, ks, kz, vc, vs, vz, bits)
    assert blk.size == group_block_bytes(bits) == {2: 3072, 3: 4096, 4: 5120}[bits]
    out = unpack_group_block(blk, bits)
    for a, b in zip(out, (kc, ks, kz, vc, vs, vz)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("section", ["key", "value"])
def test_code_positions_are_a_bijection(bits, section):
    ii, dd = np.meshgrid(np.arange(32), np.arange(128), indexing="ij")
    fn = _key_code_coords if section == "key" else _value_code_coords
    word, bit = _code_position(*fn(ii, dd), bits)
    flat_bit = word * 8 + bit
    assert np.all(bit % bits == 0)
    assert len(np.unique(flat_bit)) == 32 * 128
    assert flat_bit.min() == 0 and flat_bit.max() == 32 * 128 * bits - bits


def test_3bit_fields_are_a_bijection():
    for fn in (_key_code_coords, _value_code_coords):
        ii, dd = np.meshgrid(np.arange(32), np.arange(128), indexing="ij")
        lo, hi = _code_fields(*fn(ii, dd), 3)
        lo_bits = (lo[0] * 8 + lo[1]).ravel()
        hi_bits = (hi[0] * 8 + hi[1]).ravel()
        assert lo[2] == 2 and hi[2] == 1 and lo[3] == 0 and hi[3] == 2
        assert np.all(lo[1] % 2 == 0)
        # the low fields tile bits [0, 8192) two at a time, the high fields [8192, 12288) one at a time
        assert len(np.unique(lo_bits)) == 4096 and lo_bits.min() == 0 and lo_bits.max() == 8190
        assert len(np.unique(hi_bits)) == 4096 and hi_bits.min() == 8192 and hi_bits.max() == 12287


@pytest.mark.parametrize("entry", _load("block_layout.json")["code_positions_3bit"],
                         ids=lambda e: f'3{e["section"][0]}-{e["token"]}-{e["channel"]}')
def test_single_3bit_code_lands_at_hand_derived_positions(entry):
    kc = np.zeros((32, 128), dtype=np.uint8)
    vc = np.zeros((32, 128), dtype=np.uint8)
    target = kc if entry["section"] == "key" else vc
    target[entry["token"], entry["channel"]] = 7   # all three bits set
    z = np.zeros(128, dtype=np.float16)
    zv = np.zeros((32, 4), dtype=np.float16)
    blk = pack_group_block(kc, z, z, vc, zv, zv, 3)
    sec = blk[:1536] if entry["section"] == "key" else blk[1536:3072]
    words = sec.view("<u4")
    nz = np.nonzero(words)[0].tolist()
    assert nz == [entry["lo_word_byte"] // 4, entry["hi_word_byte"] // 4]
    assert int(words[nz[0]]) == 3 << entry["lo_bit"]
    assert int(words[nz[1]]) == 1 << entry["hi_bit"]


@pytest.mark.parametrize("entry", _load("block_layout.json")["code_positions"],
                         ids=lambda e: f'{e["bits"]}{e["section"][0]}-{e["token"]}-{e["channel"]}')
def test_single_code_lands_at_hand_derived_position(entry):
    bits = entry["bits"]
    kc = np.zeros((32, 128), dtype=np.uint8)
    vc = np.zeros((32, 128), dtype=np.uint8)
    target = kc if entry["section"] == "key" else vc
    target[entry["token"], entry["channel"]] = 1
    z = np.zeros(128, dtype=np.float16)
    zv = np.zeros((32, 4), dtype=np.float16)
    blk = pack_group_block(kc, z, z, vc, zv, zv, bits)
    cb = 32 * 128 * bits // 8
    sec = blk[:cb] if entry["section"] == "key" else blk[cb:2 * cb]
    words = sec.view("<u4")
    nz = np.nonzero(words)[0]
    assert nz.tolist() == [entry["word_byte"] // 4]
    assert int(words[nz[0]]) == 1 << entry["bit"]


@pytest.mark.parametrize("entry", _load("block_layout.json")["value_scale_index"])
def test_value_scale_lands_at_hand_derived_index(entry):
    assert _value_scale_index(entry["token"], entry["group"]) == entry["index"]
    vs = np.zeros((32, 4), dtype=np.float16)
    vs[entry["token"], entry["group"]] = np.float16(1.5)
    z = np.zeros(128, dtype=np.float16)
    c = np.zeros((32, 128), dtype=np.uint8)
    blk = pack_group_block(c, z, z, c, vs, np.zeros((32, 4), np.float16), 2)
    arr = blk[2048 + 512:2048 + 768].view("<f2")
    assert np.nonzero(arr)[0].tolist() == [entry["index"]]


def test_bits_per_element_matches_memory_ratio():
    # 2-bit codes + fp16 scale and zero-point per 32-element group = 3 bits per
    # element; against fp16 that is 16/3 = 5.33x, consistent with the 5.3x
    # memory reduction quoted in "The Asymmetric Key-Value Cache Compression
    # Framework", Summary (a loose check: the page does not name its setting).
    bits_per_elem = group_block_bytes(2) * 8 / (2 * 32 * 128)
    assert bits_per_elem == 3.0
    assert round(16 / bits_per_elem, 1) == 5.3
