"""Pins for the oracle's streaming rule and its decode attention.

Residual window: the most recent tokens stay FP16 ("The Asymmetric Key-Value
Cache Compression Framework", In practice); quantized groups are appended along
the token dimension and combined with the FP16 residual inside attention
("KV cache quantization: putting the bits in the cached vectors", full-text-skim
notes on KIVI's grouped/residual split).
"""
import math

import numpy as np
import pytest
import torch

from oracle import OracleCache, OracleHead, attention_fp64, quantized_count
from oracle.bruteforce import dense_decode, simulate_quantized_count


@pytest.mark.parametrize("R", [0, 32, 64, 128])
def test_quantized_count_closed_form_vs_simulation(R):
    for T in list(range(0, 400)) + [1000, 4097, 10000]:
        assert quantized_count(T, R, 32) == simulate_quantized_count(T, R, 32)


def test_window_size_bounds():
    for R in (32, 64, 128):
        for T in range(R, 2000):
            w = T - quantized_count(T, R)
            assert R <= w <= R + 31


def test_flush_steps_of_32k_context_r128():
    # 32768 prefill tokens, R = 128, then 64 single-token steps: groups move to the
    # quantized store when T reaches 32800 and 32832.
    flushes = [32768 + s for s in range(1, 65)
               if quantized_count(32768 + s, 128) != quantized_count(32768 + s - 1, 128)]
    assert flushes == [32800, 32832]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("R", [0, 32, 64])
@pytest.mark.parametrize("rotate", [False, True])
def test_oracle_matches_bruteforce(bits, R, rotate):
    rng = np.random.default_rng(100 + bits + R + rotate)
    T = 150
    k = (rng.standard_normal((T, 128)) * np.where(np.arange(128) % 37 == 0, 10, 1)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((3, 128)).astype(np.float16)
    head = OracleHead(bits, R, rotate)
    # append in uneven chunks to exercise flushes across calls
    for a, b in [(0, 1), (1, 40), (40, 41), (41, 100), (100, 150)]:
        head.append(k[a:b], v[a:b])
    assert head.T == T and head.Q == simulate_quantized_count(T, R, 32)
    got = head.attend(q)
    ref = dense_decode(head.prepare_query(q), head.k16, head.v16, head)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_residual_covers_everything_equals_fp16_attention():
    rng = np.random.default_rng(7)
    T = 96
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    head = OracleHead(2, 128)
    head.append(k, v)
    assert head.Q == 0
    got = head.attend(q)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None],
        torch.from_numpy(k.astype(np.float64))[None],
        torch.from_numpy(v.astype(np.float64))[None])[0].numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_rotation_preserves_attention_when_unquantized():
    rng = np.random.default_rng(8)
    T = 80
    k = (rng.standard_normal((T, 128)) * 3).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    a = OracleHead(2, 128, rotate=False)
    b = OracleHead(2, 128, rotate=True)
    a.append(k, v)
    b.append(k, v)
    # only difference: the fp16 rounding of the rotated keys
    assert np.allclose(a.attend(q), b.attend(q), atol=2e-3)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 128))
    k = rng.standard_normal((300, 128)) * 5
    ones = np.ones((300, 128))
    assert np.allclose(attention_fp64(q, k, ones, 1 / math.sqrt(128)), 1.0, atol=1e-14)


def test_gqa_head_mapping():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, n = 2, 8, 2, 70
    k = rng.standard_normal((B, n, Hkv, 128)).astype(np.float16)
    v = rng.standard_normal((B, n, Hkv, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    c = OracleCache(B, Hq, Hkv, 2, 32)
    c.append(k, v)
    out = c.decode(q)
    for b in range(B):
        for hq in range(Hq):
            h = hq // (Hq // Hkv)
            ref = c.heads[b][h].attend(q[b, hq:hq + 1])
            other = c.heads[b][1 - h].attend(q[b, hq:hq + 1])
            assert np.allclose(out[b, hq], ref[0], rtol=0, atol=1e-13)
            assert not np.allclose(out[b, hq], other[0], rtol=0, atol=1e-3)


def test_ragged_append_counts():
    rng = np.random.default_rng(12)
    c = OracleCache(3, 4, 2, 2, 32)
    k = rng.standard_normal((3, 50, 2, 128)).astype(np.float16)
    v = rng.standard_normal((3, 50, 2, 128)).astype(np.float16)
    c.append(k, v, n_tokens=[50, 0, 33])
    assert [c.seq_len(b) for b in range(3)] == [(50, 0), (0, 0), (33, 0)]
    c.append(k, v, n_tokens=[50, 31, 40])
    assert [c.seq_len(b) for b in range(3)] == [(100, 64), (31, 0), (73, 32)]


def test_empty_sequence_rejected():
    with pytest.raises(ValueError):
        OracleHead(2, 32).attend(np.zeros((1, 128), np.float16))


# ---- attention sink: token 0 stays FP16, groups start at token 1 ("KV cache
# quantization: putting the bits in the cached vectors", full-text-skim notes on
# keeping the first token in fp16) ----

@pytest.mark.parametrize("R", [0, 32, 128])
def test_sink_count_closed_form_vs_simulation(R):
    for T in list(range(0, 300)) + [1000, 4097]:
        assert quantized_count(T, R, 32, sink=True) == simulate_quantized_count(T, R, 32, sink=True)


def test_sink_window_bounds_and_first_flush():
    for R in (0, 32, 128):
        for T in range(R + 1, 1500):
            fp16 = T - quantized_count(T, R, 32, sink=True)      # window plus the sink
            assert R + 1 <= fp16 <= R + 32
        # the first group (tokens 1..32) leaves the window when T = 1 + R + 32
        assert quantized_count(R + 32, R, 32, sink=True) == 0
        assert quantized_count(R + 33, R, 32, sink=True) == 32


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("R", [0, 32])
@pytest.mark.parametrize("rotate", [False, True])
def test_sink_oracle_matches_bruteforce(bits, R, rotate):
    rng = np.random.default_rng(300 + bits + R + rotate)
    T = 140
    k = rng.standard_normal((T, 128)).astype(np.float16)
    k[0] *= np.float16(40.0)                       # a strong first token
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((2, 128)).astype(np.float16)
    head = OracleHead(bits, R, rotate, sink=True)
    for a, b in [(0, 1), (1, 2), (2, 70), (70, 140)]:
        head.append(k[a:b], v[a:b])
    assert head.Q == simulate_quantized_count(T, R, 32, sink=True)
    got = head.attend(q)
    ref = dense_decode(head.prepare_query(q), head.k16, head.v16, head)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_sink_group_zero_is_tokens_1_to_32():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((100, 128)).astype(np.float16)
    v = rng.standard_normal((100, 128)).astype(np.float16)
    a = OracleHead(2, 32, sink=True)
    a.append(k, v)
    b = OracleHead(2, 32)            # no sink, fed tokens 1..99 only
    b.append(k[1:], v[1:])
    assert a.Q == b.Q == 64
    for g in range(2):
        assert np.array_equal(a.block(g), b.block(g))


def test_sink_small_context_is_plain_fp16_attention():
    rng = np.random.default_rng(9)
    T = 33                             # R + 1 tokens: nothing quantized yet
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((3, 128)).astype(np.float16)
    head = OracleHead(2, 32, sink=True)
    head.append(k, v)
    assert head.Q == 0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None],
        torch.from_numpy(k.astype(np.float64))[None],
        torch.from_numpy(v.astype(np.float64))[None])[0].numpy()
    assert np.allclose(head.attend(q), ref, rtol=0, atol=1e-12)


def test_sink_keeps_an_outlier_first_token_out_of_group_zero():
    # token 0 far outside the range of the others: without a sink it shares group 0
    # with tokens 1..31, whose per-channel range (and so their error) it blows up;
    # with a sink it stays exact and group 0 holds ordinary tokens.
    rng = np.random.default_rng(10)
    T = 200
    k = rng.standard_normal((T, 128)).astype(np.float16)
    k[0] = np.float16(300.0)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    with_sink = OracleHead(2, 32, sink=True)
    without = OracleHead(2, 32)
    for h in (with_sink, without):
        h.append(k, v)
    ks, _ = with_sink.cache_values()
    kn, _ = without.cache_values()
    exact = k.astype(np.float64)
    assert np.array_equal(ks[-1], exact[0])                   # the sink comes last
    assert np.abs(kn[1:32] - exact[1:32]).max() > 3.0          # group 0 without a sink
    assert np.abs(ks[0:31] - exact[1:32]).max() < 1.5          # group 0 with a sink = tokens 1..32
