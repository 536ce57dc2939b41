"""Pins for the oracle's pre-RoPE option: keys are quantized before the rotary
position embedding and rotated after dequantization ("KVQuant" review, Method and
Key idea). The rotary embedding itself is not defined on the pages; the oracle
takes the standard one (channel pairs f, f + 64; theta_f = base^(-f/64)), pinned
here by hand-derived values and by the properties that define a rotary embedding.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import OracleHead, rope_fp64
from oracle.bruteforce import dense_decode, simulate_quantized_count

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_cases.json")


def test_rope_hand_derived_cases():
    g = json.load(open(GOLDEN))
    val = {"cos1": g["cos1"], "sin1": g["sin1"], "-sin1": -g["sin1"], "1": 1.0}
    assert math.isclose(g["cos1"], math.cos(1.0), rel_tol=0, abs_tol=1e-16)
    for case in g["cases"]:
        x = np.zeros((1, 128))
        x[0, case["unit_channel"]] = 1.0
        got = rope_fp64(x, [case["position"]], case["base"])[0]
        exp = np.zeros(128)
        for ch, name in case["expect"].items():
            exp[int(ch)] = val[name]
        assert np.allclose(got, exp, rtol=0, atol=1e-12), case


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((5, 128))
    assert np.array_equal(rope_fp64(x, [0] * 5), x)


def test_rope_is_orthogonal_pairwise_rotation():
    for t in (1, 77, 131071, 1048575):
        m = rope_fp64(np.eye(128), [t] * 128)        # row i: image of unit vector i
        assert np.allclose(m @ m.T, np.eye(128), rtol=0, atol=1e-12)
        # only the pairs (f, f + 64) mix
        mask = np.zeros((128, 128), dtype=bool)
        for f in range(64):
            mask[[f, f, f + 64, f + 64], [f, f + 64, f, f + 64]] = True
        assert np.all(m[~mask] == 0)


def test_rope_positions_compose():
    x = np.random.default_rng(2).standard_normal((4, 128))
    s, t = [3, 100, 4000, 9], [5, 27, 123, 0]
    a = rope_fp64(rope_fp64(x, s), t)
    b = rope_fp64(x, np.add(s, t))
    assert np.allclose(a, b, rtol=0, atol=1e-10)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    for m, n in [(0, 5), (100, 37), (5000, 5001)]:
        d1 = (rope_fp64(q, [m]) @ rope_fp64(k, [n]).T).item()
        d2 = (rope_fp64(q, [m + 11]) @ rope_fp64(k, [n + 11]).T).item()
        assert math.isclose(d1, d2, rel_tol=1e-9, abs_tol=1e-9)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("R", [0, 32])
@pytest.mark.parametrize("sink", [False, True])
def test_rope_oracle_matches_bruteforce(bits, R, sink):
    rng = np.random.default_rng(400 + bits + R + sink)
    T = 120
    k = (rng.standard_normal((T, 128)) * np.where(np.arange(128) % 29 == 0, 8, 1)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((2, 128)).astype(np.float16)
    head = OracleHead(bits, R, sink=sink, rope=True)
    for a, b in [(0, 1), (1, 50), (50, 51), (51, 120)]:
        head.append(k[a:b], v[a:b])
    assert head.Q == simulate_quantized_count(T, R, 32, sink)
    got = head.attend(q)
    ref = dense_decode(head.prepare_query(q), head.k16, head.v16, head)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_rope_unquantized_equals_textbook_attention_over_rotated_keys():
    # R >= T: every key is FP16; rotating each key by an explicit 2x2 rotation
    # matrix per channel pair and calling torch's attention must agree
    rng = np.random.default_rng(4)
    T = 30
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((3, 128)).astype(np.float16)
    head = OracleHead(2, 32, rope=True, rope_base=500.0)
    head.append(k, v)
    assert head.Q == 0
    kr = np.zeros((T, 128))
    for t in range(T):
        for f in range(64):
            th = t * 500.0 ** (-f / 64)
            rot = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
            kr[t, [f, f + 64]] = rot @ k[t, [f, f + 64]].astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None], torch.from_numpy(kr)[None],
        torch.from_numpy(v.astype(np.float64))[None])[0].numpy()
    assert np.allclose(head.attend(q), ref, rtol=0, atol=1e-12)


def test_rope_quantizes_the_keys_as_given():
    # pre-RoPE: the stored groups are those of the unrotated keys
    rng = np.random.default_rng(5)
    k = rng.standard_normal((200, 128)).astype(np.float16)
    v = rng.standard_normal((200, 128)).astype(np.float16)
    a, b = OracleHead(2, 64, rope=True), OracleHead(2, 64)
    a.append(k, v)
    b.append(k, v)
    assert a.Q == b.Q == 128
    for g in range(a.Q // 32):
        assert np.array_equal(a.block(g), b.block(g))


def test_rope_lowers_error_of_rotated_outlier_channels():
    # keys with a large fixed channel (pinned outlier): quantizing before the
    # rotation keeps the outlier in its channel, so on the outlier's channel pair
    # the dequantized-then-rotated keys are far closer to the exact rotated keys
    # than quantized rotated keys (whose per-channel range the rotation inflates)
    rng = np.random.default_rng(6)
    T = 4096
    k = rng.standard_normal((T, 128))
    k[:, 3] = 20.0 + rng.standard_normal(T)
    k = k.astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    exact = rope_fp64(k.astype(np.float64), np.arange(T))
    pre = OracleHead(2, 0, rope=True)
    pre.append(k, v)
    post = OracleHead(2, 0)
    post.append(exact.astype(np.float16), v)        # post-RoPE keys quantized
    pair = [3, 67]
    err_pre = np.abs(pre.cache_values()[0] - exact)[:, pair].mean()
    err_post = np.abs(post.cache_values()[0] - exact)[:, pair].mean()
    assert err_pre < 0.25 * err_post


def test_rope_and_hadamard_rotation_are_exclusive():
    with pytest.raises(ValueError):
        OracleHead(2, 32, rotate=True, rope=True)
