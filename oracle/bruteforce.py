"""Brute-force float64 checker used to pin the oracle on tiny inputs.

TEST INFRASTRUCTURE ONLY. It re-derives, token by token with scalar Python
loops, which tokens are quantized (by simulating the residual window one token
at a time instead of using the closed form), dequantizes each quantized token
from its group's scale and zero-point, and evaluates softmax attention with
scipy's softmax. It is deliberately written differently from kvq_oracle so that
a slip in either one shows up as a disagreement.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import softmax


def simulate_quantized_count(T: int, R: int, G: int, sink: bool = False) -> int:
    """Quantized-token count after appending T tokens one at a time.

    Rule: the most recent R tokens must stay FP16 ("Pin the most recent tokens in
    FP16"), and tokens leave the window in whole groups of G aligned to token 0.
    After each append, while the oldest FP16 group lies entirely before the last
    R tokens, it is quantized.

    With an attention sink, token 0 never enters a group: the groups tile the
    tokens after it, so only the t - 1 tokens after the sink count as history.
    """
    q = 0
    for t in range(1, T + 1):
        history = t - 1 if sink else t
        while q + G <= history - R:
            q += G
    return q


def rotate_pairs_scalar(key, t, base):
    """Rotary embedding of one key row at position t, one channel pair at a time:
    channels f and f + D/2 turn by the angle t * base^(-2f / D)."""
    D = len(key)
    half = D // 2
    out = [0.0] * D
    for f in range(half):
        ang = t * math.pow(base, -2.0 * f / D)
        c, s = math.cos(ang), math.sin(ang)
        out[f] = key[f] * c - key[f + half] * s
        out[f + half] = key[f + half] * c + key[f] * s
    return out


def dense_decode(q_rows, k16, v16, head, scale=None):
    """Attention of q_rows [H, D] over a whole sequence held by `head`.

    `head` supplies per-group quantization results (its kc/ks/kz/vc/vs/vz
    arrays) and the FP16 history k16/v16 [T, D]; this function decides per token
    which representation attention uses and dequantizes scalar by scalar. With
    `head.rope`, every key (dequantized or FP16) is then rotated at its position.
    """
    T, D = k16.shape
    G = head.G
    sink = bool(getattr(head, "sink", False))
    Qn = simulate_quantized_count(T, head.R, G, sink)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    keys = np.zeros((T, D))
    vals = np.zeros((T, D))
    for t in range(T):
        pos = t - 1 if sink else t     # position among the tokens that can be grouped
        if 0 <= pos < Qn:
            g, i = divmod(pos, G)
            for d in range(D):
                keys[t, d] = float(head.kz[g][d]) + float(head.ks[g][d]) * int(head.kc[g][i, d])
                j = d // G
                vals[t, d] = float(head.vz[g][i, j]) + float(head.vs[g][i, j]) * int(head.vc[g][i, d])
        else:
            keys[t] = k16[t].astype(np.float64)
            vals[t] = v16[t].astype(np.float64)
        if getattr(head, "rope", False):
            keys[t] = rotate_pairs_scalar([float(x) for x in keys[t]], t, head.rope_base)
    out = np.zeros((q_rows.shape[0], D))
    for h in range(q_rows.shape[0]):
        scores = np.array([sum(float(q_rows[h, d]) * keys[t, d] for d in range(D)) * scale
                           for t in range(T)])
        p = softmax(scores)
        out[h] = p @ vals
    return out
