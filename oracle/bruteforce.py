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


def dense_decode(q_rows, k16, v16, head, scale=None):
    """Attention of q_rows [H, D] over a whole sequence held by `head`.

    `head` supplies per-group quantization results (its kc/ks/kz/vc/vs/vz
    arrays) and the FP16 history k16/v16 [T, D]; this function decides per token
    which representation attention uses and dequantizes scalar by scalar.
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
    out = np.zeros((q_rows.shape[0], D))
    for h in range(q_rows.shape[0]):
        scores = np.array([sum(float(q_rows[h, d]) * keys[t, d] for d in range(D)) * scale
                           for t in range(T)])
        p = softmax(scores)
        out[h] = p @ vals
    return out
