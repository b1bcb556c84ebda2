"""Sequential (Markov) correction of the draft distributions (fp64).

Test infrastructure (see ``oracle/__init__``): never imported by the product.

"LongSpark", sec. 2.3, eqs. (7)-(8): the base logits l_j^(0) of the K_b
positions (all computed in parallel by the LM head) are refined by a
low-rank term that depends on the token sampled at the previous position,
``l_j = l_j^(0) + W_c e_c(y_{j-1})``, j = 1..K_b, with y_0 the committed
token; ``q_j = softmax(l_j)`` is sampled in order (y_j depends on y_{j-1})
and the same q_j are used for verification.  Only the correction and the
sampling are sequential (Fig. 6).  ``e_c`` is a correction embedding table
[V, r] and ``W_c`` the output mapping [V, r] (rank r, 256 on the pages).

Sampling is the Gumbel-max draw of the factorised proposal (stream 0 of the
Philox uniforms at position j), so a zero correction reproduces it exactly.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64
from .lm_head import draft_tokens, logsumexp_rows


def correction(w_c, e_c, token: int):
    """``W_c e_c(token)``: the correction of every vocab entry [V]."""
    return bf16_bits_to_f64(w_c) @ bf16_bits_to_f64(e_c[token])


def markov_sample(base_logits, q_off, anchor, w_c, e_c, req_id, seed: int, requests=None):
    """Sequential correction and sampling of every request (or ``requests``).
    ``base_logits [M, V]`` are l^(0) of the packed draft rows.  Returns dict
    (logits [M, V] corrected, lse [M], tokens [M], gap [M]); rows of other
    requests stay NaN / -1."""
    M, V = base_logits.shape
    W = bf16_bits_to_f64(w_c)
    E = bf16_bits_to_f64(e_c)
    z = np.full((M, V), np.nan)
    lse = np.full(M, np.nan)
    tok = np.full(M, -1, np.int32)
    gap = np.full(M, np.nan)
    B = len(q_off) - 1
    for b in (range(B) if requests is None else requests):
        prev = int(anchor[b])
        for j, m in enumerate(range(int(q_off[b]), int(q_off[b + 1])), start=1):
            z[m] = np.asarray(base_logits[m], np.float64) + W @ E[prev]
            lse[m] = logsumexp_rows(z[m][None])[0]
            t, g = draft_tokens(z[m][None], np.array([b]), np.array([j]), req_id, seed)
            tok[m], gap[m] = t[0], g[0]
            prev = int(tok[m])
    return dict(logits=z, lse=lse, tokens=tok, gap=gap)
