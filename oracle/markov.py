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

"DeLS-Spec" (inference fusion, and its appendix on the local head and the
unigram prior) fuses the same kind of term: the long (block-parallel) logits
plus alpha times the short-context logits minus beta times the log unigram
prior, alpha = beta = 0.3 by default (1 in the exact decomposition).  Its
Markov local head is the lookup-and-project term above (E_M, W_M [V, d_r]),
so the fused logits are ``l_j = l_j^(0) + alpha W_M e_M(y_{j-1}) + bias_v``
with ``bias = -beta log p~_0``, and LongSpark is alpha = 1, no bias.  The
prior is additively smoothed corpus counts, lambda = 1 by default:
``p~_0(v) = (c(v) + lambda) / (sum_u c(u) + lambda |V|)``.  (The page's
formulas are not printed; these are the readings of its text.)
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64
from .lm_head import draft_tokens, logsumexp_rows


def unigram_log_prior(counts, lam: float = 1.0):
    """``log p~_0(v)`` from corpus counts ``c(v)`` with additive smoothing."""
    c = np.asarray(counts, np.float64)
    with np.errstate(divide="ignore"):     # lambda = 0 and a zero count: -inf
        return np.log((c + lam) / (c.sum() + lam * len(c)))


def correction(w_c, e_c, token: int):
    """``W_c e_c(token)``: the correction of every vocab entry [V]."""
    return bf16_bits_to_f64(w_c) @ bf16_bits_to_f64(e_c[token])


def markov_sample(base_logits, q_off, anchor, w_c, e_c, req_id, seed: int, requests=None,
                  alpha: float = 1.0, vocab_bias=None, greedy: bool = False):
    """Sequential correction and sampling of every request (or ``requests``).
    ``base_logits [M, V]`` are l^(0) of the packed draft rows; ``alpha``
    scales the correction and ``vocab_bias [V]`` (optional) is added to every
    row; ``greedy`` draws the argmax of each corrected row (temperature 0,
    smallest index on ties).  Returns dict (logits [M, V] corrected, lse [M],
    tokens [M], gap [M]); rows of other requests stay NaN / -1."""
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
            z[m] = np.asarray(base_logits[m], np.float64) + alpha * (W @ E[prev])
            if vocab_bias is not None:
                z[m] = z[m] + np.asarray(vocab_bias, np.float64)
            lse[m] = logsumexp_rows(z[m][None])[0]
            t, g = draft_tokens(z[m][None], np.array([b]), np.array([j]), req_id, seed,
                                greedy=greedy)
            tok[m], gap[m] = t[0], g[0]
            prev = int(tok[m])
    return dict(logits=z, lse=lse, tokens=tok, gap=gap)
