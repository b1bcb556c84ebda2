"""Lossless speculative-sampling verification (fp64).

Test infrastructure (see ``oracle/__init__``): never imported by the product.

Per request, with target distributions ``p_1 .. p_{b+1}`` (softmax of the
target's logits at the anchor and the b verified drafts) and draft
distributions ``q_1 .. q_b``:

1. Drafts are tested in order; ``y_j`` is accepted with probability
   ``min(1, p_j(y_j) / q_j(y_j))`` ("LongSpark", sec. 2.1, eq. (1)).
2. The first rejection at position j ends the round; the correction token is
   drawn from ``[p_j - q_j]_+ / sum_u [p_j(u) - q_j(u)]_+`` ("LongSpark",
   sec. 2.1, eq. (2)).
3. If all b drafts are accepted, one more token is drawn from the target's
   next distribution ``p_{b+1}``; accepting a drafts therefore advances the
   prefix by a + 1 tokens ("LongSpark", sec. 2.1, text after eq. (2)).
4. A verify budget b smaller than the draft length d tests only the first b
   drafts; the rest are dropped unverified ("ForeSpark", sec. 4.4: the
   verified positions form a prefix of each draft and the target sees them as
   one packed batch).  b = 0 is a plain autoregressive step.

Readings where the pages are silent:
* the test is ``u < r`` with ``u`` the position's acceptance uniform in [0, 1);
* ``q_j(y_j) = 0`` gives r = 1 (such a draft has probability 0);
* if ``[p_j - q_j]_+`` sums to 0 (p_j and q_j equal) the correction is drawn
  from ``p_j``;
* draws use Gumbel-max with Philox uniforms of stream 2 at position j (or
  b + 1 for the bonus token), see ``oracle.philox``.

Variants:
* pruned drafter vocabulary ("H-Spec", App. B.2): the drafter's softmax is
  over a subset of the target vocabulary and q_j is zero outside it; the
  rules above are unchanged, so verification stays lossless.
* temperature 0 on both sides ("LongSpark", App. D.1; "H-Spec", sec. 4):
  p_j and q_j are one-hot at their argmax (smallest index on ties), so r_j is
  1 when y_j is the argmax of target row j and 0 otherwise, the residual
  [p_j - q_j]_+ is the one-hot of that argmax and the bonus is the argmax of
  row b + 1 -- the rules above applied to one-hot distributions.
"""
from __future__ import annotations

from typing import Callable, List, Sequence, Tuple

import numpy as np

from .lm_head import argmax_with_gap, gumbel_argmax, softmax_rows
from .philox import STREAM_SAMPLE, accept_uniform, gumbel_uniforms


def accept_probability(p_y, q_y):
    """``min(1, p(y) / q(y))``, and 1 when ``q(y) = 0``."""
    if q_y == 0:
        return 1
    r = p_y / q_y
    return r if r < 1 else 1


def residual_weights(p, q):
    """Unnormalised correction distribution ``[p - q]_+`` (elementwise)."""
    d = p - q
    return np.where(d > 0, d, 0 * d)


def verify_request(p_rows: Sequence, q_rows: Sequence, y: Sequence,
                   n_verify: int, accept_u: Callable[[int], float],
                   sample: Callable[[object, int], int]):
    """One request's verification.

    ``p_rows[j-1]`` / ``q_rows[j-1]`` are the target / draft distributions at
    position j, ``y[j-1]`` the draft token.  ``accept_u(j)`` returns the
    acceptance uniform of position j and ``sample(weights, j)`` draws an index
    with probability proportional to the non-negative ``weights``.
    Returns ``(accepted, next_token, tests)`` with ``tests`` a list of
    ``(j, u, r)`` for every acceptance test made."""
    tests: List[Tuple[int, float, float]] = []
    for j in range(1, n_verify + 1):
        p, q, t = p_rows[j - 1], q_rows[j - 1], int(y[j - 1])
        r = accept_probability(p[t], q[t])
        u = accept_u(j)
        tests.append((j, u, r))
        if u < r:
            continue
        res = residual_weights(p, q)
        if sum(res) > 0:
            return j - 1, sample(res, j), tests
        return j - 1, sample(p, j), tests
    return n_verify, sample(p_rows[n_verify], n_verify + 1), tests


def greedy_request(x_rows: Sequence, y: Sequence, n_verify: int):
    """Temperature-0 verification of one request from its target logit rows
    ``x_rows`` (b + 1 rows) and drafts ``y``.  Returns ``(accepted,
    next_token, gaps)`` with the top-2 logit gap of every row consulted."""
    gaps = []
    for j in range(1, n_verify + 1):
        a, g = argmax_with_gap(x_rows[j - 1])
        gaps.append(g)
        if int(y[j - 1]) != a:
            return j - 1, a, gaps
    a, g = argmax_with_gap(x_rows[n_verify])
    gaps.append(g)
    return n_verify, a, gaps


def draft_rows_full_vocab(draft_logits, draft_vocab_inv, V: int):
    """Draft distributions over the target vocabulary: softmax over the
    drafter's entries, zero for target tokens outside its vocabulary."""
    q_d = softmax_rows(np.asarray(draft_logits, np.float64))
    if draft_vocab_inv is None:
        return q_d
    inv = np.asarray(draft_vocab_inv, np.int64)
    q = np.zeros((q_d.shape[0], V))
    inside = inv >= 0
    q[:, inside] = q_d[:, inv[inside]]
    return q


def verify(target_logits: np.ndarray, t_off, draft_logits: np.ndarray,
           draft_tokens, q_off, req_id, seed: int, requests=None, greedy: bool = False,
           draft_vocab_inv=None):
    """Verification of every request (or of ``requests``).

    ``target_logits`` holds ``b_b + 1`` rows per request (rows ``t_off[b]``..),
    ``draft_logits`` and ``draft_tokens`` the packed draft rows (rows
    ``q_off[b]``..).  Returns a dict of arrays: ``accepted`` and ``next_token``
    (-1 for requests not processed), ``accept_margin`` (smallest |u - r| over
    the request's tests, inf if none), ``sample_gap`` (top-2 Gumbel key gap of
    the final draw) and ``tests`` (list per request)."""
    B = len(t_off) - 1
    V = target_logits.shape[1]
    acc = np.full(B, -1, np.int32)
    nxt = np.full(B, -1, np.int32)
    margin = np.full(B, np.inf)
    gap = np.full(B, np.nan)
    tests_all = [None] * B
    for b in (range(B) if requests is None else requests):
        t0, t1 = int(t_off[b]), int(t_off[b + 1])
        nv = t1 - t0 - 1
        q0 = int(q_off[b])
        y = np.asarray(draft_tokens[q0:q0 + nv])
        if greedy:
            a, c, gaps = greedy_request(target_logits[t0:t1].astype(np.float64), y, nv)
            acc[b], nxt[b] = a, c
            tests_all[b] = []
            tested = gaps if a < nv else gaps[:-1]   # rows whose argmax decided a test
            margin[b] = min(tested) if tested else np.inf
            gap[b] = gaps[-1]
            continue
        p_rows = softmax_rows(target_logits[t0:t1].astype(np.float64))
        if nv > 0:
            q_rows = draft_rows_full_vocab(draft_logits[q0:q0 + nv], draft_vocab_inv, V)
        else:
            q_rows = np.zeros((0, V))
        rid = int(req_id[b])
        last = {}

        def sample(w, j, rid=rid, last=last):
            with np.errstate(divide="ignore"):
                lw = np.log(np.asarray(w, np.float64))
            u = gumbel_uniforms(seed, rid, j, STREAM_SAMPLE, V)
            idx, g = gumbel_argmax(lw, u)
            last["gap"] = g
            return idx

        a, c, tests = verify_request(p_rows, q_rows, y, nv,
                                     lambda j, rid=rid: accept_uniform(seed, rid, j),
                                     sample)
        acc[b], nxt[b] = a, c
        tests_all[b] = tests
        if tests:
            margin[b] = min(abs(u - r) for _, u, r in tests)
        gap[b] = last["gap"]
    return dict(accepted=acc, next_token=nxt, accept_margin=margin,
                sample_gap=gap, tests=tests_all)
