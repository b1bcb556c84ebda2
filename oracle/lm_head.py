"""Drafter LM head, draft softmax statistics and draft sampling (fp64).

Test infrastructure (see ``oracle/__init__``): never imported by the product.

* Base logits of every draft slot come from the frozen target vocabulary
  head applied to the final draft states: ``z = h W^T`` with ``W`` the
  target's ``[V, H]`` head ("LongSpark", sec. 2.3 and App. A.1, Fig. 6; the
  target normalisation is applied by the caller before this step).
* The proposal of slot j is ``q_j = softmax(z_j)`` and the slots are sampled
  independently, so the block proposal factorises as the product of the
  ``q_j`` ("LongSpark", sec. 2.1, eq. (4); "DeLS-Spec": one forward pass
  followed by one sampling step).
* Sampling: the pages only say "sample".  Each token is drawn here as the
  Gumbel-max ``argmax_v (z_v - log(-log u_v))`` with one Philox uniform per
  vocab entry (stream 0, position j = row - q_off[b] + 1); the smallest index
  wins a tie.  Gumbel-max yields an exact sample of ``softmax(z)``.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64
from .philox import STREAM_DRAFT, gumbel_uniforms


def lm_head_logits(hidden: np.ndarray, w_vocab: np.ndarray,
                   rows=None, v_chunk: int = 8192, vocab_map=None) -> np.ndarray:
    """``z = hidden @ W^T`` in float64 from bf16 bit patterns.  With a pruned
    drafter vocabulary (``vocab_map``: target id of each drafter entry) W is
    those rows of the target's head, in map order ("H-Spec", App. B.2).  The
    vocab is processed in chunks only to bound memory; each entry is one dot
    product."""
    h = bf16_bits_to_f64(hidden if rows is None else hidden[rows])
    ids = np.arange(w_vocab.shape[0]) if vocab_map is None else np.asarray(vocab_map, np.int64)
    V = len(ids)
    z = np.empty((h.shape[0], V))
    for lo in range(0, V, v_chunk):
        z[:, lo:lo + v_chunk] = h @ bf16_bits_to_f64(w_vocab[ids[lo:lo + v_chunk]]).T
    return z


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """``log sum_v exp(z_v)`` per row, with max subtraction."""
    mx = z.max(axis=1, keepdims=True)
    return (mx + np.log(np.exp(z - mx).sum(axis=1, keepdims=True)))[:, 0]


def softmax_rows(z: np.ndarray) -> np.ndarray:
    return np.exp(z - logsumexp_rows(z)[:, None])


def gumbel_argmax(log_w: np.ndarray, u: np.ndarray):
    """``argmax_v (log_w_v - log(-log u_v))`` over entries with finite
    ``log_w``; the smallest index wins ties.  Returns (index, gap) where gap
    is the distance between the best and second-best keys (inf if only one
    candidate)."""
    key = np.full(log_w.shape, -np.inf)
    ok = np.isfinite(log_w)
    key[ok] = log_w[ok] - np.log(-np.log(u[ok]))
    idx = int(np.argmax(key))               # first maximum = smallest index
    if ok.sum() < 2:
        return idx, np.inf
    top2 = np.partition(key, -2)[-2:]
    return idx, float(top2[1] - top2[0])


def argmax_with_gap(x: np.ndarray):
    """First index of the maximum, and the gap between the two largest
    entries (inf for a single entry)."""
    idx = int(np.argmax(x))
    if len(x) < 2:
        return idx, np.inf
    top2 = np.partition(x, -2)[-2:]
    return idx, float(top2[1] - top2[0])


def draft_tokens(z: np.ndarray, row_req: np.ndarray, row_pos: np.ndarray,
                 req_id: np.ndarray, seed: int, greedy: bool = False, vocab_map=None):
    """Gumbel-max sample of ``softmax(z_r)`` for each row ``r`` (the argmax
    of ``z_r`` at temperature 0, ``greedy``).  ``row_req`` gives the request
    of each row and ``row_pos`` its 1-based position.  With a pruned
    vocabulary the drawn entry is reported as its target id."""
    M, V = z.shape
    tok = np.empty(M, np.int32)
    gap = np.empty(M)
    for r in range(M):
        if greedy:
            tok[r], gap[r] = argmax_with_gap(z[r])
        else:
            u = gumbel_uniforms(seed, int(req_id[row_req[r]]), int(row_pos[r]),
                                STREAM_DRAFT, V)
            tok[r], gap[r] = gumbel_argmax(z[r], u)
    if vocab_map is not None:
        tok = np.asarray(vocab_map, np.int32)[tok]
    return tok, gap


def row_owner(q_off: np.ndarray):
    """(request, 1-based position) of every packed draft row."""
    q_off = np.asarray(q_off, np.int64)
    B = len(q_off) - 1
    req = np.repeat(np.arange(B), np.diff(q_off))
    pos = np.arange(int(q_off[-1])) - q_off[req] + 1
    return req, pos
