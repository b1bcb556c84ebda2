"""The step run end to end on the oracle, with its near-tie audit.

Test infrastructure (see ``oracle/__init__``): never imported by the product.

Order of the step ("LongSpark", sec. 2.1 and App. A.1, Fig. 6): draft-block
attention, LM head + softmax + sampling of the K_b draft tokens, then
verification against the target's K_b + 1 rows.  The drafter's own layers
between attention and the LM head need trained weights and are not part of the
step, so the LM head consumes given draft states.

Audit (decisions excused from exact parity): an acceptance test whose
``|u - min(1, p/q)|`` is below ``NEAR_TIE`` and a Gumbel-max draw whose
top-2 key gap is below ``NEAR_TIE``.
"""
from __future__ import annotations

import numpy as np

from . import attention, lm_head, verify

NEAR_TIE = 1e-5


def run_lm_head(hidden, w_vocab, q_off, req_id, seed, rows=None, greedy=False, vocab_map=None):
    """Logits, lse, draft tokens and Gumbel gaps for all rows (or ``rows``)."""
    req, pos = lm_head.row_owner(q_off)
    z = lm_head.lm_head_logits(hidden, w_vocab, rows=rows, vocab_map=vocab_map)
    sel = np.arange(len(req)) if rows is None else np.asarray(rows)
    lse = lm_head.logsumexp_rows(z)
    tok, gap = lm_head.draft_tokens(z, req[sel], pos[sel], req_id, seed, greedy=greedy,
                                    vocab_map=vocab_map)
    return dict(rows=sel, logits=z, lse=lse, tokens=tok, gap=gap)


def run_verify(target_logits, t_off, draft_logits, draft_tokens, q_off,
               req_id, seed, requests=None, greedy=False, draft_vocab_inv=None):
    return verify.verify(target_logits, t_off, draft_logits, draft_tokens,
                         q_off, req_id, seed, requests=requests, greedy=greedy,
                         draft_vocab_inv=draft_vocab_inv)


def run_attention(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len,
                  q_off, num_heads_kv, scale, requests=None):
    return attention.draft_attn(q, k_blk, v_blk, k_cache, v_cache, page_table,
                                ctx_len, q_off, num_heads_kv, scale,
                                requests=requests)
