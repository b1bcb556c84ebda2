"""One draft-and-verify step with preallocated outputs and workspaces.

Runs the C-ABI calls back to back on one stream: draft-block attention, LM
head + draft sampling, verification ("LongSpark", sec. 2.1 and App. A.1,
Fig. 6) and, on the fixed-cost context path, the fold of the retained rows
into the context summary ("LongSpark", sec. 2.2 and App. A.2).  With a
correction rank the draws of the LM head are replaced by the sequential
(Markov) correction and sampling ("LongSpark", sec. 2.3, eqs. (7)-(8)), whose
corrected distributions verification then uses.  The drafter
layers between attention and the LM head need trained weights and are outside
the step, so the LM head consumes given draft states.

``StepOptions`` selects the variants the calls take as parameters: causal
block mask, recent window, summary entries, pruned drafter vocabulary,
temperature 0, rank of the sequential correction.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import (SD_MASK_CAUSAL, SD_MASK_NONE, draft_attn_workspace_size,
               lm_head_workspace_size, markov_workspace_size, sd_draft_attn,
               sd_lm_head_probs, sd_markov_sample, sd_summary_update, sd_verify,
               summary_workspace_size, verify_workspace_size)


@dataclass
class StepShape:
    batch: int
    total_q: int
    total_target_rows: int
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    hidden: int
    vocab: int
    max_total_ctx: int
    max_draft_k: int
    split_tokens: int = 0


@dataclass
class StepOptions:
    causal_block: bool = False   # causal mask among the draft block's rows
    window: int = 0              # 0: whole prefix; W: the last W prefix tokens
    n_summary: int = 0           # context-summary entries per KV head (0: none)
    draft_vocab: int = 0         # 0: full vocabulary; else the pruned drafter's size
    greedy: bool = False         # temperature 0 on both sides
    markov_rank: int = 0         # 0: factorised drafts; r: sequential correction of rank r
    markov_alpha: float = 1.0    # scale of the correction (logit fusion: 0.3)
    prior_beta: float = 0.0      # fusion: subtract beta x log unigram prior (t["vocab_bias"])

    def __post_init__(self):
        if self.markov_rank and self.draft_vocab:
            raise ValueError("the sequential correction works on the full drafter vocabulary")


class DraftVerifyStep:
    """``t`` (the step's device inputs) holds the attention, LM-head and
    verification tensors; with summary entries also ``summary_keys``
    [Hkv, S, D] and ``ctx_len_prev`` (prefix lengths before the rows the fold
    appends); with a pruned vocabulary ``vocab_map`` [V_d] and ``vocab_inv``
    [V]; with a correction rank ``anchor`` [B] (the committed tokens) and the
    bf16 tables ``markov_w_c``, ``markov_e_c`` [V, r]; with a prior weight
    ``vocab_bias`` [V] (-beta log p~_0, from ``sd_log_prior_bias``)."""

    def __init__(self, shape: StepShape, device, options: Optional[StepOptions] = None):
        s = shape
        o = options or StepOptions()
        self.shape, self.options = s, o
        dev = torch.device(device)
        self.device = dev
        vd = o.draft_vocab or s.vocab
        self.attn_out = torch.empty(s.total_q, s.num_heads_q, s.head_dim, dtype=torch.bfloat16,
                                    device=dev)
        self.logits = torch.empty(s.total_q, vd, dtype=torch.float32, device=dev)
        self.lse = torch.empty(s.total_q, dtype=torch.float32, device=dev)
        self.tokens = torch.empty(s.total_q, dtype=torch.int32, device=dev)
        self.accepted = torch.empty(s.batch, dtype=torch.int32, device=dev)
        self.next_token = torch.empty(s.batch, dtype=torch.int32, device=dev)
        self.ratio = torch.empty(s.total_q, dtype=torch.float32, device=dev)
        self.ws_summary = None
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(256, draft_attn_workspace_size(
            s.batch, s.num_heads_q, s.num_heads_kv, s.head_dim, s.max_draft_k, s.max_total_ctx,
            s.split_tokens)), **u8)
        self.ws_lm = torch.empty(max(256, lm_head_workspace_size(s.total_q, vd)), **u8)
        if o.n_summary:
            self.summary_values = torch.zeros(s.batch, s.num_heads_kv, o.n_summary, s.head_dim,
                                              dtype=torch.float32, device=dev)
            self.summary_lse = torch.full((s.batch, s.num_heads_kv, o.n_summary), float("-inf"),
                                          dtype=torch.float32, device=dev)
        if o.markov_rank:
            self.ws_markov = torch.empty(max(256, markov_workspace_size(s.batch, vd, s.max_draft_k)), **u8)
        self.ws_verify = torch.empty(max(256, verify_workspace_size(
            s.batch, s.total_q, s.total_target_rows, s.vocab)), **u8)

    def summary_init(self, t: Dict[str, torch.Tensor], stream=None):
        """Summary of every request's prefix before the step's new rows (its
        workspace is allocated on the first call)."""
        if self.ws_summary is None:
            s = self.shape
            need = summary_workspace_size(s.batch, s.num_heads_kv, self.options.n_summary,
                                          s.head_dim, t["page_table"].shape[1])
            self.ws_summary = torch.empty(max(256, need), dtype=torch.uint8, device=self.device)
        return sd_summary_update(t["summary_keys"], t["k_cache"], t["v_cache"], t["page_table"],
                                 t["ctx_len_prev"], None, self.summary_values, self.summary_lse,
                                 workspace=self.ws_summary, stream=stream)

    def attention(self, t: Dict[str, torch.Tensor], stream=None):
        s, o = self.shape, self.options
        summ = dict(summary_keys=t["summary_keys"], summary_values=self.summary_values) \
            if o.n_summary else {}
        return sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"],
                             t["page_table"], t["ctx_len"], t["q_off"],
                             max_draft_k=s.max_draft_k, max_total_ctx=s.max_total_ctx,
                             split_tokens=s.split_tokens,
                             block_mask=SD_MASK_CAUSAL if o.causal_block else SD_MASK_NONE,
                             window=o.window, out=self.attn_out, workspace=self.ws_attn,
                             stream=stream, **summ)

    def lm_head(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        o = self.options
        return sd_lm_head_probs(t["hidden"], t["w_vocab"], t["q_off"], t["req_id"], seed,
                                vocab_map=t["vocab_map"] if o.draft_vocab else None,
                                greedy=o.greedy, logits=self.logits, lse=self.lse,
                                draft_tokens=self.tokens, workspace=self.ws_lm, stream=stream)

    def markov(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        """Correct the LM head's logits in place and redraw the tokens in
        order (the LM head's own draws are overwritten)."""
        o = self.options
        return sd_markov_sample(self.logits, t["anchor"], t["markov_w_c"], t["markov_e_c"],
                                t["q_off"], t["req_id"], seed,
                                max_draft_k=self.shape.max_draft_k, alpha=o.markov_alpha,
                                greedy=o.greedy,
                                vocab_bias=t["vocab_bias"] if o.prior_beta else None, lse=self.lse,
                                draft_tokens=self.tokens, workspace=self.ws_markov,
                                stream=stream)

    def verify(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        o = self.options
        return sd_verify(t["target_logits"], t["t_off"], self.logits, self.lse, self.tokens,
                         t["q_off"], t["req_id"], seed,
                         draft_vocab_inv=t["vocab_inv"] if o.draft_vocab else None,
                         greedy=o.greedy, accepted_len=self.accepted,
                         next_token=self.next_token, accept_ratio=self.ratio,
                         workspace=self.ws_verify, stream=stream)

    def summary_fold(self, t: Dict[str, torch.Tensor], stream=None):
        """Fold the committed token and the accepted drafts (rows
        ctx_len_prev .. ctx_len_prev + accepted) into the summary."""
        return sd_summary_update(t["summary_keys"], t["k_cache"], t["v_cache"], t["page_table"],
                                 t["ctx_len_prev"], self.accepted, self.summary_values,
                                 self.summary_lse, stream=stream)

    def run(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        self.attention(t, stream)
        self.lm_head(t, seed, stream)
        if self.options.markov_rank:
            self.markov(t, seed, stream)
        self.verify(t, seed, stream)
        if self.options.n_summary:
            self.summary_fold(t, stream)
        return dict(attn_out=self.attn_out, logits=self.logits, lse=self.lse,
                    tokens=self.tokens, accepted=self.accepted, next_token=self.next_token,
                    ratio=self.ratio)
