"""One draft-and-verify step with preallocated outputs and workspaces.

Runs the three C-ABI calls back to back on one stream: draft-block attention,
LM head + draft sampling, verification ("LongSpark", sec. 2.1 and App. A.1,
Fig. 6).  The drafter layers between attention and the LM head need trained
weights and are outside the step, so the LM head consumes given draft states.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import (draft_attn_workspace_size, lm_head_workspace_size, sd_draft_attn,
               sd_lm_head_probs, sd_verify, verify_workspace_size)


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


class DraftVerifyStep:
    def __init__(self, shape: StepShape, device):
        s = shape
        self.shape = s
        dev = torch.device(device)
        self.device = dev
        self.attn_out = torch.empty(s.total_q, s.num_heads_q, s.head_dim, dtype=torch.bfloat16,
                                    device=dev)
        self.logits = torch.empty(s.total_q, s.vocab, dtype=torch.float32, device=dev)
        self.lse = torch.empty(s.total_q, dtype=torch.float32, device=dev)
        self.tokens = torch.empty(s.total_q, dtype=torch.int32, device=dev)
        self.accepted = torch.empty(s.batch, dtype=torch.int32, device=dev)
        self.next_token = torch.empty(s.batch, dtype=torch.int32, device=dev)
        self.ratio = torch.empty(s.total_q, dtype=torch.float32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(256, draft_attn_workspace_size(
            s.batch, s.num_heads_q, s.num_heads_kv, s.head_dim, s.max_total_ctx,
            s.split_tokens)), **u8)
        self.ws_lm = torch.empty(max(256, lm_head_workspace_size(s.total_q, s.vocab)), **u8)
        self.ws_verify = torch.empty(max(256, verify_workspace_size(
            s.batch, s.total_q, s.total_target_rows, s.vocab)), **u8)

    def attention(self, t: Dict[str, torch.Tensor], stream=None):
        s = self.shape
        return sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"],
                             t["page_table"], t["ctx_len"], t["q_off"],
                             max_draft_k=s.max_draft_k, max_total_ctx=s.max_total_ctx,
                             split_tokens=s.split_tokens, out=self.attn_out,
                             workspace=self.ws_attn, stream=stream)

    def lm_head(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        return sd_lm_head_probs(t["hidden"], t["w_vocab"], t["q_off"], t["req_id"], seed,
                                logits=self.logits, lse=self.lse, draft_tokens=self.tokens,
                                workspace=self.ws_lm, stream=stream)

    def verify(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        return sd_verify(t["target_logits"], t["t_off"], self.logits, self.lse, self.tokens,
                         t["q_off"], t["req_id"], seed, accepted_len=self.accepted,
                         next_token=self.next_token, accept_ratio=self.ratio,
                         workspace=self.ws_verify, stream=stream)

    def run(self, t: Dict[str, torch.Tensor], seed: int, stream=None):
        self.attention(t, stream)
        self.lm_head(t, seed, stream)
        self.verify(t, seed, stream)
        return dict(attn_out=self.attn_out, logits=self.logits, lse=self.lse,
                    tokens=self.tokens, accepted=self.accepted, next_token=self.next_token,
                    ratio=self.ratio)
