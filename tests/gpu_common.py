"""Helpers for the GPU parity tests (not collected by pytest)."""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import compare, step as ostep, verify as overify
from synth import StepInputs, device as sdev

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_attention(inp: StepInputs, split_tokens=0, max_draft_k=None):
    t = sdev.attention_tensors(inp, DEV)
    b = inp.budgets
    mdk = int(b.draft_k.max()) if max_draft_k is None else max_draft_k
    out = sd.sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"],
                           t["page_table"], t["ctx_len"], t["q_off"], max_draft_k=mdk,
                           max_total_ctx=inp.max_total_ctx, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return bits(out)


def oracle_attention(inp: StepInputs, requests=None):
    b = inp.budgets
    return ostep.run_attention(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache,
                               inp.page_table, b.ctx_len, b.q_off, inp.cfg.num_heads_kv,
                               inp.softmax_scale, requests=requests)


def gpu_lm_head(inp: StepInputs):
    t = sdev.lm_head_tensors(inp, DEV)
    z, lse, tok = sd.sd_lm_head_probs(t["hidden"], t["w_vocab"], t["q_off"], t["req_id"],
                                      inp.philox_seed)
    torch.cuda.synchronize()
    return z.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy()


def request_rows(q_off, requests):
    return np.concatenate([np.arange(q_off[b], q_off[b + 1]) for b in requests]).astype(np.int64)
