"""GPU test of sd_draft_attn_noalloc (the attention for callers that cannot
allocate): through the C ABI, two calls in a row -- the second with a smaller
input, so the shared scratch array still holds the first call's larger work
list and partials -- each checked against sd_draft_attn on the same inputs
(bit for bit: the same kernels run) and against the oracle (max-abs 1e-2,
relative L2 1e-2)."""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import compare
from synth import StepInputs, device as sdev
from synth.configs import C1_32K

from gpu_common import DEV, bits, log, oracle_attention, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _cfg(**kw):
    base = dict(name="noalloc", batch=5, ctx=("list", (0, 1, 37, 1000, 20000)),
                draft_k=("list", (3, 1, 16, 5, 16)), verify="full", num_heads_q=32,
                num_heads_kv=8, head_dim=128, hidden=64, vocab=64, seed=7070)
    base.update(kw)
    return C1_32K.with_(**base)


def _both(inp, split_tokens=0):
    t = sdev.attention_tensors(inp, DEV)
    b = inp.budgets
    kw = dict(max_draft_k=int(b.draft_k.max()), max_total_ctx=inp.max_total_ctx,
              split_tokens=split_tokens)
    args = (t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["page_table"],
            t["ctx_len"], t["q_off"])
    ref = sd.sd_draft_attn(*args, **kw)
    out = torch.full_like(t["q"], float("nan"))
    sd.sd_draft_attn_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    return bits(out), bits(ref)


def test_noalloc_two_calls_second_smaller():
    first = StepInputs(_cfg())
    log("noalloc call 1: 5 requests up to 20,000 tokens, split 2048")
    got, ref = _both(first, split_tokens=2048)
    assert np.array_equal(got, ref)
    rep = compare.attention_report(got, oracle_attention(first))
    log(f"noalloc call 1 vs oracle {rep}")
    assert rep["ok"] and rep["rel_l2"] < 1e-2

    second = StepInputs(_cfg(batch=2, ctx=("list", (5, 300)), draft_k=("list", (16, 2)),
                             num_heads_q=64, seed=7071))
    log("noalloc call 2: 2 requests up to 300 tokens, GQA group 8 (128-row items)")
    got, ref = _both(second, split_tokens=64)
    assert np.array_equal(got, ref)
    rep = compare.attention_report(got, oracle_attention(second))
    log(f"noalloc call 2 vs oracle {rep}")
    assert rep["ok"] and rep["rel_l2"] < 1e-2
