"""The step's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, synchronises nothing and records no memset:
with preallocated outputs and workspaces every call is a sequence of kernel
launches on the caller's stream, so a serving loop can capture a whole
draft-and-verify step once and replay it.  Each replay here follows eager work
on the same buffers (the step run eagerly with another seed, which overwrites
every output) and a synchronisation, and must reproduce the eager outputs of
the captured seed bit for bit.  The fixed-cost path also folds the accepted
rows into its summary state in place, so that state is reset from a saved
copy before every eager run and every replay, and the folded state is
compared too.
"""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from synth import StepInputs, device as sdev
from synth.configs import C1_32K

from gpu_common import DEV, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _setup(path):
    from block_drafting_sd_amd.step import DraftVerifyStep, StepOptions, StepShape

    cfg = C1_32K.with_(name=f"graph_{path}", batch=4, ctx=("list", (700, 37, 0, 1500)),
                       draft_k=("list", (16, 5, 3, 9)), verify="full", num_heads_q=8,
                       num_heads_kv=2, head_dim=64, hidden=256, vocab=4100, seed=4040)
    inp = StepInputs(cfg)
    b = inp.budgets
    opts = {
        "full": StepOptions(),
        "hspec_greedy": StepOptions(causal_block=True, window=512, draft_vocab=1000, greedy=True),
        "fusion": StepOptions(markov_rank=64, markov_alpha=0.3, prior_beta=0.3),
        "fixed": StepOptions(window=256, n_summary=16),
    }[path]
    t = {}
    t.update(sdev.attention_tensors(inp, DEV))
    t.update(sdev.lm_head_tensors(inp, DEV))
    t.update(sdev.verify_tensors(inp, DEV))
    if opts.draft_vocab:
        vmap = inp.pruned_vocab(opts.draft_vocab)
        vinv = np.full(cfg.vocab, -1, np.int32)
        vinv[vmap] = np.arange(opts.draft_vocab, dtype=np.int32)
        t["vocab_map"] = sdev.i32(vmap, DEV)
        t["vocab_inv"] = sdev.i32(vinv, DEV)
    if opts.markov_rank:
        w_c, e_c = inp.markov_tables(opts.markov_rank)
        t.update(markov_w_c=sdev.bf16(w_c, DEV), markov_e_c=sdev.bf16(e_c, DEV),
                 anchor=sdev.i32(inp.anchor_tokens(), DEV))
    if opts.prior_beta:
        t["vocab_bias"] = sd.sd_log_prior_bias(torch.from_numpy(inp.unigram_counts()).to(DEV),
                                               lam=1.0, scale=-opts.prior_beta)
    if opts.n_summary:
        # the last K_max + 1 rows of each prefix stand in for the new rows
        t["summary_keys"] = sdev.bf16(inp.summary_queries(opts.n_summary), DEV)
        t["ctx_len_prev"] = sdev.i32(np.maximum(b.ctx_len - (int(b.draft_k.max()) + 1), 0), DEV)
    shape = StepShape(batch=cfg.batch, total_q=inp.total_q, total_target_rows=inp.total_target_rows,
                      num_heads_q=cfg.num_heads_q, num_heads_kv=cfg.num_heads_kv,
                      head_dim=cfg.head_dim, hidden=cfg.hidden, vocab=cfg.vocab,
                      max_total_ctx=inp.max_total_ctx, max_draft_k=int(b.draft_k.max()))
    step = DraftVerifyStep(shape, DEV, opts)
    if opts.n_summary:
        step.summary_init(t)
    return step, t, inp.philox_seed


def _snapshot(out):
    return {k: v.clone() for k, v in out.items()}


@pytest.mark.parametrize("path", ["full", "hspec_greedy", "fusion", "fixed"])
def test_step_graph_replays_match_eager(path):
    step, t, seed = _setup(path)
    stateful = step.options.n_summary > 0
    saved = (step.summary_values.clone(), step.summary_lse.clone()) if stateful else None

    def reset():
        if stateful:
            step.summary_values.copy_(saved[0])
            step.summary_lse.copy_(saved[1])

    def outputs(out):
        d = dict(out)
        if stateful:
            d.update(summary_values=step.summary_values, summary_lse=step.summary_lse)
        return d

    reset()
    ref = _snapshot(outputs(step.run(t, seed)))
    reset()
    other = _snapshot(outputs(step.run(t, seed + 1)))
    torch.cuda.synchronize()
    # the other seed must change what the replays have to restore
    assert not torch.equal(ref["logits"], other["logits"]) or not torch.equal(ref["tokens"],
                                                                                other["tokens"]) \
        or path == "hspec_greedy"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step.run(t, seed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = outputs(step.run(t, seed))
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        step.run(t, seed + 1 + rep)                 # eager work on the same buffers
        x = torch.randn(256, 256, device=DEV)
        (x @ x).sum().item()                        # unrelated eager work, then a sync
        torch.cuda.synchronize()
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            same = torch.equal(outs[k], v) if v.dtype != torch.float32 else \
                torch.equal(outs[k].view(torch.int32), v.view(torch.int32))
            log(f"graph {path} replay {rep}: {k} identical {same}")
            assert same, f"{path}: replay {rep} differs from the eager run in {k}"
