"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one DraftVerifyStep, automatic split-K sizing).

The oracle cannot redo a whole 128K-context step in test time, so each test
checks (a) sampled outputs the oracle computes one by one -- every output row
of a few whole requests (all KV heads, so every split-K merge of those
requests), a spread of LM-head rows, and the full verification of those
requests from the oracle's own fp64 drafter logits -- and (b) properties that
hold for every output at any size: attention outputs are convex combinations
of value rows, softmax rows of the LM head are normalised, accepted lengths lie
in [0, b_b] and tokens in [0, V).

Tolerances are those of the parity suite: attention max-abs <= 1e-2 (and
relative L2 < 1e-2), probabilities <= 1e-5, tokens and lengths exact except
audited near-ties (margin < 1e-5).
"""
import numpy as np
import pytest
import torch

from block_drafting_sd_amd.step import DraftVerifyStep, StepShape
from oracle import compare, lm_head as olm, step as ostep, verify as overify
from synth import StepInputs, device as sdev
from synth.configs import C1_32K, C2_128K, C3_VERIFY, C4_RAGGED

from gpu_common import DEV, bits, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _run_step(inp: StepInputs, target=None):
    c, b = inp.cfg, inp.budgets
    t = {}
    t.update(sdev.attention_tensors(inp, DEV))
    t.update(sdev.lm_head_tensors(inp, DEV))
    tgt = inp.target_logits if target is None else target
    t.update(dict(target_logits=sdev.f32(tgt, DEV), t_off=sdev.i32(b.t_off, DEV)))
    shape = StepShape(batch=c.batch, total_q=inp.total_q, total_target_rows=inp.total_target_rows,
                      num_heads_q=c.num_heads_q, num_heads_kv=c.num_heads_kv, head_dim=c.head_dim,
                      hidden=c.hidden, vocab=c.vocab, max_total_ctx=inp.max_total_ctx,
                      max_draft_k=int(b.draft_k.max()))
    step = DraftVerifyStep(shape, DEV)
    out = step.run(t, inp.philox_seed)
    torch.cuda.synchronize()
    return t, out


def _attention_properties(inp, t, out):
    """Every output is a convex combination of its KV head's value rows:
    per (row, head, dim) it lies within [min, max] of those values, here
    bounded by the global value range (bf16 rounding allowed)."""
    o = out["attn_out"].float()
    assert torch.isfinite(o).all()
    vmax = max(t["v_cache"].float().abs().max().item(), t["v_blk"].float().abs().max().item())
    assert o.abs().max().item() <= vmax * (1 + 2 ** -7)


def _lm_properties(out, V):
    z, lse, tok = out["logits"], out["lse"], out["tokens"]
    assert torch.isfinite(z).all() and torch.isfinite(lse).all()
    q_sum = torch.exp(z - lse[:, None]).sum(1)
    assert (q_sum - 1).abs().max().item() <= 1e-4
    assert (lse >= z.max(1).values).all()
    assert ((tok >= 0) & (tok < V)).all()


def _verify_properties(inp, out):
    b = inp.budgets
    acc = out["accepted"].cpu().numpy()
    nxt = out["next_token"].cpu().numpy()
    assert np.all(acc >= 0) and np.all(acc <= b.verify_b)
    assert np.all((nxt >= 0) & (nxt < inp.cfg.vocab))


def _check_requests(inp, t, out, reqs, target=None, lm_rows_extra=()):
    """Oracle comparison of whole requests: attention rows, LM-head rows,
    draft tokens and the verification outcome."""
    c, b = inp.cfg, inp.budgets
    rows = np.concatenate([np.arange(b.q_off[r], b.q_off[r + 1]) for r in reqs]).astype(np.int64)
    # attention: all rows of the sampled requests (every KV head)
    ref_attn = ostep.run_attention(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache,
                                   inp.page_table, b.ctx_len, b.q_off, c.num_heads_kv,
                                   inp.softmax_scale, requests=reqs)
    ra = compare.attention_report(bits(out["attn_out"]), ref_attn, rows=rows)
    log(f"attention requests {list(reqs)} (N={[int(b.ctx_len[r]) for r in reqs]}): {ra}")
    assert ra["ok"] and ra["rel_l2"] < 1e-2
    # LM head: the sampled requests' rows plus a spread of others
    lm_rows = np.unique(np.concatenate([rows, np.asarray(lm_rows_extra, np.int64)]))
    ref_lm = ostep.run_lm_head(inp.hidden, inp.w_vocab, b.q_off, inp.req_id, inp.philox_seed,
                               rows=lm_rows)
    rl = compare.lm_head_report(out["logits"].cpu().numpy(), out["lse"].cpu().numpy(),
                                out["tokens"].cpu().numpy(), ref_lm)
    log(f"lm head rows {len(lm_rows)}: {rl}")
    assert rl["ok"]
    # verification end to end from the oracle's own drafter logits and tokens
    z_full = np.zeros((inp.total_q, c.vocab))
    tok_full = np.zeros(inp.total_q, np.int32)
    pos = {int(m): i for i, m in enumerate(lm_rows)}
    for m in rows:
        z_full[m] = ref_lm["logits"][pos[int(m)]]
        tok_full[m] = ref_lm["tokens"][pos[int(m)]]
    tgt = inp.target_logits if target is None else target
    ref_v = overify.verify(tgt, b.t_off, z_full, tok_full, b.q_off, inp.req_id, inp.philox_seed,
                           requests=reqs)
    excused = np.zeros(c.batch, bool)
    for r in reqs:
        sl = [pos[int(m)] for m in range(int(b.q_off[r]), int(b.q_off[r + 1]))]
        excused[r] = bool(np.any(ref_lm["gap"][sl] < ostep.NEAR_TIE))
    rv = compare.verify_report(out["accepted"].cpu().numpy(), out["next_token"].cpu().numpy(),
                               ref_v, reqs, excused)
    log(f"verify requests {list(reqs)}: {rv}")
    assert rv["ok"]


@pytest.mark.parametrize("cfg", [C1_32K, C2_128K], ids=["32k_b16", "128k_b16"])
def test_fullsize_uniform_context(cfg):
    log(f"full-size workload {cfg.name}")
    inp = StepInputs(cfg)
    t, out = _run_step(inp)
    _attention_properties(inp, t, out)
    _lm_properties(out, cfg.vocab)
    _verify_properties(inp, out)
    extra = [1, 100 % inp.total_q, inp.total_q // 2, inp.total_q - 2]
    _check_requests(inp, t, out, [0, cfg.batch - 1], lm_rows_extra=extra)


def test_fullsize_verify_heavy():
    cfg = C3_VERIFY
    log(f"full-size workload {cfg.name}")
    inp = StepInputs(cfg)
    # target = the oracle's fp64 drafter logits of every row + seeded noise
    drafter = olm.lm_head_logits(inp.hidden, inp.w_vocab)
    target = inp.target_from_drafter(drafter)
    t, out = _run_step(inp, target=target)
    _attention_properties(inp, t, out)
    _lm_properties(out, cfg.vocab)
    _verify_properties(inp, out)
    acc = out["accepted"].cpu().numpy()
    log(f"mean accepted {acc.mean():.2f} of {int(inp.budgets.verify_b[0])}")
    reqs = [int(np.argmin(inp.target_sigma)), int(np.argmax(inp.target_sigma)), 17]
    _check_requests(inp, t, out, reqs, target=target, lm_rows_extra=[5, 500, inp.total_q - 1])


def test_fullsize_ragged_mix():
    cfg = C4_RAGGED
    log(f"full-size workload {cfg.name}")
    inp = StepInputs(cfg)
    b = inp.budgets
    t, out = _run_step(inp)
    _attention_properties(inp, t, out)
    _lm_properties(out, cfg.vocab)
    _verify_properties(inp, out)
    # shortest and longest prefix, each draft budget, a partial verify budget
    n = b.ctx_len
    reqs = {int(np.argmin(n)), int(np.argmax(n))}
    for k in (4, 8, 16):
        reqs.add(int(np.flatnonzero(b.draft_k == k)[0]))
    part = np.flatnonzero(b.verify_b < b.draft_k)
    if part.size:
        reqs.add(int(part[0]))
    _check_requests(inp, t, out, sorted(reqs), lm_rows_extra=[0, inp.total_q - 1])
