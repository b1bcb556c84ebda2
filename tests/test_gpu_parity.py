"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Attention outputs within 1e-2 max-abs; probabilities within 1e-5; draft
tokens, accepted lengths and next tokens exact except audited near-ties
(|u - r| < 1e-5 or a Gumbel top-2 key gap < 1e-5).
"""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import compare, lm_head as olm, step as ostep, verify as overify
from oracle.attention import bf16_bits_to_f64 as oa_bits_to_f64
from synth import StepInputs, device as sdev
from synth.configs import C0_TINY, C1_32K, C3_VERIFY, C4_RAGGED, small

from gpu_common import (DEV, bits, gpu_attention, gpu_lm_head, log, oracle_attention,
                        request_rows, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


# ------------------------------------------------------------------ attention

def _edge_cfg(**kw):
    base = dict(name="attn_edge", batch=5, ctx=("list", (0, 1, 37, 160, 1000)),
                draft_k=("list", (3, 1, 16, 5, 8)), verify="full", num_heads_q=8,
                num_heads_kv=2, head_dim=128, hidden=64, vocab=64, seed=4242)
    base.update(kw)
    return C1_32K.with_(**base)


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("split", [0, 64, 192])
def test_attention_edge_shapes(head_dim, split):
    inp = StepInputs(_edge_cfg(head_dim=head_dim))
    log(f"attention edge D={head_dim} split={split}")
    rep = compare.attention_report(gpu_attention(inp, split_tokens=split), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 1e-2


@pytest.mark.parametrize("hq,hkv,kmax", [(40, 8, 16), (64, 8, 16), (40, 8, 15), (12, 1, 8),
                                          (128, 8, 8)])
@pytest.mark.parametrize("split", [0, 64])
def test_attention_large_groups(hq, hkv, kmax, split):
    """More than 64 query rows per (request, KV head) -- GQA groups of 5 or 8
    at K = 16, group 5 at ForeSpark's K = 15, group 12 at K = 8, group 16 at
    K = 8: work items of 128 rows (four waves over one KV stream)."""
    kb = tuple(min(kmax, k) for k in (kmax, 1, kmax - 1, 5, kmax, 3))
    inp = StepInputs(_edge_cfg(batch=6, ctx=("list", (0, 1, 37, 160, 1000, 2049)),
                               draft_k=("list", kb), num_heads_q=hq, num_heads_kv=hkv,
                               head_dim=128 if hq % 8 == 0 else 64, seed=hq * 100 + kmax))
    log(f"attention large groups Hq={hq} Hkv={hkv} K<={kmax} split={split}")
    rep = compare.attention_report(gpu_attention(inp, split_tokens=split), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 1e-2


def test_attention_many_requests():
    """1,100 ragged requests: the work list is built over two 1,024-request
    rounds, and with 64-token splits the block units, full-length splits and
    shorter last splits all occur (empty prefixes and K_b = 0 included)."""
    B = 1100
    ctx = tuple((0, 17, 64, 100, 300, 1)[i % 6] for i in range(B))
    kb = tuple((1, 2, 4, 0, 3)[i % 5] for i in range(B))
    inp = StepInputs(_edge_cfg(batch=B, ctx=("list", ctx), draft_k=("list", kb), num_heads_q=4,
                               num_heads_kv=1, head_dim=64, seed=1100))
    log("attention many requests B=1100 split=64")
    rep = compare.attention_report(gpu_attention(inp, split_tokens=64), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 1e-2


@pytest.mark.parametrize("batch,split", [(7, 0), (64, 64), (65, 64), (64, 0)])
def test_attention_launch_shapes(batch, split):
    """The call's launch shapes at their boundaries: every request within one
    split (7 or 64 requests, automatic split: one item per request and KV
    head, no work list, no merge), 64 requests with several splits each (the
    split-K workgroups scan the requests themselves) and 65 (the work-list
    kernel).  Ragged prefixes with empty ones and K_b = 0 rows."""
    ctx = tuple((0, 17, 300, 64, 1, 250, 128)[i % 7] for i in range(batch))
    kb = tuple((4, 1, 0, 16, 3)[i % 5] for i in range(batch))
    inp = StepInputs(_edge_cfg(batch=batch, ctx=("list", ctx), draft_k=("list", kb),
                               num_heads_q=8, num_heads_kv=2, head_dim=64,
                               seed=9000 + batch + split))
    log(f"attention launch shape B={batch} split={split}")
    rep = compare.attention_report(gpu_attention(inp, split_tokens=split), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 1e-2


def test_attention_tiny_workload():
    inp = StepInputs(C0_TINY)
    rep = compare.attention_report(gpu_attention(inp), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 1e-2


def test_attention_peaked_queries():
    inp = StepInputs(_edge_cfg(q_scale=8.0, seed=99))
    rep = compare.attention_report(gpu_attention(inp), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 2e-2


def test_attention_mha_and_small_groups():
    inp = StepInputs(_edge_cfg(num_heads_q=4, num_heads_kv=4, head_dim=64))
    rep = compare.attention_report(gpu_attention(inp), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"]


# -------------------------------------------------------------------- LM head

@pytest.mark.parametrize("M,H,V", [(16, 256, 1024), (5, 64, 1000), (130, 128, 1001),
                                   (257, 512, 4096), (256, 64, 768), (600, 128, 1001),
                                   (1024, 64, 5000),
                                   (16, 64, 70001), (256, 64, 65600),
                                   (16, 256, 70001), (600, 128, 65600),
                                   # 320 x 256 tiles (at least 256 of them):
                                   # ragged vocab and row tails
                                   (600, 64, 40003), (257, 128, 82001),
                                   (8, 64, 151936), (1024, 64, 20481),
                                   # 320 x 64 tiles (at most 64 rows, at least 256 tiles):
                                   # full and ragged row and vocab tails
                                   (64, 128, 90001), (33, 256, 81921),
                                   # 320 x 128 tiles (65 to 128 rows, at least 256 tiles)
                                   (128, 128, 90001), (100, 64, 81921),
                                   # 128 x 128 tiles at 65 to 128 rows of a smaller vocabulary
                                   (128, 128, 32000), (100, 64, 20001)])
def test_lm_head_shapes(M, H, V):
    cfg = C0_TINY.with_(name="lm", batch=1, draft_k=M, hidden=H, vocab=V, seed=M * 7 + V)
    inp = StepInputs(cfg)
    z, lse, tok = gpu_lm_head(inp)
    ref = ostep.run_lm_head(inp.hidden, inp.w_vocab, inp.budgets.q_off, inp.req_id,
                            inp.philox_seed)
    rep = compare.lm_head_report(z, lse, tok, ref)
    log(f"lm_head M={M} H={H} V={V} {rep}")
    assert rep["ok"]
    assert rep["logit_max_abs"] < 1e-5


def test_lm_head_qwen_vocab_sampled_rows():
    cfg = small(C1_32K, batch=3, ctx=16)
    inp = StepInputs(cfg)
    z, lse, tok = gpu_lm_head(inp)
    rows = np.array([0, 1, 15, 16, 31, 47])
    ref = ostep.run_lm_head(inp.hidden, inp.w_vocab, inp.budgets.q_off, inp.req_id,
                            inp.philox_seed, rows=rows)
    rep = compare.lm_head_report(z, lse, tok, ref)
    log(f"lm_head qwen vocab {rep}")
    assert rep["ok"]


# --------------------------------------------------------------------- verify

def _verify_gpu(inp, draft_logits, draft_tokens, draft_lse=None):
    t = sdev.verify_tensors(inp, DEV)
    dl = torch.from_numpy(draft_logits).to(DEV)
    dt = torch.from_numpy(draft_tokens.astype(np.int32)).to(DEV)
    lse = None if draft_lse is None else torch.from_numpy(draft_lse.astype(np.float32)).to(DEV)
    acc, nxt, ratio = sd.sd_verify(t["target_logits"], t["t_off"], dl, lse, dt, t["q_off"],
                                   t["req_id"], inp.philox_seed)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), ratio.cpu().numpy()


@pytest.mark.parametrize("verify_mode", ["full", "uniform", "zero"])
@pytest.mark.parametrize("V", [1000, 8193, 20000])
def test_verify_only_random_drafts(verify_mode, V):
    cfg = C0_TINY.with_(name="verify", batch=24, ctx=16, draft_k=(1, 4, 16), verify=verify_mode,
                        vocab=V, seed=V + len(verify_mode), target=("normal", 1.0))
    inp = StepInputs(cfg)
    b = inp.budgets
    dl = inp.random_draft_logits(sigma=1.0)
    dt = inp.random_draft_tokens()
    acc, nxt, ratio = _verify_gpu(inp, dl, dt)
    ref = overify.verify(inp.target_logits, b.t_off, dl, dt, b.q_off, inp.req_id,
                         inp.philox_seed)
    rep = compare.verify_report(acc, nxt, ref, range(cfg.batch))
    rr = compare.ratio_report(ratio, ref, b.q_off, range(cfg.batch))
    log(f"verify {verify_mode} V={V} {rep} ratio {rr}")
    assert rep["ok"] and rr["max_abs"] < 1e-5


@pytest.mark.parametrize("batch", [32, 64])
def test_verify_drafts_from_q_accept_often(batch):
    # target = draft logits + small noise: long accepted runs, bonus tokens
    cfg = C0_TINY.with_(name="verify_close", batch=batch, ctx=16, draft_k=8, verify="full",
                        vocab=3000, seed=5, target=("normal", 1.0))
    inp = StepInputs(cfg)
    b = inp.budgets
    dl = inp.random_draft_logits(sigma=1.0)
    rq, pos = olm.row_owner(b.q_off)
    dt, _ = olm.draft_tokens(dl.astype(np.float64), rq, pos, inp.req_id, inp.philox_seed)
    rng = np.random.default_rng(0)
    src = np.concatenate([np.r_[np.arange(b.q_off[i], b.q_off[i + 1]), b.q_off[i + 1] - 1]
                          for i in range(cfg.batch)])
    tgt = (dl[src] + rng.standard_normal((len(src), cfg.vocab)) * 0.1).astype(np.float32)
    inp.__dict__["target_logits"] = tgt
    acc, nxt, ratio = _verify_gpu(inp, dl, dt)
    ref = overify.verify(tgt, b.t_off, dl, dt, b.q_off, inp.req_id, inp.philox_seed)
    rep = compare.verify_report(acc, nxt, ref, range(cfg.batch))
    log(f"verify close {rep}")
    assert rep["ok"] and rep["mean_accepted"] > 4


@pytest.mark.parametrize("batch", [47, 48, 130])
def test_verify_either_side_of_the_decision_kernel(batch):
    # below 48 requests every sampling workgroup takes its request's decision;
    # from 48 on a separate kernel decides once per request
    cfg = C0_TINY.with_(name="verify_batches", batch=batch, ctx=16, draft_k=(0, 1, 5, 16),
                        verify="full", vocab=9000, seed=batch, target=("normal", 1.0))
    inp = StepInputs(cfg)
    b = inp.budgets
    dl = inp.random_draft_logits(sigma=1.0)
    dt = inp.random_draft_tokens()
    acc, nxt, ratio = _verify_gpu(inp, dl, dt)
    ref = overify.verify(inp.target_logits, b.t_off, dl, dt, b.q_off, inp.req_id,
                         inp.philox_seed)
    rep = compare.verify_report(acc, nxt, ref, range(cfg.batch))
    rr = compare.ratio_report(ratio, ref, b.q_off, range(cfg.batch))
    log(f"verify batch={batch} {rep} ratio {rr}")
    assert rep["ok"] and rr["max_abs"] < 1e-5


@pytest.mark.parametrize("batch", [6, 50])
def test_verify_long_drafts(batch):
    """Verify budgets past 256 positions, so the decision takes several
    passes (below and above the batch from which it has its own kernel).
    Even requests have a target equal to the drafter's logits (every draft is
    accepted and the bonus comes from row b_b + 1 > 256); odd ones add a
    little noise (long runs that end in a rejection somewhere)."""
    kbs = tuple((300, 256, 257, 600, 1, 513)[i % 6] for i in range(batch))
    cfg = C0_TINY.with_(name="verify_long", batch=batch, ctx=16, draft_k=("list", kbs),
                        verify="full", vocab=512, seed=31 + batch, target=("normal", 1.0))
    inp = StepInputs(cfg)
    b = inp.budgets
    dl = inp.random_draft_logits(sigma=1.0)
    rq, pos = olm.row_owner(b.q_off)
    dt, _ = olm.draft_tokens(dl.astype(np.float64), rq, pos, inp.req_id, inp.philox_seed)
    src = np.concatenate([np.r_[np.arange(b.q_off[i], b.q_off[i + 1]), b.q_off[i + 1] - 1]
                          for i in range(cfg.batch)])
    row_req = np.repeat(np.arange(cfg.batch), np.diff(b.t_off))
    noise = np.where(row_req % 2 == 0, 0.0, 0.004)[:, None]
    rng = np.random.default_rng(7)
    tgt = (dl[src].astype(np.float64) + rng.standard_normal((len(src), cfg.vocab)) * noise)
    tgt = tgt.astype(np.float32)
    inp.__dict__["target_logits"] = tgt
    log(f"verify long drafts batch={batch}")
    acc, nxt, ratio = _verify_gpu(inp, dl, dt)
    ref = overify.verify(tgt, b.t_off, dl, dt, b.q_off, inp.req_id, inp.philox_seed)
    rep = compare.verify_report(acc, nxt, ref, range(cfg.batch))
    rr = compare.ratio_report(ratio, ref, b.q_off, range(cfg.batch))
    log(f"verify long batch={batch} {rep} ratio {rr} accepted {ref['accepted'].tolist()}")
    assert rep["ok"] and rr["max_abs"] < 1e-5
    assert ref["accepted"].max() > 256


def test_attention_understated_total_context():
    """Prefix lengths that add up to more than max_total_ctx, so that their
    work items do not fit the partials sized from it (4 x 1,000 tokens
    against a bound of 1,000): nothing is computed and every output row
    comes back NaN, never stale.  The same buffers with the right bound then
    give the exact result."""
    inp = StepInputs(_edge_cfg(batch=4, ctx=("list", (1000, 1000, 1000, 1000)),
                               draft_k=("list", (4, 4, 4, 4)), seed=404))
    t = sdev.attention_tensors(inp, DEV)
    out = torch.full_like(t["q"], 7.0)
    ws = torch.empty(sd.draft_attn_workspace_size(4, 8, 2, 128, 4, 4000, 64), dtype=torch.uint8,
                     device=DEV)
    log("attention understated max_total_ctx")
    sd.sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["page_table"],
                     t["ctx_len"], t["q_off"], max_draft_k=4, max_total_ctx=1000, split_tokens=64,
                     out=out, workspace=ws)
    torch.cuda.synchronize()
    got = oa_bits_to_f64(bits(out))
    assert np.isnan(got).all()
    log("attention with the right bound on the same buffers")
    sd.sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["page_table"],
                     t["ctx_len"], t["q_off"], max_draft_k=4, max_total_ctx=4000, split_tokens=64,
                     out=out, workspace=ws)
    torch.cuda.synchronize()
    rep = compare.attention_report(bits(out), oracle_attention(inp))
    log(str(rep))
    assert rep["ok"] and rep["rel_l2"] < 1e-2


# ---------------------------------------------------------------- whole step

def test_step_tiny_end_to_end():
    from __graft_entry__ import smoke
    smoke()
