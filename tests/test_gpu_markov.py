"""GPU parity of the sequential (Markov) correction (sd_markov_sample).

Corrected logits and lse within 1e-5 of the oracle's fp64 values (a rank-r
bf16 product with fp32 accumulation added to fp32 logits), draws exact except
audited near-ties (Gumbel top-2 key gap < 1e-5); after a near-tie draw the
rest of that request follows another chain and is not compared.  With
W_c = 0 the draws must equal sd_lm_head_probs' own, exactly.  The
"DeLS-Spec" fusion (alpha, unigram-prior bias) is compared the same way,
with the device's bias as the oracle's input; the bias itself within 2e-6
of the fp64 prior (fp32 rounding of values up to ~6).
"""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import markov as omk
from oracle.step import NEAR_TIE
from synth import StepInputs, device as sdev
from synth.configs import C1_32K, C2_128K

from gpu_common import DEV, bits, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bf16(x):
    return (torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def _tables(V, r, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    return _bf16(rng.normal(0, scale, (V, r))), _bf16(rng.normal(0, scale, (V, r)))


def _run(base, q_off, anchor, w_c, e_c, req_id, seed, max_k):
    z = sdev.f32(base, DEV)
    _, lse, tok = sd.sd_markov_sample(z, sdev.i32(anchor, DEV), sdev.bf16(w_c, DEV),
                                      sdev.bf16(e_c, DEV), sdev.i32(q_off, DEV),
                                      sdev.i32(req_id.view(np.int32), DEV), seed,
                                      max_draft_k=max_k)
    torch.cuda.synchronize()
    return z.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy()


def _compare(got, ref, q_off, requests, tag):
    z, lse, tok = got
    worst_z = worst_l = 0.0
    compared = mism = 0
    for b in requests:
        for m in range(int(q_off[b]), int(q_off[b + 1])):
            worst_z = max(worst_z, float(np.abs(z[m] - ref["logits"][m]).max()))
            worst_l = max(worst_l, abs(float(lse[m]) - ref["lse"][m]))
            compared += 1
            if tok[m] != ref["tokens"][m]:
                assert ref["gap"][m] < NEAR_TIE, (tag, b, m, tok[m], ref["tokens"][m])
                mism += 1
                break      # the chains differ from here on
    log(f"{tag}: rows {compared}, logits max-abs {worst_z:.2e}, lse max-abs {worst_l:.2e}, "
        f"near-tie draws {mism}")
    assert worst_z <= 1e-5 and worst_l <= 1e-5


@pytest.mark.parametrize("V,r", [(1000, 32), (4096, 256)])
def test_markov_small(V, r):
    rng = np.random.default_rng(V + r)
    d = np.array([3, 16, 1, 0, 9])
    q_off = np.concatenate([[0], np.cumsum(d)]).astype(np.int32)
    base = rng.normal(0, 2.0, (int(q_off[-1]), V)).astype(np.float32)
    anchor = rng.integers(0, V, len(d)).astype(np.int32)
    req_id = rng.integers(0, 2**32, len(d), dtype=np.uint64).astype(np.uint32)
    w_c, e_c = _tables(V, r, V * r, scale=0.3)
    got = _run(base, q_off, anchor, w_c, e_c, req_id, 77, 16)
    ref = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 77)
    _compare(got, ref, q_off, range(len(d)), f"markov V={V} r={r}")


def test_markov_greedy():
    # temperature 0: each draw is the argmax of the corrected row
    V, r = 3001, 64
    rng = np.random.default_rng(55)
    d = np.array([16, 7, 1])
    q_off = np.concatenate([[0], np.cumsum(d)]).astype(np.int32)
    base = rng.normal(0, 2.0, (int(q_off[-1]), V)).astype(np.float32)
    anchor = rng.integers(0, V, len(d)).astype(np.int32)
    req_id = rng.integers(0, 2**32, len(d), dtype=np.uint64).astype(np.uint32)
    w_c, e_c = _tables(V, r, 8, scale=0.4)
    z = sdev.f32(base, DEV)
    _, lse, tok = sd.sd_markov_sample(z, sdev.i32(anchor, DEV), sdev.bf16(w_c, DEV),
                                      sdev.bf16(e_c, DEV), sdev.i32(q_off, DEV),
                                      sdev.i32(req_id.view(np.int32), DEV), 9, max_draft_k=16,
                                      greedy=True)
    torch.cuda.synchronize()
    got = (z.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy())
    ref = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 9, greedy=True)
    _compare(got, ref, q_off, range(len(d)), "markov greedy")


def test_zero_correction_reproduces_the_lm_head_draws():
    cfg = C1_32K.with_(batch=4, ctx=16, draft_k=(16, 5, 1, 9), hidden=256, vocab=5000, seed=3)
    inp = StepInputs(cfg)
    t = sdev.lm_head_tensors(inp, DEV)
    z, lse, tok = sd.sd_lm_head_probs(t["hidden"], t["w_vocab"], t["q_off"], t["req_id"],
                                      inp.philox_seed)
    zero = torch.zeros(cfg.vocab, 32, dtype=torch.bfloat16, device=DEV)
    anchor = torch.zeros(cfg.batch, dtype=torch.int32, device=DEV)
    z2 = z.clone()
    _, lse2, tok2 = sd.sd_markov_sample(z2, anchor, zero, zero, t["q_off"], t["req_id"],
                                        inp.philox_seed, max_draft_k=16)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2)
    assert torch.equal(z, z2)
    assert (lse - lse2).abs().max().item() <= 1e-6


def test_markov_full_size_128k_shapes():
    # 16 requests x K = 16 over the 151,936-token vocabulary, rank 256, the
    # base logits from the LM head; two whole requests against the oracle
    cfg = C2_128K.with_(ctx=16)
    inp = StepInputs(cfg)
    b = inp.budgets
    t = sdev.lm_head_tensors(inp, DEV)
    z, _, _ = sd.sd_lm_head_probs(t["hidden"], t["w_vocab"], t["q_off"], t["req_id"],
                                  inp.philox_seed)
    torch.cuda.synchronize()
    base = z.cpu().numpy()
    rng = np.random.default_rng(11)
    anchor = rng.integers(0, cfg.vocab, cfg.batch).astype(np.int32)
    w_c, e_c = _tables(cfg.vocab, 256, 12, scale=0.15)
    got = _run(base, b.q_off, anchor, w_c, e_c, inp.req_id, inp.philox_seed, 16)
    reqs = [0, cfg.batch - 1]
    ref = omk.markov_sample(base, b.q_off, anchor, w_c, e_c, inp.req_id, inp.philox_seed,
                            requests=reqs)
    _compare(got, ref, b.q_off, reqs, "markov 16 x 16 x 151936, r = 256")


def test_log_prior_bias_matches_the_smoothed_prior():
    # 151,936 Zipf-like counts with zeros; fp64 in the kernel, fp32 out
    rng = np.random.default_rng(21)
    V = 151936
    counts = (1e7 / np.arange(1, V + 1) ** 1.1).astype(np.int64)
    counts[rng.random(V) < 0.1] = 0
    counts = rng.permutation(counts)
    got = sd.sd_log_prior_bias(torch.from_numpy(counts).to(DEV), lam=1.0, scale=-0.3)
    torch.cuda.synchronize()
    ref = -0.3 * omk.unigram_log_prior(counts, 1.0)
    err = np.abs(got.cpu().numpy() - ref).max()
    log(f"log prior bias V={V}: max-abs {err:.2e} (values up to {np.abs(ref).max():.2f})")
    assert err <= 2e-6


@pytest.mark.parametrize("V,r", [(1001, 64), (4096, 256)])
def test_fusion_small(V, r):
    # "DeLS-Spec" fusion: alpha = 0.3, bias = -0.3 log p~_0 from the device
    rng = np.random.default_rng(V)
    d = np.array([16, 2, 7])
    q_off = np.concatenate([[0], np.cumsum(d)]).astype(np.int32)
    base = rng.normal(0, 2.0, (int(q_off[-1]), V)).astype(np.float32)
    anchor = rng.integers(0, V, len(d)).astype(np.int32)
    req_id = rng.integers(0, 2**32, len(d), dtype=np.uint64).astype(np.uint32)
    w_c, e_c = _tables(V, r, V + r, scale=0.4)
    counts = rng.integers(0, 1000, V).astype(np.int64)
    bias = sd.sd_log_prior_bias(torch.from_numpy(counts).to(DEV), lam=1.0, scale=-0.3)
    z = sdev.f32(base, DEV)
    _, lse, tok = sd.sd_markov_sample(z, sdev.i32(anchor, DEV), sdev.bf16(w_c, DEV),
                                      sdev.bf16(e_c, DEV), sdev.i32(q_off, DEV),
                                      sdev.i32(req_id.view(np.int32), DEV), 31, max_draft_k=16,
                                      alpha=0.3, vocab_bias=bias)
    torch.cuda.synchronize()
    got = (z.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy())
    ref = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 31, alpha=0.3,
                            vocab_bias=bias.cpu().numpy())        # staged: the device's bias
    _compare(got, ref, q_off, range(len(d)), f"fusion V={V} r={r}")


@pytest.mark.parametrize("batch,V,r,max_k", [
    (33, 2000, 320, 16),     # three request tiles; r > 256: the k-chunk loop
    (4, 7, 16, 16),          # tiny vocab (one partial chunk, scalar row ends); r = 16
    (5, 3001, 48, 6),        # positions beyond max_draft_k stay untouched
])
def test_markov_edges(batch, V, r, max_k):
    rng = np.random.default_rng(batch * 1000 + V + r)
    d = rng.integers(0, 17, batch)
    d[0] = 16
    q_off = np.concatenate([[0], np.cumsum(d)]).astype(np.int32)
    M = int(q_off[-1])
    base = rng.normal(0, 2.0, (M, V)).astype(np.float32)
    anchor = rng.integers(0, V, batch).astype(np.int32)
    req_id = rng.integers(0, 2**32, batch, dtype=np.uint64).astype(np.uint32)
    w_c, e_c = _tables(V, r, V * 7 + r, scale=0.3)
    z = sdev.f32(base, DEV)
    lse0 = torch.full((M,), -7.0, device=DEV)
    tok0 = torch.full((M,), -3, dtype=torch.int32, device=DEV)
    sd.sd_markov_sample(z, sdev.i32(anchor, DEV), sdev.bf16(w_c, DEV), sdev.bf16(e_c, DEV),
                        sdev.i32(q_off, DEV), sdev.i32(req_id.view(np.int32), DEV), 5,
                        max_draft_k=max_k, lse=lse0, draft_tokens=tok0)
    torch.cuda.synchronize()
    zg, lg, tg = z.cpu().numpy(), lse0.cpu().numpy(), tok0.cpu().numpy()
    # rows past max_draft_k: untouched
    pos = np.arange(M) - q_off[np.repeat(np.arange(batch), d)] + 1
    beyond = pos > max_k
    np.testing.assert_array_equal(zg[beyond], base[beyond])
    assert np.all(lg[beyond] == -7.0) and np.all(tg[beyond] == -3)
    # the oracle over the first max_k positions of every request
    dk = np.minimum(d, max_k)
    q_cut = np.concatenate([[0], np.cumsum(dk)]).astype(np.int32)
    keep = ~beyond
    ref = omk.markov_sample(base[keep], q_cut, anchor, w_c, e_c, req_id, 5)
    _compare((zg[keep], lg[keep], tg[keep]), ref, q_cut, range(batch),
             f"markov edges batch={batch} V={V} r={r} max_k={max_k}")


# ------------------------------------------------ the step with the correction

def _chain_cfg():
    return C1_32K.with_(name="markov_chain", batch=4, ctx=("list", (300, 37, 0, 600)),
                        draft_k=("list", (16, 5, 3, 9)), verify="full", num_heads_q=8,
                        num_heads_kv=2, head_dim=64, hidden=256, vocab=4100, seed=777)


@pytest.mark.parametrize("path", ["longspark", "dels", "longspark_greedy"])
def test_step_with_correction_chain(path):
    """Attention -> LM head -> sequential correction -> verification through
    DraftVerifyStep, each stage compared with the oracle on the previous
    stage's device outputs."""
    from block_drafting_sd_amd.step import DraftVerifyStep, StepOptions, StepShape
    from oracle import attention as oa, compare, lm_head as olm, verify as overify

    cfg = _chain_cfg()
    inp = StepInputs(cfg)
    b = inp.budgets
    r = 64
    if path.startswith("longspark"):
        opts = StepOptions(window=256, n_summary=16, markov_rank=r, greedy=path.endswith("greedy"))
    else:
        opts = StepOptions(markov_rank=r, markov_alpha=0.3, prior_beta=0.3)
    t = {}
    t.update(sdev.attention_tensors(inp, DEV))
    t.update(sdev.lm_head_tensors(inp, DEV))
    t.update(sdev.verify_tensors(inp, DEV))
    w_c, e_c = inp.markov_tables(r)
    anchor = inp.anchor_tokens()
    t.update(markov_w_c=sdev.bf16(w_c, DEV), markov_e_c=sdev.bf16(e_c, DEV),
             anchor=sdev.i32(anchor, DEV))
    bias = None
    if opts.prior_beta:
        counts = inp.unigram_counts()
        t["vocab_bias"] = sd.sd_log_prior_bias(torch.from_numpy(counts).to(DEV), lam=1.0,
                                               scale=-opts.prior_beta)
        bias = -opts.prior_beta * omk.unigram_log_prior(counts)
    if opts.n_summary:
        u = inp.summary_queries(opts.n_summary)
        t["summary_keys"] = sdev.bf16(u, DEV)
        t["ctx_len_prev"] = sdev.i32(np.maximum(b.ctx_len - 4, 0), DEV)
    shape = StepShape(batch=cfg.batch, total_q=inp.total_q, total_target_rows=inp.total_target_rows,
                      num_heads_q=cfg.num_heads_q, num_heads_kv=cfg.num_heads_kv,
                      head_dim=cfg.head_dim, hidden=cfg.hidden, vocab=cfg.vocab,
                      max_total_ctx=inp.max_total_ctx, max_draft_k=int(b.draft_k.max()))
    step = DraftVerifyStep(shape, DEV, opts)
    if opts.n_summary:
        step.summary_init(t)
        torch.cuda.synchronize()
        zs = step.summary_values.cpu().numpy()      # the state the attention reads
    seed = inp.philox_seed
    step.attention(t)
    step.lm_head(t, seed)
    torch.cuda.synchronize()
    base = step.logits.cpu().numpy()                # before the correction
    step.markov(t, seed)
    step.verify(t, seed)
    torch.cuda.synchronize()
    reqs = range(cfg.batch)

    # 1. attention (with the device's summary state, staged)
    kw = dict(window=256, summary_keys=u, summary_values=zs) if opts.n_summary else {}
    ref = oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache, inp.page_table,
                        b.ctx_len, b.q_off, cfg.num_heads_kv, inp.softmax_scale, **kw)
    rep = compare.attention_report(bits(step.attn_out), ref)
    log(f"{path} chain: attention {rep}")
    assert rep["ok"] and rep["rel_l2"] < 1e-2
    # 2. LM head base logits
    z_ref = olm.lm_head_logits(inp.hidden, inp.w_vocab)
    dz = np.abs(base - z_ref).max()
    # 3. correction and draws from the device's base logits
    got = (step.logits.cpu().numpy(), step.lse.cpu().numpy(), step.tokens.cpu().numpy())
    ref_m = omk.markov_sample(base, b.q_off, anchor, w_c, e_c, inp.req_id, seed,
                              alpha=opts.markov_alpha,
                              vocab_bias=None if bias is None else t["vocab_bias"].cpu().numpy(),
                              greedy=opts.greedy)
    log(f"{path} chain: base logits max-abs {dz:.2e}")
    assert dz <= 1e-5
    _compare(got, ref_m, b.q_off, reqs, f"{path} chain: correction")
    # 4. verification of the device's corrected drafts
    ref_v = overify.verify(inp.target_logits, b.t_off, got[0].astype(np.float64), got[2], b.q_off,
                           inp.req_id, seed, requests=list(reqs), greedy=opts.greedy)
    rep = compare.verify_report(step.accepted.cpu().numpy(), step.next_token.cpu().numpy(), ref_v,
                                reqs)
    log(f"{path} chain: verify {rep}")
    assert rep["ok"]
