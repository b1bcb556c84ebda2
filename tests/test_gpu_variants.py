"""GPU parity of the attention variants and the context summary.

* causal block mask, recent window, summary rows (and all three together):
  attention outputs within 1e-2 max-abs and relative L2 < 1e-2 of the oracle;
* the summary state kept by sd_summary_update (initialisation from a whole
  prefix, then a fold of a_b + 1 new rows): fp32 arithmetic over at most a
  few thousand rows here, compared with the oracle's fp64 definition within
  max-abs 1e-4 on Z (entries of size ~0.1..1) and 1e-4 relative on c;
* the fixed-cost context of the 128K workload (window 256 + 16 summary
  entries) at full size, on sampled requests: the summary state within
  max-abs 1e-4 and relative L2 1e-4 of the oracle (entries ~5e-3, 131,072
  fp32 terms each), the attention as in the parity suite;
* temperature-0 drafting and verification and the pruned drafter vocabulary:
  probabilities within 1e-5, tokens and accepted lengths exact except
  audited near-ties (as in the main parity suite), including the 128K
  workload's LM head with 32,000 drafter tokens.
"""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import attention as oa, compare, step as ostep, summary as osum, verify as overify
from synth import StepInputs, device as sdev
from synth.configs import C1_32K, C2_128K, C4_RAGGED

from gpu_common import DEV, bits, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

Z_ATOL = 1e-4
C_RTOL = 1e-4


def _cfg(**kw):
    base = dict(name="variants", batch=5, ctx=("list", (0, 1, 37, 160, 1000)),
                draft_k=("list", (3, 1, 16, 5, 8)), verify="full", num_heads_q=8,
                num_heads_kv=2, head_dim=128, hidden=64, vocab=64, seed=5151)
    base.update(kw)
    return C1_32K.with_(**base)


def _gpu_attn(inp, t=None, split_tokens=0, **kw):
    t = sdev.attention_tensors(inp, DEV) if t is None else t
    b = inp.budgets
    out = sd.sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"],
                           t["page_table"], t["ctx_len"], t["q_off"],
                           max_draft_k=int(b.draft_k.max()), max_total_ctx=inp.max_total_ctx,
                           split_tokens=split_tokens, **kw)
    torch.cuda.synchronize()
    return bits(out)


def _oracle_attn(inp, requests=None, **kw):
    b = inp.budgets
    return oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache, inp.page_table,
                         b.ctx_len, b.q_off, inp.cfg.num_heads_kv, inp.softmax_scale,
                         requests=requests, **kw)


def _check(got, ref, rows=None, tag=""):
    rep = compare.attention_report(got, ref, rows=rows)
    log(f"{tag} {rep}")
    assert rep["ok"] and rep["rel_l2"] < 1e-2


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("split", [0, 64])
def test_causal_block(head_dim, split):
    inp = StepInputs(_cfg(head_dim=head_dim))
    got = _gpu_attn(inp, split_tokens=split, block_mask=sd.SD_MASK_CAUSAL)
    _check(got, _oracle_attn(inp, block_mask="causal"), tag=f"causal D={head_dim} split={split}")


@pytest.mark.parametrize("mode", ["causal", "window", "summary"])
def test_variants_large_group(mode):
    """The variants with 128-row work items (GQA group 8, K = 16)."""
    inp = StepInputs(_cfg(num_heads_q=64, num_heads_kv=8, draft_k=("list", (16, 1, 16, 5, 9)),
                          seed=818))
    if mode == "causal":
        got = _gpu_attn(inp, split_tokens=64, block_mask=sd.SD_MASK_CAUSAL)
        ref = _oracle_attn(inp, block_mask="causal")
    elif mode == "window":
        got = _gpu_attn(inp, split_tokens=64, window=50)
        ref = _oracle_attn(inp, window=50)
    else:
        u, z = inp.summary_queries(16), inp.summary_values(16)
        got = _gpu_attn(inp, window=256, summary_keys=sdev.bf16(u, DEV),
                        summary_values=sdev.f32(z, DEV))
        ref = _oracle_attn(inp, window=256, summary_keys=u, summary_values=z)
    _check(got, ref, tag=f"large group {mode}")


def test_causal_block_mha_two_block_tiles():
    # G = 1 and K_b up to 40: the block spans two 32-key tiles
    inp = StepInputs(_cfg(num_heads_q=2, num_heads_kv=2, head_dim=64,
                          draft_k=("list", (40, 33, 1, 32, 17)), seed=77))
    got = _gpu_attn(inp, block_mask=sd.SD_MASK_CAUSAL)
    _check(got, _oracle_attn(inp, block_mask="causal"), tag="causal mha")


@pytest.mark.parametrize("window", [1, 16, 50, 256, 2048])
def test_recent_window(window):
    inp = StepInputs(_cfg())
    got = _gpu_attn(inp, split_tokens=64, window=window)
    _check(got, _oracle_attn(inp, window=window), tag=f"window {window}")


@pytest.mark.parametrize("window,causal", [(2048, True), (1500, False), (4096, True)])
def test_window_automatic_split(window, causal):
    """A long window under the automatic split: with few (request, KV head)
    pairs the window is cut into several items of at least 512 tokens
    (prefixes longer and shorter than the window, an empty one, ragged K_b)."""
    inp = StepInputs(_cfg(batch=6, ctx=("list", (20000, 0, 1500, 9000, 4099, 70)),
                          draft_k=("list", (16, 3, 16, 1, 8, 5)), num_heads_q=32,
                          num_heads_kv=8, seed=6000 + window))
    mask = sd.SD_MASK_CAUSAL if causal else sd.SD_MASK_NONE
    got = _gpu_attn(inp, window=window, block_mask=mask)
    ref = _oracle_attn(inp, window=window, block_mask="causal" if causal else "none")
    _check(got, ref, tag=f"window {window} automatic split causal={causal}")


@pytest.mark.parametrize("n_summary", [16, 40])
@pytest.mark.parametrize("causal", [False, True])
def test_fixed_cost_context(n_summary, causal):
    inp = StepInputs(_cfg(head_dim=64 if n_summary == 40 else 128))
    u, z = inp.summary_queries(n_summary), inp.summary_values(n_summary)
    t = sdev.attention_tensors(inp, DEV)
    mask = sd.SD_MASK_CAUSAL if causal else sd.SD_MASK_NONE
    got = _gpu_attn(inp, t=t, window=256, block_mask=mask,
                    summary_keys=sdev.bf16(u, DEV), summary_values=sdev.f32(z, DEV))
    ref = _oracle_attn(inp, window=256, block_mask="causal" if causal else "none",
                       summary_keys=u, summary_values=z)
    _check(got, ref, tag=f"fixed-cost S={n_summary} causal={causal}")


def _gpu_summary(inp, u, ctx, acc=None, state=None):
    t = sdev.attention_tensors(inp, DEV)
    B, hkv, S, D = inp.cfg.batch, inp.cfg.num_heads_kv, u.shape[1], u.shape[2]
    if state is None:
        z = torch.full((B, hkv, S, D), float("nan"), device=DEV)
        c = torch.full((B, hkv, S), float("nan"), device=DEV)
    else:
        z, c = state
    sd.sd_summary_update(sdev.bf16(u, DEV), t["k_cache"], t["v_cache"], t["page_table"],
                         sdev.i32(ctx, DEV), None if acc is None else sdev.i32(acc, DEV), z, c)
    torch.cuda.synchronize()
    return z, c


def _check_summary(z, c, Zr, Cr, tag):
    zg, cg = z.cpu().numpy().astype(np.float64), c.cpu().numpy().astype(np.float64)
    empty = Cr == -np.inf
    assert np.all(cg[empty] == -np.inf) and np.all(zg[empty] == 0)
    dz = np.abs(zg - Zr).max()
    dc = np.abs(cg[~empty] - Cr[~empty]) / np.maximum(1.0, np.abs(Cr[~empty]))
    log(f"{tag}: Z max-abs {dz:.3g}, c max-rel {dc.max() if dc.size else 0:.3g}")
    assert dz <= Z_ATOL and (dc.size == 0 or dc.max() <= C_RTOL)


@pytest.mark.parametrize("head_dim,n_summary", [(128, 16), (64, 64), (128, 40), (64, 5), (128, 64),
                                                (64, 17)])
def test_summary_init_then_fold(head_dim, n_summary):
    # every round appends a_b + 1 >= 1 rows; the first request starts empty
    inp = StepInputs(_cfg(head_dim=head_dim, batch=5, ctx=("list", (1, 2, 37, 160, 1000)),
                          draft_k=("list", (16, 16, 16, 16, 16))))
    b = inp.budgets
    u = inp.summary_queries(n_summary)
    hkv, scale = inp.cfg.num_heads_kv, inp.softmax_scale
    # the last a_b + 1 rows of each prefix are the new rows of the round
    acc = np.array([0, 0, 5, 16, 9], np.int32)
    old = (b.ctx_len - acc - 1).astype(np.int32)
    Z0, C0 = osum.summary_init(u, inp.k_cache, inp.v_cache, inp.page_table, old, hkv, scale)
    z, c = _gpu_summary(inp, u, old)
    _check_summary(z, c, Z0, C0, f"init D={head_dim} S={n_summary}")
    # fold from the GPU's own state: the oracle folds into the same fp32 state
    Zs = z.cpu().numpy().astype(np.float64)
    Cs = c.cpu().numpy().astype(np.float64)
    Z1, C1 = osum.summary_update(u, inp.k_cache, inp.v_cache, inp.page_table, old, acc, Zs, Cs,
                                 hkv, scale)
    z, c = _gpu_summary(inp, u, old, acc, state=(z, c))
    _check_summary(z, c, Z1, C1, f"fold D={head_dim} S={n_summary}")
    # and the result is the summary of every row (eq. (5))
    Zf, Cf = osum.summary_init(u, inp.k_cache, inp.v_cache, inp.page_table,
                               b.ctx_len.astype(np.int32), hkv, scale)
    _check_summary(z, c, Zf, Cf, "fold == summary of all rows")


@pytest.mark.parametrize("head_dim,n_summary", [(128, 16), (64, 33)])
def test_summary_init_sliced_ragged(head_dim, n_summary):
    """Initialisation over many slices: ragged prefixes (empty, shorter than a
    slice, ending inside a tile and inside a page, spanning dozens of
    slices), every slice's partial state merged by the second kernel."""
    ctx = (1, 5000, 12345, 511, 513, 31)
    inp = StepInputs(_cfg(head_dim=head_dim, batch=len(ctx), ctx=("list", ctx),
                          draft_k=("list", (1,) * len(ctx)), seed=6262))
    b = inp.budgets
    u = inp.summary_queries(n_summary)
    hkv = inp.cfg.num_heads_kv
    max_pages = inp.page_table.shape[1]
    ws = sd.summary_workspace_size(len(ctx), hkv, n_summary, head_dim, max_pages)
    log(f"sliced init: {max_pages} pages per row, workspace {ws} bytes")
    assert ws > 0
    n0 = b.ctx_len.astype(np.int32)
    n0[0] = 0                                   # an empty prefix
    Z0, C0 = osum.summary_init(u, inp.k_cache, inp.v_cache, inp.page_table, n0, hkv,
                               inp.softmax_scale)
    z, c = _gpu_summary(inp, u, n0)
    _check_summary(z, c, Z0, C0, f"sliced init D={head_dim} S={n_summary}")
    # folds that start inside a 32-token tile and end in the next one, or
    # start on a tile or page boundary
    acc = np.array([0, 40, 3, 30, 0, 20], np.int32)
    old = (b.ctx_len - acc - 1).astype(np.int32)
    z, c = _gpu_summary(inp, u, old)
    Zs = z.cpu().numpy().astype(np.float64)
    Cs = c.cpu().numpy().astype(np.float64)
    Z1, C1 = osum.summary_update(u, inp.k_cache, inp.v_cache, inp.page_table, old, acc, Zs, Cs,
                                 hkv, inp.softmax_scale)
    z, c = _gpu_summary(inp, u, old, acc, state=(z, c))
    _check_summary(z, c, Z1, C1, f"fold across tiles D={head_dim} S={n_summary}")


def test_summary_init_empty_requests_between():
    """Empty prefixes between non-empty ones inside one wavefront's run of
    the concatenated rows (the walk skips them), and more requests than one
    64-lane scan chunk."""
    ctx = (5, 0, 0, 7, 0, 600, 0, 1, 33) + (0,) * 60 + (40, 0, 513)
    inp = StepInputs(_cfg(batch=len(ctx), ctx=("list", ctx), draft_k=("list", (1,) * len(ctx)),
                          seed=7373))
    b = inp.budgets
    u = inp.summary_queries(16)
    Zr, Cr = osum.summary_init(u, inp.k_cache, inp.v_cache, inp.page_table, b.ctx_len,
                               inp.cfg.num_heads_kv, inp.softmax_scale)
    z, c = _gpu_summary(inp, u, b.ctx_len)
    _check_summary(z, c, Zr, Cr, f"init with empty requests between ({len(ctx)} requests)")


def test_summary_init_full_size_ragged():
    """The ragged serving mix at full size (128 requests, 1K-128K-token
    prefixes, 8 KV heads): with 1,024 (request, KV head) pairs every pair is
    one wavefront walking its whole prefix; its first 16 requests alone
    (128 pairs) are cut into slices and merged.  Sampled requests (the
    longest, the shortest, one between) against the oracle."""
    cfg = C4_RAGGED.with_(hidden=64, vocab=64)
    inp = StepInputs(cfg)
    t = sdev.attention_tensors(inp, DEV)
    b = inp.budgets
    hkv, D = cfg.num_heads_kv, cfg.head_dim
    u = inp.summary_queries(16)
    uu = sdev.bf16(u, DEV)
    ref = {}

    def oracle(r):
        if r not in ref:
            kl, vl = inp.logical_kv(r)
            zr, cr = np.zeros((hkv, 16, D)), np.zeros((hkv, 16))
            for g in range(hkv):
                zr[g], cr[g] = osum.summary_of_rows(u[g], kl[:, g], vl[:, g], inp.softmax_scale)
            ref[r] = (zr, cr)
        return ref[r]

    for nreq in (cfg.batch, 16):
        max_pages = t["page_table"].shape[1]
        ws = sd.summary_workspace_size(nreq, hkv, 16, D, max_pages)
        z = torch.full((nreq, hkv, 16, D), float("nan"), device=DEV)
        c = torch.full((nreq, hkv, 16), float("nan"), device=DEV)
        sd.sd_summary_update(uu, t["k_cache"], t["v_cache"], t["page_table"][:nreq].contiguous(),
                             t["ctx_len"][:nreq].contiguous(), None, z, c)
        torch.cuda.synchronize()
        n = b.ctx_len[:nreq]
        reqs = sorted({int(np.argmax(n)), int(np.argmin(n)), nreq // 2})
        zg, cg = z.cpu().numpy(), c.cpu().numpy()
        for r in reqs:
            zr, cr = oracle(r)
            dz = np.abs(zg[r] - zr).max()
            rel = np.linalg.norm(zg[r] - zr) / np.linalg.norm(zr)
            dc = (np.abs(cg[r] - cr) / np.maximum(1, np.abs(cr))).max()
            log(f"ragged summary init, {nreq} requests (workspace {ws} B), request {r} "
                f"({int(n[r])} tokens): Z max-abs {dz:.3g}, rel-L2 {rel:.3g}, c max-rel {dc:.3g}")
            assert dz <= Z_ATOL and rel <= 1e-4 and dc <= C_RTOL


def test_summary_then_attention_chain():
    inp = StepInputs(_cfg())
    u = inp.summary_queries(16)
    z, c = _gpu_summary(inp, u, inp.budgets.ctx_len)
    got = _gpu_attn(inp, window=256, summary_keys=sdev.bf16(u, DEV), summary_values=z)
    ref = _oracle_attn(inp, window=256, summary_keys=u, summary_values=z.cpu().numpy())
    _check(got, ref, tag="summary -> attention")


def test_fixed_cost_full_size_128k():
    cfg = C2_128K
    inp = StepInputs(cfg)
    u = inp.summary_queries(16)
    t = sdev.attention_tensors(inp, DEV)
    b = inp.budgets
    B, hkv, D = cfg.batch, cfg.num_heads_kv, cfg.head_dim
    z = torch.empty((B, hkv, 16, D), device=DEV)
    c = torch.empty((B, hkv, 16), device=DEV)
    uu = sdev.bf16(u, DEV)
    sd.sd_summary_update(uu, t["k_cache"], t["v_cache"], t["page_table"], t["ctx_len"], None, z, c)
    out = sd.sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"],
                           t["page_table"], t["ctx_len"], t["q_off"],
                           max_draft_k=int(b.draft_k.max()), max_total_ctx=inp.max_total_ctx,
                           window=256, summary_keys=uu, summary_values=z)
    torch.cuda.synchronize()
    reqs = [0, B - 1]
    zr = np.zeros((B, hkv, 16, D))
    cr = np.zeros((B, hkv, 16))
    for r in reqs:
        kl, vl = inp.logical_kv(r)
        for g in range(hkv):
            zr[r, g], cr[r, g] = osum.summary_of_rows(u[g], kl[:, g], vl[:, g], inp.softmax_scale)
    zg, cg = z.cpu().numpy(), c.cpu().numpy()
    dz = max(np.abs(zg[r] - zr[r]).max() for r in reqs)
    rel = max(np.linalg.norm(zg[r] - zr[r]) / np.linalg.norm(zr[r]) for r in reqs)
    dc = max((np.abs(cg[r] - cr[r]) / np.maximum(1, np.abs(cr[r]))).max() for r in reqs)
    zmag = max(np.abs(zr[r]).max() for r in reqs)
    log(f"128K summary init: Z max-abs {dz:.3g} (entries up to {zmag:.3g}), rel-L2 {rel:.3g}, "
        f"c max-rel {dc:.3g}")
    # 131,072 fp32 terms per entry, merged tile by tile: the relative error of
    # an fp32 running sum of n terms stays near sqrt(n) * 2^-24 ~ 2e-5
    assert dz <= Z_ATOL and rel <= 1e-4 and dc <= C_RTOL
    rows = np.concatenate([np.arange(b.q_off[r], b.q_off[r + 1]) for r in reqs])
    ref = _oracle_attn(inp, requests=reqs, window=256, summary_keys=u, summary_values=zg)
    _check(bits(out), ref, rows=rows, tag="128K fixed-cost attention")


# ------------------------------------------------- temperature 0, pruned vocab


def _lm_cfg(**kw):
    base = dict(name="lm_variants", batch=3, ctx=("list", (16, 16, 16)),
                draft_k=("list", (16, 5, 16)), verify="full", num_heads_q=8, num_heads_kv=2,
                head_dim=64, hidden=256, vocab=4100, seed=9090)
    base.update(kw)
    return C1_32K.with_(**base)


def _gpu_lm(inp, **kw):
    t = sdev.lm_head_tensors(inp, DEV)
    z, lse, tok = sd.sd_lm_head_probs(t["hidden"], t["w_vocab"], t["q_off"], t["req_id"],
                                      inp.philox_seed, **kw)
    torch.cuda.synchronize()
    return z, lse, tok


@pytest.mark.parametrize("pruned", [False, True])
@pytest.mark.parametrize("greedy", [False, True])
def test_lm_head_greedy_and_pruned(greedy, pruned):
    inp = StepInputs(_lm_cfg())
    vmap = inp.pruned_vocab(1000) if pruned else None
    z, lse, tok = _gpu_lm(inp, greedy=greedy,
                          vocab_map=None if vmap is None else sdev.i32(vmap, DEV))
    b = inp.budgets
    ref = ostep.run_lm_head(inp.hidden, inp.w_vocab, b.q_off, inp.req_id, inp.philox_seed,
                            greedy=greedy, vocab_map=vmap)
    rep = compare.lm_head_report(z.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy(), ref)
    log(f"lm head greedy={greedy} pruned={pruned}: {rep}")
    assert rep["ok"] and rep["logit_max_abs"] < 1e-5


def _verify_inputs(inp, rng, vd=None):
    """Seeded draft logits / tokens: a fraction of the tokens is the target
    row's argmax so that temperature-0 tests accept some drafts."""
    b = inp.budgets
    V = inp.cfg.vocab
    x = inp.target_logits
    vmap = None if vd is None else inp.pruned_vocab(vd)
    z = (rng.standard_normal((inp.total_q, V if vd is None else vd)) * 1.5).astype(np.float32)
    tok = np.empty(inp.total_q, np.int32)
    for r in range(inp.cfg.batch):
        q0, t0 = int(b.q_off[r]), int(b.t_off[r])
        for j in range(int(b.q_off[r + 1]) - q0):
            row = x[t0 + min(j, int(b.t_off[r + 1]) - t0 - 1)]
            if rng.random() < 0.8 and (vmap is None or np.argmax(row) in vmap):
                tok[q0 + j] = int(np.argmax(row))
            else:
                tok[q0 + j] = int(rng.integers(0, V)) if vmap is None else int(rng.choice(vmap))
    return z, tok, vmap


@pytest.mark.parametrize("batch", [24, 56])
@pytest.mark.parametrize("mode", ["greedy", "pruned", "greedy_pruned"])
def test_verify_greedy_and_pruned(mode, batch):
    inp = StepInputs(_lm_cfg(batch=batch, ctx=16, draft_k=(16, 7, 1), verify="uniform",
                             vocab=20000, seed=3131))
    b = inp.budgets
    greedy = mode.startswith("greedy")
    rng = np.random.default_rng(12)
    z, tok, vmap = _verify_inputs(inp, rng, vd=5000 if "pruned" in mode else None)
    inv = None
    if vmap is not None:
        inv = np.full(inp.cfg.vocab, -1, np.int32)
        inv[vmap] = np.arange(len(vmap), dtype=np.int32)
    zd = z.astype(np.float64)
    lse = (zd.max(1) + np.log(np.exp(zd - zd.max(1, keepdims=True)).sum(1))).astype(np.float32)
    t = sdev.verify_tensors(inp, DEV)
    acc, nxt, _ = sd.sd_verify(t["target_logits"], t["t_off"], sdev.f32(z, DEV),
                               sdev.f32(lse, DEV), sdev.i32(tok, DEV), t["q_off"], t["req_id"],
                               inp.philox_seed, greedy=greedy,
                               draft_vocab_inv=None if inv is None else sdev.i32(inv, DEV))
    torch.cuda.synchronize()
    ref = overify.verify(inp.target_logits, b.t_off, z, tok, b.q_off, inp.req_id,
                         inp.philox_seed, greedy=greedy, draft_vocab_inv=inv)
    rep = compare.verify_report(acc.cpu().numpy(), nxt.cpu().numpy(), ref, range(inp.cfg.batch))
    log(f"verify {mode}: {rep}")
    assert rep["ok"]
    if greedy:
        assert 0 < rep["mean_accepted"]


def test_pruned_vocab_full_size_128k_shapes():
    # the LM head of the 128K workload with the drafter restricted to 32,000
    # target tokens, then verification against the full target vocabulary
    cfg = C2_128K.with_(ctx=16)
    inp = StepInputs(cfg)
    b = inp.budgets
    vmap = inp.pruned_vocab(32000)
    inv = np.full(cfg.vocab, -1, np.int32)
    inv[vmap] = np.arange(32000, dtype=np.int32)
    z, lse, tok = _gpu_lm(inp, vocab_map=sdev.i32(vmap, DEV))
    rows = np.array([0, 1, 17, 100, inp.total_q - 1])
    ref = ostep.run_lm_head(inp.hidden, inp.w_vocab, b.q_off, inp.req_id, inp.philox_seed,
                            rows=rows, vocab_map=vmap)
    rep = compare.lm_head_report(z.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy(), ref)
    log(f"pruned LM head 256 x 4096 x 32000: {rep}")
    assert rep["ok"]
    assert np.all(np.isin(tok.cpu().numpy(), vmap))
    t = sdev.verify_tensors(inp, DEV)
    acc, nxt, _ = sd.sd_verify(t["target_logits"], t["t_off"], z, lse, tok, t["q_off"],
                               t["req_id"], inp.philox_seed, draft_vocab_inv=sdev.i32(inv, DEV))
    torch.cuda.synchronize()
    reqs = [0, 7, cfg.batch - 1]
    ref_v = overify.verify(inp.target_logits, b.t_off, z.cpu().numpy(), tok.cpu().numpy(),
                           b.q_off, inp.req_id, inp.philox_seed, requests=reqs,
                           draft_vocab_inv=inv)
    rv = compare.verify_report(acc.cpu().numpy(), nxt.cpu().numpy(), ref_v, reqs)
    log(f"pruned verify at 151936: {rv}")
    assert rv["ok"]
