"""GPU parity with non-finite values in cache slots that no query attends
(and that the context summary does not cover).

The target's cache is read in place ("H-Spec", sec. 3.3.2), so the slots of a
request's last page past its N_b tokens hold whatever the target last wrote
there (rejected drafts' KV, or never-written memory), and with a recent
window the slots of the window's first page before N_b - W are outside the
attended range.  Their weights are zero, and the output must not depend on
them at all: these tests fill every such slot of both caches with NaN and
+-infinity bf16 patterns and compare with the oracle, which never reads them.
The summary walks 32-token tiles, so its first and last tiles hold rows
outside the range it summarises; those are poisoned too.
"""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import attention as oa, compare, summary as osum
from synth import StepInputs, device as sdev
from synth.configs import C1_32K, C2_128K

from gpu_common import DEV, bits, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

# NaN (quiet, both signs), a NaN with a low payload, +inf, -inf
POISON = np.array([0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80], np.uint16)


def _poison(t, inp, window=0):
    """Overwrite the unattended slots in place; returns how many were hit."""
    kc = t["k_cache"].view(torch.int16)     # [pages, Hkv, D/8, 16, 8]
    vc = t["v_cache"].view(torch.int16)     # [pages, Hkv, D, 16]
    pt = inp.page_table
    hit = 0
    for b, n in enumerate(inp.budgets.ctx_len.tolist()):
        slots = []
        if n % 16:                                       # past N_b in the last page
            slots.append((pt[b, n // 16], n % 16, 16))
        if window and n > window and (n - window) % 16:  # before the window in its first page
            n0 = n - window
            slots.append((pt[b, n0 // 16], 0, n0 % 16))
        for page, s0, s1 in slots:
            page = int(page)
            w = s1 - s0
            pat = torch.from_numpy(np.resize(POISON, kc[page, :, :, s0:s1, :].numel())
                                   .view(np.int16).copy()).to(DEV)
            kc[page, :, :, s0:s1, :] = pat.view(kc[page, :, :, s0:s1, :].shape)
            patv = torch.from_numpy(np.resize(POISON[::-1], vc[page, :, :, s0:s1].numel())
                                    .view(np.int16).copy()).to(DEV)
            vc[page, :, :, s0:s1] = patv.view(vc[page, :, :, s0:s1].shape)
            hit += w
    torch.cuda.synchronize()
    return hit


def _run(inp, split_tokens=0, window=0):
    t = sdev.attention_tensors(inp, DEV)
    hit = _poison(t, inp, window)
    b = inp.budgets
    out = sd.sd_draft_attn(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"],
                           t["page_table"], t["ctx_len"], t["q_off"],
                           max_draft_k=int(b.draft_k.max()), max_total_ctx=inp.max_total_ctx,
                           split_tokens=split_tokens, window=window)
    torch.cuda.synchronize()
    ref = oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache, inp.page_table,
                        b.ctx_len, b.q_off, inp.cfg.num_heads_kv, inp.softmax_scale,
                        window=window)
    got = bits(out)
    return got, ref, hit


def _edge(**kw):
    base = dict(name="nonfinite", batch=5, ctx=("list", (0, 1, 37, 160, 1000)),
                draft_k=("list", (3, 1, 16, 5, 8)), verify="full", num_heads_q=8,
                num_heads_kv=2, head_dim=128, hidden=64, vocab=64, seed=606)
    base.update(kw)
    return C1_32K.with_(**base)


def _check(got, ref, tag):
    assert np.all(np.isfinite(oa.bf16_bits_to_f64(got)[np.isfinite(ref)])), f"{tag}: non-finite output"
    rep = compare.attention_report(got, ref)
    log(f"{tag} {rep}")
    assert rep["ok"] and rep["rel_l2"] < 1e-2


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("split", [0, 64, 192])
def test_nonfinite_past_prefix_end(head_dim, split):
    inp = StepInputs(_edge(head_dim=head_dim))
    log(f"nonfinite tail D={head_dim} split={split}")
    got, ref, hit = _run(inp, split_tokens=split)
    assert hit > 0
    _check(got, ref, f"nonfinite tail D={head_dim} split={split} slots={hit}")


@pytest.mark.parametrize("window", [16, 50, 256])
def test_nonfinite_outside_window(window):
    inp = StepInputs(_edge(ctx=("list", (0, 1, 37, 333, 1000))))
    log(f"nonfinite window={window}")
    got, ref, hit = _run(inp, split_tokens=64, window=window)
    assert hit > 0
    _check(got, ref, f"nonfinite window={window} slots={hit}")


def test_nonfinite_qwen_shapes():
    """The 128K workload's head shapes (32 / 8 / 128, K = 16) with ragged
    prefixes that end inside a page, including a long one."""
    cfg = C2_128K.with_(name="nonfinite_qwen", batch=4, ctx=("list", (1, 37, 1000, 65541)),
                        hidden=64, vocab=64, seed=607)
    inp = StepInputs(cfg)
    log("nonfinite qwen shapes")
    got, ref, hit = _run(inp)
    assert hit > 0
    _check(got, ref, f"nonfinite qwen slots={hit}")


def _poison_rows(t, inp, b, t0, t1):
    """Overwrite token rows [t0, t1) of request b in both caches."""
    kc = t["k_cache"].view(torch.int16)
    vc = t["v_cache"].view(torch.int16)
    for tok in range(t0, t1):
        page, slot = int(inp.page_table[b, tok // 16]), tok % 16
        pk = torch.from_numpy(np.resize(POISON, kc[page, :, :, slot, :].numel()).view(np.int16)
                              .copy()).to(DEV)
        kc[page, :, :, slot, :] = pk.view(kc[page, :, :, slot, :].shape)
        pv = torch.from_numpy(np.resize(POISON[::-1], vc[page, :, :, slot].numel()).view(np.int16)
                              .copy()).to(DEV)
        vc[page, :, :, slot] = pv.view(vc[page, :, :, slot].shape)
    return t1 - t0


@pytest.mark.parametrize("head_dim", [64, 128])
def test_nonfinite_summary(head_dim):
    """Initialisation with every slot past N_b poisoned, then a fold of
    a_b + 1 rows starting inside a 32-token tile whose earlier rows (already
    summarised) are poisoned as well."""
    inp = StepInputs(_edge(head_dim=head_dim, ctx=("list", (1, 37, 160, 1000, 77)),
                           draft_k=("list", (16, 16, 16, 16, 16))))
    t = sdev.attention_tensors(inp, DEV)
    b = inp.budgets
    n = b.ctx_len.astype(np.int32)
    acc = np.array([0, 5, 16, 9, 30], np.int32)
    old = (n - acc - 1).astype(np.int32)
    u = inp.summary_queries(16)
    hkv, D, B = inp.cfg.num_heads_kv, head_dim, len(n)
    hit = _poison(t, inp)
    assert hit > 0
    args = (sdev.bf16(u, DEV), t["k_cache"], t["v_cache"], t["page_table"])
    # initialisation over the whole prefixes: the slots past N_b are poisoned
    z = torch.full((B, hkv, 16, D), float("nan"), device=DEV)
    c = torch.full((B, hkv, 16), float("nan"), device=DEV)
    sd.sd_summary_update(*args, sdev.i32(n, DEV), None, z, c)
    torch.cuda.synchronize()
    Zr, Cr = osum.summary_init(u, inp.k_cache, inp.v_cache, inp.page_table, n, hkv,
                               inp.softmax_scale)
    zg, cg = z.cpu().numpy().astype(np.float64), c.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(zg)) and np.all(np.isfinite(cg))
    dz, dc = np.abs(zg - Zr).max(), (np.abs(cg - Cr) / np.maximum(1, np.abs(Cr))).max()
    log(f"nonfinite summary init D={head_dim} slots={hit}: Z max-abs {dz:.3g}, c max-rel {dc:.3g}")
    assert dz <= 1e-4 and dc <= 1e-4
    # the state before the new rows, then poison the rows of the fold's first
    # tile that come before it, and fold
    sd.sd_summary_update(*args, sdev.i32(old, DEV), None, z, c)
    torch.cuda.synchronize()
    Zs, Cs = z.cpu().numpy().astype(np.float64), c.cpu().numpy().astype(np.float64)
    hit2 = sum(_poison_rows(t, inp, r, int(old[r]) & ~31, int(old[r])) for r in range(B))
    torch.cuda.synchronize()
    assert hit2 > 0
    sd.sd_summary_update(*args, sdev.i32(old, DEV), sdev.i32(acc, DEV), z, c)
    torch.cuda.synchronize()
    Z1, C1 = osum.summary_update(u, inp.k_cache, inp.v_cache, inp.page_table, old, acc, Zs, Cs,
                                 hkv, inp.softmax_scale)
    zg, cg = z.cpu().numpy().astype(np.float64), c.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(zg)) and np.all(np.isfinite(cg))
    dz, dc = np.abs(zg - Z1).max(), (np.abs(cg - C1) / np.maximum(1, np.abs(C1))).max()
    log(f"nonfinite summary fold D={head_dim} slots={hit2}: Z max-abs {dz:.3g}, c max-rel {dc:.3g}")
    assert dz <= 1e-4 and dc <= 1e-4
