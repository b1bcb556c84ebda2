"""GPU parity of the ForeSpark scheduler (sd_schedule_draft / sd_schedule_verify).

Staged comparison: the estimator outputs are compared with the oracle's fp64
values (logits within 1e-4 after 2 x 4096-term fp32 dot products; scores and
probabilities within 1e-5), then the oracle takes the scheduling decisions
from the GPU's own logits / probabilities, so one near-tie cannot cascade.
Integer decisions (sum d_i, B, each d_i, each b_i) must match exactly except
audited near-ties: two bucket-pair objectives within 1e-5 (relative), or
sorted scores / survival values within 1e-5 across the selection boundary.
"""
import numpy as np
import pytest
import torch

import block_drafting_sd_amd as sd
from oracle import schedule as osch
from synth import device as sdev
from synth.schedule_inputs import ScheduleInputs

from gpu_common import DEV, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

NEAR = 1e-5


def _dev_predraft(si):
    p = si.predraft()
    t = {k: (sdev.bf16(v, DEV) if v.dtype == np.uint16 else sdev.f32(v, DEV)) for k, v in p.items()}
    caps, dl, vc, vl = si.latency_tables()
    tab = dict(draft_caps=sdev.i32(caps, DEV), draft_lat=sdev.f32(dl, DEV),
               verify_caps=sdev.i32(vc, DEV), verify_lat=sdev.f32(vl, DEV))
    return p, t, (caps, dl, vc, vl), tab


def _gpu_schedule(si, t, tab, n_nonspec):
    out = sd.sd_schedule_draft(t["ctx_feat"], t["anchor_emb"], t["w_c"], t["w_e"], t["w_o"],
                               tab["draft_caps"], tab["draft_lat"], tab["verify_caps"],
                               tab["verify_lat"], n_nonspec, b_u=t["b_u"], b_o=t["b_o"],
                               cal_scale=t["cal_scale"], cal_bias=t["cal_bias"], K=si.K)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _scores_from_logits(z, K):
    return np.stack([osch.survival_scores(osch.reward_curve(osch.survival_benefits(z[i], K), K))
                     for i in range(len(z))])


def _check_schedule(si, p, tables, got, n_nonspec, tag):
    K = si.K
    z_ref = osch.predraft_logits(p["ctx_feat"], p["anchor_emb"], p["w_c"], p["w_e"], p["w_o"],
                                 p["b_u"], p["b_o"], p["cal_scale"], p["cal_bias"])
    dz = np.abs(got["logits"] - z_ref).max()
    g_ref = _scores_from_logits(got["logits"].astype(np.float64), K)   # staged
    dg = np.abs(got["scores"] - g_ref).max()
    res = osch.joint_schedule(g_ref, n_nonspec, *tables)
    cands = sorted((c[0] for c in osch.pair_candidates(g_ref, n_nonspec, *tables)), reverse=True)
    pair_tie = len(cands) > 1 and np.isfinite(cands[1]) and \
        (cands[0] - cands[1]) <= NEAR * abs(cands[0])
    k_gpu, B_gpu = int(got["q_off"][-1]), int(got["verify_budget"][0])
    vals, owner = osch.sorted_scores(g_ref)
    k = res["k"]
    # requests owning scores within NEAR of the selection boundary: only they
    # may split the boundary differently (a run of equal scores inside one
    # request is ordered by d on both sides)
    tied = set()
    if 0 < k < len(vals):
        lo, hi = vals[k] - NEAR, vals[k - 1] + NEAR
        tied = {int(o) for v, o in zip(vals, owner) if lo <= v <= hi}
    boundary_tie = len(tied) > 1
    log(f"{tag}: logits max-abs {dz:.2e}, scores max-abs {dg:.2e}, k {k_gpu}/{k}, "
        f"B {B_gpu}/{res['budget']}, objective {got['objective'][0]:.6g}/{res['objective']:.6g}, "
        f"pair tie {pair_tie}, requests tied at the boundary {len(tied) if boundary_tie else 0}")
    assert dz <= 1e-4 and dg <= 1e-5
    assert abs(got["objective"][0] - res["objective"]) <= 1e-5 * abs(res["objective"])
    if not pair_tie:
        assert (k_gpu, B_gpu) == (k, res["budget"])
        free = np.array([i not in tied or not boundary_tie for i in range(len(got["draft_len"]))])
        np.testing.assert_array_equal(got["draft_len"][free], res["draft_len"][free])
        if boundary_tie:
            ids = sorted(tied)
            assert got["draft_len"][ids].sum() == res["draft_len"][ids].sum()
    assert np.all(np.diff(got["q_off"]) == got["draft_len"]) and got["q_off"][0] == 0
    assert np.all(got["draft_len"] <= K) and B_gpu <= k_gpu
    return res


@pytest.mark.parametrize("n,K,d_h,r", [(5, 6, 64, 32), (37, 16, 256, 64), (192, 16, 4096, 256)])
def test_schedule_draft(n, K, d_h, r):
    si = ScheduleInputs(n=n, K=K, d_h=d_h, r=r, seed=100 + n)
    p, t, tables, tab = _dev_predraft(si)
    got = _gpu_schedule(si, t, tab, n)
    _check_schedule(si, p, tables, got, n, f"schedule n={n} K={K}")


def test_schedule_draft_tight_tables():
    # a verifier bucket below N + 1 drafts, and a draft table that cannot hold
    # every request's K drafts: B is capped by the tables, not by the scores
    si = ScheduleInputs(n=64, K=8, d_h=128, r=32, seed=7)
    p, t, _, _ = _dev_predraft(si)
    caps = np.array([64, 96, 160], np.int32)
    dl = np.array([1.0, 1.5, 2.5], np.float32)
    vc = np.array([64, 80, 100], np.int32)
    vl = np.array([3.0, 3.1, 3.3], np.float32)
    tab = dict(draft_caps=sdev.i32(caps, DEV), draft_lat=sdev.f32(dl, DEV),
               verify_caps=sdev.i32(vc, DEV), verify_lat=sdev.f32(vl, DEV))
    got = _gpu_schedule(si, t, tab, 64)
    res = _check_schedule(si, p, (caps, dl, vc, vl), got, 64, "schedule tight tables")
    assert res["budget"] <= 100 - 64


def _oracle_budget(got_p, q_off, B):
    return osch.distribute_budget(got_p.astype(np.float64), q_off, B)


@pytest.mark.parametrize("n,K,H,m,V", [(6, 8, 64, 16, 300), (192, 16, 4096, 256, 151936)])
def test_schedule_verify(n, K, H, m, V):
    si = ScheduleInputs(n=n, K=K, d_h=H, m=m, V=V, seed=300 + n)
    rng = np.random.default_rng(n)
    d = rng.integers(0, K + 1, n).astype(np.int32)
    q_off = np.concatenate([[0], np.cumsum(d)]).astype(np.int32)
    rows = n * K
    pp = si.postdraft(rows)
    B = int(q_off[-1] * 0.6)
    t = dict(hidden=sdev.bf16(pp["hidden"], DEV), w_s=sdev.bf16(pp["w_s"], DEV),
             e_pred=sdev.bf16(pp["e_pred"], DEV), w=sdev.f32(pp["w"], DEV),
             temperature=sdev.f32(pp["temperature"], DEV), anchor=sdev.i32(pp["anchor"], DEV),
             tokens=sdev.i32(pp["tokens"], DEV))
    out = sd.sd_schedule_verify(t["hidden"], t["w_s"], t["e_pred"], t["w"], t["anchor"],
                                t["tokens"], sdev.i32(q_off, DEV),
                                sdev.i32(np.array([B], np.int32), DEV), bias=pp["bias"],
                                temperature=t["temperature"], K=K)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    M = int(q_off[-1])
    req = np.repeat(np.arange(n), d)
    pos = np.arange(M) - q_off[req] + 1
    prev = np.where(pos == 1, pp["anchor"][req], pp["tokens"][np.maximum(np.arange(M) - 1, 0)])
    p_ref = osch.postdraft_probs(pp["hidden"][:M], pp["w_s"], pp["e_pred"], pp["w"], prev, pos,
                                 pp["bias"], pp["temperature"])
    dp = np.abs(got["accept_prob"][:M] - p_ref).max()
    S_ref, b_ref = _oracle_budget(got["accept_prob"][:M], q_off, B)      # staged
    ds = np.abs(got["survival"][:M] - S_ref).max()
    srt = np.sort(S_ref)[::-1]
    tie = 0 < B < M and srt[B - 1] - srt[B] <= NEAR
    log(f"budget n={n}: p max-abs {dp:.2e}, S max-abs {ds:.2e}, sum b {got['verify_len'].sum()}"
        f"/{b_ref.sum()}, boundary tie {tie}")
    assert dp <= 1e-5 and ds <= 1e-5
    assert got["verify_len"].sum() == min(B, M)
    assert np.all(got["verify_len"] <= d)
    if not tie:
        np.testing.assert_array_equal(got["verify_len"], b_ref)
    np.testing.assert_array_equal(np.diff(got["t_off"]), got["verify_len"] + 1)


def test_schedule_chain_192_requests():
    # pre-draft schedule -> its q_off and B feed the budget distribution on
    # the device; the chain is compared stage by stage
    si = ScheduleInputs(n=192, K=16, d_h=4096, r=256, m=256, seed=5)
    p, t, tables, tab = _dev_predraft(si)
    out = sd.sd_schedule_draft(t["ctx_feat"], t["anchor_emb"], t["w_c"], t["w_e"], t["w_o"],
                               tab["draft_caps"], tab["draft_lat"], tab["verify_caps"],
                               tab["verify_lat"], 192, b_u=t["b_u"], b_o=t["b_o"],
                               cal_scale=t["cal_scale"], cal_bias=t["cal_bias"], K=16)
    rows = 192 * 16
    pp = si.postdraft(rows)
    post = sd.sd_schedule_verify(sdev.bf16(pp["hidden"], DEV), sdev.bf16(pp["w_s"], DEV),
                                 sdev.bf16(pp["e_pred"], DEV), sdev.f32(pp["w"], DEV),
                                 sdev.i32(pp["anchor"], DEV), sdev.i32(pp["tokens"], DEV),
                                 out["q_off"], out["verify_budget"], bias=pp["bias"],
                                 temperature=sdev.f32(pp["temperature"], DEV), K=16)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    _check_schedule(si, p, tables, got, 192, "chain: schedule")
    q_off = got["q_off"]
    M = int(q_off[-1])
    B = int(got["verify_budget"][0])
    pa = post["accept_prob"].cpu().numpy()
    S_ref, b_ref = _oracle_budget(pa[:M], q_off, B)
    vl = post["verify_len"].cpu().numpy()
    srt = np.sort(S_ref)[::-1]
    tie = 0 < B < M and srt[B - 1] - srt[B] <= NEAR
    log(f"chain: budget {B} of {M} drafted, sum b {vl.sum()}, boundary tie {tie}")
    assert vl.sum() == min(B, M)
    if not tie:
        np.testing.assert_array_equal(vl, b_ref)
