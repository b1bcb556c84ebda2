#!/usr/bin/env python3
"""Throughput of one block-parallel draft-and-verify step on one MI355X.

Default workload: 16 requests with 131072-token prefixes (Qwen3-8B shapes:
32 query / 8 KV heads, head dim 128, 16-token pages with a shuffled page
table, 8 GiB of bf16 prefix KV), a block of K = 16 drafts per request, an
LM head of 4096 x 151936, and full verification of the 16 drafts against 17
target rows per request.  A step = draft attention + LM head/sampling +
verification over one batch; inputs are resident in HBM before timing.

Prints ONE JSON line: drafted+verified tokens/s (sum of K_b per step / step
time), the attention call's achieved HBM bandwidth against the 8 TB/s peak,
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_sd_draft_attn_c2_n128k_b16.txt")
ATTN_SOURCE = os.path.join(ROOT, "block_drafting_sd_amd", "csrc", "attn.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


PATHS = {
    # the whole prefix, bidirectional block (the prefix-reading drafters)
    "full": dict(),
    # "LongSpark" fixed-cost context: recent window of 256 target KV rows and
    # 16 summary entries per KV head (App. B.1), summary folded every step
    "fixed": dict(window=256, n_summary=16),
    # "H-Spec": causal block over a 2048-token window, drafter vocabulary
    # pruned to 32,000 target tokens (sec. 3.3.2, App. B.2)
    "hspec": dict(causal_block=True, window=2048, draft_vocab=32000),
    # "LongSpark" with the sequential correction of rank 256 (sec. 2.3) on top
    # of the fixed-cost context
    "longspark": dict(window=256, n_summary=16, markov_rank=256),
    # "DeLS-Spec": the full-prefix block drafter with the Markov local head
    # fused as l_L + 0.3 l_S - 0.3 log p~_0 (rank 256: a reading)
    "dels": dict(markov_rank=256, markov_alpha=0.3, prior_beta=0.3),
}


def cpu_baseline(inp, n_req: int, target, opts, extra):
    """The oracle as it stands, on the first ``n_req`` requests of the workload
    (attention over all KV heads, LM head rows, verification and, on the
    fixed-cost path, the summary fold); scaled to drafted+verified tokens/s."""
    import numpy as np
    from oracle import step as ostep, summary as osum, verify as overify
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version') or ''}".strip()
                                 for i in pools})) or "unknown"
    except Exception:  # pragma: no cover
        threads, blas = 1, "unknown"
    b = inp.budgets
    c = inp.cfg
    reqs = list(range(n_req))
    rows = np.concatenate([np.arange(b.q_off[r], b.q_off[r + 1]) for r in reqs])
    kw = dict(block_mask="causal" if opts.causal_block else "none", window=opts.window)
    if opts.n_summary:   # summary of the prefix before the step (state, untimed)
        Z, C = osum.summary_init(extra["u"], inp.k_cache,
                                 inp.v_cache, inp.page_table[:n_req], extra["ctx_prev"][:n_req],
                                 c.num_heads_kv, inp.softmax_scale)
        Zf = np.zeros((c.batch,) + Z.shape[1:], np.float32)
        Zf[:n_req] = Z
        kw.update(summary_keys=extra["u"], summary_values=Zf)
    t0 = time.perf_counter()
    from oracle import attention as oattn
    oattn.draft_attn(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache, inp.page_table,
                     b.ctx_len, b.q_off, c.num_heads_kv, inp.softmax_scale, requests=reqs, **kw)
    t1 = time.perf_counter()
    lm = ostep.run_lm_head(inp.hidden, inp.w_vocab, b.q_off, inp.req_id, inp.philox_seed,
                           rows=rows, greedy=opts.greedy, vocab_map=extra.get("vmap"))
    full_z = np.zeros((inp.total_q, lm["logits"].shape[1]), np.float64)
    full_z[rows] = lm["logits"]
    tok = np.zeros(inp.total_q, np.int32)
    tok[rows] = lm["tokens"]
    if opts.markov_rank:
        from oracle import markov as omk
        bias = (-opts.prior_beta * omk.unigram_log_prior(extra["counts"])
                if opts.prior_beta else None)
        mk = omk.markov_sample(full_z, b.q_off, extra["anchor"], extra["w_c"], extra["e_c"],
                               inp.req_id, inp.philox_seed, requests=reqs,
                               alpha=opts.markov_alpha, vocab_bias=bias)
        full_z[rows], tok[rows] = mk["logits"][rows], mk["tokens"][rows]
    t2 = time.perf_counter()
    tgt = inp.target_logits if target is None else target
    res = overify.verify(tgt, b.t_off, full_z, tok, b.q_off, inp.req_id, inp.philox_seed,
                         requests=reqs, greedy=opts.greedy, draft_vocab_inv=extra.get("vinv"))
    t3 = time.perf_counter()
    if opts.n_summary:
        osum.summary_update(extra["u"], inp.k_cache, inp.v_cache, inp.page_table[:n_req],
                            extra["ctx_prev"][:n_req], res["accepted"][:n_req], Z, C,
                            c.num_heads_kv, inp.softmax_scale)
    t4 = time.perf_counter()
    tokens = int(sum(b.draft_k[r] for r in reqs))
    return {"value": tokens / (t4 - t0), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "blas": blas,
            "sample": (f"{n_req} of {c.batch} requests: attention over all "
                       f"{c.num_heads_kv} KV heads at N={int(b.ctx_len[0])}, LM head on "
                       f"{len(rows)} rows x {lm['logits'].shape[1]}"
                       + (f", rank-{opts.markov_rank} sequential correction"
                          if opts.markov_rank else "") + ", verification"
                       + (", summary fold" if opts.n_summary else "") +
                       f"; attn {t1 - t0:.2f}s lm {t2 - t1:.2f}s verify {t3 - t2:.2f}s"
                       + (f" fold {t4 - t3:.2f}s" if opts.n_summary else ""))}


def measured_traffic():
    """HBM bytes per sd_draft_attn call from the committed rocprofv3 PMC
    summary (FETCH_SIZE + WRITE_SIZE of the call's kernels, scaled by the same
    counters' reading for a device copy of known size), or None when the
    attention source has changed since those counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_SUMMARY):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        src = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
        if kv.get("attn_source_sha256") != src:
            return None
        return int(float(kv["traffic_bytes_per_call"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(gib: float):
    """A plain device copy of known size, for scaling PMC byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy calibration: {n * 4} bytes read and written per copy, 3 copies")


def measured_peaks(dev, read_gib: float = 4.0, mfma_iters: int = 20000, reps: int = 5):
    """The GPU's own ceilings: a plain streaming read of ``read_gib`` GiB and
    back-to-back independent bf16 MFMAs on every CU (library probes, HIP
    events on the current stream; the best of ``reps`` launches)."""
    import torch
    import block_drafting_sd_amd as sd
    buf = torch.empty(int(read_gib * (1 << 30)), dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    fsink = torch.zeros(4, dtype=torch.float32, device=dev)
    sd.sd_probe_read(buf, sink)
    sd.sd_probe_mfma(100, fsink)
    torch.cuda.synchronize()
    best_read = best_mfma = float("inf")
    flops = 0
    for _ in range(reps):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        sd.sd_probe_read(buf, sink)
        e1.record()
        flops = sd.sd_probe_mfma(mfma_iters, fsink)
        e2.record()
        torch.cuda.synchronize()
        best_read = min(best_read, e0.elapsed_time(e1))
        best_mfma = min(best_mfma, e1.elapsed_time(e2))
    del buf
    return {"hbm_read_gbs": round(read_gib * (1 << 30) / (best_read * 1e-3) / 1e9, 1),
            "mfma_bf16_tflops": round(flops / (best_mfma * 1e-3) / 1e12, 1),
            "read_bytes": int(read_gib * (1 << 30)), "mfma_flops": flops,
            "method": "sd_probe_read / sd_probe_mfma, best of %d launches" % reps}


def library_gemm(hidden, w, reps: int = 5, calls: int = 10):
    """Reference point for the LM head, not a step of the path: the vendor
    library's plain GEMM (torch.mm -> hipBLASLt) of the same bf16 operands
    with fp32 output, no softmax statistics or sampling.  Median of ``reps``
    timings of ``calls`` back-to-back calls (HIP events, current stream)."""
    import numpy as np
    import torch
    out = torch.empty(hidden.shape[0], w.shape[0], dtype=torch.float32, device=hidden.device)
    wt = w.t()
    for _ in range(3):
        torch.mm(hidden, wt, out_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            torch.mm(hidden, wt, out_dtype=torch.float32, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / calls)
    del out
    med = float(np.median(ms))
    flops = 2.0 * hidden.shape[0] * hidden.shape[1] * w.shape[0]
    return {"op": "torch.mm bf16 x bf16 -> fp32 (hipBLASLt), same operands, no epilogue",
            "ms": round(med, 4), "tflops": round(flops / (med * 1e-3) / 1e12, 1)}


def bench_schedule(args):
    """ForeSpark's scheduler between verification and drafting: pre-draft
    estimation + joint schedule, then post-draft estimation + budget
    distribution, for 192 requests ("ForeSpark", sec. 4.2-4.4)."""
    import numpy as np
    import torch
    import block_drafting_sd_amd as sd
    from synth import device as sdev
    from synth.schedule_inputs import ScheduleInputs

    sd.load()
    dev = torch.device("cuda:0")
    si = ScheduleInputs()
    p = si.predraft()
    t = {k: (sdev.bf16(v, dev) if v.dtype == np.uint16 else sdev.f32(v, dev)) for k, v in p.items()}
    caps, dl, vc, vl = si.latency_tables()
    tab = [sdev.i32(caps, dev), sdev.f32(dl, dev), sdev.i32(vc, dev), sdev.f32(vl, dev)]
    rows = si.n * si.K
    pp = si.postdraft(rows)
    tp = dict(hidden=sdev.bf16(pp["hidden"], dev), w_s=sdev.bf16(pp["w_s"], dev),
              e_pred=sdev.bf16(pp["e_pred"], dev), w=sdev.f32(pp["w"], dev),
              temperature=sdev.f32(pp["temperature"], dev), anchor=sdev.i32(pp["anchor"], dev),
              tokens=sdev.i32(pp["tokens"], dev))
    ws = torch.empty(sd.load().sd_schedule_workspace_size(si.n, si.r, rows, si.m),
                     dtype=torch.uint8, device=dev)

    def pre():
        return sd.sd_schedule_draft(t["ctx_feat"], t["anchor_emb"], t["w_c"], t["w_e"], t["w_o"],
                                    *tab, si.n, b_u=t["b_u"], b_o=t["b_o"],
                                    cal_scale=t["cal_scale"], cal_bias=t["cal_bias"], K=si.K,
                                    workspace=ws)

    def post(o):
        return sd.sd_schedule_verify(tp["hidden"], tp["w_s"], tp["e_pred"], tp["w"],
                                     tp["anchor"], tp["tokens"], o["q_off"], o["verify_budget"],
                                     bias=pp["bias"], temperature=tp["temperature"], K=si.K,
                                     workspace=ws)

    for _ in range(args.warmup):
        post(pre())
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        o = pre()
        ev[i][1].record()
        post(o)
        ev[i][2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pre_us = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    post_us = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    out = {"metric": "draft/verify scheduler latency per step (192 requests)",
           "value": round(float((pre_us + post_us).mean()), 2), "unit": "us",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(elapsed * 1e3 / args.steps, 4), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16/f32",
           "data": "synthetic (seeded estimator weights and inputs, profiled-like latency tables)",
           "config": {"workload": "forespark_scheduler_n192_k16", "requests": si.n, "K": si.K,
                      "d_h": si.d_h, "r": si.r, "selector_dims": si.m, "vocab": si.V},
           "breakdown_us": {"pre_draft_schedule": round(float(pre_us.mean()), 2),
                            "post_draft_budget": round(float(post_us.mean()), 2)}}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload index (default 2: 128K, batch 16)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=16,
                    help="requests of the workload the CPU oracle is timed on")
    ap.add_argument("--calibrate-copy", type=float, default=0.0,
                    help="GiB: also run a plain device copy of this size (PMC calibration)")
    ap.add_argument("--path", choices=sorted(PATHS), default="full",
                    help="attention context: full prefix (default), LongSpark fixed-cost "
                         "(window 256 + 16 summary entries), H-Spec (causal block, window "
                         "2048, 32,000-token drafter vocabulary), LongSpark fixed-cost with "
                         "the rank-256 sequential correction, DeLS-Spec fusion (full prefix, "
                         "Markov local head of rank 256, alpha = beta = 0.3)")
    ap.add_argument("--greedy", action="store_true", help="temperature 0 on both sides")
    ap.add_argument("--target-sigma", type=float, default=0.0,
                    help="for a drafter-plus-noise target: one noise sigma for every request "
                         "(e.g. 0.5) instead of the workload's per-request spread")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured HBM-read and MFMA ceilings (library probes, untimed) "
                         "and the library-GEMM reference of the LM head")
    ap.add_argument("--schedule", action="store_true",
                    help="time the draft / verification scheduler instead of the step "
                         "(192 requests, K = 16, d_h = 4096, r = 256)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the step is not sharded across GPUs "
                                   "(each GPU would run its own requests or KV heads)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.schedule:
        bench_schedule(args)
        return

    import block_drafting_sd_amd as sd
    from block_drafting_sd_amd.step import DraftVerifyStep, StepOptions, StepShape
    from synth import StepInputs, by_index, device as sdev

    sd.load()
    dev = torch.device("cuda:0")
    cfg = by_index(args.config)
    if args.target_sigma > 0:
        if cfg.target[0] != "drafter_plus_noise":
            print("--target-sigma applies to drafter-plus-noise targets only", file=sys.stderr)
            sys.exit(2)
        sg = args.target_sigma
        cfg = cfg.with_(name=f"{cfg.name}_sigma{sg:g}", target=("drafter_plus_noise", sg, sg))
    inp = StepInputs(cfg)
    b = inp.budgets
    t_gen = time.perf_counter()
    log(f"[bench] generating inputs for {cfg.name} ...")
    t = {}
    t.update(sdev.attention_tensors(inp, dev))
    t.update(sdev.lm_head_tensors(inp, dev))
    shape = StepShape(batch=cfg.batch, total_q=inp.total_q,
                      total_target_rows=inp.total_target_rows, num_heads_q=cfg.num_heads_q,
                      num_heads_kv=cfg.num_heads_kv, head_dim=cfg.head_dim, hidden=cfg.hidden,
                      vocab=cfg.vocab, max_total_ctx=inp.max_total_ctx,
                      max_draft_k=int(b.draft_k.max()), split_tokens=args.split_tokens)
    opts = StepOptions(greedy=args.greedy, **PATHS[args.path])
    step = DraftVerifyStep(shape, dev, opts)
    seed = inp.philox_seed
    extra = {}
    if opts.n_summary:
        # the fold appends rows ctx_len_prev .. ctx_len_prev + a_b: the last
        # K_max + 1 rows of each prefix stand in for the round's new rows
        extra["u"] = inp.summary_queries(opts.n_summary)
        extra["ctx_prev"] = np.maximum(b.ctx_len - (int(b.draft_k.max()) + 1), 0).astype(np.int32)
        t["summary_keys"] = sdev.bf16(extra["u"], dev)
        t["ctx_len_prev"] = sdev.i32(extra["ctx_prev"], dev)
    if opts.draft_vocab:
        extra["vmap"] = inp.pruned_vocab(opts.draft_vocab)
        extra["vinv"] = np.full(cfg.vocab, -1, np.int32)
        extra["vinv"][extra["vmap"]] = np.arange(opts.draft_vocab, dtype=np.int32)
        t["vocab_map"] = sdev.i32(extra["vmap"], dev)
        t["vocab_inv"] = sdev.i32(extra["vinv"], dev)
    if opts.markov_rank:
        extra["w_c"], extra["e_c"] = inp.markov_tables(opts.markov_rank)
        extra["anchor"] = inp.anchor_tokens()
        t["markov_w_c"] = sdev.bf16(extra["w_c"], dev)
        t["markov_e_c"] = sdev.bf16(extra["e_c"], dev)
        t["anchor"] = sdev.i32(extra["anchor"], dev)
    if opts.prior_beta:
        # fixed vocabulary bias from corpus counts (setup, untimed)
        extra["counts"] = inp.unigram_counts()
        t["vocab_bias"] = sd.sd_log_prior_bias(torch.from_numpy(extra["counts"]).to(dev),
                                               lam=1.0, scale=-opts.prior_beta)
    if cfg.target[0] == "normal":
        t.update(sdev.verify_tensors(inp, dev))
    else:
        # drafter-plus-noise target: seeded noise on this library's own
        # drafter logits of the same inputs (input preparation, untimed)
        step.lm_head(t, seed)
        torch.cuda.synchronize()
        t.update(sdev.verify_tensors(inp, dev, inp.target_from_drafter(step.logits.cpu().numpy())))
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t_gen:.1f}s)")

    if args.calibrate_copy > 0:
        copy_calibration(args.calibrate_copy)

    init = None
    if opts.n_summary:
        # state before the first step (setup, outside the timed steps); a
        # second, warm call is timed on its own: it reads every prefix row once
        step.summary_init(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step.summary_init(t)
        e1.record()
        torch.cuda.synchronize()
        init_ms = e0.elapsed_time(e1)
        init_bytes = (int(t["ctx_len_prev"].to(torch.int64).sum().item()) * cfg.num_heads_kv
                      * cfg.head_dim * 2 * 2)
        init = {"summary_init_ms": round(init_ms, 4), "prefix_kv_bytes": init_bytes,
                "read_gbs": round(init_bytes / (init_ms * 1e-3) / 1e9, 1)}
        log(f"[bench] summary initialisation {init_ms:.3f} ms ({init['read_gbs']} GB/s)")
    for i in range(args.warmup):
        step.run(t, seed + i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # HIP events on the calls' stream mark the stage boundaries.  Each record
    # costs a few microseconds of idle GPU between kernels, so only the
    # boundaries of stages that run are recorded, and a step's first event
    # also closes the previous step's last stage (one more event ends the
    # timed region).
    stages = ["attention", "lm_head"] + (["markov"] if opts.markov_rank else []) + ["verify"] + \
             (["summary_fold"] if opts.n_summary else [])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in stages] for _ in range(args.steps)]
    ev_end = torch.cuda.Event(enable_timing=True)
    run_stage = {"attention": lambda i: step.attention(t),
                 "lm_head": lambda i: step.lm_head(t, seed + 1000 + i),
                 "markov": lambda i: step.markov(t, seed + 1000 + i),
                 "verify": lambda i: step.verify(t, seed + 1000 + i),
                 "summary_fold": lambda i: step.summary_fold(t)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for e, name in zip(ev[i], stages):
            e.record()
            run_stage[name](i)
    ev_end.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f}s")

    # Emitted tokens (sum_b (a_b + 1), the committed tokens of a round): every
    # timed step used its own seed, so the steps are replayed untimed, in the
    # same order, and their accepted lengths read back one by one.
    emitted_steps = []
    for i in range(args.steps):
        for name in stages:
            run_stage[name](i)
        emitted_steps.append(int(step.accepted.sum().item()) + cfg.batch)
    emitted_total = int(sum(emitted_steps))

    peaks = None if args.no_peaks else measured_peaks(dev)
    lib_gemm = (library_gemm(t["hidden"], t["w_vocab"])
                if not args.no_peaks and not opts.draft_vocab else None)
    bounds = [e for row in ev for e in row] + [ev_end]
    durs = [bounds[k].elapsed_time(bounds[k + 1]) for k in range(len(bounds) - 1)]
    stage_ms = {name: np.array(durs[j::len(stages)]) for j, name in enumerate(stages)}
    zero = np.zeros(args.steps)
    attn_ms, lm_ms, ver_ms = stage_ms["attention"], stage_ms["lm_head"], stage_ms["verify"]
    mk_ms = stage_ms.get("markov", zero)
    fold_ms = stage_ms.get("summary_fold", zero)
    tokens_per_step = int(b.draft_k.sum())
    ms_per_step = elapsed * 1e3 / args.steps
    value = tokens_per_step * args.steps / elapsed

    c = cfg
    n_read = b.ctx_len.astype(np.int64)
    if opts.window:
        n_read = np.minimum(n_read, opts.window)
    kv_bytes = int(n_read.sum()) * c.num_heads_kv * c.head_dim * 2 * 2
    blk_bytes = inp.total_q * c.num_heads_kv * c.head_dim * 2 * 2
    q_out_bytes = 2 * inp.total_q * c.num_heads_q * c.head_dim * 2
    sum_bytes = (c.num_heads_kv * opts.n_summary * c.head_dim * (2 + 4 * c.batch)
                 if opts.n_summary else 0)
    attn_bytes = kv_bytes + blk_bytes + q_out_bytes + sum_bytes
    attn_avg_s = float(attn_ms.mean()) * 1e-3
    attn_gbs = attn_bytes / attn_avg_s / 1e9
    v_draft = opts.draft_vocab or c.vocab
    lm_flops = 2.0 * inp.total_q * c.hidden * v_draft
    lm_tflops = lm_flops / (float(lm_ms.mean()) * 1e-3) / 1e12

    out = {
        "metric": "drafted+verified tokens/s at 128K ctx, batch 16; attn HBM GB/s % of peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs of the workload's shapes; no trained weights)",
        "config": {"workload": c.name, "batch": c.batch, "prefix_tokens": int(b.ctx_len.max()),
                   "draft_k": int(b.draft_k.max()), "num_heads_q": c.num_heads_q,
                   "num_heads_kv": c.num_heads_kv, "head_dim": c.head_dim,
                   "page_size": c.page_size, "hidden": c.hidden, "vocab": c.vocab,
                   "split_tokens": args.split_tokens or "auto", "path": args.path,
                   "greedy": bool(args.greedy), "window": opts.window,
                   "summary_entries": opts.n_summary, "causal_block": opts.causal_block,
                   "draft_vocab": v_draft, "markov_rank": opts.markov_rank,
                   "markov_alpha": opts.markov_alpha, "prior_beta": opts.prior_beta},
        "roofline": {"kernel": "sd_draft_attn call: attn_splitk + attn_combine (+ attn_worklist "
                               "above 64 requests; attn_splitk alone when each request fits one split)",
                     "bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.path == "full" and args.config == 2
                     else None,
                     "algorithmic_bytes": attn_bytes,
                     "avg_ms": round(float(attn_ms.mean()), 4),
                     "measured_peak": peaks and peaks["hbm_read_gbs"],
                     "frac_of_measured": peaks and round(attn_gbs / peaks["hbm_read_gbs"], 4)},
        "breakdown_ms": {"attention": round(float(attn_ms.mean()), 4),
                         "lm_head": round(float(lm_ms.mean()), 4),
                         "markov": round(float(mk_ms.mean()), 4),
                         "verify": round(float(ver_ms.mean()), 4),
                         "summary_fold": round(float(fold_ms.mean()), 4)},
        "breakdown_median_ms": {k: round(float(np.median(v)), 4)
                                for k, v in (("attention", attn_ms), ("lm_head", lm_ms),
                                             ("verify", ver_ms))},
        "breakdown_p10_p90_ms": {k: [round(float(np.percentile(v, 10)), 4),
                                     round(float(np.percentile(v, 90)), 4)]
                                 for k, v in (("attention", attn_ms), ("lm_head", lm_ms),
                                              ("verify", ver_ms))},
        "lm_head": {"tflops": round(lm_tflops, 1),
                    "frac_mfma_bf16": round(lm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "frac_of_measured_mfma": peaks and round(lm_tflops / peaks["mfma_bf16_tflops"], 4),
                    "w_hbm_gbs": round(v_draft * c.hidden * 2 / (float(lm_ms.mean()) * 1e-3) / 1e9, 1),
                    "library_gemm": lib_gemm},
        "measured_peaks": peaks,
        "setup": init,
        # secondary metric: committed tokens (accepted drafts + the correction
        # or bonus token of every request) per second of the same timed steps
        "emitted_tokens_per_s": round(emitted_total / elapsed, 1),
        "emitted_tokens_per_step_mean": round(emitted_total / args.steps, 3),
        # one drafter attention layer per step is timed; projections for the
        # 3 attention modules of "H-Spec" and the 5 draft layers of "LongSpark"
        "projection_tokens_per_s": {
            f"{L}_layers": round(tokens_per_step / ((L * float(attn_ms.mean()) + float(lm_ms.mean())
                                                      + float(mk_ms.mean()) + float(ver_ms.mean())
                                                      + float(fold_ms.mean())) * 1e-3), 1)
            for L in (3, 5)},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(
            inp, args.cpu_requests,
            None if cfg.target[0] == "normal" else t["target_logits"].cpu().numpy(),
            opts, extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
