"""Block-parallel speculative draft-and-verify step for AMD MI355X (gfx950).

Thin Python binding over the C ABI declared in ``include/sd.h``; the
functions keep the C names.  PyTorch supplies device memory and the stream;
arguments are checked for dtype / contiguity / device and passed as raw
pointers.  All computation happens in ``libsd_amd.so``.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from ._lib import LIB_PATH, SdError, check, load  # noqa: F401

SD_MASK_NONE, SD_MASK_CAUSAL = 0, 1

__all__ = ["sd_draft_attn", "sd_draft_attn_noalloc", "sd_summary_update", "sd_lm_head_probs", "sd_markov_sample",
           "sd_verify",
           "sd_schedule_draft", "sd_schedule_verify", "sd_version",
           "SD_MASK_NONE", "SD_MASK_CAUSAL",
           "draft_attn_workspace_size", "lm_head_workspace_size",
           "summary_workspace_size", "verify_workspace_size", "SdError", "load"]


def _req(t: torch.Tensor, name: str, dtypes, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _need(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """Device arrays are never read on the host, so the library cannot check
    their lengths: the binding does."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} entries, needs at least {n}")


_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_U32 = (torch.int32, torch.uint32)
_F32 = (torch.float32,)


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def sd_version() -> str:
    return load().sd_version().decode()


def sd_probe_read(src, sink=None, stream=None):
    """Stream every byte of the device tensor ``src`` with plain loads
    (HBM read ceiling); see include/sd.h.  Returns the sink tensor."""
    lib = load()
    if not isinstance(src, torch.Tensor) or not src.is_contiguous():
        raise TypeError("src must be a contiguous torch.Tensor")
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=src.device)
    check("sd_probe_read", lib.sd_probe_read(_ptr(src), src.numel() * src.element_size(),
                                             _ptr(sink), _stream_handle(stream)))
    return sink


def sd_probe_mfma(iters: int, sink=None, device=None, stream=None):
    """Back-to-back independent bf16 MFMAs on every CU (MFMA ceiling).
    Returns the flop count of the launch."""
    lib = load()
    if sink is None:
        sink = torch.zeros(4, dtype=torch.float32, device=device or "cuda")
    check("sd_probe_mfma", lib.sd_probe_mfma(int(iters), _ptr(sink), _stream_handle(stream)))
    return int(lib.sd_probe_mfma_flops(int(iters)))


def draft_attn_workspace_size(batch, num_heads_q, num_heads_kv, head_dim, max_draft_k,
                              max_total_ctx, split_tokens=0) -> int:
    return int(load().sd_draft_attn_workspace_size(batch, num_heads_q, num_heads_kv, head_dim,
                                                   max_draft_k, max_total_ctx, split_tokens))


def lm_head_workspace_size(M, V) -> int:
    return int(load().sd_lm_head_workspace_size(M, V))


def markov_workspace_size(batch, V, max_draft_k) -> int:
    return int(load().sd_markov_workspace_size(batch, V, max_draft_k))


def summary_workspace_size(batch, num_heads_kv, n_summary, head_dim, max_pages,
                           page_size=16) -> int:
    return int(load().sd_summary_workspace_size(batch, num_heads_kv, n_summary, head_dim,
                                                max_pages, page_size))


def verify_workspace_size(batch, total_q, total_target_rows, V) -> int:
    return int(load().sd_verify_workspace_size(batch, total_q, total_target_rows, V))


def _workspace(ws, nbytes, device):
    if ws is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel() * ws.element_size()} < {nbytes}")
    return ws


def sd_draft_attn(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, q_off, *,
                  max_draft_k: int, max_total_ctx: int, softmax_scale: Optional[float] = None,
                  split_tokens: int = 0, block_mask: int = SD_MASK_NONE, window: int = 0,
                  summary_keys=None, summary_values=None, out=None, workspace=None,
                  stream=None):
    """Draft-block attention; see ``sd_draft_attn`` in include/sd.h."""
    lib = load()
    dev = q.device
    _req(q, "q", _BF16, dev)
    _req(k_blk, "k_blk", _BF16, dev)
    _req(v_blk, "v_blk", _BF16, dev)
    _req(k_cache, "k_cache", _BF16, dev)
    _req(v_cache, "v_cache", _BF16, dev)
    _req(page_table, "page_table", _I32, dev)
    _req(ctx_len, "ctx_len", _I32, dev)
    _req(q_off, "q_off", _I32, dev)
    total_q, hq, D = q.shape
    hkv = k_blk.shape[1]
    num_pages, _, _, page_size, _ = k_cache.shape
    batch, max_pages = page_table.shape
    _need(ctx_len, batch, "ctx_len")
    _need(q_off, batch + 1, "q_off")
    if tuple(k_blk.shape) != (total_q, hkv, D) or tuple(v_blk.shape) != (total_q, hkv, D):
        raise ValueError("k_blk and v_blk must be [total_q, Hkv, D]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    nbytes = lib.sd_draft_attn_workspace_size(batch, hq, hkv, D, max_draft_k, max_total_ctx,
                                              split_tokens)
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.numel(), "out")
    n_summary = 0
    if summary_keys is not None or summary_values is not None:
        _req(summary_keys, "summary_keys", _BF16, dev)
        _req(summary_values, "summary_values", _F32, dev)
        n_summary = summary_keys.shape[1]
        if tuple(summary_keys.shape) != (hkv, n_summary, D) or \
                tuple(summary_values.shape) != (batch, hkv, n_summary, D):
            raise ValueError("summary_keys must be [Hkv, S, D] and summary_values [batch, Hkv, S, D]")
    st = lib.sd_draft_attn(_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache),
                           _ptr(page_table), _ptr(ctx_len), _ptr(q_off), batch, total_q,
                           max_draft_k, num_pages, max_pages, page_size, hq, hkv, D,
                           int(max_total_ctx), int(split_tokens), float(softmax_scale),
                           int(block_mask), int(window), _ptr(summary_keys),
                           _ptr(summary_values), n_summary,
                           _ptr(out), _ptr(workspace), workspace.numel(), _stream_handle(stream))
    check("sd_draft_attn", st)
    return out


def sd_draft_attn_noalloc(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, q_off, *,
                          max_draft_k: int, max_total_ctx: int,
                          softmax_scale: Optional[float] = None, split_tokens: int = 0,
                          block_mask: int = SD_MASK_NONE, window: int = 0, summary_keys=None,
                          summary_values=None, out=None, stream=None):
    """Draft-block attention for callers that cannot allocate: the library's
    own per-GPU scratch array instead of a workspace; see
    ``sd_draft_attn_noalloc`` in include/sd.h.  ``out`` must be given (this
    entry point exists for code that allocates nothing)."""
    lib = load()
    dev = q.device
    for t, nm in ((q, "q"), (k_blk, "k_blk"), (v_blk, "v_blk"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _req(t, nm, _BF16, dev)
    for t, nm in ((page_table, "page_table"), (ctx_len, "ctx_len"), (q_off, "q_off")):
        _req(t, nm, _I32, dev)
    if out is None:
        raise ValueError("out must be given (the no-allocation entry point allocates nothing)")
    _req(out, "out", _BF16, dev)
    total_q, hq, D = q.shape
    hkv = k_blk.shape[1]
    num_pages, _, _, page_size, _ = k_cache.shape
    batch, max_pages = page_table.shape
    _need(ctx_len, batch, "ctx_len")
    _need(q_off, batch + 1, "q_off")
    _need(out, q.numel(), "out")
    if tuple(k_blk.shape) != (total_q, hkv, D) or tuple(v_blk.shape) != (total_q, hkv, D):
        raise ValueError("k_blk and v_blk must be [total_q, Hkv, D]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    n_summary = 0
    if summary_keys is not None or summary_values is not None:
        _req(summary_keys, "summary_keys", _BF16, dev)
        _req(summary_values, "summary_values", _F32, dev)
        n_summary = summary_keys.shape[1]
        if tuple(summary_keys.shape) != (hkv, n_summary, D) or \
                tuple(summary_values.shape) != (batch, hkv, n_summary, D):
            raise ValueError("summary_keys must be [Hkv, S, D] and summary_values [batch, Hkv, S, D]")
    st = lib.sd_draft_attn_noalloc(_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(page_table), _ptr(ctx_len), _ptr(q_off),
                                   batch, total_q, max_draft_k, num_pages, max_pages, page_size,
                                   hq, hkv, D, int(max_total_ctx), int(split_tokens),
                                   float(softmax_scale), int(block_mask), int(window),
                                   _ptr(summary_keys), _ptr(summary_values), n_summary,
                                   _ptr(out), _stream_handle(stream))
    check("sd_draft_attn_noalloc", st)
    return out


def sd_summary_update(summary_queries, k_cache, v_cache, page_table, ctx_len, accepted_len,
                      summary_values, summary_lse, *, softmax_scale: Optional[float] = None,
                      workspace=None, stream=None):
    """Fold retained target KV rows into the context summary (in place); see
    ``sd_summary_update`` in include/sd.h.  ``accepted_len=None`` initialises
    the summary from each request's whole prefix (with ``workspace`` of
    ``summary_workspace_size`` bytes, allocated here when None)."""
    lib = load()
    dev = summary_queries.device
    _req(summary_queries, "summary_queries", _BF16, dev)
    _req(k_cache, "k_cache", _BF16, dev)
    _req(v_cache, "v_cache", _BF16, dev)
    _req(page_table, "page_table", _I32, dev)
    _req(ctx_len, "ctx_len", _I32, dev)
    if accepted_len is not None:
        _req(accepted_len, "accepted_len", _I32, dev)
    _req(summary_values, "summary_values", _F32, dev)
    _req(summary_lse, "summary_lse", _F32, dev)
    hkv, n_summary, D = summary_queries.shape
    num_pages, _, _, page_size, _ = k_cache.shape
    batch, max_pages = page_table.shape
    if tuple(summary_values.shape) != (batch, hkv, n_summary, D) or \
            tuple(summary_lse.shape) != (batch, hkv, n_summary):
        raise ValueError("summary_values must be [batch, Hkv, S, D] and summary_lse [batch, Hkv, S]")
    _need(ctx_len, batch, "ctx_len")
    _need(accepted_len, batch, "accepted_len")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    ws, ws_bytes = None, 0
    if accepted_len is None:   # an initialisation keeps its pieces' partial states there
        ws = _workspace(workspace, summary_workspace_size(batch, hkv, n_summary, D, max_pages,
                                                          page_size), dev)
        ws_bytes = ws.numel() * ws.element_size()
    st = lib.sd_summary_update(_ptr(summary_queries), _ptr(k_cache), _ptr(v_cache),
                               _ptr(page_table), _ptr(ctx_len), _ptr(accepted_len), batch,
                               num_pages, max_pages, page_size, hkv, D, n_summary,
                               float(softmax_scale), _ptr(summary_values), _ptr(summary_lse),
                               _ptr(ws), ws_bytes, _stream_handle(stream))
    check("sd_summary_update", st)
    return summary_values, summary_lse


def sd_lm_head_probs(hidden, w_vocab, q_off, req_id, seed: int, *, vocab_map=None,
                     greedy: bool = False, logits=None, lse=None, draft_tokens=None,
                     workspace=None, stream=None
                     ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """LM head + softmax statistics + draft sampling; see include/sd.h.
    ``vocab_map`` (int32 [V_draft] target ids) prunes the drafter's
    vocabulary; ``greedy`` draws the argmax."""
    lib = load()
    dev = hidden.device
    _req(hidden, "hidden", _BF16, dev)
    _req(w_vocab, "w_vocab", _BF16, dev)
    _req(q_off, "q_off", _I32, dev)
    _req(req_id, "req_id", _U32, dev)
    if vocab_map is not None:
        _req(vocab_map, "vocab_map", _I32, dev)
    M, H = hidden.shape
    w_rows = w_vocab.shape[0]
    V = w_rows if vocab_map is None else vocab_map.numel()
    batch = q_off.numel() - 1
    _need(req_id, batch, "req_id")
    if logits is None:
        logits = torch.empty(M, V, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(M, dtype=torch.float32, device=dev)
    if draft_tokens is None:
        draft_tokens = torch.empty(M, dtype=torch.int32, device=dev)
    _need(logits, M * V, "logits")
    _need(lse, M, "lse")
    _need(draft_tokens, M, "draft_tokens")
    nbytes = lib.sd_lm_head_workspace_size(M, V)
    workspace = _workspace(workspace, nbytes, dev)
    st = lib.sd_lm_head_probs(_ptr(hidden), _ptr(w_vocab), M, H, V, _ptr(q_off), batch,
                              _ptr(req_id), int(seed) & ((1 << 64) - 1), _ptr(vocab_map),
                              w_rows, int(bool(greedy)), _ptr(logits), _ptr(lse),
                              _ptr(draft_tokens), _ptr(workspace), workspace.numel(),
                              _stream_handle(stream))
    check("sd_lm_head_probs", st)
    return logits, lse, draft_tokens


def sd_markov_sample(logits, anchor_tokens, w_c, e_c, q_off, req_id, seed: int, *,
                     max_draft_k: int, alpha: float = 1.0, vocab_bias=None, greedy: bool = False,
                     lse=None, draft_tokens=None, workspace=None, stream=None):
    """Sequential correction of the draft logits (in place) and sampling;
    see ``sd_markov_sample`` in include/sd.h (``alpha`` and ``vocab_bias``
    give the logit fusion).  Returns (logits, lse, tokens)."""
    lib = load()
    dev = logits.device
    _req(logits, "logits", _F32, dev)
    _req(anchor_tokens, "anchor_tokens", _I32, dev)
    _req(w_c, "w_c", _BF16, dev)
    _req(e_c, "e_c", _BF16, dev)
    _req(q_off, "q_off", _I32, dev)
    _req(req_id, "req_id", _U32, dev)
    M, V = logits.shape
    r = w_c.shape[1]
    if tuple(w_c.shape) != (V, r) or tuple(e_c.shape) != (V, r):
        raise ValueError("w_c and e_c must be [V, r]")
    if vocab_bias is not None:
        _req(vocab_bias, "vocab_bias", _F32, dev)
        if vocab_bias.numel() != V:
            raise ValueError("vocab_bias must have V entries")
    batch = q_off.numel() - 1
    _need(anchor_tokens, batch, "anchor_tokens")
    _need(req_id, batch, "req_id")
    if lse is None:
        lse = torch.empty(M, dtype=torch.float32, device=dev)
    if draft_tokens is None:
        draft_tokens = torch.empty(M, dtype=torch.int32, device=dev)
    _need(lse, M, "lse")
    _need(draft_tokens, M, "draft_tokens")
    workspace = _workspace(workspace, markov_workspace_size(batch, V, max_draft_k), dev)
    st = lib.sd_markov_sample(_ptr(logits), _ptr(lse), _ptr(draft_tokens), _ptr(anchor_tokens),
                              _ptr(w_c), _ptr(e_c), float(alpha),
                              None if vocab_bias is None else _ptr(vocab_bias), int(bool(greedy)),
                              _ptr(q_off),
                              batch, M, V, r, int(max_draft_k),
                              _ptr(req_id), int(seed) & ((1 << 64) - 1), _ptr(workspace),
                              workspace.numel(), _stream_handle(stream))
    check("sd_markov_sample", st)
    return logits, lse, draft_tokens


def sd_log_prior_bias(counts, *, lam: float = 1.0, scale: float = -0.3, out=None, stream=None):
    """``scale * log p~_0`` from int64 corpus counts [V] (additive smoothing
    ``lam``); see ``sd_log_prior_bias`` in include/sd.h.  Returns fp32 [V]."""
    lib = load()
    dev = counts.device
    _req(counts, "counts", (torch.int64,), dev)
    V = counts.numel()
    if out is None:
        out = torch.empty(V, dtype=torch.float32, device=dev)
    _req(out, "out", _F32, dev)
    check("sd_log_prior_bias", lib.sd_log_prior_bias(_ptr(counts), V, float(lam), float(scale),
                                                     _ptr(out), _stream_handle(stream)))
    return out


def sd_verify(target_logits, t_off, draft_logits, draft_lse, draft_tokens, q_off, req_id,
              seed: int, *, draft_vocab_inv=None, greedy: bool = False, accepted_len=None,
              next_token=None, accept_ratio=None, want_ratio: bool = True, workspace=None,
              stream=None):
    """Speculative-sampling verification; see include/sd.h.
    ``draft_vocab_inv`` (int32 [V]: drafter entry of each target id or -1)
    declares a pruned drafter vocabulary; ``greedy`` verifies at temperature 0.
    Returns (accepted_len, next_token, accept_ratio or None)."""
    lib = load()
    dev = target_logits.device
    _req(target_logits, "target_logits", _F32, dev)
    _req(t_off, "t_off", _I32, dev)
    _req(draft_logits, "draft_logits", _F32, dev)
    if draft_lse is not None:
        _req(draft_lse, "draft_lse", _F32, dev)
    _req(draft_tokens, "draft_tokens", _I32, dev)
    _req(q_off, "q_off", _I32, dev)
    _req(req_id, "req_id", _U32, dev)
    R, V = target_logits.shape
    total_q = draft_tokens.numel()
    batch = t_off.numel() - 1
    if accepted_len is None:
        accepted_len = torch.empty(batch, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(batch, dtype=torch.int32, device=dev)
    if accept_ratio is None and want_ratio and total_q > 0:
        accept_ratio = torch.empty(total_q, dtype=torch.float32, device=dev)
    nbytes = lib.sd_verify_workspace_size(batch, total_q, R, V)
    workspace = _workspace(workspace, nbytes, dev)
    if draft_logits.dim() != 2:
        raise ValueError("draft_logits must be [total_q, V] (or [total_q, V_draft] with "
                         "draft_vocab_inv)")
    v_draft = draft_logits.shape[1]
    if draft_vocab_inv is None and v_draft != V:
        # without a vocabulary map the library reads draft rows with the
        # target's row length
        raise ValueError(f"draft_logits has rows of {v_draft} entries; without draft_vocab_inv "
                         f"they must have V = {V}")
    if draft_vocab_inv is not None and draft_lse is None:
        raise ValueError("a pruned drafter vocabulary (draft_vocab_inv) needs draft_lse")
    _need(q_off, batch + 1, "q_off")
    _need(req_id, batch, "req_id")
    _need(draft_logits, total_q * v_draft, "draft_logits")
    _need(draft_lse, total_q, "draft_lse")
    _need(accepted_len, batch, "accepted_len")
    _need(next_token, batch, "next_token")
    _need(accept_ratio, total_q, "accept_ratio")
    if draft_vocab_inv is not None:
        _req(draft_vocab_inv, "draft_vocab_inv", _I32, dev)
        _need(draft_vocab_inv, V, "draft_vocab_inv")
    st = lib.sd_verify(_ptr(target_logits), _ptr(t_off), _ptr(draft_logits), _ptr(draft_lse),
                       _ptr(draft_tokens), _ptr(q_off), batch, total_q, R, V,
                       _ptr(draft_vocab_inv), v_draft, int(bool(greedy)), _ptr(req_id),
                       int(seed) & ((1 << 64) - 1), _ptr(accepted_len), _ptr(next_token),
                       _ptr(accept_ratio), _ptr(workspace), workspace.numel(),
                       _stream_handle(stream))
    check("sd_verify", st)
    return accepted_len, next_token, accept_ratio


def _opt_f32(t, name, dev):
    if t is not None:
        _req(t, name, _F32, dev)
    return t


def sd_schedule_draft(ctx_feat, anchor_emb, w_c, w_e, w_o, draft_caps, draft_lat, verify_caps,
                      verify_lat, n_nonspec: int, *, b_u=None, b_o=None, cal_scale=None,
                      cal_bias=None, K: Optional[int] = None, workspace=None, stream=None):
    """Pre-draft estimation and the joint draft / verification schedule; see
    ``sd_schedule_draft`` in include/sd.h.  Returns a dict of device tensors:
    logits, scores, draft_len, q_off, verify_budget, objective."""
    lib = load()
    dev = ctx_feat.device
    for t, nm in ((ctx_feat, "ctx_feat"), (anchor_emb, "anchor_emb"), (w_c, "w_c"),
                  (w_e, "w_e"), (w_o, "w_o")):
        _req(t, nm, _BF16, dev)
    _req(draft_caps, "draft_caps", _I32, dev)
    _req(verify_caps, "verify_caps", _I32, dev)
    _req(draft_lat, "draft_lat", _F32, dev)
    _req(verify_lat, "verify_lat", _F32, dev)
    for t, nm in ((b_u, "b_u"), (b_o, "b_o"), (cal_scale, "cal_scale"), (cal_bias, "cal_bias")):
        _opt_f32(t, nm, dev)
    n, d_h = ctx_feat.shape
    r = w_c.shape[0]
    T = w_o.shape[0]
    if K is None:
        K = int((math.isqrt(8 * T + 1) - 1) // 2)
    if K * (K + 1) // 2 != T:
        raise ValueError(f"w_o has {T} rows, not K(K+1)/2 for K={K}")
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(logits=torch.empty(n, T, **f32), scores=torch.empty(n, K, **f32),
               draft_len=torch.empty(n, **i32), q_off=torch.empty(n + 1, **i32),
               verify_budget=torch.empty(1, **i32), objective=torch.empty(1, **f32))
    workspace = _workspace(workspace, lib.sd_schedule_workspace_size(n, r, 0, 1), dev)
    st = lib.sd_schedule_draft(_ptr(ctx_feat), _ptr(anchor_emb), _ptr(w_c), _ptr(w_e), _ptr(b_u),
                               _ptr(w_o), _ptr(b_o), _ptr(cal_scale), _ptr(cal_bias), n, d_h, r, K,
                               _ptr(draft_caps), _ptr(draft_lat), draft_caps.numel(),
                               _ptr(verify_caps), _ptr(verify_lat), verify_caps.numel(),
                               int(n_nonspec), _ptr(out["logits"]), _ptr(out["scores"]),
                               _ptr(out["draft_len"]), _ptr(out["q_off"]),
                               _ptr(out["verify_budget"]), _ptr(out["objective"]),
                               _ptr(workspace), workspace.numel(), _stream_handle(stream))
    check("sd_schedule_draft", st)
    return out


def sd_schedule_verify(hidden, w_s, e_pred, w, anchor_tokens, draft_tokens, q_off,
                       verify_budget, *, bias: float = 0.0, temperature=None,
                       K: Optional[int] = None, workspace=None, stream=None):
    """Post-draft estimation and budget distribution; see
    ``sd_schedule_verify`` in include/sd.h.  ``hidden`` holds max_rows packed
    draft rows.  Returns a dict: accept_prob, survival, verify_len, t_off."""
    lib = load()
    dev = hidden.device
    for t, nm in ((hidden, "hidden"), (w_s, "w_s"), (e_pred, "e_pred")):
        _req(t, nm, _BF16, dev)
    _req(w, "w", _F32, dev)
    _opt_f32(temperature, "temperature", dev)
    for t, nm in ((anchor_tokens, "anchor_tokens"), (draft_tokens, "draft_tokens"),
                  (q_off, "q_off"), (verify_budget, "verify_budget")):
        _req(t, nm, _I32, dev)
    max_rows, H = hidden.shape
    m = w_s.shape[0]
    V = e_pred.shape[0]
    n = q_off.numel() - 1
    if K is None:
        K = temperature.numel() if temperature is not None else 32
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(accept_prob=torch.empty(max_rows, **f32), survival=torch.empty(max_rows, **f32),
               verify_len=torch.empty(n, **i32), t_off=torch.empty(n + 1, **i32))
    workspace = _workspace(workspace, lib.sd_schedule_workspace_size(1, 1, max_rows, m), dev)
    st = lib.sd_schedule_verify(_ptr(hidden), _ptr(w_s), _ptr(e_pred), _ptr(w), float(bias),
                                _ptr(temperature), _ptr(anchor_tokens), _ptr(draft_tokens),
                                _ptr(q_off), _ptr(verify_budget), n, max_rows, H, m, V, K,
                                _ptr(out["accept_prob"]), _ptr(out["survival"]),
                                _ptr(out["verify_len"]), _ptr(out["t_off"]), _ptr(workspace),
                                workspace.numel(), _stream_handle(stream))
    check("sd_schedule_verify", st)
    return out
