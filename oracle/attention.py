"""Draft-block attention over the target's paged prefix KV cache (fp64).

Test infrastructure (see ``oracle/__init__``): never imported by the product.

What is computed, per request b, KV head g and query head h of g's group:
every one of the request's K_b draft query rows attends, with one softmax and
no mask, to (i) all N_b prefix keys of the target's cache for head g, read in
place through the page table, and (ii) all K_b keys of the draft block itself,
its own row included.

* Bidirectional attention inside the block: "ForeSpark", sec. 1 and sec. 4.1
  (each draft layer attends bidirectionally to all draft positions and to the
  context, which enters only as extra keys and values); "LongSpark",
  App. A.1, Fig. 6 (one attention normalisation across the sources,
  bidirectional among local slots).
* Target KV reused in place, dimensions equal to the target's, one target
  layer per draft layer; block Q/K carry RoPE positions that continue the
  prefix, so the cache and the block arrive post-RoPE: "H-Spec", sec. 3.3.2.
* Full prefix (no window): the prefix-reading drafters the pages compare
  against read the whole prefix ("LongSpark", sec. 1 and Fig. 1).

Variants (keyword arguments of ``draft_attn``):

* ``window=W``: only the last W prefix rows are keys and values -- the
  recent window of the fixed-cost drafter ("LongSpark", sec. 2.2, eq. (6)),
  and the sliding window of "H-Spec", sec. 3.3.2, read here as one window
  shared by all rows of the block.
* ``summary_keys`` / ``summary_values``: the context summary enters as extra
  rows, summary queries as keys and summary values as values, under the
  same normalisation ("LongSpark", sec. 2.2, eq. (6)).  The values enter
  rounded to bf16 like every other value row (a reading: the pages do not fix
  the precision the attention consumes them in).
* ``block_mask="causal"``: block row j sees block rows 0..j only; prefix and
  summary rows stay visible ("H-Spec", sec. 3.3.2, causal attention over the
  masked block with the target KV as prefix context).
* Scores are q.k / sqrt(d): "LongSpark", App. A.2, eq. (10).
* Query head h reads KV head h // (Hq / Hkv) (grouped-query attention; the
  pages do not spell out the mapping).

``attention_lse`` and ``lse_merge`` restate "LongSpark" App. A.2 eqs. (10)
and (11); the merge is what a split-K kernel uses to combine partial results.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def gather_prefix(k_cache: np.ndarray, v_cache: np.ndarray,
                  page_table_row: np.ndarray, n_tokens: int, kv_head: int):
    """Logical prefix keys / values ``[n_tokens, D]`` (bf16 bits) of one KV
    head, read from the documented page layouts:
    ``k_cache[page, head, c, slot, e]`` is dim ``8c + e`` of the token in
    ``slot``; ``v_cache[page, head, d, slot]`` is dim ``d`` of that token."""
    P = k_cache.shape[3]
    D = k_cache.shape[2] * k_cache.shape[4]
    n_pages = (n_tokens + P - 1) // P
    pages = np.asarray(page_table_row[:n_pages], np.int64)
    kp = k_cache[pages, kv_head]                    # [n, D/8, P, 8]
    k = kp.transpose(0, 2, 1, 3).reshape(n_pages * P, D)
    vp = v_cache[pages, kv_head]                    # [n, D, P]
    v = vp.transpose(0, 2, 1).reshape(n_pages * P, D)
    return k[:n_tokens], v[:n_tokens]


def attention_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of rows ``q [m, D]`` over keys ``k [n, D]`` and values
    ``v [n, D]`` with no mask.  Returns ``(z [m, D], lse [m])`` where
    ``lse = log sum_i exp(s_i)`` and ``z = sum_i exp(s_i - lse) v_i``
    ("LongSpark", App. A.2, eq. (10)), evaluated with max subtraction."""
    s = (q @ k.T) * scale
    mx = s.max(axis=1, keepdims=True)
    w = np.exp(s - mx)
    l = w.sum(axis=1, keepdims=True)
    return (w @ v) / l, (mx + np.log(l))[:, 0]


def lse_merge(z_a, lse_a, z_b, lse_b):
    """Merge the statistics of two disjoint key sets ("LongSpark", App. A.2,
    eq. (11)): ``lse = log(e^lse_a + e^lse_b)``,
    ``z = e^(lse_a - lse) z_a + e^(lse_b - lse) z_b``."""
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    mx = np.maximum(lse_a, lse_b)
    lse = mx + np.log(np.exp(lse_a - mx) + np.exp(lse_b - mx))
    wa = np.exp(lse_a - lse)[..., None]
    wb = np.exp(lse_b - lse)[..., None]
    return wa * z_a + wb * z_b, lse


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, nearest even (finite
    inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def masked_attention(q, k, v, scale, visible):
    """Softmax attention of ``q [m, D]`` over the keys ``k [n, D]`` that
    ``visible [m, n]`` (bool) marks for each row; masked keys get weight 0."""
    s = np.where(visible, (q @ k.T) * scale, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    w = np.exp(s - mx)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def draft_attn(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, q_off,
               num_heads_kv: int, softmax_scale: float, requests=None,
               block_mask: str = "none", window: int = 0, summary_keys=None,
               summary_values=None):
    """Attention output ``[total_q, Hq, D]`` (float64) for every draft row.

    Inputs are the bf16 bit patterns the kernel receives (``summary_values``
    is fp32 ``[batch, Hkv, S, D]``, ``summary_keys`` bf16 bits
    ``[Hkv, S, D]``).  ``requests`` restricts the work to a subset of
    requests (other rows stay NaN)."""
    assert block_mask in ("none", "causal")
    total_q, Hq, D = q.shape
    G = Hq // num_heads_kv
    out = np.full((total_q, Hq, D), np.nan)
    B = len(ctx_len)
    for b in (range(B) if requests is None else requests):
        r0, r1 = int(q_off[b]), int(q_off[b + 1])
        if r1 == r0:
            continue
        kb = r1 - r0
        n = int(ctx_len[b])
        n0 = max(0, n - window) if window > 0 else 0
        for g in range(num_heads_kv):
            kp, vp = gather_prefix(k_cache, v_cache, page_table[b], n, g)
            ks = [kp[n0:], k_blk[r0:r1, g]]
            vs = [vp[n0:], v_blk[r0:r1, g]]
            n_sum = 0
            if summary_keys is not None:
                n_sum = summary_keys.shape[1]
                ks.append(summary_keys[g])
                vs.append(f32_to_bf16_bits(summary_values[b, g]))
            k_all = bf16_bits_to_f64(np.concatenate(ks, 0))
            v_all = bf16_bits_to_f64(np.concatenate(vs, 0))
            n_pre = n - n0
            visible = np.ones((kb, n_pre + kb + n_sum), bool)
            if block_mask == "causal":
                visible[:, n_pre:n_pre + kb] = np.tril(np.ones((kb, kb), bool))
            for h in range(g * G, (g + 1) * G):
                out[r0:r1, h] = masked_attention(bf16_bits_to_f64(q[r0:r1, h]), k_all,
                                                 v_all, softmax_scale, visible)
    return out
