"""Global context summary of the fixed-cost drafter (fp64).

Test infrastructure (see ``oracle/__init__``): never imported by the product.

"LongSpark", sec. 2.2, eq. (5): for fixed summary queries U (per KV head),
the summary values are the attention of U over every retained target KV row,
Z_t = Attn(U, K_{1:t}, V_{1:t}).  App. A.2, eq. (10): for a set of rows R,
c_R = log sum_{i in R} exp(s_i) and Z_R = sum_{i in R} exp(s_i - c_R) v_i
with s_i = u . k_i * scale; eq. (11): disjoint sets merge as
c = log(e^c_A + e^c_B), Z = e^(c_A - c) Z_A + e^(c_B - c) Z_B, and an empty
new set leaves the state unchanged.  After verification the committed token
and the accepted drafts (a_b + 1 rows) are folded in (sec. 2.2, Fig. 3).

The summary is kept per KV head (a reading: the pages count the entries per
layer and attention head, and the entries act as extra keys and values of the
draft attention, which are per KV head under grouped-query attention).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_lse, bf16_bits_to_f64, gather_prefix, lse_merge


def summary_of_rows(u_bits, k_bits, v_bits, scale: float):
    """(Z [S, D], c [S]) of summary queries ``u`` over rows ``k, v`` (bf16
    bits), eq. (10); the empty set gives (0, -inf)."""
    S, D = u_bits.shape
    if len(k_bits) == 0:
        return np.zeros((S, D)), np.full(S, -np.inf)
    return attention_lse(bf16_bits_to_f64(u_bits), bf16_bits_to_f64(k_bits),
                         bf16_bits_to_f64(v_bits), scale)


def fold(z, c, z_new, c_new):
    """Merge a stored state with the statistics of new rows, eq. (11); an
    empty side (c = -inf) contributes nothing."""
    z = np.asarray(z, np.float64)
    c = np.asarray(c, np.float64)
    out_z, out_c = z.copy(), c.copy()
    for i in range(len(c)):
        if c_new[i] == -np.inf:
            continue
        if c[i] == -np.inf:
            out_z[i], out_c[i] = z_new[i], c_new[i]
            continue
        zi, ci = lse_merge(z[i][None], np.array([c[i]]), z_new[i][None], np.array([c_new[i]]))
        out_z[i], out_c[i] = zi[0], ci[0]
    return out_z, out_c


def summary_init(u, k_cache, v_cache, page_table, ctx_len, num_heads_kv: int, scale: float):
    """Summary of every request's whole prefix: (Z [B, Hkv, S, D], c [B, Hkv, S])."""
    B = len(ctx_len)
    S, D = u.shape[1], u.shape[2]
    Z = np.zeros((B, num_heads_kv, S, D))
    C = np.full((B, num_heads_kv, S), -np.inf)
    for b in range(B):
        n = int(ctx_len[b])
        for g in range(num_heads_kv):
            k, v = gather_prefix(k_cache, v_cache, page_table[b], n, g)
            Z[b, g], C[b, g] = summary_of_rows(u[g], k, v, scale)
    return Z, C


def summary_update(u, k_cache, v_cache, page_table, ctx_len, accepted, Z, C,
                   num_heads_kv: int, scale: float):
    """Fold rows N_b .. N_b + a_b of every request into (Z, C), eq. (11)."""
    Z = np.array(Z, np.float64)
    C = np.array(C, np.float64)
    for b in range(len(ctx_len)):
        n, a = int(ctx_len[b]), int(accepted[b])
        for g in range(num_heads_kv):
            k, v = gather_prefix(k_cache, v_cache, page_table[b], n + a + 1, g)
            z_new, c_new = summary_of_rows(u[g], k[n:], v[n:], scale)
            Z[b, g], C[b, g] = fold(Z[b, g], C[b, g], z_new, c_new)
    return Z, C
