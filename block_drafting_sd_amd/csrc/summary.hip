// Global context summary of the fixed-cost drafter ("LongSpark", sec. 2.2,
// eq. (5), and App. A.2, eqs. (10)-(11)).
//
// Each KV head g of a request keeps, for S fixed summary queries u_i, the
// attention of u_i over every target KV row retained so far:
//     c_i = log sum_t exp(s_it),  Z_i = sum_t exp(s_it - c_i) v_t,
//     s_it = scale * u_i . k_t.
// After verification the a_b + 1 newly retained rows (the committed token
// and the accepted drafts, already written to the target's cache) are folded
// in: their own statistics (c', Z') over the new rows, then the merge of
// eq. (11), c'' = log(e^c + e^c'), Z'' = e^(c - c'') Z + e^(c' - c'') Z'.
// An empty set of new rows leaves the state as it is.
//
// summary_rows: one wavefront per (request, KV head, slice of rows).  The
// rows are walked in 32-token tiles (aligned to 32 tokens; rows outside the
// slice are masked), read in place through the page table with 16-byte
// non-temporal loads straight into MFMA operands; the next tile's loads are
// in flight while the current one is computed.  Per tile and group of 16
// summary queries:
//   * scores^T (32 tokens x 16 queries) = K U^T as two 16x16x32 bf16 MFMA
//     chains over the head dim; the A operand of chain h holds the tokens
//     8 (r / 4) + 4 h + r % 4 for row r, so that each lane's eight scores are
//     the tokens 8 (lane / 16) + [0, 8) of its query (lane % 16);
//   * an online softmax in base 2 (running max per query over the four
//     lanes of a column, sums kept per lane until the end);
//   * O (16 queries x D) += P V with P as the A operand straight from the
//     scores' registers and V's 16-byte loads (8 consecutive tokens of one
//     dim) as B.  P enters as a bf16 pair hi + lo (hi = bf16(p),
//     lo = bf16(p - hi)), two MFMAs per product, so the weights keep
//     ~2^-18 relative error; every sum is fp32.
// A fold (one slice: the new rows) merges its result into the stored state
// with eq. (11).  Initialising from whole prefixes splits the concatenation
// of every (request, KV head)'s rows into kSummaryInitWaves equal runs, one
// per wave, whatever the lengths (concat_size / find_request); each piece of
// a (request, KV head) that a wave covers leaves its partial state (max, sum,
// unnormalised O) in the workspace, and summary_merge combines a pair's
// pieces with the same rule.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kTile = 32;        // tokens per wave step
constexpr int kMergeThreads = 256;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D>
struct Tile {
  u32x4 k[2][D / 32];   // score chain h, k-step over the head dim
  u32x4 v[D / 16];      // value columns 16 nb + (lane % 16)
};

// A whole-prefix initialisation walks the concatenation of every (request,
// KV head)'s rows: request b's KV head g owns rows P_b + g N_b .. P_b +
// (g + 1) N_b, P_b = hkv * sum_{b' < b} N_b'.  Wave w takes rows w T ..
// (w + 1) T, T = max(kSummaryMinSplit, ceil(total / kSummaryInitWaves)), so
// every wave has the same work whatever the lengths; the piece of pair p that
// wave w covers goes to slot p + w (both grow along the rows, so no two
// pieces share a slot, and slots stay below B * hkv + kSummaryInitWaves).

// total rows (hkv * sum_b N_b) and T, the same in every wave
__device__ void concat_size(const SummaryArgs& a, int lane, long long& total, long long& T) {
  const int n_max = a.max_pages * 16;
  long long s = 0;
  for (int b = lane; b < a.batch; b += 64) s += clampi(a.ctx_len[b], 0, n_max);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  total = s * a.hkv;
  T = (total + kSummaryInitWaves - 1) / kSummaryInitWaves;
  T = T < kSummaryMinSplit ? kSummaryMinSplit : T;
}

// Request b and its first row P_b: with row >= 0 the request whose rows hold
// `row` (false past the last row); with row < 0 request `want`.
__device__ bool find_request(const SummaryArgs& a, long long row, int want, int lane, int& b,
                             long long& pb) {
  const int n_max = a.max_pages * 16;
  long long base = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int bb = b0 + lane;
    const long long rows = bb < a.batch ? static_cast<long long>(clampi(a.ctx_len[bb], 0, n_max)) * a.hkv : 0;
    long long incl = rows;                              // inclusive scan over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const long long chunk = __shfl(incl, 63, 64);
    int l = -1;
    if (row >= 0) {
      if (row < base + chunk) l = __ffsll(static_cast<unsigned long long>(__ballot(row < base + incl))) - 1;
    } else if (want < b0 + 64) {
      l = want - b0;
    }
    if (l >= 0) {
      b = b0 + l;
      pb = base + __shfl(incl - rows, l, 64);
      return true;
    }
    base += chunk;
  }
  return false;
}

// D: head dim; QG: groups of 16 summary queries (S <= 16 QG); FOLD: a fold
// (a.accepted given), whose stored state is loaded at the start (one group
// of queries) so that its latency overlaps the page-id and row loads.
template <int D, int QG, bool FOLD>
__global__ __launch_bounds__(64) void summary_rows(SummaryArgs a) {
  constexpr int KS = D / 32, NB = D / 16;
  const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
  const int S = a.n_summary;
  const int n_max = a.max_pages * 16;
  // a fold: request b, KV head g, its new rows [lo, hi)
  const int b = FOLD ? static_cast<int>(blockIdx.x) / a.hkv : 0;
  const int g = FOLD ? static_cast<int>(blockIdx.x) % a.hkv : 0;
  const int pair = b * a.hkv + g;

  // a fold's stored state for the entries this lane merges (below)
  constexpr bool kEarly = FOLD && QG == 1;
  float c_pre[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float z_pre[kEarly ? 4 : 1][kEarly ? NB : 1];
  if constexpr (kEarly) {
    const float* zs = a.z + static_cast<size_t>(pair) * S * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 4 * grp + i;
      c_pre[i] = q < S ? a.c[static_cast<size_t>(pair) * S + q] : 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) z_pre[i][nb] = q < S ? zs[static_cast<size_t>(q) * D + 16 * nb + col] : 0.f;
    }
  }

  bf16x8 uq[QG][KS];
  f32x4 o[QG][NB];
  float m[QG], l[QG];
  const float sl2 = a.scale * kLog2e;

  // (m, l, O) of KV head g's summary queries over rows [lo, hi) of request b;
  // l summed over the four lanes of a column at the end
  auto walk = [&](int b, int g, int lo, int hi) {
  // summary queries: B operand of the score products (query 16 qg + col)
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int q = 16 * qg + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      uq[qg][ks] = q < S ? load_bf16x8(a.u + (static_cast<size_t>(g) * S + q) * D + 32 * ks + 8 * grp)
                         : zero_bf16x8();
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    m[qg] = -INFINITY;
    l[qg] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[qg][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int* pt = a.page_table + static_cast<size_t>(b) * a.max_pages;
  // the lane's key tokens (chain h) lie in tile page col / 8, its value
  // tokens 8 grp .. 8 grp + 7 in tile page grp / 2
  auto pages = [&](int t0, int& pk, int& pv) {
    pk = clampi(pt[min((t0 >> 4) + (col >> 3), a.max_pages - 1)], 0, a.num_pages - 1);
    pv = clampi(pt[min((t0 >> 4) + (grp >> 1), a.max_pages - 1)], 0, a.num_pages - 1);
  };
  auto load = [&](int pk, int pv, Tile<D>& r) {
    const uint16_t* kb = a.k_cache + (static_cast<size_t>(pk) * a.hkv + g) * (D / 8) * 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tok = (8 * (col >> 2) + 4 * h + (col & 3)) & 15;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) r.k[h][ks] = load_nt(kb + (4 * ks + grp) * 128 + tok * 8);
    }
    const uint16_t* vb = a.v_cache + (static_cast<size_t>(pv) * a.hkv + g) * D * 16 + ((8 * grp) & 15);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) r.v[nb] = load_nt(vb + (16 * nb + col) * 16);
  };
  auto compute = [&](int t0, const Tile<D>& r) {
    const bool partial = t0 < lo || t0 + kTile > hi;       // wave-uniform
    uint32_t keep = 0xffu;                                 // bit j: token t0 + 8 grp + j is in range
    if (partial) {
      keep = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = t0 + 8 * grp + j;
        keep |= (t >= lo && t < hi) ? 1u << j : 0u;
      }
    }
    bf16x8 vv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x4 w = r.v[nb];
      if (partial) {   // rows outside the range may hold anything, even NaN
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] &= ((keep >> (2 * e)) & 1u ? 0x0000ffffu : 0u) | ((keep >> (2 * e + 1)) & 1u ? 0xffff0000u : 0u);
      }
      vv[nb] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      f32x4 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[h] = mfma16(__builtin_bit_cast(bf16x8, r.k[h][ks]), uq[qg][ks], s[h]);
      }
      float x[8];
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = (keep >> j) & 1u ? s[j >> 2][j & 3] * sl2 : -INFINITY;
        mt = fmaxf(mt, x[j]);
      }
      mt = fmaxf(mt, xor_shuffle(mt, 16));
      mt = fmaxf(mt, xor_shuffle(mt, 32));
      const float mn = fmaxf(m[qg], mt);                 // finite: every tile holds a row in range
      const float al = exp2f(m[qg] - mn);                 // 0 on the first tile
      float ls = 0.f;
      bf16x8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = exp2f(x[j] - mn);
        ls += p;
        ph[j] = static_cast<__bf16>(p);
        pl[j] = static_cast<__bf16>(p - static_cast<float>(ph[j]));
      }
      l[qg] = l[qg] * al + ls;
      m[qg] = mn;
      // row q = 16 qg + 4 grp + i of O takes the factor of column 4 grp + i
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(al, 4 * grp + i, 64);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[qg][nb][i] *= ar[i];
        o[qg][nb] = mfma16(ph, vv[nb], o[qg][nb]);
        o[qg][nb] = mfma16(pl, vv[nb], o[qg][nb]);
      }
    }
  };

  if (hi > lo) {
    // tiles first + 32 i, i < nt, in two register sets in turn; the page ids
    // run two tiles ahead of the loads that use them.  Inside the loop every
    // load is unconditional (a conditional one would make the compiler copy
    // the registers it fills, waiting for them at once); the last one or two
    // tiles are computed after it.
    const int first = lo & ~(kTile - 1);
    const int nt = (hi - first + kTile - 1) / kTile;
    int pka, pva, pkb, pvb;
    pages(first, pka, pva);
    pages(first + kTile, pkb, pvb);
    Tile<D> ra, rb;
    load(pka, pva, ra);
    int i = 0;
    for (; i + 2 < nt; i += 2) {
      pages(first + (i + 2) * kTile, pka, pva);
      load(pkb, pvb, rb);
      compute(first + i * kTile, ra);
      pages(first + (i + 3) * kTile, pkb, pvb);
      load(pka, pva, ra);
      compute(first + (i + 1) * kTile, rb);
    }
    if (i + 1 < nt) {
      load(pkb, pvb, rb);
      compute(first + i * kTile, ra);
      compute(first + (i + 1) * kTile, rb);
    } else {
      compute(first + i * kTile, ra);
    }
  }
  // per-query sums over the four lanes of a column
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    l[qg] += xor_shuffle(l[qg], 16);
    l[qg] += xor_shuffle(l[qg], 32);
  }
  };

  if constexpr (!FOLD) {
    // rows [w T, (w + 1) T) of the concatenation, piece by piece
    long long total, T;
    concat_size(a, lane, total, T);
    const long long w = blockIdx.x;
    const long long r0 = w * T, r1 = min(total, r0 + T);
    int rb;
    long long pb;
    if (r0 >= total || !find_request(a, r0, 0, lane, rb, pb)) return;   // past the last row
    long long cur = r0;
    for (;;) {
      const int n = clampi(a.ctx_len[rb], 0, n_max);   // > 0: the request holds row cur
      const int rg = static_cast<int>((cur - pb) / n);
      const long long ps = pb + static_cast<long long>(rg) * n;   // first row of (rb, rg)
      const long long pe = min(r1, ps + n);
      walk(rb, rg, static_cast<int>(cur - ps), static_cast<int>(pe - ps));
      // partial state of the piece: max (base 2), sum, unnormalised O
      const size_t base = (static_cast<size_t>(rb) * a.hkv + rg + static_cast<size_t>(w)) * S;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const int q = 16 * qg + col;
        if (grp == 0 && q < S) a.part_ml[base + q] = make_float2(m[qg], l[qg]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = 16 * qg + 4 * grp + i;
          if (qi < S) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) a.part_o[(base + qi) * D + 16 * nb + col] = o[qg][nb][i];
          }
        }
      }
      cur = pe;
      if (cur >= r1) break;
      if (rg + 1 == a.hkv) {   // the next request with rows
        pb += static_cast<long long>(n) * a.hkv;
        do {
          ++rb;
        } while (rb < a.batch && clampi(a.ctx_len[rb], 0, n_max) == 0);
        if (rb >= a.batch) break;
      }
    }
    return;
  }

  // a fold: the committed token and the accepted drafts of request b
  {
    const int lo = clampi(a.ctx_len[b], 0, n_max);
    walk(b, g, lo, min(n_max, lo + clampi(a.accepted[b], 0, n_max) + 1));
  }

  // a fold: merge with the stored state (eq. (11)); no new rows leave it as is
  float* zs = a.z + static_cast<size_t>(pair) * S * D;
  float* cs = a.c + static_cast<size_t>(pair) * S;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 16 * qg + 4 * grp + i;
      const float mq = __shfl(m[qg], 4 * grp + i, 64);
      const float lq = __shfl(l[qg], 4 * grp + i, 64);
      if (q >= S || !(lq > 0.f)) continue;
      const float c_new = (mq + log2f(lq)) * kLn2;
      float c_old;
      if constexpr (kEarly) c_old = c_pre[i];
      else c_old = cs[q];
      float* zq = zs + static_cast<size_t>(q) * D;
      float c = c_new;
      if (c_old == -INFINITY) {
        const float inv = 1.f / lq;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) zq[16 * nb + col] = o[qg][nb][i] * inv;
      } else {
        const float mx = fmaxf(c_old, c_new);
        c = mx + logf(expf(c_old - mx) + expf(c_new - mx));
        const float wo = expf(c_old - c), wn = expf(c_new - c) / lq;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float z_old;
          if constexpr (kEarly) z_old = z_pre[i][nb];
          else z_old = zq[16 * nb + col];
          zq[16 * nb + col] = wo * z_old + wn * o[qg][nb][i];
        }
      }
      if (col == 0) cs[q] = c;
    }
  }
}

// Combines the pieces of a whole-prefix initialisation: entry (q, d) of a
// (request, KV head) is sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over
// its pieces s (slots p + w for the waves w covering its rows), M = max m_s
// (base 2); c = ln 2 (M + log2 of the denominator).  A prefix without rows
// gets the empty state (Z = 0, c = -inf).
__global__ __launch_bounds__(kMergeThreads) void summary_merge(SummaryArgs a) {
  const int pair = blockIdx.x, S = a.n_summary, D = a.head_dim;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int lane = threadIdx.x & 63;
  long long total, T;
  concat_size(a, lane, total, T);
  int bb;
  long long pb;
  find_request(a, -1, b, lane, bb, pb);
  const int n = clampi(a.ctx_len[b], 0, a.max_pages * 16);
  const long long ps = pb + static_cast<long long>(g) * n;   // first row of the pair
  const int w0 = static_cast<int>(ps / T);
  const int nc = n > 0 ? static_cast<int>((ps + n - 1) / T) - w0 + 1 : 0;
  const int e = blockIdx.y * kMergeThreads + threadIdx.x;
  if (e >= S * D) return;
  const int q = e / D, d = e % D;
  const size_t base = static_cast<size_t>(pair) + w0;
  // one pass with a running maximum over groups of 16 slices whose loads go
  // out together (clamped index; an empty slice's values are never written
  // and are dropped by a select)
  constexpr int U = 16;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < nc; s0 += U) {
    float2 ml[U];
    float os[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = (base + min(s0 + u, nc - 1)) * S + q;
      ml[u] = a.part_ml[i];
      os[u] = a.part_o[i * D + d];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = s0 + u < nc && ml[u].y > 0.f;
      const float mn = live ? fmaxf(M, ml[u].x) : M;
      const float r = mn == M ? 1.f : exp2f(M - mn);    // M = -inf: 0
      const float w = live ? exp2f(ml[u].x - mn) : 0.f;
      L = L * r + (live ? ml[u].y * w : 0.f);
      O = O * r + (live ? os[u] * w : 0.f);
      M = mn;
    }
  }
  a.z[(static_cast<size_t>(pair) * S + q) * D + d] = L > 0.f ? O / L : 0.f;
  if (d == 0) a.c[static_cast<size_t>(pair) * S + q] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D, bool FOLD>
hipError_t launch_rows(const SummaryArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(64);
  if (a.n_summary <= 16) return launch_kernel(summary_rows<D, 1, FOLD>, grid, block, s, a);
  if (a.n_summary <= 32) return launch_kernel(summary_rows<D, 2, FOLD>, grid, block, s, a);
  return launch_kernel(summary_rows<D, 4, FOLD>, grid, block, s, a);
}

}  // namespace

int64_t summary_init_slots(int64_t batch, int64_t hkv) { return kSummaryInitWaves + batch * hkv; }

hipError_t launch_summary(const SummaryArgs& a, hipStream_t s) {
  const int head_dim = a.head_dim;
  if (a.accepted)   // a fold: one wave per (request, KV head)
    return head_dim == 64 ? launch_rows<64, true>(a, dim3(a.batch * a.hkv), s)
                          : launch_rows<128, true>(a, dim3(a.batch * a.hkv), s);
  // an initialisation: kSummaryInitWaves waves over the concatenated rows,
  // then the merge
  const dim3 grid(kSummaryInitWaves);
  hipError_t e = head_dim == 64 ? launch_rows<64, false>(a, grid, s) : launch_rows<128, false>(a, grid, s);
  if (e != hipSuccess) return e;
  const dim3 mgrid(a.batch * a.hkv, (a.n_summary * head_dim + kMergeThreads - 1) / kMergeThreads);
  return launch_kernel(summary_merge, mgrid, dim3(kMergeThreads), s, a);
}

}  // namespace sd
