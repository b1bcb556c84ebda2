// Speculative-sampling verification ("LongSpark", sec. 2.1, eqs. (1)-(2) and
// the bonus-token rule after eq. (2); "ForeSpark", sec. 4.4 for verify
// budgets b_b <= K_b).  Variants: temperature 0 on both sides (p_j and q_j
// one-hot at their argmax: accept iff y_j = argmax p_j, correction or bonus
// = argmax p_j; "LongSpark", App. D.1 and "H-Spec", sec. 4 evaluate greedy
// decoding) and a pruned drafter vocabulary (q_j is zero outside it; "H-Spec",
// App. B.2).
//
// Three or four launches, no host synchronisation:
//   1. verify_rowstats  grid (rows x 8192-entry chunks): per chunk (max, sum
//      exp) of every target row (and of every draft row when no draft lse is
//      given).  Each thread issues its eight 16-byte loads at once, so the
//      logits stream through in one pass: HBM-bound.  The loads are
//      non-temporal (each logit is read once here).
//   2. verify_decide    one workgroup per request: merges the row statistics
//      it needs, evaluates the request's ratio tests in parallel (256
//      positions per pass, one thread each, in two rounds of loads) and takes
//      the first rejection from wave ballots.  Only for batches of
//      kDecideBatch requests or more: below that every sampling workgroup
//      takes the decision itself and the launch is saved.
//   3. verify_sample    grid (requests x 2048-entry chunks): every workgroup
//      of a request reads the decision and draws Gumbel-max candidates of its
//      vocab chunk from the residual [p_j - q_j]_+ (and from p_j as the
//      fallback), or from p_{b+1}.  Only one row per request is read, so the
//      chunks are small to spread that row over many CUs.
//   4. verify_finalize  one wavefront per request merges the chunk candidates.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kThreads = 256;
// Positions whose ratio tests one pass of the decision holds in LDS; a
// request with more verified drafts takes several passes.
constexpr int kDecideChunk = 256;
// Batch from which the decision gets its own kernel (timed: -13 us at 128
// requests, -4 us at 64, +3 us at 16 for the extra launch).
constexpr int kDecideBatch = 48;

// (max, sum exp(x - max), first index of the max) of one vocab chunk of one
// row.  Thread t holds entries 4 (t + 256 j) + e of the chunk.
__global__ __launch_bounds__(kThreads) void verify_rowstats(VerifyArgs a) {
  __shared__ float sh[kThreads / 64];
  __shared__ float shk[kThreads / 64];
  __shared__ int shi[kThreads / 64];
  constexpr int kGroups = kVerifyChunk / (4 * kThreads);
  const int row = blockIdx.x / a.n_chunks;
  const int c = blockIdx.x % a.n_chunks;
  const bool tgt = row < a.R;
  const int len = tgt ? a.V : a.v_draft;
  const float* src = tgt ? a.target + static_cast<size_t>(row) * a.V
                         : a.draft + static_cast<size_t>(row - a.R) * a.v_draft;
  const int lo = c * kVerifyChunk;
  const bool vec_ok = (len & 3) == 0;
  f32x4 x[kGroups];
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    const int v = lo + 4 * (threadIdx.x + kThreads * j);
    if (vec_ok && v + 3 < len) {
      x[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + v));   // read once
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[j][e] = v + e < len ? src[v + e] : -INFINITY;
    }
  }
  // The first argmax is needed only at temperature 0 (greedy tests and
  // draws); sampling needs the max alone, a cheaper reduction.
  float mx;
  int amax = 0;
  if (a.greedy) {
    Cand best{-FLT_MAX, 0x7fffffff};
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = lo + 4 * (threadIdx.x + kThreads * j) + e;
        if (v < len && better(x[j][e], v, best.key, best.idx)) best = Cand{x[j][e], v};
      }
    best = block_best<kThreads>(best, shk, shi);
    mx = best.key;
    amax = best.idx;
  } else {
    float m = -FLT_MAX;   // entries past the row are -inf
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, x[j][e]);
    mx = block_reduce_max<kThreads>(m, sh);
  }
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < kGroups; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) se += __builtin_amdgcn_exp2f((x[j][e] - mx) * kLog2e);
  se = block_reduce_sum<kThreads>(se, sh);
  if (threadIdx.x == 0) a.row_part[blockIdx.x] = make_float4(mx, se, __int_as_float(amax), 0.f);
}

// Log-normaliser of a row from its n chunk partials, and with kArgmax its
// first argmax (temperature 0 only).  Loads are issued U at a time (clamped
// index, duplicates weighted zero) so their latencies overlap: when sampling,
// (max, sum) pairs 32 at a time, so at up to 32 chunks (a vocabulary of up to
// 262,144) all of a row's partials are in flight together.
template <bool kArgmax>
__device__ float merge_row(const float4* part, int n, int& amax) {
  constexpr int U = kArgmax ? 16 : 32;
  float mx = -FLT_MAX;
  float s = 0.f;
  Cand best{-FLT_MAX, 0x7fffffff};
  for (int i0 = 0; i0 < n; i0 += U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float4* pp = part + min(i0 + u, n - 1);
      if constexpr (kArgmax) {
        v[u] = *pp;
      } else {
        const float2 m2 = *reinterpret_cast<const float2*>(pp);
        v[u] = make_float4(m2.x, m2.y, 0.f, 0.f);
      }
    }
    float m2 = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m2 = fmaxf(m2, v[u].x);
      if constexpr (kArgmax) {
        const int idx = __float_as_int(v[u].z);
        if (i0 + u < n && better(v[u].x, idx, best.key, best.idx)) best = Cand{v[u].x, idx};
      }
    }
    s *= __builtin_amdgcn_exp2f((mx - m2) * kLog2e);
#pragma unroll
    for (int u = 0; u < U; ++u)
      s += i0 + u < n ? v[u].y * __builtin_amdgcn_exp2f((v[u].x - m2) * kLog2e) : 0.f;
    mx = m2;
  }
  amax = best.idx;
  return mx + logf(s);
}

__device__ __forceinline__ float merge_row(const VerifyArgs& a, const float4* part, int& amax) {
  return a.greedy ? merge_row<true>(part, a.n_chunks, amax) : merge_row<false>(part, a.n_chunks, amax);
}

// Shared memory of one request's decision.
struct DecideSmem {
  float lse_p[kDecideChunk + 1];   // the pass's rows, and the bonus row after the last one
  int amax_p[kDecideChunk + 1];
  float lse_q[kDecideChunk];
  int first_reject[kThreads / 64];   // per wave: first rejected position of the pass, or n
  int reject;                      // first rejected position (0-based), or nv
  float lse_p_dec, lse_q_dec;      // normalisers of the row the draw uses
  float4 dec;   // (accepted as int bits or -1, lse_p, lse_q, tested as int bits)
};

// Row statistics, every ratio test and the first rejection of request b, by
// one workgroup; on return sm.dec holds the decision for every thread.  With
// `writer` set the workgroup also stores accepted[b] and the accept ratios.
// The tests run kDecideChunk positions per pass; every tested position gets
// its ratio, and the first rejection over all passes decides.
__device__ void decide_request(const VerifyArgs& a, int b, bool writer, DecideSmem& sm) {
  const int tid = threadIdx.x;
  const int t0 = clampi(a.t_off[b], 0, a.R);
  const int t1 = clampi(a.t_off[b + 1], t0, a.R);
  const int q0 = clampi(a.q_off[b], 0, a.total_q);
  const int kb = clampi(a.q_off[b + 1], q0, a.total_q) - q0;
  if (t1 == t0) {   // no target row: nothing to verify (contract violation)
    if (tid == 0) {
      if (writer) a.accepted[b] = 0;
      sm.dec = make_float4(__int_as_float(-1), 0.f, 0.f, __int_as_float(0));
    }
    __syncthreads();
    return;
  }
  const int nv = min(t1 - t0 - 1, kb);
  const uint32_t rid = a.req_id[b];
  if (tid == 0) sm.reject = nv;

  for (int c0 = 0;; c0 += kDecideChunk) {
    const int n = min(kDecideChunk, nv - c0);
    const bool last = c0 + n == nv;   // this pass also holds the bonus row nv
    // A: per position (one thread each), the log-normalisers of its rows
    // and its ratio test (eq. (1)): r_j = min(1, p_j(y_j)/q_j(y_j)); at
    // temperature 0 both distributions are one-hot and r_j = [y_j = argmax
    // p_j].  The token, the row partials and the draft normaliser do not
    // depend on one another, so their loads are issued together, and the two
    // logits at y_j follow in a second round.  The thread after the last
    // position takes the bonus row.
    bool rejected = false;   // position tid of this pass was rejected
    for (int i = tid; i < n + (last ? 1 : 0); i += kThreads) {
      const bool test = i < n;
      const int j = c0 + i + 1;
      const int y = test ? clampi(a.tokens[q0 + j - 1], 0, a.V - 1) : 0;
      const float lqd = test && a.draft_lse ? a.draft_lse[q0 + j - 1] : 0.f;
      int amax;
      const float lse_p = merge_row(a, a.row_part + static_cast<size_t>(t0 + c0 + i) * a.n_chunks, amax);
      sm.lse_p[i] = lse_p;
      sm.amax_p[i] = amax;
      if (!test) continue;
      int unused;
      const float lse_q = a.draft_lse ? lqd
                                      : merge_row<false>(a.row_part + static_cast<size_t>(a.R + q0 + j - 1) * a.n_chunks,
                                                         a.n_chunks, unused);
      sm.lse_q[i] = lse_q;
      float r = 1.f;
      if (a.greedy) {
        r = y == amax ? 1.f : 0.f;
      } else {
        const int iy = a.vinv ? a.vinv[y] : y;   // y in the drafter's vocabulary
        const float lp = a.target[static_cast<size_t>(t0 + j - 1) * a.V + y] - lse_p;
        const float lq = iy >= 0 && iy < a.v_draft
                             ? a.draft[static_cast<size_t>(q0 + j - 1) * a.v_draft + iy] - lse_q
                             : -INFINITY;
        if (expf(lq) > 0.f) r = fminf(1.f, expf(lp - lq));
      }
      const u32x4 w = philox4x32_10(u32x4{0u, static_cast<uint32_t>(j), rid, kStreamAccept},
                                    a.key0, a.key1);
      rejected = !(accept_from_bits(w[0]) < r);
      if (writer && a.accept_ratio) a.accept_ratio[q0 + j - 1] = r;
    }
    {
      // first rejection of each wave's positions (position i is thread i)
      const uint64_t rj = __ballot(rejected);
      if ((tid & 63) == 0) sm.first_reject[tid >> 6] = rj ? (tid & ~63) + __builtin_ctzll(rj) : n;
    }
    __syncthreads();

    // C: the first rejection ends the round; keep the normalisers of the row
    // the draw will use (the rejected one, or the bonus row)
    if (tid == 0) {
      int first = n;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) first = min(first, sm.first_reject[w]);
      if (sm.reject == nv && first < n) {
        sm.reject = c0 + first;
        sm.lse_p_dec = sm.lse_p[first];
        sm.lse_q_dec = sm.lse_q[first];
      }
      if (last && sm.reject == nv) {
        sm.lse_p_dec = sm.lse_p[n];
        sm.lse_q_dec = 0.f;
      }
    }
    __syncthreads();   // the next pass reuses the arrays
    // after a rejection, later passes only serve the ratios of the positions
    // beyond it
    if (last || (sm.reject < nv && !(writer && a.accept_ratio))) break;
  }
  if (writer && a.accept_ratio)
    for (int i = nv + tid; i < kb; i += kThreads) a.accept_ratio[q0 + i] = __int_as_float(0x7fc00000);

  if (tid == 0) {
    const int acc = sm.reject;
    if (writer) a.accepted[b] = acc;
    const bool residual = !a.greedy && acc < nv;
    sm.dec = make_float4(__int_as_float(acc), sm.lse_p_dec, residual ? sm.lse_q_dec : 0.f,
                         __int_as_float(nv));
  }
  __syncthreads();
}

// Large batches: one workgroup per request decides once and stores the
// decision for the request's sampling workgroups.
__global__ __launch_bounds__(kThreads) void verify_decide(VerifyArgs a) {
  __shared__ DecideSmem sm;
  decide_request(a, blockIdx.x, true, sm);
  if (threadIdx.x == 0) a.decision[blockIdx.x] = sm.dec;
}

// Every workgroup of a request draws Gumbel-max candidates of its vocab chunk
// after the request's decision: from the residual [p_j - q_j]_+ (and from p_j
// as the fallback) at the first rejection, or from p_{b+1} when every test
// passed.  kDecided: the decision comes from verify_decide; otherwise every
// workgroup takes it itself (one launch fewer, for small batches).
template <bool kDecided>
__global__ __launch_bounds__(kThreads) void verify_sample(VerifyArgs a) {
  __shared__ float shk[kThreads / 64];
  __shared__ int shi[kThreads / 64];
  const int b = blockIdx.x / a.n_schunks;
  const int c = blockIdx.x % a.n_schunks;
  const int tid = threadIdx.x;
  float4 dec;
  if constexpr (kDecided) {
    dec = a.decision[b];
  } else {
    __shared__ DecideSmem sm;
    decide_request(a, b, c == 0, sm);
    dec = sm.dec;
  }
  const int acc = __float_as_int(dec.x);
  if (acc < 0) {   // no target row
    if (tid == 0) {
      a.samp_part[blockIdx.x * 2] = make_float4(-FLT_MAX, __int_as_float(-1), 0.f, 0.f);
      a.samp_part[blockIdx.x * 2 + 1] = make_float4(-FLT_MAX, __int_as_float(-1), 0.f, 0.f);
    }
    return;
  }
  const int nv = __float_as_int(dec.w);
  const int t0 = clampi(a.t_off[b], 0, a.R);
  const int q0 = clampi(a.q_off[b], 0, a.total_q);
  const uint32_t rid = a.req_id[b];
  const bool residual = !a.greedy && acc < nv;
  const int j = acc + 1;                      // position of the drawn token
  const float* xrow = a.target + static_cast<size_t>(t0 + acc) * a.V;
  const float* zrow = a.draft + static_cast<size_t>(q0 + acc) * a.v_draft;
  const float lp2 = dec.y * kLog2e;   // log-normalisers in base-2 units
  const float lq2 = dec.z * kLog2e;

  // D: Gumbel-max candidates of this vocab chunk; thread t holds entries
  // 4 (t + 256 j) + e of the chunk
  Cand best_r{-FLT_MAX, 0x7fffffff}, best_p{-FLT_MAX, 0x7fffffff};
  int any_pos = 0;
  const int lo = c * kSampleChunk;
  const bool vec_ok = (a.V & 3) == 0;
#pragma unroll
  for (int jj = 0; jj < kSampleChunk / (4 * kThreads); ++jj) {
    const int g = lo + 4 * (tid + kThreads * jj);
    if (g >= a.V) break;
    f32x4 xv, zv;
    if (vec_ok && g + 3 < a.V) {
      xv = *reinterpret_cast<const f32x4*>(xrow + g);
      if (residual && !a.vinv) zv = *reinterpret_cast<const f32x4*>(zrow + g);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[e] = g + e < a.V ? xrow[g + e] : 0.f;
        zv[e] = residual && !a.vinv && g + e < a.V ? zrow[g + e] : 0.f;
      }
    }
    if (residual && a.vinv) {
      // q is zero outside the drafter's vocabulary
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int iz = g + e < a.V ? a.vinv[g + e] : -1;
        zv[e] = iz >= 0 && iz < a.v_draft ? zrow[iz] : -INFINITY;
      }
    }
    const u32x4 w = a.greedy ? u32x4{0u, 0u, 0u, 0u}
                             : philox4x32_10(u32x4{static_cast<uint32_t>(g >> 2),
                                                   static_cast<uint32_t>(j), rid, kStreamSample},
                                             a.key0, a.key1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = g + e;
      if (v < a.V) {
        const float gn = a.greedy ? 0.f : gumbel_from_bits(w[e]);
        const float x = xv[e];
        const float kp = x + gn;
        if (better(kp, v, best_p.key, best_p.idx)) best_p = Cand{kp, v};
        if (residual) {
          // p and q by the hardware base-2 exponential of one fused
          // multiply-add each (one rounding, as x - lse alone has)
          const float res = __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -lp2)) -
                            __builtin_amdgcn_exp2f(fmaf(zv[e], kLog2e, -lq2));
          if (res > 0.f) {
            any_pos = 1;
            const float kr = kLn2 * __builtin_amdgcn_logf(res) + gn;
            if (better(kr, v, best_r.key, best_r.idx)) best_r = Cand{kr, v};
          }
        }
      }
    }
  }
  best_r = block_best<kThreads>(best_r, shk, shi);
  best_p = block_best<kThreads>(best_p, shk, shi);
  any_pos = __syncthreads_or(any_pos);
  if (tid == 0) {
    a.samp_part[blockIdx.x * 2] =
        make_float4(best_r.key, __int_as_float(best_r.idx), any_pos ? 1.f : 0.f, 0.f);
    a.samp_part[blockIdx.x * 2 + 1] = make_float4(best_p.key, __int_as_float(best_p.idx), 0.f, 0.f);
  }
}

// One wavefront per request: lanes read the chunk candidates in parallel.
__global__ __launch_bounds__(64) void verify_finalize(VerifyArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float4* p = a.samp_part + static_cast<size_t>(b) * a.n_schunks * 2;
  int any_pos = 0;
  for (int c = lane; c < a.n_schunks; c += 64) any_pos |= p[2 * c].z != 0.f;
  const int sel = __any(any_pos) ? 0 : 1;   // residual draw, else a draw from p
  Cand best{-FLT_MAX, 0x7fffffff};
  for (int c = lane; c < a.n_schunks; c += 64) {
    const float4 q = p[2 * c + sel];
    const int idx = __float_as_int(q.y);
    if (idx >= 0 && better(q.x, idx, best.key, best.idx)) best = Cand{q.x, idx};
  }
  best = wave_best(best);
  if (lane == 0) a.next_token[b] = best.idx == 0x7fffffff ? -1 : best.idx;
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
  const int rows = a.R + (a.draft_lse ? 0 : a.total_q);
  hipError_t e = hipSuccess;
  if (rows > 0) e = launch_kernel(verify_rowstats, dim3(rows * a.n_chunks), dim3(kThreads), s, a);
  const dim3 sgrid(a.batch * a.n_schunks);
  if (a.batch >= kDecideBatch) {
    if (e == hipSuccess) e = launch_kernel(verify_decide, dim3(a.batch), dim3(kThreads), s, a);
    if (e == hipSuccess) e = launch_kernel(verify_sample<true>, sgrid, dim3(kThreads), s, a);
  } else if (e == hipSuccess) {
    e = launch_kernel(verify_sample<false>, sgrid, dim3(kThreads), s, a);
  }
  if (e == hipSuccess)
    e = launch_kernel(verify_finalize, dim3(a.batch), dim3(64), s, a);
  return e;
}

}  // namespace sd
