// Work-conserving draft / verification budget scheduling ("ForeSpark",
// sec. 4.2-4.4), entirely on the device so that the host never waits:
//
//   sched_gemm       C = A1 B1^T (+ A2 B2^T), bf16 in, fp32 out, MFMA 32x32x16
//                    (four wavefronts split K per 32 x 32 tile, and K split
//                    across workgroups for the few-row pre-draft product,
//                    finished by sched_gemm_reduce); epilogue: + bias, SiLU.
//                    Serves the pre-draft estimator's hidden layer
//                    u = SiLU(W_c c + W_e e + b) (eq. (2)) and the post-draft
//                    selector projection W_s h (eq. (5)).
//   sched_tri_logits z = W_o u (+ b_o), then the per-entry calibration
//                    scale * z + bias (sec. 4.5): fp32 VALU, one wavefront per
//                    (request, triangle entry).
//   sched_rewards    survival benefits S_{d,j} (eq. (3)) and the reward curve
//                    R(d) = Reward(d, d), one thread per (request, d).
//   sched_joint      one workgroup: the upper concave envelope F of every
//                    reward curve (monotone chain, O(K) per request) and the
//                    survival scores g_d = F(d) - F(d-1); a stable merge of
//                    the requests' (already sorted) score runs in LDS; the bucket-pair search of eq. (4) against
//                    the latency tables; the draft schedule d_i (the owners of
//                    the top k scores), q_off and the budget B.
//   sched_post_logit one wavefront per draft row: p = sigmoid((w . [h; s] + c) /
//                    theta_j), s = (W_s h) * E_pred(previous token) (eq. (5)).
//   sched_budget     one workgroup: S^_j = prod_{t<=j} p_t per request, a
//                    stable merge of the requests' rows, the top B rows -> verify prefix
//                    b_i and t_off (sec. 4.4).
//
// Equal scores are ordered by (request, position), which keeps every
// selection a prefix of each request's draft.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + expf(-x)); }

// ------------------------------------------------------------------ GEMM
// One workgroup (4 wavefronts) computes a 32 x 32 tile of C[M][N] =
// A1 B1^T (+ A2 B2^T) with A [M][K], B [N][K] row-major bf16, K a multiple of
// 16, over its share (blockIdx.z of ksplit) of the 16-dim steps of both
// products; the wavefronts take interleaved steps and their partial tiles
// are summed through LDS.  Lane l feeds row l % 32 of the A (and B) tile with
// dims 8 (l / 32) .. +8 of a step; element i of a partial tile is
// C[row 8 (i/4) + 4 (l/32) + i%4][col l % 32].  Rows past M (N) load the last
// row and are not stored.  With one split the epilogue adds the bias and
// applies SiLU; with several, raw sums go to part[z] and sched_gemm_reduce
// finishes (few rows: the K splits are what fill the GPU).
constexpr int kGemmWaves = 4;

__global__ __launch_bounds__(64 * kGemmWaves) void sched_gemm(SchedGemmArgs a) {
  __shared__ float red[kGemmWaves][32 * 33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int h = lane >> 5, rr = lane & 31;
  const size_t ra = static_cast<size_t>(min(m0 + rr, a.M - 1)) * a.K + 8 * h;
  const size_t rb = static_cast<size_t>(min(n0 + rr, a.N - 1)) * a.K + 8 * h;
  f32x16 acc = {};
  const int steps = a.K / 16;
  const int total = steps * (a.a2 ? 2 : 1);
  const int per = (total + a.ksplit - 1) / a.ksplit;
  const int sb = static_cast<int>(blockIdx.z) * per, se = min(total, sb + per);
  auto opnd = [&](int g, bf16x8& x, bf16x8& y) {
    const bool second = g >= steps;
    const size_t k = static_cast<size_t>(second ? g - steps : g) * 16;
    x = load_bf16x8((second ? a.a2 : a.a1) + ra + k);
    y = load_bf16x8((second ? a.b2 : a.b1) + rb + k);
  };
  int s = sb + wave;
  for (; s + 3 * kGemmWaves < se; s += 4 * kGemmWaves) {
    bf16x8 x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) opnd(s + u * kGemmWaves, x[u], y[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = mfma_32x32x16(x[u], y[u], acc);
  }
  for (; s < se; s += kGemmWaves) {
    bf16x8 x, y;
    opnd(s, x, y);
    acc = mfma_32x32x16(x, y, acc);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) red[wave][(8 * (i >> 2) + 4 * h + (i & 3)) * 33 + rr] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * 32; e += 64 * kGemmWaves) {
    const int row = m0 + e / 32, col = n0 + e % 32;
    if (row < a.M && col < a.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kGemmWaves; ++w) v += red[w][(e / 32) * 33 + e % 32];
      if (a.ksplit > 1) {
        a.part[(static_cast<size_t>(blockIdx.z) * a.M + row) * a.N + col] = v;
      } else {
        if (a.bias) v += a.bias[col];
        if (a.silu) v = v * sigmoidf(v);
        a.c[static_cast<size_t>(row) * a.N + col] = v;
      }
    }
  }
}

// c = act(sum_z part[z] + bias), one thread per element.
__global__ __launch_bounds__(256) void sched_gemm_reduce(SchedGemmArgs a) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t mn = static_cast<size_t>(a.M) * a.N;
  if (e >= mn) return;
  float v = 0.f;
  for (int z = 0; z < a.ksplit; ++z) v += a.part[z * mn + e];
  if (a.bias) v += a.bias[e % a.N];
  if (a.silu) v = v * sigmoidf(v);
  a.c[e] = v;
}

// z[i][e] = scale[e] * (u[i] . W_o[e] + b_o[e]) + bias[e]; one wavefront per
// (request, entry), lanes across r.
__global__ __launch_bounds__(256) void sched_tri_logits(SchedArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int T = a.K * (a.K + 1) / 2;
  if (idx >= a.n * T) return;
  const int i = idx / T, e = idx % T;
  const float* u = a.u + static_cast<size_t>(i) * a.r;
  const uint16_t* w = a.w_o + static_cast<size_t>(e) * a.r;
  float z = 0.f;
  for (int k = lane; k < a.r; k += 64) z += u[k] * __uint_as_float(static_cast<uint32_t>(w[k]) << 16);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
  if (lane == 0) {
    if (a.b_o) z += a.b_o[e];
    if (a.cal_scale) z *= a.cal_scale[e];
    if (a.cal_bias) z += a.cal_bias[e];
    a.logits[idx] = z;
  }
}

// Reward curve R_i(d) = sum_{j<=d} prod_{t<=j} sigmoid(z^(d)_t) (eq. (3) and
// Reward_i(d, d)), one thread per (request, d); the row's logits are loaded
// together (a fixed, predicated loop) so their latencies overlap.
__global__ __launch_bounds__(256) void sched_rewards(SchedArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int K = a.K;
  if (e >= a.n * K) return;
  const int i = e / K, d = e % K + 1;
  const float* z = a.logits + static_cast<size_t>(i) * (K * (K + 1) / 2) + d * (d - 1) / 2;
  float zv[kSchedMaxK];
#pragma unroll
  for (int t = 0; t < kSchedMaxK; ++t) zv[t] = t < d ? z[t] : 0.f;
  float prod = 1.f, sum = 0.f;
#pragma unroll
  for (int t = 0; t < kSchedMaxK; ++t) {
    if (t < d) {
      prod *= sigmoidf(zv[t]);
      sum += prod;
    }
  }
  a.rewards[static_cast<size_t>(i) * (K + 1) + d] = sum;
}

// --------------------------------------------------- sorting in one workgroup
// Descending by value, equal values by ascending index.
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Stable merge of sorted runs in LDS.  Request i's entries occupy positions
// bounds(i) .. bounds(i + 1) - 1 and are already in "before" order (values
// non-increasing along a request, original indices increasing); own[p] is
// the request of position p.  Round r merges neighbouring groups of 2^r
// requests: an element's new position is its rank in its own group plus the
// number of elements of the partner group that go before it, found by binary
// search -- a partner element comes first if its value is larger (partner on
// the right: its original indices are all larger) or not smaller (partner on
// the left).  ceil(log2 n) rounds, one barrier each; (v, ix) hold the result.
template <int NT, typename Bounds>
__device__ void merge_runs(float*& v, int*& ix, float*& v2, int*& ix2, int total, int n,
                           const int* own, Bounds bounds) {
  for (int w = 1; w < n; w <<= 1) {
    for (int p = threadIdx.x; p < total; p += NT) {
      const int i = own[p];
      const int g0 = (i / (2 * w)) * (2 * w);
      const int lo = bounds(g0), mid = bounds(min(g0 + w, n)), hi = bounds(min(g0 + 2 * w, n));
      const float x = v[p];
      const bool left = p < mid;
      int a = left ? mid : lo, c = left ? hi : mid;   // binary search in the partner run
      while (a < c) {                                 // first partner entry that goes after x
        const int m = (a + c) >> 1;
        const bool first = left ? v[m] > x : v[m] >= x;
        if (first) a = m + 1;
        else c = m;
      }
      const int np = lo + (left ? p - lo + (a - mid) : p - mid + (a - lo));
      if (np >= 0 && np < total) {
        v2[np] = x;
        ix2[np] = ix[p];
      }
    }
    __syncthreads();
    float* tv = v;
    v = v2;
    v2 = tv;
    int* ti = ix;
    ix = ix2;
    ix2 = ti;
  }
}

// Inclusive prefix sum of x[0..P) in place (P <= 4 * NT), Hillis-Steele over
// per-thread partial sums.
template <int NT>
__device__ void prefix_sum(float* x, int P, float* tmp) {
  const int per = (P + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  float s = 0.f;
  for (int q = 0; q < per && b0 + q < P; ++q) {
    s += x[b0 + q];
    x[b0 + q] = s;
  }
  tmp[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const float add = threadIdx.x >= off ? tmp[threadIdx.x - off] : 0.f;
    __syncthreads();
    tmp[threadIdx.x] += add;
    __syncthreads();
  }
  const float base = threadIdx.x > 0 ? tmp[threadIdx.x - 1] : 0.f;
  for (int q = 0; q < per && b0 + q < P; ++q) x[b0 + q] += base;
  __syncthreads();
}

constexpr int kSchedThreads = 1024;

// ------------------------------------------------------------ joint schedule
__global__ __launch_bounds__(kSchedThreads) void sched_joint(SchedArgs a) {
  __shared__ float s_va[kSchedMaxEntries], s_vb[kSchedMaxEntries];
  __shared__ int s_ia[kSchedMaxEntries], s_ib[kSchedMaxEntries];
  __shared__ int s_own[kSchedMaxEntries];
  __shared__ float s_tmp[kSchedThreads];
  __shared__ int s_d[kSchedMaxRequests];
  __shared__ float s_best[kSchedThreads];
  __shared__ int s_bidx[kSchedThreads];
  __shared__ float s_R[kSchedMaxEntries + kSchedMaxRequests];   // [n][K + 1]
  __shared__ int s_hx[kSchedMaxEntries + kSchedMaxRequests];
  const int tid = threadIdx.x;
  const int n = a.n, K = a.K;
  const int E = n * K;
  float* s_v = s_va;
  int* s_i = s_ia;
  float* s_v2 = s_vb;
  int* s_i2 = s_ib;

  // reward curves (from sched_rewards) into LDS; then the upper concave
  // envelope and the scores, one thread per request
  for (int e = tid; e < n * (K + 1); e += kSchedThreads)
    s_R[e] = e % (K + 1) == 0 ? 0.f : a.rewards[e];
  __syncthreads();
  for (int i = tid; i < n; i += kSchedThreads) {
    const float* R = s_R + i * (K + 1);
    int* hx = s_hx + i * (K + 1);
    // upper hull of the points (d, R[d]): drop the middle point while it lies
    // on or below the chord of its neighbours
    int top = 0;
    for (int d = 0; d <= K; ++d) {
      while (top >= 2) {
        const int p0 = hx[top - 2], p1 = hx[top - 1];
        // cross((p1 - p0), (d - p0)) >= 0  <=> p1 not strictly above the chord
        const float cr = (p1 - p0) * (R[d] - R[p0]) - (R[p1] - R[p0]) * (d - p0);
        if (cr >= 0.f) --top;
        else break;
      }
      hx[top++] = d;
    }
    // scores: slope of the hull segment covering (d-1, d), non-increasing
    float prev = FLT_MAX;
    int seg = 0;
    for (int d = 1; d <= K; ++d) {
      while (hx[seg + 1] < d) ++seg;
      const int x0 = hx[seg], x1 = hx[seg + 1];
      float g = (R[x1] - R[x0]) / static_cast<float>(x1 - x0);
      g = fminf(g, prev);
      prev = g;
      a.scores[static_cast<size_t>(i) * K + d - 1] = g;
      s_v[i * K + d - 1] = g;
      s_i[i * K + d - 1] = i * K + d - 1;
      s_own[i * K + d - 1] = i;
    }
  }
  __syncthreads();
  // every request's scores are non-increasing: merge the n sorted runs
  merge_runs<kSchedThreads>(s_v, s_i, s_v2, s_i2, E, n, s_own, [K](int i) { return i * K; });

  // count of positive scores, then prefix sums of the sorted scores
  int pos = 0;
  for (int e = tid; e < E; e += kSchedThreads) pos += s_v[e] > 0.f;
  s_tmp[tid] = static_cast<float>(pos);
  __syncthreads();
  for (int off = kSchedThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_tmp[tid] += s_tmp[tid + off];
    __syncthreads();
  }
  const int n_pos = static_cast<int>(s_tmp[0]);
  __syncthreads();
  // prefix[B] = sum of the top B scores: s_v becomes the inclusive prefix sum
  prefix_sum<kSchedThreads>(s_v, E, s_tmp);

  // eq. (4): one candidate per (draft bucket, verify bucket) pair
  float best = -FLT_MAX;
  int bidx = 0x7fffffff;
  const int pairs = a.n_dbuckets * a.n_vbuckets;
  for (int q = tid; q < pairs; q += kSchedThreads) {
    const int bd = q / a.n_vbuckets, bv = q % a.n_vbuckets;
    const int k = min(a.d_caps[bd] - n, E);
    if (k < 0) continue;
    const int B = min(min(a.v_caps[bv] - a.n_nonspec, k), n_pos);
    if (B < 0) continue;
    const float num = static_cast<float>(n) + (B > 0 ? s_v[B - 1] : 0.f);
    const float obj = num / (a.d_lat[bd] + a.v_lat[bv]);
    if (obj > best || (obj == best && q < bidx)) {
      best = obj;
      bidx = q;
    }
  }
  s_best[tid] = best;
  s_bidx[tid] = bidx;
  __syncthreads();
  for (int off = kSchedThreads / 2; off > 0; off >>= 1) {
    if (tid < off) {
      const float ob = s_best[tid + off];
      const int oi = s_bidx[tid + off];
      if (ob > s_best[tid] || (ob == s_best[tid] && oi < s_bidx[tid])) {
        s_best[tid] = ob;
        s_bidx[tid] = oi;
      }
    }
    __syncthreads();
  }
  const int q = s_bidx[0];
  int k = 0, B = 0;
  if (q != 0x7fffffff) {
    const int bd = q / a.n_vbuckets, bv = q % a.n_vbuckets;
    k = min(a.d_caps[bd] - n, E);
    B = min(min(a.v_caps[bv] - a.n_nonspec, k), n_pos);
  }
  // draft schedule: owners of the top k scores
  for (int i = tid; i < n; i += kSchedThreads) s_d[i] = 0;
  __syncthreads();
  for (int r = tid; r < k; r += kSchedThreads) {
    const int e = s_i[r];   // an entry index (NaN scores could sort past padding)
    if (e >= 0 && e < E) atomicAdd(&s_d[e / K], 1);
  }
  __syncthreads();
  for (int i = tid; i < n; i += kSchedThreads) a.draft_len[i] = s_d[i];
  if (tid == 0) {
    a.budget[0] = B;
    if (a.objective) a.objective[0] = q != 0x7fffffff ? s_best[0] : -INFINITY;
    if (a.q_off) {
      int acc = 0;
      for (int i = 0; i < n; ++i) {
        a.q_off[i] = acc;
        acc += s_d[i];
      }
      a.q_off[n] = acc;
    }
  }
}

// ------------------------------------------------------- post-draft estimator
// p_m = sigmoid((w_h . h_m + w_s . (sh_m * E_pred[prev_m]) + c) / theta_j)
__global__ __launch_bounds__(64) void sched_post_logit(SchedPostArgs a) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x;
  const int total = min(a.q_off[a.n], a.M);
  if (m >= total) return;
  int lo = 0, hi = a.n;   // request of row m: largest i with q_off[i] <= m
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.q_off[mid] <= m) lo = mid;
    else hi = mid;
  }
  const int j = m - a.q_off[lo] + 1;   // 1-based position
  const int prev = clampi(j == 1 ? a.anchor[lo] : a.tokens[m - 1], 0, a.V - 1);
  const uint16_t* h = a.hidden + static_cast<size_t>(m) * a.H;
  float s = 0.f;
  for (int k = 8 * lane; k < a.H; k += 8 * 64) {
    const bf16x8 x = load_bf16x8(h + k);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += a.w[k + e] * static_cast<float>(x[e]);
  }
  const float* sh = a.sh + static_cast<size_t>(m) * a.ms;
  const uint16_t* ep = a.e_pred + static_cast<size_t>(prev) * a.ms;
  for (int k = lane; k < a.ms; k += 64)
    s += a.w[a.H + k] * sh[k] * __uint_as_float(static_cast<uint32_t>(ep[k]) << 16);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    float logit = s + a.bias;
    if (a.temperature) logit /= a.temperature[clampi(j, 1, a.K) - 1];
    a.prob[m] = sigmoidf(logit);
  }
}

__global__ __launch_bounds__(kSchedThreads) void sched_budget(SchedPostArgs a) {
  __shared__ float s_va[kSchedMaxEntries], s_vb[kSchedMaxEntries];
  __shared__ int s_ia[kSchedMaxEntries], s_ib[kSchedMaxEntries];
  __shared__ int s_own[kSchedMaxEntries];
  __shared__ int s_q[kSchedMaxRequests + 1];
  __shared__ int s_b[kSchedMaxRequests];
  const int tid = threadIdx.x;
  const int n = a.n;
  for (int i = tid; i <= n; i += kSchedThreads) s_q[i] = a.q_off[i];
  __syncthreads();
  const int total = clampi(s_q[n], 0, a.M);
  float* s_v = s_va;
  int* s_i = s_ia;
  float* s_v2 = s_vb;
  int* s_i2 = s_ib;
  for (int m = tid; m < total; m += kSchedThreads) {
    s_v[m] = a.prob[m];
    s_own[m] = 0;
  }
  __syncthreads();
  // survival along each draft (thread per request); rows keep their index,
  // which is the (request, position) order
  for (int i = tid; i < n; i += kSchedThreads) {
    const int r0 = clampi(s_q[i], 0, total), r1 = clampi(s_q[i + 1], r0, total);
    float prod = 1.f;
    for (int m = r0; m < r1; ++m) {
      prod *= s_v[m];
      s_v[m] = prod;
      s_own[m] = i;
    }
  }
  __syncthreads();
  for (int m = tid; m < total; m += kSchedThreads) {
    a.survival[m] = s_v[m];
    s_i[m] = m;
  }
  __syncthreads();
  // survival is non-increasing along each draft: merge the n sorted runs
  // (request i's rows are positions s_q[i] .. s_q[i + 1] - 1, clamped)
  merge_runs<kSchedThreads>(s_v, s_i, s_v2, s_i2, total, n, s_own,
                            [&](int i) { return clampi(s_q[i], 0, total); });
  const int B = clampi(a.budget[0], 0, total);
  for (int i = tid; i < n; i += kSchedThreads) s_b[i] = 0;
  __syncthreads();
  for (int r = tid; r < B; r += kSchedThreads) {
    const int m = s_i[r];   // a row index (NaN probabilities could sort past padding)
    if (m >= 0 && m < total) atomicAdd(&s_b[s_own[m]], 1);
  }
  __syncthreads();
  for (int i = tid; i < n; i += kSchedThreads) a.verify_len[i] = s_b[i];
  if (tid == 0 && a.t_off) {
    int acc = 0;
    for (int i = 0; i < n; ++i) {
      a.t_off[i] = acc;
      acc += s_b[i] + 1;
    }
    a.t_off[n] = acc;
  }
}

}  // namespace

hipError_t launch_sched_gemm(const SchedGemmArgs& g, hipStream_t s) {
  hipError_t e = launch_kernel(sched_gemm, dim3((g.M + 31) / 32, (g.N + 31) / 32, g.ksplit),
                               dim3(64 * kGemmWaves), s, g);
  if (e == hipSuccess && g.ksplit > 1) {
    const size_t mn = static_cast<size_t>(g.M) * g.N;
    e = launch_kernel(sched_gemm_reduce, dim3(static_cast<unsigned>((mn + 255) / 256)), dim3(256), s, g);
  }
  return e;
}

hipError_t launch_schedule_draft(const SchedGemmArgs& g, const SchedArgs& a, hipStream_t s) {
  hipError_t e = launch_sched_gemm(g, s);
  const int T = a.K * (a.K + 1) / 2;
  if (e == hipSuccess) e = launch_kernel(sched_tri_logits, dim3((a.n * T + 3) / 4), dim3(256), s, a);
  if (e == hipSuccess) e = launch_kernel(sched_rewards, dim3((a.n * a.K + 255) / 256), dim3(256), s, a);
  if (e == hipSuccess) e = launch_kernel(sched_joint, dim3(1), dim3(kSchedThreads), s, a);
  return e;
}

hipError_t launch_schedule_verify(const SchedGemmArgs& g, const SchedPostArgs& a, hipStream_t s) {
  hipError_t e = launch_sched_gemm(g, s);
  if (e == hipSuccess) e = launch_kernel(sched_post_logit, dim3(a.M), dim3(64), s, a);
  if (e == hipSuccess) e = launch_kernel(sched_budget, dim3(1), dim3(kSchedThreads), s, a);
  return e;
}

}  // namespace sd
