// Sequential (Markov) correction of the draft distributions ("LongSpark",
// sec. 2.3, eqs. (7)-(8)): l_j = l_j^(0) + W_c e_c(y_{j-1}), q_j = softmax(l_j),
// y_j drawn from q_j in order, y_0 the committed token.  The base logits of
// all positions come from the LM head in parallel; only this correction and
// the sampling run position by position.
//
//   markov_init   clears the per-(position, request) draw cells.
//   markov_step   one launch per position j.  Workgroups walk 128-row vocab
//                 chunks; a wave's 32 rows x 16 requests are two 16x16x32 MFMA
//                 products W_c[16 x r] e_c(y_{j-1})^T[r x 16] (bf16, fp32
//                 accumulation), the epilogue adds them to the logits in place
//                 and folds (max, sum exp) and the Gumbel-max candidate with
//                 the stream-0 uniforms of position j.  A lane owns 4
//                 consecutive vocab entries of one request: one Philox call.
//                 Each workgroup stores its (max, sum exp) and merges its
//                 candidate into one of the request's 16 draw cells with a
//                 64-bit atomic max on (ordered key, ~index); the next
//                 position reads y_j as the largest of the 16 cells, without
//                 a merge launch.  (All workgroups on one cell would
//                 serialise: each cell group is a separate 512-byte block.)
//   markov_final  lse of every (request, position) from the stored partials
//                 and the drawn tokens from the cells.
// The same launch computes the "DeLS-Spec" fusion with its Markov local head:
// the correction is scaled by alpha and a fixed per-vocab bias (minus beta
// times the log unigram prior, from log_prior_bias) is added to every row.
// The positions follow each other on the stream; nothing returns to the host.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kVChunk = 128;   // vocab rows per chunk (4 waves x 32)
constexpr int kRTile = 16;     // requests per workgroup
constexpr int kKSteps = 8;     // 32-wide k-steps whose operands load together
constexpr int kStepGrid = 512; // workgroups per request tile: two per CU

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// (key, index) -> 64-bit word whose unsigned order is `better`'s order:
// larger key first, then the smaller index.
__device__ __forceinline__ unsigned long long pack_cand(float key, int idx) {
  const uint32_t u = __float_as_uint(key);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(o) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int cand_index(unsigned long long w) {
  return static_cast<int>(~static_cast<uint32_t>(w));
}

// Draw cell `sub` of (position j, request b); cells of one (j, sub) group
// are contiguous, groups are cell_stride words apart.
__device__ __forceinline__ size_t cell_at(const MarkovArgs& a, int j, int sub, int b) {
  return (static_cast<size_t>(j - 1) * kMarkovCells + sub) * a.cell_stride + b;
}

// y_j of request b: the best of its cells.
__device__ __forceinline__ int drawn_token(const MarkovArgs& a, int j, int b) {
  unsigned long long w = 0;
#pragma unroll
  for (int c = 0; c < kMarkovCells; ++c) {
    const unsigned long long x = a.cell[cell_at(a, j, c, b)];
    w = x > w ? x : w;
  }
  return clampi(cand_index(w), 0, a.V - 1);
}

// Folds value x of vocab entry v into (mx, se) and the Gumbel-max candidate.
__device__ __forceinline__ void fold_entry(float x, float g, int v, float& mx, float& se, Cand& best) {
  if (x > mx) {
    se = se * __builtin_amdgcn_exp2f((mx - x) * kLog2e) + 1.f;
    mx = x;
  } else {
    se += __builtin_amdgcn_exp2f((x - mx) * kLog2e);
  }
  const float key = x + g;
  if (better(key, v, best.key, best.idx)) best = Cand{key, v};
}

__device__ __forceinline__ void merge_stats(float& mx, float& se, float omx, float ose) {
  const float nmx = fmaxf(mx, omx);
  se = se * __builtin_amdgcn_exp2f((mx - nmx) * kLog2e) + ose * __builtin_amdgcn_exp2f((omx - nmx) * kLog2e);
  mx = nmx;
}

__device__ __forceinline__ void active_row(const MarkovArgs& a, int b, int j, bool& active, int& m) {
  const int q0 = clampi(a.q_off[b], 0, a.M);
  const int kb = clampi(a.q_off[b + 1], q0, a.M) - q0;
  active = j <= kb && j <= a.max_k;
  m = q0 + j - 1;
}

__global__ __launch_bounds__(256) void markov_init(MarkovArgs a) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < static_cast<size_t>(a.max_k) * kMarkovCells * a.cell_stride) a.cell[i] = 0ull;
}

// Workgroup (p, tile) walks the chunks p, p + gridDim.x, ... for requests
// tile * 16 .. + 15.  Lane l: request column l % 16, k-group l / 16; its
// accumulator holds vocab rows 4 (l / 16) + i of the 16-row tile.
__global__ __launch_bounds__(256) void markov_step(MarkovArgs a, int j) {
  __shared__ float4 red[4][kRTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, col = lane & 15;
  const int b = blockIdx.y * kRTile + col;

  bool active = false;
  int m = 0;
  uint32_t rid = 0;
  int y = 0;
  if (b < a.batch) {
    active_row(a, b, j, active, m);
    rid = a.req_id[b];
    y = j == 1 ? clampi(a.anchor[b], 0, a.V - 1) : drawn_token(a, j - 1, b);
  }
  float* row = a.logits + static_cast<size_t>(m) * a.V;
  const uint16_t* er = a.e_c + static_cast<size_t>(y) * a.r + 8 * q;
  const bool one_k_chunk = a.r <= 32 * kKSteps;
  bf16x8 bv[kKSteps];
  if (one_k_chunk) {
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) bv[s] = 32 * s + 8 * q < a.r ? load_bf16x8(er + 32 * s) : zero_bf16x8();
  }

  float mx = -FLT_MAX, se = 0.f;
  Cand best{-FLT_MAX, 0x7fffffff};
  for (int chunk = blockIdx.x; chunk < a.n_chunks; chunk += gridDim.x) {
    const int vw = chunk * kVChunk + 32 * wave;       // first vocab row of this wave
    // base logits (and the vocab bias) first, so that their latency
    // overlaps the W_c loads
    float4 l[2], vb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int v = vw + 16 * t + 4 * q;
      if (active && a.vec4 && v + 3 < a.V) {
        l[t] = *reinterpret_cast<const float4*>(row + v);
      } else {
        l[t].x = active && v < a.V ? row[v] : 0.f;
        l[t].y = active && v + 1 < a.V ? row[v + 1] : 0.f;
        l[t].z = active && v + 2 < a.V ? row[v + 2] : 0.f;
        l[t].w = active && v + 3 < a.V ? row[v + 3] : 0.f;
      }
      vb[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.vbias && active) {
        if (a.vec4 && v + 3 < a.V) {
          vb[t] = *reinterpret_cast<const float4*>(a.vbias + v);
        } else {
          vb[t].x = v < a.V ? a.vbias[v] : 0.f;
          vb[t].y = v + 1 < a.V ? a.vbias[v + 1] : 0.f;
          vb[t].z = v + 2 < a.V ? a.vbias[v + 2] : 0.f;
          vb[t].w = v + 3 < a.V ? a.vbias[v + 3] : 0.f;
        }
      }
    }
    // A operands: W_c rows vw + 16 t + col, every k-step of a k-chunk in flight
    const uint16_t* wr0 = a.w_c + static_cast<size_t>(min(vw + col, a.V - 1)) * a.r + 8 * q;
    const uint16_t* wr1 = a.w_c + static_cast<size_t>(min(vw + 16 + col, a.V - 1)) * a.r + 8 * q;
    f32x4 acc0 = {}, acc1 = {};
    for (int k0 = 0; k0 < a.r; k0 += 32 * kKSteps) {
      bf16x8 a0[kKSteps], a1[kKSteps];
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bool in = k0 + 32 * s + 8 * q < a.r;
        a0[s] = in ? load_bf16x8(wr0 + k0 + 32 * s) : zero_bf16x8();
        a1[s] = in ? load_bf16x8(wr1 + k0 + 32 * s) : zero_bf16x8();
      }
      if (!one_k_chunk) {
#pragma unroll
        for (int s = 0; s < kKSteps; ++s)
          bv[s] = k0 + 32 * s + 8 * q < a.r ? load_bf16x8(er + k0 + 32 * s) : zero_bf16x8();
      }
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        acc0 = mfma_16x16x32(a0[s], bv[s], acc0);
        acc1 = mfma_16x16x32(a1[s], bv[s], acc1);
      }
    }
    // epilogue: corrected logits back in place, folded into the statistics
    if (active) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x4 c = t == 0 ? acc0 : acc1;
        const int v = vw + 16 * t + 4 * q;              // multiple of 4
        const float x[4] = {l[t].x + a.alpha * c[0] + vb[t].x, l[t].y + a.alpha * c[1] + vb[t].y,
                            l[t].z + a.alpha * c[2] + vb[t].z, l[t].w + a.alpha * c[3] + vb[t].w};
        if (a.vec4 && v + 3 < a.V) {
          *reinterpret_cast<float4*>(row + v) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < a.V) row[v + e] = x[e];
        }
        if (v < a.V) {
          // Gumbel-max keys; temperature 0 ranks the corrected logits themselves
          const u32x4 w = a.greedy ? u32x4{0u, 0u, 0u, 0u}
                                   : philox4x32_10(u32x4{static_cast<uint32_t>(v >> 2), static_cast<uint32_t>(j),
                                                         rid, kStreamDraft},
                                                   a.key0, a.key1);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < a.V) fold_entry(x[e], a.greedy ? 0.f : gumbel_from_bits(w[e]), v + e, mx, se, best);
        }
      }
    }
  }
  // lanes col, col + 16, col + 32, col + 48 hold the same request
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    merge_stats(mx, se, xor_shuffle(mx, o), xor_shuffle(se, o));
    const float ok = xor_shuffle(best.key, o);
    const int oi = xor_shuffle(best.idx, o);
    if (better(ok, oi, best.key, best.idx)) best = Cand{ok, oi};
  }
  if (q == 0) red[wave][col] = make_float4(mx, se, best.key, __int_as_float(best.idx));
  __syncthreads();
  if (wave == 0 && q == 0 && active) {
    float M = red[0][col].x, S = red[0][col].y;
    Cand bb{red[0][col].z, __float_as_int(red[0][col].w)};
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 p = red[w][col];
      merge_stats(M, S, p.x, p.y);
      const int pi = __float_as_int(p.w);
      if (better(p.z, pi, bb.key, bb.idx)) bb = Cand{p.z, pi};
    }
    const size_t jb = static_cast<size_t>(j - 1) * a.batch + b;
    a.part[jb * a.n_parts + blockIdx.x] = make_float2(M, S);
    atomicMax(a.cell + cell_at(a, j, blockIdx.x % kMarkovCells, b), pack_cand(bb.key, bb.idx));
  }
}

// One workgroup per (request, position): lse and the drawn token.
__global__ __launch_bounds__(256) void markov_final(MarkovArgs a) {
  __shared__ float sh[8];
  const int b = blockIdx.x, j = blockIdx.y + 1;
  bool active;
  int m;
  active_row(a, b, j, active, m);
  if (!active) return;
  const size_t jb = static_cast<size_t>(j - 1) * a.batch + b;
  const float2* p = a.part + jb * a.n_parts;
  float mx = -FLT_MAX, se = 0.f;
  for (int c = threadIdx.x; c < a.n_parts; c += 256) {
    const float2 x = p[c];
    merge_stats(mx, se, x.x, x.y);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) merge_stats(mx, se, xor_shuffle(mx, o), xor_shuffle(se, o));
  if (lane == 0) sh[wave] = mx, sh[4 + wave] = se;
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sh[0], S = sh[4];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_stats(M, S, sh[w], sh[4 + w]);
    a.lse[m] = M + logf(S);
    a.tokens[m] = drawn_token(a, j, b);
  }
}

// scale * log((c_v + lambda) / (sum_u c_u + lambda V)), one workgroup: the
// smoothed unigram log-prior, scaled (-beta for the fusion bias).
__global__ __launch_bounds__(1024) void log_prior_bias(const int64_t* counts, int V, double lam, float scale,
                                                       float* out) {
  __shared__ double sh[16];
  double s = 0.0;
  for (int v = threadIdx.x; v < V; v += 1024) s += static_cast<double>(max(counts[v], int64_t(0)));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += sh[w];
  const double den = tot + lam * V;
  for (int v = threadIdx.x; v < V; v += 1024) {
    const double c = static_cast<double>(max(counts[v], int64_t(0)));
    out[v] = static_cast<float>(scale * log((c + lam) / den));
  }
}

}  // namespace

hipError_t launch_log_prior_bias(const int64_t* counts, int V, double lam, float scale, float* out,
                                 hipStream_t s) {
  void* args[] = {const_cast<int64_t**>(&counts), &V, &lam, &scale, &out};
  return hipLaunchKernel(reinterpret_cast<const void*>(log_prior_bias), dim3(1), dim3(1024), args, 0, s);
}

hipError_t launch_markov(const MarkovArgs& a, hipStream_t s) {
  const size_t cells = static_cast<size_t>(a.max_k) * kMarkovCells * a.cell_stride;
  hipError_t e = launch_kernel(markov_init, dim3(static_cast<unsigned>((cells + 255) / 256)), dim3(256), s, a);
  const dim3 grid(a.n_parts, (a.batch + kRTile - 1) / kRTile);
  for (int j = 1; j <= a.max_k && e == hipSuccess; ++j) {
    void* args[] = {const_cast<MarkovArgs*>(&a), &j};
    e = hipLaunchKernel(reinterpret_cast<const void*>(markov_step), grid, dim3(256), args, 0, s);
  }
  if (e == hipSuccess) e = launch_kernel(markov_final, dim3(a.batch, a.max_k), dim3(256), s, a);
  return e;
}

int32_t markov_chunks(int32_t V) { return (V + kVChunk - 1) / kVChunk; }
int32_t markov_parts(int32_t V) { return min(markov_chunks(V), kStepGrid); }

}  // namespace sd
