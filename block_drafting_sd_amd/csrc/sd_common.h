// Device helpers shared by the step's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- memory
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ void store_u32x4(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Round-to-nearest-even float -> bfloat16 bits.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[i]);
  return r;
}

// ------------------------------------------------------------------ MFMA
// D = A * B + C for a 32x32 output tile, K = 16 (bf16 in, fp32 accumulate).
// Lane l holds A row (l % 32), B column (l % 32), k = 8 * (l / 32) + [0, 8);
// the output holds column (l % 32), rows 8 * (i / 4) + 4 * (l / 32) + i % 4
// for element i of the 16.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// -------------------------------------------------------------- cross-lane
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ int xor_shuffle(int v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// ------------------------------------------------------------ Philox-4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): ten rounds; each round forms the two 64-bit products of counter
// words 0 and 2 with the Philox multipliers and mixes their halves with
// words 1, 3 and the round key; the key advances by the Weyl constants
// between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    c = u32x4{hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0};
  }
  return c;
}

enum : uint32_t { kStreamDraft = 0, kStreamAccept = 1, kStreamSample = 2 };

// Gumbel noise -log(-log u) for u = (2 (x >> 9) + 1) 2^-24, in (0, 1).
// u lies in [2^-24, 1 - 2^-24] and -ln u in (2^-24, 17): both normal floats,
// so the hardware base-2 logarithm applies without the denormal and range
// handling of logf: -ln(-ln u) = -ln2 log2(-ln2 log2 u).
__device__ __forceinline__ float gumbel_from_bits(uint32_t x) {
  const float u = static_cast<float>((x >> 9) * 2u + 1u) * 5.9604644775390625e-8f;
  const float e = -kLn2 * __builtin_amdgcn_logf(u);   // -ln u > 0
  return -kLn2 * __builtin_amdgcn_logf(e);
}

// Acceptance uniform u = (x >> 8) 2^-24 in [0, 1).
__device__ __forceinline__ float accept_from_bits(uint32_t x) {
  return static_cast<float>(x >> 8) * 5.9604644775390625e-8f;
}

// Candidate (key, index) order: larger key wins, smaller index on a tie.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// ------------------------------------------------------ block reductions
template <int NT>
__device__ float block_reduce_max(float v, float* sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, xor_shuffle(v, m));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = sh[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) v = fmaxf(v, sh[i]);
  return v;
}

template <int NT>
__device__ float block_reduce_sum(float v, float* sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_shuffle(v, m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) v += sh[i];
  return v;
}

struct Cand {
  float key;
  int idx;
};

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float k = xor_shuffle(c.key, m);
    const int i = xor_shuffle(c.idx, m);
    if (better(k, i, c.key, c.idx)) c = Cand{k, i};
  }
  return c;
}

template <int NT>
__device__ Cand block_best(Cand c, float* shk, int* shi) {
  c = wave_best(c);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    shk[threadIdx.x >> 6] = c.key;
    shi[threadIdx.x >> 6] = c.idx;
  }
  __syncthreads();
  Cand r{shk[0], shi[0]};
#pragma unroll
  for (int i = 1; i < NT / 64; ++i)
    if (better(shk[i], shi[i], r.key, r.idx)) r = Cand{shk[i], shi[i]};
  return r;
}


// ------------------------------------------------- direct-to-LDS streaming
// Kernels that stream operands from HBM into a ring of LDS stages use gfx950
// direct-to-LDS loads: a load writes 16 bytes per lane straight into LDS, so
// several stages can be in flight without holding them in registers.
typedef __attribute__((address_space(3))) char lds_char;

// One direct-to-LDS load: lane l's 16 bytes at `src` land at LDS byte
// address lds + 16 l (lds wave-uniform, passed in m0).  The instruction's
// immediate offset is left at 0: the hardware adds it to the LDS address as
// well as to the global one.  Written as inline assembly so that the
// compiler does not tie later LDS reads to it with a blanket wait for every
// load in flight; the waits are explicit (wait_vmcnt) instead, so a kernel
// using it issues no other vector-memory loads inside its streaming loop.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);   // an SGPR operand
  // one wait state between the m0 write and the load that reads it
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      ::"v"(src), "s"(lds)
      : "memory", "m0");
}

// The same load with the non-temporal cache policy, for data a call reads
// once and never again (the paged KV stream): its lines are the first the
// caches give up, so the stream does not push out data that is reused.
__device__ __forceinline__ void dma16_stream(const void* src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      ::"v"(src), "s"(lds)
      : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)(p))));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for the loads of the oldest stage when `ahead` newer stages (L loads
// each) may stay in flight; ahead in [0, C].
template <int L, int C>
__device__ __forceinline__ void wait_stage(int ahead) {
  if constexpr (C == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= C) wait_vmcnt<C * L>();
    else wait_stage<L, C - 1>(ahead);
  }
}

// Workgroup barrier that the compiler may not move memory accesses across and
// that, unlike __syncthreads(), does not first drain every load in flight.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace sd
