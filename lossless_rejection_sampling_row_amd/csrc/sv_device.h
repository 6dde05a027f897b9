// sv_device.h - device helpers for the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_plan.h"

namespace sv {

// ------------------------------------------------------------------ numerics

// Temperature 0 is greedy; otherwise it must lie in [2^-14, 2^14]. NaN fails.
__device__ __forceinline__ bool temperature_ok(float T) {
  return T == 0.0f || (T >= 0x1p-14f && T <= 0x1p14f);
}

// log2(e)/T, rounded once from fp64. Every kernel derives its exponent scale
// from this one value, so all partial sums share one temperature.
__device__ __forceinline__ float scale_of(float T) {
  return (float)(1.4426950408889634 / (double)T);
}

// fl(m*c): the reference a slice's sum is taken against. An infinite maximum
// (all -inf, or a +inf logit) gives reference 0. The sum then becomes 0,
// +inf or NaN, and the row is rejected as invalid when it is merged.
__device__ __forceinline__ float ref_of(float m, float c) {
  return __builtin_isfinite(m) ? m * c : 0.0f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The smallest exponential the race can draw: -ln(1 - 2^-24), rounded down.
constexpr double kEminLow = 5.96e-8;

// ------------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11), Philox-4x32 with 10 rounds. Each round multiplies counter words 0
// and 2 by the two round constants. Word 0 of the new counter is the high half
// of the second product, xor counter word 1, xor key word 0. Word 1 is the
// low half of the second product. Words 2 and 3 follow the same pattern with
// the first product, counter word 3 and key word 1. The key advances by the
// Weyl constants after every round.
struct Philox4 {
  uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2,
                                                 uint32_t x3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t prod_a = (uint64_t)0xD2511F53u * (uint64_t)x0;
    const uint64_t prod_b = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
    const uint32_t y0 = (uint32_t)(prod_b >> 32) ^ x1 ^ k0;
    const uint32_t y2 = (uint32_t)(prod_a >> 32) ^ x3 ^ k1;
    x1 = (uint32_t)prod_b;
    x3 = (uint32_t)prod_a;
    x0 = y0;
    x2 = y2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{x0, x1, x2, x3};
}

__device__ __forceinline__ uint32_t word_of(const Philox4& p, int i) {
  return i == 0 ? p.w0 : i == 1 ? p.w1 : i == 2 ? p.w2 : p.w3;
}

// Counter layout: (block, tag, position j in the request, request b), key = seed.
constexpr uint32_t kTagAccept = 0;
constexpr uint32_t kTagRace = 1;

// Uniform on [0,1) for the accept test: top 24 bits times 2^-24 (exact in fp32).
__device__ __forceinline__ float uniform_accept(uint32_t w) { return (float)(w >> 8) * 0x1p-24f; }

// Uniform on (0,1) for the race: (2*(w >> 9) + 1) * 2^-24, exact in fp32, never 0 or 1.
__device__ __forceinline__ float uniform_open(uint32_t w) {
  return (float)((w >> 9) * 2u + 1u) * 0x1p-24f;
}

// fp32 race exponential for candidate selection. It is accurate enough to rank
// keys inside a slice; the final choice is re-evaluated in fp64. The guard
// keeps it strictly positive.
__device__ __forceinline__ float expo32(uint32_t w) {
  const float e = -__logf(uniform_open(w));
  return fmaxf(e, 1e-30f);
}

__device__ __forceinline__ double expo64(uint32_t w) { return -log((double)uniform_open(w)); }

__device__ __forceinline__ uint32_t race_word(uint64_t seed, int64_t x, int j, int b) {
  const Philox4 p = philox4x32_10((uint32_t)(x >> 2), kTagRace, (uint32_t)j, (uint32_t)b,
                                  (uint32_t)seed, (uint32_t)(seed >> 32));
  return word_of(p, (int)(x & 3));
}

// ------------------------------------------------------------------ logits

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// VEC logits held as one load. bf16 logits arrive as raw 16-bit patterns.
template <typename E, int VEC>
struct Chunk;

template <>
struct Chunk<uint16_t, 8> {
  static constexpr int kVec = 8;
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void fill_neg_inf() { v = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t d = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? bf16_hi(d) : bf16_lo(d);
  }
};

template <>
struct Chunk<float, 4> {
  static constexpr int kVec = 4;
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void fill_neg_inf() { v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY); }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};

template <>
struct Chunk<uint16_t, 1> {
  static constexpr int kVec = 1;
  uint32_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *p; }
  __device__ __forceinline__ void fill_neg_inf() { v = 0xFF80u; }
  __device__ __forceinline__ float get(int) const { return bf16_lo(v); }
};

template <>
struct Chunk<float, 1> {
  static constexpr int kVec = 1;
  float v;
  __device__ __forceinline__ void load(const float* p) { v = *p; }
  __device__ __forceinline__ void fill_neg_inf() { v = -INFINITY; }
  __device__ __forceinline__ float get(int) const { return v; }
};

__device__ __forceinline__ float logit_at(const void* base, int dtype, int64_t idx) {
  if (dtype == SV_BF16) return bf16_lo((uint32_t) reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

// ------------------------------------------------------------------ wave64 reductions
// Butterfly reductions: every lane ends with the same, order-fixed result.

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_or(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Best (key, index) under "larger key wins, then lower index".
__device__ __forceinline__ bool beats(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ void wave_best(double& k, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ko = __shfl_xor(k, o);
    const int io = __shfl_xor(i, o);
    if (beats(ko, io, k, i)) {
      k = ko;
      i = io;
    }
  }
}

// Two best fp32 keys of a slice, k1 >= k2, equal keys ordered by lower index.
struct Top2 {
  float k1, k2;
  int i1, i2;
};

__device__ __forceinline__ Top2 top2_empty() { return Top2{-1.0f, -1.0f, INT32_MAX, INT32_MAX}; }

__device__ __forceinline__ void top2_push(Top2& t, float k, int i) {
  if (k > t.k1 || (k == t.k1 && i < t.i1)) {
    t.k2 = t.k1;
    t.i2 = t.i1;
    t.k1 = k;
    t.i1 = i;
  } else if (k > t.k2 || (k == t.k2 && i < t.i2)) {
    t.k2 = k;
    t.i2 = i;
  }
}

__device__ __forceinline__ void wave_top2(Top2& t) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float a1 = __shfl_xor(t.k1, o), a2 = __shfl_xor(t.k2, o);
    const int j1 = __shfl_xor(t.i1, o), j2 = __shfl_xor(t.i2, o);
    top2_push(t, a1, j1);
    top2_push(t, a2, j2);
  }
}


// ------------------------------------------------------------------ hand-off between workgroups
// A record that one wave writes and another wave (maybe on another XCD) reads in the same
// kernel moves with agent-scope atomic loads and stores. Those are coherent across the
// per-XCD L2 caches by themselves, so no cache write-back fence is needed. The writer waits
// for its stores to complete before it takes the ticket, so the wave that draws the last
// ticket reads complete records.

__device__ __forceinline__ void store_word(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_word(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish(P1Part* dst, const P1Part& v) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  store_word(d + 0, __float_as_uint(v.m_t));
  store_word(d + 1, __float_as_uint(v.s_t));
  store_word(d + 2, __float_as_uint(v.m_d));
  store_word(d + 3, __float_as_uint(v.s_d));
  store_word(d + 4, (uint32_t)v.am_t);
  store_word(d + 5, (uint32_t)v.am_d);
  store_word(d + 6, (uint32_t)v.bad);
  store_word(d + 7, (uint32_t)v.pad);
}

__device__ __forceinline__ P1Part read_p1(const P1Part* src) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  P1Part v;
  v.m_t = __uint_as_float(load_word(s + 0));
  v.s_t = __uint_as_float(load_word(s + 1));
  v.m_d = __uint_as_float(load_word(s + 2));
  v.s_d = __uint_as_float(load_word(s + 3));
  v.am_t = (int32_t)load_word(s + 4);
  v.am_d = (int32_t)load_word(s + 5);
  v.bad = (int32_t)load_word(s + 6);
  v.pad = 0;
  return v;
}

__device__ __forceinline__ void publish(P2Part* dst, const P2Part& v) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  store_word(d + 0, __float_as_uint(v.k1));
  store_word(d + 1, __float_as_uint(v.k2));
  store_word(d + 2, (uint32_t)v.i1);
  store_word(d + 3, (uint32_t)v.i2);
  store_word(d + 4, __float_as_uint(v.rsum));
  store_word(d + 5, __float_as_uint(v.mref));
  store_word(d + 6, (uint32_t)v.bad);
  store_word(d + 7, (uint32_t)v.gidx);
}

__device__ __forceinline__ P2Part read_p2(const P2Part* src) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  P2Part v;
  v.k1 = __uint_as_float(load_word(s + 0));
  v.k2 = __uint_as_float(load_word(s + 1));
  v.i1 = (int32_t)load_word(s + 2);
  v.i2 = (int32_t)load_word(s + 3);
  v.rsum = __uint_as_float(load_word(s + 4));
  v.mref = __uint_as_float(load_word(s + 5));
  v.bad = (int32_t)load_word(s + 6);
  v.gidx = (int32_t)load_word(s + 7);
  return v;
}

// Arrive at a counter shared by `total` waves. Returns true in the wave that arrives last.
// The counter wraps back to zero on the last arrival, ready for the next call.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's published records have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t old = 0;
  if (lane == 0) old = atomicInc(counter, total - 1);
  old = __shfl(old, 0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return old == total - 1;
}

}  // namespace sv
