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

// log2 of the race's uniform by the hardware logarithm. Its relative error is about 1e-7
// over all of U's values, next to 1 included (measured on MI355X against fp64).
__device__ __forceinline__ float log2_uniform(uint32_t w) { return __builtin_amdgcn_logf(uniform_open(w)); }

constexpr float kLn2f = 0.693147181f;
constexpr float kLog2Ln2f = -0.528766373f;  // log2(ln 2)

// fp32 race exponential E = -ln(U) = -log2(U) ln 2 for ranking candidates; the final
// choice is re-evaluated in fp64. The guard keeps it strictly positive.
__device__ __forceinline__ float expo32(uint32_t w) { return fmaxf(-log2_uniform(w) * kLn2f, 1e-30f); }

// log2(E) = log2(-log2 U) + log2(ln 2), for keys in the log domain.
__device__ __forceinline__ float log2_expo32(uint32_t w) {
  return __builtin_amdgcn_logf(fmaxf(-log2_uniform(w), 1e-30f)) + kLog2Ln2f;
}

// An upper bound on E = -ln(U), for lower bounds on race keys that prune tokens. The
// relative 1e-3 and absolute 1e-6 are far above the fp32 error of expo32.
__device__ __forceinline__ float expo32_upper(uint32_t w) {
  return fmaf(-log2_uniform(w) * kLn2f, 1.001f, 1e-6f);
}

// x / y by the hardware reciprocal (about 1 ulp), for fp32 ranking keys and their bounds,
// which carry margins far above it.
__device__ __forceinline__ float div_fast(float x, float y) { return x * __builtin_amdgcn_rcpf(y); }

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
// load_nt marks the load non-temporal: logits that one kernel reads once are streamed
// past the caches instead of displacing lines that are reused.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename E, int VEC>
struct Chunk;

template <>
struct Chunk<uint16_t, 8> {
  static constexpr int kVec = 8;
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_nt(const uint16_t* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v = make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ __forceinline__ void fill_neg_inf() { v = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
  __device__ __forceinline__ void select_if(bool c, const Chunk& o) {
    v.x = c ? o.v.x : v.x;
    v.y = c ? o.v.y : v.y;
    v.z = c ? o.v.z : v.z;
    v.w = c ? o.v.w : v.w;
  }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t d = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? bf16_hi(d) : bf16_lo(d);
  }
  // Runtime element index, written as a select tree on its bits so that the compiler keeps
  // the chunk in registers instead of indexing it through memory.
  __device__ __forceinline__ float get_dyn(int e) const {
    const uint32_t lo = (e & 2) ? v.y : v.x;
    const uint32_t hi = (e & 2) ? v.w : v.z;
    const uint32_t d = (e & 4) ? hi : lo;
    return (e & 1) ? bf16_hi(d) : bf16_lo(d);
  }
};

template <>
struct Chunk<float, 4> {
  static constexpr int kVec = 4;
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void load_nt(const float* p) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v = make_float4(t.x, t.y, t.z, t.w);
  }
  __device__ __forceinline__ void fill_neg_inf() { v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY); }
  __device__ __forceinline__ void select_if(bool c, const Chunk& o) {
    v.x = c ? o.v.x : v.x;
    v.y = c ? o.v.y : v.y;
    v.z = c ? o.v.z : v.z;
    v.w = c ? o.v.w : v.w;
  }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
  __device__ __forceinline__ float get_dyn(int e) const {
    const float lo = (e & 1) ? v.y : v.x;
    const float hi = (e & 1) ? v.w : v.z;
    return (e & 2) ? hi : lo;
  }
};

template <>
struct Chunk<uint16_t, 1> {
  static constexpr int kVec = 1;
  uint32_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *p; }
  __device__ __forceinline__ void load_nt(const uint16_t* p) { v = __builtin_nontemporal_load(p); }
  __device__ __forceinline__ void fill_neg_inf() { v = 0xFF80u; }
  __device__ __forceinline__ void select_if(bool c, const Chunk& o) { v = c ? o.v : v; }
  __device__ __forceinline__ float get(int) const { return bf16_lo(v); }
  __device__ __forceinline__ float get_dyn(int) const { return bf16_lo(v); }
};

template <>
struct Chunk<float, 1> {
  static constexpr int kVec = 1;
  float v;
  __device__ __forceinline__ void load(const float* p) { v = *p; }
  __device__ __forceinline__ void load_nt(const float* p) { v = __builtin_nontemporal_load(p); }
  __device__ __forceinline__ void fill_neg_inf() { v = -INFINITY; }
  __device__ __forceinline__ void select_if(bool c, const Chunk& o) { v = c ? o.v : v; }
  __device__ __forceinline__ float get(int) const { return v; }
  __device__ __forceinline__ float get_dyn(int) const { return v; }
};

__device__ __forceinline__ float to_float(uint16_t v) { return bf16_lo((uint32_t)v); }
__device__ __forceinline__ float to_float(float v) { return v; }

__device__ __forceinline__ float logit_at(const void* base, int dtype, int64_t idx) {
  if (dtype == SV_BF16) return bf16_lo((uint32_t) reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

// ------------------------------------------------------------------ wave64 reductions
// Every lane ends with the same, order-fixed result. Inside a 16-lane row the lanes
// exchange values by DPP (quad permutations, then the half-row and row mirrors), which
// the VALU does without the LDS round trip of a shuffle. Each exchange pairs lanes by an
// involution, so the two lanes of a pair combine the same two values and agree. The four
// row results then combine in a fixed order from lanes 0, 16, 32 and 48.

enum : int {
  kDppQuadXor1 = 0xB1,        // quad_perm [1,0,3,2]: lane i reads lane i ^ 1
  kDppQuadXor2 = 0x4E,        // quad_perm [2,3,0,1]: lane i reads lane i ^ 2
  kDppRowHalfMirror = 0x141,  // lane i of each 8-lane half row reads lane 7 - i
  kDppRowMirror = 0x140       // lane i of each 16-lane row reads lane 15 - i
};

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(dpp<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ int lane_of(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_of(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double lane_of(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Combine within aligned groups of `width` lanes, width a power of two up to 16.
template <class T, class Op>
__device__ __forceinline__ T row_reduce(T x, Op op, int width) {
  if (width > 1) x = op(x, dpp<kDppQuadXor1>(x));
  if (width > 2) x = op(x, dpp<kDppQuadXor2>(x));
  if (width > 4) x = op(x, dpp<kDppRowHalfMirror>(x));
  if (width > 8) x = op(x, dpp<kDppRowMirror>(x));
  return x;
}

template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  x = row_reduce(x, op, 16);
  return op(op(lane_of(x, 0), lane_of(x, 16)), op(lane_of(x, 32), lane_of(x, 48)));
}

// Groups of 32 or 64 lanes finish with shuffles between rows.
template <class T, class Op>
__device__ __forceinline__ T seg_reduce(T x, Op op, int width) {
  x = row_reduce(x, op, width < 16 ? width : 16);
  for (int o = 16; o < width; o <<= 1) x = op(x, __shfl_xor(x, o));
  return x;
}

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
  __device__ __forceinline__ double operator()(double a, double b) const { return fmax(a, b); }
};
struct OpMin {
  __device__ __forceinline__ int operator()(int a, int b) const { return min(a, b); }
};
struct OpOr {
  __device__ __forceinline__ int operator()(int a, int b) const { return a | b; }
};
struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
  __device__ __forceinline__ double operator()(double a, double b) const { return a + b; }
};

__device__ __forceinline__ float wave_max(float x) { return wave_reduce(x, OpMax{}); }
__device__ __forceinline__ double wave_max(double x) { return wave_reduce(x, OpMax{}); }
__device__ __forceinline__ int wave_min(int x) { return wave_reduce(x, OpMin{}); }
__device__ __forceinline__ int wave_or(int x) { return wave_reduce(x, OpOr{}); }
__device__ __forceinline__ float wave_sum(float x) { return wave_reduce(x, OpSum{}); }
__device__ __forceinline__ double wave_sum(double x) { return wave_reduce(x, OpSum{}); }

// Reductions over aligned groups of `width` lanes (a power of two, at most 64): every lane
// ends with its group's result, combined in a fixed order.
__device__ __forceinline__ float seg_max(float x, int width) { return seg_reduce(x, OpMax{}, width); }
__device__ __forceinline__ float seg_sum(float x, int width) { return seg_reduce(x, OpSum{}, width); }
__device__ __forceinline__ double seg_sum(double x, int width) { return seg_reduce(x, OpSum{}, width); }
__device__ __forceinline__ int seg_min(int x, int width) { return seg_reduce(x, OpMin{}, width); }

// A value every lane of the wave holds alike, moved to a scalar register.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ double uni(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Best (key, index) under "larger key wins, then lower index".
__device__ __forceinline__ bool beats(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// The best (key, index) of the wave on every lane. "beats" is a strict order on pairs,
// so the winner does not depend on the order of the exchanges.
template <int CTRL>
__device__ __forceinline__ void best_step(double& k, int& i) {
  const double ko = dpp<CTRL>(k);
  const int io = dpp<CTRL>(i);
  if (beats(ko, io, k, i)) {
    k = ko;
    i = io;
  }
}

__device__ __forceinline__ void wave_best(double& k, int& i) {
  best_step<kDppQuadXor1>(k, i);
  best_step<kDppQuadXor2>(k, i);
  best_step<kDppRowHalfMirror>(k, i);
  best_step<kDppRowMirror>(k, i);
  double bk = lane_of(k, 0);
  int bi = lane_of(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const double kr = lane_of(k, r);
    const int ir = lane_of(i, r);
    if (beats(kr, ir, bk, bi)) {
      bk = kr;
      bi = ir;
    }
  }
  k = bk;
  i = bi;
}

// Two best fp32 keys seen by a lane or a wave, k1 >= k2, equal keys ordered by
// lower index. Each entry carries the two logits its key came from, so the
// winners can be re-evaluated in fp64 without reloading them.
struct Top2 {
  float k1, k2;
  int i1, i2;
  float a1, b1, a2, b2;
};

__device__ __forceinline__ Top2 top2_empty() {
  return Top2{-INFINITY, -INFINITY, INT32_MAX, INT32_MAX, 0.0f, 0.0f, 0.0f, 0.0f};
}

__device__ __forceinline__ void top2_push(Top2& t, float k, int i, float a, float b) {
  if (!(k > t.k2 || (k == t.k2 && i < t.i2))) return;  // most draws: not among the two best
  if (k > t.k1 || (k == t.k1 && i < t.i1)) {
    t.k2 = t.k1;
    t.i2 = t.i1;
    t.a2 = t.a1;
    t.b2 = t.b1;
    t.k1 = k;
    t.i1 = i;
    t.a1 = a;
    t.b1 = b;
  } else if (k > t.k2 || (k == t.k2 && i < t.i2)) {
    t.k2 = k;
    t.i2 = i;
    t.a2 = a;
    t.b2 = b;
  }
}

__device__ __forceinline__ void wave_top2(Top2& t) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float k1 = __shfl_xor(t.k1, o), k2 = __shfl_xor(t.k2, o);
    const int i1 = __shfl_xor(t.i1, o), i2 = __shfl_xor(t.i2, o);
    const float a1 = __shfl_xor(t.a1, o), b1 = __shfl_xor(t.b1, o);
    const float a2 = __shfl_xor(t.a2, o), b2 = __shfl_xor(t.b2, o);
    top2_push(t, k1, i1, a1, b1);
    top2_push(t, k2, i2, a2, b2);
  }
}

// ------------------------------------------------------------------ hand-off between workgroups
// A record that one wave writes and another wave (maybe on another XCD) reads in the same
// kernel moves with agent-scope atomic loads and stores. Those are coherent across the
// per-XCD L2 caches by themselves, so no cache write-back fence is needed. The writer waits
// for its stores to complete before it takes the ticket, so the wave that draws the last
// ticket reads complete records.

// Records of 8-byte words move as 64-bit agent-scope atomic stores and loads.
__device__ __forceinline__ void store_dword2(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_dword2(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N>
struct Dwords {
  uint64_t w[N];
};

template <class T>
__device__ __forceinline__ void publish64(T* dst, const T& v) {
  static_assert(sizeof(T) % 8 == 0 && alignof(T) >= 8, "records of 8-byte words");
  constexpr int n = sizeof(T) / 8;
  const Dwords<n> w = __builtin_bit_cast(Dwords<n>, v);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
  for (int i = 0; i < n; ++i) store_dword2(d + i, w.w[i]);
}

template <class T>
__device__ __forceinline__ T read_record64(const T* src) {
  constexpr int n = sizeof(T) / 8;
  Dwords<n> w;
  const uint64_t* s = reinterpret_cast<const uint64_t*>(src);
#pragma unroll
  for (int i = 0; i < n; ++i) w.w[i] = load_dword2(s + i);
  return __builtin_bit_cast(T, w);
}

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
