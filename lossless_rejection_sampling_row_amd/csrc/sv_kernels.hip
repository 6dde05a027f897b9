// sv_kernels.hip - the verify sampler's kernels and the exported C-ABI calls.
//
// Pass 1 streams the target and draft logits of every proposal row once.
// Rows are split into spans. One long-lived wave per span:
//  - reads the span with double-buffered 16-byte loads;
//  - keeps per-lane running softmax statistics (max, sum of exp2 against that
//    max) and where the maximum sits;
//  - picks up the logits at the drafted token D from registers;
//  - writes one 48-byte partial.
// There is no cross-workgroup traffic in pass 1: it is a pure stream.
//
// Pass 2 draws each request's last token.
//  - Every wave of a request first rebuilds the request from pass 1's
//    partials. It merges each row's statistics in fp64 and runs the accept
//    test row by row until the first row that is not accepted. The test
//    follows Strata PR #3416 "[Engine] Preserve target probabilities in gated
//    MTP", section Approach, with the accept form of mlxcel PR #992, section
//    What changed. The stop rule follows mlxcel PR #992, section Two metric
//    corrections.
//  - The last token comes from the row that ended the request: a residual
//    draw from (p - mu)+, a bonus draw from p, or the greedy argmax.
//  - The draw is an exponential race argmax_x w_x / E_x, with ties going to
//    the lower index.
//  - Each wave streams a span and prunes tokens that provably cannot win
//    before drawing their random numbers. It re-evaluates its two best fp32
//    candidates in fp64.
//  - The request's last wave (atomic ticket) merges and writes the outputs.
//  - Two instances: the plain call's, and the diagnostic / scheduled calls',
//    which also reports the residual mass and applies per-row gate schedules
//    and the cumulative floor (regolith audit, section schedule behavior).
//
// Other entry points reuse these pieces:
//  - the lazy verify streams row j of the still-open requests in launch j
//    (lazy_rows_kernel), then runs pass 2;
//  - the acceptance sums run pass 1, stream every proposal row again for
//    sum min(p, mu) and sum p q (sums_kernel), and add the per-wave partials
//    (merge_sums_kernel).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "sv_device.h"
#include "sv_plan.h"

namespace sv {

// One side's filter parameters: [B] device arrays, each optional (null: that filter off).
struct FilterSide {
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
};

struct FilterArgs {
  FilterSide side[2];  // target, draft
  float* theta;        // [R][2] keep-thresholds, written by thresholds_kernel
  // With segment records (16-byte rows of at most kSegCap segments): the records, [R][2][nseg],
  // and per row and side the statistics pass 1 can take instead of streaming the row.
  SegRec* seg = nullptr;
  int32_t nseg = 0;
  FiltStat* fstat = nullptr;
  // Filtered verify only: skip the row sides the verify never reads (side_unused).
  int32_t skip_unused = 0;
};

struct Inputs {
  const void* target;
  const void* draft;
  const int32_t* dt;
  const int32_t* ro;
  const float* temp;
  const float* tau;
  const float* tau_step;  // [R] per-row step thresholds, or null (tau[b] for every row)
  const float* min_cum;   // [B] cumulative floors, or null (no cumulative gate)
  uint64_t seed;
  int32_t B, R, V, dtype;
  int32_t w1;  // pass 1: waves per row
  int32_t w2;  // pass 2: waves per request
  // Filtered verify only: each row's keep-thresholds [R][2] (target, draft) and the filter
  // parameters, whose validity pass 2 checks per request.
  const float* theta = nullptr;
  FilterSide filt[2] = {{nullptr, nullptr, nullptr}, {nullptr, nullptr, nullptr}};
  // With the filter chain's segment records: [R][2] statistics of the rows it decided.
  const FiltStat* fstat = nullptr;
};

struct FilterParams {
  int k;
  float top_p, min_p;
};

__device__ __forceinline__ FilterParams filter_params(const FilterSide& f, int b) {
  FilterParams p;
  p.k = f.top_k != nullptr ? f.top_k[b] : 0;
  p.top_p = f.top_p != nullptr ? f.top_p[b] : 1.0f;
  p.min_p = f.min_p != nullptr ? f.min_p[b] : 0.0f;
  return p;
}

// Parameter ranges. NaN fails every comparison, so a NaN top_p or min_p is invalid.
__device__ __forceinline__ bool filter_valid(const FilterParams& p) {
  return p.k >= 0 && p.top_p > 0.0f && p.min_p >= 0.0f && p.min_p <= 1.0f;
}

struct Work {
  WsHeader* hdr;
  P1Part* part1;
  P2Part* part2;
  uint32_t* t2;  // pass 2: waves finished per request
  SumPart* part3;   // acceptance sums: one partial per (row, wave)
  uint32_t* done3;  // acceptance sums: rows that hold partials (reset by the merge)
  int32_t* lazy_stop;  // lazy verify: the request's window has stopped
  // Bonus races: per request, the largest (logit, token) any of its waves has seen, packed by
  // pack_best. Zero between calls: the request's merging wave clears it.
  uint64_t* bmax = nullptr;
};

struct Outputs {
  int32_t* tokens;
  int32_t* accept_len;
  sv_row_diag* diag;
  sv_batch_stats* stats;
};

__device__ __forceinline__ uint32_t seed_lo(uint64_t s) { return (uint32_t)s; }
__device__ __forceinline__ uint32_t seed_hi(uint64_t s) { return (uint32_t)(s >> 32); }

// Vector indices [begin, end) of wave g among `nwaves` waves that share a row. A row
// holds fewer than 2^28 logits, so vector indices and byte offsets within a row fit in
// 32 bits.
struct Span {
  int begin, end;
};

__device__ __forceinline__ Span wave_span(int nvec, int nwaves, int g) {
  int per = (nvec + nwaves - 1) / nwaves;
  per = (per + kWave - 1) / kWave * kWave;
  const int b = min(g * per, nvec);
  const int e = min(b + per, nvec);
  return Span{b, e};
}

__device__ __forceinline__ sv_row_diag untested_diag() {
  sv_row_diag d;
  d.p_D = d.q_D = d.mu_D = d.u = d.resid_mass = NAN;
  d.verdict = SV_ROW_UNTESTED;
  d.pad0 = d.pad1 = 0;
  return d;
}

// Temperature 0 (greedy) rows fold their logits with scale 1: their sums are not needed
// for p, but a NaN, a +inf or an all -inf row makes them non-finite or zero, which is the
// validity test.
__device__ __forceinline__ float fold_scale(float T) { return T == 0.0f ? 1.0f : scale_of(T); }

// ====================================================================== pass 1

// Pass 1 streams the potential proposal rows: every row but the last of its request. Slot
// p of the pass-1 grid is the p-th of them, row r = p + b of request b, where b is the
// largest request index with ro[b] - b <= p.
struct RowCls {
  bool proposal;  // the slot's row is tested by the method
  int r;          // the row, always inside [0, R)
  int b, lo, j;   // request, its first row, and r's position in it
  int D;          // drafted token of row r
  float T, tau;
};

// The slot's request when every request has the same number of rows.
__device__ __forceinline__ int slot_guess(const Inputs& in, int p) {
  const int np = in.R - in.B;
  return min((int)(((int64_t)p * in.B) / np), in.B - 1);
}

// Classify slot p in one round trip when the guess holds: the request's range, temperature
// and tau, and the drafted tokens of the 64 rows ending at r are requested together. A
// wrong guess (requests of different lengths) costs a binary search. Every index stays in
// bounds whatever row_offsets holds; a broken batch is caught by block 0's check and fails
// closed in pass 2.
__device__ RowCls classify_slot(const Inputs& in, int p, int b, int lane) {
  RowCls c{};
  int lo = in.ro[b], hi = in.ro[b + 1];
  float T = in.temp[b], tau = in.tau[b];
  int r = min(max(p + b, 0), in.R - 1);
  int dwin = in.dt[max(r - lane, 0)];  // lane i: drafted token of row r - i
  if (!(lo <= p + b && p + b < hi - 1)) {
    int L = 0, H = in.B - 1;  // largest b with ro[b] - b <= p
    while (L < H) {
      const int mid = (L + H + 1) >> 1;
      if (in.ro[mid] - mid <= p) L = mid; else H = mid - 1;
    }
    b = L;
    lo = in.ro[b];
    hi = in.ro[b + 1];
    T = in.temp[b];
    tau = in.tau[b];
    r = min(max(p + b, 0), in.R - 1);
    dwin = in.dt[max(r - lane, 0)];
  }
  c.r = r;
  if (!(0 <= lo && lo <= p + b && p + b < hi - 1 && hi <= in.R)) return c;
  c.b = b;
  c.lo = lo;
  c.j = r - lo;
  c.T = T;
  c.tau = tau;
  // Rows lo..r must all carry a drafted token in [0, V): the request stops at the first
  // row without one.
  bool bad = lane <= c.j && (dwin < 0 || dwin >= in.V);
  c.D = lane_of(dwin, 0);
  for (int base = kWave; base <= c.j && !__ballot(bad); base += kWave) {  // windows beyond 64 rows
    const int D = in.dt[max(r - base - lane, 0)];
    bad = base + lane <= c.j && (D < 0 || D >= in.V);
  }
  c.proposal = temperature_ok(T) && !__builtin_isnan(tau) && __ballot(bad) == 0;
  return c;
}

// Running statistics of one lane over one array.
struct Acc {
  float m;   // max logit seen
  float mc;  // ref_of(m, c): the reference of s
  float s;   // sum of exp2(l*c - mc)
  int am;    // first index holding m
};

__device__ __forceinline__ Acc acc_empty() { return Acc{-INFINITY, 0.0f, 0.0f, INT32_MAX}; }

// Fold U chunks of one array into a lane's running softmax statistics (temperature > 0).
// Chunk u of this lane sits at vector index vb + u*64. With ARG, `am` tracks the vector
// index of the first chunk that holds the lane's maximum: a cheap, branch-free hint of
// where the row's large logits are (it only steers pruning in pass 2).
// With FILT, tokens below the row's keep-threshold th add nothing to the sum; the maximum
// is taken over every token (the largest logit always survives the filters).
template <bool ARG, bool FILT = false, class CH, int U>
__device__ __forceinline__ void fold_soft(Acc& a, const CH (&x)[U], int vb, float c, float th = -INFINITY) {
  constexpr int VEC = CH::kVec;
  float vm[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float m = x[u].get(0);
#pragma unroll
    for (int e = 1; e < VEC; ++e) m = fmaxf(m, x[u].get(e));
    vm[u] = m;
  }
  float bm = vm[0];
#pragma unroll
  for (int u = 1; u < U; ++u) bm = fmaxf(bm, vm[u]);
  if (ARG) {
    int h = U - 1;
#pragma unroll
    for (int u = U - 2; u >= 0; --u) h = (vm[u] == bm) ? u : h;
    a.am = (bm > a.m) ? vb + h * kWave : a.am;
  }
  const float mn = fmaxf(a.m, bm);
  const float mcn = ref_of(mn, c);
  a.s = (a.s != 0.0f) ? a.s * fast_exp2(a.mc - mcn) : 0.0f;  // exactly 1 unless the max grew
  a.mc = mcn;
  a.m = mn;
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // Every logit of the chunk below the threshold: nothing to add. (A filtered row with a NaN
    // has th = +inf, so its sum stays 0 and the row fails; an unfiltered one has th = -inf.)
    if (FILT && vm[u] < th) continue;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float t = fast_exp2(fmaf(x[u].get(e), c, -a.mc));
      if (FILT) t = x[u].get(e) < th ? 0.0f : t;
      if ((u * VEC + e) & 1) s1 += t; else s0 += t;
    }
  }
  a.s += s0 + s1;
}

// Fold U chunks into a lane's maximum and the NaN / +inf check (greedy rows, and bonus
// rows, which no softmax sum validates). With ARG, `am` tracks the vector index of the
// first chunk holding the maximum; exact_argmax resolves the element after the span.
template <bool ARG, class CH, int U>
__device__ __forceinline__ void fold_max(Acc& a, const CH (&x)[U], int vb, int& bad) {
  constexpr int VEC = CH::kVec;
  float vm[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float v = x[u].get(e);
      m = fmaxf(m, v);
      bad |= (int)(__builtin_isnan(v) || v == INFINITY);
    }
    vm[u] = m;
  }
  float bm = vm[0];
#pragma unroll
  for (int u = 1; u < U; ++u) bm = fmaxf(bm, vm[u]);
  if (ARG) {
    int h = U - 1;
#pragma unroll
    for (int u = U - 2; u >= 0; --u) h = (vm[u] == bm) ? u : h;
    a.am = (bm > a.m) ? vb + h * kWave : a.am;
  }
  a.m = fmaxf(a.m, bm);
}

// Lowest element index holding the wave maximum wm, given each lane's maximum and the
// vector index of the first of its chunks that holds it. The lanes that hold wm re-read
// that one vector (a cache hit) and scan it.
template <class CH, typename E>
__device__ __forceinline__ int exact_argmax(const E* row, const Acc& a, float wm) {
  constexpr int VEC = CH::kVec;
  int idx = INT32_MAX;
  if (a.m == wm && wm != -INFINITY) {
    CH x;
    x.load(row + (int64_t)a.am * VEC);
#pragma unroll
    for (int e = VEC - 1; e >= 0; --e) idx = (x.get(e) == wm) ? a.am * VEC + e : idx;
  }
  idx = wave_min(idx);
  return idx == INT32_MAX ? -1 : idx;
}

// Load U chunks for lane `lane` of a wave whose chunk 0 starts at vector index wb. Every lane
// loads, with no branch around the loads so that they stay in flight together. A lane past
// the span's end re-reads the span's last vector (a cache hit) and is masked by mask_chunks.
// The row pointer is wave-uniform and the offset a 32-bit byte count, so each load takes
// a scalar base and one vector register of offset.
// With NT the loads are non-temporal (pass 1 reads each logit once).
template <bool NT, class CH, int U, typename E>
__device__ __forceinline__ void load_chunks(CH (&x)[U], const E* row, int wb, int lane, int vend) {
  constexpr uint32_t kBytes = CH::kVec * sizeof(E);
  const char* base = reinterpret_cast<const char*>(row);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = min(wb + u * kWave + lane, vend - 1);
    const E* ptr = reinterpret_cast<const E*>(base + (uint32_t)vi * kBytes);
    if (NT) x[u].load_nt(ptr);
    else x[u].load(ptr);
  }
}

// Turn the chunks of lanes past the span's end into -inf. Wave-uniform test per chunk row.
template <class CH, int U>
__device__ __forceinline__ void mask_chunks(CH (&x)[U], int wb, int lane, int vend) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int w0 = wb + u * kWave;
    if (w0 + kWave > vend) {
      CH ninf;
      ninf.fill_neg_inf();
      x[u].select_if(w0 + lane >= vend, ninf);
    }
  }
}

// Reduce a lane statistic to the wave: max, lowest index of the max, and the sum
// re-referenced to the wave maximum.
__device__ __forceinline__ void wave_stat(const Acc& a, float c, bool sums, float& m, float& s, int& am) {
  m = wave_max(a.m);
  int idx = (a.m == m && m != -INFINITY) ? a.am : INT32_MAX;
  idx = wave_min(idx);
  am = idx == INT32_MAX ? -1 : idx;
  s = 0.0f;
  if (sums) {
    const float mcw = ref_of(m, c);
    const float term = (a.s != 0.0f) ? a.s * fast_exp2(a.mc - mcw) : 0.0f;
    s = wave_sum(term);
  }
}

// Block 0 checks row_offsets for the whole batch and clears the stats. With max_rows > 0 a
// request of more rows than that also fails the batch (the lazy verify streams only that many).
__device__ void block0_duties(const Inputs& in, const Work& w, const Outputs& out, int max_rows = 0) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  if (threadIdx.x == 0) bad = (in.ro[0] != 0) || (in.ro[in.B] != in.R);
  for (int i = threadIdx.x; i < in.B; i += kBlock)
    bad |= !(in.ro[i] < in.ro[i + 1]) || (max_rows > 0 && in.ro[i + 1] - in.ro[i] > max_rows);
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) w.hdr->ro_valid = s_bad ? 0 : 1;
  constexpr int kStats = (int)(sizeof(sv_batch_stats) / sizeof(int64_t));
  if (out.stats != nullptr && threadIdx.x < kStats) reinterpret_cast<int64_t*>(out.stats)[threadIdx.x] = 0;
}



// Waves, not workgroups, are assigned to slots: wave gw of the grid streams span gw % w1 of
// slot gw / w1, so the split need not be a multiple of a workgroup's four waves.
// Stream span sp of proposal row r, both arrays, and write the wave's partial at slot g of
// the row. ta / da already hold the span's first batch (requested by the caller, so that it
// travels with the caller's own round trips).
template <typename E, int VEC, int U, bool FILT = false>
__device__ __forceinline__ void stream_span(const Inputs& in, const Work& w, int r, int g, float T, int D,
                                            const E* trow, const E* drow, Span sp, Chunk<E, VEC> (&ta)[U],
                                            Chunk<E, VEC> (&da)[U], int lane, float th_t = -INFINITY,
                                            float th_d = -INFINITY) {
  using CH = Chunk<E, VEC>;
  constexpr int step = U * kWave;
  CH tb[U], db[U];
  const bool greedy = T == 0.0f;
  const float c = fold_scale(T);
  const int dvec = D / VEC;
  const int de = D - dvec * VEC;
  const bool holds_D = dvec >= sp.begin && dvec < sp.end;  // only this span's wave reads D's logits

  Acc at = acc_empty(), ad = acc_empty();
  int found = 0;
  float ltD = 0.0f, ldD = 0.0f;

  auto fold_both = [&](const CH (&xt)[U], const CH (&xd)[U], int wb) __attribute__((always_inline)) {
    const int vb = wb + lane;
    fold_soft<true, FILT>(at, xt, vb, c, th_t);
    fold_soft<true, FILT>(ad, xd, vb, c, th_d);
    if (holds_D) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (vb + u * kWave == dvec) {
          found = 1;
          ltD = xt[u].get_dyn(de);
          ldD = xd[u].get_dyn(de);
        }
      }
    }
  };

  // Double buffering: the next batch is in flight while the current one is folded. The
  // loop leaves only at its bottom (an exit in the middle makes the compiler wait for every
  // outstanding load at the top of each step), so with an odd step count the last pass
  // folds one batch that is masked to -inf entirely, which changes nothing.
  const int nsteps = (sp.end - sp.begin + step - 1) / step;
  for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
    load_chunks<true>(tb, trow, base + step, lane, sp.end);  // past the end: clamped re-reads
    load_chunks<true>(db, drow, base + step, lane, sp.end);
    mask_chunks(ta, base, lane, sp.end);
    mask_chunks(da, base, lane, sp.end);
    fold_both(ta, da, base);
    load_chunks<true>(ta, trow, base + 2 * step, lane, sp.end);
    load_chunks<true>(da, drow, base + 2 * step, lane, sp.end);
    mask_chunks(tb, base + step, lane, sp.end);
    mask_chunks(db, base + step, lane, sp.end);
    fold_both(tb, db, base + step);
  }

  P1Part pp{};
  wave_stat(at, c, true, pp.m_t, pp.s_t, pp.am_t);
  wave_stat(ad, c, true, pp.m_d, pp.s_d, pp.am_d);
  if (greedy) {
    pp.am_t = exact_argmax<CH>(trow, at, pp.m_t);
    pp.am_d = exact_argmax<CH>(drow, ad, pp.m_d);
  } else {
    pp.am_d = -1;
  }
  const uint64_t fm = __ballot(found);
  const int src = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
  pp.lt_D = lane_of(ltD, src);
  pp.ld_D = lane_of(ldD, src);
  pp.flags = fm ? 2 : 0;
  if (lane == 0) w.part1[(int64_t)r * in.w1 + g] = pp;  // read by pass 2, after this kernel
}

// The filtered verify's rows where the filter chain decided one side only: stream the other
// side's array (side 0 target, 1 draft) as stream_span does, and take the decided side's
// statistics from the chain (wave 0 carries them whole, the others none) and its drafted-token
// logit from the same record. Rows with a chain record always hold a valid drafted token.
template <typename E, int VEC, int U, bool FILT>
__device__ __forceinline__ void stream_one(const Inputs& in, const Work& w, int r, int g, float T, int D,
                                           const E* row, Span sp, Chunk<E, VEC> (&xa)[U], int lane, float th,
                                           int side, const FiltStat& other) {
  using CH = Chunk<E, VEC>;
  constexpr int step = U * kWave;
  CH xb[U];
  const float c = fold_scale(T);
  const int dvec = D / VEC;
  const int de = D - dvec * VEC;
  const bool holds_D = dvec >= sp.begin && dvec < sp.end;
  Acc a = acc_empty();
  int found = 0;
  float lD = 0.0f;
  auto fold1 = [&](const CH (&x)[U], int wb) __attribute__((always_inline)) {
    const int vb = wb + lane;
    fold_soft<true, FILT>(a, x, vb, c, th);
    if (holds_D) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (vb + u * kWave == dvec) {
          found = 1;
          lD = x[u].get_dyn(de);
        }
      }
    }
  };
  const int nsteps = (sp.end - sp.begin + step - 1) / step;
  for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
    load_chunks<true>(xb, row, base + step, lane, sp.end);
    mask_chunks(xa, base, lane, sp.end);
    fold1(xa, base);
    load_chunks<true>(xa, row, base + 2 * step, lane, sp.end);
    mask_chunks(xb, base + step, lane, sp.end);
    fold1(xb, base + step);
  }
  float m, sum;
  int am;
  wave_stat(a, c, true, m, sum, am);
  const uint64_t fm = __ballot(found);
  const float lDw = lane_of(lD, fm ? __ffsll((unsigned long long)fm) - 1 : 0);
  const float om = g == 0 ? other.m : -INFINITY;
  const float os = g == 0 ? other.s : 0.0f;
  P1Part pp{};
  if (side == 0) {
    pp = P1Part{m, sum, om, os, am, -1, fm ? 2 : 0, lDw, other.lD, {0, 0, 0}};
  } else {
    pp = P1Part{om, os, m, sum, -1, -1, fm ? 2 : 0, other.lD, lDw, {0, 0, 0}};
  }
  if (lane == 0) w.part1[(int64_t)r * in.w1 + g] = pp;  // read by pass 2, after this kernel
}

template <typename E, int VEC, int U, bool FILT = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void pass1_kernel(Inputs in, Work w,
                                                                                             Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (blockIdx.x == 0) block0_duties(in, w, out);
  const int np = in.R - in.B;
  if (gw >= (int64_t)np * in.w1) return;
  const int p = (int)(gw / in.w1);
  const int g = (int)(gw % in.w1);

  using CH = Chunk<E, VEC>;
  const int nvec = in.V / VEC;
  const Span sp = wave_span(nvec, in.w1, g);
  const int bg = slot_guess(in, p);
  const int rg = min(p + bg, in.R - 1);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)rg * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)rg * in.V;
  CH ta[U], da[U];
  // The first batch of the guessed row (and, filtered, its keep-thresholds) is requested
  // before the slot is classified, so the row's metadata and its first logits arrive together.
  if (sp.begin < sp.end) {
    load_chunks<true>(ta, trow, sp.begin, lane, sp.end);
    load_chunks<true>(da, drow, sp.begin, lane, sp.end);
  }
  float th_t = -INFINITY, th_d = -INFINITY;
  FiltStat ft{}, fd{};
  if (FILT) {
    th_t = in.theta[2 * (int64_t)rg];
    th_d = in.theta[2 * (int64_t)rg + 1];
    if (in.fstat != nullptr) {
      ft = in.fstat[2 * (int64_t)rg];
      fd = in.fstat[2 * (int64_t)rg + 1];
    }
  }
  const RowCls cls = classify_slot(in, p, bg, lane);
  if (!cls.proposal) return;
  const int r = cls.r;
  if (FILT && r != rg) {
    th_t = in.theta[2 * (int64_t)r];
    th_d = in.theta[2 * (int64_t)r + 1];
    if (in.fstat != nullptr) {
      ft = in.fstat[2 * (int64_t)r];
      fd = in.fstat[2 * (int64_t)r + 1];
    }
  }
  if (FILT && in.fstat != nullptr && ft.ok != 0 && fd.ok != 0) {
    // The filter chain decided both sides from their candidates and kept the row's statistics:
    // wave 0's partial carries them whole (and the drafted token's logits), the others none.
    P1Part pp{};
    if (g == 0) {
      pp = P1Part{ft.m, ft.s, fd.m, fd.s, -1, -1, 2, ft.lD, fd.lD, {0, 0, 0}};
    } else {
      pp = P1Part{-INFINITY, 0.0f, -INFINITY, 0.0f, -1, -1, 0, 0.0f, 0.0f, {0, 0, 0}};
    }
    if (lane == 0) w.part1[(int64_t)r * in.w1 + g] = pp;
    return;
  }
  if (r != rg) {  // the guess missed: stream the right row
    trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
    drow = reinterpret_cast<const E*>(in.draft) + (int64_t)r * in.V;
    if (sp.begin < sp.end) {
      load_chunks<true>(ta, trow, sp.begin, lane, sp.end);
      load_chunks<true>(da, drow, sp.begin, lane, sp.end);
    }
  }

  if (FILT && in.fstat != nullptr && (ft.ok != 0) != (fd.ok != 0)) {
    if (ft.ok == 0)
      stream_one<E, VEC, U, FILT>(in, w, r, g, cls.T, cls.D, trow, sp, ta, lane, th_t, 0, fd);
    else
      stream_one<E, VEC, U, FILT>(in, w, r, g, cls.T, cls.D, drow, sp, da, lane, th_d, 1, ft);
    return;
  }
  stream_span<E, VEC, U, FILT>(in, w, r, g, cls.T, cls.D, trow, drow, sp, ta, da, lane, th_t, th_d);
}

// ====================================================================== pass 2

// One row of a request, merged from its pass-1 partials.
struct RowStat {
  float m_t, mc_t, m_d, mc_d;
  double s_t, s_d;
  int am_t, am_d;  // greedy rows: exact argmaxes
};

struct RowEval {
  int verdict;
  float p_D, q_D, mu_D, u;
  float tau_eff;  // the row's gate threshold
};

// Merge the partials of the rows held by this wave and test each row's drafted token, all
// rows at once. Row jj of the set sits in the aligned group of nw lanes starting at jj*nw
// (nw, the waves per row, is a power of two), one partial per lane; `live` marks lanes
// whose row is to be tested. Each group reduces in a fixed order with fp64 sums, so every
// lane of a group ends with its row's result. j is the lane's row position in the request
// and D its drafted token.
//
// The gate threshold of row j is its step threshold ts, raised by the cumulative floor to
// floor / (q_0(D_0) ... q_{j-1}(D_{j-1})) when floor > 0 (regolith audit, section schedule
// behavior: the product of the drafted tokens' probabilities, this row's included, must
// reach the floor). `carry` is that product over the rows before this slot set, and
// `nlive` the number of live rows in the set; `carry` returns multiplied by the set's rows.
// Without SCHED the threshold is ts on every row (no floor), as in the plain call.
// With FILT, p(D) and q(D) are 0 when D's logit is below the row's keep-threshold.
template <bool SCHED, bool FILT = false>
__device__ __forceinline__ RowEval eval_rows(const Inputs& in, const P1Part& e, bool live, int nw, int b, int j,
                                             int D, float T, float ts, float floor, double& carry, int nlive,
                                             float c, RowStat& rs, float th_t = -INFINITY, float th_d = -INFINITY) {
  const bool greedy = T == 0.0f;
  const float mt = seg_max(live ? e.m_t : -INFINITY, nw);
  const float md = seg_max(live ? e.m_d : -INFINITY, nw);
  const float mct = ref_of(mt, c), mcd = ref_of(md, c);
  double st = 0.0, sd = 0.0;
  int it = INT32_MAX, id = INT32_MAX;
  if (live) {
    if (e.s_t != 0.0f) st = (double)(e.s_t * fast_exp2(ref_of(e.m_t, c) - mct));
    if (e.s_d != 0.0f) sd = (double)(e.s_d * fast_exp2(ref_of(e.m_d, c) - mcd));
    if (e.m_t == mt && e.am_t >= 0) it = e.am_t;
    if (e.m_d == md && e.am_d >= 0) id = e.am_d;
  }
  st = seg_sum(st, nw);
  sd = seg_sum(sd, nw);
  it = seg_min(it, nw);
  id = seg_min(id, nw);
  // Exactly one partial of a row holds the drafted token's logits: the group sums pick
  // them up unchanged (x + 0 = x).
  const bool f = live && (e.flags & 2);
  const float ltD = seg_sum(f ? e.lt_D : 0.0f, nw);
  const float ldD = seg_sum(f ? e.ld_D : 0.0f, nw);
  const int nf = __float2int_rn(seg_sum(f ? 1.0f : 0.0f, nw));
  rs = RowStat{mt, mct, md, mcd, st, sd, it == INT32_MAX ? -1 : it, id == INT32_MAX ? -1 : id};

  const bool valid = __builtin_isfinite(mt) && __builtin_isfinite(md) && __builtin_isfinite(st) && st > 0.0 &&
                     __builtin_isfinite(sd) && sd > 0.0 && nf == 1 && !__builtin_isnan(ts);
  RowEval ev{};
  ev.u = NAN;
  double p, q;
  if (greedy) {  // one-hot p and q
    p = (D == rs.am_t) ? 1.0 : 0.0;
    q = (D == rs.am_d) ? 1.0 : 0.0;
  } else {
    p = exp2((double)ltD * (double)c - (double)mct) / st;
    q = exp2((double)ldD * (double)c - (double)mcd) / sd;
    if (FILT && ltD < th_t) p = 0.0;
    if (FILT && ldD < th_d) q = 0.0;
  }
  // Row group g of the set sits in lanes g*nw .. g*nw + nw - 1; every lane of a group holds
  // its row's q. The product runs over the live rows before this lane's row, in row order.
  double tau_eff = (double)ts;
  if (SCHED && floor > 0.0f) {
    double pre = carry;
    const int jj = (int)(threadIdx.x & (kWave - 1)) / nw;
    for (int g = 0; g < nlive; ++g) {
      const double qg = lane_of(q, g * nw);
      if (g < jj) pre *= qg;
      carry *= qg;
    }
    tau_eff = fmax(tau_eff, (double)floor / pre);
  }
  ev.tau_eff = (float)tau_eff;
  if (greedy) {
    ev.p_D = (float)p;
    ev.q_D = (float)q;
    const bool offered = q >= tau_eff;
    ev.mu_D = offered ? ev.q_D : 0.0f;
    // p(D) is 0 or 1 and mu(D) <= 1: u*mu(D) < p(D) holds for every u iff p(D) = 1.
    ev.verdict = !valid ? kRowInvalid : !offered ? SV_ROW_NULL : (ev.p_D == 1.0f ? SV_ROW_ACCEPT : SV_ROW_REJECT);
    return ev;
  }
  const bool offered = q >= tau_eff;
  const double mu = offered ? q : 0.0;
  ev.p_D = (float)p;
  ev.q_D = (float)q;
  ev.mu_D = (float)mu;
  if (!valid) {
    ev.verdict = kRowInvalid;
  } else if (!offered) {
    ev.verdict = SV_ROW_NULL;
  } else {
    const Philox4 ph = philox4x32_10(0u, kTagAccept, (uint32_t)j, (uint32_t)b, seed_lo(in.seed), seed_hi(in.seed));
    ev.u = uniform_accept(ph.w0);
    ev.verdict = ((double)ev.u * mu < p) ? SV_ROW_ACCEPT : SV_ROW_REJECT;
  }
  return ev;
}

// Field-by-field choice between two register-held partials (a reference to either of two
// locals would move both to memory).
__device__ __forceinline__ P1Part pick_part(bool second, const P1Part& a, const P1Part& b) {
  P1Part r;
  r.m_t = second ? b.m_t : a.m_t;
  r.s_t = second ? b.s_t : a.s_t;
  r.m_d = second ? b.m_d : a.m_d;
  r.s_d = second ? b.s_d : a.s_d;
  r.am_t = second ? b.am_t : a.am_t;
  r.am_d = second ? b.am_d : a.am_d;
  r.flags = second ? b.flags : a.flags;
  r.lt_D = second ? b.lt_D : a.lt_D;
  r.ld_D = second ? b.ld_D : a.ld_D;
  r.pad[0] = r.pad[1] = r.pad[2] = 0;
  return r;
}

// A request's range, temperature and tau: one round trip.
struct ReqHead {
  int lo, n;
  float T, tau;
  float floor;   // cumulative floor (0: no cumulative gate)
  bool filt_ok;  // both sides' filter values are valid (or unused: greedy)
};

template <bool FILT = false>
__device__ __forceinline__ ReqHead request_head(const Inputs& in, int b) {
  ReqHead h;
  h.lo = in.ro[b];
  h.n = in.ro[b + 1] - h.lo;
  h.T = in.temp[b];
  h.tau = in.tau[b];
  h.floor = in.min_cum != nullptr ? in.min_cum[b] : 0.0f;
  h.filt_ok = true;
  if (FILT) {
    const FilterParams ft = filter_params(in.filt[0], b), fd = filter_params(in.filt[1], b);
    h.filt_ok = h.T == 0.0f || (filter_valid(ft) && filter_valid(fd));
  }
  return h;
}

// A request as pass 2 rebuilds it. Every field is wave-uniform.
struct ReqState {
  int lo, n, n_prop;
  int k;              // accepted drafts
  int f;              // the row that yields the last token (lo + k)
  int kind;           // kKind*
  int final_verdict;  // verdict of row f (SV_ROW_BONUS when every proposal row was accepted)
  float T, tau, c;    // after the walk, tau is row f's gate threshold
  float floor;        // cumulative floor
  float th_t, th_d;   // row f's keep-thresholds (-inf without filters)
  RowStat stop;       // row f's statistics when f is a proposal row
  int stop_half;      // row f's partials are in e1 (1) or e0 (0) ...
  int stop_lane0;     // ... in lanes stop_lane0 .. stop_lane0 + w1 - 1
};

// The drafted tokens of rows lo .. lo+63 (lane j: row lo + j) and the pass-1 partials of
// rows lo .. lo + 128/w1 - 1 in two slots per lane: e0 holds rows lo .. lo + 64/w1 - 1,
// e1 the next 64/w1 rows, one partial per lane. Indices are clamped into the arrays, so
// this may run before lo is known to be right.
template <bool SCHED>
__device__ __forceinline__ void prefetch_rows(const Inputs& in, const Work& w, int lo, int lane, int& dt0,
                                              float& ts0, P1Part& e0, P1Part& e1) {
  dt0 = in.dt[min(lo + lane, in.R - 1)];
  ts0 = SCHED && in.tau_step != nullptr ? in.tau_step[min(lo + lane, in.R - 1)] : 0.0f;
  const int64_t base = (int64_t)lo * in.w1;
  const int64_t last = (int64_t)in.R * in.w1 - 1;
  e0 = w.part1[min(base + lane, last)];
  e1 = w.part1[min(base + lane + kWave, last)];
}

// Keep-thresholds of rows lo .. lo+63 (lane j: row lo + j), clamped into the array.
__device__ __forceinline__ void prefetch_theta(const Inputs& in, int lo, int lane, float& tht0, float& thd0) {
  const int64_t r = min(lo + lane, in.R - 1);
  tht0 = in.theta[2 * r];
  thd0 = in.theta[2 * r + 1];
}

// Rebuild request b (head h, row_offsets checked) from the inputs and pass 1's partials:
// test its proposal rows in order up to the first one that is not accepted. Every wave of
// the request does this on its own, so no wave waits for another. dt0/e0/e1 arrive
// prefetched for first row lo_pre (fetched again when that guess was wrong). The rows of
// one slot are tested together. On return e0/e1 hold the slot set with row f. With
// `diag`, each row's record is written once: tested rows by their group's first lane (the
// stop row with `stop_resid`), untested and bonus rows after the walk.
template <bool SCHED, bool FILT = false>
__device__ __forceinline__ ReqState walk_request(const Inputs& in, const Work& w, int b, const ReqHead& h,
                                                 int lo_pre, int lane, int dt0, float ts0, P1Part& e0, P1Part& e1,
                                                 sv_row_diag* diag, float stop_resid, float tht0 = -INFINITY,
                                                 float thd0 = -INFINITY) {
  ReqState q{};
  q.lo = h.lo;
  q.n = h.n;
  q.T = h.T;
  q.tau = h.tau;
  q.floor = SCHED ? h.floor : 0.0f;
  q.stop_half = 0;
  q.stop_lane0 = 0;
  q.th_t = q.th_d = -INFINITY;
  const bool req_ok = temperature_ok(q.T) && !__builtin_isnan(q.tau) && __builtin_isfinite(q.floor) &&
                      q.floor >= 0.0f && h.filt_ok;
  q.c = req_ok ? fold_scale(q.T) : 0.0f;
  const int nw = in.w1;
  const int rows_half = kWave / nw;
  const int per_group = 2 * rows_half;
  const int nd = q.n - 1;  // rows that carry a drafted token: all but the last
  if (q.lo != lo_pre) {  // requests of different lengths
    prefetch_rows<SCHED>(in, w, q.lo, lane, dt0, ts0, e0, e1);
    if (FILT) prefetch_theta(in, q.lo, lane, tht0, thd0);
  }
  // Proposal rows: the rows before the first drafted token outside [0, V).
  q.n_prop = nd;
  for (int base = 0; base < nd; base += kWave) {
    const int i = base + lane;
    const int D = base == 0 ? dt0 : in.dt[q.lo + min(i, nd - 1)];
    const uint64_t m = __ballot(i < nd && (D < 0 || D >= in.V));
    if (m != 0) {
      q.n_prop = base + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  if (!req_ok) {
    q.kind = kKindInvalid;
    q.f = q.lo;
    return q;
  }
  int k = q.n_prop;
  bool stopped = false;
  float stop_tau = q.tau;
  double carry = 1.0;  // product of q(D) over the rows before the current slot set
  const int jj = lane / nw;  // the lane's row within a slot set
  for (int j0 = 0; j0 < q.n_prop && !stopped; j0 += per_group) {
    if (j0 > 0) {  // windows longer than one group
      int unused;
      float unused_ts;
      prefetch_rows<SCHED>(in, w, q.lo + j0, lane, unused, unused_ts, e0, e1);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // unrolled: e0 and e1 stay in registers
      const int jh = j0 + half * rows_half;
      if (jh >= q.n_prop) break;
      const int j = jh + jj;
      const bool live = j < q.n_prop;
      const int jc = min(j, nd - 1);
      const int D = jc < kWave ? __shfl(dt0, jc) : in.dt[q.lo + jc];
      const float ts = !SCHED || in.tau_step == nullptr ? q.tau
                                                        : jc < kWave ? __shfl(ts0, jc) : in.tau_step[q.lo + jc];
      const int nlive = min(rows_half, q.n_prop - jh);
      float th_t = -INFINITY, th_d = -INFINITY;
      if (FILT) {
        th_t = jc < kWave ? __shfl(tht0, jc) : in.theta[2 * (int64_t)(q.lo + jc)];
        th_d = jc < kWave ? __shfl(thd0, jc) : in.theta[2 * (int64_t)(q.lo + jc) + 1];
      }
      RowStat rs;
      const RowEval ev = eval_rows<SCHED, FILT>(in, pick_part(half != 0, e0, e1), live, nw, b, j, D, q.T, ts,
                                                q.floor, carry, nlive, q.c, rs, th_t, th_d);
      const uint64_t m = __ballot(live && ev.verdict != SV_ROW_ACCEPT);
      int stop_j = INT32_MAX;
      if (m != 0) {
        const int src = __ffsll((unsigned long long)m) - 1;
        stop_j = jh + src / nw;
        k = stop_j;
        q.final_verdict = lane_of(ev.verdict, src);
        stop_tau = lane_of(ev.tau_eff, src);
        q.stop = RowStat{lane_of(rs.m_t, src), lane_of(rs.mc_t, src), lane_of(rs.m_d, src), lane_of(rs.mc_d, src),
                         lane_of(rs.s_t, src), lane_of(rs.s_d, src), lane_of(rs.am_t, src), lane_of(rs.am_d, src)};
        q.stop_half = half;
        q.stop_lane0 = (src / nw) * nw;
        stopped = true;
      }
      if (diag != nullptr && live && (lane & (nw - 1)) == 0 && j <= stop_j) {
        sv_row_diag dg;
        dg.p_D = ev.p_D;
        dg.q_D = ev.q_D;
        dg.mu_D = ev.mu_D;
        dg.u = ev.u;
        dg.resid_mass = j == stop_j ? stop_resid : NAN;
        dg.verdict = ev.verdict;
        dg.pad0 = dg.pad1 = 0;
        diag[q.lo + j] = dg;
      }
      if (stopped) break;
    }
  }
  q.k = k;
  q.f = q.lo + k;
  q.tau = stop_tau;
  if (FILT) {
    q.th_t = k < kWave ? __shfl(tht0, k) : in.theta[2 * (int64_t)q.f];
    q.th_d = k < kWave ? __shfl(thd0, k) : in.theta[2 * (int64_t)q.f + 1];
  }
  const bool greedy = q.T == 0.0f;
  if (k < q.n_prop) {
    q.kind = q.final_verdict == kRowInvalid ? kKindInvalid : greedy ? kKindGreedyDone : kKindResidual;
  } else {
    q.kind = greedy ? kKindGreedyBonus : kKindBonus;
    q.final_verdict = SV_ROW_BONUS;
  }
  if (diag != nullptr) {
    for (int j = lane; j < q.n; j += kWave) {
      if (j > k) {
        diag[q.lo + j] = untested_diag();
      } else if (j == k && q.final_verdict == SV_ROW_BONUS) {
        sv_row_diag dg = untested_diag();
        dg.verdict = SV_ROW_BONUS;
        diag[q.lo + j] = dg;
      }
    }
  }
  // Keep the request in scalar registers.
  q.n_prop = uni(q.n_prop);
  q.k = uni(q.k);
  q.f = uni(q.f);
  q.kind = uni(q.kind);
  q.final_verdict = uni(q.final_verdict);
  q.tau = uni(q.tau);
  q.th_t = uni(q.th_t);
  q.th_d = uni(q.th_d);
  q.stop.m_t = uni(q.stop.m_t);
  q.stop.mc_t = uni(q.stop.mc_t);
  q.stop.m_d = uni(q.stop.m_d);
  q.stop.mc_d = uni(q.stop.mc_d);
  q.stop.s_t = uni(q.stop.s_t);
  q.stop.s_d = uni(q.stop.s_d);
  q.stop.am_t = uni(q.stop.am_t);
  q.stop.am_d = uni(q.stop.am_d);
  q.stop_half = uni(q.stop_half);
  q.stop_lane0 = uni(q.stop_lane0);
  return q;
}

// One lane per request adds its counts (sv_batch_stats field order). D is the drafted id on
// the request's last evaluated row.
__device__ __forceinline__ void add_stats(const Outputs& out, const ReqState& q, bool invalid, int D, int V) {
  if (out.stats == nullptr) return;
  unsigned long long* s = reinterpret_cast<unsigned long long*>(out.stats);
  if (invalid) {
    atomicAdd(s + 7, 1ull);
    return;
  }
  const bool tested_final = q.final_verdict == SV_ROW_REJECT || q.final_verdict == SV_ROW_NULL;
  atomicAdd(s + 0, 1ull);
  atomicAdd(s + 1, (unsigned long long)(q.k + (tested_final ? 1 : 0)));
  if (q.k) atomicAdd(s + 2, (unsigned long long)q.k);
  if (q.final_verdict == SV_ROW_REJECT) atomicAdd(s + 3, 1ull);
  if (q.final_verdict == SV_ROW_NULL) atomicAdd(s + 4, 1ull);
  if (q.final_verdict == SV_ROW_BONUS) atomicAdd(s + 5, 1ull);
  if (q.T == 0.0f) atomicAdd(s + 6, 1ull);
  const int offered = q.k + (q.final_verdict == SV_ROW_REJECT ? 1 : 0);
  if (offered) atomicAdd(s + 8, (unsigned long long)offered);
  if (q.final_verdict == SV_ROW_BONUS && q.k < q.n - 1) {
    atomicAdd(s + 9, 1ull);
    if (D != SV_NO_PROPOSAL && (D < 0 || D >= V)) atomicAdd(s + 10, 1ull);
  }
}

// Write request b's outputs (one wave): the accepted drafts, the last token, -1 after it.
// A request that fails closed gets -1 everywhere and untested diagnostics.
// With dt_held, lane j already holds the drafted token of row lo + j (j < 64) in dt_reg, which
// saves the emitting wave a round trip.
template <bool FILT = false>
__device__ __forceinline__ void emit_request(const Inputs& in, const Work& w, const Outputs& out, int b,
                                             const ReqState& q, bool invalid, int token, float resid, int lane,
                                             bool dt_held = false, int dt_reg = 0) {
  for (int j = lane; j < q.n; j += kWave) {
    const int r = q.lo + j;
    int t = -1;
    if (!invalid) {
      if (j < q.k) t = (dt_held && j < kWave) ? dt_reg : in.dt[r];
      else if (j == q.k) t = token;
    }
    out.tokens[r] = t;
  }
  if (lane == 0) {
    out.accept_len[b] = invalid ? -1 : q.k;
    add_stats(out, q, invalid, (!invalid && q.k < q.n) ? in.dt[q.lo + q.k] : SV_NO_PROPOSAL, in.V);
  }
  if (out.diag != nullptr) {
    if (invalid) {
      for (int j = lane; j < q.n; j += kWave) out.diag[q.lo + j] = untested_diag();
    } else {
      int dt0;
      float ts0;
      P1Part e0, e1;
      float tht0 = -INFINITY, thd0 = -INFINITY;
      prefetch_rows<true>(in, w, q.lo, lane, dt0, ts0, e0, e1);
      if (FILT) prefetch_theta(in, q.lo, lane, tht0, thd0);
      walk_request<true, FILT>(in, w, b, request_head<FILT>(in, b), q.lo, lane, dt0, ts0, e0, e1, out.diag, resid,
                               tht0, thd0);
    }
  }
}

// How far below the wave's best fp32 race key a candidate is still re-evaluated exactly:
// a relative 1e-3 for ratio keys r/E, 0.01 in log2 units for log keys. Both are far above
// the keys' fp32 error outside decision-boundary requests.
constexpr float kRatioKeySlack = 1e-3f;
constexpr float kKeyErr = 1e-5f;
constexpr float kLogKeySlack = 0.01f;

// fp64 race key of token x on a residual row, from its two logits.
// Logits below a keep-threshold (th_t, th_d) give p = 0 or q = 0.
__device__ __forceinline__ double residual_key64(double lt, double ld, double c, double mct, double mcd,
                                                 double st, double sd, double tau, uint32_t word,
                                                 float th_t, float th_d) {
  const double p = (float)lt < th_t ? 0.0 : exp2(lt * c - mct) / st;
  const double q = (float)ld < th_d ? 0.0 : exp2(ld * c - mcd) / sd;
  const double mu = q >= tau ? q : 0.0;
  const double r = p - mu;
  if (!(r > 0.0)) return 0.0;
  return r / expo64(word);
}

// fp64 race key of token x in a race over p, in the log domain: ln p(x) - ln E(x) up to a
// constant shared by every token of the row.
__device__ __forceinline__ double p_logkey64(double l, double T, uint32_t word) {
  return l / T - log(expo64(word));
}

// Race candidate queue of a pass-2 instance: a fold pushes at most U * VEC / G groups per
// lane (G tokens share a Philox block), on top of the fewer than 64 that a drain leaves.
template <int VEC, int U>
constexpr int queue_cap() {
  return (U * VEC / (VEC >= 4 ? 4 : 1) + 1) * kWave;
}

// A (logit, token) pair as one 64-bit word whose unsigned order is the logit's order: the
// float's bits mapped to a monotone unsigned key in the high half, the token in the low half.
// Zero is below every pair.
__device__ __forceinline__ uint64_t pack_best(float l, int x) {
  const uint32_t u = __float_as_uint(l);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)k << 32) | (uint32_t)x;
}

__device__ __forceinline__ float best_logit(uint64_t v) {
  const uint32_t k = (uint32_t)(v >> 32);
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// A queued logit: its bf16 bits for bf16 inputs (every logit read from them is a bf16 value,
// so this is exact), the float itself for fp32 inputs.
template <typename E>
struct QLogit;
template <>
struct QLogit<uint16_t> {
  using T = uint16_t;
  static __device__ __forceinline__ T enc(float f) { return (uint16_t)(__float_as_uint(f) >> 16); }
  static __device__ __forceinline__ float dec(T h) { return __uint_as_float((uint32_t)h << 16); }
};
template <>
struct QLogit<float> {
  using T = float;
  static __device__ __forceinline__ T enc(float f) { return f; }
  static __device__ __forceinline__ float dec(T f) { return f; }
};

// The number of lanes below this one whose bit is set in m.
__device__ __forceinline__ int lane_rank(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The race winner among the lanes' fp32 top-2 candidates. Every candidate whose fp32 key
// reaches `cut` is re-evaluated exactly by `eval(index, a, b)`; the best exact key wins,
// ties to the lower index. With `cut` a safe margin below the wave's best fp32 key, no
// candidate that could win exactly is left out.
template <class F>
__device__ __forceinline__ void resolve_race(const Top2& t, float cut, F eval, double& bk, int& bi) {
  bk = -INFINITY;
  bi = INT32_MAX;
  if (t.i1 != INT32_MAX && t.k1 >= cut) {
    bk = eval(t.i1, t.a1, t.b1);
    bi = t.i1;
  }
  if (t.i2 != INT32_MAX && t.k2 >= cut) {
    const double k2 = eval(t.i2, t.a2, t.b2);
    if (beats(k2, t.i2, bk, bi)) {
      bk = k2;
      bi = t.i2;
    }
  }
  wave_best(bk, bi);
}

// A race over p read by one wave: the rare fallback for a residual with no mass.
__device__ __forceinline__ int p_race_one_wave(const Inputs& in, const ReqState& q, int b, int lane) {
  Top2 t = top2_empty();
  for (int64_t x = lane; x < in.V; x += kWave) {
    const float l = logit_at(in.target, in.dtype, (int64_t)q.f * in.V + x);
    const float a = l * q.c;
    if (a > -INFINITY && !(l < q.th_t)) {
      const uint32_t wd = race_word(in.seed, x, q.k, b);
      top2_push(t, a - log2_expo32(wd), (int)x, l, 0.0f);
    }
  }
  double bk;
  int bi;
  resolve_race(t, wave_max(t.k1) - kLogKeySlack,
               [&](int x, float l, float) { return p_logkey64((double)l, (double)q.T, race_word(in.seed, x, q.k, b)); },
               bk, bi);
  return bi;
}

// Wave gw of the grid serves span gw % w2 of request gw / w2. DIAG is the kernel of the
// diagnostic and scheduled calls: its residual waves also sum the residual mass, which needs
// every token's p and mu, and its walk applies per-row step thresholds and the cumulative
// floor.
// The plain call's waves skip, by one test in the logit domain, every 16-byte vector that
// cannot hold a race candidate: r = (p - mu)+ <= p, so a vector whose largest p is below the
// pruning threshold holds none, whatever mu is.
// With FILT (the filtered verify) every p and q is masked by its row's keep-threshold.
template <typename E, int VEC, int U, bool DIAG, bool FILT = false>
__global__ __launch_bounds__(kBlock) void pass2_kernel(Inputs in, Work w, Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  // Each wave's queue of race candidate groups (see the draw loops).
  constexpr int kQueueCap = queue_cap<VEC, U>();
  __shared__ int q_x[kWavesPerBlock][kQueueCap];
  constexpr int kQG = VEC >= 4 ? 4 : 1;  // tokens per queued group
  using QL = QLogit<E>;
  __shared__ typename QL::T q_t[kWavesPerBlock][kQueueCap * kQG];
  __shared__ typename QL::T q_d[kWavesPerBlock][kQueueCap * kQG];
  if (gw >= (int64_t)in.B * in.w2) return;
  const int b = (int)(gw / in.w2);
  const int g = (int)(gw % in.w2);
  const bool head = g == 0;

  // One round trip brings the batch check, the request's head, and its rows' drafted
  // tokens and partials at the first row the head would give if every request had the
  // same length.
  const int ro_valid = w.hdr->ro_valid;
  const ReqHead rh = request_head<FILT>(in, b);
  const int lo_pre = (int)((int64_t)b * in.R / in.B);
  int dt0;
  float ts0;
  P1Part e0, e1;
  prefetch_rows<DIAG>(in, w, lo_pre, lane, dt0, ts0, e0, e1);
  float tht0 = -INFINITY, thd0 = -INFINITY;
  if (FILT) prefetch_theta(in, lo_pre, lane, tht0, thd0);
  if (!ro_valid) {
    // Broken row_offsets: the whole batch fails closed. The head wave of request b
    // clears an even share of the rows.
    if (head) {
      const int64_t r0 = (int64_t)b * in.R / in.B, r1 = (int64_t)(b + 1) * in.R / in.B;
      for (int64_t r = r0 + lane; r < r1; r += kWave) {
        out.tokens[r] = -1;
        if (out.diag != nullptr) out.diag[r] = untested_diag();
      }
      if (lane == 0) {
        out.accept_len[b] = -1;
        if (out.stats != nullptr) atomicAdd(reinterpret_cast<unsigned long long*>(out.stats) + 7, 1ull);
      }
    }
    return;
  }

  const ReqState q = walk_request<DIAG, FILT>(in, w, b, rh, lo_pre, lane, dt0, ts0, e0, e1, nullptr, NAN, tht0, thd0);
  if (q.kind == kKindInvalid) {
    if (head) emit_request<FILT>(in, w, out, b, q, true, -1, NAN, lane);
    return;
  }
  if (q.kind == kKindGreedyDone) {
    // One-hot p and mu: the residual is empty iff the offered draft argmax is the target argmax.
    const float resid = (q.stop.am_t == q.stop.am_d && 1.0f >= q.tau) ? 0.0f : 1.0f;
    if (head) emit_request<FILT>(in, w, out, b, q, false, q.stop.am_t, resid, lane, q.lo == lo_pre, dt0);
    return;
  }

  using CH = Chunk<E, VEC>;
  const int nvec = in.V / VEC;
  const int nw = in.w2;
  const Span sp = wave_span(nvec, nw, g);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)q.f * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)q.f * in.V;
  const uint32_t k0 = seed_lo(in.seed), k1 = seed_hi(in.seed);
  constexpr int step = U * kWave;
  constexpr int G = VEC >= 4 ? 4 : 1;  // logits sharing one Philox block
  const int nsteps = (sp.end - sp.begin + step - 1) / step;

  P2Part part{};
  part.key = -INFINITY;
  part.idx = -1;
  part.rsum = 0.0f;
  part.mref = -INFINITY;
  part.bad = 0;
  part.gidx = -1;
  part.pidx = -1;
  part.pkey = -INFINITY;

  if (q.kind == kKindResidual) {
    const float c = q.c, mct = q.stop.mc_t, mcd = q.stop.mc_d, tau = q.tau;
    const float tht = q.th_t, thd = q.th_d;
    const float ist = (float)(1.0 / q.stop.s_t), isd = (float)(1.0 / q.stop.s_d);
    // Gate in the logit domain: q_x >= tau needs l_d*c - mcd >= log2(tau * s_d). The margin
    // keeps every token whose fp32 q could reach tau; for the others mu = 0 and r = p, so q
    // is computed only where the gate can pass.
    const float gate_l = tau > 0.0f ? (float)(((double)mcd + log2((double)tau * q.stop.s_d) - 1e-3) / (double)c)
                                    : -INFINITY;
    // Pruning bound. Pass 1 left, per wave of row f, the vector that held that wave's
    // target maximum; row f's partials are in this wave's registers. A lower bound on the
    // race key of (up to 128 of) those tokens bounds the winner's key from below. A token
    // whose residual r has r / E_min below half of it cannot win and draws no random number.
    // As the wave draws, the same lower bound on its own candidates' keys raises the bar.
    // The bounds shave kKeyErr off every fp32 factor, more than its rounding error.
    const int nh = in.w1 * VEC;
    const int hsrc = q.stop_half ? e1.am_t : e0.am_t;
    int hx[2];
    float hlt[2], hld[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ti = lane + s * kWave;
      const int hv = __shfl(hsrc, q.stop_lane0 + min(ti / VEC, in.w1 - 1));
      int x = (ti < nh && hv >= 0) ? hv * VEC + ti % VEC : -1;
      x = x < in.V ? x : -1;
      hx[s] = x;
      const int xc = x >= 0 ? x : 0;
      hlt[s] = to_float(trow[xc]);
      hld[s] = to_float(drow[xc]);
    }
    // The span's first batch is requested before the hint logits are used.
    CH ta[U], da[U], tb[U], db[U];
    if (nsteps > 0) {
      load_chunks<false>(ta, trow, sp.begin, lane, sp.end);
      load_chunks<false>(da, drow, sp.begin, lane, sp.end);
    }
    float kh = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float p = (FILT && hlt[s] < tht) ? 0.0f : fast_exp2(fmaf(hlt[s], c, -mct)) * ist;
      const float qq = (FILT && hld[s] < thd) ? 0.0f : fast_exp2(fmaf(hld[s], c, -mcd)) * isd;
      const float mu = qq >= tau ? qq : 0.0f;
      const float rl = fmaf(p, 1.0f - kKeyErr, -mu * (1.0f + kKeyErr));  // at most the exact residual
      if (hx[s] >= 0 && rl > 0.0f)
        kh = fmaxf(kh, div_fast(rl, expo32_upper(race_word(in.seed, hx[s], q.k, b))) * (1.0f - kKeyErr));
    }
    kh = wave_max(kh);
    float pthr = kh * (float)(kEminLow * 0.5);
    float safe = 0.0f;  // lane's best lower bound on a drawn key
    // Where the gate fails, r = p = 2^(l*c - mct) / s_t, so r >= pthr needs l*c - mct >= sthr.
    // The margin covers the fp32 error of p.
    auto sthr_of = [&](float th) __attribute__((always_inline)) {
      return th > 0.0f ? __log2f((float)((double)th * q.stop.s_t)) - 1e-3f : -INFINITY;
    };
    float sthr = sthr_of(pthr);

    float rsum = 0.0f;
    Top2 t = top2_empty();
    // With a target filter, p often has few tokens and p <= mu on all of them, which leaves
    // the residual empty: the draw then races over p. The waves track that race too, over
    // the kept tokens whose l*c is within 29 of the row maximum's (a token further below
    // cannot win a log2-key race; see the bonus race). No vector is skipped while the
    // residual may be empty: skipping needs a drawn candidate with r > 0.
    const bool prace = FILT && tht > -INFINITY;
    const float plb = q.stop.m_t * c - 29.0f;
    Top2 tq = top2_empty();
    // Candidate groups (G tokens that share a Philox block) wait in the wave's queue and are
    // drawn 64 at a time, one group per lane: a Philox block costs a wave the same whether
    // one lane needs it or all 64. A drain re-tests every token against the bound as it then
    // stands, which only drops tokens that cannot win.
    // Draw the group of G tokens starting at xg, with their target and draft logits. With
    // raise, the drawn keys also raise the pruning bound (a dense draw skips that: on a flat
    // residual the bound prunes next to nothing).
    auto draw_res = [&](int xg, const float (&lts)[G], const float (&lds)[G], auto raise) __attribute__((always_inline)) {
      const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)q.k, (uint32_t)b, k0, k1);
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const float lt = lts[e], ld = lds[e];
        const int x = xg + e;
        const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, x & 3);
        float p = fast_exp2(fmaf(lt, c, -mct)) * ist;
        if (FILT && lt < tht) p = 0.0f;
        const float qq = fast_exp2(fmaf(ld, c, -mcd)) * isd;
        const float mu = (qq >= tau && !(FILT && ld < thd)) ? qq : 0.0f;
        const float r = fmaxf(p - mu, 0.0f);
        if (r > 0.0f && r >= pthr) {
          top2_push(t, div_fast(r, expo32(wd)), x, lt, ld);
          if (decltype(raise)::value) {
            const float rl = fmaf(p, 1.0f - kKeyErr, -mu * (1.0f + kKeyErr));  // at most the exact residual
            safe = fmaxf(safe, div_fast(rl, expo32_upper(wd)) * (1.0f - kKeyErr));
          }
        }
        if (prace && !(lt < tht) && lt * c >= plb) top2_push(tq, lt * c - log2_expo32(wd), x, lt, 0.0f);
      }
    };
    auto drain = [&](int base, int cnt) __attribute__((always_inline)) {
      if (lane < cnt) {
        const int ei = base + lane;
        float lts[G], lds[G];
#pragma unroll
        for (int e = 0; e < G; ++e) {
          lts[e] = QL::dec(q_t[wave][ei * kQG + e]);
          lds[e] = QL::dec(q_d[wave][ei * kQG + e]);
        }
        draw_res(q_x[wave][ei], lts, lds, std::true_type{});
      }
    };
    int qn = 0;  // queued groups, wave-uniform
    auto fold_res = [&](const CH (&xt)[U], const CH (&xd)[U], int v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bool live = true;
        if (!DIAG || FILT) {
          float mt = xt[u].get(0);
#pragma unroll
          for (int e = 1; e < VEC; ++e) mt = fmaxf(mt, xt[u].get(e));
          // r <= p: no token of a vector whose largest p misses pthr is a candidate
          if (!DIAG) live = fmaf(mt, c, -mct) >= sthr;
          // every target logit of the vector below the keep-threshold: p = 0, r = 0, and no
          // token takes part in the race over p either
          if (FILT) live = live && !(mt < tht);
          if (!DIAG && !__any(live)) continue;  // the whole wave skips the vector
        }
        const int x0 = (v0 + u * kWave) * VEC;
        if (!DIAG) {
          // A candidate needs p >= pthr (r <= p): one test per token in the logit domain, with
          // no exponential. On a flat residual nearly every group is a candidate: the wave then
          // draws the vector's groups in place; otherwise it queues them for the drain, which
          // computes p, mu and r for the queued tokens.
          constexpr int NG = VEC / G;
          bool cg[NG];
          int ncand = 0;
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            bool any = false;
#pragma unroll
            for (int e = 0; e < G; ++e) {
              const float l = xt[u].get(gi * G + e);
              any |= fmaf(l, c, -mct) >= sthr && !(FILT && l < tht);
              if (prace) any |= !(l < tht) && l * c >= plb;
            }
            cg[gi] = live && any;
            ncand += (int)__popcll(__ballot(cg[gi]));
          }
          if (4 * ncand >= 3 * NG * kWave) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
              if (cg[gi]) {
                float lts[G], lds[G];
#pragma unroll
                for (int e = 0; e < G; ++e) {
                  lts[e] = xt[u].get(gi * G + e);
                  lds[e] = xd[u].get(gi * G + e);
                }
                draw_res(x0 + gi * G, lts, lds, std::false_type{});
              }
            }
            continue;
          }
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            const uint64_t m = __ballot(cg[gi]);
            if (cg[gi]) {
              const int pos = qn + lane_rank(m);
              q_x[wave][pos] = x0 + gi * G;
#pragma unroll
              for (int e = 0; e < G; ++e) {
                q_t[wave][pos * kQG + e] = QL::enc(xt[u].get(gi * G + e));
                q_d[wave][pos * kQG + e] = QL::enc(xd[u].get(gi * G + e));
              }
            }
            qn = uni(qn + (int)__popcll(m));
          }
          continue;
        }
        float rv[VEC], mv[VEC];
        bool gated = false;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          rv[e] = fast_exp2(fmaf(xt[u].get(e), c, -mct)) * ist;  // p; r = p where mu = 0
          if (FILT && xt[u].get(e) < tht) rv[e] = 0.0f;
          mv[e] = 0.0f;
          gated |= xd[u].get(e) >= gate_l;
        }
        if (gated) {  // rare: a token of this vector may pass the gate
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float qq = fast_exp2(fmaf(xd[u].get(e), c, -mcd)) * isd;
            mv[e] = (qq >= tau && !(FILT && xd[u].get(e) < thd)) ? qq : 0.0f;
          }
        }
#pragma unroll
        for (int gg = 0; gg < VEC; gg += G) {
          bool any = false, anyp = false;
#pragma unroll
          for (int e = 0; e < G; ++e) {
            const float r = fmaxf(rv[gg + e] - mv[gg + e], 0.0f);
            if (DIAG) rsum += r;
            any |= (r > 0.0f && r >= pthr);
            if (prace) anyp |= !(xt[u].get(gg + e) < tht) && xt[u].get(gg + e) * c >= plb;
          }
          const bool cand = live && (any || anyp);
          const uint64_t m = __ballot(cand);
          if (cand) {
            const int pos = qn + lane_rank(m);
            q_x[wave][pos] = x0 + gg;
#pragma unroll
            for (int e = 0; e < G; ++e) {
              q_t[wave][pos * kQG + e] = QL::enc(xt[u].get(gg + e));
              q_d[wave][pos * kQG + e] = QL::enc(xd[u].get(gg + e));
            }
          }
          qn = uni(qn + (int)__popcll(m));
        }
      }
      // One drain site per fold keeps the unrolled loop small in the instruction cache.
      while (qn >= kWave) {
        __builtin_amdgcn_wave_barrier();
        drain(qn - kWave, kWave);
        __builtin_amdgcn_wave_barrier();
        qn -= kWave;
      }
    };
    // Double buffering with an exit only at the bottom (see pass 1).
    for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
      load_chunks<false>(tb, trow, base + step, lane, sp.end);
      load_chunks<false>(db, drow, base + step, lane, sp.end);
      mask_chunks(ta, base, lane, sp.end);
      mask_chunks(da, base, lane, sp.end);
      fold_res(ta, da, base + lane);
      load_chunks<false>(ta, trow, base + 2 * step, lane, sp.end);
      load_chunks<false>(da, drow, base + 2 * step, lane, sp.end);
      mask_chunks(tb, base + step, lane, sp.end);
      mask_chunks(db, base + step, lane, sp.end);
      fold_res(tb, db, base + step + lane);
      pthr = fmaxf(pthr, wave_max(safe) * (float)(kEminLow * 0.5));
      if (!DIAG) sthr = sthr_of(pthr);
    }
    if (qn > 0) {
      __builtin_amdgcn_wave_barrier();
      drain(0, qn);
    }
    part.rsum = DIAG ? wave_sum(rsum) : 0.0f;
    double bk;
    int bi;
    resolve_race(t, wave_max(t.k1) * (1.0f - kRatioKeySlack),
                 [&](int x, float lt, float ld) {
                   return residual_key64((double)lt, (double)ld, (double)c, (double)mct, (double)mcd, q.stop.s_t,
                                         q.stop.s_d, (double)tau, race_word(in.seed, x, q.k, b), tht, thd);
                 },
                 bk, bi);
    part.key = bk;
    part.idx = bi == INT32_MAX ? -1 : bi;
    if (prace) {
      double pk;
      int pi;
      resolve_race(tq, wave_max(tq.k1) - kLogKeySlack,
                   [&](int x, float l, float) {
                     return p_logkey64((double)l, (double)q.T, race_word(in.seed, x, q.k, b));
                   },
                   pk, pi);
      part.pkey = pk;
      part.pidx = pi == INT32_MAX ? -1 : pi;
    }
  } else {
    // Bonus row (race over p) or greedy bonus row (argmax). Pass 1 never read it, so it is validated here.
    const bool race = q.kind == kKindBonus;
    const float c = q.c;
    Acc a = acc_empty();
    int bad = 0;
    Top2 t = top2_empty();
    float wbest = -INFINITY;  // best log2 key the wave has drawn so far
    // A span of at most KR vectors per lane is read once, all of it at once, and held in
    // registers for both steps below; a longer one is streamed twice (the second time from the
    // caches).
    constexpr int KR = VEC == 1 ? 16 : 8;
    const bool held = sp.end - sp.begin <= KR * kWave;
    CH hb[KR];
    CH ta[U], tb[U];
    // First the span's maximum (and NaN / +inf check, and for greedy rows the lowest index of
    // the maximum).
    if (held) {
      if (nsteps > 0) {
        load_chunks<false>(hb, trow, sp.begin, lane, sp.end);
        mask_chunks(hb, sp.begin, lane, sp.end);
        fold_max<true>(a, hb, sp.begin + lane, bad);
      }
    } else {
      load_chunks<false>(ta, trow, sp.begin, lane, sp.end);
      for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
        load_chunks<false>(tb, trow, base + step, lane, sp.end);
        mask_chunks(ta, base, lane, sp.end);
        fold_max<true>(a, ta, base + lane, bad);
        load_chunks<false>(ta, trow, base + 2 * step, lane, sp.end);
        mask_chunks(tb, base + step, lane, sp.end);
        fold_max<true>(a, tb, base + step + lane, bad);
      }
    }
    float m;
    float unused;
    int am;
    wave_stat(a, 0.0f, false, m, unused, am);
    const int am_w = exact_argmax<CH>(trow, a, m);
    part.mref = m;
    part.gidx = race ? -1 : am_w;
    part.bad = wave_or(bad);
    if (race && nsteps > 0) {
      // Pruning bound. A token's log2 key is l*c - log2(E) with 2^-24 < E < 16.7, so it lies
      // within (l*c - 4.06, l*c + 24): a token more than 25 below a drawn key cannot win (the
      // margin absorbs fp32 error). The waves of a request pool their best (logit, token) in
      // one word with an atomic max, and each takes the key of the best token pooled so far
      // as its starting bound: on rows with a few large logits, every wave then skips
      // nearly all of its span. The largest logit is in p's support under every filter.
      float lb = m * c - 4.1f;
      uint64_t best = 0;
      if (am_w >= 0) {
        const uint64_t mine = pack_best(m, am_w);
        uint64_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(w.bmax + b),
                                                    (unsigned long long)mine, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        old = uni64(old);
        best = old > mine ? old : mine;
      }
      if (best != 0) {
        const float mg = best_logit(best);
        const int ig = (int)(uint32_t)best;
        if (__builtin_isfinite(mg) && ig >= 0 && ig < in.V)
          lb = fmaxf(lb, mg * c - log2_expo32(race_word(in.seed, ig, q.k, b)));
      }
      // Candidate groups are queued and drawn 64 at a time, as in the residual race.
      int qn = 0;  // queued groups, wave-uniform
      auto drain = [&](int base, int cnt) __attribute__((always_inline)) {
        float lbest = -INFINITY;
        if (lane < cnt) {
          const int ei = base + lane;
          const int xg = q_x[wave][ei];
          const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)q.k, (uint32_t)b, k0, k1);
#pragma unroll
          for (int e = 0; e < G; ++e) {
            const float l = QL::dec(q_t[wave][ei * kQG + e]);
            float av = l * c;
            if (FILT && l < q.th_t) av = -INFINITY;  // outside p's support
            if (av + 25.0f >= lb) {
              const int x = xg + e;
              const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, x & 3);
              const float key = av - log2_expo32(wd);
              lbest = fmaxf(lbest, key);
              top2_push(t, key, x, l, 0.0f);
            }
          }
        }
        wbest = fmaxf(wbest, wave_max(lbest));
        lb = fmaxf(lb, wbest);
      };
      // Before its first drain, a wave that pooled early reads the pooled pair again (the
      // other waves have published by then) and drops the queued groups that the tighter
      // bound excludes.
      bool refreshed = false;
      auto refresh = [&]() __attribute__((always_inline)) {
        refreshed = true;
        const uint64_t now = uni64(__hip_atomic_load(reinterpret_cast<unsigned long long*>(w.bmax + b),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (now <= best) return;
        best = now;
        const float mg = best_logit(now);
        const int ig = (int)(uint32_t)now;
        if (!(__builtin_isfinite(mg) && ig >= 0 && ig < in.V)) return;
        const float nl = mg * c - log2_expo32(race_word(in.seed, ig, q.k, b));
        if (!(nl > lb)) return;
        lb = nl;
        __builtin_amdgcn_wave_barrier();
        int kept = 0;
        for (int base = 0; base < qn; base += kWave) {  // in order, so writes never pass reads
          const int ei = base + lane;
          bool keep = false;
          int xg = 0;
          float lt[kQG];
          if (ei < qn) {
            xg = q_x[wave][ei];
#pragma unroll
            for (int e = 0; e < kQG; ++e) {
              lt[e] = QL::dec(q_t[wave][ei * kQG + e]);
              keep |= lt[e] * c + 25.0f >= lb && !(FILT && lt[e] < q.th_t);
            }
          }
          const uint64_t mk = __ballot(keep);
          __builtin_amdgcn_wave_barrier();
          if (keep) {
            const int pos = kept + lane_rank(mk);
            q_x[wave][pos] = xg;
#pragma unroll
            for (int e = 0; e < kQG; ++e) q_t[wave][pos * kQG + e] = QL::enc(lt[e]);
          }
          __builtin_amdgcn_wave_barrier();
          kept = uni(kept + (int)__popcll(mk));
        }
        qn = kept;
      };
      auto fold_race = [&](const auto& xt, int v0) __attribute__((always_inline)) {
        constexpr int UU = sizeof(xt) / sizeof(xt[0]);
#pragma unroll
        for (int u = 0; u < UU; ++u) {
          const int x0 = (v0 + u * kWave) * VEC;
#pragma unroll
          for (int gg = 0; gg < VEC; gg += G) {
            bool any = false;
#pragma unroll
            for (int e = 0; e < G; ++e) {
              const float l = xt[u].get(gg + e);
              any |= l * c + 25.0f >= lb && !(FILT && l < q.th_t);
            }
            const uint64_t mk = __ballot(any);
            if (any) {
              const int pos = qn + lane_rank(mk);
              q_x[wave][pos] = x0 + gg;
#pragma unroll
              for (int e = 0; e < G; ++e) q_t[wave][pos * kQG + e] = QL::enc(xt[u].get(gg + e));
            }
            qn = uni(qn + (int)__popcll(mk));
          }
        }
        if (qn >= kWave && !refreshed) refresh();
        while (qn >= kWave) {  // one drain site per fold (see the residual race)
          __builtin_amdgcn_wave_barrier();
          drain(qn - kWave, kWave);
          __builtin_amdgcn_wave_barrier();
          qn -= kWave;
        }
      };
      // Then the race.
      if (held) {
#pragma unroll
        for (int k = 0; k < KR; k += U) {
          CH pair[U];
#pragma unroll
          for (int u = 0; u < U; ++u) pair[u] = hb[k + u];
          fold_race(pair, sp.begin + k * kWave + lane);
        }
      } else {
        load_chunks<false>(ta, trow, sp.begin, lane, sp.end);
        for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
          load_chunks<false>(tb, trow, base + step, lane, sp.end);
          mask_chunks(ta, base, lane, sp.end);
          fold_race(ta, base + lane);
          load_chunks<false>(ta, trow, base + 2 * step, lane, sp.end);
          mask_chunks(tb, base + step, lane, sp.end);
          fold_race(tb, base + step + lane);
        }
      }
      if (qn > 0) {
        __builtin_amdgcn_wave_barrier();
        drain(0, qn);
      }
    }
    if (race) {
      double bk;
      int bi;
      resolve_race(t, wave_max(t.k1) - kLogKeySlack,
                   [&](int x, float l, float) {
                     return p_logkey64((double)l, (double)q.T, race_word(in.seed, x, q.k, b));
                   },
                   bk, bi);
      part.key = bk;
      part.idx = bi == INT32_MAX ? -1 : bi;
    }
  }

  if (lane == 0) publish64(&w.part2[(int64_t)b * nw + g], part);
  if (!arrive_last(&w.t2[b], (uint32_t)nw, lane)) return;

  // ---- the request's last wave: merge the partials and write the outputs
  const P2Part* pp = w.part2 + (int64_t)b * nw;
  // Every wave of the request has pooled its best pair: leave the word at zero for the next call.
  if (q.kind == kKindBonus && lane == 0)
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(w.bmax + b), 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  bool invalid = false;
  int token = -1;
  float resid = NAN;
  if (q.kind == kKindResidual) {
    double R = 0.0, bk = -1.0;
    int bi = INT32_MAX;
    for (int i = lane; i < nw; i += kWave) {
      const P2Part c2 = read_record64(pp + i);
      if (DIAG) R += (double)c2.rsum;
      if (c2.idx >= 0 && beats(c2.key, c2.idx, bk, bi)) {
        bk = c2.key;
        bi = c2.idx;
      }
    }
    if (DIAG) R = wave_sum(R);
    wave_best(bk, bi);
    resid = DIAG ? (float)R : NAN;
    // A drawn candidate has r > 0 (also in fp32), so a positive best key means the residual
    // has mass, and no candidate means none outside decision-boundary requests.
    if (bk > 0.0) {
      token = bi;
    } else if (FILT && q.th_t > -INFINITY) {  // residual with no mass: the waves' race over p
      double pk = -INFINITY;
      int pi = INT32_MAX;
      for (int i = lane; i < nw; i += kWave) {
        const P2Part c2 = read_record64(pp + i);
        if (c2.pidx >= 0 && beats(c2.pkey, c2.pidx, pk, pi)) {
          pk = c2.pkey;
          pi = c2.pidx;
        }
      }
      wave_best(pk, pi);
      token = pi != INT32_MAX ? pi : p_race_one_wave(in, q, b, lane);
    } else {
      token = p_race_one_wave(in, q, b, lane);  // residual with no mass: race over p
    }
  } else {
    float M = -INFINITY;
    int bad = 0;
    double bk = -INFINITY;
    int bi = INT32_MAX;
    for (int i = lane; i < nw; i += kWave) {
      const P2Part c2 = read_record64(pp + i);
      M = fmaxf(M, c2.mref);
      bad |= c2.bad;
      if (c2.idx >= 0 && beats(c2.key, c2.idx, bk, bi)) {
        bk = c2.key;
        bi = c2.idx;
      }
    }
    M = wave_max(M);
    bad = wave_or(bad);
    wave_best(bk, bi);
    invalid = bad != 0 || M == -INFINITY;
    if (q.kind == kKindGreedyBonus) {
      int gi = INT32_MAX;
      for (int i = lane; i < nw; i += kWave) {
        const P2Part c2 = read_record64(pp + i);
        if (c2.mref == M && c2.gidx >= 0) gi = min(gi, c2.gidx);
      }
      token = wave_min(gi);
    } else {
      invalid = invalid || bi == INT32_MAX;
      token = bi;
    }
  }
  emit_request<FILT>(in, w, out, b, q, invalid, token, resid, lane, q.lo == lo_pre, dt0);
}

// ====================================================================== lazy verify

// Position-serial verify (the survey's "lazy" row): launch j streams row j of every request
// whose rows 0 .. j-1 were all accepted, so rows are read only up to each request's first
// row that is not accepted. A wave of launch j first evaluates row j-1 from its pass-1
// partials exactly as the walk does (eval_rows); a request whose row j-1 is not accepted is
// marked stopped and streams nothing more. Pass 2 then walks and draws unchanged: the
// partials of every row up to the stop are in place, and the rows behind it are never
// decisive (the walk stops at the first row that is not accepted).
template <typename E, int VEC, int U>
__global__ __launch_bounds__(kBlock) void lazy_rows_kernel(Inputs in, Work w, int j, int max_rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (j == 0 && blockIdx.x == 0) block0_duties(in, w, Outputs{nullptr, nullptr, nullptr, nullptr}, max_rows);
  const int nw = in.w1;
  if (gw >= (int64_t)in.B * nw) return;
  const int b = (int)(gw / nw), g = (int)(gw % nw);
  // One round trip: the request head, the drafted token and the stop flag.
  const int lo = in.ro[b], hi = in.ro[b + 1];
  const float T = in.temp[b], tau = in.tau[b];
  const int stop = j > 0 ? w.lazy_stop[b] : 0;
  if (!(0 <= lo && lo < hi && hi <= in.R)) return;  // broken row_offsets: pass 2 fails the batch
  if (j >= hi - lo - 1) return;                      // row j is the request's last row, or beyond
  const int r = lo + j;
  const int D = in.dt[r];
  if (stop != 0 || !temperature_ok(T) || __builtin_isnan(tau) || D < 0 || D >= in.V) return;

  using CH = Chunk<E, VEC>;
  const Span sp = wave_span(in.V / VEC, nw, g);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)r * in.V;
  CH ta[U], da[U];
  if (sp.begin < sp.end) {  // in flight while row j-1 is evaluated
    load_chunks<true>(ta, trow, sp.begin, lane, sp.end);
    load_chunks<true>(da, drow, sp.begin, lane, sp.end);
  }
  if (j > 0) {
    const P1Part e = w.part1[(int64_t)(r - 1) * nw + (lane & (nw - 1))];
    RowStat rs;
    double carry = 1.0;
    const RowEval ev = eval_rows<false>(in, e, lane < nw, nw, b, j - 1, in.dt[r - 1], T, tau, 0.0f, carry, 1,
                                        fold_scale(T), rs);
    if (lane_of(ev.verdict, 0) != SV_ROW_ACCEPT) {
      if (g == 0 && lane == 0) w.lazy_stop[b] = 1;
      return;
    }
  } else if (g == 0 && lane == 0) {
    w.lazy_stop[b] = 0;
  }
  stream_span<E, VEC, U>(in, w, r, g, T, D, trow, drow, sp, ta, da, lane);
}

// ====================================================================== acceptance sums

// Per proposal row r (row j of request b): sum_x min(p(x), mu(x)), the probability that the
// row accepts its draft given its prefix (Strata PR #3416, section Approach; mlxcel PR #992,
// section The acceptance ceiling), and sum_x p(x) q(x), the sampler-match rule's. mu is
// gated at the row's threshold: its step threshold raised by the cumulative floor over the
// drafted tokens before it (regolith audit, section schedule behavior).
//
// The grid and the row of each wave are pass 1's. A wave first evaluates rows lo .. r from
// pass 1's partials exactly as the walk does (eval_rows), in chunks of 64 / w1 rows: that
// gives row r's statistics and gate threshold, and whether every row up to r is valid. It
// then streams its span of row r and writes one partial; merge_sums_kernel adds the w1
// partials of each row in order. A row with an invalid row up to it gets NaN.
// With FILT, p and q are masked by each row's keep-thresholds, and a request whose filter
// values are invalid at T > 0 gets NaN, as the filtered verify fails it.
template <typename E, int VEC, int U, bool FILT = false>
__global__ __launch_bounds__(kBlock) void sums_kernel(Inputs in, Work w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int np = in.R - in.B;
  if (gw >= (int64_t)np * in.w1) return;
  if (!w.hdr->ro_valid) return;
  const int p = (int)(gw / in.w1);
  const int g = (int)(gw % in.w1);
  const RowCls cls = classify_slot(in, p, slot_guess(in, p), lane);
  if (!cls.proposal) return;
  const int r = cls.r, b = cls.b, lo = cls.lo, j = cls.j;
  const float T = cls.T, c = fold_scale(T);
  const float floor = in.min_cum != nullptr ? in.min_cum[b] : 0.0f;
  bool floor_ok = __builtin_isfinite(floor) && floor >= 0.0f;
  if (FILT && T != 0.0f)
    floor_ok = floor_ok && filter_valid(filter_params(in.filt[0], b)) && filter_valid(filter_params(in.filt[1], b));

  const int nw = in.w1;
  const int per = kWave / nw;  // rows per chunk
  double carry = 1.0;
  bool ok = floor_ok;
  RowStat cur{};
  float tau_cur = 0.0f;
  for (int base = 0; base <= j; base += per) {
    const int ri = base + (int)(lane / nw);
    const bool live = ri <= j;
    const int rr = lo + min(ri, j);
    const P1Part e = w.part1[(int64_t)rr * nw + (lane & (nw - 1))];
    const int Di = in.dt[rr];
    const float tsi = in.tau_step != nullptr ? in.tau_step[rr] : cls.tau;
    const int nlive = min(per, j + 1 - base);
    float th_t = -INFINITY, th_d = -INFINITY;
    if (FILT) {
      th_t = in.theta[2 * (int64_t)rr];
      th_d = in.theta[2 * (int64_t)rr + 1];
    }
    RowStat rs;
    const RowEval ev = eval_rows<true, FILT>(in, e, live, nw, b, min(ri, j), Di, T, tsi, floor_ok ? floor : 0.0f,
                                             carry, nlive, c, rs, th_t, th_d);
    ok = ok && __ballot(live && ev.verdict == kRowInvalid) == 0;
    if (base + per > j) {  // the chunk that holds row r
      const int src = (j - base) * nw;
      cur = RowStat{lane_of(rs.m_t, src), lane_of(rs.mc_t, src), lane_of(rs.m_d, src), lane_of(rs.mc_d, src),
                    lane_of(rs.s_t, src), lane_of(rs.s_d, src), lane_of(rs.am_t, src), lane_of(rs.am_d, src)};
      tau_cur = lane_of(ev.tau_eff, src);
    }
  }

  double smin = 0.0, spq = 0.0;
  if (!ok) {
    smin = spq = NAN;
  } else if (T == 0.0f) {  // one-hot p and q: both sums are [argmax p == argmax q] (the first also needs tau <= 1)
    if (g == 0) {
      smin = (cur.am_t == cur.am_d && 1.0f >= tau_cur) ? 1.0 : 0.0;
      spq = cur.am_t == cur.am_d ? 1.0 : 0.0;
    }
  } else {
    using CH = Chunk<E, VEC>;
    const int nvec = in.V / VEC;
    const Span sp = wave_span(nvec, nw, g);
    const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
    const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)r * in.V;
    const float mct = cur.mc_t, mcd = cur.mc_d, tau = tau_cur;
    const float ist = (float)(1.0 / cur.s_t), isd = (float)(1.0 / cur.s_d);
    const float tht = FILT ? in.theta[2 * (int64_t)r] : -INFINITY;
    const float thd = FILT ? in.theta[2 * (int64_t)r + 1] : -INFINITY;
    constexpr int step = U * kWave;
    float am = 0.0f, apq = 0.0f;
    CH ta[U], da[U], tb[U], db[U];
    auto fold = [&](const CH (&xt)[U], const CH (&xd)[U]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float pp = fast_exp2(fmaf(xt[u].get(e), c, -mct)) * ist;
          float qq = fast_exp2(fmaf(xd[u].get(e), c, -mcd)) * isd;
          if (FILT) {
            pp = xt[u].get(e) < tht ? 0.0f : pp;
            qq = xd[u].get(e) < thd ? 0.0f : qq;
          }
          am += fminf(pp, qq >= tau ? qq : 0.0f);
          apq = fmaf(pp, qq, apq);
        }
      }
    };
    const int nsteps = (sp.end - sp.begin + step - 1) / step;
    if (nsteps > 0) {
      load_chunks<true>(ta, trow, sp.begin, lane, sp.end);
      load_chunks<true>(da, drow, sp.begin, lane, sp.end);
    }
    for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
      load_chunks<true>(tb, trow, base + step, lane, sp.end);
      load_chunks<true>(db, drow, base + step, lane, sp.end);
      mask_chunks(ta, base, lane, sp.end);
      mask_chunks(da, base, lane, sp.end);
      fold(ta, da);
      load_chunks<true>(ta, trow, base + 2 * step, lane, sp.end);
      load_chunks<true>(da, drow, base + 2 * step, lane, sp.end);
      mask_chunks(tb, base + step, lane, sp.end);
      mask_chunks(db, base + step, lane, sp.end);
      fold(tb, db);
    }
    smin = wave_sum((double)am);
    spq = wave_sum((double)apq);
  }
  if (lane == 0) {
    w.part3[(int64_t)r * nw + g] = SumPart{smin, spq};
    if (g == 0) w.done3[r] = 1u;
  }
}

// Adds each row's w1 partials in wave order. Rows without partials get NaN. Every done flag
// is reset for the next call.
__global__ __launch_bounds__(kBlock) void merge_sums_kernel(Inputs in, Work w, float* out_min, float* out_pq) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x; r < in.R; r += stride) {
    float m = NAN, pq = NAN;
    if (w.done3[r] != 0u) {
      double sm = 0.0, sp = 0.0;
      for (int g = 0; g < in.w1; ++g) {
        const SumPart s = w.part3[r * in.w1 + g];
        sm += s.smin;
        sp += s.spq;
      }
      m = (float)sm;
      pq = (float)sp;
      w.done3[r] = 0u;
    }
    out_min[r] = m;
    out_pq[r] = pq;
  }
}

// ====================================================================== filter chain

// The sampler's filter chain (mlxcel PR #992, section What changed): temperature scale,
// top-k, then top-p on what top-k leaves, then min-p. Each filter keeps the tokens whose
// logit reaches a threshold, ties included, so one float per row and side describes the
// kept set: token x is kept iff !(l_x < theta). One workgroup finds theta for one row and
// side.
//  - Pass A reads the row for its maximum m and validity, and keeps per segment (the 64
//    vectors one wave instruction reads) its largest logit and, for top-p alone, its fp32
//    mass. min-p's threshold follows from m alone: the smallest float y with
//    (y - m) / T >= ln(min_p) in fp64.
//  - Pass B gathers into LDS the logits that can hold the thresholds: those at or above the
//    k-th largest of the segments' (or threads') maxima (top-k), or within
//    W = log2(V / (1 - top_p)) + 1 log2 units of mass below m (top-p alone, which holds its
//    crossing), and sums the fp32 mass of the others. It re-reads only the segments whose
//    maximum reaches that bound; the other segments' mass comes from their records.
//  - The candidates are sorted (bitonic, in LDS). top-k's threshold is the k-th; top-p's is
//    where the fp64 prefix mass of exp((l - m) / T) first reaches top_p times top-k's mass.
//  - When the window holds more than kCandCap logits, or fewer than top-k's k, the filters
//    are decided by bisection over the float order, one pass over the row per step: top-k
//    on counts (after which top-k's set is gathered for top-p when it fits), top-p on fp64
//    masses. Exact; the second is slow. Peaked rows keep the window small.
constexpr int kFiltBlock = 512;  // threads per (row, side); at most 80 VGPRs: 3 workgroups per CU fit
constexpr int kFiltWaves = kFiltBlock / kWave;
constexpr int kCandCap = 8192;     // candidate logits one workgroup sorts in LDS
constexpr int kFiltSegCap = 1024;  // segments one workgroup keeps records of in LDS

// Total order on non-NaN floats as int32: order_key(a) < order_key(b) iff a < b, with -0
// just below +0.
__device__ __forceinline__ int32_t order_key(float f) {
  const int32_t i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float key_float(int32_t k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }


// A segment is the kWave vectors one wave instruction of walk_row reads: vectors
// [kWave * s, kWave * s + kWave) of the row.
struct FilterSmem {
  float cand[kCandCap];
  float seg_max[kFiltSegCap];   // each segment's largest logit
  float seg_mass[kFiltSegCap];  // with top-p alone: sum of exp2((l - seg_max) * c) over the segment
  int seg_list[kFiltSegCap];    // the segments that hold candidates
  double red[kFiltWaves];
  int wcount[kFiltWaves];   // per-wave counts of an ordered compaction
  int n_cand, first, n_seg;
};

__device__ __forceinline__ double block_sum(double v, FilterSmem& s) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s.red[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kFiltWaves; ++w) t += s.red[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, FilterSmem& s) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s.red[threadIdx.x / kWave] = (double)v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int w = 0; w < kFiltWaves; ++w) t = fmaxf(t, (float)s.red[w]);
  return t;
}

// Walk a row with every thread of the workgroup: step st covers the kFiltBlock * kFiltLoads
// vectors from st * kFiltBlock * kFiltLoads on, kFiltLoads per thread, strided by kFiltBlock.
// Every lane runs every step (a lane past the row's end re-reads the row's last vector, a
// cache hit, and sees ok = false), so the step function may use wave-wide operations. Loads
// are double-buffered: the next step's vectors are in flight while step(x, ok, st) works on
// the current ones.
constexpr int kFiltLoads = 2;

template <typename E, int VEC, class S>
__device__ __forceinline__ void walk_row(const E* row, int nvec, S step) {
  using CH = Chunk<E, VEC>;
  constexpr int per = kFiltBlock * kFiltLoads;
  const int steps = (nvec + per - 1) / per;
  auto load = [&](CH (&x)[kFiltLoads], int st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kFiltLoads; ++u)
      x[u].load(row + (int64_t)min(st * per + u * kFiltBlock + (int)threadIdx.x, nvec - 1) * VEC);
  };
  auto run = [&](const CH (&x)[kFiltLoads], int st) __attribute__((always_inline)) {
    bool ok[kFiltLoads];
#pragma unroll
    for (int u = 0; u < kFiltLoads; ++u) ok[u] = st * per + u * kFiltBlock + (int)threadIdx.x < nvec;
    step(x, ok, st);
  };
  CH xa[kFiltLoads], xb[kFiltLoads];
  if (steps > 0) load(xa, 0);
  for (int st = 0; st < steps; st += 2) {  // an odd count ends with a step that is all ok = false
    load(xb, st + 1);
    run(xa, st);
    load(xa, st + 2);
    run(xb, st + 1);
  }
}

// Run f(x) on every logit of a row (no wave-wide operations in f).
template <typename E, int VEC, class F>
__device__ __forceinline__ void for_each_logit(const E* row, int nvec, F f) {
  walk_row<E, VEC>(row, nvec, [&](const Chunk<E, VEC>(&x)[kFiltLoads], const bool (&ok)[kFiltLoads], int)
                                  __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kFiltLoads; ++u)
      if (ok[u]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) f(x[u].get(e));
      }
  });
}

// Number of logits >= v.
template <typename E, int VEC>
__device__ __forceinline__ double count_ge(const E* row, int nvec, float v, FilterSmem& s) {
  int n = 0;
  for_each_logit<E, VEC>(row, nvec, [&](float x) __attribute__((always_inline)) { n += !(x < v); });
  return block_sum((double)n, s);
}

// fp64 mass of the logits >= v: sum of exp((l - m) / T).
template <typename E, int VEC>
__device__ __forceinline__ double mass_ge(const E* row, int nvec, float v, float m, double T, FilterSmem& s) {
  double t = 0.0;
  for_each_logit<E, VEC>(row, nvec, [&](float x) __attribute__((always_inline)) {
    if (!(x < v)) t += exp(((double)x - (double)m) / T);
  });
  return block_sum(t, s);
}

// Largest float v in [lo, hi] with pred(v), by bisection over order_key; pred(lo) holds and
// pred is monotone (true below some point, false above).
template <class P>
__device__ float bisect_float(float lo, float hi, P pred) {
  int64_t a = order_key(lo), z = order_key(hi);
  if (pred(key_float((int32_t)z))) return hi;
  while (z - a > 1) {
    const int64_t mid = a + (z - a) / 2;
    if (pred(key_float((int32_t)mid))) a = mid;
    else z = mid;
  }
  return key_float((int32_t)a);
}

// Keep-threshold of row r, side `side`, by the whole workgroup. With top-p alone, lo_hint
// may raise the candidate bound: a value that at least top_p of the row's mass reaches (the
// top-p scan still checks it).
template <typename E, int VEC>
__device__ __forceinline__ void thresholds_row(const Inputs& in, const FilterArgs& fa, int r, int side, FilterSmem& s,
                                               float lo_hint = -INFINITY) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float* out = fa.theta + 2 * (int64_t)r + side;

  // The row's request: the guess for equal lengths, else a binary search. Every index stays
  // in bounds whatever row_offsets holds (a broken batch fails in pass 2).
  int b = min((int)(((int64_t)r * in.B) / in.R), in.B - 1);
  if (!(in.ro[b] <= r && r < in.ro[b + 1])) {
    int L = 0, H = in.B - 1;
    while (L < H) {
      const int mid = (L + H + 1) >> 1;
      if (in.ro[mid] <= r) L = mid; else H = mid - 1;
    }
    b = L;
  }
  const float T = in.temp[b];
  const FilterParams fp = filter_params(fa.side[side], b);
  const bool topk = fp.k > 0 && fp.k < in.V;
  const bool topp = fp.top_p < 1.0f;
  const bool minp = fp.min_p > 0.0f;
  if (!(T > 0.0f) || !temperature_ok(T) || !filter_valid(fp) || !(topk || topp || minp)) {
    if (threadIdx.x == 0) *out = -INFINITY;
    return;
  }
  const E* row = reinterpret_cast<const E*>(side == 0 ? in.target : in.draft) + (int64_t)r * in.V;
  const int nvec = in.V / VEC;
  const double Td = (double)T;

  // Sort s.cand[0, n) largest first (bitonic, padded with -inf).
  auto sort_desc = [&](int n) __attribute__((always_inline)) {
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    for (int i = n + threadIdx.x; i < np2; i += kFiltBlock) s.cand[i] = -INFINITY;
    __syncthreads();
    for (int k = 2; k <= np2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = threadIdx.x; i < np2; i += kFiltBlock) {
          const int ij = i ^ j;
          if (ij > i) {
            const float a = s.cand[i], z = s.cand[ij];
            if (((i & k) == 0) ? (a < z) : (a > z)) {
              s.cand[i] = z;
              s.cand[ij] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  };
  const float c = scale_of(T);  // log2(e) / T
  // Segment records bound the candidates for top-k when k is at most the segment count, and
  // for top-p alone; the gather then reads only the segments that can hold candidates.
  const int nseg = (nvec + kWave - 1) / kWave;
  const bool seg_k = topk && fp.k <= nseg && nseg <= kFiltSegCap;
  const bool seg_p = !topk && topp && nseg <= kFiltSegCap;
  const bool segs = seg_k || seg_p;
  // ---- pass A: maximum and validity; each thread's largest logit; each segment's largest
  //      logit and, with top-p alone, its mass relative to that logit
  float mx = -INFINITY;
  int bad = 0;
  walk_row<E, VEC>(row, nvec, [&](const Chunk<E, VEC>(&x)[kFiltLoads], const bool (&ok)[kFiltLoads], int st)
                                  __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kFiltLoads; ++u) {
      float vm = -INFINITY;
      if (ok[u]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = x[u].get(e);
          vm = fmaxf(vm, v);
          bad |= (int)(__builtin_isnan(v) || v == INFINITY);
        }
      }
      mx = fmaxf(mx, vm);
      if (segs) {
        const int sg = (st * kFiltLoads + u) * kFiltWaves + wave;  // vectors [kWave * sg, + kWave)
        const float sm = wave_max(vm);
        float ms = 0.0f;
        if (seg_p) {
          if (ok[u] && sm > -INFINITY) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) ms += fast_exp2((x[u].get(e) - sm) * c);
          }
          ms = wave_sum(ms);
        }
        if (lane == 0 && sg < nseg) {
          s.seg_max[sg] = sm;
          s.seg_mass[sg] = ms;
        }
      }
    }
  });
  const float m = block_max(mx, s);
  const bool valid = block_sum((double)bad, s) == 0.0 && m != -INFINITY;
  if (!valid) {
    if (threadIdx.x == 0) *out = INFINITY;
    return;
  }
  // min-p: the smallest float y with (y - m) / T >= ln(min_p), in fp64.
  float th_m = -INFINITY;
  if (minp) {
    const double lm = log((double)fp.min_p);
    auto keep = [&](float y) { return ((double)y - (double)m) / Td >= lm; };
    float y = (float)((double)m + Td * lm);
    for (int it = 0; it < 64 && !keep(y); ++it) y = nextafterf(y, INFINITY);
    for (int it = 0; it < 64 && keep(nextafterf(y, -INFINITY)); ++it) y = nextafterf(y, -INFINITY);
    th_m = y;
  }
  if (!topk && !topp) {
    if (threadIdx.x == 0) *out = th_m;
    return;
  }

  // ---- the candidates to gather
  //  - With top-k: the logits at or above the k-th largest of the segments' maxima (k at
  //    most the segment count), else of the threads' maxima (k <= kFiltBlock). Segments and
  //    threads each split the row into disjoint parts, so at least k logits reach that
  //    value: it is at most top-k's threshold, and top-p's crossing lies above top-k's.
  //  - With top-p alone: the logits within W = log2(V / (1 - top_p)) + 1 log2 units of mass
  //    below the maximum. A logit below that has mass under 2^-W of the maximum's, so all of
  //    them together hold less than V * 2^-W < (1 - top_p) of the row's mass (which holds
  //    the maximum): the crossing lies inside.
  //  - With top-k beyond both alone: a 24-unit window, a guess checked below.
  const float W = topp ? log2f((float)in.V / (1.0f - fp.top_p)) + 1.0f : 24.0f;
  float edge = -INFINITY;
  const bool by_edge = topk && (seg_k || fp.k <= kFiltBlock);
  if (seg_k) {
    for (int i = threadIdx.x; i < nseg; i += kFiltBlock) s.cand[i] = s.seg_max[i];
    sort_desc(nseg);
    edge = s.cand[fp.k - 1];
    __syncthreads();
  } else if (by_edge) {
    s.cand[threadIdx.x] = mx;  // -inf for a thread that read nothing
    sort_desc(kFiltBlock);
    edge = s.cand[fp.k - 1];
    __syncthreads();
  }
  // One bound for both: the gathered logits are those >= lo. The window's bound sits a little
  // below m - W / c, so that fp32 rounding can only widen it.
  const float lo = by_edge ? edge : topk ? m - (W + 0.01f) / c : fmaxf(m - (W + 0.01f) / c, lo_hint);
  // ---- gather, sort, scan
  // gather(bound, ...): the logits >= the bound go to s.cand. Returns how many there are
  // (those past kCandCap are counted, not stored). Per step each lane counts its candidates
  // and, holding any, reserves their slots with one LDS atomic and stores them. With
  // sum_rest, the fp32 mass of the other logits goes to `rest` (per vector in fp32, per lane
  // in fp64).
  auto gather = [&](const float lo, const bool sum_rest, double& rest) __attribute__((always_inline)) {
    if (threadIdx.x == 0) s.n_cand = 0;
    __syncthreads();
    double tl = 0.0;
    walk_row<E, VEC>(row, nvec, [&](const Chunk<E, VEC>(&x)[kFiltLoads], const bool (&ok)[kFiltLoads], int)
                                    __attribute__((always_inline)) {
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < kFiltLoads; ++u) {
        float ts = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = x[u].get(e);
          const bool cand = ok[u] && !(v < lo);
          cnt += cand ? 1 : 0;
          if (sum_rest && ok[u] && !cand) ts += fast_exp2((v - m) * c);
        }
        if (sum_rest) tl += (double)ts;
      }
      if (cnt == 0) return;
      int slot = atomicAdd(&s.n_cand, cnt);  // candidates are sparse: one LDS atomic per lane holding any
#pragma unroll
      for (int u = 0; u < kFiltLoads; ++u) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = x[u].get(e);
          if (ok[u] && !(v < lo)) {
            if (slot < kCandCap) s.cand[slot] = v;
            ++slot;
          }
        }
      }
    });
    rest = block_sum(tl, s);  // its barriers also publish s.n_cand and s.cand
    return s.n_cand;
  };
  // gather_segments(bound, ...): the same, reading only the segments whose largest logit
  // reaches the bound; with sum_rest the other segments' mass comes from their records. Each
  // wave reads kFiltLoads listed segments per round trip.
  auto gather_segments = [&](const float lo, const bool sum_rest, double& rest) __attribute__((always_inline)) {
    if (threadIdx.x == 0) s.n_cand = 0;
    // The listed segments keep their row order (a ballot per wave and a count over the
    // waves), so every run hands each wave and lane the same segments and sums the same
    // masses in the same order.
    double tl = 0.0;
    int ns = 0;  // segments listed so far, the same in every thread
    for (int base = 0; base < nseg; base += kFiltBlock) {
      const int i = base + (int)threadIdx.x;
      bool take = false;
      if (i < nseg) {
        const float sm = s.seg_max[i];
        take = !(sm < lo);
        if (!take && sum_rest && sm > -INFINITY) tl += (double)s.seg_mass[i] * (double)fast_exp2((sm - m) * c);
      }
      const uint64_t mk = __ballot(take);
      if (lane == 0) s.wcount[wave] = (int)__popcll(mk);
      __syncthreads();
      int before = ns, total = 0;
#pragma unroll
      for (int w = 0; w < kFiltWaves; ++w) {
        before += w < wave ? s.wcount[w] : 0;
        total += s.wcount[w];
      }
      if (take) s.seg_list[before + lane_rank(mk)] = i;
      ns += total;
      __syncthreads();
    }
    for (int i0 = wave; i0 < ns; i0 += kFiltWaves * kFiltLoads) {
      Chunk<E, VEC> x[kFiltLoads];
      bool ok[kFiltLoads];
#pragma unroll
      for (int g = 0; g < kFiltLoads; ++g) {
        const int i = i0 + g * kFiltWaves;
        const int v = i < ns ? s.seg_list[i] * kWave + lane : nvec;
        ok[g] = v < nvec;
        x[g].load(row + (int64_t)min(v, nvec - 1) * VEC);
      }
      int cnt = 0;
#pragma unroll
      for (int g = 0; g < kFiltLoads; ++g) {
        float ts = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = x[g].get(e);
          const bool cand = ok[g] && !(v < lo);
          cnt += cand ? 1 : 0;
          if (sum_rest && ok[g] && !cand) ts += fast_exp2((v - m) * c);
        }
        if (sum_rest) tl += (double)ts;
      }
      if (cnt > 0) {
        int slot = atomicAdd(&s.n_cand, cnt);
#pragma unroll
        for (int g = 0; g < kFiltLoads; ++g) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float v = x[g].get(e);
            if (ok[g] && !(v < lo)) {
              if (slot < kCandCap) s.cand[slot] = v;
              ++slot;
            }
          }
        }
      }
    }
    rest = block_sum(tl, s);  // its barriers also publish s.n_cand and s.cand
    return s.n_cand;
  };
  // top-p over the sorted candidates s.cand[0, nk), which hold top-k's whole set; S1 is their
  // fp64 mass plus `extra` (the mass of top-k's set outside them). Returns the logit at the
  // first position whose prefix mass reaches top_p * S1, or NaN when the candidates hold less.
  auto top_p_scan = [&](int nk, double extra) __attribute__((always_inline)) {
    const int ch = (nk + kFiltBlock - 1) / kFiltBlock;
    const int i0 = min((int)threadIdx.x * ch, nk), i1 = min(i0 + ch, nk);
    double own = 0.0;
    for (int i = i0; i < i1; ++i) own += exp(((double)s.cand[i] - (double)m) / Td);
    double incl = own;  // inclusive prefix over the wave's lanes, then over the waves
    for (int d = 1; d < kWave; d <<= 1) {
      const double t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    __syncthreads();
    if (lane == kWave - 1) s.red[wave] = incl;
    if (threadIdx.x == 0) s.first = INT32_MAX;
    __syncthreads();
    double before = 0.0, total = 0.0;
#pragma unroll
    for (int w = 0; w < kFiltWaves; ++w) {
      before += w < wave ? s.red[w] : 0.0;
      total += s.red[w];
    }
    const double target = (double)fp.top_p * (total + extra);
    double run = before + incl - own;  // exclusive prefix of this thread's chunk
    for (int i = i0; i < i1; ++i) {
      run += exp(((double)s.cand[i] - (double)m) / Td);
      if (run >= target) {
        atomicMin(&s.first, i);
        break;
      }
    }
    __syncthreads();
    const int ip = s.first;
    const float th = ip != INT32_MAX ? s.cand[ip] : NAN;
    __syncthreads();
    return th;
  };
  // Candidates at or above th in the sorted s.cand[0, n), given that the first k are.
  auto count_prefix = [&](int n, int k, float th) __attribute__((always_inline)) {
    if (threadIdx.x == 0) s.first = n;
    __syncthreads();
    for (int i = k - 1 + threadIdx.x; i < n - 1; i += kFiltBlock)
      if (s.cand[i + 1] < th) atomicMin(&s.first, i + 1);
    __syncthreads();
    const int nk = s.first;
    __syncthreads();
    return nk;
  };

  float th_k = -INFINITY, th_p = -INFINITY;
  bool have_k = !topk;  // top-k's threshold is known
  int n = -1;           // sorted candidates in s.cand (-1: none usable)
  double rest = 0.0;    // fp32 mass of the logits outside them
  {
    const int nw = segs ? gather_segments(lo, seg_p, rest) : gather(lo, topp && !topk, rest);
    if (nw <= kCandCap) {
      n = nw;
      sort_desc(n);
      if (topk && n >= fp.k) {
        th_k = s.cand[fp.k - 1];
        have_k = true;
      }
    }
  }
  if (!have_k) {
    // More logits lie above top-k's threshold than the cut gathered: bisect on counts, then
    // gather top-k's set for top-p when it fits.
    const double kk = (double)fp.k;
    th_k = bisect_float(-INFINITY, m, [&](float v) { return count_ge<E, VEC>(row, nvec, v, s) >= kk; });
    have_k = true;
    n = -1;
    if (topp && count_ge<E, VEC>(row, nvec, th_k, s) <= (double)kCandCap) {
      n = gather(th_k, false, rest);
      sort_desc(n);
    }
  }
  if (topp) {
    float th = NAN;
    if (n >= 0) {
      if (topk) th = top_p_scan(count_prefix(n, min(fp.k, n), th_k), 0.0);  // S1: top-k's set, all gathered
      else th = top_p_scan(n, rest);                                          // S1: the whole row
    }
    if (__builtin_isnan(th)) {
      // The candidates hold less than top_p of the mass: bisect on fp64 masses.
      const double S1 = mass_ge<E, VEC>(row, nvec, th_k, m, Td, s);
      const double target = (double)fp.top_p * S1;
      th = bisect_float(th_k, m, [&](float v) { return mass_ge<E, VEC>(row, nvec, v, m, Td, s) >= target; });
    }
    th_p = th;
  }
  if (threadIdx.x == 0) *out = fmaxf(fmaxf(th_k, th_p), th_m);
}

// Workgroup i takes row i / 2, side i % 2.
template <typename E, int VEC>
__global__ __launch_bounds__(kFiltBlock) __attribute__((amdgpu_waves_per_eu(6))) void thresholds_kernel(Inputs in, FilterArgs fa) {
  __shared__ FilterSmem s;
  thresholds_row<E, VEC>(in, fa, (int)(blockIdx.x >> 1), (int)(blockIdx.x & 1), s);
}

// ====================================================================== sampler-match rule

// The comparison rule of mlxcel PR #992, section The premise correction: every tested row
// takes a fresh draw t from the target p, the drafted token is accepted iff it equals t,
// and t is emitted on both branches. Its acceptance is sum_x p(x) q(x) (the same page,
// section The acceptance ceiling). The draw on row j of request b is the race over p with
// the same random numbers as the method's race on that row; at temperature 0 it is the
// lowest-index argmax.
//
// match_rows_kernel races every row of the batch: wave gw takes span gw % nw of row
// gw / nw and writes one MatchPart. match_emit_kernel then walks each request with one
// wave, merging the partials of up to 64 / nw rows per round trip.
struct MatchPart {
  double key;    // best fp64 log key l/T - ln E of the span (T > 0)
  int32_t idx;   // its token (-1 if none)
  float m;       // largest logit of the span
  int32_t bad;   // the span holds NaN or +inf
  int32_t gidx;  // lowest index of m in the span (T = 0)
};
static_assert(sizeof(MatchPart) == 24, "MatchPart layout");

// Request of row r: the guess for equal-length requests, else a binary search. Every read
// stays in [0, B] whatever row_offsets holds; a broken batch is failed by the emit kernel.
__device__ __forceinline__ int request_of_row(const Inputs& in, int r) {
  int b = (int)((int64_t)r * in.B / in.R);
  if (in.ro[b] <= r && r < in.ro[b + 1]) return b;
  int lo = 0, hi = in.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (in.ro[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <typename E, int VEC, int U>
__global__ __launch_bounds__(kBlock) void match_rows_kernel(Inputs in, Work w, MatchPart* parts, int nw) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (blockIdx.x == 0) block0_duties(in, w, Outputs{nullptr, nullptr, nullptr, nullptr});
  if (gw >= (int64_t)in.R * nw) return;
  const int r = (int)(gw / nw), g = (int)(gw % nw);
  const int b = uni(request_of_row(in, r));
  const int j = r - in.ro[b];  // the row's position in its request (a counter word only)
  const float T = in.temp[b];
  const bool race = T != 0.0f;
  const float c = race ? scale_of(T) : 1.0f;

  using CH = Chunk<E, VEC>;
  constexpr int step = U * kWave;
  constexpr int G = VEC >= 4 ? 4 : 1;  // logits sharing one Philox block
  const Span sp = wave_span(in.V / VEC, nw, g);
  const int nsteps = (sp.end - sp.begin + step - 1) / step;
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
  const uint32_t k0 = seed_lo(in.seed), k1 = seed_hi(in.seed);

  Acc a = acc_empty();
  int bad = 0;
  Top2 t = top2_empty();
  float wbest = -INFINITY;
  CH ta[U], tb[U];
  auto fold = [&](const CH (&xt)[U], int v0) __attribute__((always_inline)) {
    if (!race) {
      fold_max<true>(a, xt, v0, bad);
      return;
    }
    fold_max<false>(a, xt, v0, bad);
    // A log2 key l*c - log2(E) lies within (l*c - 4.06, l*c + 24), so a token more than 28.1
    // below the wave's largest l*c cannot win (the bonus race's bound, with fp32 margins).
    const float lb = fmaxf(wbest, wave_max(a.m) * c - 4.1f);
    float lbest = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x0 = (v0 + u * kWave) * VEC;
#pragma unroll
      for (int gg = 0; gg < VEC; gg += G) {
        float av[G];
        bool any = false;
#pragma unroll
        for (int e = 0; e < G; ++e) {
          av[e] = xt[u].get(gg + e) * c;
          any |= av[e] + 25.0f >= lb;
        }
        if (any) {
          const int xg = x0 + gg;
          const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)j, (uint32_t)b, k0, k1);
#pragma unroll
          for (int e = 0; e < G; ++e) {
            if (av[e] + 25.0f >= lb) {
              const int x = xg + e;
              const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, x & 3);
              const float key = av[e] - log2_expo32(wd);
              lbest = fmaxf(lbest, key);
              top2_push(t, key, x, xt[u].get(gg + e), 0.0f);
            }
          }
        }
      }
    }
    wbest = fmaxf(wbest, wave_max(lbest));
  };
  if (nsteps > 0) load_chunks<true>(ta, trow, sp.begin, lane, sp.end);
  for (int i = 0, base = sp.begin; i < nsteps; i += 2, base += 2 * step) {
    load_chunks<true>(tb, trow, base + step, lane, sp.end);
    mask_chunks(ta, base, lane, sp.end);
    fold(ta, base + lane);
    load_chunks<true>(ta, trow, base + 2 * step, lane, sp.end);
    mask_chunks(tb, base + step, lane, sp.end);
    fold(tb, base + step + lane);
  }
  float m, unused;
  int am;
  wave_stat(a, 0.0f, false, m, unused, am);
  MatchPart part;
  part.m = m;
  part.bad = wave_or(bad);
  part.gidx = race ? -1 : exact_argmax<CH>(trow, a, m);
  part.key = -INFINITY;
  part.idx = -1;
  if (race) {
    double bk;
    int bi;
    resolve_race(t, wave_max(t.k1) - kLogKeySlack,
                 [&](int x, float l, float) {
                   return p_logkey64((double)l, (double)T, race_word(in.seed, x, j, b));
                 },
                 bk, bi);
    part.key = bk;
    part.idx = bi == INT32_MAX ? -1 : bi;
  }
  if (lane == 0) parts[gw] = part;
}

// Best (key, index) within aligned groups of `width` lanes (a power of two).
__device__ __forceinline__ void seg_best(double& k, int& i, int width) {
  for (int o = 1; o < width; o <<= 1) {
    const double ko = __shfl_xor(k, o);
    const int io = __shfl_xor(i, o);
    if (beats(ko, io, k, i)) {
      k = ko;
      i = io;
    }
  }
}

// One wave per request. Each round trip brings the partials of 64 / nw rows, lane
// jj * nw + g holding span g of row jj; each aligned group of nw lanes merges its row.
__global__ __launch_bounds__(kBlock) void match_emit_kernel(Inputs in, Work w, const MatchPart* parts, int nw,
                                                             Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (gw >= in.B) return;
  const int b = (int)gw;
  if (!w.hdr->ro_valid) {
    // Broken row_offsets: every output is -1. Request b clears an even share of the rows.
    const int64_t r0 = (int64_t)b * in.R / in.B, r1 = (int64_t)(b + 1) * in.R / in.B;
    for (int64_t r = r0 + lane; r < r1; r += kWave) out.tokens[r] = -1;
    if (lane == 0) out.accept_len[b] = -1;
    return;
  }
  const int lo = in.ro[b], hi = in.ro[b + 1];
  const int n = hi - lo;
  const float T = in.temp[b];
  const int per = kWave / nw;  // rows per round trip
  const int jj = lane / nw, g = lane % nw;
  int stop = -1, stop_tok = -1;
  bool invalid = !temperature_ok(T);
  for (int base = 0; base < n && stop < 0 && !invalid; base += per) {
    const int row = base + jj;
    const bool live = row < n;
    MatchPart e{-INFINITY, -1, -INFINITY, 0, -1};
    int D = -1;
    if (live) {
      e = parts[(int64_t)(lo + row) * nw + g];
      D = in.dt[lo + row];
    }
    float M = seg_max(e.m, nw);
    const int bad = seg_reduce(e.bad, OpOr{}, nw);
    double k = e.key;
    int i = e.idx >= 0 ? e.idx : INT32_MAX;
    seg_best(k, i, nw);
    const int gi = seg_min(e.m == M && e.gidx >= 0 ? e.gidx : INT32_MAX, nw);
    const int tok = T != 0.0f ? (i == INT32_MAX ? -1 : i) : (gi == INT32_MAX ? -1 : gi);
    const bool row_bad = live && (bad != 0 || M == -INFINITY || tok < 0);
    const bool bonus = row == n - 1 || D < 0 || D >= in.V;
    const bool ends = live && (row_bad || bonus || D != tok);
    // The first row of this round, in order, that ends the request.
    const uint64_t ended = __ballot(g == 0 && ends);
    if (ended != 0) {
      const int first_lane = __builtin_ctzll(ended);
      stop = base + first_lane / nw;
      stop_tok = __shfl(tok, first_lane);
      invalid = __shfl((int)row_bad, first_lane) != 0;
    }
  }
  if (!(stop >= 0) || invalid) {
    for (int r = lo + lane; r < hi; r += kWave) out.tokens[r] = -1;
    if (lane == 0) out.accept_len[b] = -1;
    return;
  }
  // Rows before the stop accepted their drafted tokens; the stop row emits its draw.
  for (int r = lo + lane; r < hi; r += kWave) {
    const int j = r - lo;
    out.tokens[r] = j < stop ? in.dt[r] : j == stop ? stop_tok : -1;
  }
  if (lane == 0) out.accept_len[b] = stop;
}

// ====================================================================== filter chain: segment records

// Row sides whose keep-threshold the verify never reads. A request stops at its first row
// without a proposal (a drafted token outside [0, V); every request's last row is one), and
// that row draws from p alone. So the draft side of such a row is never read, nor either side
// of the rows after it. Row r of request b; wave-uniform.
__device__ __forceinline__ bool side_unused(const Inputs& in, int b, int r, int side, int lane) {
  const int lo = min(max(in.ro[b], 0), r);
  for (int base = lo; base < r; base += kWave) {
    const int j = base + lane;
    const bool none = j < r && (unsigned)in.dt[j] >= (unsigned)in.V;
    if (__ballot(none) != 0) return true;
  }
  return side == 1 && (unsigned)in.dt[r] >= (unsigned)in.V;
}

// The filter chain's thresholds in two launches when rows are read in 16-byte vectors and
// hold at most kSegCap segments (thresholds_kernel alone otherwise):
//  - seg_records_kernel streams every row and side that has an active filter, nw waves each,
//    and writes one SegRec per segment (its largest logit, and with top-p alone its mass);
//  - thresholds_finish_kernel takes one workgroup per row and side and decides the thresholds
//    from the records (the candidate bound, the gather of the listed segments, top-k and
//    top-p over the candidates). The rows and sides the records cannot decide (top-k beyond
//    the segment count, too many candidates, candidates short of top_p) take the exact path
//    of thresholds_kernel (thresholds_row) in the same workgroup.

// A record's segment holds kSegLogits logits, SV 16-byte vectors per lane of a wave (one of
// bf16, two of fp32): lane l's v-th vector of segment sg is vector (sg * SV + v) * kWave + l
// of the row.

template <typename E, int VEC>
__global__ __launch_bounds__(kBlock) void seg_records_kernel(Inputs in, FilterArgs fa, int nw) {
  constexpr int SV = kSegLogits / (kWave * VEC);
  static_assert(SV >= 1 && SV * kWave * VEC == kSegLogits, "segment shape");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (gw >= (int64_t)in.R * 2 * nw) return;
  const int rs = (int)(gw / nw), g = (int)(gw % nw);
  const int r = rs >> 1, side = rs & 1;
  const int b = uni(request_of_row(in, r));
  const float T = in.temp[b];
  const FilterParams fp = filter_params(fa.side[side], b);
  const bool topk = fp.k > 0 && fp.k < in.V, topp = fp.top_p < 1.0f, minp = fp.min_p > 0.0f;
  if (!(T > 0.0f) || !temperature_ok(T) || !filter_valid(fp) || !(topk || topp || minp)) return;
  const int nseg = fa.nseg, nvec = in.V / VEC;
  const int per = (nseg + nw - 1) / nw;
  const int s0 = min(g * per, nseg), s1 = min(s0 + per, nseg);
  SegRec* rec = fa.seg + (int64_t)rs * nseg;
  if (fa.skip_unused && side_unused(in, b, r, side, lane)) {
    // Not streamed: each wave marks its first record (a negative mass, which no sum of
    // exponentials gives), and the finishing kernel writes -inf for the side.
    if (lane == 0 && s0 < s1) rec[s0] = SegRec{-INFINITY, -1.0f};
    return;
  }
  const bool mass = topp && !topk;
  const float c = scale_of(T);
  const E* row = reinterpret_cast<const E*>(side == 0 ? in.target : in.draft) + (int64_t)r * in.V;
  using CH = Chunk<E, VEC>;
  constexpr int U = 2 / SV;  // segments per step (two vectors per lane), two steps in flight
  auto vec_of = [&](int sg, int v) __attribute__((always_inline)) { return (sg * SV + v) * kWave + lane; };
  auto load = [&](CH (&x)[U][SV], int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u)  // past the wave's last segment: that segment again (a cache hit)
#pragma unroll
      for (int v = 0; v < SV; ++v) x[u][v].load_nt(row + (int64_t)min(vec_of(min(sb + u, s1 - 1), v), nvec - 1) * VEC);
  };
  auto fold = [&](const CH (&x)[U][SV], int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sg = sb + u;
      if (sg >= s1) break;  // wave-uniform
      float vm = -INFINITY;
      int bad = 0;
#pragma unroll
      for (int v = 0; v < SV; ++v) {
        if (vec_of(sg, v) < nvec) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float y = x[u][v].get(e);
            vm = fmaxf(vm, y);
            bad |= (int)(__builtin_isnan(y) || y == INFINITY);
          }
        }
      }
      const float sm = wave_max(bad ? INFINITY : vm);  // +inf marks an invalid segment
      float ms = 0.0f;
      if (mass && sm > -INFINITY && sm < INFINITY) {
#pragma unroll
        for (int v = 0; v < SV; ++v) {
          if (vec_of(sg, v) < nvec) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) ms += fast_exp2((x[u][v].get(e) - sm) * c);
          }
        }
        ms = wave_sum(ms);
      }
      if (lane == 0) rec[sg] = SegRec{sm, ms};
    }
  };
  CH xa[U][SV], xb[U][SV];
  if (s0 < s1) load(xa, s0);
  for (int sb = s0; sb < s1; sb += 2 * U) {
    load(xb, sb + U);
    fold(xa, sb);
    load(xa, sb + 2 * U);
    fold(xb, sb + U);
  }
}

// Order one wave's LDS writes before its later LDS reads by other lanes: the LDS serves a
// wave's operations in issue order, so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kRecordWaves = 8192;   // seg_records_kernel's target grid, in waves
constexpr int kFinWaves = kFiltWaves;  // waves per row and side in thresholds_finish_kernel
constexpr int kFinCap = 256;           // candidates a row and side keeps
constexpr int kFinVecs = 8;            // 16-byte vectors per lane one gather step loads
constexpr int kFinStage = 4;           // of which the LDS stage holds this many at a time

// Largest v in [lo, hi] with pred(v), pred monotone (true below some point, false above) and
// true at lo, found by bisection over order_key(v) / 2^S: with bf16 data (S = 16) every probe
// lies just below or on a bf16 value, so {x >= v} over the data is decided in 16 steps.
template <int S, class P>
__device__ __forceinline__ float bisect_key(float lo, float hi, P pred) {
  if (pred(hi)) return hi;
  int64_t a = (int64_t)(order_key(lo) >> S), z = (int64_t)(order_key(hi) >> S) + 1;
  while (z - a > 1) {
    const int64_t mid = a + (z - a) / 2;
    if (pred(key_float((int32_t)(mid * ((int64_t)1 << S))))) a = mid;
    else z = mid;
  }
  return key_float((int32_t)(a * ((int64_t)1 << S)));
}

template <typename E, int VEC>
struct FinSmem {
  int list[kSegCap];                                 // the segments to gather, in row order
  Chunk<E, VEC> stage[kFinWaves][kFinStage][kWave];  // each lane's staged vectors
  float cand[kFinWaves][kFinCap];                    // each wave's candidates, in gather order
  float all[kFinCap];                                // all of them, wave 0's first
  double e[kFinCap];                                 // masses exp((x - m) / T), 0 below the base
  int cnt[kFinWaves];
  double rest[kFinWaves];
  float th, lo, m, s;
  int ns, mode, back;
};

// One workgroup of kFiltBlock threads per row and side (grid 2R). It runs once per row and
// side, latency-bound, so the code keeps to short loops. Every wave keeps the records of
// segments lane, lane + 64, ... in registers and takes the same decisions up to the gather;
// the gather splits the listed segments over the waves (loads staged through LDS); wave 0
// then decides the thresholds alone. Selections by value are bisections over the float order
// (bisect_key) whose steps count with ballots: the k-th largest value is the largest v that
// at least k values reach. top-p's threshold is the largest candidate x whose candidates >= x
// hold at least top_p times S1: every lane sums, for its own candidates, the masses of all
// candidates at or above them. A row and side that the records cannot decide (top-k beyond
// the segment count, more than kFinCap candidates, candidates short of top_p) is decided by
// the whole workgroup as thresholds_kernel does, in the same LDS.
template <typename E, int VEC>
__global__ __launch_bounds__(kFiltBlock) __attribute__((amdgpu_waves_per_eu(6))) void thresholds_finish_kernel(Inputs in, FilterArgs fa) {
  using CH = Chunk<E, VEC>;
  constexpr int RS = kSegCap / kWave;  // record slots per lane
  constexpr int KS = sizeof(E) == 2 ? 16 : 0;  // bisection granularity: bf16 values
  constexpr int SV = kSegLogits / (kWave * VEC);
  constexpr int NS = kFinVecs / SV;  // listed segments per wave and gather step
  __shared__ union {
    FinSmem<E, VEC> f;
    FilterSmem x;
  } u;
  FinSmem<E, VEC>& F = u.f;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rs = blockIdx.x, r = rs >> 1, side = rs & 1;
  float* out = fa.theta + rs;  // theta is [R][2]
  const int b = uni(request_of_row(in, r));
  const float T = in.temp[b];
  const FilterParams fp = filter_params(fa.side[side], b);
  const bool topk = fp.k > 0 && fp.k < in.V, topp = fp.top_p < 1.0f, minp = fp.min_p > 0.0f;
  const E* row = reinterpret_cast<const E*>(side == 0 ? in.target : in.draft) + (int64_t)r * in.V;
  // The row's drafted token and its logit, for the statistics pass 1 may take from here: their
  // loads are issued now and waited for at the end.
  int Dv = -1;
  float lD = 0.0f;
  if (fa.fstat != nullptr && threadIdx.x == 0) {
    Dv = in.dt[r];
    if ((unsigned)Dv < (unsigned)in.V) lD = to_float(row[Dv]);
  }
  auto done = [&](float th) __attribute__((always_inline)) {
    if (threadIdx.x == 0) {
      *out = th;
      if (fa.fstat != nullptr) fa.fstat[rs] = FiltStat{0.0f, 0.0f, 0.0f, 0};
    }
  };
  if (!(T > 0.0f) || !temperature_ok(T) || !filter_valid(fp) || !(topk || topp || minp)) {
    done(-INFINITY);
    return;
  }
  const int nseg = fa.nseg;
  float hint = -INFINITY;  // the exact path's candidate bound with top-p alone
  if (!(topk && fp.k > nseg)) {  // else the exact path below
  const bool rest_on = topp && !topk;  // top-p alone: S1 is the whole row's mass
  const double Td = (double)T;
  const float c = scale_of(T);
  float th_m = -INFINITY;  // min-p's threshold (wave 0's)
  double tl = 0.0;         // with top-p alone, this wave's share of the mass outside the candidates
  // Wave 0 alone reads the records and decides up to the list of segments to gather; the other
  // waves wait. mode 0: the threshold is decided (th); 1: gather the logits >= lo.
  if (wave == 0) {
    const SegRec* rec = fa.seg + (int64_t)rs * nseg;
    float smax[RS], smass[RS];
    float mx = -INFINITY;
    int bad = 0, unread = 0;
#pragma unroll
    for (int t = 0; t < RS; ++t) {
      smax[t] = -INFINITY;
      smass[t] = 0.0f;
      if (t * kWave + lane < nseg) {
        const SegRec q = rec[t * kWave + lane];
        smax[t] = q.max;
        smass[t] = q.mass;
      }
      bad |= (int)!(smax[t] < INFINITY);
      unread |= (int)(smass[t] < 0.0f);
      mx = fmaxf(mx, smax[t]);
    }
    const float m = wave_max(mx);
    int mode = 1, ns = 0;
    float th = 0.0f, lo = 0.0f;
    if (fa.skip_unused && wave_or(unread) != 0) {
      mode = 0;  // a side the verify never reads, which the record kernel did not stream
      th = -INFINITY;
    } else if (wave_or(bad) != 0 || m == -INFINITY) {
      mode = 0;
      th = INFINITY;
    } else {
      // min-p: the smallest float y with (y - m) / T >= ln(min_p), in fp64 (as
      // thresholds_kernel).
      if (minp) {
        const double lm = log((double)fp.min_p);
        auto keep = [&](float y) { return ((double)y - (double)m) / Td >= lm; };
        float y = (float)((double)m + Td * lm);
        for (int it = 0; it < 64 && !keep(y); ++it) y = nextafterf(y, INFINITY);
        for (int it = 0; it < 64 && keep(nextafterf(y, -INFINITY)); ++it) y = nextafterf(y, -INFINITY);
        th_m = y;
      }
      if (!topk && !topp) {
        mode = 0;
        th = th_m;
      } else {
        // The candidate bound lo: every logit at or above the threshold to find reaches it.
        //  - top-k: the k-th largest segment maximum (k segments hold a logit that reaches it).
        //  - top-p alone: start from the window bound (as thresholds_kernel), then raise it to
        //    the largest v at which the records still prove that the logits >= v hold top_p of
        //    the row's mass: those in segments whose maximum reaches v hold at least their
        //    segments' mass less kSegLogits * exp((v - m) / T) per segment. The records'
        //    masses are fp32 sums, so the proof keeps a margin of 2e-4 of the row's mass; the
        //    top-p search below still checks that the candidates reach top_p.
        if (topk) {
          lo = bisect_key<KS>(-INFINITY, m, [&](float v) {
            int n = 0;
#pragma unroll
            for (int t = 0; t < RS; ++t) n += (int)__popcll(__ballot(!(smax[t] < v)));
            return n >= fp.k;
          });
        } else {
          // From here on smass holds each segment's mass relative to m.
          double S = 0.0;
#pragma unroll
          for (int t = 0; t < RS; ++t) {
            smass[t] = smax[t] > -INFINITY ? smass[t] * fast_exp2((smax[t] - m) * c) : 0.0f;
            S += (double)smass[t];
          }
          S = wave_sum(S);
          const float W = log2f((float)in.V / (1.0f - fp.top_p)) + 1.0f;
          const double need = (double)fp.top_p * S + 2e-4 * S;
          lo = bisect_key<KS>(m - (W + 0.01f) / c, m, [&](float v) {
            float h = 0.0f;
            int n = 0;
#pragma unroll
            for (int t = 0; t < RS; ++t) {
              const bool on = !(smax[t] < v);
              h += on ? smass[t] : 0.0f;
              n += (int)__popcll(__ballot(on));
            }
            const double held = (double)wave_sum(h);
            return held - (double)n * (double)kSegLogits * exp(((double)v - (double)m) / Td) >= need;
          });
        }
        // The segments that can hold candidates, in row order; with top-p alone the others'
        // mass.
#pragma unroll
        for (int t = 0; t < RS; ++t) {
          const bool real = t * kWave + lane < nseg;
          const bool take = real && !(smax[t] < lo);
          if (rest_on && real && !take) tl += (double)smass[t];
          const uint64_t mk = __ballot(take);
          if (take) F.list[ns + lane_rank(mk)] = t * kWave + lane;
          ns += (int)__popcll(mk);
        }
      }
    }
    if (lane == 0) {
      F.mode = mode;
      F.th = th;
      F.lo = lo;
      F.m = m;
      F.ns = ns;
    }
  }
  __syncthreads();
  if (F.mode == 0) {
    done(F.th);
    return;
  }
  const float lo = F.lo, m = F.m;
  const int ns = F.ns;
  // Gather the logits >= lo: wave w takes listed segments w, w + kFinWaves, ..., NS at a
  // time, kFinVecs vectors per lane loaded at once and worked through the LDS stage
  // kFinStage at a time. A vector whose lanes hold at most one candidate each stores each
  // lane's largest logit at the lane's rank; otherwise one ballot per element.
  const int nvec = in.V / VEC;
  float* cand = F.cand[wave];
  auto vec_of = [&](int i0, int q) __attribute__((always_inline)) {
    const int i = i0 + (q / SV) * kFinWaves;
    return i < ns ? (F.list[i] * SV + q % SV) * kWave + lane : nvec;
  };
  int nc = 0;
  uint32_t okbits = 0;  // bit q: this lane's vector q of the step lies inside the row
  auto work = [&](int q0, int nq) __attribute__((always_inline)) {
#pragma unroll 1
    for (int q = 0; q < nq; ++q) {
      const CH x = F.stage[wave][q][lane];
      const bool ok = (okbits >> (q0 + q)) & 1u;
      // The vector's largest and second largest logit: a lane holds two candidates or more
      // iff the second reaches lo.
      float a = -INFINITY, a2 = -INFINITY, ts = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = x.get(e);
        a2 = __builtin_amdgcn_fmed3f(a, a2, v);
        a = fmaxf(a, v);
        if (rest_on && ok && v < lo) ts += fast_exp2((v - m) * c);
      }
      if (rest_on) tl += (double)ts;
      const uint64_t any = __ballot(ok && !(a < lo));
      if (any == 0) continue;  // the same for every lane
      if (__ballot(ok && !(a2 < lo)) == 0) {
        if (ok && !(a < lo)) {
          const int pos = nc + lane_rank(any);
          if (pos < kFinCap) cand[pos] = a;
        }
        nc += (int)__popcll(any);
      } else {
#pragma unroll 1
        for (int e = 0; e < VEC; ++e) {
          const float v = x.get_dyn(e);
          const bool cnd = ok && !(v < lo);
          const uint64_t mk = __ballot(cnd);
          if (cnd) {
            const int pos = nc + lane_rank(mk);
            if (pos < kFinCap) cand[pos] = v;
          }
          nc += (int)__popcll(mk);
        }
      }
    }
  };
  static_assert(kFinVecs == 2 * kFinStage, "two stage fills per step");
  for (int i0 = wave; i0 < ns; i0 += NS * kFinWaves) {
    CH x[kFinVecs];
    okbits = 0;
#pragma unroll
    for (int q = 0; q < kFinVecs; ++q) {
      const int vi = vec_of(i0, q);
      okbits |= (uint32_t)(vi < nvec) << q;
      x[q].load(row + (int64_t)min(vi, nvec - 1) * VEC);
    }
    const int nv = min(NS, (ns - i0 + kFinWaves - 1) / kFinWaves) * SV;  // vectors of this step
#pragma unroll
    for (int q = 0; q < kFinStage; ++q) F.stage[wave][q][lane] = x[q];  // each lane reads back its own
    work(0, min(nv, kFinStage));
    if (nv > kFinStage) {
#pragma unroll
      for (int q = 0; q < kFinStage; ++q) F.stage[wave][q][lane] = x[kFinStage + q];
      work(kFinStage, nv - kFinStage);
    }
  }
  const double tw = wave_sum(tl);
  if (lane == 0) {
    F.cnt[wave] = nc;
    F.rest[wave] = tw;
  }
  __syncthreads();
  if (wave == 0) {
    // Wave 0: the candidates of all waves in wave order, the rest of the row's mass, then the
    // thresholds; back = 1 hands the row to the exact path below.
    int back = 1;
    float th = 0.0f;
    do {
      int n = 0;
      double rest = 0.0;
      for (int w = 0; w < kFinWaves; ++w) {
        const int cw = F.cnt[w];
        for (int j = lane; j < cw; j += kWave)
          if (n + j < kFinCap) F.all[n + j] = F.cand[w][j];
        n += cw;
        rest += F.rest[w];
      }
      if (n > kFinCap) break;
      wave_lds_sync();
      const int nt = (n + kWave - 1) / kWave;  // candidate slots per lane: j = t * 64 + lane
      // top-k: the k-th largest candidate (at least k candidates reach lo), as a candidate's
      // value.
      float th_k = -INFINITY;
      if (topk) {
        if (n < fp.k) break;
        const float v = bisect_key<KS>(lo, m, [&](float v) {
          int cnt = 0;
          for (int t = 0; t < nt; ++t) {
            const int j = t * kWave + lane;
            cnt += (int)__popcll(__ballot(j < n && !(F.all[j] < v)));
          }
          return cnt >= fp.k;
        });
        float lowest = INFINITY;
        for (int j = lane; j < n; j += kWave) lowest = !(F.all[j] < v) ? fminf(lowest, F.all[j]) : lowest;
        th_k = -wave_max(-lowest);
      }
      // top-p over top-k's set (the candidates >= th_k; all of them with top-p alone), S1
      // being the set's fp64 mass plus, with top-p alone, the rest of the row's.
      float th_p = -INFINITY;
      if (topp) {
        const float base = topk ? th_k : lo;
        double own = 0.0;
        for (int j = lane; j < n; j += kWave) {
          const double e = !(F.all[j] < base) ? exp(((double)F.all[j] - (double)m) / Td) : 0.0;
          F.e[j] = e;
          own += e;
        }
        const double target = (double)fp.top_p * (wave_sum(own) + (topk ? 0.0 : rest));
        wave_lds_sync();
        float best = -INFINITY;
        for (int t = 0; t < nt; t += 2) {
          const int i0 = t * kWave + lane, i1 = i0 + kWave;
          const float x0 = i0 < n ? F.all[i0] : INFINITY, x1 = i1 < n ? F.all[i1] : INFINITY;
          double h0 = 0.0, h1 = 0.0;
#pragma unroll 4
          for (int j = 0; j < n; ++j) {
            const float xj = F.all[j];
            const double ej = F.e[j];
            h0 += !(xj < x0) ? ej : 0.0;
            h1 += !(xj < x1) ? ej : 0.0;
          }
          if (i0 < n && !(x0 < base) && h0 >= target) best = fmaxf(best, x0);
          if (i1 < n && !(x1 < base) && h1 >= target) best = fmaxf(best, x1);
        }
        th_p = wave_max(best);
        if (th_p == -INFINITY) break;  // the candidates hold less than top_p of S1
      }
      th = fmaxf(fmaxf(th_k, th_p), th_m);
      back = 0;
      // The masked sum pass 1 would take over the row: every kept logit is a candidate.
      const float mc = ref_of(m, c);
      float acc = 0.0f;
      for (int j = lane; j < n; j += kWave) {
        const float x = F.all[j];
        if (!(x < th)) acc += fast_exp2(fmaf(x, c, -mc));
      }
      F.s = wave_sum(acc);
    } while (false);
    if (lane == 0) {
      F.th = th;
      F.back = back;
    }
  }
  __syncthreads();
  if (F.back == 0) {
    if (threadIdx.x == 0) {
      *out = F.th;
      if (fa.fstat != nullptr)
        fa.fstat[rs] = FiltStat{m, F.s, lD, (unsigned)Dv < (unsigned)in.V ? 1 : 0};
    }
    return;
  }
  if (rest_on) hint = lo;
  __syncthreads();  // the exact path reuses the LDS
  }
  if (threadIdx.x == 0 && fa.fstat != nullptr) fa.fstat[rs] = FiltStat{0.0f, 0.0f, 0.0f, 0};
  thresholds_row<E, VEC>(in, fa, r, side, u.x, hint);
}

// ====================================================================== launch

// Zero the request tickets. Every ticket wraps back to zero when a call completes, so this
// runs only when a workspace is first seen or its layout changes (see counters_ready).
__global__ __launch_bounds__(kBlock) void clear_counters_kernel(uint32_t* t, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) t[i] = 0u;
}

// Per (device, workspace address): the counter layout of the last call enqueued on it.
struct LayoutSeen {
  int device;
  const void* ws;
  size_t off_ticket2, off_trans;  // the counters' extent
};

static std::mutex g_layout_mu;
static LayoutSeen g_layout[64];
static int g_layout_n = 0;

// Make sure the workspace's ticket arrays hold zeros before pass 1 runs: clear them when
// this (device, workspace) pair was not seen with this layout by the previous call.
static hipError_t counters_ready(const Plan& p, char* ws, hipStream_t stream) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_layout_mu);
  int slot = -1;
  for (int i = 0; i < g_layout_n; ++i)
    if (g_layout[i].device == dev && g_layout[i].ws == ws) slot = i;
  if (slot >= 0 && g_layout[slot].off_ticket2 == p.off_ticket2 && g_layout[slot].off_trans == p.off_trans)
    return hipSuccess;
  const int64_t n = (int64_t)(p.off_trans - p.off_ticket2) / 4;
  const int64_t blocks = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(kBlock), 0,
                     stream, reinterpret_cast<uint32_t*>(ws + p.off_ticket2), n);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (slot < 0) slot = g_layout_n < 64 ? g_layout_n++ : (int)(reinterpret_cast<uintptr_t>(ws) / 256 % 64);
  g_layout[slot] = LayoutSeen{dev, ws, p.off_ticket2, p.off_trans};
  return hipSuccess;
}

// Waves a kernel should run on a device: the target per compute unit, or fewer if fewer
// fit (compute units times the kernel's workgroups per unit times four waves). Queried
// once per (device, kernel).
struct SlotsSeen {
  int device;
  const void* fn;
  int64_t slots;
};

static std::mutex g_slots_mu;
static SlotsSeen g_slots[64];
static int g_slots_n = 0;

static hipError_t resident_waves(const void* fn, int per_cu_target, int64_t* slots) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_slots_mu);
  for (int i = 0; i < g_slots_n; ++i)
    if (g_slots[i].device == dev && g_slots[i].fn == fn) {
      *slots = g_slots[i].slots;
      return hipSuccess;
    }
  int cus = 0, per_cu = 0;
  if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return err;
  if ((err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kBlock, 0)) != hipSuccess) return err;
  const int64_t fit = (int64_t)(per_cu > 0 ? per_cu : 1) * kWavesPerBlock;
  const int64_t s = (int64_t)(cus > 0 ? cus : 1) * (fit < per_cu_target ? fit : per_cu_target);
  if (g_slots_n < 64) g_slots[g_slots_n++] = SlotsSeen{dev, fn, s};
  *slots = s;
  return hipSuccess;
}

// The filtered verify's first kernel: every row's keep-thresholds, one workgroup per row
// and side.
template <typename E, int VEC>
hipError_t launch_thresholds(const Plan& p, const Inputs& in, FilterArgs fa, hipStream_t stream, char* ws) {
  if constexpr (VEC > 1) {
    if (p.nseg > 0 && ws != nullptr) {
      fa.seg = reinterpret_cast<SegRec*>(ws + p.off_seg);
      fa.nseg = p.nseg;
      // Waves per row and side: about 32 per compute unit in all, each streaming at least 16
      // segments (16 KB of bf16).
      const int64_t want = (kRecordWaves + 2 * (int64_t)p.R - 1) / (2 * (int64_t)p.R);
      const int64_t most = p.nseg / 16 < 1 ? 1 : p.nseg / 16;
      const int nw = (int)(want < 1 ? 1 : want > most ? most : want);
      const int64_t blocks1 = ((int64_t)p.R * 2 * nw + kWavesPerBlock - 1) / kWavesPerBlock;
      hipLaunchKernelGGL((seg_records_kernel<E, VEC>), dim3((unsigned)blocks1), dim3(kBlock), 0, stream, in, fa, nw);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL((thresholds_finish_kernel<E, VEC>), dim3((unsigned)(2 * p.R)), dim3(kFiltBlock), 0, stream,
                         in, fa);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((thresholds_kernel<E, VEC>), dim3((unsigned)(2 * p.R)), dim3(kFiltBlock), 0, stream, in, fa);
  return hipGetLastError();
}

constexpr int kSentSpread = 4;  // pass-1 wave multiplier when the filter chain leaves row statistics
constexpr int kSentWaves = 16;  // and the fewest pass-1 waves per row then

template <typename E, int VEC, bool FILT = false>
hipError_t launch_pair(const Plan& p, Inputs in, const Work& w, const Outputs& out, hipStream_t stream,
                       hipEvent_t const* ev) {
  constexpr int U1 = VEC == 1 ? 8 : 2;  // pass 1: chunks per lane per array and step (x2 buffers)
  constexpr int U2 = VEC == 1 ? 8 : 2;  // pass 2: the same
  const void* k1 = reinterpret_cast<const void*>(&pass1_kernel<E, VEC, U1, FILT>);
  const bool diag = out.diag != nullptr || in.tau_step != nullptr || in.min_cum != nullptr;
  const void* k2 = diag ? reinterpret_cast<const void*>(&pass2_kernel<E, VEC, U2, true, FILT>)
                        : reinterpret_cast<const void*>(&pass2_kernel<E, VEC, U2, false, FILT>);
  int64_t slots1 = 0, slots2 = 0;
  hipError_t err = resident_waves(k1, kTargetWavesPerCU, &slots1);
  if (err != hipSuccess) return err;
  if ((err = resident_waves(k2, kTargetWavesPerCU2, &slots2)) != hipSuccess) return err;
  // When the filter chain leaves most rows' statistics, pass 1 streams only the rest: four
  // times as many waves per row keeps their spans short.
  if (FILT && in.fstat != nullptr) slots1 *= kSentSpread;
  Launch l = pick_waves(p, slots1, slots2);
  // A batch of many rows would still give each row few waves, and the waves of the rows left
  // to stream would then take long spans: keep at least kSentWaves per row (unless a tuning
  // override sets the split).
  if (FILT && in.fstat != nullptr && tuning().w1 <= 0 && l.w1 < kSentWaves) {
    int w1 = l.w1;
    while (w1 * 2 <= kSentWaves && w1 * 2 <= p.w1max) w1 *= 2;
    const int64_t rows = p.R - p.B;
    l.w1 = w1;
    l.blocks1 = (rows * w1 + kWavesPerBlock - 1) / kWavesPerBlock;
    if (l.blocks1 < 1) l.blocks1 = 1;
  }
  in.w1 = l.w1;
  in.w2 = l.w2;
  if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
  const dim3 block(kBlock);
  hipLaunchKernelGGL((pass1_kernel<E, VEC, U1, FILT>), dim3((unsigned)l.blocks1), block, 0, stream, in, w, out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
  if (diag)
    hipLaunchKernelGGL((pass2_kernel<E, VEC, U2, true, FILT>), dim3((unsigned)l.blocks2), block, 0, stream, in, w,
                       out);
  else
    hipLaunchKernelGGL((pass2_kernel<E, VEC, U2, false, FILT>), dim3((unsigned)l.blocks2), block, 0, stream, in, w,
                       out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev && (err = hipEventRecord(ev[2], stream)) != hipSuccess) return err;
  return hipSuccess;
}

template <typename E, int VEC>
hipError_t launch_lazy(const Plan& p, Inputs in, const Work& w, const Outputs& out, hipStream_t stream,
                       int max_rows) {
  constexpr int U1 = VEC == 1 ? 8 : 2;
  constexpr int U2 = VEC == 1 ? 8 : 2;
  // As many waves per row as a row allows (a power of two): launch j streams few rows.
  int nw = 1;
  while (nw * 2 <= p.w1max) nw *= 2;
  const void* k2 = reinterpret_cast<const void*>(&pass2_kernel<E, VEC, U2, false>);
  int64_t slots2 = 0;
  hipError_t err = resident_waves(k2, kTargetWavesPerCU2, &slots2);
  if (err != hipSuccess) return err;
  const Launch l = pick_waves(p, slots2, slots2);
  in.w1 = nw;
  in.w2 = l.w2;
  const dim3 block(kBlock);
  const int64_t blocks = ((int64_t)p.B * nw + kWavesPerBlock - 1) / kWavesPerBlock;
  const int steps = max_rows > 1 ? max_rows - 1 : 1;  // launch 0 also checks the batch
  for (int j = 0; j < steps; ++j) {
    hipLaunchKernelGGL((lazy_rows_kernel<E, VEC, U1>), dim3((unsigned)blocks), block, 0, stream, in, w, j, max_rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL((pass2_kernel<E, VEC, U2, false>), dim3((unsigned)l.blocks2), block, 0, stream, in, w, out);
  return hipGetLastError();
}

template <typename E, int VEC, bool FILT = false>
hipError_t launch_sums(const Plan& p, Inputs in, const Work& w, float* out_min, float* out_pq, hipStream_t stream) {
  constexpr int U1 = VEC == 1 ? 8 : 2;
  const void* k1 = reinterpret_cast<const void*>(&pass1_kernel<E, VEC, U1, FILT>);
  int64_t slots1 = 0;
  hipError_t err = resident_waves(k1, kTargetWavesPerCU, &slots1);
  if (err != hipSuccess) return err;
  const Launch l = pick_waves(p, slots1, slots1);
  in.w1 = l.w1;
  in.w2 = l.w2;
  const Outputs none{nullptr, nullptr, nullptr, nullptr};
  const dim3 block(kBlock);
  hipLaunchKernelGGL((pass1_kernel<E, VEC, U1, FILT>), dim3((unsigned)l.blocks1), block, 0, stream, in, w, none);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((sums_kernel<E, VEC, U1, FILT>), dim3((unsigned)l.blocks1), block, 0, stream, in, w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t mb = ((int64_t)p.R + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(merge_sums_kernel, dim3((unsigned)(mb < 1024 ? mb : 1024)), block, 0, stream, in, w, out_min,
                     out_pq);
  return hipGetLastError();
}

template <typename E, int VEC>
hipError_t launch_match(const Plan& p, Inputs in, const Work& w, const Outputs& out, hipStream_t stream) {
  constexpr int U = VEC == 1 ? 8 : 2;
  const void* k = reinterpret_cast<const void*>(&match_rows_kernel<E, VEC, U>);
  int64_t slots = 0;
  hipError_t err = resident_waves(k, kTargetWavesPerCU2, &slots);
  if (err != hipSuccess) return err;
  // Waves per row: a power of two, so that the emit kernel merges rows in aligned lane groups.
  const int64_t want = slots / (p.R > 0 ? p.R : 1);
  int nw = 1;
  while (nw * 2 <= want && nw * 2 <= p.w1max) nw *= 2;
  MatchPart* parts = reinterpret_cast<MatchPart*>(reinterpret_cast<char*>(w.part1));
  const dim3 block(kBlock);
  const int64_t blocks1 = ((int64_t)p.R * nw + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((match_rows_kernel<E, VEC, U>), dim3((unsigned)blocks1), block, 0, stream, in, w, parts, nw);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t blocks2 = ((int64_t)p.B + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(match_emit_kernel, dim3((unsigned)blocks2), block, 0, stream, in, w, parts, nw, out);
  return hipGetLastError();
}

static FilterSide side_of(const sv_filter* f) {
  return f ? FilterSide{f->top_k, f->top_p, f->min_p} : FilterSide{nullptr, nullptr, nullptr};
}

static bool any_filter(const FilterSide& f) { return f.top_k || f.top_p || f.min_p; }

static sv_status run(const void* target, const void* draft, const int32_t* draft_tokens,
                     const int32_t* row_offsets, const float* temperature, const float* tau,
                     const float* tau_step, const float* min_cum,
                     uint64_t seed, int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                     void* workspace, size_t workspace_bytes, void* hip_stream,
                     sv_row_diag* diag, sv_batch_stats* stats, void* const* events,
                     const sv_filter* tfilt = nullptr, const sv_filter* dfilt = nullptr) {
  Plan p;
  const sv_status st = check_call(shape, target, draft, draft_tokens, row_offsets, temperature, tau,
                                  out_tokens, out_accept_len, workspace, workspace_bytes, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  char* ws = static_cast<char*>(workspace);
  Inputs in{target, draft, draft_tokens, row_offsets, temperature, tau, tau_step, min_cum,
            seed, p.B, p.R, p.V, p.dtype, 1, 1};
  Work w{reinterpret_cast<WsHeader*>(ws + p.off_hdr), reinterpret_cast<P1Part*>(ws + p.off_part1),
         reinterpret_cast<P2Part*>(ws + p.off_part2), reinterpret_cast<uint32_t*>(ws + p.off_ticket2),
         reinterpret_cast<SumPart*>(ws + p.off_part3), reinterpret_cast<uint32_t*>(ws + p.off_done3),
         reinterpret_cast<int32_t*>(ws + p.off_lazy), reinterpret_cast<uint64_t*>(ws + p.off_bmax)};
  Outputs out{out_tokens, out_accept_len, diag, stats};
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
  // 16-byte loads need 16-byte aligned rows: V * element size a multiple of 16 and aligned bases.
  const bool aligned = ((int64_t)p.V * p.esize) % 16 == 0 &&
                       (reinterpret_cast<uintptr_t>(target) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(draft) % 16) == 0;
  hipError_t err = counters_ready(p, ws, stream);
  if (err != hipSuccess) return SV_E_HIP;
  const FilterSide ft = side_of(tfilt), fd = side_of(dfilt);
  if (any_filter(ft) || any_filter(fd)) {
    in.theta = reinterpret_cast<float*>(ws + p.off_theta);
    in.filt[0] = ft;
    in.filt[1] = fd;
    FilterArgs fa{{ft, fd}, reinterpret_cast<float*>(ws + p.off_theta)};
    // With segment records the chain leaves the statistics of the rows it decided, and pass 1
    // takes them instead of streaming those rows; the chain skips the row sides the verify
    // never reads.
    if (aligned && p.nseg > 0) {
      fa.fstat = reinterpret_cast<FiltStat*>(ws + p.off_fstat);
      in.fstat = fa.fstat;
      fa.skip_unused = 1;
    }
    if (p.dtype == SV_BF16) {
      err = aligned ? launch_thresholds<uint16_t, 8>(p, in, fa, stream, ws) : launch_thresholds<uint16_t, 1>(p, in, fa, stream, ws);
      if (err == hipSuccess)
        err = aligned ? launch_pair<uint16_t, 8, true>(p, in, w, out, stream, ev)
                      : launch_pair<uint16_t, 1, true>(p, in, w, out, stream, ev);
    } else {
      err = aligned ? launch_thresholds<float, 4>(p, in, fa, stream, ws) : launch_thresholds<float, 1>(p, in, fa, stream, ws);
      if (err == hipSuccess)
        err = aligned ? launch_pair<float, 4, true>(p, in, w, out, stream, ev)
                      : launch_pair<float, 1, true>(p, in, w, out, stream, ev);
    }
    return err == hipSuccess ? SV_OK : SV_E_HIP;
  }
  if (p.dtype == SV_BF16) {
    err = aligned ? launch_pair<uint16_t, 8>(p, in, w, out, stream, ev)
                  : launch_pair<uint16_t, 1>(p, in, w, out, stream, ev);
  } else {
    err = aligned ? launch_pair<float, 4>(p, in, w, out, stream, ev)
                  : launch_pair<float, 1>(p, in, w, out, stream, ev);
  }
  return err == hipSuccess ? SV_OK : SV_E_HIP;
}

// The allocation-free verify's workspace: one array per GPU in the code object, so no call
// allocates. Host code never passes `scratch` itself to a kernel (on the host it only names
// the symbol); it uses the device address that hipGetSymbolAddress returns for the current
// device, kept per device.
static __device__ __align__(256) unsigned char scratch[SV_STATIC_WORKSPACE_BYTES];

struct ScratchSeen {
  int device;
  void* ptr;
};

static std::mutex g_scratch_mu;
static ScratchSeen g_scratch[64];
static int g_scratch_n = 0;

static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (int i = 0; i < g_scratch_n; ++i)
    if (g_scratch[i].device == dev) {
      *out = g_scratch[i].ptr;
      return hipSuccess;
    }
  if (g_scratch_n >= 64) return hipErrorInvalidDevice;
  void* ptr = nullptr;
  if ((err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return err;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  g_scratch[g_scratch_n++] = ScratchSeen{dev, ptr};
  *out = ptr;
  return hipSuccess;
}

}  // namespace sv

extern "C" sv_status sv_verify_batch(const void* target_logits, const void* draft_logits,
                                     const int32_t* draft_tokens, const int32_t* row_offsets,
                                     const float* temperature, const float* tau, uint64_t seed,
                                     int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                                     void* workspace, size_t workspace_bytes, void* hip_stream) {
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, nullptr, nullptr,
                 seed, out_tokens, out_accept_len, shape, workspace, workspace_bytes, hip_stream,
                 nullptr, nullptr, nullptr);
}

extern "C" sv_status sv_verify_batch_diag(const void* target_logits, const void* draft_logits,
                                          const int32_t* draft_tokens, const int32_t* row_offsets,
                                          const float* temperature, const float* tau, uint64_t seed,
                                          int32_t* out_tokens, int32_t* out_accept_len,
                                          sv_shape shape, void* workspace, size_t workspace_bytes,
                                          void* hip_stream, sv_row_diag* out_row_diag,
                                          sv_batch_stats* out_stats, void* const* hip_events) {
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, nullptr, nullptr,
                 seed, out_tokens, out_accept_len, shape, workspace, workspace_bytes, hip_stream,
                 out_row_diag, out_stats, hip_events);
}

extern "C" sv_status sv_verify_batch_lazy(const void* target_logits, const void* draft_logits,
                                          const int32_t* draft_tokens, const int32_t* row_offsets,
                                          const float* temperature, const float* tau, uint64_t seed,
                                          int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                                          void* workspace, size_t workspace_bytes, void* hip_stream,
                                          int32_t max_rows) {
  using namespace sv;
  Plan p;
  const sv_status st = check_call(shape, target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau,
                                  out_tokens, out_accept_len, workspace, workspace_bytes, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  if (max_rows < 1 || max_rows > 4096) return SV_E_SHAPE;
  char* ws = static_cast<char*>(workspace);
  Inputs in{target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, nullptr, nullptr,
            seed, p.B, p.R, p.V, p.dtype, 1, 1};
  Work w{reinterpret_cast<WsHeader*>(ws + p.off_hdr), reinterpret_cast<P1Part*>(ws + p.off_part1),
         reinterpret_cast<P2Part*>(ws + p.off_part2), reinterpret_cast<uint32_t*>(ws + p.off_ticket2),
         reinterpret_cast<SumPart*>(ws + p.off_part3), reinterpret_cast<uint32_t*>(ws + p.off_done3),
         reinterpret_cast<int32_t*>(ws + p.off_lazy), reinterpret_cast<uint64_t*>(ws + p.off_bmax)};
  Outputs out{out_tokens, out_accept_len, nullptr, nullptr};
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const bool aligned = ((int64_t)p.V * p.esize) % 16 == 0 && (reinterpret_cast<uintptr_t>(target_logits) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(draft_logits) % 16) == 0;
  hipError_t err = counters_ready(p, ws, stream);
  if (err != hipSuccess) return SV_E_HIP;
  if (p.dtype == SV_BF16) {
    err = aligned ? launch_lazy<uint16_t, 8>(p, in, w, out, stream, max_rows)
                  : launch_lazy<uint16_t, 1>(p, in, w, out, stream, max_rows);
  } else {
    err = aligned ? launch_lazy<float, 4>(p, in, w, out, stream, max_rows)
                  : launch_lazy<float, 1>(p, in, w, out, stream, max_rows);
  }
  return err == hipSuccess ? SV_OK : SV_E_HIP;
}

namespace sv {

static sv_status row_sums_run(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                              const int32_t* row_offsets, const float* temperature, const float* tau,
                              const float* tau_step, const float* min_cum, const sv_filter* tfilt,
                              const sv_filter* dfilt, float* out_sum_min, float* out_sum_pq, sv_shape shape,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  Plan p;
  const sv_status st = check_call(shape, target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau,
                                  out_sum_min, out_sum_pq, workspace, workspace_bytes, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  char* ws = static_cast<char*>(workspace);
  Inputs in{target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, tau_step, min_cum,
            0, p.B, p.R, p.V, p.dtype, 1, 1};
  Work w{reinterpret_cast<WsHeader*>(ws + p.off_hdr), reinterpret_cast<P1Part*>(ws + p.off_part1),
         reinterpret_cast<P2Part*>(ws + p.off_part2), reinterpret_cast<uint32_t*>(ws + p.off_ticket2),
         reinterpret_cast<SumPart*>(ws + p.off_part3), reinterpret_cast<uint32_t*>(ws + p.off_done3),
         reinterpret_cast<int32_t*>(ws + p.off_lazy), reinterpret_cast<uint64_t*>(ws + p.off_bmax)};
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const bool aligned = ((int64_t)p.V * p.esize) % 16 == 0 && (reinterpret_cast<uintptr_t>(target_logits) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(draft_logits) % 16) == 0;
  hipError_t err = counters_ready(p, ws, stream);
  if (err != hipSuccess) return SV_E_HIP;
  const FilterSide ft = side_of(tfilt), fd = side_of(dfilt);
  if (any_filter(ft) || any_filter(fd)) {
    in.theta = reinterpret_cast<float*>(ws + p.off_theta);
    in.filt[0] = ft;
    in.filt[1] = fd;
    FilterArgs fa{{ft, fd}, reinterpret_cast<float*>(ws + p.off_theta)};
    // With segment records the chain leaves the statistics of the rows it decided, and pass 1
    // takes them instead of streaming those rows. The sums read only proposal rows, so the
    // chain skips the row sides the verify never reads here too.
    if (aligned && p.nseg > 0) {
      fa.skip_unused = 1;
      fa.fstat = reinterpret_cast<FiltStat*>(ws + p.off_fstat);
      in.fstat = fa.fstat;
    }
    if (p.dtype == SV_BF16) {
      err = aligned ? launch_thresholds<uint16_t, 8>(p, in, fa, stream, ws) : launch_thresholds<uint16_t, 1>(p, in, fa, stream, ws);
      if (err == hipSuccess)
        err = aligned ? launch_sums<uint16_t, 8, true>(p, in, w, out_sum_min, out_sum_pq, stream)
                      : launch_sums<uint16_t, 1, true>(p, in, w, out_sum_min, out_sum_pq, stream);
    } else {
      err = aligned ? launch_thresholds<float, 4>(p, in, fa, stream, ws) : launch_thresholds<float, 1>(p, in, fa, stream, ws);
      if (err == hipSuccess)
        err = aligned ? launch_sums<float, 4, true>(p, in, w, out_sum_min, out_sum_pq, stream)
                      : launch_sums<float, 1, true>(p, in, w, out_sum_min, out_sum_pq, stream);
    }
    return err == hipSuccess ? SV_OK : SV_E_HIP;
  }
  if (p.dtype == SV_BF16) {
    err = aligned ? launch_sums<uint16_t, 8>(p, in, w, out_sum_min, out_sum_pq, stream)
                  : launch_sums<uint16_t, 1>(p, in, w, out_sum_min, out_sum_pq, stream);
  } else {
    err = aligned ? launch_sums<float, 4>(p, in, w, out_sum_min, out_sum_pq, stream)
                  : launch_sums<float, 1>(p, in, w, out_sum_min, out_sum_pq, stream);
  }
  return err == hipSuccess ? SV_OK : SV_E_HIP;
}

}  // namespace sv

extern "C" sv_status sv_row_acceptance(const void* target_logits, const void* draft_logits,
                                       const int32_t* draft_tokens, const int32_t* row_offsets,
                                       const float* temperature, const float* tau, const float* tau_step,
                                       const float* min_cum, float* out_sum_min, float* out_sum_pq, sv_shape shape,
                                       void* workspace, size_t workspace_bytes, void* hip_stream) {
  return sv::row_sums_run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, tau_step,
                          min_cum, nullptr, nullptr, out_sum_min, out_sum_pq, shape, workspace, workspace_bytes,
                          hip_stream);
}

extern "C" sv_status sv_row_acceptance_filtered(const void* target_logits, const void* draft_logits,
                                                const int32_t* draft_tokens, const int32_t* row_offsets,
                                                const float* temperature, const float* tau, const float* tau_step,
                                                const float* min_cum, const sv_filter* target_filter,
                                                const sv_filter* draft_filter, float* out_sum_min,
                                                float* out_sum_pq, sv_shape shape, void* workspace,
                                                size_t workspace_bytes, void* hip_stream) {
  return sv::row_sums_run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, tau_step,
                          min_cum, target_filter, draft_filter, out_sum_min, out_sum_pq, shape, workspace,
                          workspace_bytes, hip_stream);
}

extern "C" sv_status sv_verify_batch_sched(const void* target_logits, const void* draft_logits,
                                           const int32_t* draft_tokens, const int32_t* row_offsets,
                                           const float* temperature, const float* tau, const float* tau_step,
                                           const float* min_cum, uint64_t seed, int32_t* out_tokens,
                                           int32_t* out_accept_len, sv_shape shape, void* workspace,
                                           size_t workspace_bytes, void* hip_stream, sv_row_diag* out_row_diag,
                                           sv_batch_stats* out_stats) {
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, tau_step, min_cum,
                 seed, out_tokens, out_accept_len, shape, workspace, workspace_bytes, hip_stream,
                 out_row_diag, out_stats, nullptr);
}

extern "C" sv_status sv_verify_batch_filtered(const void* target_logits, const void* draft_logits,
                                              const int32_t* draft_tokens, const int32_t* row_offsets,
                                              const float* temperature, const float* tau, const float* tau_step,
                                              const float* min_cum, const sv_filter* target_filter,
                                              const sv_filter* draft_filter, uint64_t seed, int32_t* out_tokens,
                                              int32_t* out_accept_len, sv_shape shape, void* workspace,
                                              size_t workspace_bytes, void* hip_stream, sv_row_diag* out_row_diag,
                                              sv_batch_stats* out_stats) {
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, tau_step, min_cum,
                 seed, out_tokens, out_accept_len, shape, workspace, workspace_bytes, hip_stream,
                 out_row_diag, out_stats, nullptr, target_filter, draft_filter);
}

extern "C" sv_status sv_filter_thresholds(const void* target_logits, const void* draft_logits,
                                          const int32_t* row_offsets, const float* temperature,
                                          const sv_filter* target_filter, const sv_filter* draft_filter,
                                          float* out_theta, sv_shape shape, void* workspace,
                                          size_t workspace_bytes, void* hip_stream) {
  using namespace sv;
  Plan p;
  const sv_status st = make_plan(shape, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  if (!target_logits || !draft_logits || !row_offsets || !temperature || !out_theta || !workspace)
    return SV_E_NULLPTR;
  if (workspace_bytes < p.total) return SV_E_WORKSPACE;
  Inputs in{target_logits, draft_logits, nullptr, row_offsets, temperature, nullptr, nullptr, nullptr,
            0, p.B, p.R, p.V, p.dtype, 1, 1};
  const FilterArgs fa{{side_of(target_filter), side_of(draft_filter)}, out_theta};
  char* ws = static_cast<char*>(workspace);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const bool aligned = ((int64_t)p.V * p.esize) % 16 == 0 && (reinterpret_cast<uintptr_t>(target_logits) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(draft_logits) % 16) == 0;
  hipError_t err;
  if (p.dtype == SV_BF16)
    err = aligned ? launch_thresholds<uint16_t, 8>(p, in, fa, stream, ws) : launch_thresholds<uint16_t, 1>(p, in, fa, stream, ws);
  else
    err = aligned ? launch_thresholds<float, 4>(p, in, fa, stream, ws) : launch_thresholds<float, 1>(p, in, fa, stream, ws);
  return err == hipSuccess ? SV_OK : SV_E_HIP;
}

extern "C" sv_status sv_verify_batch_sampler_match(const void* target_logits, const int32_t* draft_tokens,
                                                   const int32_t* row_offsets, const float* temperature,
                                                   uint64_t seed, int32_t* out_tokens, int32_t* out_accept_len,
                                                   sv_shape shape, void* workspace, size_t workspace_bytes,
                                                   void* hip_stream) {
  using namespace sv;
  Plan p;
  const sv_status st = make_plan(shape, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  if (!target_logits || !draft_tokens || !row_offsets || !temperature || !out_tokens || !out_accept_len ||
      !workspace)
    return SV_E_NULLPTR;
  if (workspace_bytes < p.total) return SV_E_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  Inputs in{target_logits, nullptr, draft_tokens, row_offsets, temperature, nullptr, nullptr, nullptr,
            seed, p.B, p.R, p.V, p.dtype, 1, 1};
  Work w{reinterpret_cast<WsHeader*>(ws + p.off_hdr), reinterpret_cast<P1Part*>(ws + p.off_part1),
         nullptr, nullptr, nullptr, nullptr, nullptr};
  const Outputs out{out_tokens, out_accept_len, nullptr, nullptr};
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const bool aligned = ((int64_t)p.V * p.esize) % 16 == 0 && (reinterpret_cast<uintptr_t>(target_logits) % 16) == 0;
  hipError_t err;
  if (p.dtype == SV_BF16)
    err = aligned ? launch_match<uint16_t, 8>(p, in, w, out, stream) : launch_match<uint16_t, 1>(p, in, w, out, stream);
  else
    err = aligned ? launch_match<float, 4>(p, in, w, out, stream) : launch_match<float, 1>(p, in, w, out, stream);
  return err == hipSuccess ? SV_OK : SV_E_HIP;
}

extern "C" sv_status sv_verify_batch_static(const void* target_logits, const void* draft_logits,
                                            const int32_t* draft_tokens, const int32_t* row_offsets,
                                            const float* temperature, const float* tau, uint64_t seed,
                                            int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                                            void* hip_stream) {
  sv::Plan p;
  const sv_status st = sv::make_plan(shape, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  if (!target_logits || !draft_logits || !draft_tokens || !row_offsets || !temperature || !tau || !out_tokens ||
      !out_accept_len)
    return SV_E_NULLPTR;
  if (p.total > SV_STATIC_WORKSPACE_BYTES) return SV_E_WORKSPACE;
  void* ws = nullptr;
  if (sv::scratch_address(&ws) != hipSuccess) return SV_E_HIP;
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, nullptr, nullptr,
                 seed, out_tokens, out_accept_len, shape, ws, SV_STATIC_WORKSPACE_BYTES, hip_stream,
                 nullptr, nullptr, nullptr);
}
