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
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "sv_device.h"
#include "sv_plan.h"

namespace sv {

struct Inputs {
  const void* target;
  const void* draft;
  const int32_t* dt;
  const int32_t* ro;
  const float* temp;
  const float* tau;
  uint64_t seed;
  int32_t B, R, V, dtype;
  int32_t w1;  // pass 1: waves per row
  int32_t w2;  // pass 2: waves per request
};

struct Work {
  WsHeader* hdr;
  P1Part* part1;
  P2Part* part2;
  uint32_t* t2;  // pass 2: waves finished per request
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

struct RowCls {
  bool located;   // row r lies in a well-formed request range
  bool req_ok;    // temperature and tau are valid
  bool proposal;  // row r is tested by the method (j < n_prop)
  int b, lo, n, j;
  int n_prop;     // leading rows before the request's first no-proposal row (and before its last row)
  int D;
  float T, tau;
};

// Locate row r's request and classify it. Every index stays in bounds whatever
// row_offsets holds. A broken batch is caught by block 0's check and failed
// closed in pass 2.
__device__ RowCls classify_row(const Inputs& in, int r, int lane) {
  RowCls c{};
  int b = (int)(((int64_t)r * in.B) / in.R);
  if (b >= in.B) b = in.B - 1;
  int lo = in.ro[b], hi = in.ro[b + 1];
  if (!(lo <= r && r < hi)) {
    int L = 0, H = in.B - 1;  // largest b with ro[b] <= r
    while (L < H) {
      const int mid = (L + H + 1) >> 1;
      if (in.ro[mid] <= r) L = mid; else H = mid - 1;
    }
    b = L;
    lo = in.ro[b];
    hi = in.ro[b + 1];
  }
  c.located = 0 <= lo && lo <= r && r < hi && hi <= in.R;
  if (!c.located) return c;
  c.b = b;
  c.lo = lo;
  c.n = hi - lo;
  c.j = r - lo;
  c.T = in.temp[b];
  c.tau = in.tau[b];
  c.req_ok = temperature_ok(c.T) && !__builtin_isnan(c.tau);
  c.n_prop = c.n - 1;
  for (int base = 0; base < c.n - 1; base += kWave) {
    const int i = base + lane;
    bool badtok = false;
    if (i < c.n - 1) {
      const int D = in.dt[lo + i];
      badtok = D < 0 || D >= in.V;
    }
    const uint64_t m = __ballot(badtok);
    if (m != 0) {
      c.n_prop = base + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  c.proposal = c.req_ok && c.j < c.n_prop;
  c.D = c.proposal ? in.dt[r] : -1;
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
template <bool ARG, class CH, int U>
__device__ __forceinline__ void fold_soft(Acc& a, const CH (&x)[U], int vb, float c) {
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
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float t = fast_exp2(fmaf(x[u].get(e), c, -a.mc));
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

// Block 0 checks row_offsets for the whole batch and clears the stats.
__device__ void block0_duties(const Inputs& in, const Work& w, const Outputs& out) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  if (threadIdx.x == 0) bad = (in.ro[0] != 0) || (in.ro[in.B] != in.R);
  for (int i = threadIdx.x; i < in.B; i += kBlock) bad |= !(in.ro[i] < in.ro[i + 1]);
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) w.hdr->ro_valid = s_bad ? 0 : 1;
  if (out.stats != nullptr && threadIdx.x < 8) reinterpret_cast<int64_t*>(out.stats)[threadIdx.x] = 0;
}



// Waves, not workgroups, are assigned to rows: wave gw of the grid streams span gw % w1 of
// row gw / w1, so the split need not be a multiple of a workgroup's four waves.
template <typename E, int VEC, int U>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void pass1_kernel(Inputs in, Work w,
                                                                                             Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (blockIdx.x == 0) block0_duties(in, w, out);
  const int r = (int)min(gw / in.w1, (int64_t)in.R - 1);
  const int g = (int)(gw % in.w1);
  const bool in_grid = gw < (int64_t)in.R * in.w1;

  using CH = Chunk<E, VEC>;
  const int nvec = in.V / VEC;
  const Span sp = wave_span(nvec, in.w1, g);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)r * in.V;
  constexpr int step = U * kWave;
  CH ta[U], da[U], tb[U], db[U];
  // The first batch is requested before the row is classified, so the row's metadata and
  // its first logits arrive together. A row the method does not test drops them.
  if (sp.begin < sp.end) {
    load_chunks<true>(ta, trow, sp.begin, lane, sp.end);
    load_chunks<true>(da, drow, sp.begin, lane, sp.end);
  }
  const RowCls cls = classify_row(in, r, lane);
  if (!in_grid || !cls.proposal) return;

  const bool greedy = cls.T == 0.0f;
  const float c = fold_scale(cls.T);
  const int dvec = cls.D / VEC;
  const int de = cls.D - dvec * VEC;
  const bool holds_D = dvec >= sp.begin && dvec < sp.end;  // only this span's wave reads D's logits

  Acc at = acc_empty(), ad = acc_empty();
  int found = 0;
  float ltD = 0.0f, ldD = 0.0f;

  auto fold_both = [&](const CH (&xt)[U], const CH (&xd)[U], int wb) __attribute__((always_inline)) {
    const int vb = wb + lane;
    fold_soft<true>(at, xt, vb, c);
    fold_soft<true>(ad, xd, vb, c);
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
  pp.lt_D = __shfl(ltD, src);
  pp.ld_D = __shfl(ldD, src);
  pp.flags = fm ? 2 : 0;
  if (lane == 0) w.part1[(int64_t)r * in.w1 + g] = pp;  // read by pass 2, after this kernel
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
};

// Merge row j's partials and test its drafted token D. The wave's lanes hold the row's
// partials: slot 0 of a lane when m0 is set, slot 1 when m1 is set. The statistics are
// merged in a fixed order with fp64 sums, and every lane ends with the same result.
__device__ __forceinline__ RowEval eval_row(const Inputs& in, const P1Part& e0, const P1Part& e1, bool m0,
                                            bool m1, int b, int j, int D, float T, float tau, float c,
                                            RowStat& rs) {
  const bool greedy = T == 0.0f;
  float mt = -INFINITY, md = -INFINITY;
  if (m0) {
    mt = e0.m_t;
    md = e0.m_d;
  }
  if (m1) {
    mt = fmaxf(mt, e1.m_t);
    md = fmaxf(md, e1.m_d);
  }
  mt = wave_max(mt);
  md = wave_max(md);
  const float mct = ref_of(mt, c), mcd = ref_of(md, c);
  double st = 0.0, sd = 0.0;
  int it = INT32_MAX, id = INT32_MAX;
  if (m0) {
    if (e0.s_t != 0.0f) st += (double)(e0.s_t * fast_exp2(ref_of(e0.m_t, c) - mct));
    if (e0.s_d != 0.0f) sd += (double)(e0.s_d * fast_exp2(ref_of(e0.m_d, c) - mcd));
    if (e0.m_t == mt && e0.am_t >= 0) it = e0.am_t;
    if (e0.m_d == md && e0.am_d >= 0) id = e0.am_d;
  }
  if (m1) {
    if (e1.s_t != 0.0f) st += (double)(e1.s_t * fast_exp2(ref_of(e1.m_t, c) - mct));
    if (e1.s_d != 0.0f) sd += (double)(e1.s_d * fast_exp2(ref_of(e1.m_d, c) - mcd));
    if (e1.m_t == mt && e1.am_t >= 0) it = min(it, e1.am_t);
    if (e1.m_d == md && e1.am_d >= 0) id = min(id, e1.am_d);
  }
  st = wave_sum(st);
  sd = wave_sum(sd);
  it = wave_min(it);
  id = wave_min(id);
  const bool f0 = m0 && (e0.flags & 2), f1 = m1 && (e1.flags & 2);
  const uint64_t fm = __ballot(f0 || f1);
  const int src = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
  const float ltD = __shfl(f0 ? e0.lt_D : e1.lt_D, src);
  const float ldD = __shfl(f0 ? e0.ld_D : e1.ld_D, src);
  rs = RowStat{mt, mct, md, mcd, st, sd, it == INT32_MAX ? -1 : it, id == INT32_MAX ? -1 : id};

  const bool valid = __builtin_isfinite(mt) && __builtin_isfinite(md) && __builtin_isfinite(st) && st > 0.0 &&
                     __builtin_isfinite(sd) && sd > 0.0;
  RowEval ev{};
  ev.u = NAN;
  if (greedy) {
    ev.p_D = (D == rs.am_t) ? 1.0f : 0.0f;
    ev.q_D = (D == rs.am_d) ? 1.0f : 0.0f;
    const bool offered = ev.q_D >= tau;
    ev.mu_D = offered ? ev.q_D : 0.0f;
    // p(D) is 0 or 1 and mu(D) <= 1: u*mu(D) < p(D) holds for every u iff p(D) = 1.
    ev.verdict = !valid ? kRowInvalid : !offered ? SV_ROW_NULL : (ev.p_D == 1.0f ? SV_ROW_ACCEPT : SV_ROW_REJECT);
    return ev;
  }
  const double p = exp2((double)ltD * (double)c - (double)mct) / st;
  const double q = exp2((double)ldD * (double)c - (double)mcd) / sd;
  const bool offered = q >= (double)tau;
  const double mu = offered ? q : 0.0;
  ev.p_D = (float)p;
  ev.q_D = (float)q;
  ev.mu_D = (float)mu;
  if (!valid || fm == 0) {
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

// A request as pass 2 rebuilds it.
struct ReqState {
  int lo, n, n_prop;
  int k;              // accepted drafts
  int f;              // the row that yields the last token (lo + k)
  int kind;           // kKind*
  int final_verdict;  // verdict of row f (SV_ROW_BONUS when every proposal row was accepted)
  float T, tau, c;
  RowStat stop;       // row f's statistics when f is a proposal row
  int stop_slot;      // row f's index within the partial group held in e0/e1
};

// Rebuild request b from the inputs and pass 1's partials: walk its proposal rows in
// order up to the first one that is not accepted. Every wave of the request does this on
// its own, so no wave waits for another.
//  - Round trip 1: the request's row range, temperature and tau.
//  - Round trip 2: the drafted tokens of its first 64 rows and the partials of its first
//    128 / (waves per row) rows, fetched together into two slots per lane (e0, e1).
// On return e0/e1 hold the group of partials that contains row f. With `diag`, each row's
// record is written once: tested rows by lane 0 in the walk (the stop row with
// `stop_resid`), untested and bonus rows after it.
__device__ __forceinline__ ReqState walk_request(const Inputs& in, const Work& w, int b, int lane,
                                                 P1Part& e0, P1Part& e1, sv_row_diag* diag,
                                                 float stop_resid) {
  ReqState q{};
  q.lo = in.ro[b];
  q.n = in.ro[b + 1] - q.lo;
  q.T = in.temp[b];
  q.tau = in.tau[b];
  q.stop_slot = -1;
  const bool req_ok = temperature_ok(q.T) && !__builtin_isnan(q.tau);
  q.c = req_ok ? fold_scale(q.T) : 0.0f;
  const int nw = in.w1;
  const int per_group = (2 * kWave) / nw;
  const int nd = q.n - 1;  // rows that carry a drafted token: all but the last

  const int dt0 = in.dt[q.lo + min(lane, max(nd - 1, 0))];  // lane j: row j's drafted token (j < nd)
  {
    const int ne = min(per_group, max(nd, 1)) * nw;
    const P1Part* base = w.part1 + (int64_t)q.lo * nw;
    e0 = base[min(lane, ne - 1)];
    e1 = base[min(lane + kWave, ne - 1)];
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
  for (int j0 = 0; j0 < q.n_prop; j0 += per_group) {
    const int nrows = min(per_group, q.n_prop - j0);
    if (j0 > 0) {  // windows longer than one group
      const int ne = nrows * nw;
      const P1Part* base = w.part1 + (int64_t)(q.lo + j0) * nw;
      e0 = base[min(lane, ne - 1)];
      e1 = base[min(lane + kWave, ne - 1)];
    }
    bool stop = false;
    for (int jj = 0; jj < nrows; ++jj) {
      const int j = j0 + jj;
      const bool m0 = lane / nw == jj;
      const bool m1 = (lane + kWave) / nw == jj;
      const int D = j < kWave ? __shfl(dt0, j) : in.dt[q.lo + j];
      RowStat rs;
      const RowEval ev = eval_row(in, e0, e1, m0, m1, b, j, D, q.T, q.tau, q.c, rs);
      const bool accepted = ev.verdict == SV_ROW_ACCEPT;
      if (diag != nullptr && lane == 0) {
        sv_row_diag dg;
        dg.p_D = ev.p_D;
        dg.q_D = ev.q_D;
        dg.mu_D = ev.mu_D;
        dg.u = ev.u;
        dg.resid_mass = accepted ? NAN : stop_resid;
        dg.verdict = ev.verdict;
        dg.pad0 = dg.pad1 = 0;
        diag[q.lo + j] = dg;
      }
      if (!accepted) {
        k = j;
        q.final_verdict = ev.verdict;
        q.stop = rs;
        q.stop_slot = jj;
        stop = true;
        break;
      }
    }
    if (stop) break;
  }
  q.k = k;
  q.f = q.lo + k;
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
  return q;
}

__device__ __forceinline__ void add_stats(const Outputs& out, const ReqState& q, bool invalid) {
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
}

// Write request b's outputs (one wave): the accepted drafts, the last token, -1 after it.
// A request that fails closed gets -1 everywhere and untested diagnostics.
__device__ __forceinline__ void emit_request(const Inputs& in, const Work& w, const Outputs& out, int b,
                                             const ReqState& q, bool invalid, int token, float resid, int lane) {
  for (int j = lane; j < q.n; j += kWave) {
    const int r = q.lo + j;
    out.tokens[r] = invalid ? -1 : (j < q.k ? in.dt[r] : (j == q.k ? token : -1));
  }
  if (lane == 0) {
    out.accept_len[b] = invalid ? -1 : q.k;
    add_stats(out, q, invalid);
  }
  if (out.diag != nullptr) {
    if (invalid) {
      for (int j = lane; j < q.n; j += kWave) out.diag[q.lo + j] = untested_diag();
    } else {
      P1Part e0, e1;
      walk_request(in, w, b, lane, e0, e1, out.diag, resid);
    }
  }
}

// fp64 race key of token x on a residual row, from its two logits.
__device__ __forceinline__ double residual_key64(double lt, double ld, double c, double mct, double mcd,
                                                 double st, double sd, double tau, uint32_t word) {
  const double p = exp2(lt * c - mct) / st;
  const double q = exp2(ld * c - mcd) / sd;
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

// A race over p read by one wave: the rare fallback for a residual with no mass.
__device__ __forceinline__ int p_race_one_wave(const Inputs& in, const ReqState& q, int b, int lane) {
  Top2 t = top2_empty();
  for (int64_t x = lane; x < in.V; x += kWave) {
    const float l = logit_at(in.target, in.dtype, (int64_t)q.f * in.V + x);
    const float a = l * q.c;
    if (a > -INFINITY) {
      const uint32_t wd = race_word(in.seed, x, q.k, b);
      top2_push(t, a - __log2f(expo32(wd)), (int)x, l, 0.0f);
    }
  }
  wave_top2(t);
  double bk = -INFINITY;
  int bi = INT32_MAX;
  if (lane < 2) {
    const int x = lane == 0 ? t.i1 : t.i2;
    const float l = lane == 0 ? t.a1 : t.a2;
    if (x != INT32_MAX) {
      bk = p_logkey64((double)l, (double)q.T, race_word(in.seed, x, q.k, b));
      bi = x;
    }
  }
  wave_best(bk, bi);
  return bi;
}

// Wave gw of the grid serves span gw % w2 of request gw / w2.
template <typename E, int VEC, int U>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void pass2_kernel(Inputs in, Work w,
                                                                                             Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (gw >= (int64_t)in.B * in.w2) return;
  const int b = (int)(gw / in.w2);
  const int g = (int)(gw % in.w2);
  const bool head = g == 0;

  if (!w.hdr->ro_valid) {
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

  P1Part e0, e1;
  const ReqState q = walk_request(in, w, b, lane, e0, e1, nullptr, NAN);
  if (q.kind == kKindInvalid) {
    if (head) emit_request(in, w, out, b, q, true, -1, NAN, lane);
    return;
  }
  if (q.kind == kKindGreedyDone) {
    // One-hot p and mu: the residual is empty iff the offered draft argmax is the target argmax.
    const float resid = (q.stop.am_t == q.stop.am_d && 1.0f >= q.tau) ? 0.0f : 1.0f;
    if (head) emit_request(in, w, out, b, q, false, q.stop.am_t, resid, lane);
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

  P2Part part{};
  part.key = -INFINITY;
  part.idx = -1;
  part.rsum = 0.0f;
  part.mref = -INFINITY;
  part.bad = 0;
  part.gidx = -1;

  if (q.kind == kKindResidual) {
    const float c = q.c, mct = q.stop.mc_t, mcd = q.stop.mc_d, tau = q.tau;
    const float ist = (float)(1.0 / q.stop.s_t), isd = (float)(1.0 / q.stop.s_d);
    float rsum = 0.0f;
    Top2 t = top2_empty();
    // Pruning bound. Pass 1 left, per wave of row f, the vector that held that wave's
    // target maximum; the partials of row f are in this wave's registers. The best race key
    // among those tokens is a key some token really has, so the winner's key is at least
    // that large. A token whose residual r has r / E_min below half of it cannot win and
    // draws no random number. Only tokens with mu <= p/2 serve: there r = p - mu carries at
    // most twice the fp32 error of p, so the bound is exact to about 1e-6 and the factor 2
    // absorbs it.
    const int nw1 = in.w1;
    const int nh = nw1 * VEC;
    int hx[VEC];
    float hlt[VEC], hld[VEC];
#pragma unroll
    for (int s = 0; s < VEC; ++s) {
      const int ti = lane + s * kWave;
      const int pos = q.stop_slot * nw1 + min(ti / VEC, nw1 - 1);
      const int h0 = __shfl(e0.am_t, pos & (kWave - 1));
      const int h1 = __shfl(e1.am_t, pos & (kWave - 1));
      const int hv = pos < kWave ? h0 : h1;
      int x = (ti < nh && hv >= 0) ? hv * VEC + ti % VEC : -1;
      x = x < in.V ? x : -1;
      hx[s] = x;
      const int xc = x >= 0 ? x : 0;
      hlt[s] = to_float(trow[xc]);
      hld[s] = to_float(drow[xc]);
    }
    // The span's first batch is requested before the hint logits are used, so both
    // arrive in one round trip.
    CH ta[U], da[U];
    if (sp.begin < sp.end) {
      load_chunks<false>(ta, trow, sp.begin, lane, sp.end);
      load_chunks<false>(da, drow, sp.begin, lane, sp.end);
    }
    float kh = 0.0f;
#pragma unroll
    for (int s = 0; s < VEC; ++s) {
      const float p = fast_exp2(fmaf(hlt[s], c, -mct)) * ist;
      const float qq = fast_exp2(fmaf(hld[s], c, -mcd)) * isd;
      const float mu = qq >= tau ? qq : 0.0f;
      if (hx[s] >= 0 && p > 0.0f && mu <= 0.5f * p)
        kh = fmaxf(kh, (float)((double)(p - mu) / expo64(race_word(in.seed, hx[s], q.k, b))));
    }
    kh = wave_max(kh);
    const float pthr = kh * (float)(kEminLow * 0.5);
    auto fold_res = [&](const CH (&xt)[U], const CH (&xd)[U], int v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x0 = (v0 + u * kWave) * VEC;
#pragma unroll
        for (int gg = 0; gg < VEC; gg += G) {
          float rv[G];
          bool any = false;
#pragma unroll
          for (int e = 0; e < G; ++e) {
            const float p = fast_exp2(fmaf(xt[u].get(gg + e), c, -mct)) * ist;
            const float qq = fast_exp2(fmaf(xd[u].get(gg + e), c, -mcd)) * isd;
            const float mu = qq >= tau ? qq : 0.0f;
            const float r = fmaxf(p - mu, 0.0f);
            rsum += r;
            rv[e] = r;
            any |= (r > 0.0f && r >= pthr);
          }
          if (any) {
            const int xg = x0 + gg;
            const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)q.k, (uint32_t)b, k0, k1);
#pragma unroll
            for (int e = 0; e < G; ++e) {
              if (rv[e] > 0.0f && rv[e] >= pthr) {
                const int x = xg + e;
                const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, x & 3);
                top2_push(t, rv[e] / expo32(wd), x, xt[u].get(gg + e), xd[u].get(gg + e));
              }
            }
          }
        }
      }
    };
    // One batch per step; at the planned split a wave's span is about one batch.
    const int nsteps = (sp.end - sp.begin + step - 1) / step;
    for (int i = 0, base = sp.begin; i < nsteps; ++i, base += step) {
      mask_chunks(ta, base, lane, sp.end);
      mask_chunks(da, base, lane, sp.end);
      fold_res(ta, da, base + lane);
      if (i + 1 < nsteps) {
        load_chunks<false>(ta, trow, base + step, lane, sp.end);
        load_chunks<false>(da, drow, base + step, lane, sp.end);
      }
    }
    wave_top2(t);
    part.rsum = wave_sum(rsum);
    double bk = -INFINITY;
    int bi = INT32_MAX;
    if (lane < 2) {
      const int x = lane == 0 ? t.i1 : t.i2;
      if (x != INT32_MAX) {
        bk = residual_key64((double)(lane == 0 ? t.a1 : t.a2), (double)(lane == 0 ? t.b1 : t.b2), (double)c,
                            (double)mct, (double)mcd, q.stop.s_t, q.stop.s_d, (double)tau,
                            race_word(in.seed, x, q.k, b));
        bi = x;
      }
    }
    wave_best(bk, bi);
    part.key = bk;
    part.idx = bi == INT32_MAX ? -1 : bi;
  } else {
    // Bonus row (race over p) or greedy bonus row (argmax). Pass 1 never read it, so it is validated here.
    const bool race = q.kind == kKindBonus;
    const float c = q.c;
    Acc a = acc_empty();
    int bad = 0;
    Top2 t = top2_empty();
    float wbest = -INFINITY;  // best log2 key the wave has seen so far
    CH ta[U];
    auto fold_bonus = [&](const CH (&xt)[U], int v0) __attribute__((always_inline)) {
      if (race) fold_max<false>(a, xt, v0, bad);  // max and NaN / +inf check
      else fold_max<true>(a, xt, v0, bad);       // ... and the lowest index of the max
      if (race) {
        float lbest = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int x0 = (v0 + u * kWave) * VEC;
#pragma unroll
          for (int gg = 0; gg < VEC; gg += G) {
            // A token's log2 key is l*c - log2(E) <= l*c + 24 (E >= 2^-24). It cannot win if
            // that bound is a factor 2 below a key already seen.
            float av[G];
            bool any = false;
#pragma unroll
            for (int e = 0; e < G; ++e) {
              av[e] = xt[u].get(gg + e) * c;
              any |= av[e] + 25.0f >= wbest;
            }
            if (any) {
              const int xg = x0 + gg;
              const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)q.k, (uint32_t)b, k0, k1);
#pragma unroll
              for (int e = 0; e < G; ++e) {
                if (av[e] + 25.0f >= wbest) {
                  const int x = xg + e;
                  const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, x & 3);
                  const float key = av[e] - __log2f(expo32(wd));
                  lbest = fmaxf(lbest, key);
                  top2_push(t, key, x, xt[u].get(gg + e), 0.0f);
                }
              }
            }
          }
        }
        wbest = fmaxf(wbest, wave_max(lbest));
      }
    };
    if (sp.begin < sp.end) load_chunks<false>(ta, trow, sp.begin, lane, sp.end);
    const int nsteps = (sp.end - sp.begin + step - 1) / step;
    for (int i = 0, base = sp.begin; i < nsteps; ++i, base += step) {
      mask_chunks(ta, base, lane, sp.end);
      fold_bonus(ta, base + lane);
      if (i + 1 < nsteps) load_chunks<false>(ta, trow, base + step, lane, sp.end);
    }
    float m;
    float unused;
    int am;
    wave_stat(a, 0.0f, false, m, unused, am);
    part.mref = m;
    part.gidx = race ? -1 : exact_argmax<CH>(trow, a, m);
    part.bad = wave_or(bad);
    if (race) {
      wave_top2(t);
      double bk = -INFINITY;
      int bi = INT32_MAX;
      if (lane < 2) {
        const int x = lane == 0 ? t.i1 : t.i2;
        if (x != INT32_MAX) {
          bk = p_logkey64((double)(lane == 0 ? t.a1 : t.a2), (double)q.T, race_word(in.seed, x, q.k, b));
          bi = x;
        }
      }
      wave_best(bk, bi);
      part.key = bk;
      part.idx = bi == INT32_MAX ? -1 : bi;
    }
  }

  if (lane == 0) publish(&w.part2[(int64_t)b * nw + g], part);
  if (!arrive_last(&w.t2[b], (uint32_t)nw, lane)) return;

  // ---- the request's last wave: merge the partials and write the outputs
  const P2Part* pp = w.part2 + (int64_t)b * nw;
  bool invalid = false;
  int token = -1;
  float resid = NAN;
  if (q.kind == kKindResidual) {
    double R = 0.0, bk = -1.0;
    int bi = INT32_MAX;
    for (int i = lane; i < nw; i += kWave) {
      const P2Part c2 = read_record(pp + i);
      R += (double)c2.rsum;
      if (c2.idx >= 0 && beats(c2.key, c2.idx, bk, bi)) {
        bk = c2.key;
        bi = c2.idx;
      }
    }
    R = wave_sum(R);
    wave_best(bk, bi);
    resid = (float)R;
    if (R > 0.0 && bk > 0.0) token = bi;
    else token = p_race_one_wave(in, q, b, lane);  // residual with no mass: race over p
  } else {
    float M = -INFINITY;
    int bad = 0;
    double bk = -INFINITY;
    int bi = INT32_MAX;
    for (int i = lane; i < nw; i += kWave) {
      const P2Part c2 = read_record(pp + i);
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
        const P2Part c2 = read_record(pp + i);
        if (c2.mref == M && c2.gidx >= 0) gi = min(gi, c2.gidx);
      }
      token = wave_min(gi);
    } else {
      invalid = invalid || bi == INT32_MAX;
      token = bi;
    }
  }
  emit_request(in, w, out, b, q, invalid, token, resid, lane);
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
  size_t off_ticket2, total;
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
  if (slot >= 0 && g_layout[slot].off_ticket2 == p.off_ticket2 && g_layout[slot].total == p.total)
    return hipSuccess;
  const int64_t n = (int64_t)(p.total - p.off_ticket2) / 4;  // the ticket array sits at the end
  const int64_t blocks = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(kBlock), 0,
                     stream, reinterpret_cast<uint32_t*>(ws + p.off_ticket2), n);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (slot < 0) slot = g_layout_n < 64 ? g_layout_n++ : (int)(reinterpret_cast<uintptr_t>(ws) / 256 % 64);
  g_layout[slot] = LayoutSeen{dev, ws, p.off_ticket2, p.total};
  return hipSuccess;
}

// Resident waves per kernel on a device: compute units times the workgroups of the kernel
// that fit on one, times four waves. Queried once per (device, kernel).
struct SlotsSeen {
  int device;
  const void* fn;
  int64_t slots;
};

static std::mutex g_slots_mu;
static SlotsSeen g_slots[64];
static int g_slots_n = 0;

static hipError_t resident_waves(const void* fn, int64_t* slots) {
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
  const int64_t s = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1) * kWavesPerBlock;
  if (g_slots_n < 64) g_slots[g_slots_n++] = SlotsSeen{dev, fn, s};
  *slots = s;
  return hipSuccess;
}

template <typename E, int VEC>
hipError_t launch_pair(const Plan& p, Inputs in, const Work& w, const Outputs& out, hipStream_t stream,
                       hipEvent_t const* ev) {
  constexpr int U1 = VEC == 1 ? 12 : 3;  // pass 1: 12 logits per lane per array and step (x2 buffers)
  constexpr int U2 = VEC == 1 ? 16 : 6;  // pass 2: one larger batch per array and step
  const void* k1 = reinterpret_cast<const void*>(&pass1_kernel<E, VEC, U1>);
  const void* k2 = reinterpret_cast<const void*>(&pass2_kernel<E, VEC, U2>);
  int64_t slots1 = 0, slots2 = 0;
  hipError_t err = resident_waves(k1, &slots1);
  if (err != hipSuccess) return err;
  if ((err = resident_waves(k2, &slots2)) != hipSuccess) return err;
  const Launch l = pick_waves(p, slots1, slots2);
  in.w1 = l.w1;
  in.w2 = l.w2;
  if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
  const dim3 block(kBlock);
  hipLaunchKernelGGL((pass1_kernel<E, VEC, U1>), dim3((unsigned)l.blocks1), block, 0, stream, in, w, out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
  hipLaunchKernelGGL((pass2_kernel<E, VEC, U2>), dim3((unsigned)l.blocks2), block, 0, stream, in, w, out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev && (err = hipEventRecord(ev[2], stream)) != hipSuccess) return err;
  return hipSuccess;
}

static sv_status run(const void* target, const void* draft, const int32_t* draft_tokens,
                     const int32_t* row_offsets, const float* temperature, const float* tau,
                     uint64_t seed, int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                     void* workspace, size_t workspace_bytes, void* hip_stream,
                     sv_row_diag* diag, sv_batch_stats* stats, void* const* events) {
  Plan p;
  const sv_status st = check_call(shape, target, draft, draft_tokens, row_offsets, temperature, tau,
                                  out_tokens, out_accept_len, workspace, workspace_bytes, &p);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;
  char* ws = static_cast<char*>(workspace);
  Inputs in{target, draft, draft_tokens, row_offsets, temperature, tau, seed, p.B, p.R, p.V, p.dtype, 1, 1};
  Work w{reinterpret_cast<WsHeader*>(ws + p.off_hdr), reinterpret_cast<P1Part*>(ws + p.off_part1),
         reinterpret_cast<P2Part*>(ws + p.off_part2), reinterpret_cast<uint32_t*>(ws + p.off_ticket2)};
  Outputs out{out_tokens, out_accept_len, diag, stats};
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
  // 16-byte loads need 16-byte aligned rows: V * element size a multiple of 16 and aligned bases.
  const bool aligned = ((int64_t)p.V * p.esize) % 16 == 0 &&
                       (reinterpret_cast<uintptr_t>(target) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(draft) % 16) == 0;
  hipError_t err = counters_ready(p, ws, stream);
  if (err != hipSuccess) return SV_E_HIP;
  if (p.dtype == SV_BF16) {
    err = aligned ? launch_pair<uint16_t, 8>(p, in, w, out, stream, ev)
                  : launch_pair<uint16_t, 1>(p, in, w, out, stream, ev);
  } else {
    err = aligned ? launch_pair<float, 4>(p, in, w, out, stream, ev)
                  : launch_pair<float, 1>(p, in, w, out, stream, ev);
  }
  return err == hipSuccess ? SV_OK : SV_E_HIP;
}

}  // namespace sv

extern "C" sv_status sv_verify_batch(const void* target_logits, const void* draft_logits,
                                     const int32_t* draft_tokens, const int32_t* row_offsets,
                                     const float* temperature, const float* tau, uint64_t seed,
                                     int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                                     void* workspace, size_t workspace_bytes, void* hip_stream) {
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, seed,
                 out_tokens, out_accept_len, shape, workspace, workspace_bytes, hip_stream,
                 nullptr, nullptr, nullptr);
}

extern "C" sv_status sv_verify_batch_diag(const void* target_logits, const void* draft_logits,
                                          const int32_t* draft_tokens, const int32_t* row_offsets,
                                          const float* temperature, const float* tau, uint64_t seed,
                                          int32_t* out_tokens, int32_t* out_accept_len,
                                          sv_shape shape, void* workspace, size_t workspace_bytes,
                                          void* hip_stream, sv_row_diag* out_row_diag,
                                          sv_batch_stats* out_stats, void* const* hip_events) {
  return sv::run(target_logits, draft_logits, draft_tokens, row_offsets, temperature, tau, seed,
                 out_tokens, out_accept_len, shape, workspace, workspace_bytes, hip_stream,
                 out_row_diag, out_stats, hip_events);
}
