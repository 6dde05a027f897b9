// sv_kernels.hip - the verify sampler's kernels and the exported C-ABI calls.
//
// Pass 1 streams the target and draft logits of every proposal row once.
//  - Rows are split into spans. One long-lived wave per span reads the span
//    with double-buffered 16-byte loads and keeps per-lane running softmax
//    statistics (max, sum of exp2 against that max) and the lowest-index
//    argmax. It also picks up the logits at the drafted token D from
//    registers.
//  - The last wave of a row (atomic ticket) merges the row's partials in fp64
//    and runs the accept test. The test follows Strata PR #3416 "[Engine]
//    Preserve target probabilities in gated MTP", section Approach, with the
//    accept form of mlxcel PR #992, section What changed.
//  - The last row of a request (second ticket) walks the verdicts to the
//    first row that was not accepted (mlxcel PR #992, section Two metric
//    corrections). It writes a request descriptor for pass 2.
//
// Pass 2 draws each request's last token from the row that ended it:
//  - a residual draw from (p - mu)+ on a rejected or NULL row;
//  - a bonus draw from p;
//  - or the greedy argmax at temperature 0.
// The draw is an exponential race argmax_x w_x / E_x, with ties going to the
// lower index. Each wave streams a span, prunes tokens that provably cannot
// win before drawing their random numbers, and re-evaluates its two best fp32
// candidates in fp64. The request's last wave merges and writes the outputs.
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
  int32_t B, R, V, dtype, s1, s2;
};

struct Work {
  WsHeader* hdr;
  P1Part* part1;
  RowRec* rec;
  ReqDesc* desc;
  P2Part* part2;
  uint32_t* t_row;  // pass 1: waves finished per row
  uint32_t* t_req;  // pass 1: rows finalised per request
  uint32_t* t2;     // pass 2: waves finished per request
};

struct Outputs {
  int32_t* tokens;
  int32_t* accept_len;
  sv_row_diag* diag;
  sv_batch_stats* stats;
};

__device__ __forceinline__ uint32_t seed_lo(uint64_t s) { return (uint32_t)s; }
__device__ __forceinline__ uint32_t seed_hi(uint64_t s) { return (uint32_t)(s >> 32); }

__device__ __forceinline__ double as_double(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Vector indices [begin, end) of wave g among `nwaves` waves that share a row.
struct Span {
  int64_t begin, end;
};

__device__ __forceinline__ Span wave_span(int64_t nvec, int nwaves, int g) {
  int64_t per = (nvec + nwaves - 1) / nwaves;
  per = (per + kWave - 1) / kWave * kWave;
  int64_t b = (int64_t)g * per;
  int64_t e = b + per;
  if (b > nvec) b = nvec;
  if (e > nvec) e = nvec;
  return Span{b, e};
}

__device__ __forceinline__ sv_row_diag untested_diag() {
  sv_row_diag d;
  d.p_D = d.q_D = d.mu_D = d.u = d.resid_mass = NAN;
  d.verdict = SV_ROW_UNTESTED;
  d.pad0 = d.pad1 = 0;
  return d;
}

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
__device__ __forceinline__ void fold_soft(Acc& a, const CH (&x)[U], int64_t vb, float c) {
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
    a.am = (bm > a.m) ? (int)(vb + (int64_t)h * kWave) : a.am;
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
__device__ __forceinline__ void fold_max(Acc& a, const CH (&x)[U], int64_t vb, int& bad) {
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
    a.am = (bm > a.m) ? (int)(vb + (int64_t)h * kWave) : a.am;
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
template <class CH, int U, typename E>
__device__ __forceinline__ void load_chunks(CH (&x)[U], const E* row, int64_t wb, int lane, int64_t vend) {
  constexpr int VEC = CH::kVec;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t vi = wb + (int64_t)u * kWave + lane;
    vi = vi < vend ? vi : vend - 1;
    x[u].load(row + vi * VEC);
  }
}

// Turn the chunks of lanes past the span's end into -inf. Wave-uniform test per chunk row.
template <class CH, int U>
__device__ __forceinline__ void mask_chunks(CH (&x)[U], int64_t wb, int lane, int64_t vend) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t w0 = wb + (int64_t)u * kWave;
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

// Outputs of a request that pass 1 can finish by itself (invalid, or greedy with a
// rejected/NULL row), or its diagnostics for pass 2 to complete.
__device__ void write_request_rows(const Inputs& in, const Work& w, const Outputs& out, const RowCls& cls,
                                   const ReqDesc& d, bool emit, int lane) {
  const bool invalid = d.kind == kKindInvalid;
  for (int j = lane; j < cls.n; j += kWave) {
    const int r = cls.lo + j;
    if (emit) {
      int t = -1;
      if (!invalid) t = j < d.k ? in.dt[r] : (j == d.k ? (int32_t)load_word(reinterpret_cast<const uint32_t*>(&w.rec[d.f].am_t)) : -1);
      out.tokens[r] = t;
    }
    if (out.diag != nullptr) {
      sv_row_diag dg = untested_diag();
      if (!invalid && j <= d.k) {
        if (j == d.k && d.final_verdict == SV_ROW_BONUS) {
          dg.verdict = SV_ROW_BONUS;
        } else {
          const RowRec rr = read_record(w.rec + r);
          dg.p_D = rr.p_D;
          dg.q_D = rr.q_D;
          dg.mu_D = rr.mu_D;
          dg.u = rr.u;
          dg.verdict = rr.verdict;
          if (j == d.k && d.kind == kKindGreedyDone)  // one-hot residual: empty iff the gated draft argmax is the target argmax
            dg.resid_mass = (rr.am_t == rr.am_d && 1.0f >= d.tau) ? 0.0f : 1.0f;
        }
      }
      out.diag[r] = dg;
    }
  }
  if (emit && lane == 0) out.accept_len[cls.b] = invalid ? -1 : d.k;
}

// A request with no proposal row (or with an invalid temperature or tau): its head wave
// describes it for pass 2.
__device__ void head_without_proposals(const Inputs& in, const Work& w, const Outputs& out,
                                       const RowCls& cls, int lane) {
  ReqDesc d{};
  d.k = 0;
  d.f = cls.lo;
  d.T = cls.T;
  d.tau = cls.tau;
  if (!cls.req_ok) {
    d.kind = kKindInvalid;
    d.final_verdict = 0;
  } else {
    d.kind = cls.T == 0.0f ? kKindGreedyBonus : kKindBonus;
    d.final_verdict = SV_ROW_BONUS;
    d.c = cls.T == 0.0f ? 0.0f : scale_of(cls.T);
  }
  if (lane == 0) w.desc[cls.b] = d;
  write_request_rows(in, w, out, cls, d, d.kind == kKindInvalid, lane);
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

// The last row of a request to be finalised walks the request's verdicts.
__device__ void finalize_request(const Inputs& in, const Work& w, const Outputs& out, const RowCls& cls,
                                 int lane) {
  const bool greedy = cls.T == 0.0f;
  int k = cls.n_prop;
  for (int base = 0; base < cls.n_prop; base += kWave) {
    const int j = base + lane;
    bool stop = false;
    if (j < cls.n_prop)
      stop = (int32_t)load_word(reinterpret_cast<const uint32_t*>(&w.rec[cls.lo + j].verdict)) != SV_ROW_ACCEPT;
    const uint64_t m = __ballot(stop);
    if (m != 0) {
      k = base + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  ReqDesc d{};
  d.k = k;
  d.f = cls.lo + k;
  d.T = cls.T;
  d.tau = cls.tau;
  d.c = greedy ? 0.0f : scale_of(cls.T);
  if (k < cls.n_prop) {
    const RowRec rr = read_record(w.rec + d.f);
    d.final_verdict = rr.verdict;
    if (rr.verdict == kRowInvalid) {
      d.kind = kKindInvalid;
    } else if (greedy) {
      d.kind = kKindGreedyDone;
    } else {
      d.kind = kKindResidual;
      d.mc_t = rr.mc_t;
      d.mc_d = rr.mc_d;
      d.m_t = rr.m_t;
      d.s_t = as_double(rr.s_t_lo, rr.s_t_hi);
      d.s_d = as_double(rr.s_d_lo, rr.s_d_hi);
    }
  } else {
    d.kind = greedy ? kKindGreedyBonus : kKindBonus;
    d.final_verdict = SV_ROW_BONUS;
  }
  if (lane == 0) w.desc[cls.b] = d;
  const bool emit = d.kind == kKindInvalid || d.kind == kKindGreedyDone;
  write_request_rows(in, w, out, cls, d, emit, lane);
}

// Merge a row's partials (fixed order, fp64 sums), test the drafted token, publish the row.
__device__ void finalize_row(const Inputs& in, const Work& w, int r, const RowCls& cls, int lane) {
  const int np = in.s1 * kWavesPerBlock;
  const P1Part* pp = w.part1 + (int64_t)r * np;
  const bool greedy = cls.T == 0.0f;
  const float c = greedy ? 1.0f : scale_of(cls.T);

  float mt = -INFINITY, md = -INFINITY, ltD = 0.0f, ldD = 0.0f;
  int found = 0;
  for (int i = lane; i < np; i += kWave) {
    const P1Part q = read_record(pp + i);
    mt = fmaxf(mt, q.m_t);
    md = fmaxf(md, q.m_d);
    if (q.flags & 2) {
      found = 1;
      ltD = q.lt_D;
      ldD = q.ld_D;
    }
  }
  mt = wave_max(mt);
  md = wave_max(md);
  const uint64_t fm = __ballot(found);
  const int src = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
  ltD = __shfl(ltD, src);
  ldD = __shfl(ldD, src);
  int it = INT32_MAX, id = INT32_MAX;
  double st = 0.0, sd = 0.0;
  const float mct = ref_of(mt, c), mcd = ref_of(md, c);
  for (int i = lane; i < np; i += kWave) {
    const P1Part q = read_record(pp + i);
    if (q.m_t == mt && q.am_t >= 0) it = min(it, q.am_t);
    if (q.m_d == md && q.am_d >= 0) id = min(id, q.am_d);
    if (q.s_t != 0.0f) st += (double)(q.s_t * fast_exp2(ref_of(q.m_t, c) - mct));
    if (q.s_d != 0.0f) sd += (double)(q.s_d * fast_exp2(ref_of(q.m_d, c) - mcd));
  }
  it = wave_min(it);
  id = wave_min(id);
  st = wave_sum(st);
  sd = wave_sum(sd);

  const int D = cls.D;
  int verdict;
  float pD, qD, muD, u = NAN;
  const bool valid = __builtin_isfinite(mt) && __builtin_isfinite(md) && __builtin_isfinite(st) && st > 0.0 &&
                     __builtin_isfinite(sd) && sd > 0.0;
  if (greedy) {
    pD = (D == it) ? 1.0f : 0.0f;
    qD = (D == id) ? 1.0f : 0.0f;
    const bool offered = qD >= cls.tau;
    muD = offered ? qD : 0.0f;
    // p(D) is 0 or 1 and mu(D) <= 1: u*mu(D) < p(D) holds for every u iff p(D) = 1.
    verdict = !valid ? kRowInvalid : !offered ? SV_ROW_NULL : (pD == 1.0f ? SV_ROW_ACCEPT : SV_ROW_REJECT);
  } else {
    const double p = exp2((double)ltD * (double)c - (double)mct) / st;
    const double q = exp2((double)ldD * (double)c - (double)mcd) / sd;
    const bool offered = q >= (double)cls.tau;
    const double mu = offered ? q : 0.0;
    pD = (float)p;
    qD = (float)q;
    muD = (float)mu;
    if (!valid || fm == 0) {
      verdict = kRowInvalid;
    } else if (!offered) {
      verdict = SV_ROW_NULL;
    } else {
      const Philox4 ph = philox4x32_10(0u, kTagAccept, (uint32_t)cls.j, (uint32_t)cls.b,
                                       seed_lo(in.seed), seed_hi(in.seed));
      u = uniform_accept(ph.w0);
      verdict = ((double)u * mu < p) ? SV_ROW_ACCEPT : SV_ROW_REJECT;
    }
  }
  if (lane == 0) {
    RowRec rr{};
    rr.verdict = verdict;
    rr.am_t = it == INT32_MAX ? -1 : it;
    rr.am_d = id == INT32_MAX ? -1 : id;
    rr.c = c;
    rr.m_t = mt;
    rr.mc_t = mct;
    rr.m_d = md;
    rr.mc_d = mcd;
    const uint64_t sb = (uint64_t)__double_as_longlong(st), db = (uint64_t)__double_as_longlong(sd);
    rr.s_t_lo = (uint32_t)sb;
    rr.s_t_hi = (uint32_t)(sb >> 32);
    rr.s_d_lo = (uint32_t)db;
    rr.s_d_hi = (uint32_t)(db >> 32);
    rr.p_D = pD;
    rr.q_D = qD;
    rr.mu_D = muD;
    rr.u = u;
    publish(w.rec + r, rr);
  }
}

template <typename E, int VEC, int U>
__global__ __launch_bounds__(kBlock) void pass1_kernel(Inputs in, Work w, Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t bid = blockIdx.x;
  if (bid == 0) block0_duties(in, w, out);
  const int r = (int)(bid / in.s1);
  const int chunk = (int)(bid % in.s1);
  const RowCls cls = classify_row(in, r, lane);
  if (!cls.located) return;
  if (!cls.proposal) {
    if (cls.j == 0 && chunk == 0 && wave == 0 && (cls.n_prop == 0 || !cls.req_ok))
      head_without_proposals(in, w, out, cls, lane);
    return;
  }

  using CH = Chunk<E, VEC>;
  const int64_t nvec = in.V / VEC;
  const int nw = in.s1 * kWavesPerBlock;
  const int g = chunk * kWavesPerBlock + wave;
  const Span sp = wave_span(nvec, nw, g);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)r * in.V;
  // Greedy rows take the same fold with scale 1: their sums are not needed for p, but a
  // NaN, a +inf or an all -inf row makes them non-finite or zero, which is the validity test.
  const bool greedy = cls.T == 0.0f;
  const float c = greedy ? 1.0f : scale_of(cls.T);
  const int64_t dvec = cls.D / VEC;
  const int de = cls.D - (int)(dvec * VEC);
  const bool holds_D = dvec >= sp.begin && dvec < sp.end;  // only this span's wave reads D's logits

  Acc at = acc_empty(), ad = acc_empty();
  int found = 0;
  float ltD = 0.0f, ldD = 0.0f;
  const int64_t step = (int64_t)U * kWave;
  CH ta[U], da[U], tb[U], db[U];

  auto fold_both = [&](const CH (&xt)[U], const CH (&xd)[U], int64_t wb) __attribute__((always_inline)) {
    const int64_t vb = wb + lane;
    fold_soft<true>(at, xt, vb, c);
    fold_soft<true>(ad, xd, vb, c);
    if (holds_D) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (vb + (int64_t)u * kWave == dvec) {
          found = 1;
          ltD = xt[u].get_dyn(de);
          ldD = xd[u].get_dyn(de);
        }
      }
    }
  };

  // Double buffering: the next batch is in flight while the current one is folded.
  if (sp.begin < sp.end) {
    load_chunks(ta, trow, sp.begin, lane, sp.end);
    load_chunks(da, drow, sp.begin, lane, sp.end);
    for (int64_t base = sp.begin;;) {
      int64_t nb = base + step;
      load_chunks(tb, trow, nb, lane, sp.end);
      load_chunks(db, drow, nb, lane, sp.end);
      mask_chunks(ta, base, lane, sp.end);
      mask_chunks(da, base, lane, sp.end);
      fold_both(ta, da, base);
      if (nb >= sp.end) break;
      base = nb;
      nb = base + step;
      load_chunks(ta, trow, nb, lane, sp.end);
      load_chunks(da, drow, nb, lane, sp.end);
      mask_chunks(tb, base, lane, sp.end);
      mask_chunks(db, base, lane, sp.end);
      fold_both(tb, db, base);
      if (nb >= sp.end) break;
      base = nb;
    }
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
  if (lane == 0) publish(&w.part1[(int64_t)r * nw + g], pp);

  // The last wave of the row merges the row; the last row of the request walks the request.
  if (!arrive_last(&w.t_row[r], (uint32_t)nw, lane)) return;
  finalize_row(in, w, r, cls, lane);
  if (!arrive_last(&w.t_req[cls.b], (uint32_t)cls.n_prop, lane)) return;
  finalize_request(in, w, out, cls, lane);
}

// ====================================================================== pass 2

__device__ __forceinline__ void add_stats(const Outputs& out, const ReqDesc& d, bool invalid) {
  if (out.stats == nullptr) return;
  unsigned long long* s = reinterpret_cast<unsigned long long*>(out.stats);
  if (invalid) {
    atomicAdd(s + 7, 1ull);
    return;
  }
  const bool tested_final = d.final_verdict == SV_ROW_REJECT || d.final_verdict == SV_ROW_NULL;
  atomicAdd(s + 0, 1ull);
  atomicAdd(s + 1, (unsigned long long)(d.k + (tested_final ? 1 : 0)));
  if (d.k) atomicAdd(s + 2, (unsigned long long)d.k);
  if (d.final_verdict == SV_ROW_REJECT) atomicAdd(s + 3, 1ull);
  if (d.final_verdict == SV_ROW_NULL) atomicAdd(s + 4, 1ull);
  if (d.final_verdict == SV_ROW_BONUS) atomicAdd(s + 5, 1ull);
  if (d.T == 0.0f) atomicAdd(s + 6, 1ull);
}

// fp64 race key of token x in a race over p, in the log domain: ln p(x) - ln E(x) up to a
// constant shared by every token of the row.
__device__ __forceinline__ double p_logkey64(double l, double T, uint32_t word) {
  return l / T - log(expo64(word));
}

// A race over p read by one wave: the rare fallback for a residual with no mass.
__device__ __forceinline__ int p_race_one_wave(const Inputs& in, const ReqDesc& d, int b, int lane) {
  Top2 t = top2_empty();
  for (int64_t x = lane; x < in.V; x += kWave) {
    const float l = logit_at(in.target, in.dtype, (int64_t)d.f * in.V + x);
    const float a = l * d.c;
    if (a > -INFINITY) {
      const uint32_t wd = race_word(in.seed, x, d.k, b);
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
      bk = p_logkey64((double)l, (double)d.T, race_word(in.seed, x, d.k, b));
      bi = x;
    }
  }
  wave_best(bk, bi);
  return bi;
}

template <typename E, int VEC, int U>
__global__ __launch_bounds__(kBlock) void pass2_kernel(Inputs in, Work w, Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t bid = blockIdx.x;
  const int b = (int)(bid / in.s2);
  const int chunk = (int)(bid % in.s2);

  if (!w.hdr->ro_valid) {
    // Broken row_offsets: the whole batch fails closed. Block (b, 0) clears an even share of the slots.
    if (chunk == 0 && wave == 0) {
      const int64_t r0 = (int64_t)b * in.R / in.B, r1 = (int64_t)(b + 1) * in.R / in.B;
      for (int64_t r = r0 + lane; r < r1; r += kWave) {
        out.tokens[r] = -1;
        if (out.diag != nullptr) out.diag[r] = untested_diag();
      }
      if (lane == 0) {
        out.accept_len[b] = -1;
        // With broken offsets, rows may have disagreed about their request, so a request
        // counter can be left part-way. Reset it for the next call.
        w.t_req[b] = 0u;
        if (out.stats != nullptr) atomicAdd(reinterpret_cast<unsigned long long*>(out.stats) + 7, 1ull);
      }
    }
    return;
  }

  const ReqDesc d = w.desc[b];
  if (d.kind == kKindInvalid || d.kind == kKindGreedyDone) {
    if (chunk == 0 && wave == 0 && lane == 0) add_stats(out, d, d.kind == kKindInvalid);
    return;
  }

  using CH = Chunk<E, VEC>;
  const int64_t nvec = in.V / VEC;
  const int nw = in.s2 * kWavesPerBlock;
  const int g = chunk * kWavesPerBlock + wave;
  const Span sp = wave_span(nvec, nw, g);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)d.f * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)d.f * in.V;
  const uint32_t k0 = seed_lo(in.seed), k1 = seed_hi(in.seed);
  const int64_t step = (int64_t)U * kWave;
  constexpr int G = VEC >= 4 ? 4 : 1;  // logits sharing one Philox block

  P2Part part{};
  part.key = -INFINITY;
  part.idx = -1;
  part.rsum = 0.0f;
  part.mref = -INFINITY;
  part.bad = 0;
  part.gidx = -1;

  if (d.kind == kKindResidual) {
    const float c = d.c, mct = d.mc_t, mcd = d.mc_d, tau = d.tau;
    const float ist = (float)(1.0 / d.s_t), isd = (float)(1.0 / d.s_d);
    float rsum = 0.0f;
    Top2 t = top2_empty();
    CH ta[U], da[U], tb[U], db[U];
    if (sp.begin < sp.end) {
      load_chunks(ta, trow, sp.begin, lane, sp.end);
      load_chunks(da, drow, sp.begin, lane, sp.end);
    }
    // Pruning bound. Pass 1 left, per wave of this row, the vector that held the wave's
    // target maximum. The best race key among those tokens is a key some token really has,
    // so the winner's key is at least that large. A token whose residual r has r / E_min
    // below half of it cannot win and draws no random number. Only tokens with
    // mu <= p/2 serve: there r = p - mu carries at most twice the fp32 error of p, so the
    // bound is exact to about 1e-6 and the factor 2 absorbs it.
    float kh = 0.0f;
    {
      const int np1 = in.s1 * kWavesPerBlock;
      for (int i = lane; i < np1 * VEC; i += kWave) {
        const int hv = w.part1[(int64_t)d.f * np1 + i / VEC].am_t;
        const int64_t x = hv >= 0 ? (int64_t)hv * VEC + i % VEC : -1;
        if (x >= 0 && x < in.V) {
          const float p = fast_exp2(fmaf(logit_at(in.target, in.dtype, (int64_t)d.f * in.V + x), c, -mct)) * ist;
          const float q = fast_exp2(fmaf(logit_at(in.draft, in.dtype, (int64_t)d.f * in.V + x), c, -mcd)) * isd;
          const float mu = q >= tau ? q : 0.0f;
          if (p > 0.0f && mu <= 0.5f * p)
            kh = fmaxf(kh, (float)((double)(p - mu) / expo64(race_word(in.seed, x, d.k, b))));
        }
      }
      kh = wave_max(kh);
    }
    const float pthr = kh * (float)(kEminLow * 0.5);
    auto fold_res = [&](const CH (&xt)[U], const CH (&xd)[U], int64_t v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t x0 = (v0 + (int64_t)u * kWave) * VEC;
#pragma unroll
        for (int gg = 0; gg < VEC; gg += G) {
          float rv[G];
          bool any = false;
#pragma unroll
          for (int e = 0; e < G; ++e) {
            const float p = fast_exp2(fmaf(xt[u].get(gg + e), c, -mct)) * ist;
            const float q = fast_exp2(fmaf(xd[u].get(gg + e), c, -mcd)) * isd;
            const float mu = q >= tau ? q : 0.0f;
            const float r = fmaxf(p - mu, 0.0f);
            rsum += r;
            rv[e] = r;
            any |= (r > 0.0f && r >= pthr);
          }
          if (any) {
            const int64_t xg = x0 + gg;
            const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)d.k, (uint32_t)b, k0, k1);
#pragma unroll
            for (int e = 0; e < G; ++e) {
              if (rv[e] > 0.0f && rv[e] >= pthr) {
                const int64_t x = xg + e;
                const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, (int)(x & 3));
                top2_push(t, rv[e] / expo32(wd), (int)x, xt[u].get(gg + e), xd[u].get(gg + e));
              }
            }
          }
        }
      }
    };
    if (sp.begin < sp.end) {
      for (int64_t base = sp.begin;;) {
        int64_t nb = base + step;
        load_chunks(tb, trow, nb, lane, sp.end);
        load_chunks(db, drow, nb, lane, sp.end);
        mask_chunks(ta, base, lane, sp.end);
        mask_chunks(da, base, lane, sp.end);
        fold_res(ta, da, base + lane);
        if (nb >= sp.end) break;
        base = nb;
        nb = base + step;
        load_chunks(ta, trow, nb, lane, sp.end);
        load_chunks(da, drow, nb, lane, sp.end);
        mask_chunks(tb, base, lane, sp.end);
        mask_chunks(db, base, lane, sp.end);
        fold_res(tb, db, base + lane);
        if (nb >= sp.end) break;
        base = nb;
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
                            (double)mct, (double)mcd, d.s_t, d.s_d, (double)tau, race_word(in.seed, x, d.k, b));
        bi = x;
      }
    }
    wave_best(bk, bi);
    part.key = bk;
    part.idx = bi == INT32_MAX ? -1 : bi;
  } else {
    // Bonus row (race over p) or greedy bonus row (argmax). Pass 1 never read it, so it is validated here.
    const bool race = d.kind == kKindBonus;
    const float c = d.c;
    Acc a = acc_empty();
    int bad = 0;
    Top2 t = top2_empty();
    float wbest = -INFINITY;  // best log2 key the wave has seen so far
    CH ta[U], tb[U];
    auto fold_bonus = [&](const CH (&xt)[U], int64_t v0) __attribute__((always_inline)) {
      if (race) fold_max<false>(a, xt, v0, bad);  // max and NaN / +inf check
      else fold_max<true>(a, xt, v0, bad);       // ... and the lowest index of the max
      if (race) {
        float lbest = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t x0 = (v0 + (int64_t)u * kWave) * VEC;
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
              const int64_t xg = x0 + gg;
              const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)d.k, (uint32_t)b, k0, k1);
#pragma unroll
              for (int e = 0; e < G; ++e) {
                if (av[e] + 25.0f >= wbest) {
                  const int64_t x = xg + e;
                  const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, (int)(x & 3));
                  const float key = av[e] - __log2f(expo32(wd));
                  lbest = fmaxf(lbest, key);
                  top2_push(t, key, (int)x, xt[u].get(gg + e), 0.0f);
                }
              }
            }
          }
        }
        wbest = fmaxf(wbest, wave_max(lbest));
      }
    };
    if (sp.begin < sp.end) {
      load_chunks(ta, trow, sp.begin, lane, sp.end);
      for (int64_t base = sp.begin;;) {
        int64_t nb = base + step;
        load_chunks(tb, trow, nb, lane, sp.end);
        mask_chunks(ta, base, lane, sp.end);
        fold_bonus(ta, base + lane);
        if (nb >= sp.end) break;
        base = nb;
        nb = base + step;
        load_chunks(ta, trow, nb, lane, sp.end);
        mask_chunks(tb, base, lane, sp.end);
        fold_bonus(tb, base + lane);
        if (nb >= sp.end) break;
        base = nb;
      }
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
          bk = p_logkey64((double)(lane == 0 ? t.a1 : t.a2), (double)d.T, race_word(in.seed, x, d.k, b));
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
  if (d.kind == kKindResidual) {
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
    else token = p_race_one_wave(in, d, b, lane);  // residual with no mass: race over p
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
    if (d.kind == kKindGreedyBonus) {
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

  const int lo = in.ro[b];
  const int n = in.ro[b + 1] - lo;
  for (int j = lane; j < n; j += kWave) {
    const int r = lo + j;
    out.tokens[r] = invalid ? -1 : (j < d.k ? in.dt[r] : (j == d.k ? token : -1));
    if (out.diag != nullptr) {
      if (invalid) out.diag[r] = untested_diag();
      else if (j == d.k && d.kind == kKindResidual) out.diag[r].resid_mass = resid;
    }
  }
  if (lane == 0) {
    out.accept_len[b] = invalid ? -1 : d.k;
    add_stats(out, d, invalid);
  }
}

// ====================================================================== launch

// Zero the ticket arrays. Every ticket wraps back to zero when a call completes, so this
// runs only when a workspace is first seen or its layout changes (see counters_ready).
__global__ __launch_bounds__(kBlock) void clear_counters_kernel(uint32_t* t, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) t[i] = 0u;
}

// Per (device, workspace address): the counter layout of the last call enqueued on it.
struct LayoutSeen {
  int device;
  const void* ws;
  size_t off_ticket_row, total;
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
  if (slot >= 0 && g_layout[slot].off_ticket_row == p.off_ticket_row && g_layout[slot].total == p.total)
    return hipSuccess;
  const int64_t n = (int64_t)(p.total - p.off_ticket_row) / 4;  // the three ticket arrays sit at the end
  const int64_t blocks = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(kBlock), 0,
                     stream, reinterpret_cast<uint32_t*>(ws + p.off_ticket_row), n);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (slot < 0) slot = g_layout_n < 64 ? g_layout_n++ : (int)(reinterpret_cast<uintptr_t>(ws) / 256 % 64);
  g_layout[slot] = LayoutSeen{dev, ws, p.off_ticket_row, p.total};
  return hipSuccess;
}

template <typename E, int VEC>
hipError_t launch_pair(const Plan& p, const Inputs& in, const Work& w, const Outputs& out,
                       hipStream_t stream, hipEvent_t const* ev) {
  constexpr int U = VEC == 1 ? 16 : 4;
  hipError_t err = hipSuccess;
  if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
  const dim3 block(kBlock);
  hipLaunchKernelGGL((pass1_kernel<E, VEC, U>), dim3((unsigned)((int64_t)p.R * p.s1)), block, 0, stream, in, w, out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
  hipLaunchKernelGGL((pass2_kernel<E, VEC, U>), dim3((unsigned)((int64_t)p.B * p.s2)), block, 0, stream, in, w, out);
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
  Inputs in{target, draft, draft_tokens, row_offsets, temperature, tau, seed,
            p.B, p.R, p.V, p.dtype, p.s1, p.s2};
  Work w{reinterpret_cast<WsHeader*>(ws + p.off_hdr), reinterpret_cast<P1Part*>(ws + p.off_part1),
         reinterpret_cast<RowRec*>(ws + p.off_rec), reinterpret_cast<ReqDesc*>(ws + p.off_desc),
         reinterpret_cast<P2Part*>(ws + p.off_part2), reinterpret_cast<uint32_t*>(ws + p.off_ticket_row),
         reinterpret_cast<uint32_t*>(ws + p.off_ticket_req), reinterpret_cast<uint32_t*>(ws + p.off_ticket2)};
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
