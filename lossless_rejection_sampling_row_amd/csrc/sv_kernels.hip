// sv_kernels.hip - the verify sampler's two kernels and the exported C-ABI calls.
//
// Pass 1 (one workgroup per (row, V-chunk)) streams the target and draft
// logits of every proposal row once. Each wave reduces its slice to softmax
// statistics (max, sum of exp2 against that max) and the lowest-index argmax.
// It writes a 32-byte partial. The last wave to finish a row (atomic ticket)
// merges the row's partials in fp64 and runs the accept test. That test
// follows Strata PR #3416 "[Engine] Preserve target probabilities in gated
// MTP", section Approach, with the accept form of mlxcel PR #992, section
// What changed.
//
// Pass 2 (one workgroup per (request, V-chunk)) walks the request's verdicts
// to its first non-accepted row k. It then draws the request's last token from
// the row that ended it:
//  - a residual draw from (p - mu)+ on a rejected or NULL row;
//  - a bonus draw from p on the last row or a row with no proposal;
//  - the greedy argmax at temperature 0.
// The draw is an exponential race, argmax_x w_x / E_x, with ties going to the
// lower index.
//  - Each wave keeps its two best fp32 keys.
//  - Elements that provably cannot win are pruned before any random number is
//    drawn.
//  - The request's last wave (atomic ticket) re-evaluates every candidate in
//    fp64 and writes the outputs.
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
  uint32_t* ticket1;
  P2Part* part2;
  uint32_t* ticket2;
};

struct Outputs {
  int32_t* tokens;
  int32_t* accept_len;
  sv_row_diag* diag;
  sv_batch_stats* stats;
};

__device__ __forceinline__ uint32_t seed_lo(uint64_t s) { return (uint32_t)s; }
__device__ __forceinline__ uint32_t seed_hi(uint64_t s) { return (uint32_t)(s >> 32); }

// ====================================================================== pass 1

struct RowCls {
  bool ok;   // a proposal row the method may test
  int b, j, n, lo, D;
  float T, tau;
};

// Locate row r's request and decide whether it is a proposal row: not the
// request's last row, and every drafted token of the request up to and
// including r lies in [0, V). Rows behind a "no proposal" row are never tested.
// Every index stays in bounds whatever row_offsets holds. A broken batch is
// caught by block 0's check and failed closed in pass 2.
__device__ RowCls classify_row(const Inputs& in, int r, int lane) {
  RowCls c{};
  c.ok = false;
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
  if (!(0 <= lo && lo <= r && r < hi && hi <= in.R)) return c;
  const int n = hi - lo, j = r - lo;
  if (j == n - 1) return c;  // bonus row: pass 2's business
  const float T = in.temp[b], tau = in.tau[b];
  if (!temperature_ok(T) || __builtin_isnan(tau)) return c;
  bool stop = false;
  for (int base = 0; base <= j; base += kWave) {
    const int i = base + lane;
    bool badtok = false;
    if (i <= j) {
      const int D = in.dt[lo + i];
      badtok = D < 0 || D >= in.V;
    }
    if (__any(badtok)) { stop = true; break; }
  }
  if (stop) return c;
  c.ok = true;
  c.b = b;
  c.j = j;
  c.n = n;
  c.lo = lo;
  c.D = in.dt[r];
  c.T = T;
  c.tau = tau;
  return c;
}

struct WaveStat {
  float m, s;
  int am, bad;
};

// Softmax statistics of one wave's slice of one array. Each lane holds NV
// chunks of VEC logits, at vector indices v0 + k*64 + lane. Out-of-range
// chunks hold -inf.
template <bool GREEDY, bool ARGMAX, class CH, int NV>
__device__ __forceinline__ WaveStat slice_stats(const CH (&x)[NV], int64_t v0, int lane, float c) {
  constexpr int VEC = CH::kVec;
  float vmax[NV];
  int bad = 0;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float m = x[k].get(0);
#pragma unroll
    for (int e = 1; e < VEC; ++e) m = fmaxf(m, x[k].get(e));
    vmax[k] = m;
    if (GREEDY) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = x[k].get(e);
        bad |= (int)(__builtin_isnan(v) || v == INFINITY);
      }
    }
  }
  float mx = vmax[0];
#pragma unroll
  for (int k = 1; k < NV; ++k) mx = fmaxf(mx, vmax[k]);
  const float wm = wave_max(mx);

  WaveStat st{wm, 0.0f, -1, 0};
  if (ARGMAX) {
    int idx = INT32_MAX;
    if (mx == wm && wm != -INFINITY) {  // only lanes that hold the wave maximum scan
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          if (idx == INT32_MAX && x[k].get(e) == wm) idx = (int)((v0 + (int64_t)k * kWave + lane) * VEC + e);
        }
      }
    }
    idx = wave_min(idx);
    st.am = idx == INT32_MAX ? -1 : idx;
  }
  if (GREEDY) {
    st.bad = wave_or(bad);
  } else {
    const float mct = ref_of(mx, c);
    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += fast_exp2(fmaf(x[k].get(e), c, -mct));
      acc[k] = s;
    }
    float s = acc[0];
#pragma unroll
    for (int k = 1; k < NV; ++k) s += acc[k];
    const float mcw = ref_of(wm, c);
    const float term = (s != 0.0f) ? s * fast_exp2(mct - mcw) : 0.0f;
    st.s = wave_sum(term);
  }
  return st;
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

// Merge a row's partials (fixed order, fp64 sums) and test the drafted token.
__device__ void finalize_row(const Inputs& in, const Work& w, const Outputs& out, int r,
                             const RowCls& cls, int lane) {
  const int np = in.s1 * kWavesPerBlock;
  const P1Part* pp = w.part1 + (int64_t)r * np;
  const bool greedy = cls.T == 0.0f;
  const float c = greedy ? 0.0f : scale_of(cls.T);

  float mt = -INFINITY, md = -INFINITY;
  int bad = 0;
  for (int i = lane; i < np; i += kWave) {
    const P1Part q = read_p1(pp + i);
    mt = fmaxf(mt, q.m_t);
    md = fmaxf(md, q.m_d);
    bad |= q.bad;
  }
  mt = wave_max(mt);
  md = wave_max(md);
  bad = wave_or(bad);
  int it = INT32_MAX, id = INT32_MAX;
  double st = 0.0, sd = 0.0;
  const float mct = ref_of(mt, c), mcd = ref_of(md, c);
  for (int i = lane; i < np; i += kWave) {
    const P1Part q = read_p1(pp + i);
    if (q.m_t == mt && q.am_t >= 0) it = min(it, q.am_t);
    if (q.m_d == md && q.am_d >= 0) id = min(id, q.am_d);
    if (!greedy) {
      if (q.s_t != 0.0f) st += (double)q.s_t * exp2((double)ref_of(q.m_t, c) - (double)mct);
      if (q.s_d != 0.0f) sd += (double)q.s_d * exp2((double)ref_of(q.m_d, c) - (double)mcd);
    }
  }
  it = wave_min(it);
  id = wave_min(id);
  st = wave_sum(st);
  sd = wave_sum(sd);

  const int D = cls.D;
  int verdict;
  float pD, qD, muD, u = NAN;
  if (greedy) {
    const bool valid = !bad && mt != -INFINITY && md != -INFINITY;
    pD = (D == it) ? 1.0f : 0.0f;
    qD = (D == id) ? 1.0f : 0.0f;
    const bool offered = qD >= cls.tau;
    muD = offered ? qD : 0.0f;
    // p(D) is 0 or 1 and mu(D) <= 1: u*mu(D) < p(D) holds for every u iff p(D) = 1.
    verdict = !valid ? kRowInvalid : !offered ? SV_ROW_NULL : (pD == 1.0f ? SV_ROW_ACCEPT : SV_ROW_REJECT);
  } else {
    const bool valid = __builtin_isfinite(mt) && __builtin_isfinite(md) && __builtin_isfinite(st) &&
                       st > 0.0 && __builtin_isfinite(sd) && sd > 0.0;
    const int64_t at = (int64_t)r * in.V + D;
    const double lt = (double)logit_at(in.target, in.dtype, at);
    const double ld = (double)logit_at(in.draft, in.dtype, at);
    const double p = exp2(lt * (double)c - (double)mct) / st;
    const double q = exp2(ld * (double)c - (double)mcd) / sd;
    const bool offered = q >= (double)cls.tau;
    const double mu = offered ? q : 0.0;
    pD = (float)p;
    qD = (float)q;
    muD = (float)mu;
    if (!valid) {
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
    rr.s_t = st;
    rr.s_d = sd;
    rr.p_D = pD;
    rr.q_D = qD;
    rr.mu_D = muD;
    rr.u = u;
    w.rec[r] = rr;
    if (out.diag != nullptr) {
      sv_row_diag dg;
      dg.p_D = pD;
      dg.q_D = qD;
      dg.mu_D = muD;
      dg.u = u;
      dg.resid_mass = NAN;
      dg.verdict = verdict == kRowInvalid ? SV_ROW_UNTESTED : verdict;
      dg.pad0 = dg.pad1 = 0;
      out.diag[r] = dg;
    }
  }
}

template <typename E, int VEC, int EPT>
__global__ __launch_bounds__(kBlock) void pass1_kernel(Inputs in, Work w, Outputs out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t bid = blockIdx.x;
  if (bid == 0) block0_duties(in, w, out);
  const int r = (int)(bid / in.s1);
  const int chunk = (int)(bid % in.s1);
  const RowCls cls = classify_row(in, r, lane);
  if (!cls.ok) return;

  constexpr int NV = EPT / VEC;
  using CH = Chunk<E, VEC>;
  const int64_t nvec = in.V / VEC;
  const int64_t v0 = ((int64_t)chunk * kWavesPerBlock + wave) * (NV * kWave);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)r * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)r * in.V;
  CH xt[NV], xd[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int64_t vi = v0 + (int64_t)k * kWave + lane;
    if (vi < nvec) {
      xt[k].load(trow + vi * VEC);
      xd[k].load(drow + vi * VEC);
    } else {
      xt[k].fill_neg_inf();
      xd[k].fill_neg_inf();
    }
  }
  WaveStat a, d;
  if (cls.T == 0.0f) {
    a = slice_stats<true, true>(xt, v0, lane, 0.0f);
    d = slice_stats<true, true>(xd, v0, lane, 0.0f);
  } else {
    const float c = scale_of(cls.T);
    a = slice_stats<false, true>(xt, v0, lane, c);
    d = slice_stats<false, false>(xd, v0, lane, c);
  }
  if (lane == 0) {
    P1Part pp;
    pp.m_t = a.m;
    pp.s_t = a.s;
    pp.m_d = d.m;
    pp.s_d = d.s;
    pp.am_t = a.am;
    pp.am_d = d.am;
    pp.bad = a.bad | d.bad;
    pp.pad = 0;
    publish(&w.part1[((int64_t)r * in.s1 + chunk) * kWavesPerBlock + wave], pp);
  }
  // The last wave of the row merges every wave's partial.
  if (!arrive_last(&w.ticket1[r], (uint32_t)in.s1 * kWavesPerBlock, lane)) return;
  finalize_row(in, w, out, r, cls, lane);
}

// ====================================================================== pass 2

enum Kind : int { kInvalid = 0, kGreedyDone = 1, kResidual = 2, kBonus = 3, kGreedyBonus = 4 };

struct ReqCls {
  int kind;
  int lo, n, k, f;
  int final_verdict;
  float T, tau;
};

// Walk request b's rows in order to its first row that is not accepted.
__device__ ReqCls walk_request(const Inputs& in, const Work& w, int b, int lane) {
  ReqCls q{};
  q.lo = in.ro[b];
  q.n = in.ro[b + 1] - q.lo;
  q.T = in.temp[b];
  q.tau = in.tau[b];
  q.kind = kInvalid;
  if (!temperature_ok(q.T) || __builtin_isnan(q.tau)) return q;
  q.k = q.n - 1;
  for (int base = 0; base < q.n; base += kWave) {
    const int j = base + lane;
    bool stop = false;
    if (j < q.n) {
      const int D = in.dt[q.lo + j];
      const bool noprop = (j == q.n - 1) || D < 0 || D >= in.V;
      stop = noprop || w.rec[q.lo + j].verdict != SV_ROW_ACCEPT;
    }
    const uint64_t m = __ballot(stop);
    if (m != 0) {
      q.k = base + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  q.f = q.lo + q.k;
  const int D = in.dt[q.f];
  const bool greedy = q.T == 0.0f;
  if (q.k == q.n - 1 || D < 0 || D >= in.V) {
    q.final_verdict = SV_ROW_BONUS;
    q.kind = greedy ? kGreedyBonus : kBonus;
  } else {
    const int v = w.rec[q.f].verdict;
    q.final_verdict = v;
    if (v == SV_ROW_REJECT || v == SV_ROW_NULL) q.kind = greedy ? kGreedyDone : kResidual;
    else q.kind = kInvalid;
  }
  return q;
}

// Write request b's outputs and diagnostics (one wave).
__device__ void emit_request(const Inputs& in, const Work& w, const Outputs& out, int b,
                             const ReqCls& q, bool invalid, int token, float resid, int lane) {
  for (int j = lane; j < q.n; j += kWave) {
    const int r = q.lo + j;
    int t = -1;
    if (!invalid) t = j < q.k ? in.dt[r] : (j == q.k ? token : -1);
    out.tokens[r] = t;
    if (out.diag != nullptr) {
      if (invalid || j > q.k) {
        sv_row_diag dg;
        dg.p_D = dg.q_D = dg.mu_D = dg.u = dg.resid_mass = NAN;
        dg.verdict = SV_ROW_UNTESTED;
        dg.pad0 = dg.pad1 = 0;
        out.diag[r] = dg;
      } else if (j == q.k) {
        if (q.final_verdict == SV_ROW_BONUS) {
          sv_row_diag dg;
          dg.p_D = dg.q_D = dg.mu_D = dg.u = dg.resid_mass = NAN;
          dg.verdict = SV_ROW_BONUS;
          dg.pad0 = dg.pad1 = 0;
          out.diag[r] = dg;
        } else {
          out.diag[r].resid_mass = resid;
        }
      }
    }
  }
  if (lane == 0) {
    out.accept_len[b] = invalid ? -1 : q.k;
    if (out.stats != nullptr) {
      unsigned long long* s = reinterpret_cast<unsigned long long*>(out.stats);
      if (invalid) {
        atomicAdd(s + 7, 1ull);
      } else {
        const bool tested_final = q.final_verdict == SV_ROW_REJECT || q.final_verdict == SV_ROW_NULL;
        atomicAdd(s + 0, 1ull);
        atomicAdd(s + 1, (unsigned long long)(q.k + (tested_final ? 1 : 0)));
        if (q.k) atomicAdd(s + 2, (unsigned long long)q.k);
        if (q.final_verdict == SV_ROW_REJECT) atomicAdd(s + 3, 1ull);
        if (q.final_verdict == SV_ROW_NULL) atomicAdd(s + 4, 1ull);
        if (q.final_verdict == SV_ROW_BONUS) atomicAdd(s + 5, 1ull);
        if (q.T == 0.0f) atomicAdd(s + 6, 1ull);
      }
    }
  }
}

// fp64 race key of token x on a residual row: (p - mu)+ / E.
__device__ double residual_key64(const Inputs& in, const RowRec& rr, const ReqCls& q, int b, int x) {
  const int64_t at = (int64_t)q.f * in.V + x;
  const double lt = (double)logit_at(in.target, in.dtype, at);
  const double ld = (double)logit_at(in.draft, in.dtype, at);
  const double p = exp2(lt * (double)rr.c - (double)rr.mc_t) / rr.s_t;
  const double qq = exp2(ld * (double)rr.c - (double)rr.mc_d) / rr.s_d;
  const double mu = qq >= (double)q.tau ? qq : 0.0;
  const double r = p - mu;
  if (!(r > 0.0)) return 0.0;
  return r / expo64(race_word(in.seed, x, q.k, b));
}

// fp64 race key of token x on a p-race, up to the common factor exp(-M/T)/sum.
__device__ double p_key64(const Inputs& in, const ReqCls& q, int b, int x, double M) {
  const int64_t at = (int64_t)q.f * in.V + x;
  const double l = (double)logit_at(in.target, in.dtype, at);
  return exp((l - M) / (double)q.T) / expo64(race_word(in.seed, x, q.k, b));
}

// A race over p read by one wave: the rare fallback for a residual with no mass.
__device__ int p_race_one_wave(const Inputs& in, const RowRec& rr, const ReqCls& q, int b, int lane) {
  Top2 t = top2_empty();
  for (int64_t x = lane; x < in.V; x += kWave) {
    const float l = logit_at(in.target, in.dtype, (int64_t)q.f * in.V + x);
    const float wgt = fast_exp2(fmaf(l, rr.c, -rr.mc_t));
    if (wgt > 0.0f) top2_push(t, wgt / expo32(race_word(in.seed, x, q.k, b)), (int)x);
  }
  wave_top2(t);
  double bk = -1.0;
  int bi = INT32_MAX;
  if (lane < 2) {
    const int x = lane == 0 ? t.i1 : t.i2;
    if (x != INT32_MAX) {
      bk = p_key64(in, q, b, x, (double)rr.m_t);
      bi = x;
    }
  }
  wave_best(bk, bi);
  return bi;
}

template <typename E, int VEC, int EPT>
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
        if (out.diag != nullptr) {
          sv_row_diag dg;
          dg.p_D = dg.q_D = dg.mu_D = dg.u = dg.resid_mass = NAN;
          dg.verdict = SV_ROW_UNTESTED;
          dg.pad0 = dg.pad1 = 0;
          out.diag[r] = dg;
        }
      }
      if (lane == 0) {
        out.accept_len[b] = -1;
        if (out.stats != nullptr) atomicAdd(reinterpret_cast<unsigned long long*>(out.stats) + 7, 1ull);
      }
    }
    return;
  }

  const ReqCls q = walk_request(in, w, b, lane);
  if (q.kind == kInvalid || q.kind == kGreedyDone) {
    if (chunk == 0 && wave == 0) {
      const int tok = q.kind == kGreedyDone ? w.rec[q.f].am_t : -1;
      float resid = NAN;
      if (q.kind == kGreedyDone) {  // one-hot residual: empty iff the gated draft argmax is the target argmax
        const RowRec& rr = w.rec[q.f];
        resid = (rr.am_t == rr.am_d && 1.0f >= q.tau) ? 0.0f : 1.0f;
      }
      emit_request(in, w, out, b, q, q.kind == kInvalid, tok, resid, lane);
    }
    return;
  }

  constexpr int NV = EPT / VEC;
  using CH = Chunk<E, VEC>;
  const int64_t nvec = in.V / VEC;
  const int64_t v0 = ((int64_t)chunk * kWavesPerBlock + wave) * (NV * kWave);
  const E* trow = reinterpret_cast<const E*>(in.target) + (int64_t)q.f * in.V;
  const E* drow = reinterpret_cast<const E*>(in.draft) + (int64_t)q.f * in.V;
  const uint32_t k0 = seed_lo(in.seed), k1 = seed_hi(in.seed);

  P2Part part;
  part.k1 = part.k2 = -1.0f;
  part.i1 = part.i2 = -1;
  part.rsum = 0.0f;
  part.mref = -INFINITY;
  part.bad = 0;
  part.gidx = -1;

  CH xt[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int64_t vi = v0 + (int64_t)k * kWave + lane;
    if (vi < nvec) xt[k].load(trow + vi * VEC); else xt[k].fill_neg_inf();
  }

  if (q.kind == kResidual) {
    CH xd[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t vi = v0 + (int64_t)k * kWave + lane;
      if (vi < nvec) xd[k].load(drow + vi * VEC); else xd[k].fill_neg_inf();
    }
    const RowRec rr = w.rec[q.f];
    // Pruning bound from the row's pass-1 argmax hints. The largest fp64 key among them
    // is a key some token really has, so the winner's key is at least that large. A
    // token whose residual r satisfies r / E_min < K/2 cannot win: it needs no random number.
    double kh = 0.0;
    const int np1 = in.s1 * kWavesPerBlock;
    for (int i = lane; i < np1; i += kWave) {
      const int x = w.part1[(int64_t)q.f * np1 + i].am_t;
      if (x >= 0) kh = fmax(kh, residual_key64(in, rr, q, b, x));
    }
    kh = wave_max(kh);
    const float pthr = (float)(kh * kEminLow * 0.5);
    const float c = rr.c, mct = rr.mc_t, mcd = rr.mc_d;
    const float ist = (float)(1.0 / rr.s_t), isd = (float)(1.0 / rr.s_d);
    const float tau = q.tau;
    float rsum = 0.0f;
    Top2 t = top2_empty();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t x0 = (v0 + (int64_t)k * kWave + lane) * VEC;
      constexpr int G = VEC >= 4 ? 4 : 1;
#pragma unroll
      for (int g = 0; g < VEC; g += G) {
        float rv[G];
        bool any = false;
#pragma unroll
        for (int e = 0; e < G; ++e) {
          const float p = fast_exp2(fmaf(xt[k].get(g + e), c, -mct)) * ist;
          const float qv = fast_exp2(fmaf(xd[k].get(g + e), c, -mcd)) * isd;
          const float mu = qv >= tau ? qv : 0.0f;
          const float r = fmaxf(p - mu, 0.0f);
          rsum += r;
          rv[e] = r;
          any |= (r > 0.0f && r >= pthr);
        }
        if (any) {
          const int64_t xg = x0 + g;
          const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)q.k, (uint32_t)b, k0, k1);
#pragma unroll
          for (int e = 0; e < G; ++e) {
            if (rv[e] > 0.0f && rv[e] >= pthr) {
              const int64_t x = xg + e;
              const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, (int)(x & 3));
              top2_push(t, rv[e] / expo32(wd), (int)x);
            }
          }
        }
      }
    }
    wave_top2(t);
    part.rsum = wave_sum(rsum);
    part.k1 = t.k1;
    part.k2 = t.k2;
    part.i1 = t.i1 == INT32_MAX ? -1 : t.i1;
    part.i2 = t.i2 == INT32_MAX ? -1 : t.i2;
  } else {
    // Bonus row (p-race) or greedy bonus row (argmax). Pass 1 never read it, so it is validated here.
    float vmax[NV];
    int bad = 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float m = xt[k].get(0);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = xt[k].get(e);
        m = fmaxf(m, v);
        bad |= (int)(__builtin_isnan(v) || v == INFINITY);
      }
      vmax[k] = m;
    }
    float mx = vmax[0];
#pragma unroll
    for (int k = 1; k < NV; ++k) mx = fmaxf(mx, vmax[k]);
    const float wm = wave_max(mx);
    int idx = INT32_MAX;
    if (mx == wm && wm != -INFINITY) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          if (idx == INT32_MAX && xt[k].get(e) == wm) idx = (int)((v0 + (int64_t)k * kWave + lane) * VEC + e);
        }
      }
    }
    idx = wave_min(idx);
    part.bad = wave_or(bad);
    part.mref = wm;
    part.gidx = idx == INT32_MAX ? -1 : idx;
    if (q.kind == kBonus && wm != -INFINITY) {
      // In this wave's frame the maximum token has weight 1 and key 1/E(xm). A token with
      // weight 2^a can only beat it if 2^a / E_min >= 1/E(xm); keep a factor 2 of slack.
      const float c = scale_of(q.T);
      const float mcw = wm * c;
      const double kw = 1.0 / expo64(race_word(in.seed, idx, q.k, b));
      const float athr = (float)log2(kw * kEminLow * 0.5);
      Top2 t = top2_empty();
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int64_t x0 = (v0 + (int64_t)k * kWave + lane) * VEC;
        constexpr int G = VEC >= 4 ? 4 : 1;
#pragma unroll
        for (int g = 0; g < VEC; g += G) {
          float av[G];
          bool any = false;
#pragma unroll
          for (int e = 0; e < G; ++e) {
            av[e] = fmaf(xt[k].get(g + e), c, -mcw);
            any |= av[e] >= athr;
          }
          if (any) {
            const int64_t xg = x0 + g;
            const Philox4 ph = philox4x32_10((uint32_t)(xg >> 2), kTagRace, (uint32_t)q.k, (uint32_t)b, k0, k1);
#pragma unroll
            for (int e = 0; e < G; ++e) {
              if (av[e] >= athr) {
                const int64_t x = xg + e;
                const uint32_t wd = G == 4 ? word_of(ph, e) : word_of(ph, (int)(x & 3));
                top2_push(t, fast_exp2(av[e]) / expo32(wd), (int)x);
              }
            }
          }
        }
      }
      wave_top2(t);
      part.k1 = t.k1;
      part.k2 = t.k2;
      part.i1 = t.i1 == INT32_MAX ? -1 : t.i1;
      part.i2 = t.i2 == INT32_MAX ? -1 : t.i2;
    }
  }

  const int np2 = in.s2 * kWavesPerBlock;
  if (lane == 0) publish(&w.part2[(int64_t)b * np2 + (int64_t)chunk * kWavesPerBlock + wave], part);
  if (!arrive_last(&w.ticket2[b], (uint32_t)np2, lane)) return;

  // ---- the request's last wave: merge the partials and emit
  const P2Part* pp = w.part2 + (int64_t)b * np2;
  bool invalid = false;
  int token = -1;
  float resid = NAN;
  if (q.kind == kResidual) {
    const RowRec rr = w.rec[q.f];
    double R = 0.0, bk = -1.0;
    int bi = INT32_MAX;
    for (int i = lane; i < np2; i += kWave) {
      const P2Part c2 = read_p2(pp + i);
      R += (double)c2.rsum;
      if (c2.i1 >= 0) {
        const double k = residual_key64(in, rr, q, b, c2.i1);
        if (beats(k, c2.i1, bk, bi)) { bk = k; bi = c2.i1; }
      }
      if (c2.i2 >= 0) {
        const double k = residual_key64(in, rr, q, b, c2.i2);
        if (beats(k, c2.i2, bk, bi)) { bk = k; bi = c2.i2; }
      }
    }
    const int np1 = in.s1 * kWavesPerBlock;
    for (int i = lane; i < np1; i += kWave) {
      const int x = w.part1[(int64_t)q.f * np1 + i].am_t;
      if (x >= 0) {
        const double k = residual_key64(in, rr, q, b, x);
        if (beats(k, x, bk, bi)) { bk = k; bi = x; }
      }
    }
    R = wave_sum(R);
    wave_best(bk, bi);
    resid = (float)R;
    if (R > 0.0 && bk > 0.0) token = bi;
    else token = p_race_one_wave(in, rr, q, b, lane);  // residual with no mass: race over p
  } else {
    float M = -INFINITY;
    int bad = 0;
    for (int i = lane; i < np2; i += kWave) {
      const P2Part c2 = read_p2(pp + i);
      M = fmaxf(M, c2.mref);
      bad |= c2.bad;
    }
    M = wave_max(M);
    bad = wave_or(bad);
    invalid = bad != 0 || M == -INFINITY;
    if (!invalid) {
      double bk = -1.0;
      int bi = INT32_MAX;
      for (int i = lane; i < np2; i += kWave) {
        const P2Part c2 = read_p2(pp + i);
        if (q.kind == kGreedyBonus) {
          if (c2.mref == M && c2.gidx >= 0 && c2.gidx < bi) bi = c2.gidx;
        } else {
          if (c2.i1 >= 0) {
            const double k = p_key64(in, q, b, c2.i1, (double)M);
            if (beats(k, c2.i1, bk, bi)) { bk = k; bi = c2.i1; }
          }
          if (c2.i2 >= 0) {
            const double k = p_key64(in, q, b, c2.i2, (double)M);
            if (beats(k, c2.i2, bk, bi)) { bk = k; bi = c2.i2; }
          }
        }
      }
      if (q.kind == kGreedyBonus) bi = wave_min(bi);
      else wave_best(bk, bi);
      token = bi;
    }
  }
  emit_request(in, w, out, b, q, invalid, token, resid, lane);
}

// ====================================================================== launch

// Zero the two ticket arrays. Both tickets wrap back to zero when a call
// completes, so this runs only when a workspace is first seen or its layout
// changes (see counters_ready).
__global__ __launch_bounds__(kBlock) void clear_counters_kernel(uint32_t* t1, int64_t n1, uint32_t* t2,
                                                               int64_t n2) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n1; i += stride) t1[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n2; i += stride) t2[i] = 0u;
}

// Per (device, workspace address): the counter layout of the last call enqueued on it.
struct LayoutSeen {
  int device;
  const void* ws;
  size_t off_ticket1, off_ticket2;
  int32_t R, B;
};

static std::mutex g_layout_mu;
static LayoutSeen g_layout[64];
static int g_layout_n = 0;

// Make sure the workspace's ticket arrays hold zeros before pass 1 runs: clear them when
// this (device, workspace) pair was not seen with this counter layout by the previous call.
static hipError_t counters_ready(const Plan& p, char* ws, hipStream_t stream) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_layout_mu);
  int slot = -1;
  for (int i = 0; i < g_layout_n; ++i)
    if (g_layout[i].device == dev && g_layout[i].ws == ws) slot = i;
  if (slot >= 0 && g_layout[slot].off_ticket1 == p.off_ticket1 && g_layout[slot].off_ticket2 == p.off_ticket2 &&
      g_layout[slot].R == p.R && g_layout[slot].B == p.B)
    return hipSuccess;
  const int64_t n = p.R > p.B ? p.R : p.B;
  const unsigned grid = (unsigned)((n + kBlock - 1) / kBlock < 1024 ? (n + kBlock - 1) / kBlock : 1024);
  hipLaunchKernelGGL(clear_counters_kernel, dim3(grid), dim3(kBlock), 0, stream,
                     reinterpret_cast<uint32_t*>(ws + p.off_ticket1), (int64_t)p.R,
                     reinterpret_cast<uint32_t*>(ws + p.off_ticket2), (int64_t)p.B);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (slot < 0) {
    slot = g_layout_n < 64 ? g_layout_n++ : (int)(reinterpret_cast<uintptr_t>(ws) / 256 % 64);
  }
  g_layout[slot] = LayoutSeen{dev, ws, p.off_ticket1, p.off_ticket2, p.R, p.B};
  return hipSuccess;
}


// Logits each lane holds per array: 128 bytes in pass 1, 32 bytes in pass 2.
template <typename E> struct Ept;
template <> struct Ept<uint16_t> { static constexpr int k1 = 64, k2 = 16; };
template <> struct Ept<float> { static constexpr int k1 = 32, k2 = 8; };

template <typename E, int VEC>
hipError_t launch_pair(const Plan& p, const Inputs& in, const Work& w, const Outputs& out,
                       hipStream_t stream, hipEvent_t const* ev) {
  hipError_t err = hipSuccess;
  if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
  const dim3 block(kBlock);
  hipLaunchKernelGGL((pass1_kernel<E, VEC, Ept<E>::k1>), dim3((unsigned)((int64_t)p.R * p.s1)), block, 0,
                     stream, in, w, out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
  hipLaunchKernelGGL((pass2_kernel<E, VEC, Ept<E>::k2>), dim3((unsigned)((int64_t)p.B * p.s2)), block, 0,
                     stream, in, w, out);
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
         reinterpret_cast<RowRec*>(ws + p.off_rec), reinterpret_cast<uint32_t*>(ws + p.off_ticket1),
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
