// sv_core.cpp - host-side planning and argument validation of the verify library.
//
// Pure C++ with no HIP dependency. The shared library links it, and the CPU
// tests also build it on its own (with address and undefined-behaviour
// sanitizers) to exercise the error paths.
#include <mutex>

#include "sv_plan.h"

namespace sv {

namespace {

constexpr int64_t kMaxV = int64_t(1) << 28;
constexpr int64_t kMaxR = int64_t(1) << 26;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

sv_status make_plan(const sv_shape& s, Plan* p) {
  if (s.dtype != SV_F32 && s.dtype != SV_BF16) return SV_E_DTYPE;
  if (s.B < 0 || s.R < 0 || s.V <= 0) return SV_E_SHAPE;
  if (s.B == 0 && s.R != 0) return SV_E_SHAPE;
  if (s.R < s.B) return SV_E_SHAPE;
  if (s.V > kMaxV || s.R > kMaxR) return SV_E_UNSUPPORTED;
  Plan q{};
  q.B = s.B;
  q.R = s.R;
  q.V = s.V;
  q.dtype = s.dtype;
  q.esize = s.dtype == SV_BF16 ? 2 : 4;
  // Waves stream contiguous spans of a row, at least two batches of each array per wave.
  // A row has at most 64 waves, so that a pass-2 wave can hold one row's partials.
  const int64_t row_bytes = (int64_t)s.V * q.esize;
  const int64_t w = row_bytes / (2 * kBatchBytes);
  q.w1max = q.w2max = (int32_t)(w < 1 ? 1 : w > kMaxWavesPerRow ? kMaxWavesPerRow : w);
  if ((int64_t)q.R * q.w1max > INT32_MAX || (int64_t)q.B * q.w2max > INT32_MAX) return SV_E_UNSUPPORTED;
  // The persistent part first: the header, the lazy verify's per-request stop flags, the
  // filtered verify's keep-thresholds and row statistics, and the counters that every call
  // leaves at zero. Then the per-call part, which one call writes before it reads: the partial
  // records of passes 1 and 2 and of the acceptance sums, or, earlier in a filtered call, the
  // filter chain's segment records (the two sets are never live at once).
  size_t off = 0;
  q.off_hdr = off;
  off += sizeof(WsHeader);
  q.off_lazy = off = align_up(off, 256);
  off += (size_t)q.B * sizeof(int32_t);
  q.off_theta = off = align_up(off, 256);  // [R] (target, draft)
  off += (size_t)q.R * 2 * sizeof(float);
  q.off_fstat = off = align_up(off, 256);  // [R] (target, draft)
  off += (size_t)q.R * 2 * sizeof(FiltStat);
  q.off_ticket2 = off = align_up(off, 256);  // pass 2's request tickets
  off += (size_t)q.B * sizeof(uint32_t);
  q.off_bmax = off = align_up(off, 8);  // the bonus race's per-request best (logit, token)
  off += (size_t)q.B * sizeof(uint64_t);
  q.off_done3 = off;  // the acceptance sums' per-row done flags
  off += (size_t)q.R * sizeof(uint32_t);
  q.off_trans = off = align_up(off, 256);
  q.off_part1 = off;
  off += (size_t)q.R * q.w1max * sizeof(P1Part);
  q.off_part2 = off = align_up(off, 256);
  off += (size_t)q.B * q.w2max * sizeof(P2Part);
  q.off_part3 = off = align_up(off, 256);
  off += (size_t)q.R * q.w1max * sizeof(SumPart);
  const size_t end_parts = off;
  const int64_t nseg = ceil_div((int64_t)s.V, kSegLogits);
  q.nseg = nseg <= kSegCap ? (int32_t)nseg : 0;
  q.off_seg = off = q.off_trans;
  off += (size_t)q.R * 2 * q.nseg * sizeof(SegRec);
  off = off > end_parts ? off : end_parts;
  q.total = align_up(off, 256);
  *p = q;
  return SV_OK;
}

namespace {

std::mutex g_tuning_mu;
Tuning g_tuning{};

}  // namespace

Tuning tuning() {
  std::lock_guard<std::mutex> lock(g_tuning_mu);
  return g_tuning;
}

void set_tuning(const Tuning& t) {
  std::lock_guard<std::mutex> lock(g_tuning_mu);
  g_tuning = t;
}

Launch pick_waves(const Plan& p, int64_t slots1, int64_t slots2) {
  Launch l{};
  const Tuning t = tuning();
  // Pass 1 streams the potential proposal rows: every row but the last of each request.
  // Pass 2 merges a row's partials in aligned lane groups, so the waves per row are a
  // power of two.
  const int64_t rows = p.R - p.B;
  int64_t w1 = t.w1 > 0 ? t.w1 : rows > 0 ? slots1 / rows : 1;
  if (w1 > p.w1max) w1 = p.w1max;
  int64_t pow2 = 1;
  while (pow2 * 2 <= w1) pow2 *= 2;
  int64_t w2 = t.w2 > 0 ? t.w2 : p.B > 0 ? slots2 / p.B : 1;
  if (t.w2 <= 0 && p.B > 0) {
    // Spans of 8 KB to 24 KB, but at least about one wave per compute unit in all (slots2
    // counts kTargetWavesPerCU2 per unit): a batch of one or two requests still spreads.
    const int64_t row_bytes = (int64_t)p.V * p.esize;
    const int64_t lo = ceil_div(row_bytes, kMaxSpanBytes2), hi = ceil_div(row_bytes, kMinSpanBytes2);
    if (w2 < lo) w2 = lo;
    if (w2 > hi) w2 = hi;
    const int64_t spread = ceil_div(slots2 / kTargetWavesPerCU2, p.B);
    if (w2 < spread) w2 = spread;
  }
  l.w1 = (int32_t)pow2;
  l.w2 = (int32_t)(w2 < 1 ? 1 : w2 > p.w2max ? p.w2max : w2);
  l.blocks1 = ceil_div(rows * l.w1, kWavesPerBlock);
  if (l.blocks1 < 1) l.blocks1 = 1;  // block 0 checks row_offsets even when nothing is streamed
  l.blocks2 = ceil_div((int64_t)p.B * l.w2, kWavesPerBlock);
  return l;
}

sv_status check_call(const sv_shape& shape, const void* target, const void* draft,
                     const int32_t* draft_tokens, const int32_t* row_offsets,
                     const float* temperature, const float* tau, const void* out_tokens,
                     const void* out_accept_len, const void* workspace,
                     size_t workspace_bytes, Plan* plan) {
  const sv_status st = make_plan(shape, plan);
  if (st != SV_OK) return st;
  if (shape.B == 0) return SV_OK;  // empty batch: nothing to read or write
  if (!target || !draft || !draft_tokens || !row_offsets || !temperature || !tau || !out_tokens ||
      !out_accept_len || !workspace)
    return SV_E_NULLPTR;
  if (workspace_bytes < plan->total) return SV_E_WORKSPACE;
  return SV_OK;
}

}  // namespace sv

extern "C" size_t sv_workspace_bytes(sv_shape shape) {
  sv::Plan p;
  if (sv::make_plan(shape, &p) != SV_OK) return 0;
  return p.total;
}

extern "C" const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_E_NULLPTR: return "SV_E_NULLPTR: a required pointer is NULL";
    case SV_E_SHAPE: return "SV_E_SHAPE: invalid B, R or V";
    case SV_E_DTYPE: return "SV_E_DTYPE: dtype must be SV_F32 or SV_BF16";
    case SV_E_WORKSPACE: return "SV_E_WORKSPACE: workspace smaller than sv_workspace_bytes";
    case SV_E_UNSUPPORTED: return "SV_E_UNSUPPORTED: sizes beyond the supported range";
    case SV_E_HIP: return "SV_E_HIP: a HIP launch or event call failed";
    default: return "unknown sv_status";
  }
}

extern "C" int sv_abi_version(void) { return SV_ABI_VERSION; }

extern "C" void sv_set_tuning(const sv_tuning* t) {
  sv::Tuning v{};
  if (t != nullptr) {
    v.w1 = t->w1;
    v.w2 = t->w2;
  }
  sv::set_tuning(v);
}

extern "C" void sv_get_tuning(sv_tuning* t) {
  if (t == nullptr) return;
  const sv::Tuning v = sv::tuning();
  t->w1 = v.w1;
  t->w2 = v.w2;
}
