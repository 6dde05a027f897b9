// sv_core.cpp - host-side planning and argument validation of the verify library.
//
// Pure C++ with no HIP dependency. The shared library links it, and the CPU
// tests also build it on its own (with address and undefined-behaviour
// sanitizers) to exercise the error paths.
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
  // Long-lived waves: each one streams a contiguous span of a row. Pass 1 aims
  // at about 3072 waves (3 per SIMD on 256 CUs) so that one round of waves
  // covers the rows; pass 2 at about 4096. A row is never split into spans
  // shorter than 8192 logits.
  const int64_t max_split = s.V / 8192 > 1 ? s.V / 8192 : 1;
  const int64_t want1 = s.R > 0 ? ceil_div(768, s.R) : 1;
  const int64_t want2 = s.B > 0 ? ceil_div(1024, s.B) : 1;
  q.s1 = (int32_t)(want1 < max_split ? want1 : max_split);
  q.s2 = (int32_t)(want2 < max_split ? want2 : max_split);
  if ((int64_t)q.R * q.s1 > INT32_MAX || (int64_t)q.B * q.s2 > INT32_MAX) return SV_E_UNSUPPORTED;
  size_t off = 0;
  q.off_hdr = off;
  off += sizeof(WsHeader);
  q.off_part1 = off = align_up(off, 256);
  off += (size_t)q.R * q.s1 * kWavesPerBlock * sizeof(P1Part);
  q.off_rec = off = align_up(off, 256);
  off += (size_t)q.R * sizeof(RowRec);
  q.off_desc = off = align_up(off, 256);
  off += (size_t)q.B * sizeof(ReqDesc);
  q.off_part2 = off = align_up(off, 256);
  off += (size_t)q.B * q.s2 * kWavesPerBlock * sizeof(P2Part);
  q.off_ticket_row = off = align_up(off, 256);
  off += (size_t)q.R * sizeof(uint32_t);
  q.off_ticket_req = off = align_up(off, 256);
  off += (size_t)q.B * sizeof(uint32_t);
  q.off_ticket2 = off = align_up(off, 256);
  off += (size_t)q.B * sizeof(uint32_t);
  q.total = align_up(off, 256);
  *p = q;
  return SV_OK;
}

sv_status check_call(const sv_shape& shape, const void* target, const void* draft,
                     const int32_t* draft_tokens, const int32_t* row_offsets,
                     const float* temperature, const float* tau, const int32_t* out_tokens,
                     const int32_t* out_accept_len, const void* workspace,
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
