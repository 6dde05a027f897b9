// sv_plan.h - workspace layout and launch plan shared by the host core and the kernels.
//
// The record types below live in the caller's workspace. Their layouts are
// fixed here so that the kernels and the host-side size computation agree.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sv_verify.h"

namespace sv {

constexpr int kWave = 64;                       // CDNA wavefront width
constexpr int kBlock = 256;                     // threads per workgroup in both kernels
constexpr int kWavesPerBlock = kBlock / kWave;

// Row verdicts kept in RowRec (the public SV_ROW_* codes plus one internal code).
enum : int32_t { kRowInvalid = 5 };

// Pass 1 writes one partial per (row, chunk, wave): the wave's share of a row's
// softmax statistics, referenced to its own maximum.
struct P1Part {
  float m_t, s_t;   // max target logit; sum of exp2(l*c - fl(m_t*c)) over the wave's slice
  float m_d, s_d;   // same for the draft logits
  int32_t am_t;     // lowest index holding m_t in the slice (-1 if none)
  int32_t am_d;     // lowest index holding m_d (greedy rows only)
  int32_t bad;      // greedy rows: slice holds NaN or +inf
  int32_t pad;
};
static_assert(sizeof(P1Part) == 32, "P1Part layout");

// Pass 1's per-row record, written by the wave that finalises the row.
struct RowRec {
  int32_t verdict;  // SV_ROW_ACCEPT / REJECT / NULL, or kRowInvalid
  int32_t am_t;     // row target argmax (lowest index)
  int32_t am_d;     // row draft argmax (greedy rows)
  int32_t pad0;
  float c;          // log2(e)/T rounded to fp32: the scale every kernel uses
  float m_t, mc_t;  // row max target logit and fl(m_t*c)
  float mc_d;       // fl(m_d*c)
  double s_t, s_d;  // row sums of exp2(l*c - mc) (fp64 merge of fp32 partials)
  float p_D, q_D, mu_D, u;
  float m_d, pad1, pad2, pad3;
};
static_assert(sizeof(RowRec) == 80, "RowRec layout");

// Pass 2 writes one partial per (request, chunk, wave).
struct P2Part {
  float k1, k2;     // two best fp32 race keys in the slice (k1 >= k2)
  int32_t i1, i2;   // their token ids (-1 if none)
  float rsum;       // residual rows: sum of (p - mu)+ over the slice
  float mref;       // bonus rows: max target logit of the slice
  int32_t bad;      // slice holds NaN or +inf (rows not validated by pass 1)
  int32_t gidx;     // greedy bonus rows: lowest index of mref
};
static_assert(sizeof(P2Part) == 32, "P2Part layout");

struct WsHeader {
  int32_t ro_valid;  // row_offsets check result, written by pass 1
  int32_t pad[63];
};
static_assert(sizeof(WsHeader) == 256, "WsHeader layout");

struct Plan {
  int32_t B, R, V, dtype;
  int32_t esize;     // bytes per logit
  int32_t ept1, s1;  // pass 1: logits per lane per array, chunks per row
  int32_t ept2, s2;  // pass 2: logits per lane, chunks per final row
  size_t off_hdr, off_part1, off_rec, off_ticket1, off_part2, off_ticket2, total;
};

// Build the plan for a shape. Returns SV_OK, or the status describing why the
// shape cannot be served. Host-only, allocation-free.
sv_status make_plan(const sv_shape& shape, Plan* out);

// Validate every host-checkable argument of a verify call.
sv_status check_call(const sv_shape& shape, const void* target, const void* draft,
                     const int32_t* draft_tokens, const int32_t* row_offsets,
                     const float* temperature, const float* tau, const int32_t* out_tokens,
                     const int32_t* out_accept_len, const void* workspace,
                     size_t workspace_bytes, Plan* plan);

}  // namespace sv
