// sv_plan.h - workspace layout and launch plan shared by the host core and the kernels.
//
// The record types below live in the caller's workspace. Their layouts are
// fixed here so that the kernels and the host-side size computation agree.
// Records that one wave writes and another reads inside the same kernel move
// word by word with agent-scope atomics, so every field is 4-byte sized
// (doubles are split into two words).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sv_verify.h"

namespace sv {

constexpr int kWave = 64;                       // CDNA wavefront width
constexpr int kBlock = 256;                     // threads per workgroup in every kernel
constexpr int kWavesPerBlock = kBlock / kWave;

// Row verdict kept in RowRec besides the public SV_ROW_* codes.
enum : int32_t { kRowInvalid = 5 };

// What pass 2 does for a request.
enum : int32_t {
  kKindInvalid = 0,      // failed closed (emitted by pass 1)
  kKindGreedyDone = 1,   // greedy, stopped on a proposal row: token = that row's argmax (emitted by pass 1)
  kKindResidual = 2,     // race over (p - mu)+ on the stop row
  kKindBonus = 3,        // race over p on the bonus row
  kKindGreedyBonus = 4   // argmax of the bonus row
};

// Pass 1: one partial per (row, wave) - the wave's span of the row reduced to
// softmax statistics referenced to the span's own maximum.
struct P1Part {
  float m_t, s_t;   // max target logit; sum of exp2(l*c - fl(m_t*c)) over the span
  float m_d, s_d;   // same for the draft logits
  int32_t am_t;     // greedy rows: lowest index holding m_t in the span (-1 if none);
                    // other rows: index of the first 16-byte vector that holds m_t (a hint)
  int32_t am_d;     // greedy rows: lowest index holding m_d
  int32_t flags;    // bit 1: the span holds the drafted token
  float lt_D, ld_D; // target / draft logit at the drafted token (when flag bit 1 is set)
  int32_t pad[3];
};
static_assert(sizeof(P1Part) == 48, "P1Part layout");

// Pass 1: the row's merged statistics and verdict, written by the wave that finalises the row.
struct RowRec {
  int32_t verdict;  // SV_ROW_ACCEPT / REJECT / NULL, or kRowInvalid
  int32_t am_t;     // greedy rows: row target argmax (lowest index)
  int32_t am_d;     // greedy rows: row draft argmax
  float c;          // log2(e)/T rounded to fp32: the scale every kernel uses
  float m_t, mc_t;  // row max target logit and fl(m_t*c)
  float m_d, mc_d;  // row max draft logit and fl(m_d*c)
  uint32_t s_t_lo, s_t_hi;  // fp64 row sums of exp2(l*c - mc), split into words
  uint32_t s_d_lo, s_d_hi;
  float p_D, q_D, mu_D, u;
  int32_t pad[4];
};
static_assert(sizeof(RowRec) == 80, "RowRec layout");

// Pass 1 -> pass 2: what the request needs for its last token.
struct ReqDesc {
  int32_t kind;           // kKind*
  int32_t k;              // accepted drafts
  int32_t f;              // row that draws the last token
  int32_t final_verdict;  // SV_ROW_REJECT / NULL / BONUS
  float T, tau, c, mc_t;
  float mc_d, m_t, pad0, pad2;
  double s_t, s_d;        // residual rows: row sums
  int32_t pad1[4];
};
static_assert(sizeof(ReqDesc) == 80, "ReqDesc layout");

// Pass 2: one partial per (request, wave).
struct P2Part {
  double key;       // best fp64 race key in the span (ratio for residual rows, log for bonus rows)
  int32_t idx;      // its token (-1 if none)
  float rsum;       // residual rows: sum of (p - mu)+ over the span
  float mref;       // bonus rows: max target logit of the span
  int32_t bad;      // bonus rows: span holds NaN or +inf
  int32_t gidx;     // greedy bonus rows: lowest index of mref
  int32_t pad;
};
static_assert(sizeof(P2Part) == 32, "P2Part layout");

struct WsHeader {
  int32_t ro_valid;  // row_offsets check result, written by pass 1
  int32_t pad[63];
};
static_assert(sizeof(WsHeader) == 256, "WsHeader layout");

struct Plan {
  int32_t B, R, V, dtype;
  int32_t esize;  // bytes per logit
  int32_t s1;     // pass 1: workgroups per row (4 waves each)
  int32_t s2;     // pass 2: workgroups per request
  size_t off_hdr, off_part1, off_rec, off_desc, off_part2, off_ticket_row, off_ticket_req,
      off_ticket2, total;
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
