// sv_plan.h - workspace layout and launch plan shared by the host core and the kernels.
//
// The record types below live in the caller's workspace. Their layouts are
// fixed here so that the kernels and the host-side size computation agree.
// Pass 1's partials reach pass 2 across the kernel boundary. Pass 2's partials
// move between its own workgroups as 8-byte words with agent-scope atomics, so
// their size is a multiple of 8 bytes.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sv_verify.h"

namespace sv {

constexpr int kWave = 64;                       // CDNA wavefront width
constexpr int kBlock = 256;                     // threads per workgroup in every kernel
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxWavesPerRow = 64;             // pass-2 walks hold one row's partials in a wave
// Bytes of one array that a wave requests per loop step (two 16-byte chunks per lane);
// both passes keep two such batches per array in flight (double buffering).
constexpr int kBatchBytes = 2 * kWave * 16;
// Waves per compute unit that the streaming kernels aim for. Measured on MI355X for the
// gated B=64, T=4, V=151936 bf16 batch: about six waves per CU, each streaming long
// contiguous spans with small batches, read HBM faster than a full-occupancy grid of
// shorter spans (29.5 us against 33 us for pass 1).
constexpr int kTargetWavesPerCU = 6;
// Pass 2 draws from one row per request. Its waves are latency-bound, so it runs more of
// them: with 12 per CU, the gated batch above draws in 36 us, against 45 us with 6 per CU
// and 42 us with 16 per CU.
constexpr int kTargetWavesPerCU2 = 12;
// ... but a pass-2 wave takes between 8 KB and 24 KB of its row. Measured on MI355X:
//  - the gated B=64, V=151936 bf16 batch (latency-bound): 38 to 42 waves per request (spans of
//    about 8 KB) draw in 28.5 us, against 30.6 us for the 48 that 12 waves per CU would give;
//  - the ungated B=256, V=256000 bf16 and mixed B=512, V=152064 fp32 batches (bound by the
//    races' random numbers on flat residuals): 20 to 40 and 24 to 48 waves per request
//    (spans of 12 to 25 KB) take 452-459 and 420-430 us per step, against 481 and 473 us
//    for the 12 and 6 waves per request that 12 waves per CU would give.
constexpr int64_t kMinSpanBytes2 = 8 * kWave * 16;
constexpr int64_t kMaxSpanBytes2 = 3 * kMinSpanBytes2;

// Row verdict used inside the kernels besides the public SV_ROW_* codes.
enum : int32_t { kRowInvalid = 5 };

// What pass 2 does for a request.
enum : int32_t {
  kKindInvalid = 0,      // failed closed
  kKindGreedyDone = 1,   // greedy, stopped on a proposal row: token = that row's argmax
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

// Pass 2: one partial per (request, wave).
struct P2Part {
  double key;       // best fp64 race key in the span (ratio for residual rows, log for bonus rows)
  int32_t idx;      // its token (-1 if none)
  float rsum;       // residual rows: sum of (p - mu)+ over the span
  float mref;       // bonus rows: max target logit of the span
  int32_t bad;      // bonus rows: span holds NaN or +inf
  int32_t gidx;     // greedy bonus rows: lowest index of mref
  int32_t pidx;     // filtered residual rows: best token of the race over p (-1 if none) ...
  double pkey;      // ... and its fp64 key, the draw if the residual turns out to be empty
};
static_assert(sizeof(P2Part) == 40, "P2Part layout");

// Acceptance sums: one partial per (row, pass-1 wave) of sum min(p, mu) and sum p q.
struct SumPart {
  double smin, spq;
};
static_assert(sizeof(SumPart) == 16, "SumPart layout");

struct WsHeader {
  int32_t ro_valid;  // row_offsets check result, written by pass 1
  int32_t pad[63];
};
static_assert(sizeof(WsHeader) == 256, "WsHeader layout");

// The filter chain's segment records: a segment is kSegLogits consecutive logits of a row
// read with 16-byte vectors. Rows of more than kSegCap segments keep none.
constexpr int kSegLogits = 512;
constexpr int kSegCap = 512;
struct alignas(8) SegRec {
  float max;   // the segment's largest logit; +inf when it holds NaN or +inf
  float mass;  // with top-p alone: sum of exp2((l - max) * c) over the segment
};
static_assert(sizeof(SegRec) == 8, "SegRec layout");

// A row and side whose threshold the filter chain decided from its candidates (ok = 1): the
// row's largest logit, the masked sum of exp2(l*c - ref_of(m, c)) over the kept logits, and
// the logit at the row's drafted token. Pass 1 then writes the row's partials from it.
struct FiltStat {
  float m, s, lD;
  int32_t ok;
};
static_assert(sizeof(FiltStat) == 16, "FiltStat layout");

struct Plan {
  int32_t B, R, V, dtype;
  int32_t esize;  // bytes per logit
  int32_t w1max;  // pass 1: most waves that share one row (sizes the partial array)
  int32_t w2max;  // pass 2: most waves that share one request
  int32_t nseg;   // record segments per row and side (0: more than kSegCap)
  // Persistent: the header, lazy stop flags, keep-thresholds, then the counters every call
  // leaves at zero, [off_ticket2, off_trans). Per call, from off_trans: the partial records
  // (off_part1..3) or, earlier in the filter chain, the segment records (off_seg).
  size_t off_hdr, off_lazy, off_theta, off_fstat, off_ticket2, off_bmax, off_done3, off_trans;
  size_t off_part1, off_part2, off_part3, off_seg, total;
};

// Build the plan for a shape. Returns SV_OK, or the status describing why the
// shape cannot be served. Host-only, allocation-free.
sv_status make_plan(const sv_shape& shape, Plan* out);

// Waves per potential proposal row in pass 1 (w1, a power of two) and per request in
// pass 2 (w2), and the grids.
struct Launch {
  int32_t w1, w2;
  int64_t blocks1, blocks2;
};

// Choose the split for a device on which each kernel keeps `slots1` / `slots2` waves
// resident: one round of waves covers the work, and no split exceeds the plan's bounds.
// A tuning override (sv_set_tuning) replaces the computed splits, clamped to the bounds.
Launch pick_waves(const Plan& p, int64_t slots1, int64_t slots2);

// Host-side tuning (sv_set_tuning): zero fields keep the computed value.
struct Tuning {
  int32_t w1, w2;  // waves per potential proposal row / per request's last row
};
Tuning tuning();
void set_tuning(const Tuning& t);

// Validate every host-checkable argument of a verify call. The two outputs are only
// null-checked (the acceptance sums pass their two float arrays).
sv_status check_call(const sv_shape& shape, const void* target, const void* draft,
                     const int32_t* draft_tokens, const int32_t* row_offsets,
                     const float* temperature, const float* tau, const void* out_tokens,
                     const void* out_accept_len, const void* workspace,
                     size_t workspace_bytes, Plan* plan);

}  // namespace sv
