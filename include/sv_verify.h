/*
 * sv_verify.h - C ABI of the MI355X speculative-decoding verify sampler.
 *
 * The operation is mu-gated lossless rejection sampling over a batch of
 * speculative windows. Per request b with rows ro[b] .. ro[b+1]-1 (one row
 * per drafted position, plus a final bonus row):
 *
 *  - p = softmax(target_logits[row] / T_b), q = softmax(draft_logits[row] / T_b).
 *  - Retained measure mu = q * [q >= tau_b], not renormalised. A drafted
 *    token D whose gate fails (q(D) < tau_b) gives an explicit NULL row.
 *    (Strata PR #3416 "[Engine] Preserve target probabilities in gated
 *    MTP", section Approach.)
 *  - An offered D is accepted with probability min(1, p(D)/mu(D)). The test
 *    used is u*mu(D) < p(D), with u a Philox uniform on [0,1) keyed by
 *    (seed, b, row position). This is the strict form of the accept test in
 *    mlxcel PR #992, section What changed.
 *  - Rejection or NULL ends the request with one draw from the normalised
 *    positive part of p - mu (Strata PR #3416, section Approach). The draw
 *    is an exponential race over the vocabulary, ties going to the lower
 *    token id. A residual with zero mass draws from p instead.
 *  - A request whose drafted tokens are all accepted, or which reaches a row
 *    with no proposal, ends with a bonus draw from p (the same section).
 *  - Each request stops at its first rejection, NULL or bonus row. The rows
 *    behind it are never tested (mlxcel PR #992, section Two metric
 *    corrections; regolith audit, section schedule behavior).
 *  - Temperature 0 is greedy: p and q are one-hot argmax indicators (lowest
 *    index on ties), and no randomness is drawn (mlxcel PR #992, section
 *    Temperature 0).
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers (HIP), owned by the caller. The
 *    library never allocates or frees caller memory. It keeps no pointer
 *    after the enqueued work completes.
 *  - Work is enqueued on `hip_stream` (a hipStream_t, NULL = legacy default
 *    stream). The call returns without synchronising. Outputs are valid once
 *    the stream has passed the call.
 *  - Host-checkable problems return a non-zero sv_status before anything is
 *    enqueued, and leave the outputs untouched.
 *  - The same inputs, seed and launch split (sv_set_tuning) give bit-identical
 *    outputs. The split changes only the order of floating-point sums. A
 *    different split can therefore change a request's tokens only where a
 *    decision lies within rounding of its boundary: the accept uniform within
 *    a relative 1e-6 of p(D)/mu(D), q(D) or some residual q_x within 1e-6 of
 *    tau, the two best race keys within a relative 1e-6 of each other, or a
 *    residual mass below 1e-6.
 */
#ifndef SV_VERIFY_H
#define SV_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 2

typedef enum sv_status {
  SV_OK = 0,
  SV_E_NULLPTR = 1,     /* a required pointer is NULL                           */
  SV_E_SHAPE = 2,       /* B < 0, R < 0, V <= 0, R < B, or B == 0 with R > 0     */
  SV_E_DTYPE = 3,       /* dtype is not SV_F32 or SV_BF16                        */
  SV_E_WORKSPACE = 4,   /* workspace smaller than sv_workspace_bytes(shape)      */
  SV_E_UNSUPPORTED = 5, /* sizes beyond what the kernels index (see below)       */
  SV_E_HIP = 6          /* a HIP launch or event call failed                     */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

enum { SV_NO_PROPOSAL = -1 };

/* Row verdicts reported in sv_row_diag.verdict. */
enum {
  SV_ROW_UNTESTED = 0, /* the method never reached this row                         */
  SV_ROW_ACCEPT = 1,   /* offered and accepted                                      */
  SV_ROW_REJECT = 2,   /* offered and rejected: residual draw                       */
  SV_ROW_NULL = 3,     /* gate failed (q(D) < tau): residual draw                   */
  SV_ROW_BONUS = 4     /* last row or no proposal: draw from p                      */
};

typedef struct sv_shape {
  int32_t B;     /* requests                                                     */
  int32_t R;     /* total rows = row_offsets[B]                                  */
  int32_t V;     /* vocabulary size (row length)                                 */
  int32_t dtype; /* sv_dtype of target_logits and draft_logits                   */
} sv_shape;

/* Per-row diagnostics (32 bytes). Rows the method did not reach, and rows of
 * invalid requests, hold verdict SV_ROW_UNTESTED and NaN values. */
typedef struct sv_row_diag {
  float p_D;        /* p(D) of an offered/NULL row (fp32 copy of an fp64 value) */
  float q_D;        /* q(D)                                                     */
  float mu_D;       /* mu(D) = q(D) if offered, else 0                          */
  float u;          /* accept uniform (NaN at temperature 0)                    */
  float resid_mass; /* sum_x (p - mu)+ on the row that drew the residual        */
  int32_t verdict;  /* SV_ROW_*                                                 */
  int32_t pad0;
  int32_t pad1;
} sv_row_diag;

/* Batch counters (optional output). `rows_tested` counts drafted positions
 * that were tested, which is the right denominator for per-position
 * acceptance (mlxcel PR #992, section Two metric corrections). */
typedef struct sv_batch_stats {
  int64_t requests;     /* valid requests                                     */
  int64_t rows_tested;  /* proposal rows tested (accepted + rejected + null)  */
  int64_t accepted;
  int64_t rejected;
  int64_t null_rows;
  int64_t bonus;        /* requests that ended with a bonus draw              */
  int64_t greedy;       /* valid requests at temperature 0                    */
  int64_t invalid;      /* requests failed closed on the device               */
  int64_t offered;      /* proposal rows whose draft passed the gate and was
                           tested (accepted + rejected)                     */
  int64_t noprop;       /* requests that stopped at a row with no proposal
                           before their last row                            */
  int64_t bad_draft;    /* ... of them, those whose drafted id was neither -1
                           nor in [0, V) (read as no proposal)              */
} sv_batch_stats;

/*
 * The sampler's filter chain for one side (target or draft) of a batch
 * (mlxcel PR #992, section What changed: temperature scale, then top-k, then
 * top-p, then min-p, then the softmax of what is left). Each member is a
 * device array of B values, one per request, or NULL, which turns that filter
 * off for every request:
 *   top_k  int32. Keeps the tokens whose logit is at least the k-th largest
 *          (ties kept). 0 or >= V turns it off; a negative value is invalid.
 *   top_p  float. On the distribution top-k leaves, renormalised: keeps the
 *          fewest largest tokens whose mass reaches top_p, the crossing token
 *          and its ties included. >= 1 turns it off; NaN or <= 0 is invalid.
 *   min_p  float. Keeps the tokens whose probability is at least min_p times
 *          the largest, tested as (x - max) / T >= ln(min_p) in fp64.
 *          0 turns it off; NaN, < 0 or > 1 is invalid.
 * The kept set is the tokens at or above the largest of the three
 * thresholds, and p (or q) is the softmax over it. Filters apply only to
 * requests with T > 0; greedy requests ignore them and their values. The
 * emitted tokens follow the filtered p when each drafted token was drawn from
 * the q the verifier uses, filtered or not.
 */
typedef struct sv_filter {
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
} sv_filter;

/*
 * sv_verify_batch - verify every request of a batch.
 *
 * target_logits  [R, V] row-major, dtype. Rows that the method may read:
 *                every proposal row and the row that ends each request.
 * draft_logits   [R, V] same layout. Only proposal rows are read.
 * draft_tokens   [R] int32. Drafted token D in [0, V), drawn by the drafter
 *                from q. -1 (or any id outside [0, V)) means no proposal:
 *                that row is a bonus row. The value on a request's last row
 *                is ignored (it is always the bonus row).
 * row_offsets    [B+1] int32. row_offsets[0] = 0, strictly increasing,
 *                row_offsets[B] = R. Request b owns rows
 *                [row_offsets[b], row_offsets[b+1]).
 * temperature    [B] fp32. 0 = greedy. Otherwise it must lie in
 *                [2^-14, 2^14].
 * tau            [B] fp32. Gate threshold: the draft is offered iff
 *                q(D) >= tau. 0 = ungated (mu = q). Must not be NaN.
 * seed           64-bit Philox key. Give every verify step its own seed.
 * out_tokens     [R] int32 output. Slots row_offsets[b] ..
 *                row_offsets[b] + accept_len[b] hold the emitted tokens: the
 *                accepted drafts, then the residual or bonus token. The other
 *                slots are -1.
 * out_accept_len [B] int32 output. Number of accepted drafts k, or -1 when
 *                request b failed closed.
 * shape          sizes and dtype (see sv_shape).
 * workspace      device scratch of at least sv_workspace_bytes(shape)
 *                bytes. Its contents need no preparation. The library keeps,
 *                per device and workspace address, the counter layout of the
 *                last call. When it sees a new address or a changed layout,
 *                it clears the counters with a small kernel before the call.
 *                Every completed call leaves them at zero again. So between
 *                two calls that pass the same address with the same shape,
 *                nothing else may write to the workspace. Calls that run at
 *                the same time must not share a workspace.
 * hip_stream     hipStream_t to enqueue on.
 *
 * Errors. Host-checkable problems return before anything is enqueued:
 * SV_E_NULLPTR, SV_E_SHAPE, SV_E_DTYPE, SV_E_WORKSPACE, SV_E_UNSUPPORTED
 * (V > 2^28 or R > 2^26). B == 0 with R == 0 is an empty batch: SV_OK,
 * nothing enqueued. A failed launch returns SV_E_HIP. Bad data found on the
 * device fails closed:
 *  - temperature outside {0} U [2^-14, 2^14] or NaN, tau NaN, or an
 *    evaluated row whose logits contain NaN or +inf or are all -inf: that
 *    request gets accept_len -1 and all of its slots -1;
 *  - row_offsets that are not strictly increasing from 0 to R: every
 *    accept_len and every slot of out_tokens is -1.
 * Logits must be finite with magnitude at most 2^64, or -inf.
 */
sv_status sv_verify_batch(const void* target_logits, const void* draft_logits,
                          const int32_t* draft_tokens, const int32_t* row_offsets,
                          const float* temperature, const float* tau, uint64_t seed,
                          int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * sv_verify_batch_diag - sv_verify_batch plus optional diagnostics.
 *
 * It does the same work, with the same arguments and results.
 * out_row_diag   [R] sv_row_diag (device), or NULL.
 * out_stats      one sv_batch_stats (device), or NULL. It is overwritten.
 * hip_events     NULL, or three hipEvent_t created by the caller. They are
 *                recorded on hip_stream before the first kernel, between
 *                the two kernels, and after the second. Elapsed times between
 *                them give each kernel's duration.
 */
sv_status sv_verify_batch_diag(const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const int32_t* row_offsets,
                               const float* temperature, const float* tau, uint64_t seed,
                               int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                               void* workspace, size_t workspace_bytes, void* hip_stream,
                               sv_row_diag* out_row_diag, sv_batch_stats* out_stats,
                               void* const* hip_events);

/*
 * sv_verify_batch_sched - sv_verify_batch with a per-step gate schedule and a
 * cumulative prefix floor, plus optional diagnostics.
 *
 * Source: regolith audit "rank-1 moce and step-aware speculative retention",
 * section schedule behavior. A supplied schedule overrides the request's
 * threshold per step. The cumulative gate requires the product of the draft
 * probabilities of the drafted tokens so far, the current one included, to
 * reach a floor. Both gates must pass, equality passes, and a failed gate ends
 * the prefix like any NULL row.
 *
 * Row j of request b (r = row_offsets[b] + j) offers its drafted token D iff
 * q(D) >= tau_j, with
 *     tau_j = max(s_r, m_b / (q_0(D_0) * ... * q_{j-1}(D_{j-1})))   if m_b > 0,
 *     tau_j = s_r                                                    otherwise,
 * where s_r = tau_step[r] (tau[b] when tau_step is NULL) and m_b = min_cum[b]
 * (0 when min_cum is NULL). The product runs over the accepted rows before j,
 * in fp64. mu = q * [q >= tau_j] on that row, also for its residual draw, so
 * the method stays lossless: tau_j depends only on the accepted prefix.
 *
 * tau_step   [R] float (device), or NULL. A schedule of thresholds for steps
 *            0, 1, 2, ... with its last entry repeating is expanded into it by
 *            the caller. Entries of bonus rows are ignored. A NaN entry on a
 *            row the method tests fails its request closed.
 * min_cum    [B] float (device), or NULL. 0 turns the cumulative gate off; a
 *            value that is NaN, infinite or negative fails its request closed.
 * Every other argument, the results, ownership, the workspace and the errors
 * are those of sv_verify_batch_diag (without events). With both tau_step and
 * min_cum NULL it computes exactly what sv_verify_batch_diag computes.
 */
sv_status sv_verify_batch_sched(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const int32_t* row_offsets,
                                const float* temperature, const float* tau, const float* tau_step,
                                const float* min_cum, uint64_t seed, int32_t* out_tokens,
                                int32_t* out_accept_len, sv_shape shape, void* workspace,
                                size_t workspace_bytes, void* hip_stream, sv_row_diag* out_row_diag,
                                sv_batch_stats* out_stats);

/*
 * sv_verify_batch_lazy - sv_verify_batch, reading rows only up to each
 * request's first row that is not accepted.
 *
 * Same arguments, results, ownership, workspace and errors as
 * sv_verify_batch; the outputs are identical. max_rows bounds the rows of
 * every request (typically the number of draft positions plus one). Position j
 * of all requests is verified by launch j, max(1, max_rows - 1) launches in
 * all, so the call trades that many dependent launches for bytes: a request
 * whose draft at position j is rejected never has rows j+1... read. mlxcel
 * PR #992, section Two metric corrections: the positions behind the first
 * rejection are never tested. A batch with a request of more than max_rows
 * rows fails closed like broken row_offsets (every output -1).
 * max_rows   1 .. 4096, else SV_E_SHAPE.
 */
sv_status sv_verify_batch_lazy(const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const int32_t* row_offsets,
                               const float* temperature, const float* tau, uint64_t seed,
                               int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                               void* workspace, size_t workspace_bytes, void* hip_stream,
                               int32_t max_rows);

/*
 * sv_verify_batch_sampler_match - the sampler-match comparison rule.
 *
 * mlxcel PR #992, section The premise correction: every tested row takes a
 * fresh draw t from the target p, a drafted token is accepted iff it equals
 * t, and t is emitted on both branches, so the emitted stream is a target
 * sample. Its acceptance is sum_x p(x) q(x) (the same page, section The
 * acceptance ceiling), at most the method's sum_x min(p, mu); the pages
 * compare the method against it. It reads no draft logits and no gate.
 * Row j of request b draws by the race over p with the random numbers of the
 * method's race on that row (ties to the lower token id); at T_b = 0 the draw
 * is the lowest-index argmax, which makes the rule argmax-against-argmax.
 * The request stops at its first row whose draft differs from the draw, at
 * a row with no proposal, or at its last row; that row's draw is its last
 * token, and accept_len counts the rows before it.
 * Inputs, outputs, ownership, workspace (sv_workspace_bytes of the same
 * shape), fail-closed cases (invalid temperature, a NaN, +inf or all -inf
 * target row up to the stop, broken row_offsets) and errors are as for
 * sv_verify_batch. It streams every row of target_logits once.
 */
sv_status sv_verify_batch_sampler_match(const void* target_logits, const int32_t* draft_tokens,
                                        const int32_t* row_offsets, const float* temperature,
                                        uint64_t seed, int32_t* out_tokens, int32_t* out_accept_len,
                                        sv_shape shape, void* workspace, size_t workspace_bytes,
                                        void* hip_stream);

/*
 * sv_row_acceptance - per-row acceptance sums of a verify batch.
 *
 * For every proposal row r (row j of request b; the rows before a request's
 * first row without a proposal and before its last row):
 *   out_sum_min[r] = sum_x min(p(x), mu(x)): the probability that row r
 *                    accepts its draft given that its prefix was accepted
 *                    (Strata PR #3416, section Approach; mlxcel PR #992,
 *                    section The acceptance ceiling);
 *   out_sum_pq[r]  = sum_x p(x) q(x): the sampler-match rule's acceptance
 *                    (mlxcel PR #992, same section).
 * p and q are softmax(logits / T_b) (one-hot argmaxes at T_b = 0), and mu is
 * q gated at row r's threshold as in sv_verify_batch_sched, with the drafted
 * tokens as the prefix. Every other row gets NaN. So does a row of a request
 * whose T_b, tau_b or floor is invalid, and a row with an invalid row up to it
 * (NaN or +inf or all -inf logits, or a NaN step threshold). Broken
 * row_offsets make every row NaN.
 * out_sum_min, out_sum_pq   [R] float (device), written in full.
 * tau_step, min_cum         as in sv_verify_batch_sched (each may be NULL).
 * It reads every proposal row twice (statistics, then sums) and draws no
 * random numbers. Arguments, workspace and errors are as for sv_verify_batch.
 */
sv_status sv_row_acceptance(const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const int32_t* row_offsets,
                            const float* temperature, const float* tau, const float* tau_step,
                            const float* min_cum, float* out_sum_min, float* out_sum_pq,
                            sv_shape shape, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * sv_filter_thresholds - each row's keep-threshold under the filter chain.
 *
 * For every row r of request b (T_b > 0) and each side, out_theta[2r] (target)
 * and out_theta[2r + 1] (draft) hold a float theta such that the kept tokens
 * are exactly those with logit >= theta: sv_filter's definition, computed
 * exactly (top-p's masses in fp64). Rows with no active filter, and greedy
 * requests, get -inf. A row whose logits contain NaN or +inf or are all -inf
 * gets +inf. Values of an invalid filter are treated as off here; the verify
 * call fails such a request.
 * target_filter, draft_filter   host pointers to sv_filter, or NULL (no filter).
 * out_theta      [R, 2] float (device), written in full.
 * It reads every row of each side that has a filter at least once. Every
 * other argument, the workspace and the errors are as for sv_verify_batch.
 */
sv_status sv_filter_thresholds(const void* target_logits, const void* draft_logits,
                               const int32_t* row_offsets, const float* temperature,
                               const sv_filter* target_filter, const sv_filter* draft_filter,
                               float* out_theta, sv_shape shape, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/*
 * sv_verify_batch_filtered - sv_verify_batch_sched with p and q filtered.
 *
 * p (target) and q (draft) are the filtered distributions of sv_filter, each
 * side with its own parameters, for every row the method evaluates: the
 * accept test, the gate mu = q * [q >= tau_j], the residual (p - mu)+ and the
 * bonus race over p. A request with T > 0 and an invalid filter value fails
 * closed (accept_len -1, slots -1). A filtered target's support is never left:
 * an accepted draft has p(D) > 0, and both draws put no mass outside p's
 * support.
 * target_filter, draft_filter   host pointers to sv_filter, or NULL.
 * The call first computes the rows' thresholds (as sv_filter_thresholds, into
 * the workspace), then runs the two passes of sv_verify_batch with the masks.
 * It skips the row sides the method never reads: the draft side of a row with
 * no proposal (every request's last row is one) and both sides of the rows
 * after it. A row side that the threshold step decided from the logits at or
 * above a bound it keeps (the masked sums are then at hand) is not streamed
 * again by the first pass; its sums differ from a streamed side's only in
 * summation order. Every other argument, the results and the errors are those of
 * sv_verify_batch_sched. With both filters NULL it computes exactly what
 * sv_verify_batch_sched computes.
 */
sv_status sv_verify_batch_filtered(const void* target_logits, const void* draft_logits,
                                   const int32_t* draft_tokens, const int32_t* row_offsets,
                                   const float* temperature, const float* tau, const float* tau_step,
                                   const float* min_cum, const sv_filter* target_filter,
                                   const sv_filter* draft_filter, uint64_t seed, int32_t* out_tokens,
                                   int32_t* out_accept_len, sv_shape shape, void* workspace,
                                   size_t workspace_bytes, void* hip_stream, sv_row_diag* out_row_diag,
                                   sv_batch_stats* out_stats);

/*
 * sv_row_acceptance_filtered - sv_row_acceptance with p and q filtered.
 *
 * The same sums, sum_x min(p, mu) and sum_x p q per proposal row, with p and
 * q the filtered distributions of sv_filter (mlxcel PR #992, section What
 * changed), so that sum_x min(p, mu) is the row's acceptance probability under the
 * sampler's own configuration. A request whose filter values are invalid at
 * T > 0 gets NaN, as sv_verify_batch_filtered fails it. The call computes the
 * thresholds first, skipping the row sides sv_verify_batch_filtered skips (no
 * proposal row's sum reads them). target_filter, draft_filter: host pointers to
 * sv_filter, or NULL. Every other argument, the results and the errors are
 * those of sv_row_acceptance; with both filters NULL it computes what
 * sv_row_acceptance computes.
 */
sv_status sv_row_acceptance_filtered(const void* target_logits, const void* draft_logits,
                                     const int32_t* draft_tokens, const int32_t* row_offsets,
                                     const float* temperature, const float* tau, const float* tau_step,
                                     const float* min_cum, const sv_filter* target_filter,
                                     const sv_filter* draft_filter, float* out_sum_min, float* out_sum_pq,
                                     sv_shape shape, void* workspace, size_t workspace_bytes,
                                     void* hip_stream);

/*
 * Launch tuning (host-only, process-wide). The verify calls split each
 * potential proposal row over w1 waves and each request's last row over w2
 * waves. A field of 0 keeps the library's choice for the device; w1 is
 * rounded down to a power of two, and both are clamped to what the workspace
 * holds (at most 64). Outputs depend on the split only as the determinism
 * note at the top of this header states. It exists for measurements and for
 * tests of that independence; normal use does not need it. It applies to
 * calls enqueued after it returns, from any thread. sv_set_tuning(NULL)
 * restores the defaults; sv_get_tuning reads the current values.
 */
typedef struct sv_tuning {
  int32_t w1, w2;
} sv_tuning;

void sv_set_tuning(const sv_tuning* t);
void sv_get_tuning(sv_tuning* t);

/*
 * sv_verify_batch_static - sv_verify_batch without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc.
 *
 * Inputs, outputs, results and errors are those of sv_verify_batch (the same
 * kernels run). The workspace is a device array of SV_STATIC_WORKSPACE_BYTES
 * inside the library, one per GPU, held until the process ends. Its address
 * is looked up on the first call on each device. A shape whose
 * sv_workspace_bytes exceeds SV_STATIC_WORKSPACE_BYTES returns
 * SV_E_WORKSPACE before anything is enqueued. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (on different streams, or
 * from several threads without ordering) race and give undefined outputs.
 * Calls in one stream are ordered and safe. The first call on a device, and
 * a call whose shape changes the workspace layout, enqueue a small kernel
 * that zeroes the array's counters.
 */
#define SV_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)

sv_status sv_verify_batch_static(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const int32_t* row_offsets,
                                 const float* temperature, const float* tau, uint64_t seed,
                                 int32_t* out_tokens, int32_t* out_accept_len, sv_shape shape,
                                 void* hip_stream);

/* Bytes of workspace the call needs for this shape; 0 when the shape is invalid. Host-only. */
size_t sv_workspace_bytes(sv_shape shape);

/* Static, human-readable name of a status code. Host-only. */
const char* sv_status_string(int status);

/* SV_ABI_VERSION of the loaded library. Host-only. */
int sv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SV_VERIFY_H */
