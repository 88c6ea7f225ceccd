/*
 * dspark.h -- C ABI of the DSpark-style draft / schedule / verify hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * What the three calls compute (sources are the DSpark write-ups):
 *   dspark_draft_sample  Markov-head draft: for every request and draft
 *       position k, p_d(x_k | x_{k-1}) = softmax((base_logit_k + bias) / T)
 *       with bias_v = A[x_{k-1}, :] . W[:, v], a rank-r factorisation of the
 *       V x V transition matrix; x_k is drawn from it and fed to step k+1
 *       (yage.ai "DSpark: speculative decoding and hardware scheduling",
 *       paragraph on the first-order Markov head; freeaitool.com "DeepSeek
 *       DSpark complete guide", section 3.1).
 *   dspark_schedule  confidence-scheduled prefix selection: survival products
 *       S_k = c_1 ... c_k per request, then a greedy sort of all (request,
 *       position) items by S with an early stop against a token budget and an
 *       optional throughput curve (freeaitool guide, sections 4.1-4.2; yage.ai
 *       analysis, scheduler paragraph; legalagi.cn "Reading DSpark as a
 *       lawyer", section 5).
 *   dspark_verify  lossless rejection-sampling verification with strict
 *       prefix semantics: accept x_j with probability min(1, p_t/p_d), on the
 *       first rejection resample from normalise(max(0, p_t - p_d)), append a
 *       bonus token from the target when every verified position is accepted
 *       (yage.ai analysis, paragraphs on prefix matching and on rejection
 *       sampling; legalagi.cn reading, section 3).
 *
 * Random draws: Philox4x32-10 (Salmon et al., SC'11) keyed by the 64-bit seed
 * (low word, high word) with counter (v >> 2, position, request, tag), word
 * v & 3; uniform u = ((w >> 9) + 0.5) * 2^-23; Gumbel G = -log(-log u).
 * Every token draw is a Gumbel-max over the whole vocabulary with one draw per
 * entry v.  These are the only tags the library uses:
 *   0  draft Gumbel of entry v at position k = 1..K;
 *   1  accept uniform of position j (v = 0);
 *   2  Gumbel of entry v for the residual, fallback or bonus draw at the
 *      position of the row it is drawn from.
 * Temperature: per request; T > 0 multiplies logits by the fp32 reciprocal
 * 1/T on both the draft and the target side, T == 0 is greedy on both sides
 * (argmax, ties to the smallest index).  T must be finite and >= 0.
 *
 * Conventions shared by every call:
 *   - Every array pointer is DEVICE memory owned by the caller, except the
 *     schedule curve arrays, which are HOST memory read during the call.
 *   - Layouts are row-major with the vocabulary innermost.
 *   - The library allocates nothing: scratch memory comes in `workspace`
 *     (size from the matching *_workspace_bytes query, 256-byte aligned),
 *     except for dspark_draft_sample_noalloc, whose scratch is a fixed
 *     per-device array the library holds.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns without synchronising.  Calls on different
 *     streams with different workspaces may run concurrently.
 *   - Host-side validation failures return a status and launch nothing;
 *     dspark_last_error() (per thread) then describes the failure.  Launch
 *     failures return DSPARK_ERR_HIP.  Non-finite logits give undefined
 *     (but memory-safe) results.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dspark_status {
    DSPARK_OK = 0,
    DSPARK_ERR_INVALID_ARG = 1,        /* NULL pointer, bad size or out-of-range value */
    DSPARK_ERR_UNSUPPORTED_DTYPE = 2,  /* dtype not in dspark_dtype */
    DSPARK_ERR_WORKSPACE_TOO_SMALL = 3,
    DSPARK_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} dspark_status;

typedef enum dspark_dtype {
    DSPARK_F32 = 0,
    DSPARK_BF16 = 1
} dspark_dtype;

/* Library version string (static storage). */
const char* dspark_version(void);

/* Message for the last failed call on this thread ("" if none). */
const char* dspark_last_error(void);

/* ------------------------------------------------------------------ draft */
/* Workspace bytes dspark_draft_sample needs for these sizes (any dtype). */
size_t dspark_draft_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t r);

/*
 * Markov-head draft sampling of K tokens for each of B requests.
 *   base_logits  [B, K, V]  logit_dt    backbone logits per draft position
 *   A            [V, r]     factor_dt   transition factor looked up by the previous token
 *   W            [r, V]     factor_dt   transition factor over the next token
 *   prev_token   [B] int32              x_0, the last committed token (0 <= x_0 < V;
 *                                       an id outside is clamped to [0, V))
 *   temperature  [B] float              T per request
 *   seed                                Philox key
 * Outputs (device):
 *   draft_tokens [B, K] int32           x_1 .. x_K
 *   draft_logp   [B, K] float           log p_d(x_k) = z_{x_k} - lse_d (0 for T == 0); nullable
 *   draft_lse    [B, K] float           lse_d = log sum_v exp(z_v), z = (base + bias)/T
 *                                       (the row maximum for T == 0); nullable
 * Draws: for T > 0, x_k = argmax_v z_v + G_v with the tag-0 draw of each entry
 * v, keyed by (seed, request, position k, v): an exact sample of p_d; for
 * T == 0, x_k is the argmax of base + bias (smallest index on ties).
 * Sizes: B >= 0, K >= 0 (either 0 is a no-op), 1 <= V < 2^30, 1 <= r <= 1024.
 * A = W = NULL drafts without the Markov head: p_d(x_k) = softmax(base_k / T)
 * for every position on its own (the transition bias is zero, as with W = 0,
 * and the draws are the same), so all B x K rows are drawn in one pass;
 * x_0 is unused, r and factor_dt are ignored, and the logits must be bf16 with
 * V % 8 == 0 and a 16-byte aligned base (ERR_INVALID_ARG otherwise).  Passing
 * only one of A and W is ERR_INVALID_ARG.
 */
dspark_status dspark_draft_sample(const void* base_logits, dspark_dtype logit_dt, const void* A,
                                  const void* W, dspark_dtype factor_dt,
                                  const int32_t* prev_token, const float* temperature,
                                  uint64_t seed, int32_t B, int32_t K, int32_t V, int32_t r,
                                  int32_t* draft_tokens, float* draft_logp, float* draft_lse,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the per-device scratch behind dspark_draft_sample_noalloc (64 MiB). */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * dspark_draft_sample without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation).  Arguments, outputs, draws and errors are those of
 * dspark_draft_sample, which it shares its kernels with; the results are
 * bit-identical.  Its scratch is a fixed array of DSPARK_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends
 * (the device is the current one; `stream` must belong to it).  Sizes whose
 * dspark_draft_workspace_bytes exceeds that are refused with
 * ERR_WORKSPACE_TOO_SMALL (for K <= 2374 that admits B <= 1413 at V = 151936
 * and B <= 1638 at V = 131072).
 * The call allocates nothing: the first call on a device looks up the
 * array's address and keeps it.  Every call on a device shares the one array,
 * and nothing in it needs clearing between calls (each call writes what it
 * reads): calls that overlap on one device (on different streams, or from
 * different threads without ordering) race and give undefined results.
 */
dspark_status dspark_draft_sample_noalloc(const void* base_logits, dspark_dtype logit_dt,
                                          const void* A, const void* W, dspark_dtype factor_dt,
                                          const int32_t* prev_token, const float* temperature,
                                          uint64_t seed, int32_t B, int32_t K, int32_t V,
                                          int32_t r, int32_t* draft_tokens, float* draft_logp,
                                          float* draft_lse, void* stream);

/* --------------------------------------------------------------- schedule */
size_t dspark_schedule_workspace_bytes(int32_t B, int32_t K);

/*
 * Confidence-scheduled verification lengths.
 *   conf        [B, K] float in [0, 1]  c_k: probability that draft token k is
 *                                       accepted given that tokens 1..k-1 were
 *   budget_tokens                       target batch tokens for this step; it
 *                                       counts the B root tokens, so at most
 *                                       D = max(0, budget - B) draft tokens are chosen
 *   curve_n, curve_latency [n_points]   HOST arrays: piecewise-linear step
 *                                       latency tau(N) of the target over N batch
 *                                       tokens (strictly increasing N; constant left
 *                                       of the first point, last slope right of the
 *                                       last).  NULL / 0 = budget only.  n_points <= 64.
 * Items (b, k) are taken in order of S = c_1..c_k descending (ties: smaller k,
 * then smaller b) while fewer than D are taken, S > 0 and, with a curve, the
 * objective (B + sum of taken S) / tau(B + taken) rises strictly.
 * Outputs (device):
 *   lengths     [B] int32               L_b in [0, K], the number of draft tokens to verify
 *   row_offsets [B + 1] int64           exclusive scan of L_b + 1 (row_offsets[B] = rows)
 *   survival    [B, K] float            S (sequential fp32 products); nullable
 * Sizes: B >= 0, 0 <= K <= 64, B * K <= 2^22.
 */
dspark_status dspark_schedule(const float* conf, int32_t B, int32_t K, int64_t budget_tokens,
                              const float* curve_n, const float* curve_latency, int32_t n_points,
                              int32_t* lengths, int64_t* row_offsets, float* survival,
                              void* workspace, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------- verify */
size_t dspark_verify_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t r);

/*
 * Rejection-sampling verification of the drafted tokens.
 *   draft_tokens [B, K] int32, prev_token [B] int32, draft_logp / draft_lse
 *   [B, K] float: as written by dspark_draft_sample.
 *   base_logits [B, K, V], A [V, r], W [r, V]: the draft inputs (the draft row
 *   at the first rejected position is recomputed for the residual).  A = W =
 *   NULL verifies tokens drafted without the Markov head (zero transition
 *   bias, as dspark_draft_sample with A = W = NULL); passing only one of them
 *   is ERR_INVALID_ARG.
 *   target_logits [rows, V] logit_dt: request b's verify rows j = 1 .. L_b + 1
 *   are rows target_row_offsets[b] + j - 1 (row L_b + 1 gives the bonus).
 *   Dense layout: offsets b * (K + 1); ragged layout: dspark_schedule's
 *   row_offsets (its first B entries).
 *   n_target_rows: rows in target_logits.  A request whose rows do not lie in
 *   [0, n_target_rows) gets accepted = 0 and next_token = -1 (nothing is read).
 *   lengths [B] int32 in [0, K]: verified draft tokens per request; NULL = K.
 *   Out-of-range lengths are clamped to [0, K]; token ids are clamped to
 *   [0, V) before they index A or a target row.
 * Draws: accept x_j iff log u_j < log p_t(x_j) - log p_d(x_j) (tag 1); after
 * the first rejection, next = argmax over the entries with p_t > p_d of
 * log(p_t - p_d) + G_v (tag 2, position j*), or, if no entry is positive
 * (rounding only), argmax_v y_v + G_v with the same draws; after a full
 * acceptance, next = argmax_v y_v + G_v on row L_b + 1 (tag 2, position
 * L_b + 1).  T == 0: argmax of the target row.
 * Outputs (device):
 *   accepted    [B] int32   a_b = number of leading accepted draft tokens (<= L_b)
 *   next_token  [B] int32   residual sample at a_b + 1 when a_b < L_b, else the bonus
 *   row_lse_t   [rows] float  target log-normaliser per visited row (row maximum
 *                             for T == 0); nullable
 *   row_logratio [rows] float log p_t(x_j) - log p_d(x_j) for rows j <= L_b
 *                             (T == 0: 0 if x_j is the target argmax, else -inf;
 *                             bonus row: 0); nullable
 * Rows that belong to no request are not touched.
 * Rows read: with row_lse_t or row_logratio given, every row j = 1 .. L_b + 1
 * of every request is read and reported.  With both NULL only the rows that
 * can decide accepted and next_token are read (strict prefix: a row after the
 * first rejection changes nothing).  Positions are then verified in two
 * launches, 1 .. min(4, K + 1) and 5 .. K + 1, and a request whose first
 * rejection lies in the first is not read in the second.  accepted and
 * next_token are the same either way.
 */
dspark_status dspark_verify(const int32_t* draft_tokens, const int32_t* prev_token,
                            const float* draft_logp, const float* draft_lse,
                            const void* base_logits, dspark_dtype logit_dt, const void* A,
                            const void* W, dspark_dtype factor_dt, const void* target_logits,
                            int64_t n_target_rows, const int64_t* target_row_offsets,
                            const int32_t* lengths,
                            const float* temperature, uint64_t seed, int32_t B, int32_t K,
                            int32_t V, int32_t r, int32_t* accepted, int32_t* next_token,
                            float* row_lse_t, float* row_logratio, void* workspace,
                            size_t ws_bytes, void* stream);

/* -------------------------------------------------------------- profiling */
/*
 * Per-kernel timing with HIP events, a measurement aid beside the three calls
 * above (no page defines it).  While a session is open, each launch of a
 * kernel whose bit (1 << dspark_kernel) is in kernel_mask is bracketed by two
 * events recorded on its launch stream; the time between them is the launch's
 * duration on that stream.
 * The session is the library's one piece of process-wide state (a mutex, an
 * event pool created by begin and destroyed by end, and launch counters): one
 * session at a time, opened and closed from any thread; launches from any
 * thread or stream are recorded while it is open.  With no session open the
 * three calls above touch no state beyond their arguments and are re-entrant
 * across threads and streams (apart from per-device caches of the device's
 * compute-unit count and kernel LDS limits, filled once with atomics).
 */
typedef enum dspark_kernel {
    DSPARK_KERNEL_DRAFT_STRIP = 0,       /* draft: bias GEMM + logits + per-entry keys over vocab strips */
    DSPARK_KERNEL_DRAFT_COMBINE = 1,     /* draft: merge of the partials (token, logp, lse) */
    DSPARK_KERNEL_VERIFY_ROWS = 2,       /* verify: target normaliser and accept test per row (both launches) */
    DSPARK_KERNEL_VERIFY_RESOLVE = 3,    /* verify: strict-prefix resolution per request */
    DSPARK_KERNEL_RESIDUAL_STRIP = 4,    /* verify: residual / fallback Gumbel over a vocab strip */
    DSPARK_KERNEL_RESIDUAL_COMBINE = 5,  /* verify: merge of the residual partials */
    DSPARK_KERNEL_SCHEDULE = 6,          /* schedule: survival, selection and row offsets */
    DSPARK_KERNEL_COUNT = 7
} dspark_kernel;

/* Open a session timing at most max_launches launches (events are created
 * here; later launches are counted, not timed).  ERR_INVALID_ARG if a session
 * is already open, kernel_mask is 0 or max_launches is outside [1, 2^20];
 * ERR_HIP if events cannot be created. */
dspark_status dspark_profile_begin(uint32_t kernel_mask, int32_t max_launches);

/* Close the session: wait for every recorded event, then write per kernel id
 * (arrays of DSPARK_KERNEL_COUNT host entries, each nullable) the summed
 * milliseconds of the timed launches, the launches seen and the launches
 * timed.  Closing with no open session returns zeros. */
dspark_status dspark_profile_end(double* total_ms, int64_t* launches, int64_t* timed);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
