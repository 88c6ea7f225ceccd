/*
 * dspark_oracle.c -- plain, slow, single-threaded CPU oracle for the
 * DSpark-style draft-sample / verify / schedule hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library; the HIP product path
 * never does, and the two share no code, header, table or helper.
 *
 * Every floating-point reduction here is accumulated in fp64.  Inputs are
 * fp32 (bf16 inputs are widened exactly by the caller).  Where a float result
 * decides an integer (an argmax, an accept bit) the decision is taken on fp32
 * values, the precision of the GPU kernels.
 *
 * Sources (DSpark write-ups; "page" names the web page, then the passage):
 *   [yage]  yage.ai, "DSpark: speculative decoding and hardware scheduling",
 *           paragraph on the first-order Markov head (the softmax of the
 *           backbone logit plus a transition bias looked up from the previous
 *           token in a rank-256 V x V matrix; rejection sampling needs the
 *           exact single-step draft probability), paragraph on prefix
 *           matching, paragraph on the scheduler (survival-ordered greedy
 *           selection that stops before the throughput-curve knee).
 *   [guide] freeaitool.com, "DeepSeek DSpark complete guide", section 3.1
 *           (sequential head: after each sampling step the previous token is
 *           fed into the next distribution), section 4.1 (c_k = probability
 *           that token k is accepted given all earlier tokens were), section
 *           4.2 (greedy sort + early stop against a profiled throughput
 *           curve).
 *   [lawyer] legalagi.cn, "Reading DSpark as a lawyer", section 3
 *           (speculative decoding keeps the longest accepted prefix and is
 *           lossless), section 5 (greedy global throughput maximisation with
 *           an early stop that keeps decoding lossless).
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *           Easy as 1, 2, 3", SC'11, section 3 (the Philox bijection).
 *
 * Readings where the pages are silent (each stated once, used throughout):
 *   - random draws: Philox4x32-10 with key (seed lo32, seed hi32) and counter
 *     (v >> 2, position, request, tag); the draw for vocab index v is output
 *     word v & 3.  Tags: 0 draft Gumbel, 1 accept uniform (v = 0),
 *     2 residual / fallback / bonus Gumbel.
 *   - uniform u = ((w >> 9) + 0.5) * 2^-23, exact in fp32, in (0, 1).
 *   - Gumbel G = -log(-log u), evaluated in fp64 and rounded to fp32.
 *   - temperature T > 0 multiplies logits by the fp32 reciprocal 1/T on both
 *     the draft and the target side; T == 0 means greedy on both sides.
 *   - argmax ties go to the smallest index.
 *   - every draw is a plain Gumbel-max over the whole vocabulary, each entry
 *     with its own key: draft token x_k = argmax_v fp32(z_v + G(tag 0, v));
 *     after a rejection at row j the residual draw is argmax over the entries
 *     with r_v = p_t(v) - p_d(v) > 0 (fp64) of fp32(log r_v) + G(tag 2, v),
 *     falling back to argmax_v fp32(y_v + G(tag 2, v)) when no entry is
 *     positive (rounding only); the bonus token is argmax_v fp32(y_v + G(tag 2,
 *     v)) on row L + 1.  Gumbel-max is an exact softmax sample: the argmax of
 *     log p_v + G_v over independent standard Gumbels G_v lands on v with
 *     probability p_v.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

enum { TAG_DRAFT = 0, TAG_ACCEPT = 1, TAG_RESAMPLE = 2 };

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (SC'11, section 3).  One round multiplies words 0 and 2 by
 * the two round constants; the high halves are xored with the other two
 * words and the round key, the low halves pass through; the words are then
 * re-ordered.  The key is advanced by the two Weyl constants between rounds.
 */
ORACLE_API void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                     uint32_t out[4]) {
    const uint32_t mult0 = 0xD2511F53u, mult1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t prod0 = (uint64_t)mult0 * (uint64_t)x0;
        uint64_t prod1 = (uint64_t)mult1 * (uint64_t)x2;
        uint32_t y0 = (uint32_t)(prod1 >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)prod1;
        uint32_t y2 = (uint32_t)(prod0 >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)prod0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        k0 += weyl0;
        k1 += weyl1;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The 32-bit random word for (seed, request b, position pos, tag, vocab v). */
static uint32_t random_word(uint64_t seed, uint32_t b, uint32_t pos, uint32_t tag, uint32_t v) {
    uint32_t ctr[4] = {v >> 2, pos, b, tag};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[v & 3u];
}

ORACLE_API float oracle_uniform(uint64_t seed, uint32_t b, uint32_t pos, uint32_t tag, uint32_t v) {
    uint32_t w = random_word(seed, b, pos, tag, v);
    double u = ((double)(w >> 9) + 0.5) * (1.0 / 8388608.0); /* 2^-23 */
    return (float)u; /* exact: at most 24 significant bits */
}

ORACLE_API float oracle_gumbel(uint64_t seed, uint32_t b, uint32_t pos, uint32_t tag, uint32_t v) {
    double u = (double)oracle_uniform(seed, b, pos, tag, v);
    return (float)(-log(-log(u)));
}

/* ------------------------------------------------------------------------ */
/* Markov-head draft logits for one position ([yage] Markov-head paragraph):
 *   bias_v = sum_i A[prev, i] * W[i, v]          (rank-r factor lookup)
 *   s_v    = base_v + bias_v                     (fp32)
 *   z_v    = s_v * (1/T)  for T > 0, else s_v    (fp32)
 */
static float inv_temperature(float T) { return 1.0f / T; }

static void draft_logits(const float* base_k, const float* A, const float* W, int V, int r,
                         int prev, float T, float* s, float* z, double* scratch) {
    for (int v = 0; v < V; ++v) scratch[v] = 0.0;
    const float* a_row = A + (size_t)prev * (size_t)r;
    for (int i = 0; i < r; ++i) {
        const double a = (double)a_row[i];
        const float* w_row = W + (size_t)i * (size_t)V;
        for (int v = 0; v < V; ++v) scratch[v] += a * (double)w_row[v];
    }
    for (int v = 0; v < V; ++v) {
        float bias = (float)scratch[v];
        s[v] = base_k[v] + bias;
    }
    if (T > 0.0f) {
        const float it = inv_temperature(T);
        for (int v = 0; v < V; ++v) z[v] = s[v] * it;
    } else {
        for (int v = 0; v < V; ++v) z[v] = s[v];
    }
}

/* log sum_v exp(z_v), accumulated in fp64 around the maximum. */
static double log_sum_exp(const float* z, int V) {
    double m = -INFINITY;
    for (int v = 0; v < V; ++v)
        if ((double)z[v] > m) m = (double)z[v];
    double acc = 0.0;
    for (int v = 0; v < V; ++v) acc += exp((double)z[v] - m);
    return m + log(acc);
}

/* argmax_v z_v, smallest index on ties; *gap = best - second best. */
static int plain_argmax(const float* z, int V, double* gap) {
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (z[v] > z[best]) best = v;
    double second = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (v != best && (double)z[v] > second) second = (double)z[v];
    if (gap) *gap = (double)z[best] - second;
    return best;
}

/* Gumbel-max over v in [lo, hi): argmax_v fp32(z_v + G_v) with G keyed by
 * (seed, b, pos, tag, v). */
static int gumbel_argmax_range(const float* z, int lo, int hi, uint64_t seed, uint32_t b,
                               uint32_t pos, uint32_t tag, double* gap) {
    int best = -1;
    float best_val = -INFINITY, second_val = -INFINITY;
    for (int v = lo; v < hi; ++v) {
        float pert = z[v] + oracle_gumbel(seed, b, pos, tag, (uint32_t)v);
        if (best < 0 || pert > best_val) {
            second_val = best_val;
            best_val = pert;
            best = v;
        } else if (pert > second_val) {
            second_val = pert;
        }
    }
    if (gap) *gap = (double)best_val - (double)second_val;
    return best;
}

/* Residual draw: res[v] = p_t(v) - p_d(v) in fp64; the token is the argmax
 * over the entries with res[v] > 0 of fp32(log res[v]) + G(tag 2, v).  Returns
 * -1 when no entry is positive (the caller then falls back to p_t). */
static int residual_gumbel_argmax(const double* res, int V, uint64_t seed, uint32_t b,
                                  uint32_t pos, double* gap) {
    int best = -1;
    float best_val = -INFINITY, second_val = -INFINITY;
    for (int v = 0; v < V; ++v) {
        if (!(res[v] > 0.0)) continue;
        const float pert =
            (float)log(res[v]) + oracle_gumbel(seed, b, pos, TAG_RESAMPLE, (uint32_t)v);
        if (best < 0 || pert > best_val) {
            second_val = best_val;
            best_val = pert;
            best = v;
        } else if (pert > second_val) {
            second_val = pert;
        }
    }
    if (gap) *gap = (double)best_val - (double)second_val;
    return best;
}

/* ------------------------------------------------------------------------ */
/* Exact single-step probabilities (used by the enumeration pins).            */

/* Draft distribution p_d(. | prev) at one position; one-hot at the argmax for
 * T == 0.  The caller passes V floats of base logits for that position. */
ORACLE_API void oracle_draft_probs(const float* base_k, const float* A, const float* W, int V,
                                   int r, int prev, float T, double* p) {
    float* s = (float*)malloc(sizeof(float) * (size_t)V);
    float* z = (float*)malloc(sizeof(float) * (size_t)V);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)V);
    draft_logits(base_k, A, W, V, r, prev, T, s, z, scratch);
    if (T > 0.0f) {
        double lse = log_sum_exp(z, V);
        for (int v = 0; v < V; ++v) p[v] = exp((double)z[v] - lse);
    } else {
        int x = plain_argmax(s, V, NULL);
        for (int v = 0; v < V; ++v) p[v] = (v == x) ? 1.0 : 0.0;
    }
    free(s);
    free(z);
    free(scratch);
}

/* Target distribution of one target row under temperature T. */
ORACLE_API void oracle_target_probs(const float* t_row, int V, float T, double* p) {
    if (T > 0.0f) {
        const float it = inv_temperature(T);
        float* y = (float*)malloc(sizeof(float) * (size_t)V);
        for (int v = 0; v < V; ++v) y[v] = t_row[v] * it;
        double lse = log_sum_exp(y, V);
        for (int v = 0; v < V; ++v) p[v] = exp((double)y[v] - lse);
        free(y);
    } else {
        int x = plain_argmax(t_row, V, NULL);
        for (int v = 0; v < V; ++v) p[v] = (v == x) ? 1.0 : 0.0;
    }
}

/* ------------------------------------------------------------------------ */
/* Draft for one request ([yage] Markov head; [guide] 3.1 sequential head).
 * For k = 1..K: draft logits with the previous token (x_0 = prev0), then
 * x_k = Gumbel-argmax of z over the whole vocabulary (T > 0, tag-0 keys) or
 * argmax of s (T == 0).
 * Outputs per position: token, log p_d(x_k) = z_{x_k} - lse_d, lse_d (for T == 0
 * lse_d is the row maximum and log p_d is 0: p_d is one-hot), and the top-2
 * gap of the values the argmax was taken over. */
ORACLE_API void oracle_draft_request(const float* base /* [K][V] */, const float* A,
                                     const float* W, int V, int r, int K, int32_t prev0,
                                     float T, uint64_t seed, uint32_t b, int32_t* tokens,
                                     float* logp, float* lse, double* gap) {
    float* s = (float*)malloc(sizeof(float) * (size_t)V);
    float* z = (float*)malloc(sizeof(float) * (size_t)V);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)V);
    int prev = prev0;
    for (int k = 0; k < K; ++k) {
        const uint32_t pos = (uint32_t)(k + 1);
        draft_logits(base + (size_t)k * (size_t)V, A, W, V, r, prev, T, s, z, scratch);
        int x;
        double g;
        if (T > 0.0f) {
            double l = log_sum_exp(z, V);
            x = gumbel_argmax_range(z, 0, V, seed, b, pos, TAG_DRAFT, &g);
            lse[k] = (float)l;
            logp[k] = (float)((double)z[x] - l);
        } else {
            x = plain_argmax(s, V, &g);
            lse[k] = s[x];
            logp[k] = 0.0f;
        }
        tokens[k] = x;
        if (gap) gap[k] = g;
        prev = x;
    }
    free(s);
    free(z);
    free(scratch);
}

/* Batch form: request b uses base[b], prev0[b], T[b]. */
ORACLE_API void oracle_draft_batch(const float* base /* [B][K][V] */, const float* A,
                                   const float* W, int B, int K, int V, int r,
                                   const int32_t* prev0, const float* T, uint64_t seed,
                                   int32_t* tokens, float* logp, float* lse, double* gap) {
    for (int b = 0; b < B; ++b) {
        const size_t o = (size_t)b * (size_t)K;
        oracle_draft_request(base + o * (size_t)V, A, W, V, r, K, prev0[b], T[b], seed,
                             (uint32_t)b, tokens + o, logp + o, lse + o, gap ? gap + o : NULL);
    }
}

/* ------------------------------------------------------------------------ */
/* Verify for one request ([yage] prefix matching and Markov-head paragraphs:
 * rejection sampling against the exact draft probability; [lawyer] section 3:
 * the longest accepted prefix is kept and the result is lossless).
 *
 *   rows j = 1..L+1 of the target (row L+1 supplies the bonus token)
 *   accept x_j  iff  log u_j < log p_t(x_j) - log p_d(x_j)      (T > 0)
 *                iff  x_j == argmax t_j                          (T == 0)
 *   a = number of leading accepts (strict prefix)
 *   a < L : next ~ normalise(max(0, p_t - p_d)) at j* = a + 1, by Gumbel-max
 *           over log of the positive residual entries (tag 2); if no residual
 *           mass is left (rounding only) next ~ p_t by Gumbel-max over y.
 *           T == 0: next = argmax t_{j*}.
 *   a = L : next ~ p_t at row L + 1 (bonus), Gumbel-max over y (tag 2).
 *           T == 0: argmax t_{L+1}.
 *
 * p_d is recomputed here from the draft definition (it does not trust any
 * passed-in draft probability).
 * row_logratio[j-1] = log p_t(x_j) - log p_d(x_j) for every j <= L (T > 0);
 * for T == 0 it is 0 when x_j is the target argmax and -inf otherwise; the
 * bonus row's entry is 0.  row_lse_t is the target log-normaliser (the row
 * maximum for T == 0).
 * accept_gap = min over the decided positions of |log u - log ratio|
 * (the top-2 target gap for T == 0); next_gap = top-2 gap of the final argmax.
 * branch (nullable) says how next was drawn: 0 bonus (a = L), 1 residual (or
 * the target argmax for T == 0), 2 fallback to p_t (rejected, but no entry of
 * p_t - p_d is positive).
 */
ORACLE_API void oracle_verify_request(const int32_t* tokens /* [K] */, int32_t prev0,
                                      const float* base /* [K][V] */, const float* A,
                                      const float* W, int V, int r, int K,
                                      const float* target /* [L+1][V] */, int L, float T,
                                      uint64_t seed, uint32_t b, int32_t* accepted,
                                      int32_t* next_token, float* row_lse_t,
                                      float* row_logratio, double* accept_gap,
                                      double* next_gap, int32_t* branch) {
    float* s = (float*)malloc(sizeof(float) * (size_t)V);
    float* z = (float*)malloc(sizeof(float) * (size_t)V);
    float* y = (float*)malloc(sizeof(float) * (size_t)V);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)V);
    const float it = (T > 0.0f) ? inv_temperature(T) : 1.0f;
    double min_gap = INFINITY;
    int a = 0;
    int decided = 0;

    /* Per-row target log-normaliser and log ratio for every drafted row. */
    for (int j = 1; j <= L + 1; ++j) {
        const float* t = target + (size_t)(j - 1) * (size_t)V;
        double lse_t;
        if (T > 0.0f) {
            for (int v = 0; v < V; ++v) y[v] = t[v] * it;
            lse_t = log_sum_exp(y, V);
        } else {
            int am = plain_argmax(t, V, NULL);
            lse_t = (double)t[am];
        }
        row_lse_t[j - 1] = (float)lse_t;
        if (j == L + 1) {
            row_logratio[j - 1] = 0.0f;
            continue;
        }
        const int x = tokens[j - 1];
        const int prev = (j == 1) ? prev0 : tokens[j - 2];
        if (T > 0.0f) {
            draft_logits(base + (size_t)(j - 1) * (size_t)V, A, W, V, r, prev, T, s, z, scratch);
            double lse_d = log_sum_exp(z, V);
            double logp_d = (double)z[x] - lse_d;
            double logp_t = (double)y[x] - lse_t;
            float ratio = (float)(logp_t - logp_d);
            row_logratio[j - 1] = ratio;
            if (!decided) {
                float lu = (float)log((double)oracle_uniform(seed, b, (uint32_t)j, TAG_ACCEPT, 0));
                double g = fabs((double)lu - (double)ratio);
                if (g < min_gap) min_gap = g;
                if (lu < ratio) a++;
                else decided = 1;
            }
        } else {
            double g;
            int am = plain_argmax(t, V, &g);
            row_logratio[j - 1] = (x == am) ? 0.0f : -INFINITY;
            if (!decided) {
                if (g < min_gap) min_gap = g;
                if (x == am) a++;
                else decided = 1;
            }
        }
    }

    int next, br;
    double ng;
    if (a < L) {
        const int js = a + 1;
        const float* t = target + (size_t)(js - 1) * (size_t)V;
        if (T > 0.0f) {
            const int prev = (js == 1) ? prev0 : tokens[js - 2];
            draft_logits(base + (size_t)(js - 1) * (size_t)V, A, W, V, r, prev, T, s, z, scratch);
            double lse_d = log_sum_exp(z, V);
            for (int v = 0; v < V; ++v) y[v] = t[v] * it;
            double lse_t = log_sum_exp(y, V);
            for (int v = 0; v < V; ++v)
                scratch[v] = exp((double)y[v] - lse_t) - exp((double)z[v] - lse_d);
            next = residual_gumbel_argmax(scratch, V, seed, b, (uint32_t)js, &ng);
            if (next >= 0) {
                br = 1;
            } else {  /* no positive residual mass (rounding only): draw from p_t */
                next = gumbel_argmax_range(y, 0, V, seed, b, (uint32_t)js, TAG_RESAMPLE, &ng);
                br = 2;
            }
        } else {
            next = plain_argmax(t, V, &ng);
            br = 1;
        }
    } else {
        const float* t = target + (size_t)L * (size_t)V;
        if (T > 0.0f) {
            for (int v = 0; v < V; ++v) y[v] = t[v] * it;
            next = gumbel_argmax_range(y, 0, V, seed, b, (uint32_t)(L + 1), TAG_RESAMPLE, &ng);
        } else {
            next = plain_argmax(t, V, &ng);
        }
        br = 0;
    }
    *accepted = a;
    *next_token = next;
    if (branch) *branch = br;
    if (accept_gap) *accept_gap = min_gap;
    if (next_gap) *next_gap = ng;
    free(s);
    free(z);
    free(y);
    free(scratch);
}

/* Batch form over ragged target rows: request b's rows start at row_offset[b]
 * of target [rows][V]; L[b] rows are verified (L == NULL means K). */
ORACLE_API void oracle_verify_batch(const int32_t* tokens /* [B][K] */, const int32_t* prev0,
                                    const float* base /* [B][K][V] */, const float* A,
                                    const float* W, int B, int K, int V, int r,
                                    const float* target, const int64_t* row_offset,
                                    const int32_t* L, const float* T, uint64_t seed,
                                    int32_t* accepted, int32_t* next_token, float* row_lse_t,
                                    float* row_logratio, double* accept_gap, double* next_gap,
                                    int32_t* branch) {
    for (int b = 0; b < B; ++b) {
        const int Lb = L ? L[b] : K;
        const size_t ro = (size_t)row_offset[b];
        oracle_verify_request(tokens + (size_t)b * (size_t)K, prev0[b],
                              base + (size_t)b * (size_t)K * (size_t)V, A, W, V, r, K,
                              target + ro * (size_t)V, Lb, T[b], seed, (uint32_t)b,
                              accepted + b, next_token + b, row_lse_t + ro, row_logratio + ro,
                              accept_gap ? accept_gap + b : NULL, next_gap ? next_gap + b : NULL,
                              branch ? branch + b : NULL);
    }
}

/* ------------------------------------------------------------------------ */
/* Confidence-scheduled prefix selection ([guide] 4.1-4.2, [yage] scheduler
 * paragraph, [lawyer] section 5).
 *   S[b][k] = c[b][0] * ... * c[b][k]     (sequential fp32 products)
 *   D = max(0, budget - B)                 (the budget counts B root tokens)
 *   items (b, k) ordered by S descending, then k ascending, then b ascending
 *   take item n (0-based) while n < D and S > 0 and, if a throughput curve
 *   tau(N) is given, the objective f(N) = (B + sum of taken S) / tau(N) rises
 *   strictly when N goes from B + n to B + n + 1; stop at the first failure.
 *   L[b] = number of taken items of request b; row_offsets = exclusive scan of
 *   L[b] + 1 (B + 1 entries).
 * tau is piecewise linear through (curve_n[i], curve_tau[i]); constant left of
 * the first point, extended with the last segment's slope right of the last.
 */
typedef struct {
    float S;
    int32_t k;
    int32_t b;
} sched_item;

static int sched_cmp(const void* pa, const void* pb) {
    const sched_item* a = (const sched_item*)pa;
    const sched_item* b = (const sched_item*)pb;
    if (a->S > b->S) return -1;
    if (a->S < b->S) return 1;
    if (a->k != b->k) return a->k < b->k ? -1 : 1;
    if (a->b != b->b) return a->b < b->b ? -1 : 1;
    return 0;
}

ORACLE_API double oracle_curve_tau(const double* cn, const double* ct, int n_points, double N) {
    if (n_points <= 0) return 1.0;
    if (n_points == 1 || N <= cn[0]) return ct[0];
    for (int i = 1; i < n_points; ++i) {
        if (N <= cn[i]) {
            double f = (N - cn[i - 1]) / (cn[i] - cn[i - 1]);
            return ct[i - 1] + f * (ct[i] - ct[i - 1]);
        }
    }
    double slope = (ct[n_points - 1] - ct[n_points - 2]) / (cn[n_points - 1] - cn[n_points - 2]);
    return ct[n_points - 1] + slope * (N - cn[n_points - 1]);
}

ORACLE_API int oracle_schedule(const float* conf /* [B][K] */, int B, int K, int64_t budget,
                               const double* curve_n, const double* curve_tau, int n_points,
                               int32_t* lengths, int64_t* row_offsets, float* survival) {
    const size_t n_items = (size_t)B * (size_t)K;
    sched_item* items = (sched_item*)malloc(sizeof(sched_item) * (n_items ? n_items : 1));
    for (int b = 0; b < B; ++b) {
        float S = 1.0f;
        for (int k = 0; k < K; ++k) {
            S = S * conf[(size_t)b * (size_t)K + (size_t)k];
            survival[(size_t)b * (size_t)K + (size_t)k] = S;
            items[(size_t)b * (size_t)K + (size_t)k] = (sched_item){S, k, b};
        }
        lengths[b] = 0;
    }
    qsort(items, n_items, sizeof(sched_item), sched_cmp);
    int64_t D = budget - (int64_t)B;
    if (D < 0) D = 0;
    double E = (double)B;
    int64_t n = 0;
    for (size_t i = 0; i < n_items; ++i) {
        if (n >= D) break;
        const sched_item* it = &items[i];
        if (!(it->S > 0.0f)) break;
        if (n_points > 0) {
            double N = (double)B + (double)n;
            double f_now = E / oracle_curve_tau(curve_n, curve_tau, n_points, N);
            double f_next = (E + (double)it->S) / oracle_curve_tau(curve_n, curve_tau, n_points, N + 1.0);
            if (!(f_next > f_now)) break;
        }
        E += (double)it->S;
        lengths[it->b] += 1;
        n++;
    }
    row_offsets[0] = 0;
    for (int b = 0; b < B; ++b) row_offsets[b + 1] = row_offsets[b] + (int64_t)lengths[b] + 1;
    free(items);
    return (int)n;
}
