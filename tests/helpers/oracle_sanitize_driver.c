/*
 * oracle_sanitize_driver.c -- runs every entry point of the CPU oracle
 * (oracle/dspark_oracle.c) on small seeded inputs, edge cases included, so that
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer can report any
 * out-of-bounds access, leak or undefined operation.  Exits non-zero if an
 * output leaves its documented range.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
float oracle_uniform(uint64_t seed, uint32_t b, uint32_t pos, uint32_t tag, uint32_t v);
float oracle_gumbel(uint64_t seed, uint32_t b, uint32_t pos, uint32_t tag, uint32_t v);
void oracle_draft_probs(const float* base_k, const float* A, const float* W, int V, int r, int prev,
                        float T, double* p);
void oracle_target_probs(const float* t_row, int V, float T, double* p);
void oracle_draft_batch(const float* base, const float* A, const float* W, int B, int K, int V,
                        int r, const int32_t* prev0, const float* T, uint64_t seed,
                        int32_t* tokens, float* logp, float* lse, double* gap);
void oracle_verify_batch(const int32_t* tokens, const int32_t* prev0, const float* base,
                         const float* A, const float* W, int B, int K, int V, int r,
                         const float* target, const int64_t* row_offset, const int32_t* L,
                         const float* T, uint64_t seed, int32_t* accepted, int32_t* next_token,
                         float* row_lse_t, float* row_logratio, double* accept_gap,
                         double* next_gap, int32_t* branch);
double oracle_curve_tau(const double* cn, const double* ct, int n_points, double N);
int oracle_schedule(const float* conf, int B, int K, int64_t budget, const double* curve_n,
                    const double* curve_tau, int n_points, int32_t* lengths,
                    int64_t* row_offsets, float* survival);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double unif(void) {  /* xorshift64*, enough for test inputs */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normal(double sd) {
    double u1 = unif() + 1e-12, u2 = unif();
    return (float)(sd * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            failures++;                                                 \
        }                                                               \
    } while (0)

static void draft_and_verify(int B, int K, int V, int r, const float* temps, int ntemps,
                             int with_lengths) {
    float* base = malloc(sizeof(float) * (size_t)B * K * V + 4);
    float* A = malloc(sizeof(float) * (size_t)V * r);
    float* W = malloc(sizeof(float) * (size_t)r * V);
    int32_t* prev = malloc(sizeof(int32_t) * (size_t)B);
    float* T = malloc(sizeof(float) * (size_t)B);
    for (size_t i = 0; i < (size_t)B * K * V; ++i) base[i] = normal(2.0);
    for (size_t i = 0; i < (size_t)V * r; ++i) A[i] = normal(0.3);
    for (size_t i = 0; i < (size_t)r * V; ++i) W[i] = normal(0.3);
    for (int b = 0; b < B; ++b) {
        prev[b] = (int32_t)(unif() * V) % V;
        T[b] = temps[b % ntemps];
    }
    int32_t* tok = malloc(sizeof(int32_t) * (size_t)B * K + 4);
    float* logp = malloc(sizeof(float) * (size_t)B * K + 4);
    float* lse = malloc(sizeof(float) * (size_t)B * K + 4);
    double* gap = malloc(sizeof(double) * (size_t)B * K + 8);
    oracle_draft_batch(base, A, W, B, K, V, r, prev, T, 42, tok, logp, lse, gap);
    for (size_t i = 0; i < (size_t)B * K; ++i) {
        CHECK(tok[i] >= 0 && tok[i] < V);
        CHECK(logp[i] <= 1e-6f);
    }
    int32_t* L = malloc(sizeof(int32_t) * (size_t)B);
    int64_t* offs = malloc(sizeof(int64_t) * (size_t)(B + 1));
    offs[0] = 0;
    for (int b = 0; b < B; ++b) {
        L[b] = with_lengths ? (int32_t)(unif() * (K + 1)) % (K + 1) : K;
        offs[b + 1] = offs[b] + L[b] + 1;
    }
    const size_t rows = (size_t)offs[B];
    float* target = malloc(sizeof(float) * rows * V);
    for (size_t i = 0; i < rows * (size_t)V; ++i) target[i] = normal(2.0);
    int32_t* acc = malloc(sizeof(int32_t) * (size_t)B);
    int32_t* nxt = malloc(sizeof(int32_t) * (size_t)B);
    int32_t* br = malloc(sizeof(int32_t) * (size_t)B);
    float* rl = malloc(sizeof(float) * rows);
    float* rr = malloc(sizeof(float) * rows);
    double* ag = malloc(sizeof(double) * (size_t)B);
    double* ng = malloc(sizeof(double) * (size_t)B);
    oracle_verify_batch(tok, prev, base, A, W, B, K, V, r, target, offs,
                        with_lengths ? L : NULL, T, 42, acc, nxt, rl, rr, ag, ng, br);
    for (int b = 0; b < B; ++b) {
        CHECK(acc[b] >= 0 && acc[b] <= L[b]);
        CHECK(nxt[b] >= 0 && nxt[b] < V);
        CHECK(br[b] >= 0 && br[b] <= 2);
    }
    double* p = malloc(sizeof(double) * (size_t)V);
    if (K > 0) {
        oracle_draft_probs(base, A, W, V, r, prev[0], temps[0], p);
        double sum = 0.0;
        for (int v = 0; v < V; ++v) sum += p[v];
        CHECK(fabs(sum - 1.0) < 1e-9);
    }
    oracle_target_probs(target, V, temps[0], p);
    free(p);
    free(base); free(A); free(W); free(prev); free(T); free(tok); free(logp); free(lse);
    free(gap); free(L); free(offs); free(target); free(acc); free(nxt); free(br); free(rl);
    free(rr); free(ag); free(ng);
}

/* The rejection whose residual has no positive entry (fallback to p_t). */
static void fallback_case(void) {
    enum { V = 40, r = 2 };
    float base[V], A[V * r] = {0}, W[r * V] = {0}, target[2 * V];
    for (int v = 0; v < V; ++v) base[v] = normal(1.0);
    base[7] = -200.0f;
    for (int v = 0; v < V; ++v) {
        target[v] = base[v];
        target[V + v] = normal(1.0);
    }
    target[7] = -201.0f;
    int32_t tok = 7, prev = 0, L = 1, acc, nxt, br;
    int64_t off = 0;
    float T = 1.0f, rl[2], rr[2];
    double ag, ng;
    int fallbacks = 0;
    for (uint64_t seed = 0; seed < 64; ++seed) {
        oracle_verify_batch(&tok, &prev, base, A, W, 1, 1, V, r, target, &off, &L, &T, seed,
                            &acc, &nxt, rl, rr, &ag, &ng, &br);
        CHECK(nxt >= 0 && nxt < V);
        CHECK(br == 0 || (br == 2 && acc == 0 && nxt != 7));  /* x = 7 has no mass left */
        fallbacks += (br == 2);
    }
    CHECK(fallbacks > 0);
}

static void schedule_cases(void) {
    const double cn[2] = {16.0, 32.0}, ct[2] = {1.0, 2.5};
    for (int B = 0; B <= 9; B += 3) {
        for (int K = 0; K <= 5; K += 1) {
            float* conf = malloc(sizeof(float) * (size_t)B * K + 4);
            float* surv = malloc(sizeof(float) * (size_t)B * K + 4);
            int32_t* len = malloc(sizeof(int32_t) * (size_t)B + 4);
            int64_t* offs = malloc(sizeof(int64_t) * (size_t)(B + 1));
            for (int i = 0; i < B * K; ++i) conf[i] = (float)unif();
            if (B * K > 0) conf[0] = 0.0f;
            for (int64_t budget = 0; budget <= 40; budget += 7) {
                for (int curve = 0; curve < 2; ++curve) {
                    int n = oracle_schedule(conf, B, K, budget, curve ? cn : NULL,
                                            curve ? ct : NULL, curve ? 2 : 0, len, offs, surv);
                    CHECK(n >= 0);
                    CHECK(offs[0] == 0);
                    for (int b = 0; b < B; ++b) CHECK(len[b] >= 0 && len[b] <= K);
                }
            }
            free(conf); free(surv); free(len); free(offs);
        }
    }
    CHECK(oracle_curve_tau(cn, ct, 2, 48.0) > 2.5);
    CHECK(oracle_curve_tau(cn, ct, 0, 1.0) == 1.0);
}

int main(void) {
    uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4];
    oracle_philox4x32_10(ctr, key, out);
    for (uint32_t v = 0; v < 64; ++v) {
        float u = oracle_uniform(7, 1, 2, 0, v);
        CHECK(u > 0.0f && u < 1.0f);
        CHECK(isfinite(oracle_gumbel(7, 1, 2, 2, v)));
    }
    const float mixed[3] = {0.0f, 0.7f, 1.0f};
    const float one[1] = {1.0f};
    draft_and_verify(5, 3, 37, 4, mixed, 3, 1);
    draft_and_verify(4, 2, 1, 3, one, 1, 0);   /* V = 1 */
    draft_and_verify(3, 1, 9, 16, mixed, 3, 0);
    draft_and_verify(6, 4, 130, 8, mixed, 3, 1);
    draft_and_verify(2, 0, 11, 2, one, 1, 0);  /* K = 0: bonus only */
    fallback_case();
    schedule_cases();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
