/*
 * oracle_sanitize_main.c -- drives every entry point of oracle/pisa_oracle.c on small
 * inputs so that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks the
 * oracle's memory accesses and integer arithmetic (tests/test_oracle_sanitize.py builds and
 * runs it on the CPU). Exit status 0 when every call returned what is expected.
 *
 * Cases: ragged lengths, group sizes 1..16, budgets K = 1..32, all three scores, walk
 * traces, node scores, attention, and near-tie validation -- a valid tied alternative, and
 * an invalid target whose tied ancestors fill the band while K - 1 candidates are surely
 * kept (the case where the candidate list holds up to 2K - 1 entries before the check).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int pisa_oracle_num_levels(int64_t N, int C, int g);
int pisa_oracle_level_sizes(int64_t N, int C, int g, int64_t* sizes, int max_levels);
int pisa_oracle_build_pyramid(const float* k, int64_t N, int Hkv, int d, int C, int g, double* pyr, int nthreads);
int pisa_oracle_walk(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const float* k, const double* pyr,
                     int64_t N, int Hq, int Hkv, int d, int C, int g, int topk, int score, int32_t* out_idx,
                     double* min_gap, int32_t* gap_level, int nthreads);
int pisa_oracle_walk_trace(const float* q_row, int64_t t, int j, const float* k, const double* pyr, int64_t N, int Hq,
                           int Hkv, int d, int C, int g, int topk, int score_mode, int32_t* out_idx, int32_t* lvl,
                           int64_t* node, double* score, int32_t* kept, int cap);
double pisa_oracle_node_score(const float* q_row, int64_t t, int j, const float* k, const double* pyr, int64_t N,
                              int Hq, int Hkv, int d, int C, int g, int l, int64_t node, int score);
int pisa_oracle_validate(const float* q_row, int64_t t, int j, const float* k, const double* pyr, int64_t N, int Hq,
                         int Hkv, int d, int C, int g, int topk, int score, const int32_t* target, double eps,
                         long budget);
int pisa_oracle_attention(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const float* k, const float* v,
                          const int32_t* idx, int64_t N, int Hq, int Hkv, int d, int C, int topk, double* out,
                          int nthreads);
int pisa_oracle_flat_select(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const double* pyr,
                            int64_t N, int Hq, int Hkv, int d, int C, int topk, int32_t* out_idx,
                            double* min_gap, int nthreads);
int pisa_oracle_flat_validate(const float* q_row, int64_t t, int j, const double* pyr, int64_t N, int Hq,
                              int Hkv, int d, int C, int topk, const int32_t* target, double eps);
int pisa_oracle_flat_exact_select(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const float* k,
                                  int64_t N, int Hq, int Hkv, int d, int C, int topk, int32_t* out_idx,
                                  double* min_gap, int nthreads);
int pisa_oracle_flat_exact_validate(const float* q_row, int64_t t, int j, const float* k, int64_t N, int Hq,
                                    int Hkv, int d, int C, int topk, const int32_t* target, double eps);

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            ++failures;                                    \
        }                                                  \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static float uniform_pm1(void) {   /* xorshift64*, mapped to [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    const uint64_t x = rng_state * 0x2545f4914f6cdd1dull;
    return (float)((double)(x >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static float* rand_array(size_t n) {
    float* a = (float*)malloc(sizeof(float) * n);
    for (size_t i = 0; i < n; ++i) a[i] = uniform_pm1();
    return a;
}

static int64_t pyr_rows(int64_t N) {
    int64_t sizes[64];
    const int L = pisa_oracle_level_sizes(N, 64, 2, sizes, 64);
    int64_t tot = 0;
    for (int l = 0; l < L; ++l) tot += sizes[l];
    return tot;
}

/* random inputs: every position walked, traced at a few positions, node scores, attention */
static void random_case(int64_t N, int Hq, int Hkv, int K, int score) {
    const int d = 64, C = 64, g = 2;
    float* q = rand_array((size_t)N * Hq * d);
    float* k = rand_array((size_t)N * Hkv * d);
    float* v = rand_array((size_t)N * Hkv * d);
    const int64_t P = pyr_rows(N);
    double* pyr = (double*)malloc(sizeof(double) * (size_t)Hkv * P * d);
    CHECK(pisa_oracle_build_pyramid(k, N, Hkv, d, C, g, pyr, 2) == 0, "build N=%lld", (long long)N);
    /* every position of short sequences; every 9th one (and the last) of longer ones */
    const int64_t stride = (N * Hq > 8000) ? 9 : 1;
    const int64_t nt = (N - 1) / stride + 1 + ((N - 1) % stride != 0);
    int64_t* ts = (int64_t*)malloc(sizeof(int64_t) * (size_t)nt);
    for (int64_t i = 0; i < nt; ++i) ts[i] = (i * stride < N) ? i * stride : N - 1;
    /* query rows of the walked positions */
    float* qr = (float*)malloc(sizeof(float) * (size_t)nt * Hq * d);
    for (int64_t i = 0; i < nt; ++i) memcpy(qr + i * Hq * d, q + ts[i] * Hq * d, sizeof(float) * Hq * d);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)nt * Hkv * K);
    double* gap = (double*)malloc(sizeof(double) * (size_t)nt * Hkv);
    int32_t* lvl = (int32_t*)malloc(sizeof(int32_t) * (size_t)nt * Hkv);
    CHECK(pisa_oracle_walk(qr, ts, nt, k, pyr, N, Hq, Hkv, d, C, g, K, score, idx, gap, lvl, 2) == 0, "walk");
    for (int64_t i = 0; i < nt; i += (nt > 7 ? nt / 7 : 1)) {
        const int64_t t = ts[i];
        for (int j = 0; j < Hkv; ++j) {
            const int cap = 4096;
            int32_t out[64], lv[4096], kept[4096];
            int64_t nd[4096];
            double sc[4096];
            const int n = pisa_oracle_walk_trace(q + t * Hq * d, t, j, k, pyr, N, Hq, Hkv, d, C, g, K, score, out, lv,
                                                 nd, sc, kept, cap);
            CHECK(n >= 1, "trace t=%lld", (long long)t);
            CHECK(memcmp(out, idx + (i * Hkv + j) * K, sizeof(int32_t) * K) == 0, "trace result t=%lld", (long long)t);
            /* a validated exact result is always reachable */
            CHECK(pisa_oracle_validate(q + t * Hq * d, t, j, k, pyr, N, Hq, Hkv, d, C, g, K, score,
                                       idx + (i * Hkv + j) * K, 1e-3, 200000) != 0,
                  "validate own result t=%lld", (long long)t);
            const double s = pisa_oracle_node_score(q + t * Hq * d, t, j, k, pyr, N, Hq, Hkv, d, C, g, 1, t / C, score);
            CHECK(isfinite(s), "node score t=%lld", (long long)t);
        }
    }
    double* att = (double*)malloc(sizeof(double) * (size_t)nt * Hq * d);
    CHECK(pisa_oracle_attention(qr, ts, nt, k, v, idx, N, Hq, Hkv, d, C, K, att, 2) == 0, "attention");
    free(att);
    /* both flat selections, each validating its own result */
    int32_t* fidx = (int32_t*)malloc(sizeof(int32_t) * (size_t)nt * Hkv * K);
    double* fgap = (double*)malloc(sizeof(double) * (size_t)nt * Hkv);
    CHECK(pisa_oracle_flat_select(qr, ts, nt, pyr, N, Hq, Hkv, d, C, K, fidx, fgap, 2) == 0, "flat");
    CHECK(pisa_oracle_flat_validate(qr, ts[0], 0, pyr, N, Hq, Hkv, d, C, K, fidx, 1e-3) == 1, "flat validate");
    CHECK(pisa_oracle_flat_exact_select(qr, ts, nt, k, N, Hq, Hkv, d, C, K, fidx, fgap, 2) == 0, "flat exact");
    CHECK(pisa_oracle_flat_exact_validate(qr, ts[0], 0, k, N, Hq, Hkv, d, C, K, fidx, 1e-3) == 1,
          "flat exact validate");
    free(fidx);
    free(fgap);
    free(q); free(qr); free(k); free(v); free(pyr); free(ts); free(idx); free(gap); free(lvl);
}

/*
 * Invalid target over a tied band: 16 leaves (N = 1024, K = 8, one head), so only the leaf
 * level is scored. Leaves 0..6 hold keys whose first coordinate is 1 (score log 64 + 1/8
 * with q = e_0), leaves 7..15 hold zero keys (score log 64, an exact 9-way tie). The oracle
 * keeps 0..7. Target {8..15} omits seven surely kept leaves and forces eight band leaves:
 * it must be rejected (0). Target {0..6, 15} resolves the tie differently: valid (1).
 */
static void band_case(void) {
    const int64_t N = 1024;
    const int Hq = 1, Hkv = 1, d = 64, C = 64, g = 2, K = 8;
    float* q = (float*)calloc((size_t)N * Hq * d, sizeof(float));
    float* k = (float*)calloc((size_t)N * Hkv * d, sizeof(float));
    for (int64_t r = 0; r < N; ++r) q[r * d] = 1.0f;
    for (int64_t r = 0; r < 7 * C; ++r) k[r * d] = 1.0f;
    const int64_t P = pyr_rows(N);
    double* pyr = (double*)malloc(sizeof(double) * (size_t)P * d);
    CHECK(pisa_oracle_build_pyramid(k, N, Hkv, d, C, g, pyr, 1) == 0, "band build");
    const int64_t t = N - 1;
    int32_t out[8];
    double gap;
    int32_t lvl;
    CHECK(pisa_oracle_walk(q + t * d, &t, 1, k, pyr, N, Hq, Hkv, d, C, g, K, 0, out, &gap, &lvl, 1) == 0, "band walk");
    for (int i = 0; i < K; ++i) CHECK(out[i] == i, "band walk slot %d = %d", i, out[i]);
    CHECK(gap == 0.0, "band gap %g", gap);
    const int32_t bad[8] = {8, 9, 10, 11, 12, 13, 14, 15};
    CHECK(pisa_oracle_validate(q + t * d, t, 0, k, pyr, N, Hq, Hkv, d, C, g, K, 0, bad, 1e-3, 200000) == 0,
          "band invalid target accepted");
    const int32_t alt[8] = {0, 1, 2, 3, 4, 5, 6, 15};
    CHECK(pisa_oracle_validate(q + t * d, t, 0, k, pyr, N, Hq, Hkv, d, C, g, K, 0, alt, 1e-3, 200000) == 1,
          "band alternative rejected");
    const int32_t dup[8] = {0, 1, 2, 3, 4, 5, 6, 6};
    CHECK(pisa_oracle_validate(q + t * d, t, 0, k, pyr, N, Hq, Hkv, d, C, g, K, 0, dup, 1e-3, 200000) == 0,
          "duplicate leaf accepted");
    /* a target missing a surely kept leaf is rejected */
    const int32_t late[8] = {1, 2, 3, 4, 5, 6, 14, 15};
    CHECK(pisa_oracle_validate(q + t * d, t, 0, k, pyr, N, Hq, Hkv, d, C, g, K, 0, late, 1e-3, 200000) == 0,
          "target without a surely kept leaf accepted");
    free(q); free(k); free(pyr);
}

/* Every level a 2-way or wider exact tie (zero keys), K = 1..32: validate enumerates bands. */
static void zero_keys_case(int K) {
    const int64_t N = 5000;
    const int Hq = 4, Hkv = 2, d = 64, C = 64, g = 2;
    float* q = rand_array((size_t)N * Hq * d);
    float* k = (float*)calloc((size_t)N * Hkv * d, sizeof(float));
    const int64_t P = pyr_rows(N);
    double* pyr = (double*)malloc(sizeof(double) * (size_t)Hkv * P * d);
    CHECK(pisa_oracle_build_pyramid(k, N, Hkv, d, C, g, pyr, 2) == 0, "zero build");
    const int64_t ts[3] = {N - 1, N / 2, 64 * K};
    for (int i = 0; i < 3; ++i) {
        const int64_t t = ts[i] < N ? ts[i] : N - 1;
        int32_t out[64];
        double gap[2];
        int32_t lvl[2];
        CHECK(pisa_oracle_walk(q + t * Hq * d, &t, 1, k, pyr, N, Hq, Hkv, d, C, g, K, 0, out, gap, lvl, 1) == 0,
              "zero walk");
        for (int j = 0; j < Hkv; ++j) {
            const int r = pisa_oracle_validate(q + t * Hq * d, t, j, k, pyr, N, Hq, Hkv, d, C, g, K, 0, out + j * K,
                                               1e-3, 2000);
            CHECK(r != 0, "zero-key walk rejected K=%d t=%lld", K, (long long)t);
            /* the reversed leaf set of the same size: reachable or undecided, never a crash */
            int32_t rev[64];
            int n = 0;
            for (int s = 0; s < K; ++s) if (out[j * K + s] >= 0) ++n;
            const int64_t nleaf = t / C + 1;
            for (int s = 0; s < K; ++s) rev[s] = (s < n) ? (int32_t)(nleaf - 1 - s) : -1;
            (void)pisa_oracle_validate(q + t * Hq * d, t, j, k, pyr, N, Hq, Hkv, d, C, g, K, 0, rev, 1e-3, 2000);
        }
    }
    free(q); free(k); free(pyr);
}

int main(void) {
    CHECK(pisa_oracle_num_levels(262144, 64, 2) == 13, "levels at 256K");
    CHECK(pisa_oracle_num_levels(0, 64, 2) == -1, "levels of an empty sequence");
    band_case();
    const int64_t lengths[] = {1, 2, 63, 64, 65, 1000, 2500};
    const int groups[][2] = {{4, 1}, {32, 2}, {6, 3}, {16, 16}};
    const int budgets[] = {1, 4, 8, 32};
    int c = 0;
    for (size_t a = 0; a < sizeof(lengths) / sizeof(lengths[0]); ++a)
        for (size_t b = 0; b < sizeof(groups) / sizeof(groups[0]); ++b) {
            const int K = budgets[c % 4];
            random_case(lengths[a], groups[b][0], groups[b][1], K, c % 3);
            ++c;
        }
    for (int K = 1; K <= 32; K *= 2) zero_keys_case(K);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
