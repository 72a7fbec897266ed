/*
 * pisa_oracle.c -- plain fp64 CPU oracle for the pyramid Top-K block selection.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library. The HIP library shares no code,
 * header, table or helper with it, and it never calls the HIP library.
 *
 * What it computes, and where the method is described:
 *   - "Block Sparse Attention with Log-Linear Complexity" (qqtang-code reading
 *     note), section 3.1: level 0 is the raw keys, level 1 holds leaf blocks of
 *     C keys (ceil(N/C) of them), and every level above merges g adjacent
 *     nodes; each summary is the mean pooling of its children, which for equal
 *     groups is the mean of all raw keys under the node.
 *   - same note, section 3.2: the walk starts at the single coarsest node and,
 *     level by level, considers only the children of the previous survivors,
 *     keeps the K best and ends with the leaf-block set; a level that has at
 *     most K candidates keeps all of them without scoring.
 *   - same note, "Scoring: LogSumExp": a candidate's score is the LogSumExp
 *     of the query's dot products with its children's summaries (raw keys at
 *     the leaf level, which makes the leaf score the exact raw-key LSE).
 *   - same note, section 4.1: the query heads of one GQA group add their
 *     LSE scores into one block score and share the selection.
 *   - same note, "Scoring: LogSumExp" (the Taylor expansion that follows
 *     it): dropping log m from the expansion of the LSE of m logits around
 *     their mean and truncating it gives the two ablation scores, the mean
 *     of the logits (first order, "PISA-1") and the mean plus half their
 *     variance (second order, "PISA-2"). The walk takes any of the three.
 *   - same note, the two-stage formulation it opens with: the second stage
 *     computes attention only over the raw key and value rows that belong to
 *     the picked blocks; the attention function below is that softmax
 *     attention, causally masked.
 *   - same note, "Background: two stages, and the bottleneck in the first"
 *     (and the ai4snews summary's first paragraph): the conventional stage one
 *     the pyramid replaces scores every block summary against the query and
 *     keeps the best K -- the flat selection below, with the leaf means as the
 *     summaries; its exact counterpart scores every eligible leaf as the walk
 *     scores a leaf candidate (the LSE over its raw keys).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *   logit = q.k / sqrt(d); level sizes M_{l+1} = ceil(M_l / g) up to one node;
 *   a ragged node's summary is the mean of all raw keys it covers; a node is
 *   eligible for query position t iff its first key index is <= t, and only
 *   eligible children enter a parent's LSE (at the leaf level: raw keys > t are
 *   masked); the "at most K" rule counts eligible candidates; GQA head h maps
 *   to KV head h / (Hq/Hkv); ties rank the lower node index first; the output
 *   is the leaf set in ascending order, padded with -1; the variance of the
 *   second-order score is the population variance (1/m) of the m eligible
 *   children's logits, the one the expansion produces.
 *
 * Arithmetic: every sum, dot product, exp and log is in double precision. The
 * inputs are float arrays holding exactly the values the GPU sees (bf16 values
 * are exact in float), widened to double on use. Plain loops, no blocking.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_LEVELS 64
#define ORACLE_MAX_TOPK 256

/* candidate scores per head over the eligible children's logits z_1..z_m */
enum { SCORE_LSE = 0, SCORE_MEAN = 1, SCORE_MEAN_HALF_VAR = 2 };

typedef struct {
    int64_t N;      /* number of keys */
    int Hq, Hkv, d, C, g, topk;
    int score;      /* SCORE_* */
    int L;          /* number of levels above the raw keys */
    int64_t M[ORACLE_MAX_LEVELS + 1];     /* M[l] nodes at level l (1..L) */
    int64_t span[ORACLE_MAX_LEVELS + 1];  /* raw keys covered by a full node at level l */
    int64_t off[ORACLE_MAX_LEVELS + 1];   /* row offset of level l inside one head's pyramid */
    int64_t total;                        /* nodes over all levels 1..L */
} geom_t;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Level geometry of the pyramid over N keys (reading note, section 3.1). */
static int make_geom(geom_t* G, int64_t N, int Hq, int Hkv, int d, int C, int g, int topk) {
    memset(G, 0, sizeof(*G));
    if (N <= 0 || C <= 0 || g < 2 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0) return -1;
    G->N = N; G->Hq = Hq; G->Hkv = Hkv; G->d = d; G->C = C; G->g = g; G->topk = topk;
    int64_t m = ceil_div(N, C), sp = C, off = 0;
    int l = 1;
    for (;;) {
        if (l > ORACLE_MAX_LEVELS) return -1;
        G->M[l] = m; G->span[l] = sp; G->off[l] = off;
        off += m;
        if (m == 1) break;
        m = ceil_div(m, g);
        sp *= g;
        l++;
    }
    G->L = l;
    G->total = off;
    return 0;
}

int pisa_oracle_num_levels(int64_t N, int C, int g) {
    geom_t G;
    if (make_geom(&G, N, 1, 1, 1, C, g, 1) != 0) return -1;
    return G.L;
}

/* Writes M_1..M_L into sizes[0..L-1]; returns L. */
int pisa_oracle_level_sizes(int64_t N, int C, int g, int64_t* sizes, int max_levels) {
    geom_t G;
    if (make_geom(&G, N, 1, 1, 1, C, g, 1) != 0) return -1;
    if (G.L > max_levels) return -1;
    for (int l = 1; l <= G.L; l++) sizes[l - 1] = G.M[l];
    return G.L;
}

/*
 * Summary of every node: the arithmetic mean of all raw keys the node covers
 * (reading note, section 3.1; the mean recursion equals this for equal groups,
 * and this form also defines ragged nodes).
 * k:   float [N, Hkv, d]     (one batch element)
 * pyr: double [Hkv, total, d], level l at row offset sum_{j<l} M_j.
 */
int pisa_oracle_build_pyramid(const float* k, int64_t N, int Hkv, int d, int C, int g,
                              double* pyr, int nthreads) {
    geom_t G;
    if (make_geom(&G, N, Hkv, Hkv, d, C, g, 1) != 0) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int l = 1; l <= G.L; l++) {
        const int64_t M = G.M[l], sp = G.span[l];
        #pragma omp parallel for schedule(dynamic, 1) collapse(2)
        for (int j = 0; j < Hkv; j++) {
            for (int64_t i = 0; i < M; i++) {
                const int64_t lo = i * sp;
                const int64_t hi = (lo + sp < N) ? lo + sp : N;
                double* out = pyr + ((int64_t)j * G.total + G.off[l] + i) * d;
                for (int e = 0; e < d; e++) out[e] = 0.0;
                for (int64_t r = lo; r < hi; r++) {
                    const float* kr = k + (r * Hkv + j) * (int64_t)d;
                    for (int e = 0; e < d; e++) out[e] += (double)kr[e];
                }
                const double cnt = (double)(hi - lo);
                for (int e = 0; e < d; e++) out[e] /= cnt;
            }
        }
    }
    return 0;
}

/* First raw-key index covered by node i of level l (level 0: the key itself). */
static int64_t first_key(const geom_t* G, int l, int64_t i) {
    return l == 0 ? i : i * G->span[l];
}

static int node_exists(const geom_t* G, int l, int64_t i) {
    return l == 0 ? (i < G->N) : (i < G->M[l]);
}

/* Summary vector of node i at level l for KV head j, widened to double. */
static void node_vec(const geom_t* G, const float* k, const double* pyr, int j, int l, int64_t i,
                     double* v) {
    if (l == 0) {
        const float* kr = k + (i * G->Hkv + j) * (int64_t)G->d;
        for (int e = 0; e < G->d; e++) v[e] = (double)kr[e];
    } else {
        const double* p = pyr + ((int64_t)j * G->total + G->off[l] + i) * G->d;
        for (int e = 0; e < G->d; e++) v[e] = p[e];
    }
}

/*
 * Score of candidate `node` at level l >= 1 for query row q (all Hq heads) at
 * position t, KV head j: the sum over the group's heads of the LogSumExp of
 * the scaled dot products with the node's eligible children (reading note,
 * "Scoring: LogSumExp" and section 4.1), or of their mean, or of their mean
 * plus half their variance (the truncated expansions that follow it).
 */
static double node_score(const geom_t* G, const float* q, const float* k, const double* pyr,
                         int64_t t, int j, int l, int64_t node, double* scratch) {
    const int GQ = G->Hq / G->Hkv, d = G->d;
    const int nchild_max = (l == 1) ? G->C : G->g;
    const int64_t first_child = (l == 1) ? node * G->C : node * G->g;
    double* z = scratch;                   /* [nchild_max] */
    double* v = scratch + nchild_max;      /* [d] */
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double S = 0.0;
    for (int hh = 0; hh < GQ; hh++) {
        const int h = j * GQ + hh;
        const float* qh = q + (int64_t)h * d;
        int nz = 0;
        for (int c = 0; c < nchild_max; c++) {
            const int64_t r = first_child + c;
            if (!node_exists(G, l - 1, r)) break;
            if (first_key(G, l - 1, r) > t) break;        /* not eligible */
            node_vec(G, k, pyr, j, l - 1, r, v);
            double dot = 0.0;
            for (int e = 0; e < d; e++) dot += (double)qh[e] * v[e];
            z[nz++] = dot * inv_sqrt_d;
        }
        if (G->score == SCORE_LSE) {
            /* log(sum exp(z)), evaluated around the maximum for range safety */
            double m = -INFINITY;
            for (int c = 0; c < nz; c++) if (z[c] > m) m = z[c];
            double s = 0.0;
            for (int c = 0; c < nz; c++) s += exp(z[c] - m);
            S += m + log(s);
        } else {
            double mean = 0.0;
            for (int c = 0; c < nz; c++) mean += z[c];
            mean /= nz;
            double var = 0.0;
            for (int c = 0; c < nz; c++) var += (z[c] - mean) * (z[c] - mean);
            var /= nz;
            S += (G->score == SCORE_MEAN) ? mean : mean + 0.5 * var;
        }
    }
    return S;
}

typedef struct { double s; int64_t node; } scored_t;

/* higher score first; equal scores: lower node index first */
static int cmp_scored(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->node < y->node) ? -1 : (x->node > y->node);
}

static int cmp_i64(const void* a, const void* b) {
    const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x < y) ? -1 : (x > y);
}

/* Eligible, existing children at level l of the nodes in surv (level l+1). */
static int expand(const geom_t* G, int l, const int64_t* surv, int nsurv, int64_t t, int64_t* cand) {
    int n = 0;
    for (int s = 0; s < nsurv; s++) {
        for (int c = 0; c < G->g; c++) {
            const int64_t ch = surv[s] * G->g + c;
            if (ch < G->M[l] && first_key(G, l, ch) <= t) cand[n++] = ch;
        }
    }
    qsort(cand, n, sizeof(int64_t), cmp_i64);
    return n;
}

typedef struct {
    int n, cap;
    int32_t* level;
    int64_t* node;
    double* score;
    int32_t* kept;
} trace_t;

static void trace_add(trace_t* tr, int l, int64_t node, double s, int kept) {
    if (!tr || tr->n >= tr->cap) { if (tr) tr->n++; return; }
    tr->level[tr->n] = l; tr->node[tr->n] = node; tr->score[tr->n] = s; tr->kept[tr->n] = kept;
    tr->n++;
}

/*
 * One coarse-to-fine walk (reading note, section 3.2) for query position t and
 * KV head j. Writes the ascending leaf set (-1 padded) to out[topk]; returns
 * the smallest gap S_(K) - S_(K+1) over the scored levels (INFINITY if no level
 * was scored) and the level where it occurred.
 */
static void walk_one(const geom_t* G, const float* q, const float* k, const double* pyr,
                     int64_t t, int j, int32_t* out, double* min_gap, int32_t* gap_level,
                     trace_t* tr) {
    const int K = G->topk;
    const int maxc = G->g * K + 1;
    int64_t* cand = (int64_t*)malloc(sizeof(int64_t) * maxc);
    int64_t* surv = (int64_t*)malloc(sizeof(int64_t) * maxc);
    scored_t* sc = (scored_t*)malloc(sizeof(scored_t) * maxc);
    double* scratch = (double*)malloc(sizeof(double) * (G->C + G->g + G->d + 8));
    int nsurv = 0;
    double mg = INFINITY;
    int32_t ml = -1;
    for (int l = G->L; l >= 1; l--) {
        int ncand;
        if (l == G->L) { cand[0] = 0; ncand = 1; }   /* the root covers key 0, always eligible */
        else ncand = expand(G, l, surv, nsurv, t, cand);
        if (ncand <= K) {                             /* at most K candidates: keep all, no scoring */
            for (int c = 0; c < ncand; c++) { surv[c] = cand[c]; trace_add(tr, l, cand[c], NAN, 1); }
            nsurv = ncand;
            continue;
        }
        for (int c = 0; c < ncand; c++) {
            sc[c].node = cand[c];
            sc[c].s = node_score(G, q, k, pyr, t, j, l, cand[c], scratch);
        }
        qsort(sc, ncand, sizeof(scored_t), cmp_scored);
        const double gap = sc[K - 1].s - sc[K].s;
        if (gap < mg) { mg = gap; ml = l; }
        for (int c = 0; c < ncand; c++) trace_add(tr, l, sc[c].node, sc[c].s, c < K);
        for (int c = 0; c < K; c++) surv[c] = sc[c].node;
        nsurv = K;
    }
    qsort(surv, nsurv, sizeof(int64_t), cmp_i64);
    for (int c = 0; c < K; c++) out[c] = (c < nsurv) ? (int32_t)surv[c] : -1;
    if (min_gap) *min_gap = mg;
    if (gap_level) *gap_level = ml;
    free(cand); free(surv); free(sc); free(scratch);
}

/*
 * Batch of walks. q_rows: float [n_rows, Hq, d], the query rows of positions
 * t_rows[i]; k: float [N, Hkv, d]; pyr from pisa_oracle_build_pyramid.
 * Outputs: out_idx int32 [n_rows, Hkv, topk], min_gap double [n_rows, Hkv],
 * gap_level int32 [n_rows, Hkv] (may be NULL).
 */
int pisa_oracle_walk(const float* q_rows, const int64_t* t_rows, int64_t n_rows,
                     const float* k, const double* pyr, int64_t N, int Hq, int Hkv, int d,
                     int C, int g, int topk, int score, int32_t* out_idx, double* min_gap,
                     int32_t* gap_level, int nthreads) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -1;
    if (make_geom(&G, N, Hq, Hkv, d, C, g, topk) != 0) return -1;
    if (score < SCORE_LSE || score > SCORE_MEAN_HALF_VAR) return -1;
    G.score = score;
    for (int64_t i = 0; i < n_rows; i++) if (t_rows[i] < 0 || t_rows[i] >= N) return -2;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t total = n_rows * Hkv;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t w = 0; w < total; w++) {
        const int64_t i = w / Hkv;
        const int j = (int)(w % Hkv);
        walk_one(&G, q_rows + i * (int64_t)Hq * d, k, pyr, t_rows[i], j,
                 out_idx + w * topk, min_gap ? min_gap + w : NULL,
                 gap_level ? gap_level + w : NULL, NULL);
    }
    return 0;
}

/*
 * One walk with every considered candidate recorded: level, node, score (NaN
 * when the level was kept whole without scoring) and whether it survived.
 * Returns the number of entries (may exceed cap; then only cap are written).
 */
int pisa_oracle_walk_trace(const float* q_row, int64_t t, int j, const float* k, const double* pyr,
                           int64_t N, int Hq, int Hkv, int d, int C, int g, int topk, int score_mode,
                           int32_t* out_idx, int32_t* lvl, int64_t* node, double* score,
                           int32_t* kept, int cap) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -1;
    if (make_geom(&G, N, Hq, Hkv, d, C, g, topk) != 0) return -1;
    if (score_mode < SCORE_LSE || score_mode > SCORE_MEAN_HALF_VAR) return -1;
    G.score = score_mode;
    if (t < 0 || t >= N || j < 0 || j >= Hkv) return -2;
    trace_t tr = {0, cap, lvl, node, score, kept};
    walk_one(&G, q_row, k, pyr, t, j, out_idx, NULL, NULL, &tr);
    return tr.n;
}

/* Exposes one node score (for the brute-force pins). */
double pisa_oracle_node_score(const float* q_row, int64_t t, int j, const float* k,
                              const double* pyr, int64_t N, int Hq, int Hkv, int d, int C,
                              int g, int l, int64_t node, int score) {
    geom_t G;
    if (make_geom(&G, N, Hq, Hkv, d, C, g, 1) != 0) return NAN;
    if (score < SCORE_LSE || score > SCORE_MEAN_HALF_VAR) return NAN;
    G.score = score;
    if (l < 1 || l > G.L || node < 0 || node >= G.M[l]) return NAN;
    if (first_key(&G, l, node) > t) return NAN;
    double* scratch = (double*)malloc(sizeof(double) * (G.C + G.g + G.d + 8));
    const double s = node_score(&G, q_row, k, pyr, t, j, l, node, scratch);
    free(scratch);
    return s;
}

/*
 * Near-tie validation. A result is valid if some resolution of near-ties
 * reaches it: at every scored level, each candidate scoring more than eps
 * above the K-th score is kept, each scoring more than eps below it is
 * dropped, and the candidates within eps of it fill the remaining places in
 * any combination. The search is pruned by the target: every ancestor of a
 * target leaf must survive its level.
 */
typedef struct {
    const geom_t* G;
    const float *q, *k;
    const double* pyr;
    int64_t t;
    int j;
    double eps;
    const int64_t* target;   /* sorted ascending, ntarget entries */
    int ntarget;
    long budget;
    double* scratch;
} vctx_t;

static int is_required(const vctx_t* V, int l, int64_t node) {
    /* node at level l is an ancestor of some target leaf */
    const int64_t div = V->G->span[l] / V->G->C;   /* leaves per full node at level l */
    for (int i = 0; i < V->ntarget; i++) if (V->target[i] / div == node) return 1;
    return 0;
}

static int same_set(const int64_t* a, int na, const int64_t* b, int nb) {
    if (na != nb) return 0;
    for (int i = 0; i < na; i++) if (a[i] != b[i]) return 0;
    return 1;
}

static int vwalk(vctx_t* V, int l, const int64_t* surv, int nsurv);

/* choose `need` more nodes from band[from..] into chosen[], then recurse */
static int vchoose(vctx_t* V, int l, int64_t* chosen, int nch, const int64_t* band, int nband,
                   int from, int need) {
    if (need == 0) {
        int64_t* s = (int64_t*)malloc(sizeof(int64_t) * (nch + 1));
        memcpy(s, chosen, sizeof(int64_t) * nch);
        qsort(s, nch, sizeof(int64_t), cmp_i64);
        const int r = vwalk(V, l - 1, s, nch);
        free(s);
        return r;
    }
    int unverified = 0;
    for (int i = from; i <= nband - need; i++) {
        if (--V->budget < 0) return -1;
        chosen[nch] = band[i];
        const int r = vchoose(V, l, chosen, nch + 1, band, nband, i + 1, need - 1);
        if (r == 1) return 1;
        if (r < 0) unverified = 1;
    }
    return unverified ? -1 : 0;
}

/* surv: survivors at level l+1 (sorted); explores level l and below */
static int vwalk(vctx_t* V, int l, const int64_t* surv, int nsurv) {
    const geom_t* G = V->G;
    const int K = G->topk;
    if (l == 0) {
        return same_set(surv, nsurv, V->target, V->ntarget);
    }
    const int maxc = G->g * K + 1;
    int64_t* cand = (int64_t*)malloc(sizeof(int64_t) * maxc);
    int ncand;
    if (l == G->L) { cand[0] = 0; ncand = 1; }
    else ncand = expand(G, l, surv, nsurv, V->t, cand);
    int result;
    if (ncand <= K) {
        result = vwalk(V, l - 1, cand, ncand);
        free(cand);
        return result;
    }
    scored_t* sc = (scored_t*)malloc(sizeof(scored_t) * ncand);
    for (int c = 0; c < ncand; c++) {
        sc[c].node = cand[c];
        sc[c].s = node_score(G, V->q, V->k, V->pyr, V->t, V->j, l, cand[c], V->scratch);
    }
    qsort(sc, ncand, sizeof(scored_t), cmp_scored);
    const double sK = sc[K - 1].s;
    /* surely kept (< K of them) plus band members forced by the target (up to K) can
     * exceed K before the check below: room for every candidate */
    int64_t* chosen = (int64_t*)malloc(sizeof(int64_t) * ncand);
    int64_t* band = (int64_t*)malloc(sizeof(int64_t) * ncand);
    int nch = 0, nband = 0, ok = 1;
    for (int c = 0; c < ncand; c++) {
        const int req = is_required(V, l, sc[c].node);
        if (sc[c].s > sK + V->eps) chosen[nch++] = sc[c].node;         /* surely kept */
        else if (sc[c].s < sK - V->eps) { if (req) ok = 0; }           /* surely dropped */
        else if (req) chosen[nch++] = sc[c].node;                       /* band, forced by target */
        else band[nband++] = sc[c].node;
    }
    if (!ok || nch > K) result = 0;
    else result = vchoose(V, l, chosen, nch, band, nband, 0, K - nch);
    free(chosen); free(band); free(sc); free(cand);
    return result;
}

/*
 * Returns 1 if `target` (topk entries, -1 padded, any order) is reachable by a
 * resolution of near-ties within eps, 0 if it is not, -1 if the search budget
 * ran out first.
 */
int pisa_oracle_validate(const float* q_row, int64_t t, int j, const float* k, const double* pyr,
                         int64_t N, int Hq, int Hkv, int d, int C, int g, int topk, int score,
                         const int32_t* target, double eps, long budget) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -2;
    if (make_geom(&G, N, Hq, Hkv, d, C, g, topk) != 0) return -2;
    if (score < SCORE_LSE || score > SCORE_MEAN_HALF_VAR) return -2;
    G.score = score;
    if (t < 0 || t >= N || j < 0 || j >= Hkv) return -2;
    int64_t tg[ORACLE_MAX_TOPK];
    int nt = 0;
    for (int i = 0; i < topk; i++) if (target[i] >= 0) tg[nt++] = target[i];
    qsort(tg, nt, sizeof(int64_t), cmp_i64);
    for (int i = 1; i < nt; i++) if (tg[i] == tg[i - 1]) return 0;   /* duplicate leaf */
    vctx_t V;
    V.G = &G; V.q = q_row; V.k = k; V.pyr = pyr; V.t = t; V.j = j; V.eps = eps;
    V.target = tg; V.ntarget = nt; V.budget = budget;
    V.scratch = (double*)malloc(sizeof(double) * (G.C + G.g + G.d + 8));
    const int r = vwalk(&V, G.L, NULL, 0);
    free(V.scratch);
    return r;
}

/*
 * Stage two: attention over the selected blocks ("Block Sparse Attention with
 * Log-Linear Complexity", the two-stage formulation at the top of the note:
 * the second stage restricts attention to the raw key/value rows of the picked
 * blocks). For query row i at position t and query head h (KV head j = h / GQ),
 * the keys are those of the blocks idx[i][j][0..topk-1] (entries < 0 ignored;
 * block b holds keys b*C .. min((b+1)*C, N) - 1) that are <= t (causal); the
 * output is the softmax of q.k / sqrt(d) over those keys applied to their value
 * rows. A row whose key set is empty gets zeros.
 *   q_rows [n_rows][Hq][d], k and v [N][Hkv][d], idx [n_rows][Hkv][topk],
 *   out [n_rows][Hq][d] (double).
 */
int pisa_oracle_attention(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const float* k,
                          const float* v, const int32_t* idx, int64_t N, int Hq, int Hkv, int d, int C,
                          int topk, double* out, int nthreads) {
    if (n_rows < 0 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1 || C < 1 || topk < 1) return -1;
    const int GQ = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)d);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t i = 0; i < n_rows; i++) {
        const int64_t t = t_rows[i];
        if (t < 0 || t >= N) { bad = 1; continue; }
        double* z = (double*)malloc(sizeof(double) * (size_t)topk * (size_t)C);
        int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)topk * (size_t)C);
        for (int h = 0; h < Hq; h++) {
            const int j = h / GQ;
            const float* q = q_rows + (i * Hq + h) * (int64_t)d;
            /* the key set: every key <= t of every selected block */
            int64_t nk = 0;
            for (int s = 0; s < topk; s++) {
                const int64_t b = idx[(i * Hkv + j) * (int64_t)topk + s];
                if (b < 0) continue;
                for (int64_t r = b * C; r < (b + 1) * C && r < N && r <= t; r++) key[nk++] = r;
            }
            double* o = out + (i * Hq + h) * (int64_t)d;
            for (int e = 0; e < d; e++) o[e] = 0.0;
            if (nk == 0) continue;
            double zmax = -INFINITY;
            for (int64_t a = 0; a < nk; a++) {
                const float* kr = k + (key[a] * Hkv + j) * (int64_t)d;
                double dot = 0.0;
                for (int e = 0; e < d; e++) dot += (double)q[e] * (double)kr[e];
                z[a] = dot * scale;
                if (z[a] > zmax) zmax = z[a];
            }
            double den = 0.0;
            for (int64_t a = 0; a < nk; a++) {
                z[a] = exp(z[a] - zmax);
                den += z[a];
            }
            for (int64_t a = 0; a < nk; a++) {
                const float* vr = v + (key[a] * Hkv + j) * (int64_t)d;
                const double w = z[a] / den;
                for (int e = 0; e < d; e++) o[e] += w * (double)vr[e];
            }
        }
        free(z);
        free(key);
    }
    return bad ? -1 : 0;
}


/*
 * Flat stage-one selection ("Block Sparse Attention with Log-Linear Complexity",
 * "Background: two stages, and the bottleneck in the first"; ai4snews summary, first
 * paragraph): every leaf block has a mean-pooled summary (level 1 of the pyramid), and
 * each query scores ALL of them and keeps the K best -- no hierarchy. Readings (the score
 * formula is stripped on the pages): the score of block b for query position t and KV
 * head j is the sum over the group's query heads of q_{t,h} . kbar_b / sqrt(d), the
 * group aggregation the note's section 4.1 gives for the pyramid's scores; block b is
 * eligible iff its first key b*C <= t (its summary covers all its keys, as at the upper
 * levels of the walk); equal scores rank the lower index first; the output is the
 * selected set in ascending order, -1 padded (all eligible blocks when at most K are).
 */
static double flat_score(const geom_t* G, const float* q, const double* pyr, int j, int64_t b) {
    const int GQ = G->Hq / G->Hkv, d = G->d;
    const double* kb = pyr + ((int64_t)j * G->total + G->off[1] + b) * d;
    double S = 0.0;
    for (int hh = 0; hh < GQ; hh++) {
        const float* qh = q + (int64_t)(j * GQ + hh) * d;
        double dot = 0.0;
        for (int e = 0; e < d; e++) dot += (double)qh[e] * kb[e];
        S += dot / sqrt((double)d);
    }
    return S;
}

/* Scores of the eligible blocks of position t, sorted in selection order; returns their count. */
static int64_t flat_sorted(const geom_t* G, const float* q, const double* pyr, int64_t t, int j, scored_t* sc) {
    int64_t n = t / G->C + 1;
    if (n > G->M[1]) n = G->M[1];
    for (int64_t b = 0; b < n; b++) {
        sc[b].node = b;
        sc[b].s = flat_score(G, q, pyr, j, b);
    }
    qsort(sc, (size_t)n, sizeof(scored_t), cmp_scored);
    return n;
}

/* The K best of a sorted candidate list, ascending, -1 padded; the gap S_(K) - S_(K+1)
 * (INFINITY when at most K candidates are eligible). */
static void flat_keep(const scored_t* sc, int64_t n, int topk, int32_t* out, double* gap) {
    int64_t keep[ORACLE_MAX_TOPK];
    const int nk = (n < topk) ? (int)n : topk;
    for (int c = 0; c < nk; c++) keep[c] = sc[c].node;
    qsort(keep, (size_t)nk, sizeof(int64_t), cmp_i64);
    for (int c = 0; c < topk; c++) out[c] = (c < nk) ? (int32_t)keep[c] : -1;
    if (gap) *gap = (n > topk) ? sc[topk - 1].s - sc[topk].s : INFINITY;
}

/* 1 if `target` (topk entries, -1 padded, any order) is the K best of the sorted list sc[0..n)
 * under some resolution of the scores within eps of the K-th score: it holds min(K, n)
 * distinct eligible candidates, every one scoring more than eps above the K-th, and none
 * scoring more than eps below it. */
static int flat_check(const scored_t* sc, int64_t n, int topk, const int32_t* target, double eps) {
    const int want = (n < topk) ? (int)n : topk;
    int ok = 1, cnt = 0;
    for (int c = 0; c < topk && ok; c++) {
        const int32_t b = target[c];
        if (b < 0) continue;
        if (b >= n) { ok = 0; break; }                       /* not eligible */
        for (int e = 0; e < c; e++) if (target[e] == b) ok = 0;   /* duplicate */
        cnt++;
    }
    if (ok && cnt != want) ok = 0;
    if (ok && n > topk) {
        const double sK = sc[topk - 1].s;
        for (int64_t r = 0; r < n && ok; r++) {
            int in = 0;
            for (int c = 0; c < topk; c++) if (target[c] == sc[r].node) in = 1;
            if (sc[r].s > sK + eps && !in) ok = 0;           /* surely kept, missing */
            if (sc[r].s < sK - eps && in) ok = 0;            /* surely dropped, present */
        }
    }
    return ok;
}

/*
 * Flat selection for the query rows of positions t_rows (one batch element).
 * q_rows: float [n_rows, Hq, d]; pyr from pisa_oracle_build_pyramid over N keys.
 * Outputs: out_idx int32 [n_rows, Hkv, topk] (ascending, -1 padded), min_gap double
 * [n_rows, Hkv] = S_(K) - S_(K+1) (INFINITY when at most K blocks are eligible).
 */
int pisa_oracle_flat_select(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const double* pyr,
                            int64_t N, int Hq, int Hkv, int d, int C, int topk, int32_t* out_idx,
                            double* min_gap, int nthreads) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -1;
    if (make_geom(&G, N, Hq, Hkv, d, C, 2, topk) != 0) return -1;
    for (int64_t i = 0; i < n_rows; i++) if (t_rows[i] < 0 || t_rows[i] >= N) return -2;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t total = n_rows * Hkv;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t w = 0; w < total; w++) {
        const int64_t i = w / Hkv;
        const int j = (int)(w % Hkv);
        scored_t* sc = (scored_t*)malloc(sizeof(scored_t) * (size_t)G.M[1]);
        const int64_t n = flat_sorted(&G, q_rows + i * (int64_t)Hq * d, pyr, t_rows[i], j, sc);
        flat_keep(sc, n, topk, out_idx + w * topk, min_gap ? min_gap + w : NULL);
        free(sc);
    }
    return 0;
}

/* Near-tie check of a flat selection (flat_check) for position t, KV head j. */
int pisa_oracle_flat_validate(const float* q_row, int64_t t, int j, const double* pyr, int64_t N, int Hq,
                              int Hkv, int d, int C, int topk, const int32_t* target, double eps) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -2;
    if (make_geom(&G, N, Hq, Hkv, d, C, 2, topk) != 0) return -2;
    if (t < 0 || t >= N || j < 0 || j >= Hkv) return -2;
    scored_t* sc = (scored_t*)malloc(sizeof(scored_t) * (size_t)G.M[1]);
    const int64_t n = flat_sorted(&G, q_row, pyr, t, j, sc);
    const int ok = flat_check(sc, n, topk, target, eps);
    free(sc);
    return ok;
}

/*
 * Flat selection by the exact leaf score (the exhaustive selection by the walk's own leaf
 * score, against which the walk's choice of blocks is measured): every eligible leaf block b
 * (b*C <= t) is scored the way the walk scores a candidate at the leaf level -- the sum over
 * the group's heads of the LogSumExp of the scaled dot products with the block's raw keys up
 * to t (node_score at level 1; reading note, "Scoring: LogSumExp" and section 4.1) -- and the
 * K best are kept, with no hierarchy. Equal scores rank the lower block first.
 */
static int64_t flat_exact_sorted(const geom_t* G, const float* q, const float* k, int64_t t, int j,
                                 scored_t* sc, double* scratch) {
    int64_t n = t / G->C + 1;
    if (n > G->M[1]) n = G->M[1];
    for (int64_t b = 0; b < n; b++) {
        sc[b].node = b;
        sc[b].s = node_score(G, q, k, NULL, t, j, 1, b, scratch);
    }
    qsort(sc, (size_t)n, sizeof(scored_t), cmp_scored);
    return n;
}

/*
 * Exact flat selection for the query rows of positions t_rows (one batch element).
 * q_rows: float [n_rows, Hq, d]; k: float [N, Hkv, d] raw keys. Outputs as
 * pisa_oracle_flat_select.
 */
int pisa_oracle_flat_exact_select(const float* q_rows, const int64_t* t_rows, int64_t n_rows, const float* k,
                                  int64_t N, int Hq, int Hkv, int d, int C, int topk, int32_t* out_idx,
                                  double* min_gap, int nthreads) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -1;
    if (make_geom(&G, N, Hq, Hkv, d, C, 2, topk) != 0) return -1;
    G.score = SCORE_LSE;
    for (int64_t i = 0; i < n_rows; i++) if (t_rows[i] < 0 || t_rows[i] >= N) return -2;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t total = n_rows * Hkv;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t w = 0; w < total; w++) {
        const int64_t i = w / Hkv;
        const int j = (int)(w % Hkv);
        scored_t* sc = (scored_t*)malloc(sizeof(scored_t) * (size_t)G.M[1]);
        double* scratch = (double*)malloc(sizeof(double) * (size_t)(C + d));
        const int64_t n = flat_exact_sorted(&G, q_rows + i * (int64_t)Hq * d, k, t_rows[i], j, sc, scratch);
        flat_keep(sc, n, topk, out_idx + w * topk, min_gap ? min_gap + w : NULL);
        free(scratch);
        free(sc);
    }
    return 0;
}

/* Near-tie check of an exact flat selection (flat_check) for position t, KV head j. */
int pisa_oracle_flat_exact_validate(const float* q_row, int64_t t, int j, const float* k, int64_t N, int Hq,
                                    int Hkv, int d, int C, int topk, const int32_t* target, double eps) {
    geom_t G;
    if (topk < 1 || topk > ORACLE_MAX_TOPK) return -2;
    if (make_geom(&G, N, Hq, Hkv, d, C, 2, topk) != 0) return -2;
    G.score = SCORE_LSE;
    if (t < 0 || t >= N || j < 0 || j >= Hkv) return -2;
    scored_t* sc = (scored_t*)malloc(sizeof(scored_t) * (size_t)G.M[1]);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(C + d));
    const int64_t n = flat_exact_sorted(&G, q_row, k, t, j, sc, scratch);
    const int ok = flat_check(sc, n, topk, target, eps);
    free(scratch);
    free(sc);
    return ok;
}
