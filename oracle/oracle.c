/*
 * oracle.c -- plain CPU oracle for the DynamiQ hot path (TEST INFRASTRUCTURE).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this.  It shares no code with the HIP library.  See oracle.h for the
 * passages followed; each function below names the reading it implements.
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -fno-fast-math -fPIC
 *        -shared oracle.c -o liboracle.so -lm
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FAST_MATH__)
#error "the oracle must be built without fast-math"
#endif

/* ------------------------------------------------------------------ */
/* small helpers                                                       */
/* ------------------------------------------------------------------ */

static float f_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

static float bf16_to_f32(uint16_t h) { return f_from_bits((uint32_t)h << 16); }

static float load_elem(const void *g, int32_t dtype, int64_t idx) {
    if (dtype == OR_BF16) return bf16_to_f32(((const uint16_t *)g)[idx]);
    return ((const float *)g)[idx];
}

void or_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int or_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Philox4x32 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as  */
/* easy as 1, 2, 3", SC'11).  One round: two 32x32->64 products of the   */
/* even counter words with the two multipliers; the high halves are     */
/* xored with the odd words and the key, and the words are permuted.     */
/* The key advances by the two Weyl constants between rounds.           */
/* ------------------------------------------------------------------ */

void or_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds,
                   uint32_t out[4]) {
    const uint32_t MA = 0xD2511F53u, MB = 0xCD9E8D57u;
    const uint32_t WA = 0x9E3779B9u, WB = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < rounds; r++) {
        if (r > 0) { k0 += WA; k1 += WB; }
        uint64_t pa = (uint64_t)MA * (uint64_t)x0;
        uint64_t pb = (uint64_t)MB * (uint64_t)x2;
        uint32_t y0 = (uint32_t)(pb >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)pb;
        uint32_t y2 = (uint32_t)(pa >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)pa;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* ------------------------------------------------------------------ */
/* Non-uniform level table (scribe notes, "Key idea and contribution":   */
/* more levels near zero; pith review ledger: levels f(eps, r), eps not  */
/* stated).  Reading: 2^q symmetric levels on the grid                   */
/*   u_r = (2r + 1 - 2^q) / (2^q - 1),  L[r] = sign(u) phi(|u|),         */
/*   phi(t) = t * (eps + (1 - eps) t),                                   */
/* evaluated in fp64 and rounded once to fp32.  eps = 1 is the uniform   */
/* grid.  W[r] = fl32(65536 / (L[r+1] - L[r])) with the fp32 levels      */
/* widened to fp64.                                                      */
/* ------------------------------------------------------------------ */

void or_levels(int q, double eps, float *L, float *W) {
    const int Q = 1 << q;
    for (int r = 0; r < Q; r++) {
        double u = (double)(2 * r + 1 - Q) / (double)(Q - 1);
        double t = fabs(u);
        double phi = t * (eps + (1.0 - eps) * t);
        L[r] = (float)(u < 0 ? -phi : phi);
    }
    for (int r = 0; r + 1 < Q; r++)
        W[r] = (float)(65536.0 / ((double)L[r + 1] - (double)L[r]));
}

/* ------------------------------------------------------------------ */
/* context                                                             */
/* ------------------------------------------------------------------ */

struct or_ctx {
    int64_t d, J;
    int32_t n, topo, log2n;
    float budget;
    uint64_t seed;
    uint32_t round;
    int32_t rounding;
    int32_t alloc;
    int32_t own;
    double eps;
    int32_t qmax;             /* widest class: 8, or 16 with the 16-bit class */
    int32_t ncls;             /* 3 classes (2, 4, 8) or 4 (2, 4, 8, 16) */
    float Lb[3][256], Wb[3][256];
    float *L16, *W16;         /* 65536 levels of the 16-bit class (qmax 16) */
    const float *L[4], *W[4]; /* level and weight tables of each class */
    float *sum, *F, *mu;      /* J, original order */
    int32_t stats_done;
    int allocated, reordered;
    uint32_t rho_bits;
    uint8_t *width;           /* J */
    int32_t *perm, *inv;      /* J */
    int64_t C[4];             /* class counts (q = 2, 4, 8, 16) */
};

static const int Q_OF_CLASS[4] = {2, 4, 8, 16};

static int class_of_width(int q) { return q == 2 ? 0 : (q == 4 ? 1 : (q == 8 ? 2 : 3)); }

static void build_tables(or_ctx *c) {
    for (int k = 0; k < 3; k++) {
        or_levels(Q_OF_CLASS[k], c->eps, c->Lb[k], c->Wb[k]);
        c->L[k] = c->Lb[k];
        c->W[k] = c->Wb[k];
    }
    c->L[3] = c->W[3] = NULL;
    if (c->qmax == 16) {
        if (!c->L16) {
            c->L16 = (float *)malloc(65536 * sizeof(float));
            c->W16 = (float *)malloc(65536 * sizeof(float));
        }
        or_levels(16, c->eps, c->L16, c->W16);
        c->L[3] = c->L16;
        c->W[3] = c->W16;
    }
}

or_ctx *or_create(int64_t n_coords, int32_t n_workers, int32_t topology,
                  float avg_bits) {
    if (n_coords <= 0 || n_coords % OR_SG != 0 || n_workers < 1) return NULL;
    if (topology != OR_RING && topology != OR_BUTTERFLY) return NULL;
    int32_t lg = 0;
    while ((1 << lg) < n_workers) lg++;
    if (topology == OR_BUTTERFLY && (1 << lg) != n_workers) return NULL;
    if (!(avg_bits >= 2.0f)) return NULL;
    or_ctx *c = (or_ctx *)calloc(1, sizeof(or_ctx));
    c->d = n_coords;
    c->J = n_coords / OR_SG;
    c->n = n_workers;
    c->topo = topology;
    c->log2n = lg;
    c->budget = avg_bits;
    c->seed = 1;
    c->round = 0;
    c->rounding = OR_STRATIFIED;
    c->eps = 0.5;
    c->qmax = 8;
    c->ncls = 3;
    build_tables(c);
    c->sum = (float *)calloc((size_t)c->J, sizeof(float));
    c->F = (float *)calloc((size_t)c->J, sizeof(float));
    c->mu = (float *)calloc((size_t)c->J, sizeof(float));
    c->width = (uint8_t *)calloc((size_t)c->J, 1);
    c->perm = (int32_t *)calloc((size_t)c->J, sizeof(int32_t));
    c->inv = (int32_t *)calloc((size_t)c->J, sizeof(int32_t));
    return c;
}

void or_destroy(or_ctx *c) {
    if (!c) return;
    free(c->sum); free(c->F); free(c->mu);
    free(c->width); free(c->perm); free(c->inv);
    free(c->L16); free(c->W16);
    free(c);
}

void or_set_seed(or_ctx *c, uint64_t seed) { c->seed = seed; }
void or_set_round(or_ctx *c, uint32_t round) { c->round = round; }
void or_set_rounding(or_ctx *c, int32_t mode) { c->rounding = mode; }
void or_set_own(or_ctx *c, int32_t mode) { c->own = mode; }

void or_set_alloc(or_ctx *c, int32_t mode) {
    c->alloc = mode;
    c->allocated = 0;
    c->reordered = 0;
}

void or_set_eps(or_ctx *c, double eps) { c->eps = eps; build_tables(c); }

int or_set_max_width(or_ctx *c, int32_t q) {
    if (q != 8 && q != 16) return -1;
    c->qmax = q;
    c->ncls = q == 16 ? 4 : 3;
    build_tables(c);
    c->allocated = 0;
    c->reordered = 0;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stage 1: statistics (scribe notes, "Key idea and contribution": per    */
/* super-group mean and squared l2 norm, all-reduced).  Reading of the     */
/* summation order: 32 sequential partial sums of 8 consecutive entries,   */
/* then a pairwise tree P_k += P_{k+delta} for delta = 16, 8, 4, 2, 1.     */
/* Squares are fl(e*e), summed the same way.  Workers fold in rank order.  */
/* ------------------------------------------------------------------ */

static float tree_sum_256(const float *e) {
    float P[32];
    for (int k = 0; k < 32; k++) {
        float s = e[8 * k];
        for (int t = 1; t < 8; t++) s = s + e[8 * k + t];
        P[k] = s;
    }
    for (int delta = 16; delta >= 1; delta /= 2)
        for (int k = 0; k < delta; k++) P[k] = P[k] + P[k + delta];
    return P[0];
}

int or_stats(or_ctx *c, int32_t worker, const void *grad, int32_t dtype) {
    if (worker != c->stats_done) return -3;
    if (dtype != OR_BF16 && dtype != OR_F32) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < c->J; j++) {
        float e[OR_SG], e2[OR_SG];
        for (int i = 0; i < OR_SG; i++) {
            e[i] = load_elem(grad, dtype, j * OR_SG + i);
            e2[i] = e[i] * e[i];
        }
        float s = tree_sum_256(e), sq = tree_sum_256(e2);
        if (worker == 0) { c->sum[j] = s; c->F[j] = sq; }
        else { c->sum[j] = c->sum[j] + s; c->F[j] = c->F[j] + sq; }
    }
    c->stats_done++;
    c->allocated = c->reordered = 0;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stage 2: allocation (pith review, "What carries the argument": widths   */
/* {2,4,8}, thresholds locked to T12 = 5/32 T24 and T24 = 17/512 T48, one  */
/* scalar selects the whole allocation; Fig. 3 caption: thresholds over    */
/* F_j, the summed squared norm).  Reading: scalar rho >= 0 (fp32) with     */
/*   T12 = fl(85 rho), T24 = fl(544 rho), T48 = fl(16384 rho),              */
/* q_j = 8 if F_j >= T48, else 4 if F_j >= T24, else 2 (the clamp to {2,4,8}*/
/* makes T12 inert), and rho = the smallest non-negative fp32 for which     */
/* sum_j q_j <= avg_bits * J.  The count is non-increasing in rho, so the   */
/* smallest rho is found by bisection on the fp32 bit pattern.              */
/* ------------------------------------------------------------------ */

int64_t or_budget_bits(const or_ctx *c) {
    /* sum_j q_j never exceeds qmax J, so every budget of qmax bits or more */
    /* is the same constraint; capping it keeps the product finite (B may be */
    /* +inf) */
    const double cap = (double)c->qmax;
    const double b = (double)c->budget < cap ? (double)c->budget : cap;
    return (int64_t)floor(b * (double)c->J);
}

/* Threshold multipliers: T = fl(K rho).  Widths {2,4,8}: K12, K24, K48 =
 * 85, 544, 16384 (ratios 5/32 and 17/512).  With the 16-bit class the chain
 * continues with T48 / T816 = 257 / 2^17 (Fig. 3 caption); all four are
 * scaled by 257 so that they stay integers exact in fp32: 21845, 139808,
 * 4210688, 2^31. */
static void multipliers(int qmax, float K[4]) {
    if (qmax == 16) {
        K[0] = 21845.0f; K[1] = 139808.0f; K[2] = 4210688.0f; K[3] = 2147483648.0f;
    } else {
        K[0] = 85.0f; K[1] = 544.0f; K[2] = 16384.0f; K[3] = INFINITY;
    }
}

/* Widths {2,4,8} (Fig. 3 caption: the chain stops at 8 unless the 16-bit
 * class is on): 16 only with that class, so a key of +inf (an overflowed
 * squared norm) gets 8 and never a width outside the plan's set. */
static int width_of(float F, float t4, float t8, float t16, int qmax) {
    if (qmax == 16 && F >= t16) return 16;
    if (F >= t8) return 8;
    if (F >= t4) return 4;
    return 2;
}

/* the thresholds T24, T48 and T816 of rho (T816 is +inf without the 16-bit
 * class, and width_of does not consult it then) */
static void thresholds_of(int qmax, uint32_t rho_bits, float *t4, float *t8, float *t16) {
    float K[4];
    multipliers(qmax, K);
    const float rho = f_from_bits(rho_bits);
    *t4 = K[1] * rho;
    *t8 = K[2] * rho;
    *t16 = qmax == 16 ? K[3] * rho : INFINITY;
}

void or_thresholds(uint32_t rho_bits, float out[3]) {
    float rho = f_from_bits(rho_bits);
    out[0] = 85.0f * rho;     /* T12 (inert under the {2,4,8} clamp) */
    out[1] = 544.0f * rho;    /* T24 */
    out[2] = 16384.0f * rho;  /* T48 */
}

/* The squared norm of the mean-subtracted values (pith.science review,
 * referee major 1): G_j = F_j - n S mu_j^2 with S = 256, as fl(F_j -
 * fl(fl(256 n) * fl(mu_j * mu_j))), negative results (rounding) set to 0.
 * Needs mu (computed at the start of the allocation). */
static void mean_corrected_key(const or_ctx *c, float *G) {
    const float denom = (float)(256 * c->n);
    for (int64_t j = 0; j < c->J; j++) {
        const float m2 = c->mu[j] * c->mu[j];
        const float t = denom * m2;
        const float g = c->F[j] - t;
        G[j] = g < 0.0f ? 0.0f : g;
    }
}

void or_get_alloc_key(const or_ctx *c, float *out) {
    if (c->alloc == OR_ALLOC_MEAN_CORRECTED) mean_corrected_key(c, out);
    else memcpy(out, c->F, (size_t)c->J * sizeof(float));
}

static int64_t count_bits_on(const float *key, int64_t J, int qmax, uint32_t rho_bits) {
    float t4, t8, t16;
    thresholds_of(qmax, rho_bits, &t4, &t8, &t16);
    int64_t total = 0;
#pragma omp parallel for reduction(+ : total) schedule(static)
    for (int64_t j = 0; j < J; j++) total += width_of(key[j], t4, t8, t16, qmax);
    return total;
}

int64_t or_count_bits(const or_ctx *c, uint32_t rho_bits) {
    return count_bits_on(c->F, c->J, c->qmax, rho_bits);
}

void or_thresholds_wide(uint32_t rho_bits, float out[4]) {
    float K[4];
    multipliers(16, K);
    const float rho = f_from_bits(rho_bits);
    for (int k = 0; k < 4; k++) out[k] = K[k] * rho;
}

/* ------------------------------------------------------------------ */
/* Exact allocation (pith.science review, referee major 1 and "What would  */
/* settle it": compare the threshold rule with an exhaustive search over   */
/* all allocations of the same bit budget).  The error model of "What      */
/* carries the argument" charges a super-group F_j 4^-q_j; the exact       */
/* allocation minimises sum_j F_j 4^-q_j over q_j in {2,4,8} subject to    */
/* sum_j q_j <= budget_bits.  Dynamic programme over super-groups and the  */
/* bits spent above 2 per super-group, in units of 2 bits (a super-group   */
/* takes 0, 1 or 3 units), costs in fp64; ties go to fewer units.  Work    */
/* and memory grow with J times the budget: J is limited to 4096.          */
/* Returns the minimal cost, or -1 if J is out of range.                   */
/* ------------------------------------------------------------------ */

double or_alloc_exact_q(const float *F, int64_t J, int64_t budget_bits, int32_t qmax, uint8_t *widths) {
    if (J < 1 || J > 4096 || budget_bits < 2 * J || (qmax != 8 && qmax != 16)) return -1.0;
    const int ncls = qmax == 16 ? 4 : 3;
    const int units[4] = {0, 1, 3, 7};
    const double inv4q[4] = {1.0 / 16.0, 1.0 / 256.0, 1.0 / 65536.0, 1.0 / 4294967296.0};
    int64_t U = (budget_bits - 2 * J) / 2;
    if (U > (int64_t)units[ncls - 1] * J) U = (int64_t)units[ncls - 1] * J;
    double *best = (double *)malloc((size_t)(U + 1) * sizeof(double));
    double *next = (double *)malloc((size_t)(U + 1) * sizeof(double));
    uint8_t *choice = (uint8_t *)malloc((size_t)J * (size_t)(U + 1));
    /* best[u]: least cost of the super-groups so far spending exactly u units */
    for (int64_t u = 0; u <= U; u++) best[u] = u == 0 ? 0.0 : INFINITY;
    for (int64_t j = 0; j < J; j++) {
        for (int64_t u = 0; u <= U; u++) {
            double b = INFINITY;
            uint8_t ch = 0;
            for (int k = 0; k < ncls; k++) {
                if (units[k] > u) break;
                const double v = best[u - units[k]] + (double)F[j] * inv4q[k];
                if (v < b) { b = v; ch = (uint8_t)k; }
            }
            next[u] = b;
            choice[(size_t)j * (size_t)(U + 1) + (size_t)u] = ch;
        }
        double *t = best; best = next; next = t;
    }
    int64_t us = 0;
    for (int64_t u = 1; u <= U; u++)
        if (best[u] < best[us]) us = u;
    const double cost = best[us];
    for (int64_t j = J - 1; j >= 0; j--) {
        const int k = choice[(size_t)j * (size_t)(U + 1) + (size_t)us];
        widths[j] = (uint8_t)Q_OF_CLASS[k];
        us -= units[k];
    }
    free(best);
    free(next);
    free(choice);
    return cost;
}

double or_alloc_exact(const float *F, int64_t J, int64_t budget_bits, uint8_t *widths) {
    return or_alloc_exact_q(F, J, budget_bits, 8, widths);
}

int or_allocate(or_ctx *c) {
    if (c->stats_done != c->n) return -3;
    const float denom = (float)(256 * c->n);
    for (int64_t j = 0; j < c->J; j++) c->mu[j] = c->sum[j] / denom;
    const int64_t budget = or_budget_bits(c);
    c->C[0] = c->C[1] = c->C[2] = c->C[3] = 0;
    if (c->alloc == OR_ALLOC_EXACT) {
        /* the exact minimiser of the error model under the budget; no scalar */
        if (or_alloc_exact_q(c->F, c->J, budget, c->qmax, c->width) < 0.0) return -1;
        for (int64_t j = 0; j < c->J; j++) c->C[class_of_width(c->width[j])]++;
        c->rho_bits = 0x7FC00000u;
        c->allocated = 1;
        c->reordered = 0;
        return 0;
    }
    if (c->alloc == OR_ALLOC_UNIFORM) {
        /* widest q of the width set with q <= B, i.e. q J <= floor(B J) */
        const int q = (c->qmax == 16 && c->budget >= 16.0f) ? 16
                      : (c->budget >= 8.0f ? 8 : (c->budget >= 4.0f ? 4 : 2));
        for (int64_t j = 0; j < c->J; j++) c->width[j] = (uint8_t)q;
        c->C[class_of_width(q)] = c->J;
        c->rho_bits = 0x7FC00000u;
        c->allocated = 1;
        c->reordered = 0;
        return 0;
    }
    const float *key = c->F;
    float *G = NULL;
    if (c->alloc == OR_ALLOC_MEAN_CORRECTED) {
        G = (float *)malloc((size_t)c->J * sizeof(float));
        mean_corrected_key(c, G);
        key = G;
    }
    uint32_t rho;
    if (count_bits_on(key, c->J, c->qmax, 0u) <= budget) {
        rho = 0u;
    } else {
        /* at +inf every finite key has width 2; keys of +inf (overflowed
         * squared norms) keep theirs, and if the budget is missed even there,
         * rho stays at the end of the range, +inf */
        uint32_t lo = 0u, hi = 0x7F800000u;
        while (hi - lo > 1u) {
            uint32_t mid = lo + (hi - lo) / 2u;
            if (count_bits_on(key, c->J, c->qmax, mid) <= budget) hi = mid; else lo = mid;
        }
        rho = hi;
    }
    c->rho_bits = rho;
    float t4, t8, t16;
    thresholds_of(c->qmax, rho, &t4, &t8, &t16);
    for (int64_t j = 0; j < c->J; j++) {
        int q = width_of(key[j], t4, t8, t16, c->qmax);
        c->width[j] = (uint8_t)q;
        c->C[class_of_width(q)]++;
    }
    free(G);
    c->allocated = 1;
    c->reordered = 0;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stage 3: reorder (scribe notes: super-groups reordered so equal widths  */
/* are contiguous).  Reading: stable partition, widths 2, then 4, then 8.  */
/* ------------------------------------------------------------------ */

int or_reorder(or_ctx *c) {
    if (!c->allocated) return -3;
    int64_t p = 0;
    for (int k = 0; k < c->ncls; k++)
        for (int64_t j = 0; j < c->J; j++)
            if (c->width[j] == Q_OF_CLASS[k]) {
                c->perm[p] = (int32_t)j;
                c->inv[j] = (int32_t)p;
                p++;
            }
    c->reordered = 1;
    return 0;
}

void or_get_stats(const or_ctx *c, float *sum, float *F, float *mu) {
    if (sum) memcpy(sum, c->sum, (size_t)c->J * sizeof(float));
    if (F) memcpy(F, c->F, (size_t)c->J * sizeof(float));
    if (mu) memcpy(mu, c->mu, (size_t)c->J * sizeof(float));
}
uint32_t or_get_rho_bits(const or_ctx *c) { return c->rho_bits; }
void or_get_widths(const or_ctx *c, uint8_t *w) { memcpy(w, c->width, (size_t)c->J); }
void or_get_perm(const or_ctx *c, int32_t *perm, int32_t *inv) {
    if (perm) memcpy(perm, c->perm, (size_t)c->J * sizeof(int32_t));
    if (inv) memcpy(inv, c->inv, (size_t)c->J * sizeof(int32_t));
}
void or_get_class_counts(const or_ctx *c, int64_t counts[3]) {
    counts[0] = c->C[0]; counts[1] = c->C[1]; counts[2] = c->C[2];
}
void or_get_class_counts4(const or_ctx *c, int64_t counts[4]) {
    for (int k = 0; k < 4; k++) counts[k] = c->C[k];
}

/* ------------------------------------------------------------------ */
/* Parts and region layout (readings; the pages give no wire format).      */
/* Part c of m: for each width class k, stream positions                   */
/*   [base_k + floor(c C_k / m), base_k + floor((c+1) C_k / m)).           */
/* Region bytes for a part holding n_2, n_4, n_8 super-groups (N total):    */
/*   codes of the 2-bit SGs (64 B each), 4-bit (128 B), 8-bit (256 B),     */
/*   then N fp32 scale units s, zero padding to a multiple of 16 bytes,    */
/*   then N x 16 UINT8 group codes.  SGs appear in stream order.            */
/*   Code i of an SG sits at bit q*i of its payload, LSB first.             */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t lo[4], cnt[4];    /* stream positions per class */
    int64_t N;
    int64_t off_codes[4], off_s, off_c, bytes;
} part_layout;

static void layout_part(const or_ctx *c, int64_t m, int64_t part, part_layout *pl) {
    int64_t base = 0;
    pl->N = 0;
    for (int k = 0; k < 4; k++) pl->lo[k] = pl->cnt[k] = pl->off_codes[k] = 0;
    for (int k = 0; k < c->ncls; k++) {
        int64_t a = part * c->C[k] / m, b = (part + 1) * c->C[k] / m;
        pl->lo[k] = base + a;
        pl->cnt[k] = b - a;
        pl->N += b - a;
        base += c->C[k];
    }
    int64_t off = 0;
    for (int k = 0; k < c->ncls; k++) {
        pl->off_codes[k] = off;
        off += pl->cnt[k] * 32 * Q_OF_CLASS[k];
    }
    pl->off_s = off;
    off += 4 * pl->N;
    off = (off + 15) / 16 * 16;
    pl->off_c = off;
    off += 16 * pl->N;
    pl->bytes = off;
}

int64_t or_region_bytes(const or_ctx *c, int64_t m, int64_t part, int64_t counts_out[4]) {
    part_layout pl;
    layout_part(c, m, part, &pl);
    if (counts_out) for (int k = 0; k < 4; k++) counts_out[k] = pl.cnt[k];
    return pl.bytes;
}

/* index of a super-group in its part (stream order) */
static int64_t part_index(const part_layout *pl, int k, int64_t idx_in_class) {
    int64_t before = 0;
    for (int t = 0; t < k; t++) before += pl->cnt[t];
    return before + idx_in_class;
}

/* pointers to the pieces of one super-group inside a region */
typedef struct { uint8_t *codes; uint8_t *s; uint8_t *cg; int q; int k; } sg_slot;

static void slot_of(const part_layout *pl, uint8_t *region, int k, int64_t idx_in_class,
                    sg_slot *sl) {
    int64_t before = 0;
    for (int t = 0; t < k; t++) before += pl->cnt[t];
    int64_t local = before + idx_in_class;     /* index in the part, stream order */
    sl->q = Q_OF_CLASS[k];
    sl->k = k;
    sl->codes = region + pl->off_codes[k] + idx_in_class * 32 * sl->q;
    sl->s = region + pl->off_s + 4 * local;
    sl->cg = region + pl->off_c + 16 * local;
}

/* ------------------------------------------------------------------ */
/* Codec for one super-group (scribe notes: per-group scale factors with a */
/* second level of quantisation to UINT8, non-uniform levels, unbiased     */
/* stochastic rounding; pith review summary: hierarchical UINT8 group      */
/* scaling).  Readings:                                                    */
/*   a_g = max |y| over group g, A = max_g a_g;                            */
/*   s = fl(A/255), raised to the next fp32 while fl(255 s) < A;           */
/*   c_g = smallest integer in [0,255] with fl(c_g s) >= a_g;              */
/*   sigma_g = fl(c_g s);  inv_g = fl(1/sigma_g), or 0 when sigma_g = 0;   */
/*   v = clamp(fl(y inv_g), -1, 1), and v = 0 where y = 0 (which differs   */
/*   only where 1/sigma_g overflows, sigma_g < 2^-128: y * inf is NaN);    */
/*   r = largest r <= 2^q - 2 with L[r] <= v;                              */
/*   code = r + [ d + 0.5 <= fl(fl(v - L[r]) W[r]) ], d the 16-bit dither */
/*   (d + 0.5 is exact in fp32; a tie rounds up, so P(up) is              */
/*   floor(65536 p + 1/2) / 65536 for the interval fraction p, within     */
/*   2^-17 of p);  decode: fl(fl(c_g s) L[code]).                          */
/* ------------------------------------------------------------------ */

static float step_of(float A) {
    float s = A / 255.0f;
    while (255.0f * s < A) s = nextafterf(s, INFINITY);
    return s;
}

static void encode_sg(const float *y, int q, const float *L, const float *W,
                      const uint16_t *d, uint16_t *codes, float *s_out, uint8_t *cg) {
    const int Q = 1 << q;
    float a[OR_NGROUPS];
    float A = 0.0f;
    for (int g = 0; g < OR_NGROUPS; g++) {
        float m = 0.0f;
        for (int i = 0; i < OR_GROUP; i++) {
            float v = fabsf(y[g * OR_GROUP + i]);
            if (v > m) m = v;
        }
        a[g] = m;
        if (m > A) A = m;
    }
    float s = step_of(A);
    *s_out = s;
    for (int g = 0; g < OR_NGROUPS; g++) {
        int cc = 0;
        while (cc < 255 && (float)cc * s < a[g]) cc++;
        cg[g] = (uint8_t)cc;
        float sigma = (float)cc * s;
        float inv = (sigma == 0.0f) ? 0.0f : 1.0f / sigma;
        for (int i = 0; i < OR_GROUP; i++) {
            int idx = g * OR_GROUP + i;
            float v = (y[idx] == 0.0f) ? 0.0f : y[idx] * inv;
            if (v < -1.0f) v = -1.0f;
            if (v > 1.0f) v = 1.0f;
            int r;
            if (q <= 8) {
                r = Q - 2;
                while (r > 0 && L[r] > v) r--;
            } else {
                /* 65536 levels: bisection for the same r (L is increasing) */
                int lo = 0, hi = Q - 2;          /* L[lo] <= v always (L[0] = -1) */
                while (lo < hi) {
                    int mid = lo + (hi - lo + 1) / 2;
                    if (L[mid] <= v) lo = mid; else hi = mid - 1;
                }
                r = lo;
            }
            float p65536 = (v - L[r]) * W[r];
            float dd = (float)d[idx] + 0.5f;
            codes[idx] = (uint16_t)(r + (dd <= p65536 ? 1 : 0));
        }
    }
}

static void decode_sg(const uint16_t *codes, int q, const float *L, float s,
                      const uint8_t *cg, float *x) {
    (void)q;
    for (int g = 0; g < OR_NGROUPS; g++) {
        float sigma = (float)cg[g] * s;
        for (int i = 0; i < OR_GROUP; i++) {
            int idx = g * OR_GROUP + i;
            x[idx] = sigma * L[codes[idx]];
        }
    }
}

/* code i at bit q i of the payload, least significant bit first; a 16-bit
   code takes two bytes, low byte first */
static void pack_codes(const uint16_t *codes, int q, uint8_t *out) {
    memset(out, 0, (size_t)(32 * q));
    for (int i = 0; i < OR_SG; i++) {
        int bit = q * i;
        if (q == 16) {
            out[bit / 8] = (uint8_t)(codes[i] & 0xFF);
            out[bit / 8 + 1] = (uint8_t)(codes[i] >> 8);
        } else {
            out[bit / 8] |= (uint8_t)(codes[i] << (bit % 8));
        }
    }
}

static void unpack_codes(const uint8_t *in, int q, uint16_t *codes) {
    const int mask = (1 << q) - 1;
    for (int i = 0; i < OR_SG; i++) {
        int bit = q * i;
        if (q == 16) codes[i] = (uint16_t)(in[bit / 8] | (in[bit / 8 + 1] << 8));
        else codes[i] = (uint16_t)((in[bit / 8] >> (bit % 8)) & mask);
    }
}

static void write_sg(const sg_slot *sl, const uint16_t *codes, float s, const uint8_t *cg) {
    pack_codes(codes, sl->q, sl->codes);
    memcpy(sl->s, &s, 4);
    memcpy(sl->cg, cg, 16);
}

static void read_sg(const or_ctx *c, const sg_slot *sl, float *x) {
    uint16_t codes[OR_SG];
    float s;
    unpack_codes(sl->codes, sl->q, codes);
    memcpy(&s, sl->s, 4);
    decode_sg(codes, sl->q, c->L[sl->k], s, sl->cg, x);
}

/* ------------------------------------------------------------------ */
/* Dithers (scribe notes: correlated rounding shares randomness across    */
/* workers).  Reading: Philox4x32-10, key = (seed lo32, seed hi32),        */
/* counter = (i >> 3, j, round, tag) for coordinate i of super-group j     */
/* (original index); coordinate i takes word (i & 7) >> 1, its low 16 bits */
/* when i is even and its high 16 bits when odd.                           */
/*   correlated:  tag 0, d = (d0 + floor(w 65536 / n)) mod 65536, w the    */
/*                rank of the quantising worker;                           */
/*   independent: tag 1 + event, d = d0.                                   */
/* ------------------------------------------------------------------ */

void or_dithers_tagged(uint64_t seed, uint32_t round, int64_t j, uint32_t tag, uint32_t stagger,
                       uint16_t *d) {
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    for (int blk = 0; blk < 32; blk++) {
        uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)j, round, tag};
        uint32_t out[4];
        or_philox4x32(ctr, key, 10, out);
        for (int t = 0; t < 8; t++) {
            int i = blk * 8 + t;
            uint32_t word = out[t >> 1];
            uint32_t d0 = (t & 1) ? (word >> 16) : (word & 0xFFFFu);
            d[i] = (uint16_t)((d0 + stagger) & 0xFFFFu);
        }
    }
}

void or_dithers(uint64_t seed, uint32_t round, int64_t j, int32_t mode,
                int32_t worker, int32_t n_workers, int32_t event, uint16_t *d) {
    uint32_t tag = (mode == OR_CORRELATED) ? 0u : (uint32_t)(1 + event);
    uint32_t stagger = (mode == OR_CORRELATED)
                           ? (uint32_t)(((uint64_t)worker * 65536u) / (uint64_t)n_workers)
                           : 0u;
    or_dithers_tagged(seed, round, j, tag, stagger, d);
}

/* Level-stratified dithers (reading of correlated rounding that keeps every  */
/* hop unbiased; correlated-quantisation reference of the pith.science       */
/* review, "Circularity"): the workers that quantise the same coordinate in  */
/* parallel -- whose inputs do not depend on each other's rounding -- share  */
/* one uniform, staggered by their index among those workers; quantisations */
/* in series (a compress and the hops that consume it, one level and the    */
/* next) take fresh uniforms.                                                */
/*   ring:      the chain of a part is serial: step t takes tag 1 + t, no    */
/*              stagger (each part's coordinates are quantised by one worker */
/*              per step);                                                   */
/*   butterfly: the compress (sending half) takes tag 1 and the n/2 senders  */
/*              of a half are staggered by w mod (n/2); the hop of level s   */
/*              takes tag 1 + s and the 2^(L-s) workers on a part are        */
/*              staggered by w mod 2^(L-s);                                  */
/*   n = 1:     tag 1, no stagger.                                           */
/* Stagger for index k of P workers: floor(k 65536 / P).                     */
static void stratified_params(const or_ctx *c, int32_t w, int32_t step, int is_compress,
                              uint32_t *tag, uint32_t *stagger) {
    uint32_t P = 1, k = 0;
    if (c->n == 1) {
        *tag = 1u;
    } else if (c->topo == OR_RING) {
        *tag = 1u + (uint32_t)step;
    } else if (is_compress) {
        *tag = 1u;
        P = (uint32_t)(c->n / 2);
        k = (uint32_t)w % P;
    } else {
        *tag = 1u + (uint32_t)step;
        P = 1u << (c->log2n - step);
        k = (uint32_t)w % P;
    }
    *stagger = (uint32_t)(((uint64_t)k * 65536u) / P);
}

/* dithers of super-group j for the quantisation event (worker, step) */
static void event_dithers(const or_ctx *c, int64_t j, int32_t worker, int32_t step, int is_compress,
                          int32_t event, uint16_t *d) {
    if (c->rounding == OR_STRATIFIED) {
        uint32_t tag, stagger;
        stratified_params(c, worker, step, is_compress, &tag, &stagger);
        or_dithers_tagged(c->seed, c->round, j, tag, stagger, d);
    } else {
        or_dithers(c->seed, c->round, j, c->rounding, worker, c->n, event, d);
    }
}

static int event_of(const or_ctx *c, int32_t worker, int32_t step) {
    if (c->topo == OR_BUTTERFLY && c->n > 1) return (step - 1) * c->n + worker;
    return worker;
}

/* ------------------------------------------------------------------ */
/* Schedules (scribe notes: ring and butterfly multi-hop all-reduce;       */
/* readings).  Ring: worker w compresses part w at step 0; at step t it    */
/* runs the hop on part (w - t) mod n with the region worker w-1 produced  */
/* at step t-1; worker w ends with part (w+1) mod n.                       */
/* Butterfly (recursive halving, L = log2 n levels): at level s the        */
/* partner is w ^ (n >> s); after level s worker w holds part              */
/* c_s = w >> (L - s) of m = 2^s.  Level 1: compress the sibling half      */
/* (2, c_1 ^ 1), hop on (2, c_1) with the raw local gradient.  Level s>=2: */
/* hop on (2^s, c_s) with the worker's own packed child as the local       */
/* operand.  Hops below the last level write the two children of their    */
/* part (2^(s+1), 2 c_s) and (2^(s+1), 2 c_s + 1).                         */
/* ------------------------------------------------------------------ */

typedef struct { int64_t m, part; int two_children; } sched_part;

static int compress_part(const or_ctx *c, int32_t w, int32_t step, sched_part *sp) {
    sp->two_children = 0;
    if (c->n == 1) {
        if (step != 0) return -1;
        sp->m = 1; sp->part = 0; return 0;
    }
    if (c->topo == OR_RING) {
        if (step != 0) return -1;
        sp->m = c->n; sp->part = w; return 0;
    }
    if (step != 1) return -1;
    sp->m = 2;
    sp->part = ((int64_t)w >> (c->log2n - 1)) ^ 1;
    return 0;
}

static int hop_part(const or_ctx *c, int32_t w, int32_t step, sched_part *sp) {
    if (c->n == 1) return -1;
    if (c->topo == OR_RING) {
        if (step < 1 || step >= c->n) return -1;
        sp->m = c->n;
        sp->part = ((int64_t)w - step % c->n + c->n) % c->n;
        sp->two_children = 0;
        return 0;
    }
    if (step < 1 || step > c->log2n) return -1;
    sp->m = (int64_t)1 << step;
    sp->part = (int64_t)w >> (c->log2n - step);
    sp->two_children = step < c->log2n;
    return 0;
}

int64_t or_final_part(const or_ctx *c, int32_t worker) {
    if (c->n == 1) return 0;
    if (c->topo == OR_RING) return (worker + 1) % c->n;
    return worker;
}

/* enumerate (class, index-in-class) of the part's SGs, optionally filtered */
typedef struct { int k; int64_t idx; int64_t pos; } sg_ref;

static int64_t collect_refs(const part_layout *pl, const int64_t *filter, int64_t nf,
                            sg_ref **out) {
    int64_t cap = pl->N;
    sg_ref *refs = (sg_ref *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(sg_ref));
    int64_t n = 0;
    for (int k = 0; k < 4; k++) {
        int64_t lo = pl->lo[k], hi = pl->lo[k] + pl->cnt[k];
        if (!filter) {
            for (int64_t p = lo; p < hi; p++) { refs[n].k = k; refs[n].idx = p - lo; refs[n].pos = p; n++; }
        } else {
            for (int64_t f = 0; f < nf; f++) {
                int64_t p = filter[f];
                if (p >= lo && p < hi) { refs[n].k = k; refs[n].idx = p - lo; refs[n].pos = p; n++; }
            }
        }
    }
    *out = refs;
    return n;
}

int or_compress(or_ctx *c, int32_t worker, int32_t step, const void *grad,
                int32_t dtype, uint8_t *region_out, const int64_t *filter, int64_t nf) {
    if (!c->reordered) return -3;
    if (worker < 0 || worker >= c->n) return -1;
    if (dtype != OR_BF16 && dtype != OR_F32) return -1;
    sched_part sp;
    if (compress_part(c, worker, step, &sp)) return -1;
    part_layout pl;
    layout_part(c, sp.m, sp.part, &pl);
    sg_ref *refs;
    int64_t nr = collect_refs(&pl, filter, nf, &refs);
    const int event = event_of(c, worker, step);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nr; t++) {
        const int k = refs[t].k;
        const int64_t j = c->perm[refs[t].pos];
        const float mu = c->mu[j];
        float y[OR_SG];
        for (int i = 0; i < OR_SG; i++) y[i] = load_elem(grad, dtype, j * OR_SG + i) - mu;
        uint16_t d[OR_SG];
        event_dithers(c, j, worker, step, 1, event, d);
        uint16_t codes[OR_SG];
        uint8_t cg[16];
        float s;
        encode_sg(y, Q_OF_CLASS[k], c->L[k], c->W[k], d, codes, &s, cg);
        sg_slot sl;
        slot_of(&pl, region_out, k, refs[t].idx, &sl);
        write_sg(&sl, codes, s, cg);
    }
    free(refs);
    return 0;
}

int or_hop(or_ctx *c, int32_t worker, int32_t step, const uint8_t *region_in,
           const void *local, int32_t local_kind, uint8_t *out0, uint8_t *out1,
           const int64_t *filter, int64_t nf) {
    if (!c->reordered) return -3;
    if (worker < 0 || worker >= c->n) return -1;
    sched_part sp;
    if (hop_part(c, worker, step, &sp)) return -1;
    /* butterfly levels >= 2 take the worker's own kept child as the local
       operand: packed, or fp32 partial sums under OR_OWN_F32 */
    const int own32 = c->topo == OR_BUTTERFLY && c->own == OR_OWN_F32;
    const int want_own = (c->topo == OR_BUTTERFLY && step >= 2);
    const int own_kind = own32 ? OR_PARTIAL : OR_PACKED;
    if (want_own != (local_kind == own_kind)) return -1;
    if (!want_own && local_kind != OR_BF16 && local_kind != OR_F32) return -1;
    if (sp.two_children && !out1) return -1;
    /* the child this worker keeps for the next level (the other is sent) */
    const int keep = sp.two_children ? (worker >> (c->log2n - step - 1)) & 1 : -1;
    part_layout pl, ch[2];
    layout_part(c, sp.m, sp.part, &pl);
    if (sp.two_children) {
        layout_part(c, 2 * sp.m, 2 * sp.part, &ch[0]);
        layout_part(c, 2 * sp.m, 2 * sp.part + 1, &ch[1]);
    }
    sg_ref *refs;
    int64_t nr = collect_refs(&pl, filter, nf, &refs);
    const int event = event_of(c, worker, step);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nr; t++) {
        const int k = refs[t].k;
        const int64_t j = c->perm[refs[t].pos];
        const float mu = c->mu[j];
        float xin[OR_SG], y[OR_SG];
        sg_slot sin;
        slot_of(&pl, (uint8_t *)region_in, k, refs[t].idx, &sin);
        read_sg(c, &sin, xin);
        if (local_kind == OR_PACKED) {
            /* the worker's own packed partial for this part; it has the same
               layout as the incoming region */
            float xown[OR_SG];
            sg_slot sown;
            slot_of(&pl, (uint8_t *)local, k, refs[t].idx, &sown);
            read_sg(c, &sown, xown);
            for (int i = 0; i < OR_SG; i++) y[i] = xin[i] + xown[i];
        } else if (local_kind == OR_PARTIAL) {
            /* the worker's own fp32 partial sums, part order */
            const float *own = (const float *)local + part_index(&pl, k, refs[t].idx) * OR_SG;
            for (int i = 0; i < OR_SG; i++) y[i] = xin[i] + own[i];
        } else {
            for (int i = 0; i < OR_SG; i++)
                y[i] = xin[i] + (load_elem(local, local_kind, j * OR_SG + i) - mu);
        }
        const int h = sp.two_children ? (refs[t].pos < ch[0].lo[k] + ch[0].cnt[k] ? 0 : 1) : 0;
        if (own32 && h == keep) {
            /* the kept child stays fp32: no quantisation */
            float *dst = (float *)(h == 0 ? out0 : out1) +
                         part_index(&ch[h], k, refs[t].pos - ch[h].lo[k]) * OR_SG;
            memcpy(dst, y, sizeof(y));
            continue;
        }
        uint16_t d[OR_SG];
        event_dithers(c, j, worker, step, 0, event, d);
        uint16_t codes[OR_SG];
        uint8_t cg[16];
        float s;
        encode_sg(y, Q_OF_CLASS[k], c->L[k], c->W[k], d, codes, &s, cg);
        sg_slot so;
        if (sp.two_children) {
            slot_of(&ch[h], h == 0 ? out0 : out1, k, refs[t].pos - ch[h].lo[k], &so);
        } else {
            slot_of(&pl, out0, k, refs[t].idx, &so);
        }
        write_sg(&so, codes, s, cg);
    }
    free(refs);
    return 0;
}

/* Finalize (scribe notes: restore the original super-group order and add  */
/* back the subtracted mean).  Reading: the output is the sum over workers, */
/* out = fl(xhat + fl(n mu_j)) at the super-group's original position.      */
int or_finalize(or_ctx *c, int64_t part, const uint8_t *region, float *out,
                const int64_t *filter, int64_t nf) {
    if (!c->reordered) return -3;
    if (part < 0 || part >= c->n) return -1;
    part_layout pl;
    layout_part(c, c->n, part, &pl);
    sg_ref *refs;
    int64_t nr = collect_refs(&pl, filter, nf, &refs);
    const float nf32 = (float)c->n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nr; t++) {
        const int k = refs[t].k;
        const int64_t j = c->perm[refs[t].pos];
        const float add = nf32 * c->mu[j];
        float x[OR_SG];
        sg_slot sl;
        slot_of(&pl, (uint8_t *)region, k, refs[t].idx, &sl);
        read_sg(c, &sl, x);
        for (int i = 0; i < OR_SG; i++) out[j * OR_SG + i] = x[i] + add;
    }
    free(refs);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Whole round                                                         */
/* ------------------------------------------------------------------ */

static int64_t worst_region_bytes(const or_ctx *c) {
    /* every region is at most one part of m >= 2 (or the whole vector), each
       super-group at most 32 qmax code bytes + 20 */
    int64_t N = c->J + 3;
    return N * (32 * c->qmax + 20) + 64;
}

int or_allreduce(or_ctx *c, const void *const *grads, int32_t dtype, float *out) {
    int rc;
    c->stats_done = 0;
    for (int w = 0; w < c->n; w++)
        if ((rc = or_stats(c, w, grads[w], dtype))) return rc;
    if ((rc = or_allocate(c))) return rc;
    if ((rc = or_reorder(c))) return rc;
    const int64_t RB = worst_region_bytes(c);
    const int n = c->n;
    if (n == 1) {
        uint8_t *reg = (uint8_t *)calloc((size_t)RB, 1);
        rc = or_compress(c, 0, 0, grads[0], dtype, reg, NULL, 0);
        if (!rc) rc = or_finalize(c, 0, reg, out, NULL, 0);
        free(reg);
        return rc;
    }
    if (c->topo == OR_RING) {
        uint8_t *buf = (uint8_t *)calloc((size_t)(2 * n) * (size_t)RB, 1);
#define RING_BUF(w, t) (buf + ((size_t)((t) & 1) * n + (w)) * (size_t)RB)
        for (int w = 0; w < n && !rc; w++)
            rc = or_compress(c, w, 0, grads[w], dtype, RING_BUF(w, 0), NULL, 0);
        for (int t = 1; t < n && !rc; t++)
            for (int w = 0; w < n && !rc; w++)
                rc = or_hop(c, w, t, RING_BUF((w - 1 + n) % n, t - 1), grads[w], dtype,
                            RING_BUF(w, t), NULL, NULL, 0);
        for (int w = 0; w < n && !rc; w++)
            rc = or_finalize(c, or_final_part(c, w), RING_BUF(w, n - 1), out, NULL, 0);
#undef RING_BUF
        free(buf);
        return rc;
    }
    /* butterfly: per worker a compress buffer and two child buffers per level
       (sized for an fp32 partial when the kept child stays fp32) */
    const int L = c->log2n;
    const int own32 = c->own == OR_OWN_F32;
    const int64_t RBp = (c->J / 2 + 3) * OR_SG * (int64_t)sizeof(float);
    const int64_t RB2 = own32 && RBp > RB ? RBp : RB;
    uint8_t *buf = (uint8_t *)calloc((size_t)n * (size_t)(1 + 2 * L) * (size_t)RB2, 1);
#define BF_CMP(w) (buf + ((size_t)(w) * (1 + 2 * L)) * (size_t)RB2)
#define BF_OUT(w, s, h) (buf + ((size_t)(w) * (1 + 2 * L) + 1 + 2 * ((s) - 1) + (h)) * (size_t)RB2)
    for (int w = 0; w < n && !rc; w++)
        rc = or_compress(c, w, 1, grads[w], dtype, BF_CMP(w), NULL, 0);
    for (int s = 1; s <= L && !rc; s++) {
        for (int w = 0; w < n && !rc; w++) {
            const int partner = w ^ (n >> s);
            const int keep = (w >> (L - s)) & 1; /* which child of the level s-1 part */
            const uint8_t *in = (s == 1) ? BF_CMP(partner) : BF_OUT(partner, s - 1, keep);
            const void *local = (s == 1) ? grads[w] : (const void *)BF_OUT(w, s - 1, keep);
            const int kind = (s == 1) ? dtype : (own32 ? OR_PARTIAL : OR_PACKED);
            rc = or_hop(c, w, s, in, local, kind, BF_OUT(w, s, 0),
                        s < L ? BF_OUT(w, s, 1) : NULL, NULL, 0);
        }
    }
    for (int w = 0; w < n && !rc; w++)
        rc = or_finalize(c, or_final_part(c, w), BF_OUT(w, L, 0), out, NULL, 0);
#undef BF_CMP
#undef BF_OUT
    free(buf);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Codec entry points for statistical pins                             */
/* ------------------------------------------------------------------ */

void or_roundtrip_sg(const float *y, int32_t q, const uint16_t *dither, double eps,
                     float *decoded, uint16_t *codes_out, float *scale, uint8_t *cg_out) {
    float *L = (float *)malloc(65536 * sizeof(float)), *W = (float *)malloc(65536 * sizeof(float));
    or_levels(q, eps, L, W);
    uint16_t codes[OR_SG];
    uint8_t cg[16];
    float s;
    encode_sg(y, q, L, W, dither, codes, &s, cg);
    decode_sg(codes, q, L, s, cg, decoded);
    if (codes_out) memcpy(codes_out, codes, sizeof(codes));
    if (scale) *scale = s;
    if (cg_out) memcpy(cg_out, cg, 16);
    free(L);
    free(W);
}

void or_roundtrip_batch(const float *y, int64_t K, int32_t q, const uint16_t *dither,
                        double eps, float *decoded) {
    float *L = (float *)malloc(65536 * sizeof(float)), *W = (float *)malloc(65536 * sizeof(float));
    or_levels(q, eps, L, W);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < K; t++) {
        uint16_t codes[OR_SG];
        uint8_t cg[16];
        float s;
        encode_sg(y + t * OR_SG, q, L, W, dither + t * OR_SG, codes, &s, cg);
        decode_sg(codes, q, L, s, cg, decoded + t * OR_SG);
    }
    free(L);
    free(W);
}

/* ------------------------------------------------------------------ */
/* MX reference quantisers (OCP Microscaling Formats v1.0; the pages cite  */
/* MXFP8 as a baseline and MXFP4/6 as estimated baselines: pith.science    */
/* review, referee major 3).  Blocks of 32 consecutive values share an     */
/* E8M0 scale X = 2^(floor(log2 max|v|) - emax), emax = exponent of the    */
/* element format's largest normal, clamped to [2^-127, 2^127]; each v / X */
/* is rounded to nearest-even on the element grid (mbits mantissa bits,    */
/* normals from 2^emin, subnormal quantum 2^(emin - mbits)) and saturated  */
/* at the largest finite element value.                                    */
/*   E4M3 (FP8): mbits 3, emin -6, emax 8, max 448                         */
/*   E3M2 (FP6): mbits 2, emin -2, emax 4, max 28                          */
/*   E2M3 (FP6): mbits 3, emin  0, emax 2, max 7.5                         */
/*   E2M1 (FP4): mbits 1, emin  0, emax 2, max 6                           */
/* ------------------------------------------------------------------ */

typedef struct { int mbits, emin, emax; double max; } mx_elem;
static const mx_elem MX_ELEM[4] = {{3, -6, 8, 448.0}, {2, -2, 4, 28.0}, {3, 0, 2, 7.5}, {1, 0, 2, 6.0}};

static double mx_elem_round(const mx_elem *f, double v) {
    double a = fabs(v);
    if (a >= f->max) return v < 0 ? -f->max : f->max;
    if (a == 0.0) return 0.0;
    int e;
    frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) -> floor(log2 a) = e - 1 */
    int ex = e - 1;
    if (ex < f->emin) ex = f->emin;
    double quantum = ldexp(1.0, ex - f->mbits);
    double r = nearbyint(a / quantum) * quantum;
    if (r > f->max) r = f->max;
    return v < 0 ? -r : r;
}

void or_mx_roundtrip(int32_t fmt, const float *x, int64_t n, float *out) {
    const mx_elem *f = &MX_ELEM[fmt];
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (n + 31) / 32; b++) {
        int64_t lo = b * 32, hi = lo + 32 < n ? lo + 32 : n;
        double amax = 0.0;
        for (int64_t i = lo; i < hi; i++) {
            double a = fabs((double)x[i]);
            if (a > amax) amax = a;
        }
        int se = -127;
        if (amax > 0.0) {
            int e;
            frexp(amax, &e);
            se = (e - 1) - f->emax;
            if (se < -127) se = -127;
            if (se > 127) se = 127;
        }
        double X = ldexp(1.0, se);
        for (int64_t i = lo; i < hi; i++) out[i] = (float)(mx_elem_round(f, (double)x[i] / X) * X);
    }
}

void or_mxfp8_roundtrip(const float *x, int64_t n, float *out) { or_mx_roundtrip(OR_MX_E4M3, x, n, out); }

/* ------------------------------------------------------------------ */
/* MX codecs in the same schedule (reading: the pages compare DynamiQ     */
/* with MX all-reduce, scribe notes "Evaluation").  No mean subtraction   */
/* and no reorder: part c of m is super-groups [floor(cJ/m),              */
/* floor((c+1)J/m)) of the original order.  Every compress and hop        */
/* re-encodes; a hop adds the decoded incoming values and the local       */
/* values in fp32.                                                        */
/* Regions are kept as their decoded fp32 values (decoding is exact).     */
/* ------------------------------------------------------------------ */

static void mx_part(const or_ctx *c, int64_t m, int64_t part, int64_t *lo, int64_t *hi) {
    *lo = part * c->J / m * OR_SG;
    *hi = (part + 1) * c->J / m * OR_SG;
}

int or_mx_allreduce(or_ctx *c, int32_t fmt, const void *const *grads, int32_t dtype, float *out) {
    if (fmt < 0 || fmt > 3) return -1;
    const int n = c->n;
    const int64_t d = c->d;
    float *tmp = (float *)malloc((size_t)d * sizeof(float));
    if (n == 1) {
        for (int64_t i = 0; i < d; i++) tmp[i] = load_elem(grads[0], dtype, i);
        or_mx_roundtrip(fmt, tmp, d, out);
        free(tmp);
        return 0;
    }
    /* cur[w]: worker w's quantised partial on its current part (full-length
       buffers indexed by original coordinate) */
    float **cur = (float **)malloc((size_t)n * sizeof(float *));
    float **nxt = (float **)malloc((size_t)n * sizeof(float *));
    for (int w = 0; w < n; w++) {
        cur[w] = (float *)calloc((size_t)d, sizeof(float));
        nxt[w] = (float *)calloc((size_t)d, sizeof(float));
    }
    int64_t lo, hi;
    if (c->topo == OR_RING) {
        for (int w = 0; w < n; w++) {
            mx_part(c, n, w, &lo, &hi);
            for (int64_t i = lo; i < hi; i++) tmp[i] = load_elem(grads[w], dtype, i);
            or_mx_roundtrip(fmt, tmp + lo, hi - lo, cur[w] + lo);
        }
        for (int t = 1; t < n; t++) {
            for (int w = 0; w < n; w++) {
                const int src = (w - 1 + n) % n;
                mx_part(c, n, ((int64_t)w - t % n + n) % n, &lo, &hi);
                for (int64_t i = lo; i < hi; i++) tmp[i] = cur[src][i] + load_elem(grads[w], dtype, i);
                or_mx_roundtrip(fmt, tmp + lo, hi - lo, nxt[w] + lo);
            }
            float **sw = cur; cur = nxt; nxt = sw;
        }
        for (int w = 0; w < n; w++) {
            mx_part(c, n, (w + 1) % n, &lo, &hi);
            memcpy(out + lo, cur[w] + lo, (size_t)(hi - lo) * sizeof(float));
        }
    } else {
        const int L = c->log2n;
        /* level 1: each worker quantises the half it sends */
        for (int w = 0; w < n; w++) {
            mx_part(c, 2, ((int64_t)w >> (L - 1)) ^ 1, &lo, &hi);
            for (int64_t i = lo; i < hi; i++) tmp[i] = load_elem(grads[w], dtype, i);
            or_mx_roundtrip(fmt, tmp + lo, hi - lo, nxt[w] + lo);   /* nxt = sent halves */
        }
        for (int s = 1; s <= L; s++) {
            for (int w = 0; w < n; w++) {
                const int partner = w ^ (n >> s);
                mx_part(c, (int64_t)1 << s, (int64_t)w >> (L - s), &lo, &hi);
                for (int64_t i = lo; i < hi; i++) {
                    const float own = (s == 1) ? load_elem(grads[w], dtype, i) : cur[w][i];
                    const float in = (s == 1) ? nxt[partner][i] : cur[partner][i];
                    tmp[i] = in + own;
                }
                /* write into a scratch then swap after all workers of the level */
                or_mx_roundtrip(fmt, tmp + lo, hi - lo, (s == 1 ? cur[w] : nxt[w]) + lo);
            }
            if (s > 1) {
                for (int w = 0; w < n; w++) {
                    mx_part(c, (int64_t)1 << s, (int64_t)w >> (L - s), &lo, &hi);
                    memcpy(cur[w] + lo, nxt[w] + lo, (size_t)(hi - lo) * sizeof(float));
                }
            }
        }
        for (int w = 0; w < n; w++) {
            mx_part(c, n, w, &lo, &hi);
            memcpy(out + lo, cur[w] + lo, (size_t)(hi - lo) * sizeof(float));
        }
    }
    for (int w = 0; w < n; w++) { free(cur[w]); free(nxt[w]); }
    free(cur); free(nxt); free(tmp);
    return 0;
}

int or_mxfp8_allreduce(or_ctx *c, const void *const *grads, int32_t dtype, float *out) {
    return or_mx_allreduce(c, OR_MX_E4M3, grads, dtype, out);
}
