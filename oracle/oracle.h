/*
 * oracle.h -- plain, slow CPU oracle for the DynamiQ hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  The product
 * path (the HIP library and its Python binding) never calls it, and the two
 * share no code, headers, tables or constants.
 *
 * What is computed follows the DynamiQ pages:
 *   - scribe notes (everythinginsigcomm), "Key idea and contribution":
 *     groups of 16 and super-groups of 256 consecutive coordinates, per
 *     super-group mean and squared l2 norm all-reduced, identical bit
 *     allocation on every worker, reorder by bitwidth, hop-by-hop
 *     decompress-accumulate-recompress, restore order and add back the mean,
 *     non-uniform levels, hierarchical UINT8 group scales, correlated rounding;
 *   - pith.science review, "What carries the argument" and Fig. 3 caption:
 *     widths {2,4,8}, thresholds locked by T12 = 5/32 T24, T24 = 17/512 T48,
 *     one scalar selects the allocation.
 * Every step the pages leave open is fixed by one stated reading, given in
 * the comment of the function that implements it; the oracle implements
 * those readings literally.
 *
 * Floating point: IEEE fp32, round to nearest even, no contraction (built with
 * -ffp-contract=off, no fast-math), denormals preserved.
 *
 * Threading: OpenMP over super-groups; every per-super-group computation is
 * independent and every reduction is sequential or integer, so results do not
 * depend on the thread count.
 *
 * Pins: tests/test_oracle_pins.py checks every function here against
 * something other than itself: exact rationals and hand-derived fixtures
 * (tests/golden/), closed forms, brute force on small inputs, Monte Carlo
 * unbiasedness, and independent implementations (rocRAND's Philox4x32-10,
 * torch's float8_e4m3fn rounding).  No function is left unpinned.
 */
#ifndef DQ_ORACLE_H
#define DQ_ORACLE_H
#include <stdint.h>
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { OR_SG = 256, OR_GROUP = 16, OR_NGROUPS = 16 };
enum { OR_RING = 0, OR_BUTTERFLY = 1 };
enum { OR_BF16 = 0, OR_F32 = 1, OR_PACKED = 2, OR_PARTIAL = 3 };
/* The worker's own operand at butterfly levels >= 2 (scribe notes: no
 * intermediate tensors, so the method re-quantises the half it keeps;
 * the fp32 variant keeps that half unquantised, as fp32 partial sums in the
 * part's stream order, 256 floats per super-group):
 *   OR_OWN_PACKED  the kept child is a packed region, local kind OR_PACKED
 *   OR_OWN_F32     the kept child is fp32, local kind OR_PARTIAL */
enum { OR_OWN_PACKED = 0, OR_OWN_F32 = 1 };
/* Rounding modes (scribe notes, "Key idea and contribution": correlated
 * rounding, shared randomness across workers; pith.science review, "Core
 * claim": unbiased at each hop):
 *   OR_CORRELATED   one shared uniform per coordinate for every quantisation
 *                   of every worker, staggered by the quantising worker's
 *                   rank (biased along serial hops)
 *   OR_INDEPENDENT  a fresh uniform per quantisation event
 *   OR_STRATIFIED   a fresh uniform per level (serial events independent, so
 *                   every hop is unbiased), shared and staggered among the
 *                   workers that quantise a coordinate in parallel */
enum { OR_CORRELATED = 0, OR_INDEPENDENT = 1, OR_STRATIFIED = 2 };
/* Allocation variants (pith.science review, referee major 1: the thresholds
 * see F_j although the quantised values have squared norm F_j - n S mu_j^2,
 * and Table 6 compares variable with uniform widths):
 *   OR_ALLOC_THRESHOLD      the method: thresholds on F_j
 *   OR_ALLOC_MEAN_CORRECTED thresholds on G_j = max(F_j - fl(256 n) mu_j^2, 0)
 *   OR_ALLOC_UNIFORM        every super-group at the widest q in {2,4,8}
 *                           with q <= B (rho reported as NaN) */
enum { OR_ALLOC_THRESHOLD = 0, OR_ALLOC_MEAN_CORRECTED = 1, OR_ALLOC_UNIFORM = 2, OR_ALLOC_EXACT = 3 };
/* OR_ALLOC_EXACT: the minimiser of sum_j F_j 4^-q_j under the same budget
 * (exhaustive in effect: a dynamic programme; J <= 4096), the comparison the
 * review's referee asks for; rho is reported as NaN. */

typedef struct or_ctx or_ctx;

/* threads (0 = OpenMP default) */
void or_set_threads(int n);
int or_get_threads(void);

/* Philox4x32 with R rounds (the oracle uses R = 10). */
void or_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds,
                   uint32_t out[4]);

/* Level table for width q with shape parameter eps (the method uses 1/2):
 *   L[r], r = 0..2^q-1;  W[r] = fl32(65536 / (L[r+1] - L[r])), r = 0..2^q-2. */
void or_levels(int q, double eps, float *L, float *W);

/* Context for one simulated round.  n_coords % 256 == 0. */
or_ctx *or_create(int64_t n_coords, int32_t n_workers, int32_t topology,
                  float avg_bits);
void or_destroy(or_ctx *c);
void or_set_seed(or_ctx *c, uint64_t seed);
void or_set_round(or_ctx *c, uint32_t round);
void or_set_rounding(or_ctx *c, int32_t mode);
void or_set_eps(or_ctx *c, double eps);
void or_set_alloc(or_ctx *c, int32_t mode);
void or_set_own(or_ctx *c, int32_t mode);
/* Width set: qmax 8 gives {2,4,8} (the method: the clamp of the review's
 * referee minor 2), qmax 16 adds the 16-bit class of the threshold chain of
 * the review's Fig. 3 caption (T48 = 257/2^17 T816).  Returns -1 for any
 * other value. */
int or_set_max_width(or_ctx *c, int32_t qmax);

/* Stage 1: per-worker statistics, called in rank order 0..n-1. */
int or_stats(or_ctx *c, int32_t worker, const void *grad, int32_t dtype);
/* Stage 2: global mean, allocation scalar rho and widths. */
int or_allocate(or_ctx *c);
/* Stage 3: stable partition by width. */
int or_reorder(or_ctx *c);

/* Accessors (host copies). */
void or_get_stats(const or_ctx *c, float *sum, float *F, float *mu);
uint32_t or_get_rho_bits(const or_ctx *c);
/* the values the thresholds were applied to (F, or G for the mean-corrected
 * variant); valid after or_allocate */
void or_get_alloc_key(const or_ctx *c, float *out);
void or_get_widths(const or_ctx *c, uint8_t *w);
void or_get_perm(const or_ctx *c, int32_t *perm, int32_t *inv);
void or_get_class_counts(const or_ctx *c, int64_t counts[3]);
/* with the 16-bit class (counts[3] is 0 without it) */
void or_get_class_counts4(const or_ctx *c, int64_t counts[4]);
int64_t or_budget_bits(const or_ctx *c);
int64_t or_count_bits(const or_ctx *c, uint32_t rho_bits);
/* Widths q_j in {2,4,8} minimising sum_j F_j 4^-q_j subject to
 * sum_j q_j <= budget_bits (J <= 4096, budget_bits >= 2 J); returns that
 * minimum (fp64), or -1 on bad arguments. */
double or_alloc_exact(const float *F, int64_t J, int64_t budget_bits, uint8_t *widths);
/* the same over the width set of qmax (8 or 16) */
double or_alloc_exact_q(const float *F, int64_t J, int64_t budget_bits, int32_t qmax, uint8_t *widths);
/* T12, T24, T48 for the scalar with bit pattern rho_bits. */
void or_thresholds(uint32_t rho_bits, float out[3]);
/* With the 16-bit class: T12, T24, T48, T816 = fl(K rho) with the chain
 * scaled by 257, K = 21845, 139808, 4210688, 2^31. */
void or_thresholds_wide(uint32_t rho_bits, float out[4]);

/* Region of part (m, part): bytes and per-class counts (4 entries; the
 * last is 0 without the 16-bit class). */
int64_t or_region_bytes(const or_ctx *c, int64_t m, int64_t part,
                        int64_t counts_out[4]);

/* Schedule steps.  `filter` (sorted global stream positions, may be NULL)
 * restricts the work to those super-groups; other bytes are left untouched.
 *   ring:      compress at step 0, hop at steps 1..n-1
 *   butterfly: compress at level 1 (step 1), hop at levels 1..log2 n
 *   n == 1:    compress at step 0 only */
int or_compress(or_ctx *c, int32_t worker, int32_t step, const void *grad,
                int32_t dtype, uint8_t *region_out, const int64_t *filter,
                int64_t n_filter);
int or_hop(or_ctx *c, int32_t worker, int32_t step, const uint8_t *region_in,
           const void *local, int32_t local_kind, uint8_t *out0, uint8_t *out1,
           const int64_t *filter, int64_t n_filter);
int or_finalize(or_ctx *c, int64_t part, const uint8_t *region, float *out,
                const int64_t *filter, int64_t n_filter);

/* Part that worker `worker` ends the reduction with. */
int64_t or_final_part(const or_ctx *c, int32_t worker);

/* Whole simulated round (stats .. finalize); grads[w] are n_coords each. */
int or_allreduce(or_ctx *c, const void *const *grads, int32_t dtype,
                 float *out);

/* Codec on one super-group with explicit 16-bit dithers (for statistical
 * pins): encodes y[256] at width q (2, 4, 8 or 16) and returns the decoded
 * values, the codes, the scale unit and the group codes. */
void or_roundtrip_sg(const float *y, int32_t q, const uint16_t *dither,
                     double eps, float *decoded, uint16_t *codes, float *scale,
                     uint8_t *cg);
/* Batch: K rows of y and dithers -> K rows of decoded values. */
void or_roundtrip_batch(const float *y, int64_t K, int32_t q,
                        const uint16_t *dither, double eps, float *decoded);
/* The 256 dithers of super-group j for Philox counter tag `tag`, each
 * raised by `stagger` modulo 65536. */
void or_dithers_tagged(uint64_t seed, uint32_t round, int64_t j, uint32_t tag, uint32_t stagger,
                       uint16_t *d);
/* The 256 dithers the oracle uses for super-group j in one quantisation
 * event (mode OR_CORRELATED or OR_INDEPENDENT, worker rank, event index). */
void or_dithers(uint64_t seed, uint32_t round, int64_t j, int32_t mode,
                int32_t worker, int32_t n_workers, int32_t event,
                uint16_t *d);

/* MX formats (OCP MX v1.0: block 32, E8M0 shared scale; elements FP8 E4M3,
 * FP6 E3M2 or E2M3, FP4 E2M1).  The mxfp8 names are the E4M3 case. */
enum { OR_MX_E4M3 = 0, OR_MX_E3M2 = 1, OR_MX_E2M3 = 2, OR_MX_E2M1 = 3 };
void or_mx_roundtrip(int32_t fmt, const float *x, int64_t n, float *out);
void or_mxfp8_roundtrip(const float *x, int64_t n, float *out);
/* The schedule of the context with MX re-encoding at every hop, on parts of
 * the original order; out = the decoded all-reduced sum. */
int or_mxfp8_allreduce(or_ctx *c, const void *const *grads, int32_t dtype, float *out);
int or_mx_allreduce(or_ctx *c, int32_t fmt, const void *const *grads, int32_t dtype, float *out);

#ifdef __cplusplus
}
#endif
#endif
