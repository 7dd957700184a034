/*
 * ddl_oracle.h -- CPU oracle for the gradient all-reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library: it is rebuilt here from the pages.
 *
 * Sources (the four pages the method is taken from):
 *  - Baidu Ring-Allreduce article (Chinese translation, part 4), section
 *    "总结" (Summary): gradients are averaged across devices with the ring
 *    all-reduce from HPC; reference 4 there (Patarasuk & Yuan, bandwidth
 *    optimal all-reduce) names the reduce-scatter + all-gather ring.
 *  - Same article, opening paragraphs: the all-reduce works on subsets of the
 *    parameters, output layer first.
 *  - "[论文解读] PowerAI DDL" review, ABSTRACT and "提出的方法": a multi-ring
 *    communication pattern.
 *  - Sony "224秒训练ResNet-50" article, section "2D-Torus All-reduce", Fig. 1
 *    and Fig. 2: GPUs on a 2D grid; reduce-scatter, all-reduce, all-gather in
 *    horizontal and vertical rings.
 *  - Same article, "训练设置" (training settings): the gradient exchange is
 *    done in half precision (FP16), and the weights are updated with LARS
 *    (coefficient 0.01, eps 1e-6).
 *
 * Parity status of each function is in the header comment of ddl_oracle.c.
 */
#ifndef DDL_ORACLE_H
#define DDL_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_F16 = 1 };
enum { ORC_SUM = 0, ORC_MEAN = 1 };
enum { ORC_RING = 0, ORC_MULTIRING = 1, ORC_TORUS2D = 2 };

/* Walk the all-reduce schedule step by step, as message passing between
 * ranks, over host buffers.
 *
 *  bufs[r]      rank r's buffer; bufs[r][e - win_lo] holds element e.
 *               May be NULL (all of them) to count traffic only.
 *  P            number of ranks (>= 1)
 *  n            elements per rank
 *  dtype, op    ORC_F32 / ORC_F16, ORC_SUM / ORC_MEAN
 *  kind         ORC_RING (k ignored, one ring), ORC_MULTIRING (k rings over
 *               k parts of every bucket) or ORC_TORUS2D (rows x cols == P)
 *  ring_order   NULL (identity) or k*P ints; ring j visits ring_order[j*P+x]
 *               at position x.  Must be NULL for the torus.
 *  bucket_off/len  the bucket list, walked in the given order; together the
 *               buckets must tile [0, n) without overlap.
 *  q            split quantum in elements (>= 1)
 *  win_lo/hi    only elements in [win_lo, win_hi) are read or written
 *  sent         NULL or P counters; each rank's sent elements are ADDED
 *               (whole chunks, independent of the window)
 *
 * Returns 0, or -1 on bad arguments (nothing is touched then).
 */
int ddl_oracle_allreduce(void *const *bufs, int P, uint64_t n, int dtype, int op,
                         int kind, int k, int rows, int cols, const int *ring_order,
                         const uint64_t *bucket_off, const uint64_t *bucket_len,
                         int nbuckets, uint64_t q, uint64_t win_lo, uint64_t win_hi,
                         uint64_t *sent);

/* Plain SGD step after the all-reduce (the Baidu article, "总结": the
 * all-reduce serves synchronous stochastic gradient descent):
 * for every replica r < nweights and element e < count
 *     w_r[e] = w_r[e] - lr * y[e]
 * in binary32, two roundings (the product, then the difference), where y is
 * the all-reduced gradient (identical on every rank) widened to binary32.
 * weights: nweights binary32 host arrays; y: count elements of dtype. */
int ddl_oracle_sgd(float *const *weights, int nweights, const void *y, uint64_t count,
                   int dtype, float lr);

/* LARS step after the all-reduce (Sony article, "训练设置": LARS, reference
 * 9 there, coefficient 0.01, eps 1e-6; the update is You, Gitman and
 * Ginsburg's layer-wise trust ratio without weight decay or momentum).
 * Layer l covers elements [layer_off[l], layer_off[l] + layer_len[l]).  For
 * each layer, from replica 0's weights and the all-reduced gradient y:
 *     W = sum w_0[e]^2, G = sum y[e]^2       (binary64, index order)
 *     trust = coeff * sqrt(W) / (sqrt(G) + eps), or 1 if W or G is 0
 *     rate = binary32(lr * trust)
 * then every replica takes w_r[e] = w_r[e] - rate * y[e] (binary32, the
 * product rounded before the difference).  All rates are computed before
 * any weight changes.  rates_out: NULL or nlayers floats.  Returns -1 for
 * bad arguments (negative or non-finite coeff or eps), touching nothing. */
int ddl_oracle_lars(float *const *weights, int nweights, const void *y,
                    const uint64_t *layer_off, const uint64_t *layer_len, int nlayers,
                    int dtype, float lr, double coeff, double eps, float *rates_out);

/* The plain definition: out[e] = sum over ranks of g_r[e] in binary64,
 * divided by P for ORC_MEAN.  Reference for tolerance checks. */
int ddl_oracle_sum_f64(const void *const *bufs, int P, uint64_t count, int dtype,
                       int op, double *out);

/* Boundaries of the split of a length-L segment into m pieces with quantum q:
 * out[0..m], piece c is [out[c], out[c+1]). */
void ddl_oracle_split(uint64_t L, int m, uint64_t q, uint64_t *out);

/* The oracle's own binary16 helpers, exported for their pin tests. */
void ddl_oracle_f16_to_f32(const uint16_t *in, float *out, uint64_t count);
void ddl_oracle_f32_to_f16(const float *in, uint16_t *out, uint64_t count);
void ddl_oracle_f16_add(const uint16_t *a, const uint16_t *b, uint16_t *out, uint64_t count);
void ddl_oracle_f16_div(const uint16_t *a, int P, uint16_t *out, uint64_t count);

#ifdef __cplusplus
}
#endif
#endif
