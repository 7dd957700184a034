/*
 * ddl_oracle.c -- plain, slow, single-threaded CPU oracle of the gradient
 * all-reduce.  TEST INFRASTRUCTURE ONLY: the HIP library never links, loads
 * or includes any of this.
 *
 * What it computes (the pages' statement of the problem): every rank ends
 * with the sum -- or the average -- of all ranks' gradients, identical on
 * every rank (Baidu Ring-Allreduce article, "总结"; Sony article, the
 * paragraph on synchronising and averaging gradients before
 * "Batch Size Control").
 *
 * How it gets there matters for the bits, because floating-point addition is
 * not associative.  The oracle therefore walks the schedule: ring
 * reduce-scatter then ring all-gather, as message passing.  In every step each
 * ring position first sends one chunk (copied into a message), then every
 * position combines the chunk it received with its own.  The pages name the
 * ring (Baidu, "总结" and reference 4) but omit its steps; the reading taken is
 * the textbook bandwidth-optimal ring:
 *
 *   chunks c = 0..m-1 of the segment come from split(L, m, q)
 *   reduce-scatter step t = 0..m-2: position x sends chunk (x - t) mod m to
 *     position x+1, which sets own = own (+) received
 *   all-gather step t = 0..m-2: position x sends chunk (x + 1 - t) mod m to
 *     position x+1, which sets own = received
 *
 * Multi-ring ("[论文解读] PowerAI DDL", ABSTRACT / "提出的方法"): every bucket is
 * split into k parts, part j goes round ring j.  2D torus (Sony article,
 * "2D-Torus All-reduce", Fig. 1, Fig. 2): rank (i, j) = i*cols + j; ring
 * reduce-scatter along each row, then a ring all-reduce (reduce-scatter +
 * all-gather) down each column on the chunk that column holds, then ring
 * all-gather along each row.
 *
 * (+) is binary32 addition (round to nearest even, subnormals kept), or for
 * half precision (Sony article, "训练设置": gradients are exchanged in FP16)
 * fp16_rne(f32(a) + f32(b)): the partial sum on the wire is binary16.  The
 * mean is one correctly rounded division by P at the add that completes each
 * chunk's sum (the last reduce-scatter step that covers all P ranks), before
 * any copy, so every rank receives the same bits.
 *
 * After the all-reduce, ddl_oracle_sgd is the plain SGD step w = w - lr*y
 * that synchronous SGD takes with the averaged gradient, and ddl_oracle_lars
 * the layer-wise adaptive step the Sony article trains with ("训练设置": LARS,
 * its reference 9, coefficient 0.01, eps 1e-6; the formula itself is not on
 * the page).  LARS as You, Gitman and Ginsburg publish it scales each layer's
 * learning rate by a trust ratio coeff * ||w|| / ||grad||; the reading taken
 * (no weight decay or momentum is stated, so neither is applied):
 *
 *   per layer l:  W = sum of w_0[e]^2, G = sum of y[e]^2 over the layer,
 *                 in binary64 (each square of a binary32 value is exact),
 *                 element by element in index order;
 *   trust = coeff * sqrt(W) / (sqrt(G) + eps)   if W > 0 and G > 0,
 *           1                                    otherwise (a zero layer
 *                                                 would never move);
 *   rate  = binary32(lr * trust), one rounding from binary64;
 *   every replica: w_r[e] = w_r[e] - rate * y[e], the SGD step with rate.
 *
 * The norms use replica 0: synchronous SGD keeps every replica identical.
 * All rates are taken from the weights before any of them is updated.
 *
 * Parity pins (tests/test_oracle_*.py): closed forms, exact small-integer
 * sums, hand-worked adversarial examples of the chain order, rank identity,
 * the traffic identity and the pages' "about 2.4 GB", reductions between the
 * three schedules, exhaustive binary16 conversion and addition against numpy,
 * and fp64 error bounds; for LARS, closed-form rates, the gradient-scale
 * invariance, the zero-layer fallback to the plain SGD step and exact
 * rational norms on small layers.  No function here is "parity unpinned";
 * the association order itself is this reading of an omitted passage.
 *
 * Build: plain C11, -O2 -ffp-contract=off, no fast-math, SSE scalar floats.
 * The MXCSR flush-to-zero / denormals-are-zero bits are cleared for the
 * duration of every call, and round-to-nearest-even is forced.
 */
#include "ddl_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

/* ------------------------------------------------------------------------ */
/* floating-point environment                                                */
/* ------------------------------------------------------------------------ */

static unsigned int fpenv_enter(void)
{
    unsigned int saved = _mm_getcsr();
    /* bit 15 FTZ, bit 6 DAZ, bits 13-14 rounding control (00 = nearest) */
    _mm_setcsr(saved & ~((1u << 15) | (1u << 6) | (3u << 13)));
    return saved;
}

static void fpenv_leave(unsigned int saved) { _mm_setcsr(saved); }

/* ------------------------------------------------------------------------ */
/* binary16, written from the IEEE 754 definition of the format               */
/* ------------------------------------------------------------------------ */

/* sign(1) exponent(5, bias 15) fraction(10).  Exponent 0: subnormal,
 * value = fraction * 2^-24.  Exponent 31: infinity or NaN. */
static float h2f(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Nearest binary16 to x, ties to even. */
static uint16_t f2h(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    float a = fabsf(x);
    if (isnan(x))
        return sign | 0x7e00;
    if (isinf(x))
        return sign | 0x7c00;
    /* spacing of binary16 values around a: 2^-24 below 2^-14, else
     * 2^(floor(log2 a) - 10) */
    int qexp;
    if (a < 0x1p-14f) {
        qexp = -24;
    } else {
        int e2;
        frexpf(a, &e2); /* a = m * 2^e2, m in [0.5, 1) */
        qexp = e2 - 1 - 10;
    }
    float s = ldexpf(a, -qexp); /* exact: a power-of-two scaling, s < 2048 */
    float fl = floorf(s);
    float frac = s - fl; /* exact */
    if (frac > 0.5f || (frac == 0.5f && fmodf(fl, 2.0f) == 1.0f))
        fl += 1.0f;
    uint32_t nq = (uint32_t)fl; /* value = nq * 2^qexp */
    if (qexp == -24)              /* nq <= 1024; 1024 encodes 2^-14 itself */
        return sign | (uint16_t)nq;
    int E = qexp + 25; /* biased exponent of nq * 2^qexp for nq in [1024, 2048) */
    if (nq == 2048) {
        nq = 1024;
        E += 1;
    }
    if (E >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(E << 10) | (uint16_t)(nq - 1024);
}

/* ------------------------------------------------------------------------ */
/* element operations                                                        */
/* ------------------------------------------------------------------------ */

/* own (+) received, stored in the wire/storage type */
static void add_elem(int dtype, void *own, const void *recv)
{
    if (dtype == ORC_F32) {
        float a, b;
        memcpy(&a, own, 4);
        memcpy(&b, recv, 4);
        a = a + b;
        memcpy(own, &a, 4);
    } else {
        uint16_t a, b;
        memcpy(&a, own, 2);
        memcpy(&b, recv, 2);
        a = f2h(h2f(a) + h2f(b));
        memcpy(own, &a, 2);
    }
}

/* x / P, correctly rounded (binary16: through binary32, then to nearest) */
static void div_elem(int dtype, void *x, int P)
{
    if (dtype == ORC_F32) {
        float a;
        memcpy(&a, x, 4);
        a = a / (float)P;
        memcpy(x, &a, 4);
    } else {
        uint16_t a;
        memcpy(&a, x, 2);
        a = f2h(h2f(a) / (float)P);
        memcpy(x, &a, 2);
    }
}

/* ------------------------------------------------------------------------ */
/* the split of a segment into pieces                                        */
/* ------------------------------------------------------------------------ */

/* Piece c of m is [b_c, b_{c+1}), b_c = min(L, q * floor(c * ceil(L/q) / m)),
 * b_m = L.  With q = 1 this is the balanced split floor(c*L/m); with q > 1
 * every piece starts on a multiple of q. */
void ddl_oracle_split(uint64_t L, int m, uint64_t q, uint64_t *out)
{
    uint64_t U = (L + q - 1) / q;
    for (int c = 0; c < m; ++c) {
        uint64_t v = q * (((uint64_t)c * U) / (uint64_t)m);
        out[c] = v < L ? v : L;
    }
    out[m] = L;
}

/* ------------------------------------------------------------------------ */
/* the ring, as message passing                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    void *const *bufs;
    int P;
    int dtype;
    size_t esz;
    uint64_t q;
    uint64_t win_lo, win_hi;
    uint64_t *sent;
    unsigned char *msg; /* message area, indexed like the window */
} walk_t;

static int pmod(int a, int m) { return ((a % m) + m) % m; }

/* elements of [lo, hi) that fall inside the window, as [*a, *b) */
static int clip(const walk_t *w, uint64_t lo, uint64_t hi, uint64_t *a, uint64_t *b)
{
    *a = lo > w->win_lo ? lo : w->win_lo;
    *b = hi < w->win_hi ? hi : w->win_hi;
    return *a < *b;
}

static unsigned char *at(const walk_t *w, int rank, uint64_t e)
{
    return (unsigned char *)w->bufs[rank] + (e - w->win_lo) * w->esz;
}

/* rank "sends" elements [lo, hi): they are copied into the message area */
static void send_chunk(walk_t *w, int rank, uint64_t lo, uint64_t hi)
{
    uint64_t a, b;
    if (w->sent)
        w->sent[rank] += hi - lo;
    if (!w->bufs || !clip(w, lo, hi, &a, &b))
        return;
    memcpy(w->msg + (a - w->win_lo) * w->esz, at(w, rank, a), (b - a) * w->esz);
}

/* rank receives elements [lo, hi) and combines them with its own */
static void recv_reduce(walk_t *w, int rank, uint64_t lo, uint64_t hi, int divide)
{
    uint64_t a, b;
    if (!w->bufs || !clip(w, lo, hi, &a, &b))
        return;
    for (uint64_t e = a; e < b; ++e) {
        unsigned char *own = at(w, rank, e);
        add_elem(w->dtype, own, w->msg + (e - w->win_lo) * w->esz);
        if (divide)
            div_elem(w->dtype, own, w->P);
    }
}

/* rank receives elements [lo, hi) and keeps them */
static void recv_copy(walk_t *w, int rank, uint64_t lo, uint64_t hi)
{
    uint64_t a, b;
    if (!w->bufs || !clip(w, lo, hi, &a, &b))
        return;
    memcpy(at(w, rank, a), w->msg + (a - w->win_lo) * w->esz, (b - a) * w->esz);
}

/* Ring reduce-scatter of segment [off, off+L) among the m ranks ring[0..m-1]
 * (ring[x] is the rank at position x).  When `divide` is set, the add of the
 * last step -- the one that completes every chunk's sum -- is followed by the
 * division by P.  Afterwards position (c-1) mod m holds the reduced chunk c. */
static void ring_reduce_scatter(walk_t *w, const int *ring, int m, uint64_t off,
                                uint64_t L, int divide)
{
    uint64_t *b = malloc(sizeof(uint64_t) * (size_t)(m + 1));
    ddl_oracle_split(L, m, w->q, b);
    for (int t = 0; t <= m - 2; ++t) {
        for (int x = 0; x < m; ++x) {
            int c = pmod(x - t, m);
            send_chunk(w, ring[x], off + b[c], off + b[c + 1]);
        }
        for (int x = 0; x < m; ++x) {
            int c = pmod(x - t, m);
            recv_reduce(w, ring[(x + 1) % m], off + b[c], off + b[c + 1],
                        divide && t == m - 2);
        }
    }
    free(b);
}

/* Ring all-gather of segment [off, off+L), starting from the state the
 * reduce-scatter leaves (position (c-1) mod m holds chunk c). */
static void ring_all_gather(walk_t *w, const int *ring, int m, uint64_t off, uint64_t L)
{
    uint64_t *b = malloc(sizeof(uint64_t) * (size_t)(m + 1));
    ddl_oracle_split(L, m, w->q, b);
    for (int t = 0; t <= m - 2; ++t) {
        for (int x = 0; x < m; ++x) {
            int c = pmod(x + 1 - t, m);
            send_chunk(w, ring[x], off + b[c], off + b[c + 1]);
        }
        for (int x = 0; x < m; ++x) {
            int c = pmod(x + 1 - t, m);
            recv_copy(w, ring[(x + 1) % m], off + b[c], off + b[c + 1]);
        }
    }
    free(b);
}

/* ------------------------------------------------------------------------ */
/* the three schedules on one bucket                                         */
/* ------------------------------------------------------------------------ */

/* k rings, ring j over part j of split(L, k); ring j's order is
 * order[j*P .. j*P+P-1] (identity when order is NULL). */
static void multiring_bucket(walk_t *w, int k, const int *order, uint64_t off,
                             uint64_t L, int mean)
{
    int P = w->P;
    uint64_t *parts = malloc(sizeof(uint64_t) * (size_t)(k + 1));
    int *ring = malloc(sizeof(int) * (size_t)P);
    ddl_oracle_split(L, k, w->q, parts);
    for (int j = 0; j < k; ++j) {
        for (int x = 0; x < P; ++x)
            ring[x] = order ? order[j * P + x] : x;
        uint64_t poff = off + parts[j], plen = parts[j + 1] - parts[j];
        ring_reduce_scatter(w, ring, P, poff, plen, mean);
        ring_all_gather(w, ring, P, poff, plen);
    }
    free(ring);
    free(parts);
}

/* rows x cols grid, rank (i, j) = i*cols + j. */
static void torus_bucket(walk_t *w, int R, int C, uint64_t off, uint64_t L, int mean)
{
    int *ring = malloc(sizeof(int) * (size_t)(R > C ? R : C));
    uint64_t *cb = malloc(sizeof(uint64_t) * (size_t)(C + 1));
    ddl_oracle_split(L, C, w->q, cb);

    /* 1. reduce-scatter along every row (the division lands here only when
     *    there is no column phase, R == 1) */
    for (int i = 0; i < R; ++i) {
        for (int j = 0; j < C; ++j)
            ring[j] = i * C + j;
        ring_reduce_scatter(w, ring, C, off, L, mean && R == 1);
    }
    /* 2. all-reduce down every column on the chunk the column holds:
     *    column j holds row-chunk (j + 1) mod C */
    for (int j = 0; j < C; ++j) {
        int c = (j + 1) % C;
        for (int i = 0; i < R; ++i)
            ring[i] = i * C + j;
        ring_reduce_scatter(w, ring, R, off + cb[c], cb[c + 1] - cb[c], mean && R > 1);
        ring_all_gather(w, ring, R, off + cb[c], cb[c + 1] - cb[c]);
    }
    /* 3. all-gather along every row */
    for (int i = 0; i < R; ++i) {
        for (int j = 0; j < C; ++j)
            ring[j] = i * C + j;
        ring_all_gather(w, ring, C, off, L);
    }
    free(cb);
    free(ring);
}

/* ------------------------------------------------------------------------ */
/* entry points                                                              */
/* ------------------------------------------------------------------------ */

static int check_args(int P, uint64_t n, int dtype, int op, int kind, int k, int rows,
                      int cols, const int *ring_order, const uint64_t *boff,
                      const uint64_t *blen, int nb, uint64_t q, uint64_t wlo, uint64_t whi)
{
    if (P < 1 || q < 1 || nb < 0 || wlo > whi || whi > n)
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_F16)
        return -1;
    if (op != ORC_SUM && op != ORC_MEAN)
        return -1;
    if (kind == ORC_MULTIRING && k < 1)
        return -1;
    if (kind == ORC_TORUS2D && (rows < 1 || cols < 1 || rows * cols != P || ring_order))
        return -1;
    if (kind != ORC_RING && kind != ORC_MULTIRING && kind != ORC_TORUS2D)
        return -1;
    if (ring_order) {
        int kk = kind == ORC_MULTIRING ? k : 1;
        char *seen = malloc((size_t)P);
        for (int j = 0; j < kk; ++j) {
            memset(seen, 0, (size_t)P);
            for (int x = 0; x < P; ++x) {
                int r = ring_order[j * P + x];
                if (r < 0 || r >= P || seen[r]) {
                    free(seen);
                    return -1;
                }
                seen[r] = 1;
            }
        }
        free(seen);
    }
    /* the buckets must tile [0, n): in range, lengths adding up to n, and no
     * two of them overlapping */
    if (nb > 0 && (!boff || !blen))
        return -1;
    uint64_t total = 0;
    for (int b = 0; b < nb; ++b) {
        if (boff[b] > n || blen[b] > n - boff[b])
            return -1;
        total += blen[b];
    }
    if (total != n)
        return -1;
    /* pairwise overlap check: quadratic, fine for an oracle */
    for (int a = 0; a < nb; ++a)
        for (int b = a + 1; b < nb; ++b)
            if (blen[a] && blen[b] && boff[a] < boff[b] + blen[b] && boff[b] < boff[a] + blen[a])
                return -1;
    return 0;
}

int ddl_oracle_allreduce(void *const *bufs, int P, uint64_t n, int dtype, int op,
                         int kind, int k, int rows, int cols, const int *ring_order,
                         const uint64_t *bucket_off, const uint64_t *bucket_len,
                         int nbuckets, uint64_t q, uint64_t win_lo, uint64_t win_hi,
                         uint64_t *sent)
{
    if (check_args(P, n, dtype, op, kind, k, rows, cols, ring_order, bucket_off,
                   bucket_len, nbuckets, q, win_lo, win_hi))
        return -1;
    unsigned int env = fpenv_enter();
    walk_t w;
    w.bufs = bufs;
    w.P = P;
    w.dtype = dtype;
    w.esz = dtype == ORC_F32 ? 4 : 2;
    w.q = q;
    w.win_lo = win_lo;
    w.win_hi = win_hi;
    w.sent = sent;
    w.msg = bufs ? malloc((size_t)((win_hi - win_lo) * w.esz) + 1) : NULL;
    int mean = op == ORC_MEAN;
    for (int b = 0; b < nbuckets; ++b) {
        if (kind == ORC_TORUS2D)
            torus_bucket(&w, rows, cols, bucket_off[b], bucket_len[b], mean);
        else
            multiring_bucket(&w, kind == ORC_MULTIRING ? k : 1, ring_order,
                             bucket_off[b], bucket_len[b], mean);
    }
    free(w.msg);
    fpenv_leave(env);
    return 0;
}

int ddl_oracle_sgd(float *const *weights, int nweights, const void *y, uint64_t count,
                   int dtype, float lr)
{
    if (nweights < 1 || !weights || (!y && count))
        return -1;
    unsigned int env = fpenv_enter();
    for (int r = 0; r < nweights; ++r) {
        for (uint64_t e = 0; e < count; ++e) {
            float g = dtype == ORC_F32 ? ((const float *)y)[e] : h2f(((const uint16_t *)y)[e]);
            float step = lr * g;
            weights[r][e] = weights[r][e] - step;
        }
    }
    fpenv_leave(env);
    return 0;
}

int ddl_oracle_lars(float *const *weights, int nweights, const void *y,
                    const uint64_t *layer_off, const uint64_t *layer_len, int nlayers,
                    int dtype, float lr, double coeff, double eps, float *rates_out)
{
    if (nweights < 1 || !weights || nlayers < 0 || (nlayers > 0 && (!layer_off || !layer_len)))
        return -1;
    if (!(coeff >= 0.0) || !(eps >= 0.0) || coeff > 1e300 || eps > 1e300)
        return -1;
    for (int l = 0; l < nlayers; ++l)
        if (layer_len[l] && (!y || !weights[0]))
            return -1;
    float *rate = malloc(sizeof(float) * (size_t)(nlayers > 0 ? nlayers : 1));
    if (!rate)
        return -1;
    unsigned int env = fpenv_enter();
    /* every layer's rate, from the weights as they are before the step */
    for (int l = 0; l < nlayers; ++l) {
        double W = 0.0, G = 0.0;
        for (uint64_t e = layer_off[l]; e < layer_off[l] + layer_len[l]; ++e) {
            double w = (double)weights[0][e];
            double g = dtype == ORC_F32 ? (double)((const float *)y)[e]
                                        : (double)h2f(((const uint16_t *)y)[e]);
            W += w * w;
            G += g * g;
        }
        double trust = 1.0;
        if (W > 0.0 && G > 0.0)
            trust = coeff * sqrt(W) / (sqrt(G) + eps);
        rate[l] = (float)((double)lr * trust);
        if (rates_out)
            rates_out[l] = rate[l];
    }
    /* then the SGD step of every layer with its own rate */
    for (int l = 0; l < nlayers; ++l) {
        for (int r = 0; r < nweights; ++r) {
            for (uint64_t e = layer_off[l]; e < layer_off[l] + layer_len[l]; ++e) {
                float g = dtype == ORC_F32 ? ((const float *)y)[e]
                                           : h2f(((const uint16_t *)y)[e]);
                float step = rate[l] * g;
                weights[r][e] = weights[r][e] - step;
            }
        }
    }
    fpenv_leave(env);
    free(rate);
    return 0;
}

int ddl_oracle_sum_f64(const void *const *bufs, int P, uint64_t count, int dtype,
                       int op, double *out)
{
    if (P < 1 || !bufs || !out)
        return -1;
    unsigned int env = fpenv_enter();
    for (uint64_t e = 0; e < count; ++e) {
        double s = 0.0;
        for (int r = 0; r < P; ++r) {
            if (dtype == ORC_F32)
                s += (double)((const float *)bufs[r])[e];
            else
                s += (double)h2f(((const uint16_t *)bufs[r])[e]);
        }
        out[e] = op == ORC_MEAN ? s / (double)P : s;
    }
    fpenv_leave(env);
    return 0;
}

void ddl_oracle_f16_to_f32(const uint16_t *in, float *out, uint64_t count)
{
    unsigned int env = fpenv_enter();
    for (uint64_t i = 0; i < count; ++i)
        out[i] = h2f(in[i]);
    fpenv_leave(env);
}

void ddl_oracle_f32_to_f16(const float *in, uint16_t *out, uint64_t count)
{
    unsigned int env = fpenv_enter();
    for (uint64_t i = 0; i < count; ++i)
        out[i] = f2h(in[i]);
    fpenv_leave(env);
}

void ddl_oracle_f16_add(const uint16_t *a, const uint16_t *b, uint16_t *out, uint64_t count)
{
    unsigned int env = fpenv_enter();
    for (uint64_t i = 0; i < count; ++i) {
        uint16_t x = a[i];
        add_elem(ORC_F16, &x, &b[i]);
        out[i] = x;
    }
    fpenv_leave(env);
}

void ddl_oracle_f16_div(const uint16_t *a, int P, uint16_t *out, uint64_t count)
{
    unsigned int env = fpenv_enter();
    for (uint64_t i = 0; i < count; ++i) {
        uint16_t x = a[i];
        div_elem(ORC_F16, &x, P);
        out[i] = x;
    }
    fpenv_leave(env);
}
