/*
 * c_abi_check.c -- a plain C program that uses libddl.so the way an MPI or
 * framework program written in C would: HIP runtime C API for memory,
 * streams and events, include/ddl.h for the all-reduce, no Python and no
 * torch.  Test program only (it links the CPU oracle to check the results).
 *
 * The operation is the one the pages define: every rank ends with the sum
 * or the average of all ranks' gradients (Baidu Ring-Allreduce article,
 * "总结"), by ring, multi-ring ("[论文解读] PowerAI DDL", ABSTRACT) or 2D
 * torus (Sony "224秒训练ResNet-50" article, "2D-Torus All-reduce").
 *
 * Checks, each printed before it runs:
 *  - ddl_allreduce and ddl_plan_execute on device buffers from hipMalloc,
 *    every rank byte-equal to the oracle's walk of the same schedule
 *    (seeded synthetic inputs from synth/), in both modes and both fused
 *    forms;
 *  - the closed form: rank r holding r + 1 gives P (P + 1) / 2 (sum) or
 *    (P + 1) / 2 (mean) in every element of every rank;
 *  - per-bucket ready events on a second stream and a done event;
 *  - the error codes of bad arguments, with nothing enqueued and the
 *    buffers untouched.
 * Exit status 0 when everything holds, 1 on a mismatch, 2 on a HIP error,
 * 77 when no GPU is visible.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ddl.h"
#include "ddl_oracle.h"
#include "synth.h"

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

#define CHECK(c, ...)                                                          \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "c_abi_check: FAILED: " __VA_ARGS__);              \
            fprintf(stderr, "\n");                                             \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

typedef struct {
    const char *name;
    int P;
    size_t n;
    ddl_dtype dtype;
    ddl_op op;
    int kind, k, rows, cols;
    int nbuckets;  /* equal buckets, issued last-first */
} Case;

static size_t esize(ddl_dtype d) { return d == DDL_F32 ? 4 : 2; }

/* equal buckets over [0, n), in reverse order (output layer first) */
static void make_buckets(size_t n, int nb, ddl_bucket *b, uint64_t *off, uint64_t *len) {
    for (int i = 0; i < nb; ++i) {
        const size_t lo = n * (size_t)i / (size_t)nb, hi = n * (size_t)(i + 1) / (size_t)nb;
        const int j = nb - 1 - i;
        b[j].offset = lo;
        b[j].count = hi - lo;
        b[j].ready_event = NULL;
        off[j] = lo;
        len[j] = hi - lo;
    }
}

/* device buffers from host images; returns the device pointers */
static void upload(void **d, void **h, int P, size_t bytes) {
    for (int r = 0; r < P; ++r)
        HIP_OK(hipMemcpy(d[r], h[r], bytes, hipMemcpyHostToDevice));
}

static void compare(const Case *c, void **d, void **ref, size_t bytes, const char *what) {
    void *got = malloc(bytes);
    CHECK(got != NULL, "host allocation");
    for (int r = 0; r < c->P; ++r) {
        HIP_OK(hipMemcpy(got, d[r], bytes, hipMemcpyDeviceToHost));
        if (memcmp(got, ref[r], bytes) != 0) {
            size_t e = 0;
            const size_t s = esize(c->dtype);
            while (e * s < bytes && memcmp((char *)got + e * s, (char *)ref[r] + e * s, s) == 0)
                ++e;
            CHECK(0, "%s %s: rank %d differs from the oracle at element %zu", c->name, what, r, e);
        }
    }
    free(got);
}

static void run_case(const Case *c, uint64_t seed) {
    const size_t bytes = c->n * esize(c->dtype);
    const uint64_t q = 16 / esize(c->dtype);
    void *d[DDL_MAX_RANKS], *in[DDL_MAX_RANKS], *ref[DDL_MAX_RANKS];
    ddl_bucket bk[64];
    uint64_t boff[64], blen[64];
    make_buckets(c->n, c->nbuckets, bk, boff, blen);
    ddl_topo topo = {c->kind, c->k, c->rows, c->cols, NULL};
    for (int r = 0; r < c->P; ++r) {
        HIP_OK(hipMalloc(&d[r], bytes));
        in[r] = malloc(bytes);
        ref[r] = malloc(bytes);
        CHECK(in[r] && ref[r], "host allocation");
        synth_fill_host(in[r], c->dtype == DDL_F32 ? SYNTH_F32 : SYNTH_F16, SYNTH_NORMAL, seed,
                        r, 0, c->n, 1e-2);
        memcpy(ref[r], in[r], bytes);
    }
    CHECK(ddl_oracle_allreduce(ref, c->P, c->n, c->dtype == DDL_F32 ? ORC_F32 : ORC_F16,
                               c->op == DDL_SUM ? ORC_SUM : ORC_MEAN, c->kind, c->k, c->rows,
                               c->cols, NULL, boff, blen, c->nbuckets, q, 0, c->n, NULL) == 0,
          "%s: oracle rejected the case", c->name);

    /* the one-shot form, both modes, on the default stream */
    for (int mode = DDL_STEPWISE; mode <= DDL_FUSED; ++mode) {
        printf("c_abi_check: %s ddl_allreduce %s\n", c->name, mode ? "fused" : "stepwise");
        fflush(stdout);
        upload(d, in, c->P, bytes);
        int rc = ddl_allreduce(d, c->P, c->n, c->dtype, c->op, &topo, bk, c->nbuckets,
                               (ddl_mode)mode, NULL, NULL);
        CHECK(rc == DDL_OK, "%s: ddl_allreduce returned %d (%s)", c->name, rc, ddl_strerror(rc));
        HIP_OK(hipDeviceSynchronize());
        compare(c, d, ref, bytes, mode ? "fused" : "stepwise");
    }

    /* a plan in each fused form, buckets gated by events recorded on a
     * second stream, done event waited on from the host */
    hipStream_t s, prod;
    HIP_OK(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    HIP_OK(hipStreamCreateWithFlags(&prod, hipStreamNonBlocking));
    hipEvent_t ev[64], done;
    void *evp[64];
    for (int b = 0; b < c->nbuckets; ++b) {
        HIP_OK(hipEventCreateWithFlags(&ev[b], hipEventDisableTiming));
        evp[b] = ev[b];
    }
    HIP_OK(hipEventCreateWithFlags(&done, hipEventDisableTiming));
    ddl_plan plan;
    int rc = ddl_plan_create(&plan, c->P, c->n, c->dtype, c->op, &topo, bk, c->nbuckets, DDL_FUSED);
    CHECK(rc == DDL_OK, "%s: ddl_plan_create returned %d", c->name, rc);
    for (int passes = 1; passes <= 2; ++passes) {
        printf("c_abi_check: %s plan, %d kernel(s) per pass, ready events\n", c->name, passes);
        fflush(stdout);
        CHECK(ddl_plan_set_fused_passes(plan, passes) == DDL_OK, "set_fused_passes");
        upload(d, in, c->P, bytes);
        for (int b = 0; b < c->nbuckets; ++b)
            HIP_OK(hipEventRecord(ev[b], prod));
        rc = ddl_plan_execute(plan, d, evp, s, done);
        CHECK(rc == DDL_OK, "%s: ddl_plan_execute returned %d (%s)", c->name, rc, ddl_strerror(rc));
        HIP_OK(hipEventSynchronize(done));
        compare(c, d, ref, bytes, passes == 1 ? "one-kernel plan" : "two-kernel plan");
    }
    HIP_OK(hipStreamSynchronize(s));
    CHECK(ddl_plan_destroy(plan) == DDL_OK, "ddl_plan_destroy");
    for (int b = 0; b < c->nbuckets; ++b)
        HIP_OK(hipEventDestroy(ev[b]));
    HIP_OK(hipEventDestroy(done));
    HIP_OK(hipStreamDestroy(s));
    HIP_OK(hipStreamDestroy(prod));
    for (int r = 0; r < c->P; ++r) {
        HIP_OK(hipFree(d[r]));
        free(in[r]);
        free(ref[r]);
    }
}

/* rank r holds r + 1: the sum P (P + 1) / 2 and the mean (P + 1) / 2 are
 * exact in binary32 */
static void closed_form(int P, size_t n, ddl_op op, const ddl_topo *topo) {
    printf("c_abi_check: closed form P=%d n=%zu %s\n", P, n, op == DDL_SUM ? "sum" : "mean");
    fflush(stdout);
    void *d[DDL_MAX_RANKS];
    float *h = (float *)malloc(n * sizeof(float));
    CHECK(h != NULL, "host allocation");
    for (int r = 0; r < P; ++r) {
        HIP_OK(hipMalloc(&d[r], n * sizeof(float)));
        for (size_t i = 0; i < n; ++i)
            h[i] = (float)(r + 1);
        HIP_OK(hipMemcpy(d[r], h, n * sizeof(float), hipMemcpyHostToDevice));
    }
    ddl_bucket b = {0, n, NULL};
    CHECK(ddl_allreduce(d, P, n, DDL_F32, op, topo, &b, 1, DDL_FUSED, NULL, NULL) == DDL_OK,
          "closed form: ddl_allreduce");
    HIP_OK(hipDeviceSynchronize());
    const float want = op == DDL_SUM ? (float)(P * (P + 1) / 2) : (float)(P + 1) / 2.0f;
    for (int r = 0; r < P; ++r) {
        HIP_OK(hipMemcpy(h, d[r], n * sizeof(float), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < n; ++i)
            CHECK(h[i] == want, "closed form P=%d: rank %d element %zu is %g, not %g", P, r, i,
                  (double)h[i], (double)want);
        HIP_OK(hipFree(d[r]));
    }
    free(h);
}

/* bad arguments: an error code, nothing enqueued, the buffers untouched */
static void errors(void) {
    printf("c_abi_check: error codes\n");
    fflush(stdout);
    enum { P = 4 };
    const size_t n = 4096;
    void *d[P];
    float *h = (float *)malloc(n * sizeof(float));
    CHECK(h != NULL, "host allocation");
    for (size_t i = 0; i < n; ++i)
        h[i] = 1.0f;
    for (int r = 0; r < P; ++r) {
        HIP_OK(hipMalloc(&d[r], (n + 4) * sizeof(float)));
        HIP_OK(hipMemcpy(d[r], h, n * sizeof(float), hipMemcpyHostToDevice));
    }
    ddl_topo ring = {DDL_RING, 1, 0, 0, NULL};
    ddl_bucket whole = {0, n, NULL};
    ddl_bucket gap[2] = {{0, 100, NULL}, {200, n - 200, NULL}};
    void *misaligned[P] = {d[0], (char *)d[1] + 4, d[2], d[3]};
    int rc;
    rc = ddl_allreduce(misaligned, P, n, DDL_F32, DDL_SUM, &ring, &whole, 1, DDL_FUSED, NULL, NULL);
    CHECK(rc == DDL_E_ALIGN, "misaligned buffer gave %d, not DDL_E_ALIGN", rc);
    rc = ddl_allreduce(d, P, n, DDL_F32, DDL_SUM, &ring, gap, 2, DDL_FUSED, NULL, NULL);
    CHECK(rc == DDL_E_BUCKETS, "buckets with a gap gave %d, not DDL_E_BUCKETS", rc);
    rc = ddl_allreduce(d, 0, n, DDL_F32, DDL_SUM, &ring, &whole, 1, DDL_FUSED, NULL, NULL);
    CHECK(rc == DDL_E_ARG, "P = 0 gave %d, not DDL_E_ARG", rc);
    ddl_topo torus = {DDL_TORUS2D, 1, 3, 3, NULL};
    rc = ddl_allreduce(d, P, n, DDL_F32, DDL_SUM, &torus, &whole, 1, DDL_FUSED, NULL, NULL);
    CHECK(rc == DDL_E_ARG, "a 3x3 torus over 4 ranks gave %d, not DDL_E_ARG", rc);
    rc = ddl_allreduce(NULL, P, n, DDL_F32, DDL_SUM, &ring, &whole, 1, DDL_FUSED, NULL, NULL);
    CHECK(rc == DDL_E_NULL, "NULL buffers gave %d, not DDL_E_NULL", rc);
    for (int code = 0; code >= -8; --code)
        CHECK(ddl_strerror(code) != NULL && ddl_strerror(code)[0] != '\0', "ddl_strerror(%d)", code);
    HIP_OK(hipDeviceSynchronize());
    for (int r = 0; r < P; ++r) {
        HIP_OK(hipMemcpy(h, d[r], n * sizeof(float), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < n; ++i)
            CHECK(h[i] == 1.0f, "rank %d changed by a rejected call", r);
        HIP_OK(hipFree(d[r]));
    }
    free(h);
}

int main(void) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        printf("c_abi_check: no GPU\n");
        return 77;
    }
    HIP_OK(hipSetDevice(0));
    const Case cases[] = {
        {"ring P=5 f32 sum", 5, 1000003, DDL_F32, DDL_SUM, DDL_RING, 1, 0, 0, 3},
        {"multiring k=3 P=6 f16 mean", 6, 777777, DDL_F16, DDL_MEAN, DDL_MULTIRING, 3, 0, 0, 2},
        {"torus 2x3 f32 mean", 6, 500001, DDL_F32, DDL_MEAN, DDL_TORUS2D, 1, 2, 3, 4},
        {"torus 4x4 f16 mean", 16, 300007, DDL_F16, DDL_MEAN, DDL_TORUS2D, 1, 4, 4, 1},
        {"ring P=40 f32 mean", 40, 262147, DDL_F32, DDL_MEAN, DDL_RING, 1, 0, 0, 5},
    };
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i)
        run_case(&cases[i], 900 + i);
    const ddl_topo ring = {DDL_RING, 1, 0, 0, NULL};
    const ddl_topo torus = {DDL_TORUS2D, 1, 4, 10, NULL};
    closed_form(4, 1 << 20, DDL_SUM, &ring);
    closed_form(40, 100003, DDL_MEAN, &torus);
    errors();
    CHECK(ddl_cache_clear() == DDL_OK, "ddl_cache_clear");
    printf("c_abi_check: ok\n");
    return 0;
}
