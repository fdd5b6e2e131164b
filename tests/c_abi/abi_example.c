/*
 * A plain C program that uses libdtcoll.so through include/dt.h only: device
 * buffers from hipMalloc, host pointer arrays, explicit counts, dtype, op and
 * stream.  No Python and no PyTorch.  Every result is copied back and
 * compared bit for bit with the CPU oracle (oracle/oracle.c, linked in as
 * test infrastructure).  Prints "ok" and exits 0 when everything matches.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dt.h"

/* the oracle's functions (oracle/oracle.c) */
int oracle_allreduce(const void* const* x, void* const* y, int nranks, size_t count, int dtype, int op);
int oracle_reduce_scatter(const void* const* x, void* const* y, int nranks, size_t m, int dtype, int op);
int oracle_all_gather(const void* const* x, void* const* y, int nranks, const size_t* counts, size_t esize);
int oracle_all_to_all(const void* const* x, void* const* y, int nranks, const size_t* splits, size_t esize);
int oracle_bucket_allreduce(void* const* grads, const size_t* numels, int ntensors, int nranks,
                            size_t bucket_bytes, void* const* flat, int dtype, int op);
int oracle_barrier(int32_t* window, int nranks, int first_generation, int generations);

#define HIP_OK(x)                                                                      \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)
#define DT_OK_(x)                                                                       \
    do {                                                                                \
        dt_status s_ = (x);                                                             \
        if (s_ != DT_OK) {                                                              \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, dt_status_string(s_), \
                    dt_last_error());                                                   \
            exit(3);                                                                    \
        }                                                                               \
    } while (0)

static uint64_t rng = 0x853c49e6748fea9bull;
static uint32_t next32(void) { /* PCG-style LCG step, top bits */
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng >> 32);
}
/* fp32 words uniform in [-1, 1): a 23-bit mantissa fraction, random sign */
static void fill_f32(float* p, size_t n) {
    for (size_t i = 0; i < n; i++) {
        uint32_t r = next32();
        p[i] = ((float)(r >> 9) / 8388608.0f) * ((r & 1) ? -1.0f : 1.0f);
    }
}
/* bf16 bit patterns with exponents in [2^-8, 2^8): never NaN or inf */
static void fill_bf16(uint16_t* p, size_t n) {
    for (size_t i = 0; i < n; i++) {
        uint32_t r = next32();
        uint32_t exp = 119 + (r % 16);
        p[i] = (uint16_t)(((r >> 31) << 15) | (exp << 7) | ((r >> 8) & 0x7F));
    }
}
static void fill_i32(int32_t* p, size_t n) {
    for (size_t i = 0; i < n; i++) p[i] = (int32_t)next32();
}

static int failures = 0;
static void same(const void* got, const void* want, size_t bytes, const char* what) {
    if (memcmp(got, want, bytes) != 0) {
        fprintf(stderr, "mismatch: %s\n", what);
        failures++;
    }
}

static void* dev(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

/* AllReduce fp32 sum, P=4, ragged length, on a user stream */
static void check_allreduce(hipStream_t s) {
    enum { P = 4 };
    const size_t n = 1000003;
    void *hx[P], *hy[P], *hw[P], *dx[P], *dy[P];
    for (int r = 0; r < P; r++) {
        hx[r] = malloc(n * 4); hy[r] = malloc(n * 4); hw[r] = malloc(n * 4);
        fill_f32((float*)hx[r], n);
        dx[r] = dev(n * 4); dy[r] = dev(n * 4);
        HIP_OK(hipMemcpy(dx[r], hx[r], n * 4, hipMemcpyHostToDevice));
    }
    DT_OK_(dt_allreduce((const void* const*)dx, dy, P, n, DT_FLOAT32, DT_SUM, s));
    HIP_OK(hipStreamSynchronize(s));
    oracle_allreduce((const void* const*)hx, hw, P, n, DT_FLOAT32, DT_SUM);
    for (int r = 0; r < P; r++) {
        HIP_OK(hipMemcpy(hy[r], dy[r], n * 4, hipMemcpyDeviceToHost));
        same(hy[r], hw[r], n * 4, "allreduce");
        free(hx[r]); free(hy[r]); free(hw[r]);
        HIP_OK(hipFree(dx[r])); HIP_OK(hipFree(dy[r]));
    }
}

/* ReduceScatter bf16 max then AllGather, P=8 */
static void check_reduce_scatter(hipStream_t s) {
    enum { P = 8 };
    const size_t m = 4099;
    void *hx[P], *hs[P], *hw[P], *dx[P], *ds[P];
    for (int r = 0; r < P; r++) {
        hx[r] = malloc(P * m * 2); hs[r] = malloc(m * 2); hw[r] = malloc(m * 2);
        fill_bf16((uint16_t*)hx[r], P * m);
        dx[r] = dev(P * m * 2); ds[r] = dev(m * 2);
        HIP_OK(hipMemcpy(dx[r], hx[r], P * m * 2, hipMemcpyHostToDevice));
    }
    DT_OK_(dt_reduce_scatter((const void* const*)dx, ds, P, m, DT_BFLOAT16, DT_MAX, s));
    HIP_OK(hipStreamSynchronize(s));
    oracle_reduce_scatter((const void* const*)hx, hw, P, m, DT_BFLOAT16, DT_MAX);
    for (int r = 0; r < P; r++) {
        HIP_OK(hipMemcpy(hs[r], ds[r], m * 2, hipMemcpyDeviceToHost));
        same(hs[r], hw[r], m * 2, "reduce_scatter");
        free(hx[r]); free(hs[r]); free(hw[r]);
        HIP_OK(hipFree(dx[r])); HIP_OK(hipFree(ds[r]));
    }
}

/* uneven AllGather int32 (one empty rank), P=5 */
static void check_all_gather(hipStream_t s) {
    enum { P = 5 };
    const size_t counts[P] = {7, 0, 100000, 13, 4096};
    size_t total = 0;
    for (int r = 0; r < P; r++) total += counts[r];
    void *hx[P], *hy[P], *hw[P], *dx[P], *dy[P];
    for (int r = 0; r < P; r++) {
        hx[r] = malloc(counts[r] * 4 + 4);
        fill_i32((int32_t*)hx[r], counts[r]);
        dx[r] = counts[r] ? dev(counts[r] * 4) : NULL;  /* an empty rank may pass NULL */
        if (counts[r]) HIP_OK(hipMemcpy(dx[r], hx[r], counts[r] * 4, hipMemcpyHostToDevice));
        hy[r] = malloc(total * 4); hw[r] = malloc(total * 4);
        dy[r] = dev(total * 4);
    }
    DT_OK_(dt_all_gather((const void* const*)dx, dy, P, counts, 0, DT_INT32, s));
    HIP_OK(hipStreamSynchronize(s));
    oracle_all_gather((const void* const*)hx, hw, P, counts, 4);
    for (int r = 0; r < P; r++) {
        HIP_OK(hipMemcpy(hy[r], dy[r], total * 4, hipMemcpyDeviceToHost));
        same(hy[r], hw[r], total * 4, "all_gather");
        free(hx[r]); free(hy[r]); free(hw[r]);
        if (dx[r]) HIP_OK(hipFree(dx[r]));
        HIP_OK(hipFree(dy[r]));
    }
}

/* AllToAll fp32 with a split matrix holding empty blocks, P=3 */
static void check_all_to_all(hipStream_t s) {
    enum { P = 3 };
    const size_t splits[P * P] = {5, 0, 70000, 1, 3, 0, 4096, 9, 2};
    size_t rows[P] = {0}, cols[P] = {0};
    for (int i = 0; i < P; i++)
        for (int j = 0; j < P; j++) { rows[i] += splits[i * P + j]; cols[j] += splits[i * P + j]; }
    void *hx[P], *hy[P], *hw[P], *dx[P], *dy[P];
    for (int r = 0; r < P; r++) {
        hx[r] = malloc(rows[r] * 4); fill_f32((float*)hx[r], rows[r]);
        dx[r] = dev(rows[r] * 4);
        HIP_OK(hipMemcpy(dx[r], hx[r], rows[r] * 4, hipMemcpyHostToDevice));
        hy[r] = malloc(cols[r] * 4); hw[r] = malloc(cols[r] * 4); dy[r] = dev(cols[r] * 4);
    }
    DT_OK_(dt_all_to_all((const void* const*)dx, dy, P, splits, DT_FLOAT32, s));
    HIP_OK(hipStreamSynchronize(s));
    oracle_all_to_all((const void* const*)hx, hw, P, splits, 4);
    for (int r = 0; r < P; r++) {
        HIP_OK(hipMemcpy(hy[r], dy[r], cols[r] * 4, hipMemcpyDeviceToHost));
        same(hy[r], hw[r], cols[r] * 4, "all_to_all");
        free(hx[r]); free(hy[r]); free(hw[r]);
        HIP_OK(hipFree(dx[r])); HIP_OK(hipFree(dy[r]));
    }
}

/* fused-bucket AllReduce, bf16 sum, P=2, three tensors, 4 KiB buckets, in place */
static void check_bucket(hipStream_t s) {
    enum { P = 2, T = 3 };
    const size_t numels[T] = {3000, 17, 5000};
    size_t total = 0;
    for (int t = 0; t < T; t++) total += numels[t];
    void *hg[P * T], *dg[P * T], *flat[P];
    for (int r = 0; r < P; r++) {
        flat[r] = malloc(total * 2);
        for (int t = 0; t < T; t++) {
            hg[r * T + t] = malloc(numels[t] * 2);
            fill_bf16((uint16_t*)hg[r * T + t], numels[t]);
            dg[r * T + t] = dev(numels[t] * 2);
            HIP_OK(hipMemcpy(dg[r * T + t], hg[r * T + t], numels[t] * 2, hipMemcpyHostToDevice));
        }
    }
    DT_OK_(dt_bucket_allreduce(dg, numels, T, P, 4096, NULL, DT_BFLOAT16, DT_SUM, s));
    HIP_OK(hipStreamSynchronize(s));
    oracle_bucket_allreduce(hg, numels, T, P, 4096, flat, DT_BFLOAT16, DT_SUM);
    for (int i = 0; i < P * T; i++) {
        const size_t bytes = numels[i % T] * 2;
        void* got = malloc(bytes);
        HIP_OK(hipMemcpy(got, dg[i], bytes, hipMemcpyDeviceToHost));
        same(got, hg[i], bytes, "bucket_allreduce");
        free(got); free(hg[i]);
        HIP_OK(hipFree(dg[i]));
    }
    for (int r = 0; r < P; r++) free(flat[r]);
}

/* barrier, P=16, 1000 generations in one launch: windows against the model.
 * The packed layout (a plain launch): this program runs beside another
 * process on the GPU, where the runtime may refuse a cooperative launch. */
static void check_barrier(hipStream_t s) {
    enum { P = 16 };
    int32_t* win[P];
    int32_t* model = calloc(P * P, sizeof(int32_t));
    int32_t* status = (int32_t*)dev(4);
    HIP_OK(hipMemset(status, 0, 4));
    for (int r = 0; r < P; r++) {
        win[r] = (int32_t*)dev(P * 4);
        HIP_OK(hipMemset(win[r], 0, P * 4));
    }
    DT_OK_(dt_barrier(win, P, 1, 1000, status, 0, DT_BARRIER_PACKED, s));
    HIP_OK(hipStreamSynchronize(s));
    int32_t st = -1;
    HIP_OK(hipMemcpy(&st, status, 4, hipMemcpyDeviceToHost));
    if (st != DT_OK) { fprintf(stderr, "barrier status %d\n", st); failures++; }
    if (oracle_barrier(model, P, 1, 1000) != 1000) failures++;
    for (int r = 0; r < P; r++) {
        int32_t row[P];
        HIP_OK(hipMemcpy(row, win[r], P * 4, hipMemcpyDeviceToHost));
        same(row, model + r * P, P * 4, "barrier window");
        HIP_OK(hipFree(win[r]));
    }
    HIP_OK(hipFree(status));
    free(model);
}

/* the error path: no launch, a status and a message */
static void check_errors(void) {
    const void* send[1] = {NULL};
    void* recv[1] = {NULL};
    if (dt_allreduce(send, recv, 0, 4, DT_FLOAT32, DT_SUM, NULL) != DT_ERR_ARG) failures++;
    if (strlen(dt_last_error()) == 0) failures++;
    if (dt_allreduce(send, recv, 1, 4, DT_FLOAT32, DT_SUM, NULL) != DT_ERR_ARG) failures++;
}

int main(void) {
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    printf("%s\n", dt_version());
    check_errors();
    check_allreduce(s);
    check_reduce_scatter(s);
    check_all_gather(s);
    check_all_to_all(s);
    check_bucket(s);
    check_barrier(s);
    HIP_OK(hipStreamDestroy(s));
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
