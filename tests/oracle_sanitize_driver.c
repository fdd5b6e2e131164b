/*
 * Memory-safety and undefined-behaviour driver for oracle/oracle.c.
 *
 * Built by tests/test_oracle_sanitizers.py with gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer (CPU only).  Every oracle function runs on small
 * seeded cases -- empty, one-element and ragged sizes, every dtype and op,
 * 1 to 16 ranks -- with each buffer in its own exact-size heap block, so a
 * read or write one element past any buffer, a signed overflow or a bad
 * shift aborts the run.  Values are not checked here (the pins do that);
 * the driver prints "ok" when every call returned OR_OK.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (oracle/oracle.c) */
uint16_t oracle_float_to_bf16(float f);
void oracle_float_to_bf16_array(const float* in, uint16_t* out, size_t n);
int oracle_allreduce(const void* const* x, void* const* y, int nranks, size_t count, int dtype, int op);
int oracle_reduce_scatter(const void* const* x, void* const* y, int nranks, size_t m, int dtype, int op);
int oracle_all_gather(const void* const* x, void* const* y, int nranks, const size_t* counts, size_t esize);
int oracle_all_to_all(const void* const* x, void* const* y, int nranks, const size_t* splits, size_t esize);
int oracle_bucket_allreduce(void* const* grads, const size_t* numels, int ntensors, int nranks,
                            size_t bucket_bytes, void* const* flat, int dtype, int op);
int oracle_hsdp_layer(const void* const* grads, void* const* out, const size_t* numels, int ntensors,
                      int replicate, int shard, size_t bucket_bytes, void* const* work, int dtype, int op);
int oracle_broadcast(const void* x_root, void* const* y, int nranks, size_t nbytes);
int oracle_replicate_to_shard(const void* const* x, void* const* y, int nranks, size_t m, size_t esize);
int oracle_all_gather_into_vec(const void* const* x, void* const* y, int nranks, const size_t* counts,
                               size_t esize);
int oracle_all_to_all_dims(const void* const* x, void* const* y, int nranks, size_t rows, size_t cols,
                           int src_dim, int dst_dim, size_t esize);
int oracle_barrier(int32_t* window, int nranks, int first_generation, int generations);
int oracle_barrier_exchange(const void* const* x, void* const* y, int nranks, size_t nbytes);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{ /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static size_t below(size_t n) { return n ? (size_t)(next_u64() % n) : 0; }

/* an exact-size block (one byte for an empty buffer, never dereferenced) */
static void* block(size_t bytes)
{
    unsigned char* p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    for (size_t i = 0; i < bytes; i++)
        p[i] = (unsigned char)next_u64();
    return p;
}
static void** blocks(int n, size_t bytes)
{
    void** v = malloc(sizeof(void*) * (size_t)(n ? n : 1));
    for (int i = 0; i < n; i++)
        v[i] = block(bytes);
    return v;
}
static void free_blocks(void** v, int n)
{
    for (int i = 0; i < n; i++)
        free(v[i]);
    free(v);
}

static int failures = 0;
static void expect_ok(int rc, const char* what)
{
    if (rc != 0) {
        fprintf(stderr, "%s returned %d\n", what, rc);
        failures++;
    }
}

static const size_t kEsize[3] = {4, 2, 4}; /* fp32, bf16, int32 */
static const int kRanks[] = {1, 2, 3, 4, 8, 16};
static const size_t kCounts[] = {0, 1, 7, 33};

static void reductions(void)
{
    for (int dt = 0; dt < 3; dt++)
        for (int op = 0; op < 4; op++)
            for (size_t pi = 0; pi < sizeof kRanks / sizeof *kRanks; pi++)
                for (size_t ci = 0; ci < sizeof kCounts / sizeof *kCounts; ci++) {
                    int p = kRanks[pi];
                    size_t m = kCounts[ci], es = kEsize[dt];
                    void** x = blocks(p, (size_t)p * m * es);
                    void** y = blocks(p, (size_t)p * m * es);
                    void** s = blocks(p, m * es);
                    expect_ok(oracle_allreduce((const void* const*)x, y, p, (size_t)p * m, dt, op), "allreduce");
                    expect_ok(oracle_reduce_scatter((const void* const*)x, s, p, m, dt, op), "reduce_scatter");
                    free_blocks(x, p);
                    free_blocks(y, p);
                    free_blocks(s, p);
                }
}

static void copies(void)
{
    for (size_t pi = 0; pi < sizeof kRanks / sizeof *kRanks; pi++)
        for (int rep = 0; rep < 4; rep++) {
            int p = kRanks[pi];
            size_t es = kEsize[rep % 3];
            size_t counts[16], total = 0;
            void* x[16];
            for (int r = 0; r < p; r++) {
                counts[r] = below(rep == 0 ? 2 : 40);
                total += counts[r];
                x[r] = block(counts[r] * es);
            }
            void** y = blocks(p, total * es);
            expect_ok(oracle_all_gather((const void* const*)x, y, p, counts, es), "all_gather");
            void** vec = malloc(sizeof(void*) * (size_t)p * (size_t)p);
            for (int q = 0; q < p; q++)
                for (int r = 0; r < p; r++)
                    vec[q * p + r] = block(counts[r] * es);
            expect_ok(oracle_all_gather_into_vec((const void* const*)x, vec, p, counts, es), "all_gather_into_vec");
            free_blocks(vec, p * p);
            free_blocks(y, p);
            void** b = blocks(p, counts[0] * es);
            expect_ok(oracle_broadcast(x[0], b, p, counts[0] * es), "broadcast");
            free_blocks(b, p);
            for (int r = 0; r < p; r++)
                free(x[r]);

            /* all-to-all with a random split matrix, zero blocks included */
            size_t splits[256], rows[16] = {0}, cols[16] = {0};
            for (int i = 0; i < p; i++)
                for (int j = 0; j < p; j++) {
                    splits[i * p + j] = below(rep == 0 ? 2 : 9);
                    rows[i] += splits[i * p + j];
                    cols[j] += splits[i * p + j];
                }
            void* ax[16];
            void* ay[16];
            for (int i = 0; i < p; i++) {
                ax[i] = block(rows[i] * es);
                ay[i] = block(cols[i] * es);
            }
            expect_ok(oracle_all_to_all((const void* const*)ax, ay, p, splits, es), "all_to_all");
            expect_ok(oracle_barrier_exchange((const void* const*)ax, ay, p, 0), "barrier_exchange(0)");
            for (int i = 0; i < p; i++) {
                free(ax[i]);
                free(ay[i]);
            }

            /* replicate -> shard, P-way exchange */
            size_t m = below(12);
            void** rx = blocks(p, (size_t)p * m * es);
            void** ry = blocks(p, m * es);
            expect_ok(oracle_replicate_to_shard((const void* const*)rx, ry, p, m, es), "replicate_to_shard");
            expect_ok(oracle_barrier_exchange((const void* const*)rx, ry, p, m * es), "barrier_exchange");
            free_blocks(rx, p);
            free_blocks(ry, p);

            /* shard-dimension all-to-all: every (src, dst) pair */
            size_t nr = (size_t)p * (1 + below(3)), nc = (size_t)p * (1 + below(3));
            for (int sd = 0; sd < 2; sd++)
                for (int dd = 0; dd < 2; dd++) {
                    size_t nsrc = sd == 0 ? (nr / (size_t)p) * nc : nr * (nc / (size_t)p);
                    size_t ndst = dd == 0 ? (nr / (size_t)p) * nc : nr * (nc / (size_t)p);
                    void** dx = blocks(p, nsrc * es);
                    void** dy = blocks(p, ndst * es);
                    expect_ok(oracle_all_to_all_dims((const void* const*)dx, dy, p, nr, nc, sd, dd, es),
                              "all_to_all_dims");
                    free_blocks(dx, p);
                    free_blocks(dy, p);
                }
        }
}

static void buckets(void)
{
    const size_t numels[] = {0, 3, 17, 1, 40, 0, 8};
    const int nt = (int)(sizeof numels / sizeof *numels);
    size_t total = 0;
    for (int t = 0; t < nt; t++)
        total += numels[t];
    const size_t bucket_bytes[] = {4, 16, 64, 1u << 20};
    for (int dt = 0; dt < 3; dt++)
        for (int op = 0; op < 4; op++)
            for (size_t pi = 0; pi < sizeof kRanks / sizeof *kRanks; pi++)
                for (size_t bi = 0; bi < sizeof bucket_bytes / sizeof *bucket_bytes; bi++) {
                    int p = kRanks[pi];
                    size_t es = kEsize[dt];
                    if (bucket_bytes[bi] < es)
                        continue;
                    void** g = malloc(sizeof(void*) * (size_t)p * (size_t)nt);
                    for (int r = 0; r < p; r++)
                        for (int t = 0; t < nt; t++)
                            g[r * nt + t] = block(numels[t] * es);
                    void** flat = blocks(p, total * es);
                    expect_ok(oracle_bucket_allreduce(g, numels, nt, p, bucket_bytes[bi], flat, dt, op),
                              "bucket_allreduce");
                    free_blocks(flat, p);
                    free_blocks(g, p * nt);
                }
    /* the HSDP layer: numels divisible by every shard size used */
    const size_t hn[] = {48, 0, 16, 96};
    const int hnt = 4;
    const int meshes[][2] = {{1, 1}, {2, 1}, {1, 2}, {2, 2}, {2, 4}, {4, 2}, {1, 16}, {16, 1}};
    for (int dt = 0; dt < 3; dt++)
        for (int op = 0; op < 4; op++)
            for (size_t mi = 0; mi < sizeof meshes / sizeof *meshes; mi++) {
                int rep = meshes[mi][0], sh = meshes[mi][1], p = rep * sh;
                size_t es = kEsize[dt], shard_total = 0;
                for (int t = 0; t < hnt; t++)
                    shard_total += hn[t] / (size_t)sh;
                void** g = malloc(sizeof(void*) * (size_t)p * hnt);
                void** o = malloc(sizeof(void*) * (size_t)p * hnt);
                for (int r = 0; r < p; r++)
                    for (int t = 0; t < hnt; t++) {
                        g[r * hnt + t] = block(hn[t] * es);
                        o[r * hnt + t] = block(hn[t] / (size_t)sh * es);
                    }
                void** work = blocks(p, shard_total * es);
                expect_ok(oracle_hsdp_layer((const void* const*)g, o, hn, hnt, rep, sh, 12 * es, work, dt, op),
                          "hsdp_layer");
                free_blocks(work, p);
                free_blocks(g, p * hnt);
                free_blocks(o, p * hnt);
            }
}

static void barrier_and_bf16(void)
{
    for (size_t pi = 0; pi < sizeof kRanks / sizeof *kRanks; pi++) {
        int p = kRanks[pi];
        int32_t* w = calloc((size_t)p * (size_t)p, sizeof(int32_t));
        if (oracle_barrier(w, p, 1, 1000) != 1000) {
            fprintf(stderr, "barrier P=%d did not pass every generation\n", p);
            failures++;
        }
        free(w);
    }
    float specials[] = {0.0f, -0.0f, 1.0f, -1.0f, 3.4e38f, -3.4e38f, 1e-45f, 1.17e-38f};
    uint16_t out[8];
    oracle_float_to_bf16_array(specials, out, 8);
    for (int i = 0; i < 1 << 20; i++) {
        uint32_t u = (uint32_t)next_u64();
        float f;
        memcpy(&f, &u, sizeof f);
        (void)oracle_float_to_bf16(f);
    }
}

int main(void)
{
    reductions();
    copies();
    buckets();
    barrier_and_bf16();
    if (failures) {
        fprintf(stderr, "%d calls failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
