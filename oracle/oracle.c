/*
 * oracle.c -- plain, slow, single-threaded CPU definition of the same-device
 * collective primitives.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP
 * library and must never sit on the product path.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark load it.  It shares no
 * code, header, table or helper with the GPU library.
 *
 * Sources (the four pages of the collective-communication reading list):
 *  [DTorch]  "集合通信组件" (DTorch developer guide, tensor communication):
 *            sec. 2.1 ThreadGroup primitives, sec. 2.3 same-device backend
 *            AllReduce listing, sec. 2.5 placement-transition dispatch.
 *  [c10d]    "PyTorch 通信栈: ProcessGroupNCCL 与 stream" (arganzheng.life):
 *            sec. 6.1 alpha-beta accounting, sec. 6.5 coalescing and DDP bucket.
 *  [pypto]   "Barrier：仅信号（Signals Only）" (pypto distributed step 04):
 *            "The idea", "Walkthrough", "Edge cases".
 *  [HSDP]    "异步融合 AllReduce 流水线优化" (hyper-parallel issue 120):
 *            "修改方案" pipeline, sec. 6 AllReduceParamGroup.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): left fold over ranks 0..P-1 per element; fp32 accumulation for fp32
 * and bf16 inputs with ONE round-to-nearest-even rounding back to bf16 at the
 * end (the DTorch listing adds in the tensor dtype; the required precision is
 * fp32 accumulation); int32 sums wrap modulo 2^32; max/min use a strict compare
 * that keeps the earlier rank on ties and lets the first NaN met win.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * No FMA contraction, no reassociation, SSE scalar float (IEEE binary32).
 * The same source built with -fopenmp spreads the independent outer loops of
 * the AllReduce, ReduceScatter and AllGather over the host's cores (the
 * all-cores leg of the CPU timing).  Each thread takes whole elements (or
 * whole outputs) and every element is still folded by one thread in rank
 * order, so both builds give the same bits; without -fopenmp the loops are
 * the plain single-threaded ones.
 *
 * Pins: every function here is checked by the CPU test suite against brute
 * force on tiny inputs, closed forms, numpy/torch library special cases,
 * Higham's recursive-summation error bound and the pages' printed patterns.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#define OR_PARALLEL_FOR _Pragma("omp parallel for schedule(static)")
#else
#define OR_PARALLEL_FOR
#endif

enum { OR_FLOAT32 = 0, OR_BFLOAT16 = 1, OR_INT32 = 2 };
enum { OR_SUM = 0, OR_MAX = 1, OR_MIN = 2, OR_AVG = 3 };
enum { OR_OK = 0, OR_BAD_ARG = 1 };

/* Threads the parallel loops use: 1 unless built with -fopenmp. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 word. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, IEEE-754 round to nearest, ties to even, from the bit
 * pattern.  A NaN stays a NaN: sign and top payload bits are kept and the
 * quiet bit is set.  Overflow to +-inf falls out of the rounding itself. */
uint16_t oracle_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower_half_keep_bit = (u >> 16) & 1u;
    u += 0x7FFFu + lower_half_keep_bit;
    return (uint16_t)(u >> 16);
}

void oracle_float_to_bf16_array(const float* in, uint16_t* out, size_t n)
{
    for (size_t i = 0; i < n; i++)
        out[i] = oracle_float_to_bf16(in[i]);
}

/* ------------------------------------------------------------ operators --- */

static int is_nan_f(float v) { return v != v; }

/* a (+) v for floats.  Sum: one IEEE binary32 addition.  Max/min: strict
 * compare; the accumulator keeps its value on ties (earlier rank wins,
 * including +0/-0), and a NaN, once met, is kept. */
static float combine_f(float a, float v, int op)
{
    if (op == OR_SUM)
        return a + v;
    if (is_nan_f(a))
        return a;
    if (is_nan_f(v))
        return v;
    if (op == OR_MAX)
        return (v > a) ? v : a;
    return (v < a) ? v : a;
}

static int32_t combine_i(int32_t a, int32_t v, int op)
{
    if (op == OR_SUM)
        return (int32_t)((uint32_t)a + (uint32_t)v); /* two's-complement wrap */
    if (op == OR_MAX)
        return (v > a) ? v : a;
    return (v < a) ? v : a;
}

/* Element e of rank r, widened to the accumulation type. */
static float load_as_float(const void* base, size_t e, int dtype)
{
    if (dtype == OR_BFLOAT16)
        return bf16_bits_to_float(((const uint16_t*)base)[e]);
    return ((const float*)base)[e];
}

static void store_from_float(void* base, size_t e, float v, int dtype)
{
    if (dtype == OR_BFLOAT16)
        ((uint16_t*)base)[e] = oracle_float_to_bf16(v);
    else
        ((float*)base)[e] = v;
}

static size_t elem_size(int dtype)
{
    return dtype == OR_BFLOAT16 ? 2u : 4u;
}

static int valid(int nranks, int dtype, int op)
{
    return nranks >= 1 && (dtype == OR_FLOAT32 || dtype == OR_BFLOAT16 || dtype == OR_INT32) &&
           (op == OR_SUM || op == OR_MAX || op == OR_MIN || op == OR_AVG);
}

/* The fold of [DTorch] sec. 2.3: start from rank 0's element, then combine
 * ranks 1..P-1 in rank order.  Inputs are x[r] + offset, element e.
 * AVG ([HSDP] sec. 6 divides the summed gradient by the group size): the
 * same sum, then one division by P in the accumulation type (IEEE binary32
 * division; C's truncating division for int32) before the final rounding. */
static void fold_one(const void* const* x, size_t offset, int nranks, size_t e, int dtype, int op,
                     void* out, size_t out_e)
{
    const int fold_op = op == OR_AVG ? OR_SUM : op;
    if (dtype == OR_INT32) {
        int32_t acc = ((const int32_t*)x[0])[offset + e];
        for (int r = 1; r < nranks; r++)
            acc = combine_i(acc, ((const int32_t*)x[r])[offset + e], fold_op);
        if (op == OR_AVG)
            acc = acc / nranks;
        ((int32_t*)out)[out_e] = acc;
    } else {
        float acc = load_as_float(x[0], offset + e, dtype);
        for (int r = 1; r < nranks; r++)
            acc = combine_f(acc, load_as_float(x[r], offset + e, dtype), fold_op);
        if (op == OR_AVG)
            acc = acc / (float)nranks;
        store_from_float(out, out_e, acc, dtype);
    }
}

/* --------------------------------------------------------- primitives --- */

/* AllReduce, Partial -> Replicate ([DTorch] sec. 2.1, sec. 2.5): every rank q
 * receives y_q[e] = fold_r x_r[e].  The page's backend aliases rank 0's result
 * for all ranks; here each of the P outputs is written. */
int oracle_allreduce(const void* const* x, void* const* y, int nranks, size_t count, int dtype, int op)
{
    if (!valid(nranks, dtype, op))
        return OR_BAD_ARG;
    OR_PARALLEL_FOR
    for (size_t e = 0; e < count; e++) {
        fold_one(x, 0, nranks, e, dtype, op, y[0], e);
        for (int q = 1; q < nranks; q++)
            memcpy((char*)y[q] + e * elem_size(dtype), (const char*)y[0] + e * elem_size(dtype),
                   elem_size(dtype));
    }
    return OR_OK;
}

/* ReduceScatterTensor, Partial -> Shard(0) ([DTorch] sec. 2.1, sec. 2.5): each
 * rank's input has P*m elements; rank r keeps chunk r of the reduction:
 * y_r[i] = fold_q x_q[r*m + i]. */
int oracle_reduce_scatter(const void* const* x, void* const* y, int nranks, size_t m, int dtype, int op)
{
    if (!valid(nranks, dtype, op))
        return OR_BAD_ARG;
    for (int r = 0; r < nranks; r++) {
        OR_PARALLEL_FOR
        for (size_t i = 0; i < m; i++)
            fold_one(x, (size_t)r * m, nranks, i, dtype, op, y[r], i);
    }
    return OR_OK;
}

/* AllGather into one tensor, Shard(0) -> Replicate ([DTorch] sec. 2.1: the
 * equal-shape form and the uneven form whose per-rank sizes come from the
 * operand).  Output = the ranks' pieces concatenated in rank order, so rank r's
 * piece starts at the sum of the counts of ranks before it. */
int oracle_all_gather(const void* const* x, void* const* y, int nranks, const size_t* counts,
                      size_t esize)
{
    if (nranks < 1 || esize == 0)
        return OR_BAD_ARG;
    OR_PARALLEL_FOR
    for (int q = 0; q < nranks; q++) {
        size_t at = 0;
        for (int r = 0; r < nranks; r++) {
            memcpy((char*)y[q] + at * esize, x[r], counts[r] * esize);
            at += counts[r];
        }
    }
    return OR_OK;
}

/* AllToAll, Shard -> Shard ([DTorch] sec. 2.1, sec. 2.5), split-matrix form:
 * splits[i*P + j] elements travel from rank i to rank j.  Rank i's input holds
 * its outgoing blocks ordered by destination; rank j's output holds its
 * incoming blocks ordered by source. */
int oracle_all_to_all(const void* const* x, void* const* y, int nranks, const size_t* splits,
                      size_t esize)
{
    if (nranks < 1 || esize == 0)
        return OR_BAD_ARG;
    for (int i = 0; i < nranks; i++) {
        for (int j = 0; j < nranks; j++) {
            size_t send_off = 0; /* blocks i -> 0..j-1 come first in x_i */
            for (int jj = 0; jj < j; jj++)
                send_off += splits[(size_t)i * nranks + jj];
            size_t recv_off = 0; /* blocks 0..i-1 -> j come first in y_j */
            for (int ii = 0; ii < i; ii++)
                recv_off += splits[(size_t)ii * nranks + j];
            memcpy((char*)y[j] + recv_off * esize, (const char*)x[i] + send_off * esize,
                   splits[(size_t)i * nranks + j] * esize);
        }
    }
    return OR_OK;
}

/* DDP-style fused bucket AllReduce ([c10d] sec. 6.5): per rank, flatten the
 * listed tensors in order into one contiguous buffer, cut it into consecutive
 * buckets of at most bucket_bytes, AllReduce each bucket (the fold above),
 * then copy the result back into each tensor.  grads[r*ntensors + t] is rank
 * r's tensor t, reduced in place.  flat[r] is a host work buffer per rank
 * that holds sum(numels) elements. */
int oracle_bucket_allreduce(void* const* grads, const size_t* numels, int ntensors, int nranks,
                            size_t bucket_bytes, void* const* flat, int dtype, int op)
{
    if (!valid(nranks, dtype, op) || ntensors < 0)
        return OR_BAD_ARG;
    size_t es = elem_size(dtype);
    size_t per_bucket = bucket_bytes / es;
    if (per_bucket == 0)
        return OR_BAD_ARG;
    size_t total = 0;
    for (int t = 0; t < ntensors; t++)
        total += numels[t];

    /* flatten */
    for (int r = 0; r < nranks; r++) {
        size_t at = 0;
        for (int t = 0; t < ntensors; t++) {
            memcpy((char*)flat[r] + at * es, grads[(size_t)r * ntensors + t], numels[t] * es);
            at += numels[t];
        }
    }
    /* reduce bucket by bucket, in place on the flat buffers */
    for (size_t start = 0; start < total; start += per_bucket) {
        size_t len = total - start < per_bucket ? total - start : per_bucket;
        for (size_t e = 0; e < len; e++) {
            fold_one((const void* const*)flat, start, nranks, e, dtype, op, (char*)flat[0] + start * es, e);
            for (int q = 1; q < nranks; q++)
                memcpy((char*)flat[q] + (start + e) * es, (char*)flat[0] + (start + e) * es, es);
        }
    }
    /* unflatten */
    for (int r = 0; r < nranks; r++) {
        size_t at = 0;
        for (int t = 0; t < ntensors; t++) {
            memcpy(grads[(size_t)r * ntensors + t], (char*)flat[r] + at * es, numels[t] * es);
            at += numels[t];
        }
    }
    return OR_OK;
}

/* One layer of the HSDP gradient reduction ([HSDP] "修改方案"): ranks form a
 * replicate x shard mesh, rank = i*shard + j.  Step 1, ReduceScatter of every
 * tensor over the shard group {i*shard .. i*shard+shard-1} along dim 0
 * (chunk j to member j), result rounded to the tensor dtype.  Step 2, the
 * shards of rank (i,j) are flattened in tensor order into one fused buffer
 * and AllReduced over the replicate group {j, shard+j, 2*shard+j, ...} in
 * buckets of at most bucket_bytes.  Step 3, each parameter's reduced shard
 * is the matching view of the fused buffer.
 *   grads[r*ntensors + t]  rank r's full gradient t (numels[t] elements,
 *                          numels[t] divisible by shard)
 *   out[r*ntensors + t]    rank r's reduced shard of t (numels[t]/shard)
 *   work[r]                host buffer of sum(numels)/shard elements per rank */
int oracle_hsdp_layer(const void* const* grads, void* const* out, const size_t* numels, int ntensors,
                      int replicate, int shard, size_t bucket_bytes, void* const* work, int dtype, int op)
{
    int nranks = replicate * shard;
    if (!valid(nranks, dtype, op) || replicate < 1 || shard < 1 || ntensors < 0)
        return OR_BAD_ARG;
    size_t es = elem_size(dtype);
    for (int t = 0; t < ntensors; t++)
        if (numels[t] % (size_t)shard != 0)
            return OR_BAD_ARG;

    /* step 1: ReduceScatter inside each shard group, written straight into the
       fused buffer of each member (flatten order = tensor order) */
    const void* members[64];
    if (shard > 64 || replicate > 64)
        return OR_BAD_ARG;
    for (int i = 0; i < replicate; i++) {
        size_t at = 0;
        for (int t = 0; t < ntensors; t++) {
            size_t m = numels[t] / (size_t)shard;
            for (int jj = 0; jj < shard; jj++)
                members[jj] = grads[(size_t)(i * shard + jj) * ntensors + t];
            for (int j = 0; j < shard; j++)
                for (size_t e = 0; e < m; e++)
                    fold_one(members, (size_t)j * m, shard, e, dtype, op, work[i * shard + j], at + e);
            at += m;
        }
    }

    /* step 2: bucketed AllReduce across each replicate group */
    size_t total = 0;
    for (int t = 0; t < ntensors; t++)
        total += numels[t] / (size_t)shard;
    size_t per_bucket = bucket_bytes / es;
    if (per_bucket == 0)
        return OR_BAD_ARG;
    void* group[64];
    for (int j = 0; j < shard; j++) {
        for (int i = 0; i < replicate; i++)
            group[i] = work[i * shard + j];
        for (size_t start = 0; start < total; start += per_bucket) {
            size_t len = total - start < per_bucket ? total - start : per_bucket;
            for (size_t e = 0; e < len; e++) {
                fold_one((const void* const*)group, start, replicate, e, dtype, op, group[0], start + e);
                for (int i = 1; i < replicate; i++)
                    memcpy((char*)group[i] + (start + e) * es, (char*)group[0] + (start + e) * es, es);
            }
        }
    }

    /* step 3: unflatten into per-parameter shards */
    for (int r = 0; r < nranks; r++) {
        size_t at = 0;
        for (int t = 0; t < ntensors; t++) {
            size_t m = numels[t] / (size_t)shard;
            memcpy(out[(size_t)r * ntensors + t], (char*)work[r] + at * es, m * es);
            at += m;
        }
    }
    return OR_OK;
}

/* Broadcast ([DTorch] sec. 2.2 lists it among the backend's collectives):
 * every rank's output is a copy of the root rank's tensor. */
int oracle_broadcast(const void* x_root, void* const* y, int nranks, size_t nbytes)
{
    if (nranks < 1)
        return OR_BAD_ARG;
    for (int q = 0; q < nranks; q++)
        memcpy(y[q], x_root, nbytes);
    return OR_OK;
}

/* ReplicateToShard, Replicate -> Shard(0) ([DTorch] sec. 2.1, sec. 2.5: no
 * communication, each rank keeps its own slice): x_r holds P*m elements,
 * y_r = slice r of x_r. */
int oracle_replicate_to_shard(const void* const* x, void* const* y, int nranks, size_t m, size_t esize)
{
    if (nranks < 1 || esize == 0)
        return OR_BAD_ARG;
    for (int r = 0; r < nranks; r++)
        memcpy(y[r], (const char*)x[r] + (size_t)r * m * esize, m * esize);
    return OR_OK;
}

/* AllGatherIntoVec ([DTorch] sec. 2.1): the gathered pieces stay separate
 * tensors; rank q's vector entry r is rank r's piece: y[q*P + r] = x_r. */
int oracle_all_gather_into_vec(const void* const* x, void* const* y, int nranks, const size_t* counts,
                               size_t esize)
{
    if (nranks < 1 || esize == 0)
        return OR_BAD_ARG;
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < nranks; r++)
            memcpy(y[(size_t)q * nranks + r], x[r], counts[r] * esize);
    return OR_OK;
}

/* AllToAll between shard dimensions of a row-major [rows, cols] tensor G
 * ([DTorch] sec. 2.1 AllToAll(input, srcDim, destDim), sec. 2.5 S -> S).
 * Shard(0): rank i holds rows [i*rows/P, (i+1)*rows/P), a [rows/P, cols]
 * block.  Shard(1): rank i holds columns [i*cols/P, (i+1)*cols/P), a
 * [rows, cols/P] block.  Element by element: rebuild G's element (a, b)
 * from its owner under src_dim, store it at its place under dst_dim. */
int oracle_all_to_all_dims(const void* const* x, void* const* y, int nranks, size_t rows, size_t cols,
                           int src_dim, int dst_dim, size_t esize)
{
    if (nranks < 1 || esize == 0 || src_dim < 0 || src_dim > 1 || dst_dim < 0 || dst_dim > 1)
        return OR_BAD_ARG;
    if ((src_dim == 0 || dst_dim == 0) && rows % (size_t)nranks != 0)
        return OR_BAD_ARG;
    if ((src_dim == 1 || dst_dim == 1) && cols % (size_t)nranks != 0)
        return OR_BAD_ARG;
    size_t rp = rows / (size_t)nranks, cp = cols / (size_t)nranks;
    for (size_t a = 0; a < rows; a++) {
        for (size_t b = 0; b < cols; b++) {
            const char* from;
            if (src_dim == 0)
                from = (const char*)x[a / rp] + ((a % rp) * cols + b) * esize;
            else
                from = (const char*)x[b / cp] + (a * cp + b % cp) * esize;
            char* to;
            if (dst_dim == 0)
                to = (char*)y[a / rp] + ((a % rp) * cols + b) * esize;
            else
                to = (char*)y[b / cp] + (a * cp + b % cp) * esize;
            memcpy(to, from, esize);
        }
    }
    return OR_OK;
}

/* Signal-window barrier ([pypto] "The idea", "Walkthrough"): window[p*P + s]
 * is cell s of rank p's window.  One generation: every rank r adds 1 to cell r
 * of every other rank's window (never its own), then waits until every cell
 * s != r of its own window has reached the generation number g (Ge compare,
 * threshold raised by one per reuse, "Edge cases" table).  Run sequentially
 * here: all notifies of a generation, then the wait checks.  Returns the
 * number of generations whose waits all passed. */
int oracle_barrier(int32_t* window, int nranks, int first_generation, int generations)
{
    int passed = 0;
    for (int k = 0; k < generations; k++) {
        int g = first_generation + k;
        for (int r = 0; r < nranks; r++)
            for (int p = 0; p < nranks; p++)
                if (p != r)
                    window[(size_t)p * nranks + r] += 1;
        int ok = 1;
        for (int r = 0; r < nranks; r++)
            for (int s = 0; s < nranks; s++)
                if (s != r && window[(size_t)r * nranks + s] < g)
                    ok = 0;
        passed += ok;
    }
    return passed;
}

/* The built-in barrier demonstration of [pypto] "Walkthrough": each rank
 * stages its slice, meets the barrier, then loads the next rank's slice, so
 * y_r = x_{(r+1) mod P}. */
int oracle_barrier_exchange(const void* const* x, void* const* y, int nranks, size_t nbytes)
{
    if (nranks < 1)
        return OR_BAD_ARG;
    for (int r = 0; r < nranks; r++)
        memcpy(y[r], x[(r + 1) % nranks], nbytes);
    return OR_OK;
}
