/*
 * dt.h -- C ABI of the same-device collective library (libdtcoll.so).
 *
 * P logical ranks whose buffers all live in one GPU's HBM exchange data
 * through HIP kernels.  This is the same-device backend described in the
 * DTorch developer guide page "集合通信组件" (sec. 2.3,
 * ThreadGroupSameDeviceBackend): several ranks bound to one GPU, which NCCL
 * cannot serve.  Here a whole collective is one kernel launch instead of a
 * host-thread handshake through a tensor store.
 *
 * Conventions for every call:
 *  - Counts are in ELEMENTS, as in the ncclAllReduce(sendbuf, recvbuf, count,
 *    dtype, op, comm, stream) shape quoted on the page "PyTorch communication
 *    stack: ProcessGroupNCCL and streams" (arganzheng.life), sec. 4.1.
 *  - send/recv are HOST arrays of nranks DEVICE pointers (rank r's buffer is
 *    send[r]); each rank buffer is one contiguous row-major allocation on the
 *    current HIP device.  The host arrays are read during the call only.
 *  - Every call is enqueue-only on `stream` (a hipStream_t; NULL = the null
 *    stream): it never blocks the host on the GPU.  As in that page's sec. 4.2
 *    and 4.4, returning means "queued", not "done"; the caller orders
 *    producers and consumers with stream order or events (dt_work_* below).
 *  - Device buffers are caller-owned.  They must stay allocated and must not
 *    be written by other streams until the stream has passed the call (the
 *    lifetime rules of that page's sec. 5).  The library allocates no device
 *    memory and keeps no device state between calls.
 *  - 1 <= nranks <= DT_MAX_RANKS.  count == 0 is a no-op that returns DT_OK.
 *  - Element types: fp32, bf16 (accumulated in fp32, rounded once to nearest
 *    even), int32 (sums wrap modulo 2^32).  Reductions fold the ranks in rank
 *    order 0, 1, ..., P-1 for every element, so results are deterministic.
 *  - Errors: DT_ERR_ARG for NULL pointers, bad enums, out-of-range sizes or
 *    buffers that overlap where a launch would race (a written byte range
 *    meeting another written or read one; exact in-place operands are
 *    allowed where a call says so); DT_ERR_HIP when a launch fails.  Nothing throws across
 *    the ABI; dt_last_error() gives this thread's last message.
 *  - Fast path: 16-byte aligned buffers and offsets.  A fold whose buffers
 *    all sit at one offset past an alignment boundary (4 KiB, 1 KiB, 128 or
 *    16 bytes: the deepest one they share) folds the elements before that
 *    boundary, with the ragged end, in one element launch and the rest the
 *    fast way; a two-shot AllReduce does the same for line-aligned buffers
 *    that share an offset within 1 KiB (its tiles then start on 1 KiB
 *    boundaries).  Folds over element-aligned buffers at offsets of their
 *    own (inputs and outputs apart, or rank by rank), and ReduceScatters
 *    whose chunks of the inputs do not all start on 128-byte lines, tile
 *    over each output's 128-byte lines, load every input's lines whole and
 *    shift them into place: the ReduceScatter always, the AllReduce from
 *    P * S = 160 MiB for 6 <= P <= 12, 256 MiB otherwise (S the bytes per
 *    rank) on (as a ReduceScatter into
 *    each output's own chunk and a fan-out of the chunks; 16-byte aligned
 *    inputs off their lines take this form too where the two-shot form
 *    pays); smaller AllReduces over buffers at offsets of their own fold
 *    element by element.  The copy engines
 *    store whole 128-byte lines of every destination that does not start
 *    on one, built from aligned loads whatever the source offset (the
 *    fan-out over each destination's own line grid when the destinations
 *    of a piece do not share one offset within a line).  Every path gives the
 *    same bits.
 */
#ifndef DT_H
#define DT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DT_MAX_RANKS 16

typedef enum { DT_FLOAT32 = 0, DT_BFLOAT16 = 1, DT_INT32 = 2 } dt_dtype;
/* DT_AVG: the rank-order sum divided once by the number of ranks in the
 * collective (fp32 IEEE division before the bf16 rounding; truncating
 * division of the wrapped sum for int32).  The hyper-parallel issue's
 * AllReduceParamGroup (sec. 6) divides the summed gradient by the group size. */
typedef enum { DT_SUM = 0, DT_MAX = 1, DT_MIN = 2, DT_AVG = 3 } dt_op;
typedef enum {
    DT_OK = 0,
    DT_ERR_ARG = 1,
    DT_ERR_UNSUPPORTED = 2,
    DT_ERR_HIP = 3,
    DT_ERR_TIMEOUT = 4
} dt_status;

/* AllReduce, Partial -> Replicate: recv[q][e] = fold_{r=0..P-1} send[r][e]
 * for every rank q.  DTorch page "集合通信组件" sec. 2.1 (AllReduce) and
 * sec. 2.3 (the same-device listing folds rank 0 then ranks 1..P-1 on one
 * rank and hands the result to all).  Usually one launch: each element is
 * read once per rank and written once per rank (the one-shot form of the
 * c10d page, sec. 9.4).  From 12 MiB per rank up for P >= 16, from 16 to
 * 256 MiB for 11 <= P <= 15, from 24 to 256 MiB for 8 <= P <= 10, from 32
 * to 256 MiB for 5 <= P <= 7 and from 128 to 192 MiB for P = 4, with
 * 16-byte aligned buffers, it runs as a
 * ReduceScatter into chunk r of recv[r] (chunks of whole 1 KiB tiles, the
 * last one shorter) followed by an in-place AllGather of the chunks, which
 * is faster there (elements past the last whole vector take the element
 * path).  Beyond 256 MiB per rank for P >= 5 it runs window by
 * window (64 MiB per rank at P >= 16, 128 MiB at P = 5-15), each window an
 * AllReduce of its own in the two-shot form, so the window's chunks are
 * still in the Infinity Cache when they fan out.  Buffers at offsets of
 * their own take the two-shot form over line grids from nranks * count *
 * element size = 160 MiB for 6 <= P <= 12, 256 MiB otherwise (see the
 * alignment convention above).  All forms
 * fold in the
 * same order and give identical bits.  In place is allowed (send[r] ==
 * recv[r]); any other overlap of a recv buffer with a send or recv buffer
 * is refused (DT_ERR_ARG).  send[r] and recv[r] hold `count` elements. */
dt_status dt_allreduce(const void* const* send, void* const* recv, int nranks, size_t count,
                       dt_dtype dtype, dt_op op, hipStream_t stream);

/* ReduceScatter, Partial -> Shard(0): send[r] holds nranks*recvcount
 * elements; recv[r][i] = fold_q send[q][r*recvcount + i].  DTorch page
 * sec. 2.1 (ReduceScatterTensor) and sec. 2.5 (P -> S0).  recv buffers must
 * overlap neither any send buffer nor each other (DT_ERR_ARG). */
dt_status dt_reduce_scatter(const void* const* send, void* const* recv, int nranks, size_t recvcount,
                            dt_dtype dtype, dt_op op, hipStream_t stream);

/* AllGather into one tensor, Shard(0) -> Replicate: recv[q] = send[0] ++
 * send[1] ++ ... ++ send[P-1] for every q.  DTorch page sec. 2.1: the
 * equal-shape form (sendcounts == NULL, every rank sends equal_count) and
 * the uneven form (sendcounts = host array of nranks element counts; rank
 * r's piece lands at the sum of the counts before it).  A byte copy: dtype
 * only sets the element size.  recv[q] holds sum(sendcounts) elements. */
dt_status dt_all_gather(const void* const* send, void* const* recv, int nranks, const size_t* sendcounts,
                        size_t equal_count, dt_dtype dtype, hipStream_t stream);

/* AllGatherIntoVec (DTorch page sec. 2.1): the gathered pieces stay separate
 * tensors.  recv[q*nranks + r] (sendcounts[r] elements, or equal_count when
 * sendcounts is NULL) receives a copy of send[r] for every rank q: one launch,
 * each piece read once and written nranks times. */
dt_status dt_all_gather_into_vec(const void* const* send, void* const* recv, int nranks, const size_t* sendcounts,
                                 size_t equal_count, dt_dtype dtype, hipStream_t stream);

/* Broadcast (DTorch page sec. 2.2 lists broadcast among the backend's
 * collectives): recv[q] = root_send (count elements) for every q.  One read of
 * the root's buffer, nranks writes.  recv[root] may equal root_send. */
dt_status dt_broadcast(const void* root_send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                       hipStream_t stream);

/* ReplicateToShard, Replicate -> Shard(0) (DTorch page sec. 2.1 and 2.5; no
 * exchange between ranks): recv[r] = elements [r*recvcount, (r+1)*recvcount)
 * of send[r], where send[r] holds nranks*recvcount elements. */
dt_status dt_replicate_to_shard(const void* const* send, void* const* recv, int nranks, size_t recvcount,
                                dt_dtype dtype, hipStream_t stream);

/* AllToAll between shard dimensions (DTorch page sec. 2.1 AllToAll(input,
 * srcDim, destDim) and sec. 2.5 S -> S) of a row-major [rows, cols] tensor.
 * Under Shard(0) rank r holds rows [r*rows/P, (r+1)*rows/P) as a contiguous
 * [rows/P, cols] block; under Shard(1) it holds columns [r*cols/P,
 * (r+1)*cols/P) as a contiguous [rows, cols/P] block.  send[r] is rank r's
 * block under src_dim, recv[r] receives its block under dst_dim.  The
 * sharded dimension(s) must divide by nranks (DT_ERR_ARG otherwise);
 * src_dim == dst_dim copies each rank's block. */
dt_status dt_all_to_all_dims(const void* const* send, void* const* recv, int nranks, size_t rows, size_t cols,
                             int src_dim, int dst_dim, dt_dtype dtype, hipStream_t stream);

/* AllToAll, Shard -> Shard, split-matrix form: splits is a host array of
 * nranks*nranks element counts, splits[i*nranks + j] = elements rank i sends
 * to rank j.  send[i] holds its outgoing blocks ordered by destination;
 * recv[j] holds its incoming blocks ordered by source.  DTorch page sec. 2.1
 * (AllToAll) and sec. 2.5 (S -> S).  Each split must be below 2^40 and the
 * per-launch tile count below 2^31 (DT_ERR_ARG otherwise). */
dt_status dt_all_to_all(const void* const* send, void* const* recv, int nranks, const size_t* splits,
                        dt_dtype dtype, hipStream_t stream);

/* DDP-style fused-bucket gradient AllReduce, in place.  c10d page sec. 6.5:
 * the tensors are flattened in the listed order into one contiguous buffer,
 * cut into buckets of at most bucket_bytes (the page's default cap is 25
 * MB; this library reads it as 25 MiB), each bucket is AllReduced, and the
 * result is copied back.  grads[r*ntensors + t] is rank r's tensor t with
 * numels[t] elements.
 *   bucket_ws != NULL: nranks device buffers of at least bucket_bytes each;
 *     each bucket is copied in by one multi-tensor launch, reduced in place,
 *     and copied back by one launch (the page's flatten/unflatten).
 *   bucket_ws == NULL: the buckets are reduced straight out of the tensors
 *     and back into them (no staging copies).  A tensor of at least 16 MiB
 *     per rank is AllReduced on its own, exactly as dt_allreduce would do
 *     it; the pieces of the smaller tensors go out together in as few
 *     multi-tensor launches as the piece tables allow: one for up to
 *     min(32, 320 / nranks) pieces, else one per min(512, 4096 / nranks).
 * Both forms give the same bits as dt_allreduce on each tensor.  bucket_bytes
 * must be a positive multiple of 16. */
dt_status dt_bucket_allreduce(void* const* grads, const size_t* numels, int ntensors, int nranks,
                              size_t bucket_bytes, void* const* bucket_ws, dt_dtype dtype, dt_op op,
                              hipStream_t stream);

/* Size of the static staging buffer of dt_bucket_allreduce_noalloc, bytes. */
#define DT_SCRATCH_BYTES (256u << 20)

/* dt_bucket_allreduce with staging (bucket_ws != NULL) for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Instead of caller workspaces,
 * rank r's buckets are staged in a static device array of DT_SCRATCH_BYTES
 * (256 MiB), at byte offset r * bucket_bytes, so nranks * bucket_bytes may
 * not exceed DT_SCRATCH_BYTES (DT_ERR_ARG otherwise; eight ranks of the
 * default 25 MiB bucket fit).  Everything else is as dt_bucket_allreduce with
 * a workspace: the same plan, kernels and bits.  The call allocates nothing:
 * each GPU holds its own copy of the array, set up by the first call with
 * that device current (make that first call outside graph capture) and kept
 * until the process ends.  All calls on one GPU share that GPU's array, so
 * calls that may overlap in time on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  No part of the array needs to
 * start at zero: every byte a call reads back was written by the same call. */
dt_status dt_bucket_allreduce_noalloc(void* const* grads, const size_t* numels, int ntensors, int nranks,
                                      size_t bucket_bytes, dt_dtype dtype, dt_op op, hipStream_t stream);

/* Where the ranks of a barrier launch run.  The spread layout needs a
 * cooperative launch, which the HIP runtime may refuse (DT_ERR_HIP, with its
 * message in dt_last_error) while another process shares the GPU; the
 * packed layout is an ordinary launch and always runs. */
typedef enum {
    DT_BARRIER_PACKED = 0, /* one workgroup, one 64-wide wave per rank: always co-resident, plain launch */
    DT_BARRIER_SPREAD = 1  /* one workgroup per rank on different CUs, cooperative launch */
} dt_barrier_layout;

/* Coalesced AllReduce, in place: many separate tensors reduced in one
 * launch, the all_reduce_coalesced / _coalescing_manager form of the c10d
 * page sec. 6.5 (several non-contiguous tensors, one launch and one event,
 * no flattening).  tensors[r*ntensors + t] is rank r's tensor t with
 * numels[t] elements; every tensor gets the same bits as dt_allreduce on it.
 * Up to 4096/nranks tensors (at most 512) per launch; more take several
 * launches.  Empty tensors may pass NULL. */
dt_status dt_allreduce_coalesced(void* const* tensors, const size_t* numels, int ntensors, int nranks, dt_dtype dtype,
                                 dt_op op, hipStream_t stream);

/* Signal-window barrier.  pypto page "Barrier：仅信号（Signals Only）",
 * "The idea" and "Walkthrough": windows[p] is rank p's window of nranks int32
 * cells in device memory (zeroed once by the caller before its first use).
 * In generation g every rank r atomically adds 1 to cell r of every other
 * rank's window, then waits until every cell s != r of its own window is
 * >= g, with atomics at device scope when the ranks are spread over
 * workgroups and at workgroup scope when they share one.  The launch orders
 * only the windows; dt_barrier_exchange below orders data.  Generations
 * first_generation .. first_generation + generations - 1 run back to back in
 * ONE launch; `layout` places the ranks (dt_barrier_layout).  Reusing a
 * window means passing the next generation number (the page's "Edge cases":
 * raise the threshold on reuse).  Each wait gives up after timeout_ns
 * nanoseconds (0 = 10 s): it then stores DT_ERR_TIMEOUT into *status_dev and
 * that rank stops; every wave exits normally.  *status_dev (device int32)
 * must hold DT_OK before the call. */
dt_status dt_barrier(int32_t* const* windows, int nranks, int32_t first_generation, int32_t generations,
                     int32_t* status_dev, uint64_t timeout_ns, int layout, hipStream_t stream);

/* The barrier ordering a data exchange, as in the pypto page's built-in
 * demonstration: every rank r copies src[r] (nbytes) to stage[r], meets the
 * barrier of generation `generation` on `windows`, then copies stage[(r+1) %
 * nranks] to dst[r].  A release fence separates the staging from the
 * notifies and an acquire fence the waits from the reads, so every rank's
 * staged bytes are visible to its reader.  Afterwards dst[r] ==
 * src[(r+1) % nranks].  Timeout, status and layout as dt_barrier. */
dt_status dt_barrier_exchange(const void* const* src, void* const* stage, void* const* dst, size_t nbytes,
                              int32_t* const* windows, int nranks, int32_t generation, int32_t* status_dev,
                              uint64_t timeout_ns, int layout, hipStream_t stream);

/* ---- host planning (no GPU work) -------------------------------------- */

/* One contiguous part of one tensor inside one bucket. */
typedef struct {
    int32_t tensor;    /* index into numels */
    int32_t bucket;    /* bucket number */
    size_t offset;     /* first element of the part inside the tensor */
    size_t length;     /* elements */
    size_t bucket_pos; /* first element of the part inside its bucket */
} dt_piece;

/* The bucket plan dt_bucket_allreduce uses: the concatenation of the
 * tensors, cut into consecutive buckets of floor(bucket_bytes/elem_size)
 * elements (c10d page sec. 6.5; where bucket boundaries fall is left open
 * there, so tensors may straddle buckets).  Writes up to `capacity` pieces
 * and sets *npieces and *nbuckets to the full counts (call with capacity 0
 * to size the arrays).  Empty tensors yield no piece. */
dt_status dt_bucket_plan(const size_t* numels, int ntensors, size_t elem_size, size_t bucket_bytes,
                         dt_piece* pieces, size_t capacity, size_t* npieces, size_t* nbuckets);

/* ---- stream/event ordering ------------------------------------------- */

/* A work handle: the pair of events of the c10d page sec. 4.3 and 4.4.
 * dt_work_begin records an event on `producer` and makes `comm` wait on it,
 * so a collective queued next on `comm` sees everything queued before on
 * `producer`.  dt_work_end records the end event on `comm` after the
 * collective.  dt_work_wait makes `consumer` wait on the end event (a stream
 * wait: the host does not block).  dt_work_query returns 1 when the end
 * event has completed, 0 if not yet, negative on error.  The handle owns two
 * HIP events and is released by dt_work_free. */
typedef struct dt_work dt_work;
dt_status dt_work_begin(hipStream_t producer, hipStream_t comm, dt_work** work);
dt_status dt_work_end(dt_work* work, hipStream_t comm);
dt_status dt_work_wait(dt_work* work, hipStream_t consumer);
int dt_work_query(dt_work* work);
dt_status dt_work_free(dt_work* work);

/* ---- per-layer ReduceScatter -> fused AllReduce pipeline -------------- */

/* HSDP gradient reduction of the hyper-parallel issue "异步融合 AllReduce
 * 流水线优化" ("修改方案" and the sec. 6 AllReduceParamGroup methods).  Ranks
 * form a replicate x shard mesh, rank = i*shard + j.  For each layer, in
 * backward order, dt_hsdp_post_backward:
 *   1. makes the AllReduce stream wait for the previous layer's
 *      ReduceScatter ("wait prev RS"),
 *   2. queues this layer's ReduceScatter on rs_stream after everything
 *      queued so far on `producer`: every tensor t of shard group i is
 *      reduce-scattered along dim 0 straight into fused[r] at the running
 *      offset of t (sum of numels[t']/shard for t' < t), so the fused buffer
 *      is the flattened shard set,
 *   3. queues the previous layer's fused AllReduce on ar_stream: replicate
 *      group j = {j, shard+j, ...} reduces its fused buffers in place in
 *      buckets of at most bucket_bytes.
 * dt_hsdp_finish queues the last layer's AllReduce and makes `consumer`
 * wait for every AllReduce issued (the root backward hook); each parameter's
 * reduced shard is then the matching slice of its layer's fused buffers.
 * fused[r] holds sum(numels)/shard elements and must stay valid until the
 * consumer has waited.  numels[t] must be divisible by shard.  fused buffers
 * may overlap neither each other, nor the layer's gradients, nor the previous
 * layer's fused buffers while that layer's AllReduce is still pending, i.e.
 * until dt_hsdp_finish (DT_ERR_ARG): reusing one fused set for every layer
 * needs a finish between layers.  dt_hsdp_destroy waits until any queued
 * ReduceScatter or AllReduce of the handle has finished writing; a layer
 * posted but not finished gets no AllReduce.  The handle
 * owns its events and keeps a host copy of the previous layer's fused
 * pointers and total size until it queues that layer's AllReduce.
 * rs_stream and ar_stream may be the same stream: the phases then run back
 * to back in the order above, which on one device (both phases drawing on
 * the same HBM) is the faster schedule, and no wait between the phases is
 * queued.  When the producer stream is rs_stream as well, no event is
 * recorded or waited per layer at all (each cross-stream wait leaves a gap
 * of several microseconds in the queue). */
typedef struct dt_hsdp dt_hsdp;
dt_status dt_hsdp_create(int replicate, int shard, size_t bucket_bytes, dt_dtype dtype, dt_op op,
                         hipStream_t rs_stream, hipStream_t ar_stream, dt_hsdp** handle);
dt_status dt_hsdp_post_backward(dt_hsdp* handle, const void* const* grads, const size_t* numels, int ntensors,
                                void* const* fused, hipStream_t producer);
dt_status dt_hsdp_finish(dt_hsdp* handle, hipStream_t consumer);
dt_status dt_hsdp_destroy(dt_hsdp* handle);

/* ---- diagnostics ------------------------------------------------------ */

const char* dt_status_string(dt_status status);
/* This thread's last error message ("" if none). */
const char* dt_last_error(void);
/* Library version string. */
const char* dt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DT_H */
