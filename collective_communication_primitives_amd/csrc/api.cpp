// api.cpp -- the C ABI of include/dt.h: argument checks, offset and tile
// tables, bucket planning, work handles and the HSDP pipeline.  Every data
// movement happens in the HIP kernels (reduce.hip, copy.hip, barrier.hip);
// this file only validates, plans and enqueues.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "dt.h"
#include "dt_launch.h"

static_assert(sizeof(dt::ReduceArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::PieceArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::GatherArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::AllToAllArgs) <= 8192, "all-to-all block table must stay well below the 64 KB verified");
static_assert(sizeof(dt::ExchangeArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::SegReduceScatterArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::SegCopyArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::DimsArgs) <= 4096, "kernel arguments must stay below 4 KiB");
static_assert(sizeof(dt::CoalescedArgs) <= 48 * 1024, "large piece table must stay well below the 64 KB verified");
static_assert(DT_MAX_RANKS == dt::kMaxRanksHost, "rank limit mismatch");
static_assert(DT_SCRATCH_BYTES == dt::kScratchBytes, "static staging size mismatch");

namespace {

thread_local std::string g_last_error;

dt_status fail(dt_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

dt_status check_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return DT_OK;
    return fail(DT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(dt_dtype d) { return d == DT_FLOAT32 || d == DT_BFLOAT16 || d == DT_INT32; }
bool valid_op(dt_op o) { return o == DT_SUM || o == DT_MAX || o == DT_MIN || o == DT_AVG; }
size_t esize_of(dt_dtype d) { return d == DT_BFLOAT16 ? 2 : 4; }
size_t vec_elems(dt_dtype d) { return 16 / esize_of(d); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// The copy engines' stores start on the destination's 128-byte lines: a
// destination off its lines (even at a 16-byte boundary) takes the line grid.
bool line_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & (dt::kGridAlign - 1)) == 0; }
bool elem_aligned(const void* p, size_t es) { return (reinterpret_cast<uintptr_t>(p) & (es - 1)) == 0; }
const char* cptr(const void* p) { return static_cast<const char*>(p); }

dt_status check_ranks(int nranks) {
    if (nranks < 1 || nranks > DT_MAX_RANKS)
        return fail(DT_ERR_ARG, "nranks=%d outside [1, %d]", nranks, DT_MAX_RANKS);
    return DT_OK;
}

template <typename T>
dt_status check_ptr_array(T const* arr, int n, const char* name) {
    if (arr == nullptr) return fail(DT_ERR_ARG, "%s is NULL", name);
    for (int i = 0; i < n; i++)
        if (arr[i] == nullptr) return fail(DT_ERR_ARG, "%s[%d] is NULL", name, i);
    return DT_OK;
}

// A byte range [lo, lo + n) of device memory, tagged for error messages:
// `name`[`index`].
struct Span {
    uintptr_t lo;
    size_t n;
    const char* name;
    int index;
};

void add_span(std::vector<Span>& v, const void* p, size_t n, const char* name, int index) {
    if (p != nullptr && n > 0) v.push_back(Span{reinterpret_cast<uintptr_t>(p), n, name, index});
}

// Refuses (DT_ERR_ARG) when two written ranges overlap, or when a read range
// overlaps a written one, unless the two are the very same range (an
// in-place operand: the kernel reads each element before writing it, from
// the same workgroup).  Kernels of different workgroups store and load
// concurrently, so any other overlap would be a data race.  O(n log n).
dt_status check_disjoint(std::vector<Span>& writes, const std::vector<Span>& reads, const char* what) {
    std::sort(writes.begin(), writes.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < writes.size(); i++) {
        const Span& a = writes[i - 1];
        const Span& b = writes[i];
        if (b.lo < a.lo + a.n)
            return fail(DT_ERR_ARG, "%s: %s[%d] and %s[%d] overlap", what, a.name, a.index, b.name, b.index);
    }
    for (const Span& r : reads) {
        // the last written range starting at or before r.lo, and the first one after it
        auto it = std::upper_bound(writes.begin(), writes.end(), r.lo,
                                   [](uintptr_t lo, const Span& s) { return lo < s.lo; });
        if (it != writes.end() && it->lo < r.lo + r.n)
            return fail(DT_ERR_ARG, "%s: %s[%d] overlaps %s[%d]", what, r.name, r.index, it->name, it->index);
        if (it != writes.begin()) {
            const Span& w = *(it - 1);
            const bool same = w.lo == r.lo && w.n == r.n;
            if (!same && r.lo < w.lo + w.n)
                return fail(DT_ERR_ARG, "%s: %s[%d] overlaps %s[%d]", what, r.name, r.index, w.name, w.index);
        }
    }
    return DT_OK;
}

// Wall-clock ticks per nanosecond budget on the current device.
uint64_t timeout_ticks(uint64_t timeout_ns) {
    static std::mutex mu;
    static int rate_khz[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int rate = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        rate = rate_khz[dev];
        if (rate == 0) {
            if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate <= 0)
                rate = 100000;  // 100 MHz, the usual constant-rate counter
            rate_khz[dev] = rate;
        }
    }
    if (timeout_ns == 0) timeout_ns = 10ull * 1000 * 1000 * 1000;
    const long double ticks = (long double)timeout_ns * (long double)rate / 1.0e6L;
    return ticks > 1.8e19L ? UINT64_MAX : (uint64_t)ticks + 1;
}

dt_status fan_out(const void* const* src, const size_t* counts, void* const* table, int nranks, size_t es,
                  hipStream_t stream, const char* what, int nsources = -1);

// ------------------------------------------------------------ reductions --
// Whether the two-shot form of the AllReduce is the faster one: a
// ReduceScatter that leaves chunk r of the result in recv[r], then an
// in-place AllGather of the chunks.  It moves (2P+1)S bytes against the
// one-shot fold's 2PS, but as a P-to-1 fold and a 1-to-P fan-out whose
// sources (S bytes in all) are still in the 256 MB Infinity Cache when the
// fan-out reads them.  Measured on the MI355X against the one-shot kernel
// (in-process A/B, graph replay, fp32 unless noted):
//   P = 16: 4-10% faster from 16 MiB per rank up; with the fan-out's two
//     workgroups per tile (from 9 ranks on) also 5-8% faster at 12 MiB, and
//     8-10% slower at 4-8 MiB;
//   P = 11-15: with that fan-out 6-11% faster at 16 MiB (P = 12 bf16: 6%),
//     within 1% at 12 MiB;
//   P = 8: 2-15% faster from 24 to 256 MiB (bf16 at 96 MiB: 1-4% slower);
//   P = 9, 12, 15: 3-15% faster from 24 MiB to 256 MiB, 2-14% slower at 8 MiB;
//     P = 9 4% slower and P = 10 even at 16 MiB, P = 10 2% faster at 20 MiB;
//   P = 5-7: 2-11% faster from 32 to 256 MiB, 2-24% slower at 8-16 MiB,
//     within 5% at 24 MiB;
//   P = 4: 0-7% faster at 128-192 MiB, mixed at 96 and 256 MiB, 18-26%
//     slower at 320 MiB.
// P = 2-3 keep the one-shot form.  Below these windows the second launch
// costs more than the pattern saves.
bool two_shot_pays(int nranks, uint64_t bytes_per_rank) {
    constexpr uint64_t MiB = 1ull << 20;
    if (nranks >= 16) return bytes_per_rank >= 12 * MiB;
    if (nranks >= 11) return bytes_per_rank >= 16 * MiB && bytes_per_rank <= 256 * MiB;
    if (nranks >= 8) return bytes_per_rank >= 24 * MiB && bytes_per_rank <= 256 * MiB;
    if (nranks >= 5) return bytes_per_rank >= 32 * MiB && bytes_per_rank <= 256 * MiB;
    if (nranks == 4) return bytes_per_rank >= 128 * MiB && bytes_per_rank <= 192 * MiB;
    return false;
}

// Per-rank window of a large AllReduce, or 0 for one call over the whole
// range.  Each element's result depends only on that element, so the
// AllReduce of a long range is the AllReduces of consecutive windows of it.
// A window runs in the two-shot form, and its ReduceScatter leaves the
// window's chunks in the Infinity Cache for the fan-out right after it,
// where one call over the whole range needs a read pass per fan-out window
// (P >= 16) or runs the one-shot kernel (P = 5-15).  Measured on the MI355X,
// in-process A/B under two buffer placements, graph replay, bit-identical:
//   P=16 fp32, 64 MiB windows against one call: 2.0-4.8% faster at 320 MiB
//     to 1 GiB per rank (1 GiB: 5516 against 5648 us, 5703 against 5816);
//     128 MiB windows -1.3..+0.2% and 256 MiB windows -1.9..+2.1% against
//     64 MiB ones; at 256 MiB one call stays faster (1371 against 1404 us);
//   P=8 bf16, 128 MiB windows against the one-shot kernel: 0.4-1.9% slower
//     at some placements, 7.6-9.5% faster at others (512 MiB, 1 GiB), so
//     the windows are the steadier choice (0.775-0.797 of peak throughout);
//     fp32 1 GiB 4741 -> 2734 us at one placement;
//   P=4: no windows: the one-shot kernel is 3-5% faster at 224-256 MiB and
//     within placement noise (+-8%) beyond.
// Each window lies inside two_shot_pays' range for its rank count.
uint64_t allreduce_window(int nranks, uint64_t bytes_per_rank) {
    constexpr uint64_t MiB = 1ull << 20;
    if (nranks >= 16) return bytes_per_rank > 256 * MiB ? 64 * MiB : 0;
    if (nranks >= 5) return bytes_per_rank > 256 * MiB ? 128 * MiB : 0;
    return 0;
}

// Validated AllReduce over one contiguous range per rank, in one call.
// ReduceScatter over line grids (dt::GridFoldArgs): chunk c is elements
// [c * in_stride, c * in_stride + n_c) of every input, n_c = count but
// last_count for the last chunk, folded into out[c].  For element-aligned
// buffers that share no offset.  The tiles follow each output's lines; the
// kernel loads every input's lines whole and shifts them in LDS, so both
// sides move whole lines whatever the offsets.
dt_status reduce_scatter_grid(const void* const* send, void* const* out, int nranks, size_t in_stride, size_t count,
                              size_t last_count, dt_dtype dtype, dt_op op, hipStream_t stream, const char* what) {
    dt::GridFoldArgs g = {};
    for (int r = 0; r < nranks; r++) {
        g.src[r] = send[r];
        g.dst[r] = out[r];
        g.lead[r] = uint32_t(reinterpret_cast<uintptr_t>(out[r]) & (dt::kGridAlign - 1));
    }
    g.in_stride = in_stride;
    g.count = count;
    g.last_count = last_count;
    g.nranks = nranks;
    g.nchunks = nranks;
    return check_hip(dt::launch_reduce_scatter_grid(g, dtype, op, stream), what);
}

// Whether an AllReduce over element-aligned buffers that share no offset
// takes the two-shot form over line grids (the grid ReduceScatter into each
// output's own chunk, then the fan-out) rather than the element kernel: once
// its footprint, 2 * P * S bytes, has clearly left the 256 MB Infinity Cache.
// Graph replays, outputs 2 bytes off and inputs aligned (or the reverse),
// element kernel against the two-shot form: at P * S = 160 MiB, P=6 fp32
// 57-60 against 55-58 us, P=8 bf16 79-88 against 62 us, P=10 bf16 70-77
// against 64-70 us, P=12 bf16 76-82 against 75-81 us; but P=4 fp32 63-66
// against 66-68 us and P=16 fp32 67-68 against 67-73 us, which only break
// even from 192-240 MiB; at P * S = 128 MiB the element kernel wins at every
// rank count measured (P=8 bf16 47 against 52-54 us, P=16 fp32 43 against
// 54-61 us).
bool grid_two_shot_pays(int nranks, uint64_t bytes_per_rank) {
    const uint64_t ps = uint64_t(nranks) * bytes_per_rank;
    if (nranks >= 6 && nranks <= 12) return ps >= (160ull << 20);
    return ps >= (256ull << 20);
}

dt_status allreduce_one(const void* const* send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                        dt_op op, hipStream_t stream) {
    dt::ReduceArgs a = {};
    bool vec = true, lines = true;
    for (int r = 0; r < nranks; r++) {
        a.src[r] = send[r];
        a.dst[r] = recv[r];
        vec = vec && aligned16(send[r]) && aligned16(recv[r]);
        lines = lines && line_aligned(send[r]);
    }
    a.nranks = nranks;
    a.rs = 0;
    const size_t v = vec_elems(dtype);
    const size_t es = esize_of(dtype);
    // Vector-aligned inputs off their lines: where the two-shot form runs
    // past the Infinity Cache, its ReduceScatter goes over the line grid,
    // which loads whole input lines (P=8 bf16 128 MiB per rank, inputs 16
    // bytes off: 364 -> 343 us, in-process A/B).
    const bool grid_first = vec && !lines && nranks > 1 && two_shot_pays(nranks, uint64_t(count) * es) &&
                            grid_two_shot_pays(nranks, uint64_t(count) * es);
    // Two-shot chunks are whole multiples of kChunkVecs vectors (1 KiB, the
    // ReduceScatter tile), all but the last, which takes the rest: every
    // chunk then starts on a cache-line boundary at any rank count, so no
    // line of an output is written by two workgroups.  Equal chunks of
    // count / P elements (the earlier cut) put the chunk starts of P = 5-15
    // off the lines, and the two-shot form then ran 15-80% slower than the
    // one-shot kernel at most sizes (in-process A/B, P = 5-7, 9, 10, 12, 15).
    constexpr uint64_t kChunkVecs = 64;
    const uint64_t nv = count / v;
    const uint64_t per = (nv + nranks - 1) / nranks;                      // vectors per chunk, rounded up
    const uint64_t mc = (per + kChunkVecs - 1) / kChunkVecs * kChunkVecs;  // ... to whole tiles
    if (vec && !grid_first && mc * uint64_t(nranks - 1) < nv && two_shot_pays(nranks, uint64_t(count) * es)) {
        const uint64_t last = nv - mc * uint64_t(nranks - 1);  // 0 < last <= mc
        const uint64_t cb = mc * 16;                           // chunk stride in bytes
        dt::ReduceArgs rs = a;
        const void* own[dt::kMaxRanksHost];
        size_t counts[dt::kMaxRanksHost];
        void* table[dt::kMaxRanksHost * dt::kMaxRanksHost];
        for (int r = 0; r < nranks; r++) {
            rs.dst[r] = static_cast<char*>(recv[r]) + r * cb;
            own[r] = rs.dst[r];
            counts[r] = size_t((r + 1 < nranks ? mc : last) * v);
            for (int q = 0; q < nranks; q++) table[size_t(r) * nranks + q] = static_cast<char*>(recv[q]) + r * cb;
        }
        rs.rs = 1;
        rs.first = 0;
        rs.count = mc;
        rs.last_count = last;
        rs.chunk_stride = mc;
        rs.chunk_elems = size_t(mc * v);
        dt_status st = check_hip(dt::launch_reduce_vec(rs, dtype, op, stream), "allreduce (reduce_scatter) launch");
        if (st != DT_OK) return st;
        if ((st = fan_out(own, counts, table, nranks, es, stream, "allreduce (all_gather) launch")) != DT_OK) return st;
        if (nv * v == count) return DT_OK;
        a.first = size_t(nv * v);  // the ragged end, fewer than one vector per rank: element path
        a.count = count - a.first;
        return check_hip(dt::launch_reduce_elems(a, dtype, op, stream), "allreduce (element path) launch");
    }
    if ((!vec || grid_first) && nranks > 1 && grid_two_shot_pays(nranks, uint64_t(count) * es)) {
        bool el = true;
        for (int r = 0; r < nranks; r++) el = el && elem_aligned(send[r], es) && elem_aligned(recv[r], es);
        // chunks of whole 1 KiB of elements, all but the last, as above
        const size_t te = size_t(dt::kGridChunkGrain) / es;
        const size_t mce = ((count + nranks - 1) / nranks + te - 1) / te * te;
        if (el && mce * size_t(nranks - 1) < count) {
            const size_t last = count - mce * size_t(nranks - 1);
            void* own[dt::kMaxRanksHost];
            size_t counts[dt::kMaxRanksHost];
            void* table[dt::kMaxRanksHost * dt::kMaxRanksHost];
            for (int r = 0; r < nranks; r++) {
                own[r] = static_cast<char*>(recv[r]) + r * mce * es;
                counts[r] = r + 1 < nranks ? mce : last;
                for (int q = 0; q < nranks; q++) table[size_t(r) * nranks + q] = static_cast<char*>(recv[q]) + r * mce * es;
            }
            dt_status st = reduce_scatter_grid(send, own, nranks, mce, mce, last, dtype, op, stream,
                                               "allreduce (grid reduce_scatter) launch");
            if (st != DT_OK) return st;
            return fan_out(own, counts, table, nranks, es, stream, "allreduce (all_gather) launch");
        }
    }
    // The one-shot vector kernel stores whole 16-byte vectors to every output;
    // outputs 16, 32 or 48 bytes into a 64-byte half line make each wave's
    // stores split lines unevenly, and the element kernel is faster there
    // (graph replays, outputs 16 bytes off: P=8 bf16 256 KiB / 1 / 16 MiB per
    // rank 4.4 / 5.5 / 51.4 -> 2.6 / 4.2 / 45.8 us, P=16 fp32 256 KiB / 1 / 4
    // MiB 5.9 / 8.1 / 27.3 -> 2.9 / 6.2 / 23.0 us, P=4 fp32 4 / 16 MiB 6.5 /
    // 24.5 -> 5.9 / 21.8 us; at 64 bytes off the two are even).
    bool halves = true;
    for (int r = 0; r < nranks; r++) halves = halves && (reinterpret_cast<uintptr_t>(recv[r]) & 63u) == 0;
    size_t body = 0;
    if (vec && halves) {
        a.first = 0;
        a.count = count / v;
        body = a.count * v;
        if (a.count) {
            dt_status st = check_hip(dt::launch_reduce_vec(a, dtype, op, stream), "allreduce launch");
            if (st != DT_OK) return st;
        }
    }
    if (body < count) {
        a.first = body;
        a.count = count - body;
        return check_hip(dt::launch_reduce_elems(a, dtype, op, stream), "allreduce (element path) launch");
    }
    return DT_OK;
}

// Bytes to peel off the front of every send and recv buffer of a fold whose
// buffers are not 128-byte aligned, so that the vector kernels' tiles start
// on an alignment boundary: the largest grain of 4096, 1024 or 128 bytes at
// which every buffer shares one offset and `stride` (the bytes between the
// starts of the ranges one launch folds, e.g. ReduceScatter chunks; 0 for
// none) keeps it; failing that, the bytes up to the next 16-byte boundary
// when every buffer shares its offset within a vector.  0 when none of these
// applies or the buffers are line-aligned already, except that with
// `to_tile`, line-aligned buffers that share a nonzero offset within 1 KiB
// (the fold kernels' tile) peel up to the next 1 KiB boundary.  Tiles that
// straddle 1 KiB boundaries cost the two-shot AllReduce 4-6% (P=8 bf16 at
// 128 MiB per rank, in-process A/B: buffers at 128 to 512 bytes past a
// 1 KiB boundary 0.753-0.761 of peak, at 0, 1 or 2 KiB 0.799-0.805); the
// 1 KiB peel wins that back less its element launch (0.781-0.785), but
// costs the one-shot kernel 1-4%.
size_t peel_bytes(const void* const* send, void* const* recv, int nranks, size_t stride, bool to_tile = false) {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(send[0]);
    auto shared = [&](uintptr_t grain) {
        if (stride % grain != 0) return false;
        for (int r = 0; r < nranks; r++)
            if ((reinterpret_cast<uintptr_t>(send[r]) & (grain - 1)) != (s0 & (grain - 1)) ||
                (reinterpret_cast<uintptr_t>(recv[r]) & (grain - 1)) != (s0 & (grain - 1)))
                return false;
        return true;
    };
    if (shared(128) && (s0 & 127) == 0)
        return to_tile && shared(1024) && (s0 & 1023) != 0 ? size_t(1024 - (s0 & 1023)) : 0;
    for (const uintptr_t grain : {uintptr_t(4096), uintptr_t(1024), uintptr_t(128)})
        if (shared(grain)) return size_t(grain - (s0 & (grain - 1)));
    if (shared(16) && (s0 & 15) != 0) return size_t(16 - (s0 & 15));
    return 0;
}

dt_status allreduce_windows(const void* const* send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                            dt_op op, hipStream_t stream);

// Validated AllReduce over one contiguous range per rank.  When every buffer
// sits at the same offset past an alignment boundary (peel_bytes), the whole
// vectors from that boundary on take the vector path (allreduce_windows) and
// the elements before it, with the ragged end, one element launch.
dt_status allreduce_impl(const void* const* send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                         dt_op op, hipStream_t stream) {
    const size_t es = esize_of(dtype), v = vec_elems(dtype);
    const uint64_t bytes = uint64_t(count) * es;
    const bool two_shot = two_shot_pays(nranks, bytes) || allreduce_window(nranks, bytes) != 0;
    const size_t peel = peel_bytes(send, recv, nranks, 0, two_shot);
    if (peel != 0) {
        const size_t h = peel / es;  // a whole number of elements for element-aligned buffers
        if (count > h && peel % es == 0) {
            // the whole vectors after the head on the vector path; the head
            // and the ragged end together in one element launch (each
            // extra launch here cost 2-3% of the AllReduce at 128 MiB)
            const size_t body = (count - h) / v * v;
            const void* s[dt::kMaxRanksHost];
            void* d[dt::kMaxRanksHost];
            dt::ReduceArgs a = {};
            for (int r = 0; r < nranks; r++) {
                a.src[r] = send[r];
                a.dst[r] = recv[r];
                s[r] = cptr(send[r]) + h * es;
                d[r] = static_cast<char*>(recv[r]) + h * es;
            }
            if (body != 0) {
                const dt_status st = allreduce_windows(s, d, nranks, body, dtype, op, stream);
                if (st != DT_OK) return st;
            }
            a.nranks = nranks;
            a.first = 0;
            a.count = h;
            a.first2 = h + body;
            a.count2 = count - h - body;
            return check_hip(dt::launch_reduce_elems(a, dtype, op, stream), "allreduce (head and tail) launch");
        }
    }
    return allreduce_windows(send, recv, nranks, count, dtype, op, stream);
}

// The AllReduce of buffers that need no peel: window by window where
// allreduce_window says so, else in one call.
dt_status allreduce_windows(const void* const* send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                            dt_op op, hipStream_t stream) {
    const size_t es = esize_of(dtype);
    const uint64_t win = allreduce_window(nranks, uint64_t(count) * es);
    if (win == 0) return allreduce_one(send, recv, nranks, count, dtype, op, stream);
    const size_t win_elems = size_t(win / es);  // whole vectors: every window keeps each buffer's alignment
    const void* s[dt::kMaxRanksHost];
    void* d[dt::kMaxRanksHost];
    for (size_t e0 = 0; e0 < count; e0 += win_elems) {
        const size_t n = std::min(win_elems, count - e0);
        for (int r = 0; r < nranks; r++) {
            s[r] = cptr(send[r]) + e0 * es;
            d[r] = static_cast<char*>(recv[r]) + e0 * es;
        }
        const dt_status st = allreduce_one(s, d, nranks, n, dtype, op, stream);
        if (st != DT_OK) return st;
    }
    return DT_OK;
}

// ReduceScatter of many independent segments, as few launches as the
// argument block allows.  seg_src[k][j] / seg_dst[k][j]: member j of segment k.
dt_status reduce_scatter_segments(const std::vector<std::vector<const void*>>& seg_src,
                                  const std::vector<std::vector<void*>>& seg_dst, const std::vector<size_t>& seg_m,
                                  int nranks, dt_dtype dtype, dt_op op, hipStream_t stream) {
    const size_t v = vec_elems(dtype);
    const uint64_t tile_elems = dt::seg_rs_tile_vecs(nranks) * v;
    const int per_launch = std::min(dt::kMaxSegs, dt::kSegPtrs / nranks);
    dt::SegReduceScatterArgs a = {};
    auto flush = [&]() -> dt_status {
        if (a.nsegs == 0) return DT_OK;
        dt_status st = check_hip(dt::launch_reduce_scatter_segs(a, dtype, op, stream), "segmented reduce_scatter");
        a = dt::SegReduceScatterArgs{};
        return st;
    };
    uint64_t tiles = 0;
    for (size_t k = 0; k < seg_m.size(); k++) {
        if (seg_m[k] == 0) continue;
        if (a.nsegs == per_launch) {
            dt_status st = flush();
            if (st != DT_OK) return st;
            tiles = 0;
        }
        const int i = a.nsegs++;
        a.nranks = nranks;
        bool al = seg_m[k] % v == 0;
        for (int j = 0; j < nranks; j++) {
            a.src[i * nranks + j] = seg_src[k][j];
            a.dst[i * nranks + j] = seg_dst[k][j];
            al = al && aligned16(seg_src[k][j]) && aligned16(seg_dst[k][j]);
        }
        if (al) a.aligned |= 1u << i;
        a.m[i] = seg_m[k];
        a.tiles_per_chunk[i] = uint32_t((seg_m[k] + tile_elems - 1) / tile_elems);
        a.tile_start[i] = uint32_t(tiles);
        tiles += uint64_t(a.tiles_per_chunk[i]) * nranks;
        if (tiles > 0x7FFFFFFFull) return fail(DT_ERR_ARG, "segmented reduce_scatter too large for one launch");
        a.tile_start[i + 1] = uint32_t(tiles);
    }
    return flush();
}

// Workgroups per fan-out source tile, as a power of two: each writes the
// destinations q with q mod 2^s equal to its part.  From 9 ranks on, two
// single-wave workgroups per tile, each with half the destinations: in-process
// A/B, P=16 fp32 AllGather 0.742 -> 0.815 of peak at 64 MiB and 0.818 ->
// 0.843 at 256 MiB per rank, P=12 0.782 -> 0.827, the P=16 two-shot
// AllReduce 0.749 -> 0.783 at 64 MiB and 0.748 -> 0.764 at 1 GiB; four
// workgroups lost to two everywhere, and splitting at P=8 cost 4-17%.
uint32_t gather_split_log2(int nranks) {
    return nranks >= 9 ? 1u : 0u;
}

// One fan-out launch over pieces k < n: piece k is bytes[k] at src[k], going to
// dst[k][q] for every q (host arrays, P entries each), in single-wave 1 KiB
// tiles (`wave`) or 128-thread 2 KiB ones; a read pass (`touch_first`, 2 KiB
// tiles only) goes first.
dt_status fan_out_launch(const void* const* src, const uint64_t* bytes, void* const* const* dst, int n,
                         int nranks, bool touch_first, bool wave, hipStream_t stream, const char* what) {
    dt::GatherArgs a = {};
    a.nranks = nranks;
    const uint64_t tile_bytes = wave ? dt::kGatherWaveTileBytes : dt::kGatherTileBytes;
    a.tile_bytes = uint32_t(tile_bytes);
    a.split_log2 = gather_split_log2(nranks);
    uint64_t tiles = 0;
    for (int k = 0; k < n; k++) {
        a.src[k] = src[k];
        a.bytes[k] = bytes[k];
        a.tile_start[k] = uint32_t(tiles);
        bool same = true;  // every destination at the same offset within a 128-byte line
        const uintptr_t md = bytes[k] ? reinterpret_cast<uintptr_t>(dst[k][0]) & (dt::kGridAlign - 1) : 0;
        for (int q = 0; q < nranks; q++) {
            void* d = bytes[k] ? dst[k][q] : nullptr;
            a.dst[k * nranks + q] = d;
            same = same && (reinterpret_cast<uintptr_t>(d) & (dt::kGridAlign - 1)) == md;
        }
        if (same && md == 0 && aligned16(src[k])) {  // every destination on a line: tiles follow the source
            a.aligned |= 1u << k;
            tiles += (bytes[k] + tile_bytes - 1) / tile_bytes;
        } else if (same) {  // tiles over the destinations' line grid
            a.shifted |= 1u << k;
            a.lead[k] = uint32_t(md) | uint32_t((reinterpret_cast<uintptr_t>(src[k]) - md) & 15u) << 16;
            tiles += dt::grid_tiles(bytes[k], md, tile_bytes);
        } else {  // each destination over its own line grid: tiles for the deepest lead
            tiles += bytes[k] ? dt::grid_tiles(bytes[k], dt::kGridAlign - 1, tile_bytes) : 0;
        }
        if ((tiles << a.split_log2) > 0x7FFFFFFFull) return fail(DT_ERR_ARG, "fan-out too large for one launch");
    }
    for (int k = n; k <= nranks; k++) a.tile_start[k] = uint32_t(tiles);
    if (tiles == 0) return DT_OK;
    dt_status st = DT_OK;
    if (touch_first && (st = check_hip(dt::launch_gather_touch(a, uint32_t(tiles), stream), what)) != DT_OK) return st;
    return check_hip(dt::launch_gather(a, uint32_t(tiles), stream), what);
}

// Fan-out of `nsources` pieces (default: nranks): piece r (counts[r]
// elements at src[r]) goes to table[r*nranks + q] for every q.  Sources up to
// kFanOutDirectBytes go in one launch.  Larger ones go window by window: a
// read pass pulls the window's source bytes into the Infinity Cache, then the
// window fans out reading from there, so HBM serves the window's reads and its
// writes in two separate phases instead of interleaved.
dt_status fan_out(const void* const* src, const size_t* counts, void* const* table, int nranks, size_t es,
                  hipStream_t stream, const char* what, int nsources) {
    if (nsources < 0) nsources = nranks;
    uint64_t total = 0;
    for (int r = 0; r < nsources; r++) total += uint64_t(counts[r]) * es;
    const void* wsrc[dt::kMaxRanksHost];
    uint64_t wbytes[dt::kMaxRanksHost];
    void* wdst[dt::kMaxRanksHost][dt::kMaxRanksHost];
    void* const* wdst_rows[dt::kMaxRanksHost];
    for (int k = 0; k < dt::kMaxRanksHost; k++) wdst_rows[k] = wdst[k];
    if (total <= dt::kFanOutDirectBytes) {
        for (int r = 0; r < nsources; r++) {
            wsrc[r] = src[r];
            wbytes[r] = uint64_t(counts[r]) * es;
            for (int q = 0; q < nranks; q++) wdst[r][q] = table[size_t(r) * nranks + q];
        }
        return fan_out_launch(wsrc, wbytes, wdst_rows, nsources, nranks, false, total <= dt::kGatherWaveBytes, stream,
                              what);
    }
    int n = 0;
    uint64_t fill = 0;
    dt_status st = DT_OK;
    for (int r = 0; r < nsources; r++) {
        const uint64_t bytes = uint64_t(counts[r]) * es;
        uint64_t off = 0;
        while (off < bytes) {
            uint64_t take = std::min(bytes - off, dt::kFanOutWindowBytes - fill);
            if (off + take < bytes) take &= ~uint64_t(15);  // cut inside a source on 16-byte boundaries
            if (take == 0) take = std::min<uint64_t>(bytes - off, 16);
            wsrc[n] = cptr(src[r]) + off;
            wbytes[n] = take;
            for (int q = 0; q < nranks; q++) wdst[n][q] = static_cast<char*>(table[size_t(r) * nranks + q]) + off;
            n++;
            off += take;
            fill += take;
            if (fill >= dt::kFanOutWindowBytes || n == nranks) {
                if ((st = fan_out_launch(wsrc, wbytes, wdst_rows, n, nranks, true, false, stream, what)) != DT_OK) return st;
                n = 0;
                fill = 0;
            }
        }
    }
    if (n > 0) return fan_out_launch(wsrc, wbytes, wdst_rows, n, nranks, true, false, stream, what);
    return DT_OK;
}

// Independent 1:1 byte copies, in as few launches as the argument block allows.
dt_status copy_segments(const std::vector<const void*>& src, const std::vector<void*>& dst,
                        const std::vector<size_t>& bytes, hipStream_t stream, const char* what) {
    dt::SegCopyArgs a = {};
    uint64_t tiles = 0;
    auto flush = [&]() -> dt_status {
        if (a.nsegs == 0) return DT_OK;
        a.tile_start[a.nsegs] = uint32_t(tiles);
        dt_status st = check_hip(dt::launch_copy_segments(a, stream), what);
        a = dt::SegCopyArgs{};
        tiles = 0;
        return st;
    };
    for (size_t k = 0; k < src.size(); k++) {
        if (bytes[k] == 0) continue;
        if (a.nsegs == dt::kMaxCopySegs) {
            dt_status st = flush();
            if (st != DT_OK) return st;
        }
        const int i = a.nsegs++;
        a.src[i] = src[k];
        a.dst[i] = dst[k];
        a.bytes[i] = bytes[k];
        a.tile_start[i] = uint32_t(tiles);
        if (aligned16(src[k]) && line_aligned(dst[k])) {
            a.aligned |= 1ull << i;
            tiles += (bytes[k] + dt::kSegCopyTileBytes - 1) / dt::kSegCopyTileBytes;
        } else {  // tiles over the destination's line grid
            tiles += dt::grid_tiles(bytes[k], reinterpret_cast<uintptr_t>(dst[k]) & (dt::kGridAlign - 1),
                                    dt::kSegCopyTileBytes);
        }
        if (tiles > 0x7FFFFFFFull) return fail(DT_ERR_ARG, "copy too large for one launch");
    }
    return flush();
}

// ------------------------------------------------------------ piece lists --
// One contiguous part of a tensor on every rank: ptr[r] is rank r's start.
struct PieceRef {
    void* ptr[DT_MAX_RANKS];
    size_t len;   // elements
    size_t wpos;  // element position inside the bucket buffer (staging only)
};

void set_aligned(dt::PieceArgs& a, int k) { a.aligned |= 1u << k; }
void set_aligned(dt::CoalescedArgs& a, int k) { a.aligned[k >> 5] |= 1u << (k & 31); }

// Fill a piece table with pieces [first, first + n).
template <typename Args>
dt_status fill_pieces(Args& a, const std::vector<PieceRef>& pieces, size_t first, int n, int nranks, size_t es,
                      void* const* ws) {
    a.nranks = nranks;
    a.npieces = n;
    uint64_t tiles = 0;
    for (int k = 0; k < n; k++) {
        const PieceRef& p = pieces[first + k];
        bool al = true;
        for (int r = 0; r < nranks; r++) {
            a.ptr[k * nranks + r] = p.ptr[r];
            al = al && aligned16(p.ptr[r]);
        }
        if (ws) {
            for (int r = 0; r < nranks; r++) al = al && aligned16(ws[r]);
            al = al && (p.wpos * es) % 16 == 0;
        }
        if (al) set_aligned(a, k);
        a.len[k] = p.len;
        a.wpos[k] = p.wpos;
        a.tile_start[k] = uint32_t(tiles);
        tiles += (p.len * es + dt::kPieceTileVecs * 16 - 1) / (dt::kPieceTileVecs * 16);
        if (tiles > 0x7FFFFFFFull) return fail(DT_ERR_ARG, "piece table too large for one launch");
    }
    a.tile_start[n] = uint32_t(tiles);
    if (ws)
        for (int r = 0; r < nranks; r++) a.ws[r] = ws[r];
    return DT_OK;
}

// What to do with a piece list: fold in place, or copy to / from the bucket
// buffers.
enum PieceAction { kFold, kFlatten, kUnflatten };

// Run `action` over all pieces in as few launches as the tables allow: the
// small table (3.3 KiB of kernel arguments) when the list fits in one, the
// large one (about 43 KiB) otherwise.
dt_status run_pieces(const std::vector<PieceRef>& pieces, int nranks, dt_dtype dtype, dt_op op, void* const* ws,
                     PieceAction action, hipStream_t stream) {
    const size_t es = esize_of(dtype);
    const int small_cap = std::min(dt::kMaxPieces, dt::kPiecePtrs / nranks);
    const int large_cap = std::min(dt::kCoalMaxPieces, dt::kCoalPtrs / nranks);
    dt_status st = DT_OK;
    if (pieces.size() <= size_t(small_cap)) {
        dt::PieceArgs a = {};
        if ((st = fill_pieces(a, pieces, 0, int(pieces.size()), nranks, es, ws)) != DT_OK) return st;
        if (action == kFold) return check_hip(dt::launch_reduce_pieces(a, dtype, op, stream), "piece reduce launch");
        return check_hip(dt::launch_copy_pieces(a, int(es), action == kFlatten, stream), "piece copy launch");
    }
    std::unique_ptr<dt::CoalescedArgs> a(new dt::CoalescedArgs());  // too large for a thread's stack
    for (size_t first = 0; first < pieces.size(); first += large_cap) {
        std::memset(a.get(), 0, sizeof(dt::CoalescedArgs));
        const int n = int(std::min<size_t>(large_cap, pieces.size() - first));
        if ((st = fill_pieces(*a, pieces, first, n, nranks, es, ws)) != DT_OK) return st;
        if (action == kFold)
            st = check_hip(dt::launch_reduce_coalesced(*a, dtype, op, stream), "coalesced reduce launch");
        else
            st = check_hip(dt::launch_copy_coalesced(*a, int(es), action == kFlatten, stream), "coalesced copy launch");
        if (st != DT_OK) return st;
    }
    return DT_OK;
}

// ---------------------------------------------------------- bucket plan --
struct Piece {
    int tensor;
    int bucket;
    size_t offset, length, bucket_pos;
};

std::vector<Piece> plan_buckets(const size_t* numels, int ntensors, size_t per_bucket, size_t* nbuckets) {
    std::vector<Piece> out;
    size_t pos = 0;  // position in the flattened concatenation
    for (int t = 0; t < ntensors; t++) {
        size_t off = 0;
        while (off < numels[t]) {
            const size_t bucket = pos / per_bucket;
            const size_t in_bucket = pos - bucket * per_bucket;
            const size_t len = std::min(numels[t] - off, per_bucket - in_bucket);
            out.push_back(Piece{t, int(bucket), off, len, in_bucket});
            off += len;
            pos += len;
        }
    }
    *nbuckets = (pos + per_bucket - 1) / per_bucket;
    return out;
}

}  // namespace

extern "C" {

const char* dt_status_string(dt_status st) {
    switch (st) {
        case DT_OK: return "DT_OK";
        case DT_ERR_ARG: return "DT_ERR_ARG: invalid argument";
        case DT_ERR_UNSUPPORTED: return "DT_ERR_UNSUPPORTED: unsupported dtype/op combination";
        case DT_ERR_HIP: return "DT_ERR_HIP: HIP runtime error";
        case DT_ERR_TIMEOUT: return "DT_ERR_TIMEOUT: barrier wait exceeded its budget";
    }
    return "unknown dt_status";
}

const char* dt_last_error(void) { return g_last_error.c_str(); }

const char* dt_version(void) { return "dtcoll 0.1 (gfx950)"; }

dt_status dt_allreduce(const void* const* send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                       dt_op op, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype) || !valid_op(op)) return fail(DT_ERR_ARG, "bad dtype %d or op %d", dtype, op);
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    if (count == 0) return DT_OK;  // empty buffers may carry NULL pointers
    if ((st = check_ptr_array(send, nranks, "send")) != DT_OK) return st;
    if ((st = check_ptr_array(recv, nranks, "recv")) != DT_OK) return st;
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < nranks; r++) {
            if (r != q && recv[q] == send[r])
                return fail(DT_ERR_ARG, "recv[%d] aliases send[%d]; only in place (recv[r] == send[r]) is allowed", q,
                            r);
            if (r != q && recv[q] == recv[r]) return fail(DT_ERR_ARG, "recv[%d] equals recv[%d]", q, r);
        }
    {
        const size_t bytes = count * esize_of(dtype);
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            add_span(w, recv[r], bytes, "recv", r);
            add_span(rd, send[r], bytes, "send", r);
        }
        if ((st = check_disjoint(w, rd, "allreduce")) != DT_OK) return st;
    }
    return allreduce_impl(send, recv, nranks, count, dtype, op, stream);
}

dt_status dt_reduce_scatter(const void* const* send, void* const* recv, int nranks, size_t recvcount,
                            dt_dtype dtype, dt_op op, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype) || !valid_op(op)) return fail(DT_ERR_ARG, "bad dtype %d or op %d", dtype, op);
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    if (recvcount == 0) return DT_OK;  // empty buffers may carry NULL pointers
    if ((st = check_ptr_array(send, nranks, "send")) != DT_OK) return st;
    if ((st = check_ptr_array(recv, nranks, "recv")) != DT_OK) return st;
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < nranks; r++) {
            if (recv[q] == send[r]) return fail(DT_ERR_ARG, "recv[%d] aliases send[%d]", q, r);
            if (r != q && recv[q] == recv[r]) return fail(DT_ERR_ARG, "recv[%d] equals recv[%d]", q, r);
        }
    {
        const size_t es = esize_of(dtype);
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            add_span(w, recv[r], recvcount * es, "recv", r);
            add_span(rd, send[r], size_t(nranks) * recvcount * es, "send", r);
        }
        if ((st = check_disjoint(w, rd, "reduce_scatter")) != DT_OK) return st;
    }
    dt::ReduceArgs a = {};
    // The vector kernel where every chunk of every input starts on a line;
    // inputs off their lines take the line grid, which loads whole input
    // lines (P=8 bf16 128 MiB per rank, inputs 16 bytes off: 208 -> 191 us,
    // in-process A/B).  Outputs off their lines cost the vector kernel
    // nothing measurable.
    bool vec = recvcount % vec_elems(dtype) == 0 && (recvcount * esize_of(dtype)) % dt::kGridAlign == 0;
    for (int r = 0; r < nranks; r++) {
        a.src[r] = send[r];
        a.dst[r] = recv[r];
        vec = vec && aligned16(send[r]) && aligned16(recv[r]) && line_aligned(send[r]);
    }
    a.nranks = nranks;
    a.rs = 1;
    a.chunk_elems = recvcount;
    if (vec) {
        a.first = 0;
        a.count = a.last_count = a.chunk_stride = recvcount / vec_elems(dtype);
        return check_hip(dt::launch_reduce_vec(a, dtype, op, stream), "reduce_scatter launch");
    }
    // Every buffer and chunk start at the same offset within a line (or a
    // vector): the first h elements of each chunk go to the element path, the
    // aligned body of every chunk to the vector kernel, the ragged end back
    // to the element path.
    const size_t es = esize_of(dtype), v = vec_elems(dtype);
    const size_t peel = peel_bytes(send, recv, nranks, recvcount * es);
    const size_t h = peel / es;
    if (peel != 0 && peel % es == 0 && recvcount >= h + v) {
        dt::ReduceArgs body = a;
        for (int r = 0; r < nranks; r++) {
            body.src[r] = cptr(send[r]) + h * es;
            body.dst[r] = static_cast<char*>(recv[r]) + h * es;
        }
        body.count = body.last_count = (recvcount - h) / v;
        body.chunk_stride = recvcount / v;
        if ((st = check_hip(dt::launch_reduce_vec(body, dtype, op, stream), "reduce_scatter (body) launch")) != DT_OK)
            return st;
        a.first = 0;  // the head and the ragged end of every chunk, one launch
        a.count = h;
        a.first2 = h + body.count * v;
        a.count2 = recvcount - a.first2;
        return check_hip(dt::launch_reduce_elems(a, dtype, op, stream), "reduce_scatter (head and tail) launch");
    }
    bool el = true;  // element-aligned buffers at offsets of their own: the line-grid kernel
    for (int r = 0; r < nranks; r++) el = el && elem_aligned(send[r], es) && elem_aligned(recv[r], es);
    if (el)
        return reduce_scatter_grid(send, recv, nranks, recvcount, recvcount, recvcount, dtype, op, stream,
                                   "reduce_scatter (grid) launch");
    a.first = 0;
    a.count = recvcount;
    return check_hip(dt::launch_reduce_elems(a, dtype, op, stream), "reduce_scatter (element path) launch");
}

dt_status dt_all_gather(const void* const* send, void* const* recv, int nranks, const size_t* sendcounts,
                        size_t equal_count, dt_dtype dtype, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype)) return fail(DT_ERR_ARG, "bad dtype %d", dtype);
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    const size_t es = esize_of(dtype);
    std::vector<size_t> counts(nranks);
    size_t total = 0;
    for (int r = 0; r < nranks; r++) {
        counts[r] = sendcounts ? sendcounts[r] : equal_count;
        if (counts[r] > (size_t(1) << 40)) return fail(DT_ERR_ARG, "sendcount[%d]=%zu too large", r, counts[r]);
        if (counts[r] > 0 && send[r] == nullptr) return fail(DT_ERR_ARG, "send[%d] is NULL", r);
        total += counts[r];
    }
    if (total == 0) return DT_OK;  // nothing to gather; empty buffers may be NULL
    if ((st = check_ptr_array(recv, nranks, "recv")) != DT_OK) return st;
    // in place (NCCL-style) is send[r] == recv[r] + offset[r]; any other alias is refused
    size_t off = 0;
    std::vector<size_t> offset(nranks);
    for (int r = 0; r < nranks; r++) {
        offset[r] = off;
        off += counts[r] * es;
    }
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < nranks; r++) {
            if (counts[r] && cptr(send[r]) >= cptr(recv[q]) && cptr(send[r]) < cptr(recv[q]) + off &&
                !(q == r && cptr(send[r]) == cptr(recv[r]) + offset[r]))
                return fail(DT_ERR_ARG, "send[%d] lies inside recv[%d] other than at its own slot", r, q);
            if (r != q && recv[q] == recv[r]) return fail(DT_ERR_ARG, "recv[%d] equals recv[%d]", q, r);
        }
    {
        // a piece already in its own slot of its own output (in place) is not
        // copied: it is read only, and only its own slot holds it
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            add_span(w, recv[r], off, "recv", r);
            if (cptr(send[r]) != cptr(recv[r]) + offset[r]) add_span(rd, send[r], counts[r] * es, "send", r);
        }
        if ((st = check_disjoint(w, rd, "all_gather")) != DT_OK) return st;
    }
    std::vector<void*> table(size_t(nranks) * nranks);
    for (int r = 0; r < nranks; r++)
        for (int q = 0; q < nranks; q++) table[size_t(r) * nranks + q] = static_cast<char*>(recv[q]) + offset[r];
    return fan_out(send, counts.data(), table.data(), nranks, es, stream, "all_gather launch");
}

dt_status dt_all_gather_into_vec(const void* const* send, void* const* recv, int nranks, const size_t* sendcounts,
                                 size_t equal_count, dt_dtype dtype, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype)) return fail(DT_ERR_ARG, "bad dtype %d", dtype);
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    const size_t es = esize_of(dtype);
    std::vector<size_t> counts(nranks);
    std::vector<void*> table(size_t(nranks) * nranks);
    for (int r = 0; r < nranks; r++) {
        counts[r] = sendcounts ? sendcounts[r] : equal_count;
        if (counts[r] > (size_t(1) << 40)) return fail(DT_ERR_ARG, "sendcount[%d]=%zu too large", r, counts[r]);
        if (counts[r] == 0) continue;  // empty pieces may carry NULL pointers
        if (send[r] == nullptr) return fail(DT_ERR_ARG, "send[%d] is NULL", r);
        for (int q = 0; q < nranks; q++) {
            void* d = recv[size_t(q) * nranks + r];
            if (d == nullptr) return fail(DT_ERR_ARG, "recv[%d] (rank %d's copy of rank %d) is NULL", q * nranks + r, q, r);
            if (d == send[r]) return fail(DT_ERR_ARG, "recv[%d] aliases send[%d]", q * nranks + r, r);
            table[size_t(r) * nranks + q] = d;
        }
    }
    {
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            if (counts[r] == 0) continue;
            add_span(rd, send[r], counts[r] * es, "send", r);
            for (int q = 0; q < nranks; q++) add_span(w, recv[size_t(q) * nranks + r], counts[r] * es, "recv", q * nranks + r);
        }
        if ((st = check_disjoint(w, rd, "all_gather_into_vec")) != DT_OK) return st;
    }
    return fan_out(send, counts.data(), table.data(), nranks, es, stream, "all_gather_into_vec launch");
}

dt_status dt_broadcast(const void* root_send, void* const* recv, int nranks, size_t count, dt_dtype dtype,
                       hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype)) return fail(DT_ERR_ARG, "bad dtype %d", dtype);
    if (recv == nullptr) return fail(DT_ERR_ARG, "recv array is NULL");
    if (count == 0) return DT_OK;
    if (count > (size_t(1) << 40)) return fail(DT_ERR_ARG, "count=%zu too large", count);
    if (root_send == nullptr) return fail(DT_ERR_ARG, "root_send is NULL");
    if ((st = check_ptr_array(recv, nranks, "recv")) != DT_OK) return st;
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < q; r++)
            if (recv[q] == recv[r]) return fail(DT_ERR_ARG, "recv[%d] equals recv[%d]", q, r);
    {
        // the root's buffer may be one of the outputs (it is then not copied onto itself)
        std::vector<Span> w, rd;
        for (int q = 0; q < nranks; q++) add_span(w, recv[q], count * esize_of(dtype), "recv", q);
        add_span(rd, root_send, count * esize_of(dtype), "root_send", 0);
        if ((st = check_disjoint(w, rd, "broadcast")) != DT_OK) return st;
    }
    // the fan-out engine with one source: rank slot 0 carries the root's data
    const void* src[1] = {root_send};
    size_t counts[1] = {count};
    return fan_out(src, counts, recv, nranks, esize_of(dtype), stream, "broadcast launch", /*nsources=*/1);
}

dt_status dt_replicate_to_shard(const void* const* send, void* const* recv, int nranks, size_t recvcount,
                                dt_dtype dtype, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype)) return fail(DT_ERR_ARG, "bad dtype %d", dtype);
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    if (recvcount == 0) return DT_OK;
    if ((st = check_ptr_array(send, nranks, "send")) != DT_OK) return st;
    if ((st = check_ptr_array(recv, nranks, "recv")) != DT_OK) return st;
    const size_t es = esize_of(dtype);
    std::vector<const void*> src(nranks);
    std::vector<void*> dst(nranks);
    std::vector<size_t> bytes(nranks, recvcount * es);
    std::vector<Span> w, rd;
    for (int r = 0; r < nranks; r++) {
        src[r] = cptr(send[r]) + size_t(r) * recvcount * es;
        dst[r] = recv[r];
        add_span(w, recv[r], recvcount * es, "recv", r);
        add_span(rd, src[r], recvcount * es, "send slice", r);
    }
    // only slice r of send[r] is read (an output that is exactly its own slice copies onto itself)
    if ((st = check_disjoint(w, rd, "replicate_to_shard")) != DT_OK) return st;
    return copy_segments(src, dst, bytes, stream, "replicate_to_shard launch");
}

dt_status dt_all_to_all_dims(const void* const* send, void* const* recv, int nranks, size_t rows, size_t cols,
                             int src_dim, int dst_dim, dt_dtype dtype, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype)) return fail(DT_ERR_ARG, "bad dtype %d", dtype);
    if (src_dim < 0 || src_dim > 1 || dst_dim < 0 || dst_dim > 1)
        return fail(DT_ERR_ARG, "src_dim %d / dst_dim %d must be 0 or 1", src_dim, dst_dim);
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    const size_t P = size_t(nranks);
    if ((src_dim == 0 || dst_dim == 0) && rows % P != 0) return fail(DT_ERR_ARG, "rows=%zu not divisible by %d", rows, nranks);
    if ((src_dim == 1 || dst_dim == 1) && cols % P != 0) return fail(DT_ERR_ARG, "cols=%zu not divisible by %d", cols, nranks);
    if (rows == 0 || cols == 0) return DT_OK;
    if (rows > (size_t(1) << 31) || cols > (size_t(1) << 31)) return fail(DT_ERR_ARG, "tensor too large");
    if ((st = check_ptr_array(send, nranks, "send")) != DT_OK) return st;
    if ((st = check_ptr_array(recv, nranks, "recv")) != DT_OK) return st;
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < nranks; r++)
            if (recv[q] == send[r]) return fail(DT_ERR_ARG, "recv[%d] aliases send[%d]", q, r);
    const size_t es = esize_of(dtype);
    {
        const size_t sblock = (src_dim == 0 ? rows / P * cols : rows * (cols / P)) * es;
        const size_t dblock = (dst_dim == 0 ? rows / P * cols : rows * (cols / P)) * es;
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            add_span(w, recv[r], dblock, "recv", r);
            add_span(rd, send[r], sblock, "send", r);
        }
        if ((st = check_disjoint(w, rd, "all_to_all_dims")) != DT_OK) return st;
    }
    if (src_dim == dst_dim) {  // no exchange: each rank copies its own block
        const size_t block = (src_dim == 0 ? rows / P * cols : rows * (cols / P)) * es;
        std::vector<const void*> src(send, send + nranks);
        std::vector<void*> dst(recv, recv + nranks);
        std::vector<size_t> bytes(nranks, block);
        return copy_segments(src, dst, bytes, stream, "all_to_all_dims copy launch");
    }
    dt::DimsArgs a = {};
    bool vec = true, el = true;
    for (int r = 0; r < nranks; r++) {
        a.src[r] = send[r];
        a.dst[r] = recv[r];
        vec = vec && aligned16(send[r]) && aligned16(recv[r]);
        el = el && elem_aligned(send[r], es) && elem_aligned(recv[r], es);
    }
    a.rows = rows;
    a.cols = cols;
    a.rp = rows / P;
    a.cp = cols / P;
    a.esize = uint32_t(es);
    a.nranks = nranks;
    a.dir = src_dim == 0 ? 0 : 1;
    a.nruns = uint64_t(rows) * P;
    const uint64_t run_bytes = a.cp * es;
    a.vec = (vec && run_bytes % 16 == 0) ? 1u : 0u;
    a.elems = (!a.vec && el) ? 1u : 0u;
    uint64_t blocks;
    if (a.vec && run_bytes >= dt::kDimsWaveTileBytes) {
        a.wave = 1;
        a.tiles_per_run = uint32_t((run_bytes + dt::kDimsWaveTileBytes - 1) / dt::kDimsWaveTileBytes);
        a.runs_per_block = 1;
        blocks = a.nruns * a.tiles_per_run;
    } else if (run_bytes >= dt::kDimsTileBytes) {
        a.tiles_per_run = uint32_t((run_bytes + dt::kDimsTileBytes - 1) / dt::kDimsTileBytes);
        a.runs_per_block = 1;
        blocks = a.nruns * a.tiles_per_run;
    } else {
        a.tiles_per_run = 1;
        a.runs_per_block = uint32_t(std::min<uint64_t>(dt::kDimsMaxRunsPerBlock,
                                                        std::max<uint64_t>(1, dt::kDimsTileBytes / run_bytes)));
        blocks = (a.nruns + a.runs_per_block - 1) / a.runs_per_block;
    }
    if (blocks > 0x7FFFFFFFull) return fail(DT_ERR_ARG, "all_to_all_dims too large for one launch");
    return check_hip(dt::launch_all_to_all_dims(a, uint32_t(blocks), stream), "all_to_all_dims launch");
}

dt_status dt_all_to_all(const void* const* send, void* const* recv, int nranks, const size_t* splits,
                        dt_dtype dtype, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype)) return fail(DT_ERR_ARG, "bad dtype %d", dtype);
    if (splits == nullptr) return fail(DT_ERR_ARG, "splits is NULL");
    if (send == nullptr || recv == nullptr) return fail(DT_ERR_ARG, "send/recv array is NULL");
    // a rank that sends (receives) nothing may pass NULL for its input (output)
    std::vector<size_t> row(nranks, 0), col(nranks, 0);
    for (int i = 0; i < nranks; i++)
        for (int j = 0; j < nranks; j++) {
            row[i] += splits[i * nranks + j];
            col[j] += splits[i * nranks + j];
        }
    for (int r = 0; r < nranks; r++) {
        if (row[r] > 0 && send[r] == nullptr) return fail(DT_ERR_ARG, "send[%d] is NULL", r);
        if (col[r] > 0 && recv[r] == nullptr) return fail(DT_ERR_ARG, "recv[%d] is NULL", r);
    }
    for (int q = 0; q < nranks; q++)
        for (int r = 0; r < nranks; r++) {
            if (col[q] > 0 && row[r] > 0 && recv[q] == send[r])
                return fail(DT_ERR_ARG, "recv[%d] aliases send[%d]", q, r);
            if (r != q && col[q] > 0 && col[r] > 0 && recv[q] == recv[r])
                return fail(DT_ERR_ARG, "recv[%d] equals recv[%d]", q, r);
        }
    for (int s = 0; s < nranks * nranks; s++)
        if (splits[s] > (size_t(1) << 40)) return fail(DT_ERR_ARG, "splits[%d]=%zu too large", s, splits[s]);
    const size_t es = esize_of(dtype);
    {
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            add_span(w, recv[r], col[r] * es, "recv", r);
            add_span(rd, send[r], row[r] * es, "send", r);
        }
        if ((st = check_disjoint(w, rd, "all_to_all")) != DT_OK) return st;
    }
    dt::AllToAllArgs a = {};
    uint64_t tiles = 0;
    auto flush = [&]() -> dt_status {
        if (a.nblocks == 0) return DT_OK;
        a.tile_start[a.nblocks] = uint32_t(tiles);
        for (int k = a.nblocks + 1; k <= dt::kA2ABlocks; k++) a.tile_start[k] = UINT32_MAX;
        for (int g = 0; g < dt::kA2ABlocks / dt::kA2AGroup; g++) a.group_start[g] = a.tile_start[g * dt::kA2AGroup];
        const dt_status st = check_hip(dt::launch_all_to_all(a, uint32_t(tiles), stream), "all_to_all launch");
        a = dt::AllToAllArgs{};
        tiles = 0;
        return st;
    };
    // send offsets run along rows, receive offsets down columns
    std::vector<uint64_t> recv_off(nranks, 0);
    for (int i = 0; i < nranks; i++) {
        uint64_t so = 0;
        for (int j = 0; j < nranks; j++) {
            const uint64_t bytes = uint64_t(splits[i * nranks + j]) * es;
            if (bytes > 0) {
                const char* from = cptr(send[i]) + so;
                char* to = static_cast<char*>(recv[j]) + recv_off[j];
                const bool al = aligned16(from) && line_aligned(to);
                // other blocks' tiles cover their destination's line grid
                const uint64_t t = al ? (bytes + dt::kCopyTileBytes - 1) / dt::kCopyTileBytes
                                      : dt::grid_tiles(bytes, reinterpret_cast<uintptr_t>(to) & (dt::kGridAlign - 1),
                                                       dt::kCopyTileBytes);
                if (a.nblocks == dt::kA2ABlocks || tiles + t > 0x7FFFFFFFull) {
                    const dt_status st = flush();
                    if (st != DT_OK) return st;
                }
                const int k = a.nblocks++;
                a.from[k] = from;
                a.to[k] = to;
                a.bytes[k] = bytes;
                a.tile_start[k] = uint32_t(tiles);
                if (al) a.aligned[k >> 6] |= 1ull << (k & 63);
                tiles += t;
            }
            so += bytes;
            recv_off[j] += bytes;
        }
    }
    return flush();
}

dt_status dt_bucket_plan(const size_t* numels, int ntensors, size_t elem_size, size_t bucket_bytes, dt_piece* pieces,
                         size_t capacity, size_t* npieces, size_t* nbuckets) {
    g_last_error.clear();
    if (ntensors < 0 || (ntensors > 0 && numels == nullptr) || npieces == nullptr || nbuckets == nullptr)
        return fail(DT_ERR_ARG, "bad arguments to dt_bucket_plan");
    if (elem_size == 0 || bucket_bytes < elem_size) return fail(DT_ERR_ARG, "bucket_bytes smaller than one element");
    if (capacity > 0 && pieces == nullptr) return fail(DT_ERR_ARG, "pieces is NULL");
    size_t nb = 0;
    std::vector<Piece> plan = plan_buckets(numels, ntensors, bucket_bytes / elem_size, &nb);
    for (size_t i = 0; i < plan.size() && i < capacity; i++)
        pieces[i] = dt_piece{plan[i].tensor, plan[i].bucket, plan[i].offset, plan[i].length, plan[i].bucket_pos};
    *npieces = plan.size();
    *nbuckets = nb;
    return DT_OK;
}

// Tensors at least this large (bytes per rank) get an AllReduce of their own
// in the in-place bucket path.  Measured on the 32-layer data-parallel
// workload (32 and 86 MiB tensors, P=8 bf16, in-process): one AllReduce per
// tensor took 34.8 ms (35.4 ms with the one-shot kernel only) against 36.3
// ms for the multi-tensor fold of every piece.
constexpr size_t kOwnAllReduceBytes = size_t(16) << 20;

}  // extern "C"

namespace {

// Arguments shared by the bucket AllReduce entry points.  Every tensor is
// reduced in place, so no two of them (over all ranks) may overlap, and the
// bucket buffers, when given, may overlap neither the tensors nor each other.
dt_status bucket_check(void* const* grads, const size_t* numels, int ntensors, int nranks, size_t bucket_bytes,
                       void* const* bucket_ws, dt_dtype dtype, dt_op op) {
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype) || !valid_op(op)) return fail(DT_ERR_ARG, "bad dtype %d or op %d", dtype, op);
    if (ntensors < 0) return fail(DT_ERR_ARG, "ntensors=%d", ntensors);
    if (ntensors == 0) return DT_OK;
    if (numels == nullptr) return fail(DT_ERR_ARG, "numels is NULL");
    if (bucket_bytes == 0 || bucket_bytes % 16 != 0)
        return fail(DT_ERR_ARG, "bucket_bytes=%zu must be a positive multiple of 16", bucket_bytes);
    if (grads == nullptr) return fail(DT_ERR_ARG, "grads is NULL");
    for (int r = 0; r < nranks; r++)  // an empty tensor may carry a NULL pointer
        for (int t = 0; t < ntensors; t++)
            if (numels[t] > 0 && grads[size_t(r) * ntensors + t] == nullptr)
                return fail(DT_ERR_ARG, "grads[%d] (rank %d, tensor %d) is NULL", r * ntensors + t, r, t);
    if (bucket_ws && (st = check_ptr_array(bucket_ws, nranks, "bucket_ws")) != DT_OK) return st;
    const size_t es = esize_of(dtype);
    std::vector<Span> w;
    for (int r = 0; r < nranks; r++) {
        for (int t = 0; t < ntensors; t++) add_span(w, grads[size_t(r) * ntensors + t], numels[t] * es, "grads", r * ntensors + t);
        if (bucket_ws) add_span(w, bucket_ws[r], bucket_bytes, "bucket_ws", r);
    }
    return check_disjoint(w, {}, "bucket_allreduce");
}

// The bucket AllReduce after validation; bucket_ws is NULL (in place) or
// nranks buffers of bucket_bytes.
dt_status bucket_allreduce_impl(void* const* grads, const size_t* numels, int ntensors, int nranks, size_t bucket_bytes,
                                void* const* bucket_ws, dt_dtype dtype, dt_op op, hipStream_t stream) {
    dt_status st;
    const size_t es = esize_of(dtype);
    size_t nbuckets = 0;
    const std::vector<Piece> plan = plan_buckets(numels, ntensors, bucket_bytes / es, &nbuckets);
    auto piece_ref = [&](const Piece& p) {
        PieceRef ref = {};
        for (int r = 0; r < nranks; r++)
            ref.ptr[r] = static_cast<char*>(grads[size_t(r) * ntensors + p.tensor]) + p.offset * es;
        ref.len = p.length;
        ref.wpos = p.bucket_pos;
        return ref;
    };
    std::vector<PieceRef> pieces;
    if (!bucket_ws) {
        // Reduced in place, straight out of the tensors: each element's fold is
        // independent, so bucket boundaries do not matter here.  A tensor of at
        // least kOwnAllReduceBytes per rank is AllReduced on its own, as
        // dt_allreduce does it (the two-shot form where that is faster); the
        // pieces of all smaller tensors go out together, in as few launches as
        // the piece tables allow.
        auto own = [&](int t) { return numels[t] * es >= kOwnAllReduceBytes; };
        for (int t = 0; t < ntensors; t++) {
            if (!own(t)) continue;
            void* ptrs[DT_MAX_RANKS];
            for (int r = 0; r < nranks; r++) ptrs[r] = grads[size_t(r) * ntensors + t];
            if ((st = allreduce_impl(ptrs, ptrs, nranks, numels[t], dtype, op, stream)) != DT_OK) return st;
        }
        for (const Piece& p : plan)
            if (!own(p.tensor)) pieces.push_back(piece_ref(p));
        if (pieces.empty()) return DT_OK;
        return run_pieces(pieces, nranks, dtype, op, nullptr, kFold, stream);
    }
    size_t i = 0;
    while (i < plan.size()) {
        const int bucket = plan[i].bucket;
        size_t end = i;
        while (end < plan.size() && plan[end].bucket == bucket) end++;
        size_t bucket_len = 0;
        pieces.clear();
        for (size_t k = i; k < end; k++) {
            pieces.push_back(piece_ref(plan[k]));
            bucket_len = std::max(bucket_len, plan[k].bucket_pos + plan[k].length);
        }
        // the page's flatten -> AllReduce -> unflatten, bucket by bucket through the workspace
        if ((st = run_pieces(pieces, nranks, dtype, op, bucket_ws, kFlatten, stream)) != DT_OK) return st;
        if ((st = allreduce_impl(bucket_ws, bucket_ws, nranks, bucket_len, dtype, op, stream)) != DT_OK) return st;
        if ((st = run_pieces(pieces, nranks, dtype, op, bucket_ws, kUnflatten, stream)) != DT_OK) return st;
        i = end;
    }
    return DT_OK;
}

}  // namespace

extern "C" {

dt_status dt_bucket_allreduce(void* const* grads, const size_t* numels, int ntensors, int nranks, size_t bucket_bytes,
                              void* const* bucket_ws, dt_dtype dtype, dt_op op, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = bucket_check(grads, numels, ntensors, nranks, bucket_bytes, bucket_ws, dtype, op);
    if (st != DT_OK || ntensors == 0) return st;
    return bucket_allreduce_impl(grads, numels, ntensors, nranks, bucket_bytes, bucket_ws, dtype, op, stream);
}

dt_status dt_bucket_allreduce_noalloc(void* const* grads, const size_t* numels, int ntensors, int nranks,
                                      size_t bucket_bytes, dt_dtype dtype, dt_op op, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = bucket_check(grads, numels, ntensors, nranks, bucket_bytes, nullptr, dtype, op);
    if (st != DT_OK || ntensors == 0) return st;
    if (uint64_t(nranks) * bucket_bytes > dt::kScratchBytes)
        return fail(DT_ERR_ARG, "nranks * bucket_bytes = %d * %zu exceeds the %llu-byte static staging buffer", nranks,
                    bucket_bytes, (unsigned long long)dt::kScratchBytes);
    char* scratch = nullptr;
    if ((st = check_hip(dt::scratch_base(reinterpret_cast<void**>(&scratch)), "static staging buffer")) != DT_OK)
        return st;
    // rank r stages its buckets at scratch + r * bucket_bytes (16-byte aligned: bucket_bytes is a multiple of 16)
    void* ws[DT_MAX_RANKS];
    for (int r = 0; r < nranks; r++) ws[r] = scratch + size_t(r) * bucket_bytes;
    return bucket_allreduce_impl(grads, numels, ntensors, nranks, bucket_bytes, ws, dtype, op, stream);
}

dt_status dt_allreduce_coalesced(void* const* tensors, const size_t* numels, int ntensors, int nranks, dt_dtype dtype,
                                 dt_op op, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if (!valid_dtype(dtype) || !valid_op(op)) return fail(DT_ERR_ARG, "bad dtype %d or op %d", dtype, op);
    if (ntensors < 0) return fail(DT_ERR_ARG, "ntensors=%d", ntensors);
    if (ntensors == 0) return DT_OK;
    if (numels == nullptr || tensors == nullptr) return fail(DT_ERR_ARG, "tensors/numels is NULL");
    for (int r = 0; r < nranks; r++)
        for (int t = 0; t < ntensors; t++)
            if (numels[t] > 0 && tensors[size_t(r) * ntensors + t] == nullptr)
                return fail(DT_ERR_ARG, "tensors[%d] (rank %d, tensor %d) is NULL", r * ntensors + t, r, t);
    {
        // every tensor is reduced in place: no two may overlap
        std::vector<Span> w;
        for (int r = 0; r < nranks; r++)
            for (int t = 0; t < ntensors; t++)
                add_span(w, tensors[size_t(r) * ntensors + t], numels[t] * esize_of(dtype), "tensors", r * ntensors + t);
        if ((st = check_disjoint(w, {}, "allreduce_coalesced")) != DT_OK) return st;
    }
    std::vector<PieceRef> pieces;
    for (int t = 0; t < ntensors; t++) {
        if (numels[t] == 0) continue;
        PieceRef ref = {};
        for (int r = 0; r < nranks; r++) ref.ptr[r] = tensors[size_t(r) * ntensors + t];
        ref.len = numels[t];
        pieces.push_back(ref);
    }
    if (pieces.empty()) return DT_OK;
    return run_pieces(pieces, nranks, dtype, op, nullptr, kFold, stream);
}

dt_status dt_barrier(int32_t* const* windows, int nranks, int32_t first_generation, int32_t generations,
                     int32_t* status_dev, uint64_t timeout_ns, int layout, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if ((st = check_ptr_array(windows, nranks, "windows")) != DT_OK) return st;
    if (status_dev == nullptr) return fail(DT_ERR_ARG, "status_dev is NULL");
    if (first_generation < 1 || generations < 0 || int64_t(first_generation) + generations - 1 > INT32_MAX)
        return fail(DT_ERR_ARG, "generations %d..%d out of range", first_generation, first_generation + generations - 1);
    if (layout != DT_BARRIER_PACKED && layout != DT_BARRIER_SPREAD) return fail(DT_ERR_ARG, "bad layout %d", layout);
    if (generations == 0) return DT_OK;
    dt::BarrierArgs a = {};
    for (int r = 0; r < nranks; r++) a.win[r] = windows[r];
    a.status = status_dev;
    a.timeout_ticks = timeout_ticks(timeout_ns);
    a.nranks = nranks;
    a.first_generation = first_generation;
    a.generations = generations;
    return check_hip(dt::launch_barrier(a, layout == DT_BARRIER_SPREAD, stream), "barrier launch");
}

dt_status dt_barrier_exchange(const void* const* src, void* const* stage, void* const* dst, size_t nbytes,
                              int32_t* const* windows, int nranks, int32_t generation, int32_t* status_dev,
                              uint64_t timeout_ns, int layout, hipStream_t stream) {
    g_last_error.clear();
    dt_status st = check_ranks(nranks);
    if (st != DT_OK) return st;
    if ((st = check_ptr_array(windows, nranks, "windows")) != DT_OK) return st;
    if ((st = check_ptr_array(src, nranks, "src")) != DT_OK) return st;
    if ((st = check_ptr_array(stage, nranks, "stage")) != DT_OK) return st;
    if ((st = check_ptr_array(dst, nranks, "dst")) != DT_OK) return st;
    if (status_dev == nullptr) return fail(DT_ERR_ARG, "status_dev is NULL");
    if (generation < 1) return fail(DT_ERR_ARG, "generation %d must be >= 1", generation);
    if (layout != DT_BARRIER_PACKED && layout != DT_BARRIER_SPREAD) return fail(DT_ERR_ARG, "bad layout %d", layout);
    dt::ExchangeArgs a = {};
    for (int r = 0; r < nranks; r++) {
        a.bar.win[r] = windows[r];
        a.src[r] = src[r];
        a.stage[r] = stage[r];
        a.dst[r] = dst[r];
    }
    a.bar.status = status_dev;
    a.bar.timeout_ticks = timeout_ticks(timeout_ns);
    a.bar.nranks = nranks;
    a.bar.first_generation = generation;
    a.bar.generations = 1;
    a.nbytes = nbytes;
    return check_hip(dt::launch_exchange(a, layout == DT_BARRIER_SPREAD, stream), "barrier exchange launch");
}

// ------------------------------------------------------------ work handles --
struct dt_work {
    hipEvent_t start = nullptr;
    hipEvent_t end = nullptr;
};

dt_status dt_work_begin(hipStream_t producer, hipStream_t comm, dt_work** work) {
    g_last_error.clear();
    if (work == nullptr) return fail(DT_ERR_ARG, "work is NULL");
    dt_work* w = new dt_work();
    dt_status st = check_hip(hipEventCreateWithFlags(&w->start, hipEventDisableTiming), "hipEventCreate");
    if (st == DT_OK) st = check_hip(hipEventCreateWithFlags(&w->end, hipEventDisableTiming), "hipEventCreate");
    if (st == DT_OK) st = check_hip(hipEventRecord(w->start, producer), "hipEventRecord(producer)");
    if (st == DT_OK) st = check_hip(hipStreamWaitEvent(comm, w->start, 0), "hipStreamWaitEvent(comm)");
    if (st != DT_OK) {
        dt_work_free(w);
        return st;
    }
    *work = w;
    return DT_OK;
}

dt_status dt_work_end(dt_work* work, hipStream_t comm) {
    g_last_error.clear();
    if (work == nullptr) return fail(DT_ERR_ARG, "work is NULL");
    return check_hip(hipEventRecord(work->end, comm), "hipEventRecord(comm)");
}

dt_status dt_work_wait(dt_work* work, hipStream_t consumer) {
    g_last_error.clear();
    if (work == nullptr) return fail(DT_ERR_ARG, "work is NULL");
    return check_hip(hipStreamWaitEvent(consumer, work->end, 0), "hipStreamWaitEvent(consumer)");
}

int dt_work_query(dt_work* work) {
    if (work == nullptr) return -1;
    hipError_t e = hipEventQuery(work->end);
    if (e == hipSuccess) return 1;
    if (e == hipErrorNotReady) return 0;
    g_last_error = hipGetErrorString(e);
    return -1;
}

dt_status dt_work_free(dt_work* work) {
    if (work == nullptr) return DT_OK;
    if (work->start) (void)hipEventDestroy(work->start);
    if (work->end) (void)hipEventDestroy(work->end);
    delete work;
    return DT_OK;
}

// ---------------------------------------------------------- HSDP pipeline --
struct dt_hsdp {
    int replicate = 1, shard = 1;
    size_t bucket_bytes = 0;
    dt_dtype dtype = DT_BFLOAT16;
    dt_op op = DT_SUM;
    hipStream_t rs_stream = nullptr, ar_stream = nullptr;
    hipEvent_t produced = nullptr;   // producer stream position at post_backward
    hipEvent_t rs_done[2] = {nullptr, nullptr};  // ping-pong: previous / current layer's RS end
    int prev_slot = 0;
    std::vector<hipEvent_t> ar_done;  // one per issued fused AllReduce
    std::vector<hipEvent_t> spare;
    bool has_prev = false;
    std::vector<void*> prev_fused;    // previous layer's fused buffers (caller-owned)
    size_t prev_total = 0;            // elements per fused buffer
};

namespace {

// "wait prev RS": the AllReduce stream waits for the previous layer's
// ReduceScatter.  Queued before the current layer re-records anything.
dt_status hsdp_wait_prev_rs(dt_hsdp* h) {
    // on one stream the order of issue already puts the ReduceScatter first;
    // a wait there would only add a barrier packet (and its gap) to the queue
    if (h->ar_stream == h->rs_stream) return DT_OK;
    return check_hip(hipStreamWaitEvent(h->ar_stream, h->rs_done[h->prev_slot], 0), "AR stream waits prev RS");
}

// "issue prev AR": the previous layer's fused buffers, AllReduced in place
// inside each replicate group {j, shard+j, ...}, bucket by bucket.
dt_status hsdp_issue_prev_allreduce(dt_hsdp* h, bool last) {
    dt_status st;
    const size_t es = esize_of(h->dtype);
    const size_t per_bucket = h->bucket_bytes / es;
    // with one replica the fused shards already are the result: the AllReduce
    // of a group of one folds nothing, so only its end event is recorded
    const size_t fold_total = h->replicate > 1 ? h->prev_total : 0;
    // one launch per bucket covers every replicate group: piece j is group j's
    // slice [start, start + len) of its members' fused buffers, reduced in place
    const int per_launch = std::min(dt::kMaxPieces, dt::kPiecePtrs / h->replicate);
    for (size_t start = 0; start < fold_total; start += per_bucket) {
        const size_t len = std::min(per_bucket, fold_total - start);
        for (int j0 = 0; j0 < h->shard; j0 += per_launch) {
            dt::PieceArgs a = {};
            a.nranks = h->replicate;
            a.npieces = std::min(per_launch, h->shard - j0);
            uint64_t tiles = 0;
            for (int k = 0; k < a.npieces; k++) {
                bool al = true;
                for (int i = 0; i < h->replicate; i++) {
                    char* p = static_cast<char*>(h->prev_fused[size_t(i) * h->shard + j0 + k]) + start * es;
                    a.ptr[k * h->replicate + i] = p;
                    al = al && aligned16(p);
                }
                if (al) a.aligned |= 1u << k;
                a.len[k] = len;
                a.tile_start[k] = uint32_t(tiles);
                tiles += (len * es + dt::kPieceTileVecs * 16 - 1) / (dt::kPieceTileVecs * 16);
            }
            if (tiles > 0x7FFFFFFFull) return fail(DT_ERR_ARG, "bucket too large for one launch");
            a.tile_start[a.npieces] = uint32_t(tiles);
            if ((st = check_hip(dt::launch_reduce_pieces(a, h->dtype, h->op, h->ar_stream), "fused AllReduce")) != DT_OK)
                return st;
        }
    }
    h->has_prev = false;
    // on one stream only the last AllReduce of a pass needs an end event: the
    // stream's order covers the ones before it (each record is a queue entry)
    if (h->ar_stream == h->rs_stream && !last) return DT_OK;
    hipEvent_t ev = nullptr;
    if (!h->spare.empty()) {
        ev = h->spare.back();
        h->spare.pop_back();
    } else if ((st = check_hip(hipEventCreateWithFlags(&ev, hipEventDisableTiming), "hipEventCreate")) != DT_OK) {
        return st;
    }
    h->ar_done.push_back(ev);
    return check_hip(hipEventRecord(ev, h->ar_stream), "record AR done");
}

}  // namespace

dt_status dt_hsdp_create(int replicate, int shard, size_t bucket_bytes, dt_dtype dtype, dt_op op, hipStream_t rs_stream,
                         hipStream_t ar_stream, dt_hsdp** handle) {
    g_last_error.clear();
    if (handle == nullptr) return fail(DT_ERR_ARG, "handle is NULL");
    if (replicate < 1 || shard < 1 || replicate * shard > DT_MAX_RANKS)
        return fail(DT_ERR_ARG, "mesh %d x %d outside 1..%d ranks", replicate, shard, DT_MAX_RANKS);
    if (!valid_dtype(dtype) || !valid_op(op)) return fail(DT_ERR_ARG, "bad dtype %d or op %d", dtype, op);
    if (bucket_bytes == 0 || bucket_bytes % 16 != 0)
        return fail(DT_ERR_ARG, "bucket_bytes=%zu must be a positive multiple of 16", bucket_bytes);
    dt_hsdp* h = new dt_hsdp();
    h->replicate = replicate;
    h->shard = shard;
    h->bucket_bytes = bucket_bytes;
    h->dtype = dtype;
    h->op = op;
    h->rs_stream = rs_stream;
    h->ar_stream = ar_stream;
    dt_status st = check_hip(hipEventCreateWithFlags(&h->produced, hipEventDisableTiming), "hipEventCreate");
    for (int k = 0; k < 2 && st == DT_OK; k++)
        st = check_hip(hipEventCreateWithFlags(&h->rs_done[k], hipEventDisableTiming), "hipEventCreate");
    if (st != DT_OK) {
        dt_hsdp_destroy(h);
        return st;
    }
    *handle = h;
    return DT_OK;
}

dt_status dt_hsdp_post_backward(dt_hsdp* h, const void* const* grads, const size_t* numels, int ntensors,
                                void* const* fused, hipStream_t producer) {
    g_last_error.clear();
    if (h == nullptr) return fail(DT_ERR_ARG, "handle is NULL");
    const int nranks = h->replicate * h->shard;
    dt_status st;
    if (ntensors < 1 || numels == nullptr || grads == nullptr) return fail(DT_ERR_ARG, "no tensors");
    size_t total = 0;
    for (int t = 0; t < ntensors; t++) total += numels[t];
    for (int r = 0; r < nranks; r++)  // an empty tensor may carry a NULL pointer
        for (int t = 0; t < ntensors; t++)
            if (numels[t] > 0 && grads[size_t(r) * ntensors + t] == nullptr)
                return fail(DT_ERR_ARG, "grads[%d] (rank %d, tensor %d) is NULL", r * ntensors + t, r, t);
    if (total > 0 && (st = check_ptr_array(fused, nranks, "fused")) != DT_OK) return st;
    for (int t = 0; t < ntensors; t++)
        if (numels[t] % size_t(h->shard) != 0)
            return fail(DT_ERR_ARG, "numels[%d]=%zu not divisible by shard=%d", t, numels[t], h->shard);
    const size_t es = esize_of(h->dtype);
    if (total > 0) {
        // The ReduceScatter writes fused[r] while it reads the gradients, and
        // the previous layer's fused buffers still wait for their AllReduce
        // (queued below, after this ReduceScatter): reusing them before
        // dt_hsdp_finish would overwrite shards that are not yet reduced.
        std::vector<Span> w, rd;
        for (int r = 0; r < nranks; r++) {
            add_span(w, fused[r], total / size_t(h->shard) * es, "fused", r);
            for (int t = 0; t < ntensors; t++) add_span(rd, grads[size_t(r) * ntensors + t], numels[t] * es, "grads", r * ntensors + t);
            if (h->has_prev) add_span(rd, h->prev_fused[r], h->prev_total * es, "previous layer's fused", r);
        }
        // an exact match is an in-place operand for check_disjoint, never valid here
        for (const Span& x : rd)
            for (const Span& y : w)
                if (x.lo == y.lo && x.n == y.n)
                    return fail(DT_ERR_ARG, "hsdp post_backward: %s[%d] is %s[%d]", x.name, x.index, y.name, y.index);
        if ((st = check_disjoint(w, rd, "hsdp post_backward")) != DT_OK) return st;
    }

    // 1. wait prev RS
    if (h->has_prev && (st = hsdp_wait_prev_rs(h)) != DT_OK) return st;
    // 2. issue this layer's ReduceScatter, after everything the producer
    //    queued: tensor t of shard group i lands in fused[r] at offset `at`
    if (producer != h->rs_stream) {  // on the producer's own stream the order already holds
        if ((st = check_hip(hipEventRecord(h->produced, producer), "record producer")) != DT_OK) return st;
        if ((st = check_hip(hipStreamWaitEvent(h->rs_stream, h->produced, 0), "RS stream waits producer")) != DT_OK)
            return st;
    }
    // every tensor of every shard group is one segment of one launch
    std::vector<std::vector<const void*>> seg_src;
    std::vector<std::vector<void*>> seg_dst;
    std::vector<size_t> seg_m;
    size_t at = 0;
    for (int t = 0; t < ntensors; t++) {
        const size_t m = numels[t] / size_t(h->shard);
        for (int i = 0; i < h->replicate; i++) {
            std::vector<const void*> src(h->shard);
            std::vector<void*> dst(h->shard);
            for (int j = 0; j < h->shard; j++) {
                const int r = i * h->shard + j;
                src[j] = grads[size_t(r) * ntensors + t];
                dst[j] = static_cast<char*>(fused[r]) + at * es;
            }
            seg_src.push_back(src);
            seg_dst.push_back(dst);
            seg_m.push_back(m);
        }
        at += m;
    }
    if ((st = reduce_scatter_segments(seg_src, seg_dst, seg_m, h->shard, h->dtype, h->op, h->rs_stream)) != DT_OK)
        return st;
    const int cur_slot = h->prev_slot ^ 1;
    // the AllReduce stream's wait for this ReduceScatter (one stream: its order)
    if (h->ar_stream != h->rs_stream &&
        (st = check_hip(hipEventRecord(h->rs_done[cur_slot], h->rs_stream), "record RS done")) != DT_OK)
        return st;
    // 3. issue the previous layer's fused AllReduce (its wait is queued above)
    if (h->has_prev && (st = hsdp_issue_prev_allreduce(h, false)) != DT_OK) return st;
    // this layer becomes the previous one
    h->prev_slot = cur_slot;
    if (fused)
        h->prev_fused.assign(fused, fused + nranks);
    else
        h->prev_fused.assign(size_t(nranks), nullptr);  // an empty layer: nothing to reduce
    h->prev_total = at;
    h->has_prev = true;
    return DT_OK;
}

dt_status dt_hsdp_finish(dt_hsdp* h, hipStream_t consumer) {
    g_last_error.clear();
    if (h == nullptr) return fail(DT_ERR_ARG, "handle is NULL");
    dt_status st;
    if (h->has_prev) {  // drain: the last layer's RS, then its fused AllReduce
        if ((st = hsdp_wait_prev_rs(h)) != DT_OK) return st;
        if ((st = hsdp_issue_prev_allreduce(h, true)) != DT_OK) return st;
    }
    for (hipEvent_t ev : h->ar_done) {
        if (consumer != h->ar_stream &&
            (st = check_hip(hipStreamWaitEvent(consumer, ev, 0), "consumer waits AR")) != DT_OK)
            return st;
        h->spare.push_back(ev);
    }
    h->ar_done.clear();
    return DT_OK;
}

dt_status dt_hsdp_destroy(dt_hsdp* h) {
    if (h == nullptr) return DT_OK;
    for (hipEvent_t ev : h->ar_done) {
        (void)hipEventSynchronize(ev);
        (void)hipEventDestroy(ev);
    }
    for (hipEvent_t ev : h->spare) {
        (void)hipEventSynchronize(ev);
        (void)hipEventDestroy(ev);
    }
    if (h->produced) (void)hipEventDestroy(h->produced);
    // a layer posted but never finished still has its ReduceScatter writing
    // the caller's fused buffers: wait for it before the caller may free them
    // (its AllReduce is dropped, not queued); on one stream, whose unfinished
    // work carries no events, wait for the stream
    if (h->ar_stream == h->rs_stream) (void)hipStreamSynchronize(h->rs_stream);
    for (hipEvent_t ev : h->rs_done)
        if (ev) {
            (void)hipEventSynchronize(ev);
            (void)hipEventDestroy(ev);
        }
    delete h;
    return DT_OK;
}

}  // extern "C"
