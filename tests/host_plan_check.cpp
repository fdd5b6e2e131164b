// Host-side check of the library's planning code under AddressSanitizer and
// UndefinedBehaviorSanitizer (CPU only, no GPU, no HIP runtime).
//
// api.cpp (the C ABI: validation, offset and tile tables, bucket plan, work
// handles, HSDP schedule) is compiled for the host and linked against this
// file, which stands in for two things:
//   * the kernel launchers of dt_launch.h: instead of launching, each one
//     walks the grid it was given the way its kernel indexes memory and
//     checks that every byte range a workgroup would read or write lies
//     inside a buffer the test registered (reads: inputs or in-place
//     buffers; writes: outputs), that tile tables start at 0, grow by the
//     kernel's tile size and match the grid, and that every "aligned" flag
//     is backed by 16-byte aligned addresses;
//   * the few HIP runtime calls api.cpp makes (events, stream waits, device
//     attributes), as no-ops.
// The "device buffers" are host heap blocks of exact size, so the sanitizer
// also catches any host-side overrun in the table builders themselves.
// The program prints "ok <launches>" when every call behaved.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "dt.h"
#include "dt_launch.h"

namespace {

int g_fail = 0;
long g_launches = 0;

#define CHECK(cond, ...)                                                     \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: ", __FILE__, __LINE__);                  \
            fprintf(stderr, __VA_ARGS__);                                    \
            fprintf(stderr, "\n");                                           \
            ++g_fail;                                                        \
            exit(1);                                                         \
        }                                                                    \
    } while (0)

// ------------------------------------------------------------ registry --
struct Buf {
    size_t size;
    bool writable;
};
std::map<const char*, Buf> g_bufs;  // by base address; the buffers never overlap

void reg(const void* p, size_t n, bool writable) {
    if (p) g_bufs[static_cast<const char*>(p)] = Buf{n, writable};
}

// [p + off, p + off + n) must lie inside one registered buffer.
void touch(const void* p, uint64_t off, uint64_t n, bool write, const char* what) {
    if (n == 0) return;
    const char* lo = static_cast<const char*>(p) + off;
    auto it = g_bufs.upper_bound(lo);  // first buffer starting after lo
    if (it != g_bufs.begin()) {
        --it;
        if (lo + n <= it->first + it->second.size) {
            CHECK(!write || it->second.writable, "%s writes a read-only buffer", what);
            return;
        }
    }
    CHECK(false, "%s touches %llu bytes at %p (offset %llu) outside every buffer", what, (unsigned long long)n,
          static_cast<const void*>(lo), (unsigned long long)off);
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool line_al(const void* p) { return (reinterpret_cast<uintptr_t>(p) & (dt::kGridAlign - 1)) == 0; }
size_t esize(int dtype) { return dtype == DT_BFLOAT16 ? 2 : 4; }
uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// a tile table: starts at 0, piece k spans want[k] tiles, total = grid
void check_tiles(const uint32_t* tile_start, const std::vector<uint64_t>& want, uint64_t grid, const char* what) {
    CHECK(tile_start[0] == 0, "%s: tile_start[0] = %u", what, tile_start[0]);
    for (size_t k = 0; k < want.size(); k++)
        CHECK(tile_start[k + 1] - tile_start[k] == want[k], "%s: piece %zu has %u tiles, expected %llu", what, k,
              tile_start[k + 1] - tile_start[k], (unsigned long long)want[k]);
    CHECK(tile_start[want.size()] == grid, "%s: table ends at %u, grid %llu", what, tile_start[want.size()],
          (unsigned long long)grid);
}

}  // namespace

// ------------------------------------------------------ HIP stand-ins --
extern "C" {
hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
    *value = 100000;
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stand-in"; }
// Events the library has recorded since they were created: a stream wait on
// one it never recorded would order nothing, a planning bug.
std::set<hipEvent_t> g_recorded;
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    *e = reinterpret_cast<hipEvent_t>(malloc(64));
    g_recorded.erase(*e);
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    g_recorded.erase(e);
    free(e);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
    CHECK(e != nullptr, "record on a null event");
    g_recorded.insert(e);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipEventQuery(hipEvent_t e) {
    CHECK(e != nullptr, "query of a null event");
    return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
    CHECK(e != nullptr, "sync on a null event");
    return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned) {
    CHECK(e != nullptr, "wait on a null event");
    CHECK(g_recorded.count(e) == 1, "a stream waits on an event that was never recorded");
    return hipSuccess;
}
}

// ------------------------------------------------- launcher stand-ins --
namespace dt {

// While g_log_folds is set, the reduce, piece-fold and gather stand-ins
// record every byte range they write on rank 0 (start, bytes): an in-place
// AllReduce plan must write each element of rank 0's tensors exactly once.
bool g_log_folds = false;
std::vector<std::pair<const char*, uint64_t>> g_fold_log;
void log_fold(const void* p, uint64_t bytes) {
    if (g_log_folds && bytes) g_fold_log.push_back({static_cast<const char*>(p), bytes});
}

// The static staging buffer: a fake device range (never dereferenced),
// registered as writable on every lookup since the driver clears the
// registry between cases.
int g_scratch_lookups = 0;
hipError_t scratch_base(void** ptr) {
    g_scratch_lookups++;
    char* p = reinterpret_cast<char*>(uintptr_t(3) << 44);
    reg(p, kScratchBytes, true);
    *ptr = p;
    return hipSuccess;
}

// Output vectors per tile of the segmented ReduceScatter.  Deliberately not
// the library's value: the planning code must take the tile size from this
// function, never from a constant of its own.
uint64_t seg_rs_tile_vecs(int) { return 384; }

int g_rs_launches = 0;  // ReduceScatter-mode launches (a.rs) since the last reset

hipError_t launch_reduce_vec(const ReduceArgs& a, int, int, hipStream_t) {
    g_launches++;
    if (a.rs) g_rs_launches++;
    CHECK(a.nranks >= 1 && a.nranks <= kMaxRanksHost, "reduce_vec nranks %d", a.nranks);
    const uint64_t bytes = a.count * 16;
    if (!a.rs) {
        log_fold(a.dst[0], bytes);
        for (int r = 0; r < a.nranks; r++) {
            CHECK(al16(a.src[r]) && al16(a.dst[r]), "reduce_vec buffers not 16-byte aligned");
            touch(a.src[r], 0, bytes, false, "reduce_vec read");
            touch(a.dst[r], 0, bytes, true, "reduce_vec write");
        }
        return hipSuccess;
    }
    // ReduceScatter: chunk c starts c * chunk_stride vectors into every input and
    // holds count vectors, the last chunk last_count (the kernel's early exit)
    CHECK(a.last_count >= 1 && a.last_count <= a.count, "reduce_scatter: last chunk %llu of %llu vectors",
          (unsigned long long)a.last_count, (unsigned long long)a.count);
    CHECK(a.chunk_stride >= a.count, "reduce_scatter: chunk stride %llu below the count %llu",
          (unsigned long long)a.chunk_stride, (unsigned long long)a.count);
    const uint64_t last = a.last_count * 16;
    log_fold(a.dst[0], a.nranks == 1 ? last : bytes);
    for (int r = 0; r < a.nranks; r++) {
        CHECK(al16(a.src[r]) && al16(a.dst[r]), "reduce_vec buffers not 16-byte aligned");
        for (int c = 0; c < a.nranks; c++)
            touch(a.src[r], c * a.chunk_stride * 16, c + 1 == a.nranks ? last : bytes, false, "reduce_scatter read");
        touch(a.dst[r], 0, r + 1 == a.nranks ? last : bytes, true, "reduce_scatter write");
    }
    return hipSuccess;
}

hipError_t launch_reduce_elems(const ReduceArgs& a, int dtype, int, hipStream_t) {
    g_launches++;
    const size_t es = esize(dtype);
    const uint64_t firsts[2] = {a.first, a.first2}, counts[2] = {a.count, a.count2};
    for (int k = 0; k < 2; k++) {  // the launch's two element ranges
        const uint64_t first = firsts[k], count = counts[k];
        if (count == 0) continue;
        log_fold(static_cast<const char*>(a.dst[0]) + first * es, count * es);
        for (int r = 0; r < a.nranks; r++) {
            if (a.rs) {
                for (int c = 0; c < a.nranks; c++)
                    touch(a.src[r], (c * a.chunk_elems + first) * es, count * es, false, "reduce_elems read");
            } else {
                touch(a.src[r], first * es, count * es, false, "reduce_elems read");
            }
            touch(a.dst[r], first * es, count * es, true, "reduce_elems write");
        }
    }
    CHECK(a.count2 == 0 || a.first2 >= a.first + a.count, "reduce_elems: ranges overlap or out of order");
    return hipSuccess;
}

template <typename Args>
void check_piece_table(const Args& a, int npieces_cap, int ptr_cap, size_t es, bool fold, int to_ws, const char* what) {
    CHECK(a.npieces >= 1 && a.npieces <= npieces_cap, "%s: %d pieces", what, a.npieces);
    CHECK(a.npieces * a.nranks <= ptr_cap, "%s: %d pointers", what, a.npieces * a.nranks);
    std::vector<uint64_t> want;
    for (int k = 0; k < a.npieces; k++) want.push_back(ceil_div(a.len[k] * es, kPieceTileVecs * 16));
    check_tiles(a.tile_start, want, a.tile_start[a.npieces], what);
    for (int k = 0; k < a.npieces; k++) {
        CHECK(a.len[k] > 0, "%s: empty piece %d", what, k);
        for (int r = 0; r < a.nranks; r++) {
            const void* p = a.ptr[k * a.nranks + r];
            if (fold) {
                if (r == 0) log_fold(p, a.len[k] * es);
                touch(p, 0, a.len[k] * es, true, what);  // reduced in place
            } else {
                touch(p, 0, a.len[k] * es, !to_ws, what);
                touch(a.ws[r], a.wpos[k] * es, a.len[k] * es, to_ws != 0, what);
            }
        }
    }
}
bool piece_aligned(const PieceArgs& a, int k) { return (a.aligned >> k) & 1u; }
bool piece_aligned(const CoalescedArgs& a, int k) { return (a.aligned[k >> 5] >> (k & 31)) & 1u; }
template <typename Args>
void check_piece_alignment(const Args& a, size_t es, bool with_ws, const char* what) {
    for (int k = 0; k < a.npieces; k++) {
        if (!piece_aligned(a, k)) continue;
        for (int r = 0; r < a.nranks; r++) {
            CHECK(al16(a.ptr[k * a.nranks + r]), "%s: aligned flag on an unaligned piece", what);
            if (with_ws) CHECK(al16(static_cast<const char*>(a.ws[r]) + a.wpos[k] * es), "%s: unaligned ws", what);
        }
    }
}

hipError_t launch_reduce_pieces(const PieceArgs& a, int dtype, int, hipStream_t) {
    g_launches++;
    check_piece_table(a, kMaxPieces, kPiecePtrs, esize(dtype), true, 0, "reduce_pieces");
    check_piece_alignment(a, esize(dtype), false, "reduce_pieces");
    return hipSuccess;
}
hipError_t launch_reduce_coalesced(const CoalescedArgs& a, int dtype, int, hipStream_t) {
    g_launches++;
    check_piece_table(a, kCoalMaxPieces, kCoalPtrs, esize(dtype), true, 0, "reduce_coalesced");
    check_piece_alignment(a, esize(dtype), false, "reduce_coalesced");
    return hipSuccess;
}
hipError_t launch_copy_pieces(const PieceArgs& a, int es, int to_ws, hipStream_t) {
    g_launches++;
    check_piece_table(a, kMaxPieces, kPiecePtrs, size_t(es), false, to_ws, "copy_pieces");
    check_piece_alignment(a, size_t(es), true, "copy_pieces");
    return hipSuccess;
}
hipError_t launch_copy_coalesced(const CoalescedArgs& a, int es, int to_ws, hipStream_t) {
    g_launches++;
    check_piece_table(a, kCoalMaxPieces, kCoalPtrs, size_t(es), false, to_ws, "copy_coalesced");
    check_piece_alignment(a, size_t(es), true, "copy_coalesced");
    return hipSuccess;
}

hipError_t launch_reduce_scatter_segs(const SegReduceScatterArgs& a, int dtype, int, hipStream_t) {
    g_launches++;
    const size_t es = esize(dtype), v = 16 / es;
    CHECK(a.nsegs >= 1 && a.nsegs <= kMaxSegs && a.nsegs * a.nranks <= kSegPtrs, "segs: %d x %d", a.nsegs, a.nranks);
    std::vector<uint64_t> want;
    for (int k = 0; k < a.nsegs; k++) {
        CHECK(a.tiles_per_chunk[k] == ceil_div(a.m[k], seg_rs_tile_vecs(a.nranks) * v), "segs: tiles per chunk");
        want.push_back(uint64_t(a.tiles_per_chunk[k]) * a.nranks);
        for (int j = 0; j < a.nranks; j++) {
            touch(a.src[k * a.nranks + j], 0, a.m[k] * a.nranks * es, false, "segs read");
            touch(a.dst[k * a.nranks + j], 0, a.m[k] * es, true, "segs write");
            if (j == 0) log_fold(a.dst[k * a.nranks], a.m[k] * es);  // member 0's folded chunk
            if ((a.aligned >> k) & 1u) {
                CHECK(a.m[k] % v == 0, "segs: aligned flag with a ragged chunk");
                CHECK(al16(a.src[k * a.nranks + j]) && al16(a.dst[k * a.nranks + j]), "segs: unaligned");
            }
        }
    }
    check_tiles(a.tile_start, want, a.tile_start[a.nsegs], "segs");
    return hipSuccess;
}

// The line-grid ReduceScatter: chunk c of every input (c * in_stride
// elements in, count elements, last_count for the last chunk) folds into
// dst[c], lead[c] bytes into its line.
int g_grid_rs_launches = 0;
hipError_t launch_reduce_scatter_grid(const GridFoldArgs& a, int dtype, int, hipStream_t) {
    g_launches++;
    g_grid_rs_launches++;
    const uint64_t es = esize(dtype);
    CHECK(a.nranks >= 1 && a.nranks <= kMaxRanksHost && a.nchunks == a.nranks, "grid rs: %d ranks, %d chunks",
          a.nranks, a.nchunks);
    CHECK(a.last_count >= 1 && a.last_count <= a.count && a.in_stride >= a.count,
          "grid rs: chunks of %llu elements, the last %llu, stride %llu", (unsigned long long)a.count,
          (unsigned long long)a.last_count, (unsigned long long)a.in_stride);
    for (int c = 0; c < a.nchunks; c++) {
        const uint64_t n = (c + 1 == a.nchunks ? a.last_count : a.count) * es;
        const uintptr_t d = reinterpret_cast<uintptr_t>(a.dst[c]);
        // the tiles follow the output's lines: every store is a whole aligned vector
        CHECK(a.lead[c] == (d & (kGridAlign - 1)), "grid rs: chunk %d lead %u for an output at %llu mod 128", c,
              a.lead[c], (unsigned long long)(d & (kGridAlign - 1)));
        CHECK(d % es == 0, "grid rs: output %d not element-aligned", c);
        touch(a.dst[c], 0, n, true, "grid reduce_scatter write");
        for (int r = 0; r < a.nranks; r++) {
            CHECK(reinterpret_cast<uintptr_t>(a.src[r]) % es == 0, "grid rs: input %d not element-aligned", r);
            touch(a.src[r], c * a.in_stride * es, n, false, "grid reduce_scatter read");
        }
    }
    log_fold(a.dst[0], (a.nchunks == 1 ? a.last_count : a.count) * es);
    return hipSuccess;
}

// Every gather piece launched since the last reset: (source, bytes, first
// destination), for the coverage check of the windowed fan-out.
struct GatherPiece {
    const char* src;
    uint64_t bytes;
    const char* dst0;
};
std::vector<GatherPiece> g_gather_pieces;
int g_touch_launches = 0;

// Tiles of gather piece r: over its bytes, or, for a shifted piece, over its
// destinations' aligned 16-byte grid (all of them off alignment by md).
uint64_t gather_tiles(const GatherArgs& a, int r) {
    CHECK(a.tile_bytes == kGatherTileBytes || a.tile_bytes == kGatherWaveTileBytes, "gather: tile of %u bytes",
          a.tile_bytes);
    if (((a.shifted >> r) & 1u) && a.bytes[r]) {
        CHECK(!((a.aligned >> r) & 1u), "gather: piece %d both aligned and shifted", r);
        // the kernel stores grid vector v of destination q at dst[q] - lead +
        // 16 v and loads the source at src + 16 v - lead - sm: every grid
        // start must sit on a 128-byte line, and sm must put the loads on
        // vectors
        const uint32_t lead = a.lead[r] & 0xFFFFu, sm = a.lead[r] >> 16;
        CHECK(lead < kGridAlign && sm < 16, "gather: piece %d lead %u sm %u", r, lead, sm);
        for (int q = 0; q < a.nranks; q++)
            CHECK(((reinterpret_cast<uintptr_t>(a.dst[r * a.nranks + q]) - lead) & (kGridAlign - 1)) == 0,
                  "gather: shifted piece %d: destination %d off its grid (lead %u)", r, q, lead);
        CHECK(((reinterpret_cast<uintptr_t>(a.src[r]) - lead - sm) & 15u) == 0,
              "gather: shifted piece %d: source loads off the vectors (lead %u sm %u)", r, lead, sm);
        return ceil_div(lead + a.bytes[r], a.tile_bytes);
    }
    CHECK(a.lead[r] == 0, "gather: lead %u on piece %d that is not shifted", a.lead[r], r);
    if ((a.aligned >> r) & 1u) return ceil_div(a.bytes[r], a.tile_bytes);
    // destinations at offsets of their own: each over its own line grid,
    // grid byte g being piece byte g - (dst mod 128); tiles for a lead of 127
    return a.bytes[r] ? ceil_div(kGridAlign - 1 + a.bytes[r], a.tile_bytes) : 0;
}

hipError_t launch_gather_touch(const GatherArgs& a, uint32_t tiles, hipStream_t) {
    g_launches++;
    g_touch_launches++;
    CHECK(a.tile_bytes == kGatherTileBytes, "gather touch: %u-byte tiles", a.tile_bytes);
    std::vector<uint64_t> want;
    for (int r = 0; r < a.nranks; r++) want.push_back(gather_tiles(a, r));
    check_tiles(a.tile_start, want, tiles, "gather touch");
    for (int r = 0; r < a.nranks; r++) {
        touch(a.src[r], 0, a.bytes[r], false, "gather touch read");
        if ((a.aligned >> r) & 1u) CHECK(al16(a.src[r]), "gather touch: unaligned source");
    }
    return hipSuccess;
}

hipError_t launch_gather(const GatherArgs& a, uint32_t tiles, hipStream_t) {
    g_launches++;
    CHECK(a.split_log2 <= 2 && (uint64_t(tiles) << a.split_log2) <= 0x7FFFFFFFull, "gather: split %u of %u tiles",
          a.split_log2, tiles);
    for (int r = 0; r < a.nranks; r++)
        if (a.bytes[r]) {
            g_gather_pieces.push_back(GatherPiece{static_cast<const char*>(a.src[r]), a.bytes[r],
                                                  static_cast<const char*>(a.dst[r * a.nranks])});
            if (a.dst[r * a.nranks] != a.src[r]) log_fold(a.dst[r * a.nranks], a.bytes[r]);
        }
    std::vector<uint64_t> want;
    for (int r = 0; r < a.nranks; r++) want.push_back(gather_tiles(a, r));
    check_tiles(a.tile_start, want, tiles, "gather");
    for (int r = 0; r < a.nranks; r++) {
        if (a.bytes[r] == 0) continue;
        touch(a.src[r], 0, a.bytes[r], false, "gather read");
        for (int q = 0; q < a.nranks; q++) {
            touch(a.dst[r * a.nranks + q], 0, a.bytes[r], true, "gather write");
            if ((a.aligned >> r) & 1u)
                CHECK(line_al(a.dst[r * a.nranks + q]), "gather: aligned piece with a destination off its line");
        }
        if ((a.aligned >> r) & 1u) CHECK(al16(a.src[r]), "gather: unaligned source");
    }
    return hipSuccess;
}

struct A2ABlock {
    const char* from;
    const char* to;
    uint64_t bytes;
};
std::vector<A2ABlock> g_a2a_blocks;  // every block of every all-to-all launch, in launch order

hipError_t launch_all_to_all(const AllToAllArgs& a, uint32_t tiles, hipStream_t) {
    g_launches++;
    CHECK(a.nblocks >= 1 && a.nblocks <= kA2ABlocks, "all_to_all: %d blocks", a.nblocks);
    std::vector<uint64_t> want;
    for (int k = 0; k < a.nblocks; k++) {
        CHECK(a.bytes[k] > 0, "all_to_all: empty block %d", k);
        const bool al = (a.aligned[k >> 6] >> (k & 63)) & 1ull;  // else tiles over the destination's aligned grid
        want.push_back(ceil_div((al ? 0 : reinterpret_cast<uintptr_t>(a.to[k]) & (kGridAlign - 1)) + a.bytes[k], kCopyTileBytes));
    }
    check_tiles(a.tile_start, want, tiles, "all_to_all");
    for (int k = a.nblocks + 1; k <= kA2ABlocks; k++)
        CHECK(a.tile_start[k] == UINT32_MAX, "all_to_all: tile_start[%d] = %u past the last block", k, a.tile_start[k]);
    for (int g = 0; g < kA2ABlocks / kA2AGroup; g++)
        CHECK(a.group_start[g] == a.tile_start[g * kA2AGroup], "all_to_all: group_start[%d] = %u", g, a.group_start[g]);
    for (int k = 0; k < a.nblocks; k++) {
        touch(a.from[k], 0, a.bytes[k], false, "all_to_all read");
        touch(a.to[k], 0, a.bytes[k], true, "all_to_all write");
        if ((a.aligned[k >> 6] >> (k & 63)) & 1ull)
            CHECK(al16(a.from[k]) && line_al(a.to[k]), "all_to_all: aligned flag on a block off its lines");
        g_a2a_blocks.push_back(A2ABlock{static_cast<const char*>(a.from[k]), static_cast<const char*>(a.to[k]),
                                        a.bytes[k]});
    }
    return hipSuccess;
}

hipError_t launch_copy_segments(const SegCopyArgs& a, hipStream_t) {
    g_launches++;
    CHECK(a.nsegs >= 1 && a.nsegs <= kMaxCopySegs, "copy_segments: %d segments", a.nsegs);
    std::vector<uint64_t> want;
    for (int k = 0; k < a.nsegs; k++) {
        const bool al = (a.aligned >> k) & 1ull;  // else tiles over the destination's aligned grid
        want.push_back(ceil_div((al ? 0 : reinterpret_cast<uintptr_t>(a.dst[k]) & (kGridAlign - 1)) + a.bytes[k], kSegCopyTileBytes));
        touch(a.src[k], 0, a.bytes[k], false, "copy_segments read");
        touch(a.dst[k], 0, a.bytes[k], true, "copy_segments write");
        if ((a.aligned >> k) & 1ull) CHECK(al16(a.src[k]) && line_al(a.dst[k]), "copy_segments: off its lines");
    }
    check_tiles(a.tile_start, want, a.tile_start[a.nsegs], "copy_segments");
    return hipSuccess;
}

hipError_t launch_all_to_all_dims(const DimsArgs& a, uint32_t blocks, hipStream_t) {
    g_launches++;
    const uint64_t es = a.esize, run_bytes = a.cp * es, P = uint64_t(a.nranks);
    CHECK(a.rp * P == a.rows && a.cp * P == a.cols, "dims: shapes");
    CHECK(a.nruns == a.rows * P, "dims: %llu runs", (unsigned long long)a.nruns);
    CHECK(a.runs_per_block >= 1 && a.runs_per_block <= kDimsMaxRunsPerBlock && a.tiles_per_run >= 1,
          "dims: blocking");
    if (a.wave) {
        CHECK(a.vec && run_bytes >= kDimsWaveTileBytes && a.runs_per_block == 1, "dims: single-wave path");
        CHECK(a.tiles_per_run == ceil_div(run_bytes, kDimsWaveTileBytes), "dims: wave tiles per run");
    } else {
        CHECK(!(a.vec && run_bytes >= kDimsWaveTileBytes), "dims: vector runs of a tile or more take the wave path");
        CHECK(a.tiles_per_run == (run_bytes >= kDimsTileBytes ? ceil_div(run_bytes, kDimsTileBytes) : 1),
              "dims: tiles per run");
    }
    CHECK(!(a.vec && a.elems), "dims: both the vector and the element path");
    if (a.elems)  // whole-element copies need every base element-aligned
        for (int r = 0; r < a.nranks; r++)
            CHECK(reinterpret_cast<uintptr_t>(a.src[r]) % es == 0 && reinterpret_cast<uintptr_t>(a.dst[r]) % es == 0,
                  "dims: element path with rank %d's buffers off element alignment", r);
    if (a.wave || a.tiles_per_run > 1)
        CHECK(blocks == a.nruns * a.tiles_per_run, "dims: grid %u", blocks);
    else
        CHECK(blocks == ceil_div(a.nruns, a.runs_per_block), "dims: grid %u", blocks);
    // the run decode of dt_launch.h, for every run: a whole run of cp elements
    const uint64_t block_src = (a.dir == 0 ? a.rp * a.cols : a.rows * a.cp) * es;
    const uint64_t block_dst = (a.dir == 0 ? a.rows * a.cp : a.rp * a.cols) * es;
    for (int r = 0; r < a.nranks; r++) {
        touch(a.src[r], 0, block_src, false, "dims source block");
        touch(a.dst[r], 0, block_dst, true, "dims destination block");
    }
    for (uint64_t k = 0; k < a.nruns; k++) {
        uint64_t i, j, src_off, dst_off;
        if (a.dir == 0) {
            j = k / a.rows;
            const uint64_t row = k % a.rows;
            i = row / a.rp;
            src_off = ((row % a.rp) * a.cols + j * a.cp) * es;
            dst_off = row * a.cp * es;
        } else {
            j = k / (a.rp * P);
            const uint64_t row = (k / P) % a.rp;
            i = k % P;
            src_off = (j * a.rp + row) * a.cp * es;
            dst_off = (row * a.cols + i * a.cp) * es;
        }
        CHECK(i < P && j < P, "dims: run %llu decodes to ranks %llu, %llu", (unsigned long long)k,
              (unsigned long long)i, (unsigned long long)j);
        if (i >= P || j >= P) break;
        touch(a.src[i], src_off, run_bytes, false, "dims run read");
        touch(a.dst[j], dst_off, run_bytes, true, "dims run write");
        if (a.vec)
            CHECK(run_bytes % 16 == 0 && al16(static_cast<const char*>(a.src[i]) + src_off) &&
                      al16(static_cast<const char*>(a.dst[j]) + dst_off),
                  "dims: vector flag on an unaligned run");
    }
    return hipSuccess;
}

hipError_t launch_barrier(const BarrierArgs& a, int, hipStream_t) {
    g_launches++;
    for (int r = 0; r < a.nranks; r++) touch(a.win[r], 0, uint64_t(a.nranks) * 4, true, "barrier window");
    touch(a.status, 0, 4, true, "barrier status");
    CHECK(a.timeout_ticks > 0, "barrier without a time budget");
    return hipSuccess;
}

hipError_t launch_exchange(const ExchangeArgs& a, int spread, hipStream_t s) {
    const hipError_t e = launch_barrier(a.bar, spread, s);
    for (int r = 0; r < a.bar.nranks; r++) {
        touch(a.src[r], 0, a.nbytes, false, "exchange read");
        touch(a.stage[r], 0, a.nbytes, true, "exchange stage");
        touch(a.dst[r], 0, a.nbytes, true, "exchange write");
    }
    return e;
}

}  // namespace dt

// ---------------------------------------------------------------- driver --
namespace {

std::mt19937_64 rng(12345);
size_t below(size_t n) { return n ? size_t(rng() % n) : 0; }

// exact-size host blocks posing as device buffers, at an element offset
struct Pool {
    std::vector<char*> raw;
    ~Pool() {
        for (char* p : raw) free(p);
    }
    // a buffer of n bytes starting `skew` bytes into a 16-aligned block
    char* get(size_t n, size_t skew, bool writable) {
        char* p = static_cast<char*>(aligned_alloc(16, ((n + skew + 15) / 16) * 16 + 16));
        raw.push_back(p);
        reg(p + skew, n, writable);
        return p + skew;
    }
};

void expect(dt_status st, dt_status want, const char* what) {
    CHECK(st == want, "%s returned %d (%s), expected %d", what, st, dt_last_error(), want);
}

void reductions() {
    for (int it = 0; it < 120; it++) {
        Pool pool;
        g_bufs.clear();
        const int p = 1 + int(below(16));
        const dt_dtype dtype = dt_dtype(below(3));
        const dt_op op = dt_op(below(4));
        const size_t es = esize(dtype);
        // sizes up to about 1 MiB per rank (past the line-grid two-shot
        // threshold), buffers aligned, at one shared offset, or each at an
        // offset of its own (up to 158 elements)
        const size_t m = below(4) == 0 ? below(3) : below(5) == 0 ? 20000 + below(20000) : below(3000);
        const int mode = int(below(3));
        const size_t shared_skew = es * below(4);
        auto skew = [&]() { return mode == 0 ? size_t(0) : mode == 1 ? shared_skew : es * below(80); };
        std::vector<const void*> send(p);
        std::vector<void*> recv(p), shard(p);
        for (int r = 0; r < p; r++) {
            send[r] = pool.get(p * m * es, skew(), false);
            recv[r] = pool.get(p * m * es, skew(), true);
            shard[r] = pool.get(m * es, skew(), true);
        }
        expect(dt_allreduce(send.data(), recv.data(), p, p * m, dtype, op, nullptr), DT_OK, "allreduce");
        expect(dt_reduce_scatter(send.data(), shard.data(), p, m, dtype, op, nullptr), DT_OK, "reduce_scatter");
        // in place
        for (int r = 0; r < p; r++) send[r] = recv[r];
        expect(dt_allreduce(send.data(), recv.data(), p, p * m, dtype, op, nullptr), DT_OK, "allreduce in place");
        expect(dt_replicate_to_shard(send.data(), shard.data(), p, m, dtype, nullptr), DT_OK, "replicate_to_shard");
    }
}

void copies() {
    using dt::A2ABlock;
    using dt::g_a2a_blocks;
    for (int it = 0; it < 120; it++) {
        Pool pool;
        g_bufs.clear();
        const int p = 1 + int(below(16));
        const dt_dtype dtype = dt_dtype(below(3));
        const size_t es = esize(dtype);
        const size_t skew = below(3) == 0 ? es * below(4) : 0;
        std::vector<size_t> counts(p);
        size_t total = 0;
        for (int r = 0; r < p; r++) total += counts[r] = below(3) == 0 ? 0 : below(below(2) ? 5000 : 40);
        std::vector<const void*> send(p);
        std::vector<void*> recv(p), vec(size_t(p) * p), bcast(p);
        for (int r = 0; r < p; r++) send[r] = counts[r] ? pool.get(counts[r] * es, skew, false) : nullptr;
        for (int q = 0; q < p; q++) recv[q] = pool.get(total * es, skew, true);
        expect(dt_all_gather(send.data(), recv.data(), p, counts.data(), 0, dtype, nullptr), DT_OK, "all_gather");
        for (int q = 0; q < p; q++)
            for (int r = 0; r < p; r++) vec[q * p + r] = counts[r] ? pool.get(counts[r] * es, skew, true) : nullptr;
        expect(dt_all_gather_into_vec(send.data(), vec.data(), p, counts.data(), 0, dtype, nullptr), DT_OK,
               "all_gather_into_vec");
        const size_t n0 = 1 + below(3000);
        const void* root = pool.get(n0 * es, skew, false);
        for (int q = 0; q < p; q++) bcast[q] = pool.get(n0 * es, skew, true);
        expect(dt_broadcast(root, bcast.data(), p, n0, dtype, nullptr), DT_OK, "broadcast");
        // equal counts
        const size_t c = 1 + below(2000);
        std::vector<const void*> send_eq(p);
        std::vector<void*> recv_eq(p);
        for (int r = 0; r < p; r++) send_eq[r] = pool.get(c * es, skew, false);
        for (int q = 0; q < p; q++) recv_eq[q] = pool.get(p * c * es, skew, true);
        expect(dt_all_gather(send_eq.data(), recv_eq.data(), p, nullptr, c, dtype, nullptr), DT_OK,
               "all_gather equal");

        // all-to-all with a random split matrix (zero blocks, empty ranks)
        std::vector<size_t> splits(size_t(p) * p);
        std::vector<size_t> row(p, 0), col(p, 0);
        const size_t hi = below(2) ? 3 : 1500;
        for (int i = 0; i < p; i++)
            for (int j = 0; j < p; j++) {
                splits[i * p + j] = below(4) == 0 ? 0 : below(hi);
                row[i] += splits[i * p + j];
                col[j] += splits[i * p + j];
            }
        std::vector<const void*> a_send(p);
        std::vector<void*> a_recv(p);
        for (int r = 0; r < p; r++) {
            a_send[r] = row[r] ? pool.get(row[r] * es, skew, false) : nullptr;
            a_recv[r] = col[r] ? pool.get(col[r] * es, skew, true) : nullptr;
        }
        g_a2a_blocks.clear();
        expect(dt_all_to_all(a_send.data(), a_recv.data(), p, splits.data(), dtype, nullptr), DT_OK, "all_to_all");
        // the blocks, in (i, j) order: rank i's send offset runs along its row, rank j's receive offset down its column
        size_t nb = 0;
        std::vector<size_t> down(p, 0);
        for (int i = 0; i < p; i++) {
            size_t along = 0;
            for (int j = 0; j < p; j++) {
                const size_t bytes = splits[i * p + j] * es;
                if (bytes) {
                    CHECK(nb < g_a2a_blocks.size(), "all_to_all: block %d -> %d missing", i, j);
                    const A2ABlock& g = g_a2a_blocks[nb++];
                    CHECK(g.from == static_cast<const char*>(a_send[i]) + along &&
                              g.to == static_cast<const char*>(a_recv[j]) + down[j] && g.bytes == bytes,
                          "all_to_all: block %d -> %d misplaced", i, j);
                }
                along += bytes;
                down[j] += bytes;
            }
        }
        CHECK(nb == g_a2a_blocks.size(), "all_to_all: %zu blocks launched, %zu expected", g_a2a_blocks.size(), nb);

        // shard-dimension all-to-all, every (src, dst) pair
        const size_t rows = p * (1 + below(6)), cols = p * (1 + below(below(2) ? 6 : 3000));
        for (int sd = 0; sd < 2; sd++)
            for (int dd = 0; dd < 2; dd++) {
                const size_t ns = sd == 0 ? rows / p * cols : rows * (cols / p);
                const size_t nd = dd == 0 ? rows / p * cols : rows * (cols / p);
                std::vector<const void*> ds(p);
                std::vector<void*> dd_(p);
                for (int r = 0; r < p; r++) {
                    ds[r] = pool.get(ns * es, skew, false);
                    dd_[r] = pool.get(nd * es, skew, true);
                }
                expect(dt_all_to_all_dims(ds.data(), dd_.data(), p, rows, cols, sd, dd, dtype, nullptr), DT_OK,
                       "all_to_all_dims");
            }
    }
}

void buckets() {
    for (int it = 0; it < 80; it++) {
        Pool pool;
        g_bufs.clear();
        const int p = 1 + int(below(16));
        const dt_dtype dtype = dt_dtype(below(3));
        const dt_op op = dt_op(below(4));
        const size_t es = esize(dtype);
        const int nt = 1 + int(below(below(4) == 0 ? 700 : 40));
        std::vector<size_t> numels(nt);
        for (int t = 0; t < nt; t++) numels[t] = below(5) == 0 ? 0 : below(below(2) ? 50 : 5000);
        std::vector<void*> grads(size_t(p) * nt);
        for (int r = 0; r < p; r++)
            for (int t = 0; t < nt; t++)
                grads[r * nt + t] = numels[t] ? pool.get(numels[t] * es, es * below(4), true) : nullptr;
        const size_t bucket = 16 * (below(2) ? 1 + below(8) : 64 + below(4000));
        expect(dt_bucket_allreduce(grads.data(), numels.data(), nt, p, bucket, nullptr, dtype, op, nullptr), DT_OK,
               "bucket in place");
        std::vector<void*> ws(p);
        for (int r = 0; r < p; r++) ws[r] = pool.get(bucket, 0, true);
        expect(dt_bucket_allreduce(grads.data(), numels.data(), nt, p, bucket, ws.data(), dtype, op, nullptr), DT_OK,
               "bucket staged");
        expect(dt_bucket_allreduce_noalloc(grads.data(), numels.data(), nt, p, bucket, dtype, op, nullptr), DT_OK,
               "bucket staged in the static buffer");
        expect(dt_allreduce_coalesced(grads.data(), numels.data(), nt, p, dtype, op, nullptr), DT_OK, "coalesced");

        // the bucket plan: every element exactly once, buckets within bounds
        size_t npieces = 0, nb = 0;
        expect(dt_bucket_plan(numels.data(), nt, es, bucket, nullptr, 0, &npieces, &nb), DT_OK, "plan count");
        std::vector<dt_piece> pieces(npieces + 1);
        expect(dt_bucket_plan(numels.data(), nt, es, bucket, pieces.data(), npieces, &npieces, &nb), DT_OK, "plan");
        std::vector<size_t> covered(nt, 0);
        for (size_t k = 0; k < npieces; k++) {
            const dt_piece& pc = pieces[k];
            CHECK(pc.tensor >= 0 && pc.tensor < nt && size_t(pc.bucket) < nb, "plan: piece %zu", k);
            CHECK(pc.offset == covered[pc.tensor], "plan: piece %zu out of order", k);
            CHECK((pc.bucket_pos + pc.length) * es <= bucket, "plan: piece %zu overflows its bucket", k);
            covered[pc.tensor] += pc.length;
        }
        for (int t = 0; t < nt; t++) CHECK(covered[t] == numels[t], "plan: tensor %d covered %zu", t, covered[t]);
    }
}

// In place, tensors of at least 16 MiB per rank take an AllReduce of their
// own (two-shot or one-shot with a ragged tail) and the rest one fold: rank
// 0's copy of every tensor is written exactly once, with no gap or overlap.
void bucket_big_case(int p, const std::vector<size_t>& numel_list) {
    const int nt = int(numel_list.size());
    const size_t es = 2;
    const size_t* numels = numel_list.data();
    g_bufs.clear();
    char* base = reinterpret_cast<char*>(uintptr_t(1) << 44);  // fake, never dereferenced
    std::vector<void*> grads(size_t(p) * nt);
    for (int r = 0; r < p; r++)
        for (int t = 0; t < nt; t++) {
            grads[r * nt + t] = base + (uint64_t(r) << 36) + (uint64_t(t) << 30);
            reg(grads[r * nt + t], numels[t] * es, true);
        }
    dt::g_fold_log.clear();
    dt::g_log_folds = true;
    expect(dt_bucket_allreduce(grads.data(), numels, nt, p, size_t(25) << 20, nullptr, DT_BFLOAT16, DT_SUM, nullptr),
           DT_OK, "bucket in place, large tensors");
    dt::g_log_folds = false;
    for (int t = 0; t < nt; t++) {
        const char* t0 = static_cast<const char*>(grads[t]);
        const uint64_t bytes = numels[t] * es;
        std::vector<std::pair<const char*, uint64_t>> in;
        for (const auto& e : dt::g_fold_log)
            if (e.first < t0 + bytes && e.first + e.second > t0) in.push_back(e);
        std::sort(in.begin(), in.end());
        uint64_t at = 0;
        for (const auto& e : in) {
            CHECK(e.first == t0 + at, "bucket in place: tensor %d written at +%lld, expected +%llu", t,
                  (long long)(e.first - t0), (unsigned long long)at);
            at += e.second;
        }
        CHECK(at == bytes, "bucket in place: tensor %d covered %llu of %llu bytes", t, (unsigned long long)at,
              (unsigned long long)bytes);
    }
    g_bufs.clear();
}

void bucket_big() {
    const size_t MiE = size_t(1) << 20;  // elements
    // two-shot 32 and 88 MiB tensors, a ragged one, small ones folded
    bucket_big_case(8, {16 * MiE, 4096, 8 * MiE + 3, 100, 44 * MiE, 8 * MiE - 8});
    // P=16: five two-shot 40 MiB tensors, one of 16 MiB, a small one
    bucket_big_case(16, {20 * MiE, 20 * MiE, 20 * MiE, 20 * MiE, 20 * MiE, 8 * MiE, 7});
    // P=4: one-shot 48 MiB tensors
    bucket_big_case(4, {24 * MiE, 24 * MiE, 24 * MiE});
}

void hsdp_and_sync() {
    const int meshes[][2] = {{2, 4}, {1, 8}, {8, 1}, {4, 4}, {2, 2}, {1, 1}, {16, 1}, {1, 16}};
    for (auto& mesh : meshes) {
        Pool pool;
        g_bufs.clear();
        const int rep = mesh[0], sh = mesh[1], p = rep * sh;
        const dt_dtype dtype = DT_BFLOAT16;
        const size_t es = 2;
        // stream layouts (fake handles, never dereferenced): everything on one
        // stream; one side stream apart from the producer; two side streams
        const hipStream_t s1 = reinterpret_cast<hipStream_t>(uintptr_t(0x1000)),
                          s2 = reinterpret_cast<hipStream_t>(uintptr_t(0x2000)),
                          s3 = reinterpret_cast<hipStream_t>(uintptr_t(0x3000));
        const hipStream_t layouts[3][3] = {{nullptr, nullptr, nullptr}, {s1, s1, s3}, {s1, s2, s3}};
        for (const auto& lay : layouts) {
        dt_hsdp* h = nullptr;
        expect(dt_hsdp_create(rep, sh, 16 * (1 + below(100)), dtype, DT_SUM, lay[0], lay[1], &h), DT_OK, "hsdp");
        for (int layer = 0; layer < 5; layer++) {
            const int nt = 1 + int(below(9));
            std::vector<size_t> numels(nt);
            size_t total = 0;
            for (int t = 0; t < nt; t++) total += numels[t] = sh * (below(4) == 0 ? 0 : 1 + below(700));
            std::vector<void*> grads(size_t(p) * nt), fused(p);
            for (int r = 0; r < p; r++) {
                for (int t = 0; t < nt; t++) grads[r * nt + t] = numels[t] ? pool.get(numels[t] * es, 0, false) : nullptr;
                fused[r] = pool.get(total / sh * es, 0, true);
            }
            expect(dt_hsdp_post_backward(h, grads.data(), numels.data(), nt, fused.data(), lay[2]), DT_OK,
                   "hsdp post_backward");
        }
        expect(dt_hsdp_finish(h, lay[2]), DT_OK, "hsdp finish");
        expect(dt_hsdp_destroy(h), DT_OK, "hsdp destroy");
        }

        // barrier and exchange
        std::vector<int32_t*> win(p);
        for (int r = 0; r < p; r++) win[r] = reinterpret_cast<int32_t*>(pool.get(size_t(p) * 4, 0, true));
        int32_t* status = reinterpret_cast<int32_t*>(pool.get(4, 0, true));
        for (int layout = 0; layout < 2; layout++)
            expect(dt_barrier(win.data(), p, 1, 10, status, 0, layout, nullptr), DT_OK, "barrier");
        const size_t nbytes = below(5000);
        std::vector<const void*> src(p);
        std::vector<void*> stage(p), dst(p);
        for (int r = 0; r < p; r++) {
            src[r] = pool.get(nbytes, 0, false);
            stage[r] = pool.get(nbytes, 0, true);
            dst[r] = pool.get(nbytes, 0, true);
        }
        expect(dt_barrier_exchange(src.data(), stage.data(), dst.data(), nbytes, win.data(), p, 11, status, 0,
                                   DT_BARRIER_PACKED, nullptr),
               DT_OK, "exchange");
    }
}

void validation() {
    Pool pool;
    g_bufs.clear();
    const void* a = pool.get(64, 0, false);
    void* b = pool.get(64, 0, true);
    const void* send[2] = {a, a};
    void* recv[2] = {b, b};
    expect(dt_allreduce(send, recv, 0, 4, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "nranks 0");
    expect(dt_allreduce(send, recv, 17, 4, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "nranks 17");
    expect(dt_allreduce(send, recv, 2, 4, dt_dtype(7), DT_SUM, nullptr), DT_ERR_ARG, "bad dtype");
    expect(dt_allreduce(send, recv, 2, 4, DT_FLOAT32, dt_op(9), nullptr), DT_ERR_ARG, "bad op");
    expect(dt_allreduce(send, recv, 2, 4, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "recv aliases");
    size_t numels[1] = {4};
    void* g[1] = {b};
    expect(dt_bucket_allreduce(g, numels, 1, 1, 24, nullptr, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG,
           "bucket not a multiple of 16");
    size_t np = 0, nb = 0;
    expect(dt_bucket_plan(numels, 1, 4, 2, nullptr, 0, &np, &nb), DT_ERR_ARG, "bucket smaller than an element");
    // the static staging buffer holds nranks * bucket_bytes at most
    void* g8[8];
    size_t numels8[1] = {4};
    for (int r = 0; r < 8; r++) g8[r] = pool.get(16, 0, true);
    expect(dt_bucket_allreduce_noalloc(g8, numels8, 1, 8, size_t(32) << 20, DT_FLOAT32, DT_SUM, nullptr), DT_OK,
           "noalloc, 8 x 32 MiB buckets");
    expect(dt_bucket_allreduce_noalloc(g8, numels8, 1, 8, (size_t(32) << 20) + 16, DT_FLOAT32, DT_SUM, nullptr),
           DT_ERR_ARG, "noalloc, buckets beyond the static buffer");
    expect(dt_bucket_allreduce_noalloc(g8, numels8, 1, 8, 24, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG,
           "noalloc, bucket not a multiple of 16");
}

// Partial overlaps between buffers that a launch writes and buffers it reads
// or writes elsewhere: the kernels would race, so every entry point refuses
// them, while exact in-place operands stay allowed.
void overlaps() {
    Pool pool;
    g_bufs.clear();
    const size_t n = 1024;  // fp32 elements per rank
    char* big = pool.get(16 * n * 4, 0, true);  // one block, carved into overlapping views
    const void* send[2] = {big, big + 4 * n * 4};
    void* recv[2] = {big + 8 * n * 4, big + 12 * n * 4};
    expect(dt_allreduce(send, recv, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_OK, "allreduce, disjoint views");
    recv[1] = big + 8 * n * 4 + 2048;  // inside recv[0]
    expect(dt_allreduce(send, recv, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "allreduce, recv overlap");
    recv[1] = big + 12 * n * 4;
    send[1] = big + 8 * n * 4 + 64;  // reads inside recv[0]
    expect(dt_allreduce(send, recv, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "allreduce, send inside recv");
    void* inplace[2] = {big, big + 4 * n * 4};
    const void* inplace_c[2] = {big, big + 4 * n * 4};
    expect(dt_allreduce(inplace_c, inplace, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_OK, "allreduce in place");
    const void* skewed[2] = {big + 64, big + 4 * n * 4};  // in place for rank 1 only; send[0] overlaps recv[0]
    expect(dt_allreduce(skewed, inplace, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "allreduce, shifted self");

    // ReduceScatter: send[r] holds 2n, recv[r] n
    const void* rs_send[2] = {big, big + 2 * n * 4};
    void* rs_recv[2] = {big + 8 * n * 4, big + 3 * n * 4};  // recv[1] inside send[1]
    expect(dt_reduce_scatter(rs_send, rs_recv, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG, "rs, recv inside send");
    rs_recv[1] = big + 10 * n * 4;
    expect(dt_reduce_scatter(rs_send, rs_recv, 2, n, DT_FLOAT32, DT_SUM, nullptr), DT_OK, "rs, disjoint");

    // AllGather: a source that starts before an output and runs into it
    const void* ag_send[2] = {big + 8 * n * 4 - 64, big};
    void* ag_recv[2] = {big + 8 * n * 4, big + 12 * n * 4};
    expect(dt_all_gather(ag_send, ag_recv, 2, nullptr, n, DT_FLOAT32, nullptr), DT_ERR_ARG, "ag, send runs into recv");
    const void* ag_inplace[2] = {big + 8 * n * 4, big + 12 * n * 4 + n * 4};  // each in its own slot
    expect(dt_all_gather(ag_inplace, ag_recv, 2, nullptr, n, DT_FLOAT32, nullptr), DT_OK, "ag in place");

    // AllToAll: recv[0] overlapping send[1]
    const size_t splits[4] = {n, n, n, n};
    const void* a_send[2] = {big, big + 2 * n * 4};
    void* a_recv[2] = {big + 3 * n * 4, big + 8 * n * 4};
    expect(dt_all_to_all(a_send, a_recv, 2, splits, DT_FLOAT32, nullptr), DT_ERR_ARG, "a2a, recv overlaps send");
    a_recv[0] = big + 4 * n * 4;
    expect(dt_all_to_all(a_send, a_recv, 2, splits, DT_FLOAT32, nullptr), DT_OK, "a2a, disjoint");

    // bucket / coalesced: two tensors of one rank overlapping
    size_t numels[2] = {n, n};
    void* g[4] = {big, big + 2 * n * 4, big + 4 * n * 4, big + 4 * n * 4 + 8};
    expect(dt_bucket_allreduce(g, numels, 2, 2, 4096, nullptr, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG,
           "bucket, overlapping tensors");
    expect(dt_allreduce_coalesced(g, numels, 2, 2, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG,
           "coalesced, overlapping tensors");
    g[3] = big + 6 * n * 4;
    void* ws[2] = {big + 8 * n * 4, big + 6 * n * 4 + 16};  // ws[1] inside grads[3]
    expect(dt_bucket_allreduce(g, numels, 2, 2, 4096, ws, DT_FLOAT32, DT_SUM, nullptr), DT_ERR_ARG,
           "bucket, workspace inside a tensor");
    ws[1] = big + 12 * n * 4;
    expect(dt_bucket_allreduce(g, numels, 2, 2, 4096, ws, DT_FLOAT32, DT_SUM, nullptr), DT_OK, "bucket, disjoint");

    // HSDP: one fused set reused for the next layer before finish() is refused
    dt_hsdp* h = nullptr;
    expect(dt_hsdp_create(2, 2, 4096, DT_BFLOAT16, DT_SUM, nullptr, nullptr, &h), DT_OK, "hsdp create");
    const size_t hn[1] = {2 * n};  // bf16, shard 2: fused holds n elements
    const void* hg[4] = {big, big + 4 * n, big + 8 * n, big + 12 * n};
    void* fused_a[4] = {big + 16 * n, big + 18 * n, big + 20 * n, big + 22 * n};
    void* fused_b[4] = {big + 24 * n, big + 26 * n, big + 28 * n, big + 30 * n};
    expect(dt_hsdp_post_backward(h, hg, hn, 1, fused_a, nullptr), DT_OK, "hsdp layer 0");
    expect(dt_hsdp_post_backward(h, hg, hn, 1, fused_a, nullptr), DT_ERR_ARG, "hsdp, fused reused before finish");
    void* fused_c[4] = {big + 24 * n, big + 26 * n, big + 17 * n, big + 30 * n};  // fused[2] inside layer 0's fused[0]
    expect(dt_hsdp_post_backward(h, hg, hn, 1, fused_c, nullptr), DT_ERR_ARG, "hsdp, fused overlaps previous");
    expect(dt_hsdp_post_backward(h, hg, hn, 1, fused_b, nullptr), DT_OK, "hsdp layer 1");
    expect(dt_hsdp_finish(h, nullptr), DT_OK, "hsdp finish");
    expect(dt_hsdp_post_backward(h, hg, hn, 1, fused_a, nullptr), DT_OK, "hsdp, fused reused after finish");
    void* fused_g[4] = {big + 2 * n, big + 26 * n, big + 28 * n, big + 30 * n};  // fused[0] inside grads[0]
    expect(dt_hsdp_finish(h, nullptr), DT_OK, "hsdp finish");
    expect(dt_hsdp_post_backward(h, hg, hn, 1, fused_g, nullptr), DT_ERR_ARG, "hsdp, fused overlaps a gradient");
    expect(dt_hsdp_destroy(h), DT_OK, "hsdp destroy");

    // HSDP with one replica: the fused AllReduce folds nothing, so it launches nothing
    expect(dt_hsdp_create(1, 4, 4096, DT_BFLOAT16, DT_SUM, nullptr, nullptr, &h), DT_OK, "hsdp 1x4");
    const size_t hn4[1] = {4 * n};
    const void* hg4[4] = {big, big + 8 * n, big + 16 * n, big + 24 * n};
    void* f4[4] = {big + 32 * n, big + 34 * n, big + 36 * n, big + 38 * n};
    const long before = g_launches;
    expect(dt_hsdp_post_backward(h, hg4, hn4, 1, f4, nullptr), DT_OK, "hsdp 1x4 layer");
    expect(dt_hsdp_finish(h, nullptr), DT_OK, "hsdp 1x4 finish");
    CHECK(g_launches - before == 1, "hsdp 1x4: %ld launches, expected the ReduceScatter only", g_launches - before);
    expect(dt_hsdp_destroy(h), DT_OK, "hsdp 1x4 destroy");
    g_bufs.clear();
}

}  // namespace

// The windowed fan-out of large sources: fake device ranges (never touched)
// of a few hundred MiB, odd sizes, one empty rank.  Every source byte must be
// launched exactly once, at the matching destination offset, with a read
// pass before each window.
void big_fan_out() {
    using dt::g_gather_pieces;
    using dt::g_touch_launches;
    using dt::GatherPiece;
    g_bufs.clear();
    const int p = 6;
    const size_t counts[p] = {3, (size_t(40) << 20) + 1, 7, (size_t(100) << 20) + 3, 0, (size_t(35) << 20) + 5};
    size_t total = 0;
    for (int r = 0; r < p; r++) total += counts[r];
    const size_t es = 2;  // bf16
    char* base = reinterpret_cast<char*>(uintptr_t(1) << 44);  // a fake, 16-byte aligned address range
    const void* send[p];
    void* recv[p];
    for (int r = 0; r < p; r++) {
        send[r] = counts[r] ? base + (uint64_t(r) << 32) : nullptr;
        if (counts[r]) reg(send[r], counts[r] * es, false);
        recv[r] = base + (uint64_t(16 + r) << 32);
        reg(recv[r], total * es, true);
    }
    g_gather_pieces.clear();
    g_touch_launches = 0;
    expect(dt_all_gather(send, recv, p, counts, 0, DT_BFLOAT16, nullptr), DT_OK, "big all_gather");
    CHECK(g_touch_launches > 1, "big all_gather: %d read passes", g_touch_launches);
    uint64_t at = 0;  // destination offset of rank r's piece
    for (int r = 0; r < p; r++) {
        const char* s0 = static_cast<const char*>(send[r]);
        uint64_t covered = 0;
        for (const GatherPiece& g : g_gather_pieces) {
            if (!s0 || g.src < s0 || g.src >= s0 + counts[r] * es) continue;
            CHECK(g.src == s0 + covered, "big all_gather: rank %d piece out of order", r);
            CHECK(g.dst0 == static_cast<const char*>(recv[0]) + at + covered, "big all_gather: rank %d offset", r);
            covered += g.bytes;
        }
        CHECK(covered == counts[r] * es, "big all_gather: rank %d covered %llu of %llu bytes", r,
              (unsigned long long)covered, (unsigned long long)(counts[r] * es));
        at += counts[r] * es;
    }
    // a large broadcast goes through the same windows
    g_touch_launches = 0;
    void* out[p];
    for (int q = 0; q < p; q++) out[q] = recv[q];
    const size_t root_count = size_t(150) << 20;  // 300 MiB of bf16
    const char* root = base + (uint64_t(40) << 32);
    reg(root, root_count * es, false);
    expect(dt_broadcast(root, out, p, root_count, DT_BFLOAT16, nullptr), DT_OK, "big broadcast");
    CHECK(g_touch_launches > 1, "big broadcast: %d read passes", g_touch_launches);
    g_bufs.clear();
}

// The two-shot AllReduce (P >= 16 from 16 MiB per rank, P = 8-15 at 24-256
// MiB, P = 5-7 at 32-256 MiB, P = 4 at 128-192 MiB) and, beyond that (P >=
// 16 above 256 MiB in 64 MiB windows, P = 5-15 above 256 MiB in 128 MiB
// windows), window by window: fake device ranges.  For every case, rank 0's
// output is written exactly once (ReduceScatter chunk 0, fan-outs of the
// other chunks, one-shot tails), each fan-out piece copies a range of rank
// r's own output to the same offset of output 0, and the number of two-shot
// windows (ReduceScatter launches) is the expected one.
namespace dt {
extern int g_rs_launches;
}
void two_shot() {
    using dt::g_gather_pieces;
    using dt::GatherPiece;
    struct Case {
        int p;
        dt_dtype dtype;
        size_t count;
        bool in_place;
        int windows;     // two-shot windows expected (0: one-shot only)
        size_t skew = 0; // bytes past a 4 KiB boundary, the same for every buffer: a peeled head
        size_t send_skew = SIZE_MAX;  // the inputs' own offset (default: skew)
        size_t rank_step = 0;         // rank r's buffers a further r * rank_step bytes in
        int grid = 0;                 // line-grid ReduceScatter launches expected
    };
    const size_t M = size_t(1) << 20;
    const Case cases[] = {
        {8, DT_BFLOAT16, 64 * M, false, 1},           // 128 MiB per rank
        {8, DT_BFLOAT16, 64 * M, true, 1},
        {8, DT_BFLOAT16, 12 * M, false, 1},           // 24 MiB: the lower edge at P=8
        {8, DT_BFLOAT16, 12 * M - 64, false, 0},      // just below it
        {8, DT_FLOAT32, 64 * M, false, 1},            // 256 MiB: the upper edge at P=8
        {8, DT_FLOAT32, 64 * M + 32, false, 2},       // beyond it: two 128 MiB windows and a one-shot tail
        {8, DT_BFLOAT16, 192 * M, true, 3},           // 384 MiB in place: three windows
        {16, DT_FLOAT32, 3 * M, false, 1},            // 12 MiB: the lower edge at P=16
        {16, DT_FLOAT32, 3 * M - 64, false, 0},       // just below it
        {16, DT_FLOAT32, 4 * M, false, 1},            // 16 MiB
        {12, DT_FLOAT32, 4 * M, false, 1},            // 16 MiB: the lower edge at P=11-15
        {12, DT_FLOAT32, 4 * M - 64, false, 0},       // just below it
        {10, DT_FLOAT32, 4 * M, false, 0},            // 16 MiB at P=10: one-shot
        {11, DT_BFLOAT16, 8 * M, false, 1},           // 16 MiB at P=11
        {16, DT_FLOAT32, 8 * M, false, 1},            // 32 MiB
        {16, DT_FLOAT32, 64 * M, true, 1},            // 256 MiB: still one call
        {16, DT_FLOAT32, 96 * M + 64, false, 6},      // 384 MiB + 256 B: six 64 MiB windows and a one-shot tail
        {16, DT_FLOAT32, 80 * M + 4096, true, 5},     // 320 MiB + 16 KiB: five windows and a one-shot tail
        {12, DT_INT32, 48 * M, false, 1},             // 192 MiB
        {12, DT_INT32, 72 * M, false, 3},             // 288 MiB at P=12: windows of whole vectors per chunk
        {12, DT_BFLOAT16, 200 * M + 96, false, 4},    // 400 MiB + 192 B at P=12: three windows, a two-shot 16 MiB tail
        {8, DT_BFLOAT16, 64 * M + 8, false, 1},       // not a multiple of P vectors: a shorter last chunk
        {12, DT_FLOAT32, 48 * M + 4, false, 1},       // 192 MiB + 16 B at P=12: chunks of whole 1 KiB tiles
        {8, DT_BFLOAT16, 64 * M + 4, false, 1},       // not a whole number of vectors: two-shot, an element tail
        {8, DT_BFLOAT16, 12 * M + 3, false, 1},       // 24 MiB + 6 B
        {4, DT_FLOAT32, 32 * M, false, 1},            // 128 MiB at P=4
        {4, DT_FLOAT32, 48 * M, true, 1},             // 192 MiB at P=4
        {4, DT_FLOAT32, 16 * M, false, 0},            // 64 MiB at P=4
        {4, DT_FLOAT32, 48 * M + 16, false, 0},       // just beyond 192 MiB at P=4: one-shot
        {4, DT_FLOAT32, 64 * M, false, 0},            // 256 MiB at P=4: one-shot, no windows
        {2, DT_FLOAT32, 32 * M, false, 0},            // P=2
        {6, DT_FLOAT32, 48 * M, false, 1},            // 192 MiB at P=6: two-shot
        {6, DT_FLOAT32, 4 * M, false, 0},             // 16 MiB at P=6: one-shot
        {7, DT_FLOAT32, 96 * M + 4, false, 3},        // 384 MiB + 16 B at P=7: three 128 MiB windows, a one-shot tail
        {8, DT_BFLOAT16, 64 * M, false, 1, 2},        // 2 bytes off: a 4094-byte head, a ragged end, one element launch
        {8, DT_BFLOAT16, 64 * M + 3, true, 1, 130},   // in place, 130 bytes off
        {16, DT_FLOAT32, 96 * M + 64, false, 6, 12},  // windows after a peeled head
        {5, DT_INT32, 40 * M, false, 1, 1028},        // 1028 bytes off: the 4 KiB grain
        {8, DT_BFLOAT16, 64 * M, false, 1, 512},      // line-aligned, 512 bytes into a 1 KiB tile: a 1 KiB peel
        {16, DT_FLOAT32, 96 * M, true, 6, 256},       // the same before windows, in place
        {4, DT_FLOAT32, 16 * M, false, 0, 512},       // one-shot: no peel for line-aligned buffers
        // offsets that differ between inputs and outputs or between ranks:
        // the line-grid two-shot form from P * S = 256 MiB, window by window
        {8, DT_BFLOAT16, 16 * M + 5, false, 0, 0, 2, 0, 1},       // inputs 2 bytes off, 32 MiB + 10 B
        {8, DT_BFLOAT16, 10 * M, false, 0, 0, 2, 0, 1},           // P * S = 160 MiB: the edge at P = 6-12
        {8, DT_BFLOAT16, 10 * M - 8, false, 0, 0, 2, 0, 0},       // just below: the element kernel
        {12, DT_BFLOAT16, 6 * M + 3, false, 0, 0, 2, 0, 0},       // P=12, 144 MiB: the element kernel
        {6, DT_FLOAT32, 7 * M, false, 0, 0, 4, 0, 1},             // P=6, 168 MiB
        {4, DT_FLOAT32, 12 * M, false, 0, 0, 4, 0, 0},            // P=4, 192 MiB: the element kernel
        {4, DT_FLOAT32, 16 * M, false, 0, 0, 4, 0, 1},            // P=4, 256 MiB
        {16, DT_FLOAT32, 3 * M, false, 0, 0, 4, 0, 0},            // P=16, 192 MiB: the element kernel
        {16, DT_FLOAT32, 16 * M + 3, false, 0, 4, 0, 0, 1},       // outputs 4 bytes off
        {3, DT_BFLOAT16, 48 * M + 1, true, 0, 0, 0, 2, 1},        // in place, rank r 2r bytes off
        {5, DT_INT32, 16 * M + 7, false, 0, 16, 8, 4, 1},         // every buffer at an offset of its own
        {8, DT_BFLOAT16, 160 * M + 3, false, 0, 2, 0, 0, 3},      // 320 MiB: three 128 MiB windows
        // vector-aligned inputs 16 bytes off their lines: the line grid where
        // the two-shot form pays and P * S >= 256 MiB, else the vector forms
        {8, DT_BFLOAT16, 64 * M, false, 0, 0, 16, 0, 1},          // 128 MiB per rank
        {16, DT_FLOAT32, 4 * M, false, 0, 0, 16, 0, 1},           // 16 MiB at P=16: P * S = 256 MiB
        {16, DT_FLOAT32, 3 * M, false, 1, 0, 16, 0, 0},           // 12 MiB at P=16: the vector two-shot
        {8, DT_BFLOAT16, 160 * M, false, 0, 0, 16, 0, 3},         // 320 MiB: three windows on the grid
        {4, DT_FLOAT32, 16 * M, false, 0, 0, 16, 0, 0},           // 64 MiB at P=4: one-shot
    };
    char* base = reinterpret_cast<char*>(uintptr_t(1) << 45);  // fake, never dereferenced
    for (const Case& c : cases) {
        g_bufs.clear();
        const size_t es = esize(c.dtype), bytes = c.count * es;
        const void* send[16];
        void* recv[16];
        const size_t send_skew = c.send_skew == SIZE_MAX ? c.skew : c.send_skew;
        for (int r = 0; r < c.p; r++) {
            recv[r] = base + (uint64_t(r) << 33) + c.skew + r * c.rank_step;
            reg(recv[r], bytes, true);
            if (c.in_place) {
                send[r] = recv[r];
            } else {
                send[r] = base + (uint64_t(32 + r) << 33) + send_skew + r * c.rank_step;
                reg(send[r], bytes, false);
            }
        }
        g_gather_pieces.clear();
        dt::g_rs_launches = 0;
        dt::g_grid_rs_launches = 0;
        dt::g_fold_log.clear();
        dt::g_log_folds = true;
        expect(dt_allreduce(send, recv, c.p, c.count, c.dtype, DT_SUM, nullptr), DT_OK, "two-shot allreduce");
        dt::g_log_folds = false;
        CHECK(dt::g_rs_launches == c.windows, "allreduce of %zu bytes per rank at P=%d: %d two-shot windows, expected %d",
              bytes, c.p, dt::g_rs_launches, c.windows);
        CHECK(dt::g_grid_rs_launches == c.grid, "allreduce of %zu bytes per rank at P=%d: %d line-grid launches, expected %d",
              bytes, c.p, dt::g_grid_rs_launches, c.grid);
        if (c.windows == 0 && c.grid == 0) CHECK(g_gather_pieces.empty(), "one-shot allreduce with a fan-out");
        // every fan-out piece: a range of rank r's own output, copied to the same offset of output 0
        for (const GatherPiece& g : g_gather_pieces) {
            int owner = -1;
            for (int r = 0; r < c.p; r++)
                if (g.src >= static_cast<const char*>(recv[r]) && g.src < static_cast<const char*>(recv[r]) + bytes)
                    owner = r;
            CHECK(owner >= 0, "two-shot allreduce: a fan-out source outside the outputs");
            const uint64_t off = uint64_t(g.src - static_cast<const char*>(recv[owner]));
            CHECK(g.dst0 == static_cast<const char*>(recv[0]) + off, "two-shot allreduce: fan-out piece moved");
        }
        // rank 0's output: written exactly once, no gap, no overlap
        std::vector<std::pair<const char*, uint64_t>> w = dt::g_fold_log;
        std::sort(w.begin(), w.end());
        uint64_t at = 0;
        const char* r0 = static_cast<const char*>(recv[0]);
        for (const auto& e : w) {
            CHECK(e.first == r0 + at, "allreduce: output 0 written at +%lld, expected +%llu", (long long)(e.first - r0),
                  (unsigned long long)at);
            at += e.second;
        }
        CHECK(at == bytes, "allreduce: output 0 covered %llu of %llu bytes", (unsigned long long)at,
              (unsigned long long)bytes);
    }
    g_bufs.clear();
}

// ReduceScatters whose buffers share no offset, with the grid each should
// take: the inputs' lines when the inputs share one offset and every
// chunk's output starts at most 16 bytes before a line of its grid, else the
// outputs' lines.  Chunk strides off the lines make the input offset differ
// from chunk to chunk.
void grid_reduce_scatter() {
    struct Case {
        int p;
        dt_dtype dtype;
        size_t recvcount;
        size_t send_skew[4];
        size_t recv_skew[4];
    };
    const Case cases[] = {
        // bf16, 2000-byte chunks (80 mod 128): inputs 2 bytes off, outputs 2 bytes before each chunk's input line
        {4, DT_BFLOAT16, 1000, {2, 2, 2, 2}, {0, 80, 32, 112}},
        // the outputs 4 bytes past each chunk's input offset instead
        {4, DT_BFLOAT16, 1000, {2, 2, 2, 2}, {6, 86, 38, 118}},
        // fp32, inputs at two offsets (4000-byte chunks, 32 mod 128), outputs on their chunks' lines
        {2, DT_FLOAT32, 1000, {0, 4}, {0, 32}},
        // fp32, inputs 8 bytes off, outputs aligned, chunks of whole lines: 120 bytes into a line
        {3, DT_FLOAT32, 4096 * 3, {8, 8, 8}, {0, 0, 0}},
        // the same with chunks 20 bytes past whole lines: later chunks' outputs fall inside lines
        {3, DT_FLOAT32, 4096 * 3 + 5, {8, 8, 8}, {0, 0, 0}},
        // vector-aligned inputs 16 bytes off their lines: the grid, not the vector kernel
        {2, DT_FLOAT32, 4096, {16, 16}, {0, 0}},
        // aligned buffers, chunks of 4000 bytes: later chunks' inputs off their lines
        {2, DT_FLOAT32, 1000, {0, 0}, {0, 0}},
    };
    char* base = reinterpret_cast<char*>(uintptr_t(5) << 44);  // fake, never dereferenced
    for (const Case& c : cases) {
        g_bufs.clear();
        const size_t es = esize(c.dtype);
        const void* send[4];
        void* recv[4];
        for (int r = 0; r < c.p; r++) {
            send[r] = base + (uint64_t(r) << 33) + c.send_skew[r];
            reg(send[r], c.p * c.recvcount * es, false);
            recv[r] = base + (uint64_t(16 + r) << 33) + c.recv_skew[r];
            reg(recv[r], c.recvcount * es, true);
        }
        const int before = dt::g_grid_rs_launches;
        expect(dt_reduce_scatter(send, recv, c.p, c.recvcount, c.dtype, DT_SUM, nullptr), DT_OK,
               "reduce_scatter over line grids");
        CHECK(dt::g_grid_rs_launches == before + 1, "reduce_scatter P=%d: %d grid launches, expected one", c.p,
              dt::g_grid_rs_launches - before);
    }
    g_bufs.clear();
}

int main() {
    validation();
    overlaps();
    big_fan_out();
    two_shot();
    grid_reduce_scatter();
    dt::g_grid_rs_launches = 0;
    reductions();
    // the random reductions reach the line-grid ReduceScatter (buffers at
    // offsets of their own)
    CHECK(dt::g_grid_rs_launches >= 20, "the line-grid ReduceScatter ran %d times", dt::g_grid_rs_launches);
    copies();
    buckets();
    bucket_big();
    hsdp_and_sync();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("ok %ld\n", g_launches);
    return 0;
}
