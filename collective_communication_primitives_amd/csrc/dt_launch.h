// dt_launch.h -- kernel argument blocks and launchers (host side), shared by
// the kernel sources and the C ABI in api.cpp.  Every argument block is
// passed by value and stays below 4 KiB, so no device-side tables are
// needed and the library allocates nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dt {

constexpr int kMaxRanksHost = 16;

// AllReduce / ReduceScatter over one contiguous range per rank.
struct ReduceArgs {
    const void* src[kMaxRanksHost];
    void* dst[kMaxRanksHost];
    uint64_t first;        // first element handled by this launch (element path)
    uint64_t count;        // elements per chunk handled by this launch (vector path: vectors)
    uint64_t first2;       // element path: a second range [first2, first2 + count2) in the same
    uint64_t count2;       //   launch (a misaligned buffer's head and ragged tail together)
    uint64_t last_count;   // vector ReduceScatter: vectors of the last chunk (<= count)
    uint64_t chunk_stride; // vector ReduceScatter: vectors between chunk starts in each input (>= count)
    uint64_t chunk_elems;  // ReduceScatter: elements per output chunk
    int nranks;
    int rs;                // 1: ReduceScatter (grid.y = chunk), 0: AllReduce
};

// ReduceScatter over a 128-byte line grid, for element-aligned buffers that
// share no offset (the vector kernels need every buffer 16-byte aligned, or
// all at one offset).  Chunk c is elements [c * in_stride, c * in_stride +
// n_c) of every input, n_c = count for every chunk but the last
// (last_count); it goes to dst[c].  The tiles follow each output's lines:
// lead[c] = dst[c] & (kGridAlign - 1).
struct GridFoldArgs {
    const void* src[kMaxRanksHost];
    void* dst[kMaxRanksHost];
    uint32_t lead[kMaxRanksHost];
    uint64_t in_stride;
    uint64_t count;
    uint64_t last_count;
    int nranks;
    int nchunks;
};
// The AllReduce's grid two-shot form cuts its chunks in whole KiB, so every
// chunk of a buffer sits at that buffer's offset within a line.
constexpr uint64_t kGridChunkGrain = 1024;

// Multi-tensor pieces of one bucket.  Piece k of rank r starts at
// ptr[k*nranks + r]; ws[r] + wpos[k] is its place in rank r's bucket buffer.
constexpr int kPiecePtrs = 320;
constexpr int kMaxPieces = 32;
struct PieceArgs {
    void* ptr[kPiecePtrs];
    void* ws[kMaxRanksHost];
    uint64_t len[kMaxPieces];
    uint64_t wpos[kMaxPieces];
    uint32_t tile_start[kMaxPieces + 1];
    uint32_t aligned;      // bit k: piece k may use 16-byte vectors
    int npieces;
    int nranks;
};

// Coalesced AllReduce of many separate tensors in one launch (in place).
// Piece k of rank r starts at ptr[k*nranks + r].  The table travels in the
// kernel arguments (about 39 KiB; launches with up to 64 KB of arguments
// were verified on gfx950 with ROCm 7.2).
constexpr int kCoalPtrs = 4096;
constexpr int kCoalMaxPieces = 512;
struct CoalescedArgs {
    void* ptr[kCoalPtrs];
    void* ws[kMaxRanksHost];          // bucket buffers (flatten / unflatten only)
    uint64_t len[kCoalMaxPieces];
    uint64_t wpos[kCoalMaxPieces];    // element position inside the bucket buffer
    uint32_t tile_start[kCoalMaxPieces + 1];
    uint32_t aligned[kCoalMaxPieces / 32];
    int npieces;
    int nranks;
};

// Several independent ReduceScatters in one launch (one per segment, all of
// nranks members): segment k's member j reads src[k*nranks + j] (nranks*m[k]
// elements) and writes chunk j of the fold to dst[k*nranks + j] (m[k]).
constexpr int kSegPtrs = 160;
constexpr int kMaxSegs = 32;
struct SegReduceScatterArgs {
    const void* src[kSegPtrs];
    void* dst[kSegPtrs];
    uint64_t m[kMaxSegs];
    uint32_t tile_start[kMaxSegs + 1];
    uint32_t tiles_per_chunk[kMaxSegs];
    uint32_t aligned;      // bit k: segment k may use 16-byte vectors
    int nsegs;
    int nranks;
};

// Fan-out copy (AllGather, AllGatherIntoVec, Broadcast): rank r's bytes
// [0, bytes[r]) are written to dst[r*nranks + q] for every q.
struct GatherArgs {
    const void* src[kMaxRanksHost];
    void* dst[kMaxRanksHost * kMaxRanksHost];
    uint64_t bytes[kMaxRanksHost];
    uint32_t tile_start[kMaxRanksHost + 1];
    uint32_t aligned;      // bit r: rank r's source is 16-byte aligned and every destination
                           // starts on a 128-byte line; tiles follow the source
    uint32_t shifted;      // bit r (not aligned): rank r's destinations share one offset within a
                           // 128-byte line; its tiles then follow their grid (grid_tiles)
    uint32_t lead[kMaxRanksHost];  // shifted piece r: bits 0-15 the grid bytes before its first byte
                                   // (the destinations' offset within the grid's grain), bits 16-19
                                   // the source's offset within a vector at the grid's vector starts
    uint32_t tile_bytes;   // kGatherTileBytes or kGatherWaveTileBytes: the launch's workgroup shape
    uint32_t split_log2;   // each source tile's destinations go to 2^split_log2 workgroups (q mod 2^s)
    int nranks;
};

// Tiles of a copy whose destination does not start on a 128-byte line: the
// tiles cover a grid that starts at the line holding the destination's first
// byte, md = dst & (kGridAlign - 1) bytes before it, so that no line is
// written by two workgroups, and every interior 16-byte vector is one aligned
// store, built from aligned loads of the source (funnel16).  Stores that start
// off the lines are costly even when 16-byte aligned: a fan-out to
// destinations 16 or 32 bytes past a line ran 1.7x slower than on the line
// grid (P=8 bf16, 24 MiB pieces, 444 against 282 us).
constexpr uint64_t kGridAlign = 128;
inline uint64_t grid_tiles(uint64_t bytes, uint64_t md, uint64_t tile_bytes) {
    return (md + bytes + tile_bytes - 1) / tile_bytes;
}

// 1:1 copies of independent byte ranges (ReplicateToShard and other
// per-rank copies): segment k copies bytes[k] from src[k] to dst[k].
constexpr int kMaxCopySegs = 64;
struct SegCopyArgs {
    const void* src[kMaxCopySegs];
    void* dst[kMaxCopySegs];
    uint64_t bytes[kMaxCopySegs];
    uint32_t tile_start[kMaxCopySegs + 1];
    uint64_t aligned;      // bit k: segment k allows 16-byte vectors
    int nsegs;
};

// AllToAll between shard dimensions of a row-major [rows, cols] tensor.
// Every exchange is a set of runs of cp = cols/P contiguous elements:
//   dir 0 (Shard(0) -> Shard(1)): run k = (j, a), j = k / rows, a = k % rows:
//     x_{a/rp} + ((a % rp) * cols + j * cp)  ->  y_j + a * cp
//   dir 1 (Shard(1) -> Shard(0)): run k = (j, a, i), j = k / (rp*P),
//     a = (k / P) % rp, i = k % P:
//     x_i + (j * rp + a) * cp  ->  y_j + a * cols + i * cp
// A workgroup copies runs_per_block whole runs, or one 1/tiles_per_run
// slice of a long run.
struct DimsArgs {
    const void* src[kMaxRanksHost];
    void* dst[kMaxRanksHost];
    uint64_t rows, cols, rp, cp;   // elements
    uint32_t esize;
    uint32_t runs_per_block;       // >= 1
    uint32_t tiles_per_run;        // >= 1 (only one of the two exceeds 1)
    uint32_t vec;                  // 1: runs and bases allow 16-byte vectors
    uint32_t elems;                // 1 (vec 0): every base element-aligned, so runs copy whole elements
    uint32_t wave;                 // 1: one kDimsWaveTileBytes slice of one run per single-wave workgroup
    uint64_t nruns;
    int nranks;
    int dir;
};

// AllToAll: block k of a launch copies bytes[k] from `from[k]` to `to[k]`.
// The blocks are the non-empty i -> j blocks of the split matrix in (i, j)
// order, with their byte offsets resolved on the host; kA2ABlocks covers a
// full 16 x 16 matrix, so one launch serves any rank count.
// A workgroup finds its block in two rounds: group_start[g] = tile_start[16 g]
// gives the group of sixteen blocks, then that group's sixteen starts give the
// block.  Entries past the last block hold UINT32_MAX (after tile_start
// [nblocks], the tile total), so no comparison needs a bound.
constexpr int kA2ABlocks = kMaxRanksHost * kMaxRanksHost;
constexpr int kA2AGroup = 16;
struct AllToAllArgs {
    const void* from[kA2ABlocks];
    void* to[kA2ABlocks];
    uint64_t bytes[kA2ABlocks];
    uint32_t tile_start[kA2ABlocks + 1];
    uint32_t group_start[kA2ABlocks / kA2AGroup];
    uint64_t aligned[kA2ABlocks / 64];  // bit k: block k allows 16-byte vectors
    int nblocks;
};

struct BarrierArgs {
    int32_t* win[kMaxRanksHost];
    int32_t* status;
    uint64_t timeout_ticks;  // wall-clock ticks per wait
    int nranks;
    int first_generation;
    int generations;
};

struct ExchangeArgs {
    BarrierArgs bar;
    const void* src[kMaxRanksHost];
    void* stage[kMaxRanksHost];
    void* dst[kMaxRanksHost];
    uint64_t nbytes;
};

// Tile sizes (bytes of one rank's data per workgroup).
constexpr uint64_t kCopyTileBytes = 1024;    // all-to-all: one wave, one vector per thread
// Gather (fan-out) tiles, one vector per thread: single-wave workgroups (1
// KiB source tiles) for a direct fan-out of at most kGatherWaveBytes of
// sources; 128-thread workgroups (2 KiB) for a larger direct one, for the
// windows of a large one and for their read passes.
constexpr int kGatherU = 1;
constexpr int kGatherBlock = 128;
constexpr uint64_t kGatherTileBytes = uint64_t(kGatherU) * kGatherBlock * 16;
constexpr int kGatherWaveBlock = 64;
constexpr uint64_t kGatherWaveTileBytes = uint64_t(kGatherU) * kGatherWaveBlock * 16;
constexpr uint64_t kGatherWaveBytes = 128ull << 20;
constexpr uint64_t kPieceTileVecs = 512;     // bucket pieces: 512 x 16 B

// Launchers: return the HIP error of the launch.  dtype/op are the dt_dtype /
// dt_op enum values.  `vector` selects the 16-byte path (caller checked
// alignment and divisibility).
hipError_t launch_reduce_vec(const ReduceArgs& a, int dtype, int op, hipStream_t s);
hipError_t launch_reduce_elems(const ReduceArgs& a, int dtype, int op, hipStream_t s);
hipError_t launch_reduce_scatter_grid(const GridFoldArgs& a, int dtype, int op, hipStream_t s);
hipError_t launch_reduce_pieces(const PieceArgs& a, int dtype, int op, hipStream_t s);
hipError_t launch_reduce_coalesced(const CoalescedArgs& a, int dtype, int op, hipStream_t s);
hipError_t launch_copy_coalesced(const CoalescedArgs& a, int esize, int to_ws, hipStream_t s);
hipError_t launch_reduce_scatter_segs(const SegReduceScatterArgs& a, int dtype, int op, hipStream_t s);
// Output vectors per workgroup tile of the segmented ReduceScatter for P ranks.
uint64_t seg_rs_tile_vecs(int nranks);
hipError_t launch_copy_pieces(const PieceArgs& a, int esize, int to_ws, hipStream_t s);
// The table counts kGatherTileBytes tiles.
hipError_t launch_gather(const GatherArgs& a, uint32_t tiles, hipStream_t s);
// Read pass over the gather's source tiles (plain loads, nothing stored).
hipError_t launch_gather_touch(const GatherArgs& a, uint32_t tiles, hipStream_t s);
constexpr uint64_t kFanOutDirectBytes = 256ull << 20;  // sources up to this size: one launch
constexpr uint64_t kFanOutWindowBytes = 128ull << 20;   // larger sources: windows of this size
hipError_t launch_all_to_all(const AllToAllArgs& a, uint32_t tiles, hipStream_t s);
hipError_t launch_copy_segments(const SegCopyArgs& a, hipStream_t s);
hipError_t launch_all_to_all_dims(const DimsArgs& a, uint32_t blocks, hipStream_t s);
constexpr uint64_t kSegCopyTileBytes = 1024;
constexpr uint64_t kDimsTileBytes = 16384;
constexpr uint32_t kDimsMaxRunsPerBlock = 64;
constexpr uint64_t kDimsWaveTileBytes = 1024;  // the single-wave path: 64 lanes x 16 bytes
// The static staging buffer of the allocation-free bucket AllReduce
// (scratch.hip): its device address on the current device, looked up once per
// device.  kScratchBytes holds eight ranks' 25 MiB buckets (or sixteen of 16 MiB).
constexpr uint64_t kScratchBytes = 256ull << 20;
hipError_t scratch_base(void** ptr);
hipError_t launch_barrier(const BarrierArgs& a, int spread, hipStream_t s);
hipError_t launch_exchange(const ExchangeArgs& a, int spread, hipStream_t s);

}  // namespace dt
