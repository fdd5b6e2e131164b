// copy.hip -- the gather and all-to-all copy engines.
//
// Both are byte copies driven by an offset table carried in the kernel
// arguments (no device-side tables).  The work is cut into 1 or 2 KiB (gather)
// or 1 KiB (all-to-all) tiles of source data; one workgroup copies one tile, so
// uneven pieces (1 row or 16384 rows, an empty all-to-all block or a 4096-row
// one) balance across the whole chip.  A workgroup finds its piece from an
// exclusive prefix sum of tile counts: a linear scan over at most 16 ranks for
// the gather, a two-level batched lookup over at most 256 non-empty blocks
// for the all-to-all.
//
// AllGather fans out: each source tile is read once and written to every
// rank's output, (1 + P) bytes of HBM traffic per gathered byte.  Stores go
// out as whole 128-byte lines of the destinations: destinations that do not
// start on a line (even at a 16-byte boundary) take tiles over their line
// grid, each vector built from aligned loads of the source; destinations
// that share no offset within a line each take their own grid, their
// vectors shifted out of the source lines staged in LDS.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

// The all-to-all copies 1 KiB tiles with single-wave workgroups: in-process A/B
// 3.7-3.9% faster than 4 KiB tiles of 256 threads (and than 2 KiB of 128)
// on three split matrices at P=8 and P=16.
constexpr int kA2AThreads = 64;
constexpr int kCopyU = int(kCopyTileBytes / 16 / kA2AThreads);  // 16-byte vectors per thread per tile
static_assert(kCopyU >= 1, "an all-to-all tile holds at least one vector per thread");

// PMAX bounds the rank count; EXACT (P == PMAX) unrolls the P destination
// stores.  A tile is U vectors per thread of BLOCK threads of one rank's
// source.
template <int PMAX, bool EXACT, int U, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_gather(GatherArgs a) {
    constexpr uint64_t kTile = uint64_t(U) * BLOCK * 16;
    // 2^split_log2 workgroups share one source tile, each writing the
    // destinations q with q mod 2^split_log2 == its part
    const uint32_t b = blockIdx.x >> a.split_log2;
    const int part = int(blockIdx.x & ((1u << a.split_log2) - 1u));
    const int nparts = 1 << a.split_log2;
    const int nr = EXACT ? PMAX : a.nranks;
    int r = 0;
    while (r + 1 < nr && a.tile_start[r + 1] <= b) r++;
    const char* src = static_cast<const char*>(a.src[r]);
    void* const* dsts = a.dst + r * nr;
    const uint64_t b0 = uint64_t(b - a.tile_start[r]) * kTile;
    const uint64_t b1 = min(a.bytes[r], b0 + kTile);
    if ((a.aligned >> r) & 1u) {
        const uint64_t v1 = b1 / 16;
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * BLOCK;
            if (v < v1) x[u] = load16_h<false>(src + v * 16);  // writes dominate 1:P
        }
        // Buffer stores, non-temporal with device scope, one resource per
        // destination over the tile's whole vectors (the range drops the lanes
        // past them; the ragged bytes go below).  In-process A/B against plain
        // non-temporal global stores: 1.4-4.3% faster on every fan-out workload
        // on two machines, and no slower at any of 13 output placements.
        const uint32_t vbytes = uint32_t(v1 * 16 - b0);
#pragma unroll
        for (int q = 0; q < PMAX; q++) {
            if (q < nr && (q & (nparts - 1)) == part && dsts[q] != src) {  // an in-place piece sits in its slot
                const rsrc_t out = make_rsrc(static_cast<char*>(dsts[q]) + b0, vbytes);
#pragma unroll
                for (int u = 0; u < U; u++) bstore16<kPolNT | kPolDevice>(out, (threadIdx.x + u * BLOCK) * 16, x[u]);
            }
        }
        const uint64_t t = v1 * 16 + threadIdx.x;  // ragged end: fewer than 16 bytes
        if (t < b1 && part == 0) {
            const char c = src[t];
            for (int q = 0; q < nr; q++)
                if (dsts[q] != src) static_cast<char*>(dsts[q])[t] = c;
        }
    } else if ((a.shifted >> r) & 1u) {
        // The destinations share one offset, `lead` bytes into their grid:
        // tile b covers bytes [b0, b0 + kTile) of the grid, grid byte g being
        // byte g - lead of the piece.  A grid vector inside the piece is
        // built from aligned loads of the source (the source sits sm bytes
        // into a vector at the grid's vector starts) and stored with one
        // aligned store to each destination of this part; the partial
        // vectors at the piece's two ends are loaded through a window over
        // the piece and stored byte by byte, in part 0, their loads all
        // issued before any store.  Both offsets come from the host, so the
        // first load waits on no destination pointer.
        const uint32_t lead = a.lead[r] & 0xFFFFu;
        const uint32_t sm = a.lead[r] >> 16;
        const int64_t bytes = int64_t(a.bytes[r]);
        u32x4 x[U];
        bool full[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t p0 = int64_t(b0) + int64_t(threadIdx.x + u * BLOCK) * 16 - int64_t(lead);
            full[u] = p0 >= 0 && p0 + 16 <= bytes;
            if (full[u]) x[u] = load16_any<false>(src + p0, sm);
        }
#pragma unroll
        for (int q = 0; q < PMAX; q++) {
            if (q < nr && (q & (nparts - 1)) == part && dsts[q] != src) {
                // the aligned path's stores, addressed from the tile's grid start
                const rsrc_t out = make_rsrc(static_cast<char*>(dsts[q]) - lead + b0, uint32_t(kTile));
#pragma unroll
                for (int u = 0; u < U; u++)
                    if (full[u]) bstore16<kPolNT | kPolDevice>(out, (threadIdx.x + u * BLOCK) * 16, x[u]);
            }
        }
        if (part == 0 && (int64_t(b0) < int64_t(lead) || int64_t(b0) - lead + int64_t(kTile) > bytes)) {
            // a tile at one of the piece's ends: its partial vectors, loaded
            // through a window over the piece, stored byte by byte
            const LoadWindow w = load_window(src, bytes, int64_t(b0) - lead - sm, int64_t(kTile) + 16);
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t p0 = int64_t(b0) + int64_t(threadIdx.x + u * BLOCK) * 16 - int64_t(lead);
                if (full[u] || p0 + 16 <= 0 || p0 >= bytes) continue;
                const u32x4 y = window_load_shifted<0>(w, p0 - int64_t(sm), sm);
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    if (p0 + j < 0 || p0 + j >= bytes) continue;
                    const char c = vec_byte(y, j);
                    for (int q = 0; q < nr; q++)
                        if (dsts[q] != src) static_cast<char*>(dsts[q])[p0 + j] = c;
                }
            }
        }
    } else {
        // Destinations at offsets of their own: each destination q tiles over
        // its own line grid, tile b covering bytes [b0, b0 + kTile) of it,
        // grid byte g being byte g - lead_q of the piece (lead_q = dsts[q]
        // mod 128, so the host counts tiles for a lead of 127).  The piece
        // bytes that any destination's tile b needs lie in [b0 - 127, b0 +
        // kTile): the workgroup stages them once in LDS as aligned source
        // vectors (through a window over the piece: nothing outside its
        // aligned vectors is read), then each lane builds its vector for each
        // destination of this part from two LDS vectors and one byte shift
        // (uniform per destination) and stores it aligned, whole lines of
        // the destination, or at the piece's two ends byte by byte.  The
        // stage starts sm bytes before a vector boundary of the source, at
        // piece byte b0 - 128 - sm, so the loads are aligned.
        constexpr int V = U * BLOCK;  // vectors per tile
        constexpr int SV = V + 9;     // staged: piece bytes [b0 - 128 - sm, b0 + kTile + 16 - sm)
        __shared__ u32x4 stage[SV];
        const uint32_t sm = uint32_t(reinterpret_cast<uintptr_t>(src) & 15u);
        const int64_t bytes = int64_t(a.bytes[r]);
        const int64_t s_lo = int64_t(b0) - 128 - int64_t(sm);
        const LoadWindow w = load_window(src, bytes, s_lo, int64_t(SV) * 16);
        u32x4 y[U + 1];
#pragma unroll
        for (int u = 0; u <= U; u++) {
            const int i = int(threadIdx.x) + u * BLOCK;
            if (i < SV) y[u] = window_load<0>(w, s_lo + int64_t(i) * 16);
        }
#pragma unroll
        for (int u = 0; u <= U; u++) {
            const int i = int(threadIdx.x) + u * BLOCK;
            if (i < SV) stage[i] = y[u];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PMAX; q++) {
            if (!(q < nr && (q & (nparts - 1)) == part && dsts[q] != src)) continue;
            char* d = static_cast<char*>(dsts[q]);
            const int64_t lead = int64_t(reinterpret_cast<uintptr_t>(d) & uint64_t(kGridAlign - 1));
            const rsrc_t out = make_rsrc(d - lead + b0, uint32_t(kTile));
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int l = int(threadIdx.x) + u * BLOCK;
                const int64_t s0 = int64_t(b0) + int64_t(l) * 16 - lead;  // the piece byte of this grid vector
                if (s0 + 16 <= 0 || s0 >= bytes) continue;
                const uint32_t o = uint32_t(int64_t(l) * 16 - lead + 128 + int64_t(sm));  // 1 .. 16 V + 127
                const uint32_t s = o & 15u;
                const u32x4 lo = stage[o >> 4];
                const u32x4 x = s != 0 ? funnel16(lo, stage[(o >> 4) + 1], s) : lo;
                if (s0 >= 0 && s0 + 16 <= bytes) {
                    bstore16<kPolNT | kPolDevice>(out, uint32_t(l) * 16, x);
                } else {
#pragma unroll
                    for (int j = 0; j < 16; j++)
                        if (s0 + j >= 0 && s0 + j < bytes) d[s0 + j] = vec_byte(x, j);
                }
            }
        }
    }
}

// A 1:1 copy of `bytes` bytes from src to dst (dst not on a 128-byte line
// or src not 16-byte aligned), tile `tile` of TILE bytes over dst's line grid
// (grid_tiles), THREADS lanes with TILE / 16 / THREADS vectors each: a
// vector inside the copy is built from aligned loads of the source and
// stored aligned; the partial vectors at the copy's two ends are loaded
// through a window over the source (load_window) and stored byte by byte.
template <int THREADS, uint64_t TILE>
__device__ __forceinline__ void copy_shifted(const char* src, char* dst, uint64_t bytes, uint64_t tile) {
    constexpr int U = int(TILE / 16 / THREADS);
    const uint32_t md = uint32_t(reinterpret_cast<uintptr_t>(dst) & (kGridAlign - 1));
    const uint32_t sm = uint32_t((reinterpret_cast<uintptr_t>(src) - md) & 15u);
    const int64_t n = int64_t(bytes);
    const int64_t g0 = int64_t(tile * TILE) - int64_t(md);  // copy byte at the tile's grid start
    const rsrc_t out = make_rsrc(dst + g0, uint32_t(TILE));
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int64_t p0 = g0 + int64_t(threadIdx.x + u * THREADS) * 16;
        if (p0 >= 0 && p0 + 16 <= n)
            bstore16<kPolNT | kPolDevice>(out, (threadIdx.x + u * THREADS) * 16, load16_any<true>(src + p0, sm));
    }
    if (g0 >= 0 && g0 + int64_t(TILE) <= n) return;
    const LoadWindow w = load_window(src, n, g0 - int64_t(sm), int64_t(TILE) + 16);
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int64_t p0 = g0 + int64_t(threadIdx.x + u * THREADS) * 16;
        if ((p0 >= 0 && p0 + 16 <= n) || p0 + 16 <= 0 || p0 >= n) continue;
        const u32x4 x = window_load_shifted<kPolNT>(w, p0 - int64_t(sm), sm);
#pragma unroll
        for (int j = 0; j < 16; j++)
            if (p0 + j >= 0 && p0 + j < n) dst[p0 + j] = vec_byte(x, j);
    }
}

// Read pass over a gather table's source tiles: plain loads, which leave the
// bytes in the Infinity Cache for the fan-out launched right after.  The
// empty asm keeps the loads (each waits for its own, which a read pass can
// afford: it only has to touch the lines); nothing is stored.
__global__ __launch_bounds__(kGatherBlock) void k_gather_touch(GatherArgs a) {
    constexpr int U = kGatherU;
    constexpr uint64_t kTile = kGatherTileBytes;
    const uint32_t b = blockIdx.x;
    const int nr = a.nranks;
    int r = 0;
    while (r + 1 < nr && a.tile_start[r + 1] <= b) r++;
    const char* src = static_cast<const char*>(a.src[r]);
    const uint64_t b0 = uint64_t(b - a.tile_start[r]) * kTile;
    if ((a.aligned >> r) & 1u) {
        const uint64_t v1 = min(a.bytes[r], b0 + kTile) / 16;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kGatherBlock;
            if (v < v1) {
                const u32x4 x = load16_h<false>(src + v * 16);
                asm volatile("" ::"v"(x));
            }
        }
    } else if ((a.shifted >> r) & 1u) {
        // the same grid as k_gather: each lane reads the aligned source vector
        // holding the first byte its grid vector needs
        const uint32_t md = a.lead[r] & 0xFFFFu;
        const int64_t bytes = int64_t(a.bytes[r]);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t p0 = int64_t(b0) + int64_t(threadIdx.x + u * kGatherBlock) * 16 - int64_t(md);
            if (p0 + 16 > 0 && p0 < bytes) {
                const char* at = src + (p0 > 0 ? p0 : 0);
                const u32x4 x = load16_h<false>(at - (reinterpret_cast<uintptr_t>(at) & 15u));
                asm volatile("" ::"v"(x));
            }
        }
    }
}

// Block of tile b: the last k with tile_start[k] <= b (blocks are non-empty,
// so the starts increase, and padding entries never qualify), and that start.
// Two rounds of one batched scalar load each: the sixteen group starts, then
// the sixteen starts of the group.
__device__ __forceinline__ int a2a_block(const AllToAllArgs& a, uint32_t b, uint32_t& start) {
    constexpr int G = kA2AGroup;
    int g = 0;
#pragma unroll
    for (int k = 1; k < kA2ABlocks / G; k++) g += a.group_start[k] <= b ? 1 : 0;
    const int g0 = G * g;
    int s = g0;
    start = a.group_start[g];
#pragma unroll
    for (int j = 1; j < G; j++) {
        const uint32_t ts = a.tile_start[g0 + j];
        const bool in = ts <= b;
        s += in ? 1 : 0;
        start = in ? ts : start;
    }
    return s;
}

__global__ __launch_bounds__(kA2AThreads) void k_all_to_all(AllToAllArgs a) {
    const uint32_t b = blockIdx.x;
    uint32_t start;
    const int k = a2a_block(a, b, start);
    const char* src = static_cast<const char*>(a.from[k]);
    char* dst = static_cast<char*>(a.to[k]);
    const uint64_t b0 = uint64_t(b - start) * kCopyTileBytes;
    const uint64_t b1 = min(a.bytes[k], b0 + kCopyTileBytes);
    if ((a.aligned[k >> 6] >> (k & 63)) & 1ull) {
        const uint64_t v1 = b1 / 16;
        u32x4 x[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kA2AThreads;
            if (v < v1) x[u] = load16(src + v * 16);
        }
        // stores: buffer instructions, non-temporal with device scope, over the
        // tile's whole vectors (0.3-0.6% faster than non-temporal global stores)
        const rsrc_t out = make_rsrc(dst + b0, uint32_t(v1 * 16 - b0));
#pragma unroll
        for (int u = 0; u < kCopyU; u++) bstore16<kPolNT | kPolDevice>(out, (threadIdx.x + u * kA2AThreads) * 16, x[u]);
        const uint64_t t = v1 * 16 + threadIdx.x;
        if (t < b1) dst[t] = src[t];
    } else {
        copy_shifted<kA2AThreads, kCopyTileBytes>(src, dst, a.bytes[k], b - start);
    }
}

namespace {
template <int PMAX, int BLOCK>
hipError_t gather_pb(const GatherArgs& a, uint32_t tiles, hipStream_t s) {
    const uint32_t grid = tiles << a.split_log2;  // the host keeps tiles << split_log2 below 2^31
    if (a.nranks == PMAX)
        k_gather<PMAX, true, kGatherU, BLOCK><<<grid, BLOCK, 0, s>>>(a);
    else
        k_gather<PMAX, false, kGatherU, BLOCK><<<grid, BLOCK, 0, s>>>(a);
    return hipGetLastError();
}
// The two workgroup shapes, measured by in-process A/B over output placements
// on the MI355X: single waves fan out up to 128 MiB of sources 1-4% faster
// (the bench step's AllGather at six placements, the P=16 AllReduce's 64 MiB
// windows), 128 threads are 1% faster at 256 MiB and 4% faster in the windows
// of the uneven AllGather.
template <int PMAX>
hipError_t gather_p(const GatherArgs& a, uint32_t tiles, hipStream_t s) {
    return a.tile_bytes == kGatherWaveTileBytes ? gather_pb<PMAX, kGatherWaveBlock>(a, tiles, s)
                                                : gather_pb<PMAX, kGatherBlock>(a, tiles, s);
}
}  // namespace

// ------------------------------------------------------- segment copy --
// Independent 1:1 byte copies in 1 KiB tiles of single-wave workgroups
// (in-process A/B: 6-7% faster than 16 KiB tiles of 256 threads, for
// ReplicateToShard at 128 MiB and 1 GiB per rank); a workgroup finds its
// segment by binary search over the tile prefix.
constexpr int kSegCopyBlock = 64;
__global__ __launch_bounds__(kSegCopyBlock) void k_copy_segments(SegCopyArgs a) {
    constexpr int U = int(kSegCopyTileBytes / 16 / kSegCopyBlock);
    static_assert(U >= 1, "a segment-copy tile holds at least one vector per thread");
    const uint32_t b = blockIdx.x;
    int lo = 0, hi = a.nsegs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_start[mid] <= b) lo = mid;
        else hi = mid;
    }
    const int k = lo;
    const char* src = static_cast<const char*>(a.src[k]);
    char* dst = static_cast<char*>(a.dst[k]);
    const uint64_t b0 = uint64_t(b - a.tile_start[k]) * kSegCopyTileBytes;
    const uint64_t b1 = min(a.bytes[k], b0 + kSegCopyTileBytes);
    if ((a.aligned >> k) & 1ull) {
        const uint64_t v1 = b1 / 16;
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kSegCopyBlock;
            if (v < v1) x[u] = load16(src + v * 16);
        }
        // stores: buffer instructions, non-temporal with device scope, over the
        // tile's whole vectors (ReplicateToShard 2.9-3.5% faster than with
        // non-temporal global stores)
        const rsrc_t out = make_rsrc(dst + b0, uint32_t(v1 * 16 - b0));
#pragma unroll
        for (int u = 0; u < U; u++) bstore16<kPolNT | kPolDevice>(out, (threadIdx.x + u * kSegCopyBlock) * 16, x[u]);
        const uint64_t t = v1 * 16 + threadIdx.x;
        if (t < b1) dst[t] = src[t];
    } else {
        copy_shifted<kSegCopyBlock, kSegCopyTileBytes>(src, dst, a.bytes[k], b - a.tile_start[k]);
    }
}

// ------------------------------------------------- shard-dimension A2A --
__device__ __forceinline__ void dims_run(const DimsArgs& a, uint64_t k, const char** src, char** dst) {
    const uint64_t es = a.esize;
    if (a.dir == 0) {
        const uint64_t j = k / a.rows, row = k - j * a.rows, i = row / a.rp;
        *src = static_cast<const char*>(a.src[i]) + ((row - i * a.rp) * a.cols + j * a.cp) * es;
        *dst = static_cast<char*>(a.dst[j]) + row * a.cp * es;
    } else {
        const uint64_t P = uint64_t(a.nranks);
        const uint64_t j = k / (a.rp * P), rem = k - j * a.rp * P, row = rem / P, i = rem - row * P;
        *src = static_cast<const char*>(a.src[i]) + (j * a.rp + row) * a.cp * es;
        *dst = static_cast<char*>(a.dst[j]) + (row * a.cols + i * a.cp) * es;
    }
}

__global__ __launch_bounds__(kBlock) void k_all_to_all_dims(DimsArgs a) {
    __shared__ const char* run_src[kDimsMaxRunsPerBlock];
    __shared__ char* run_dst[kDimsMaxRunsPerBlock];
    const uint64_t run_bytes = a.cp * a.esize;
    const uint64_t b = blockIdx.x;
    uint64_t k0, nk, lo, hi;  // runs [k0, k0 + nk), byte slice [lo, hi) of each
    if (a.tiles_per_run > 1) {
        k0 = b / a.tiles_per_run;
        nk = 1;
        lo = (b - k0 * a.tiles_per_run) * kDimsTileBytes;
        hi = min(run_bytes, lo + kDimsTileBytes);
    } else {
        k0 = b * a.runs_per_block;
        nk = min(uint64_t(a.runs_per_block), a.nruns - k0);
        lo = 0;
        hi = run_bytes;
    }
    if (threadIdx.x < nk) {  // decode each run once per workgroup
        const char* from;
        char* to;
        dims_run(a, k0 + threadIdx.x, &from, &to);
        run_src[threadIdx.x] = from + lo;
        run_dst[threadIdx.x] = to + lo;
    }
    __syncthreads();
    const uint64_t span = hi - lo;
    if (a.vec) {
        const uint32_t sv = uint32_t(span / 16);
        const uint32_t total = uint32_t(nk) * sv;
        constexpr int U = 4;
        for (uint32_t t0 = threadIdx.x; t0 < total; t0 += kBlock * U) {
            u32x4 x[U];
            char* to[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint32_t t = t0 + u * kBlock;
                to[u] = nullptr;
                if (t < total) {
                    const uint32_t rk = t / sv, v = t - rk * sv;
                    x[u] = load16(run_src[rk] + uint64_t(v) * 16);
                    to[u] = run_dst[rk] + uint64_t(v) * 16;
                }
            }
#pragma unroll
            for (int u = 0; u < U; u++)
                if (to[u]) store16(to[u], x[u]);
        }
    } else if (a.elems) {
        // runs off 16-byte alignment at element-aligned bases: whole
        // elements (runs are element multiples), U per thread with every
        // load issued before the stores (a byte loop here waited for each
        // byte's load in turn)
        constexpr int U = 8;
        const uint64_t es = a.esize;
        const uint64_t ne = span / es;  // elements per run slice
        const uint64_t total = nk * ne;
        for (uint64_t t0 = threadIdx.x; t0 < total; t0 += uint64_t(kBlock) * U) {
            uint32_t w[U];
            char* to[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t t = t0 + uint64_t(u) * kBlock;
                to[u] = nullptr;
                if (t < total) {
                    const uint64_t rk = t / ne, c = (t - rk * ne) * es;
                    w[u] = es == 2 ? uint32_t(*reinterpret_cast<const uint16_t*>(run_src[rk] + c))
                                   : *reinterpret_cast<const uint32_t*>(run_src[rk] + c);
                    to[u] = run_dst[rk] + c;
                }
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (!to[u]) continue;
                if (es == 2) *reinterpret_cast<uint16_t*>(to[u]) = uint16_t(w[u]);
                else *reinterpret_cast<uint32_t*>(to[u]) = w[u];
            }
        }
    } else {
        const uint64_t total = nk * span;
        for (uint64_t t = threadIdx.x; t < total; t += kBlock) {
            const uint64_t rk = t / span, c = t - rk * span;
            run_dst[rk][c] = run_src[rk][c];
        }
    }
}

// Runs of at least one tile with 16-byte aligned bases and lengths: one
// workgroup of a single wave per 1 KiB slice of one run, the copy engine of
// the split-matrix all-to-all (a vector per lane, buffer stores that are
// non-temporal with device scope).  The last slice of a run may be shorter:
// its store range ends at the run's end, which drops the lanes past it.
constexpr int kDimsWaveThreads = 64;
static_assert(kDimsWaveTileBytes == uint64_t(kDimsWaveThreads) * 16, "one vector per lane");
__global__ __launch_bounds__(kDimsWaveThreads) void k_all_to_all_dims_wave(DimsArgs a) {
    const uint64_t run_bytes = a.cp * a.esize;
    const uint64_t b = blockIdx.x;
    const uint64_t k = b / a.tiles_per_run;
    const uint64_t lo = (b - k * a.tiles_per_run) * kDimsWaveTileBytes;
    const uint64_t hi = min(run_bytes, lo + kDimsWaveTileBytes);
    const char* from;
    char* to;
    dims_run(a, k, &from, &to);
    const uint32_t off = threadIdx.x * 16;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (lo + off < hi) x = load16(from + lo + off);
    const rsrc_t out = make_rsrc(to + lo, uint32_t(hi - lo));
    bstore16<kPolNT | kPolDevice>(out, off, x);
}

hipError_t launch_copy_segments(const SegCopyArgs& a, hipStream_t s) {
    const uint32_t tiles = a.tile_start[a.nsegs];
    if (tiles == 0) return hipSuccess;
    k_copy_segments<<<tiles, kSegCopyBlock, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_all_to_all_dims(const DimsArgs& a, uint32_t blocks, hipStream_t s) {
    if (blocks == 0) return hipSuccess;
    if (a.wave)
        k_all_to_all_dims_wave<<<blocks, kDimsWaveThreads, 0, s>>>(a);
    else
        k_all_to_all_dims<<<blocks, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, uint32_t tiles, hipStream_t s) {
    if (tiles == 0) return hipSuccess;
    if (a.tile_bytes != kGatherTileBytes && a.tile_bytes != kGatherWaveTileBytes) return hipErrorInvalidValue;
    if (a.split_log2 > 2 || (uint64_t(tiles) << a.split_log2) > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const int p = a.nranks;
    return p <= 1 ? gather_p<1>(a, tiles, s) : p <= 2 ? gather_p<2>(a, tiles, s) : p <= 4 ? gather_p<4>(a, tiles, s)
           : p <= 8 ? gather_p<8>(a, tiles, s) : gather_p<16>(a, tiles, s);
}

hipError_t launch_gather_touch(const GatherArgs& a, uint32_t tiles, hipStream_t s) {
    if (tiles == 0) return hipSuccess;
    if (a.tile_bytes != kGatherTileBytes) return hipErrorInvalidValue;  // the read pass walks 2 KiB tiles
    k_gather_touch<<<tiles, kGatherBlock, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_all_to_all(const AllToAllArgs& a, uint32_t tiles, hipStream_t s) {
    if (tiles == 0) return hipSuccess;
    k_all_to_all<<<tiles, kA2AThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace dt
