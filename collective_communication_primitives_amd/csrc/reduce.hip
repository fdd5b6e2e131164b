// reduce.hip -- the rank-fold kernels: AllReduce (one-shot), ReduceScatter
// (on 16-byte aligned buffers, or over 128-byte line grids with every input
// shifted into place when the buffers share no offset), the element path
// and the multi-tensor bucket reduce.
//
// Work layout.  Rank buffers are P separate contiguous allocations in HBM.
// Each thread owns whole 16-byte vectors: it issues the loads of its vectors
// from every rank before folding, so a workgroup keeps P tiles of reads in
// flight (one per rank, 1-8 KiB each by kernel), then folds in rank order and
// writes the result (to every rank for AllReduce, to the owning rank for
// ReduceScatter).  Every HBM byte is
// touched once: AllReduce moves 2*P*S bytes, ReduceScatter (P+1)*S.
//
// The rank count P (1..16) is a template parameter of every fold kernel
// (the element kernel's too), so each fold is fully unrolled with no
// per-rank predicate and the P loads of a vector go out back to back.  (With a runtime count below a template
// bound, the compiler turned the per-rank guards into branches and waited
// for each load in turn: the ReduceScatter of P = 5-7 took 2x as long.)
#include <type_traits>

#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

// One wave, one vector per thread: the tile of the ReduceScatter.
constexpr int kWaveBlock = 64;

// ------------------------------------------------------------- AllReduce --
// grid.x covers a.count vectors in tiles of BLOCK*U.
//
// Issue order: all of rank 0's vectors, then rank 1's, ...; stores output by
// output.  Each wave then sends U KiB-long runs to one buffer before moving to
// the next, which the MI355X's HBM serves faster than interleaving the P
// buffers vector by vector (measured: +3% for the P-to-P AllReduce pattern).
// BST: store through buffer instructions (see the store loop).
template <int DT, int OP, int P, int U, int BLOCK, bool BST = false>
__global__ __launch_bounds__(BLOCK) void k_reduce_vec(ReduceArgs a) {
    const uint64_t base = uint64_t(blockIdx.x) * (BLOCK * U) + threadIdx.x;
    // Loads without branches, so that all P * U of them are in flight at
    // once: a lane past the end re-reads the last vector (its result is not
    // stored).  A per-lane guard around each load compiled into a wait after
    // every load.
    u32x4 x[U][P];
#pragma unroll
    for (int r = 0; r < P; r++) {
        const char* src = static_cast<const char*>(a.src[r]);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = base + uint64_t(u) * BLOCK;
            x[u][r] = load16(src + (v < a.count ? v : a.count - 1) * 16);
        }
    }
    u32x4 y[U];
#pragma unroll
    for (int u = 0; u < U; u++) y[u] = fold_vec<DT, OP, P>(x[u], P);
    if constexpr (BST) {
        // Buffer stores, non-temporal with device scope, where they measured
        // faster than non-temporal global stores (in-process A/B): every P >= 2
        // up to kBufferStoreAllReduceBytes per rank (graph-replay times at 1-8
        // MiB: P=2 and P=4 6-20% faster, P=8 5-10% in eager loops).  Beyond
        // that (P=8 at 16-20 MiB, P=16 at 8 MiB in one run) they were up to 8%
        // slower.
        const uint64_t t0 = uint64_t(blockIdx.x) * (BLOCK * U);
        const uint64_t left = a.count - t0;
        const uint32_t tb = uint32_t((left < uint64_t(BLOCK * U) ? left : uint64_t(BLOCK * U)) * 16);
#pragma unroll
        for (int q = 0; q < P; q++) {
            const rsrc_t out = make_rsrc(static_cast<char*>(a.dst[q]) + t0 * 16, tb);
#pragma unroll
            for (int u = 0; u < U; u++) bstore16<kPolNT | kPolDevice>(out, (threadIdx.x + u * BLOCK) * 16, y[u]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < P; q++) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t v = base + uint64_t(u) * BLOCK;
                if (v < a.count) store16(static_cast<char*>(a.dst[q]) + v * 16, y[u]);
            }
        }
    }
}

// --------------------------------------------------------- ReduceScatter --
// grid.x covers a.count vectors of one chunk in tiles of BLOCK*U; grid.y =
// output chunk.  Chunk c starts c * a.chunk_stride vectors into every input
// and holds a.count vectors; the last chunk holds a.last_count (the two-shot
// AllReduce cuts its chunks in whole tiles, so the last one may be shorter),
// and its tiles past that end return at once.  The stride exceeds the count
// when a misaligned head of every chunk went to the element path.  Buffer instructions: one resource per rank for the tile's
// range (the same lane offsets serve all P ranks), non-temporal loads and
// device-scope stores; the resource range cuts off the last tile.  Measured
// against the same kernel with 64-bit global addressing: 2-3% faster for
// P=8 bf16 at 16 MiB per chunk.  BLOCK threads x U vectors per tile: one
// wave with one vector per thread (1 KiB of every rank per workgroup) for
// every P.  In-process A/B: 2.5% faster than 512 threads x 1 vector at P=8
// bf16 and no slower at any of 13 placements of the inputs tried; 5-7%
// faster than 256 threads x 4 vectors at P=4 and no slower at P=2.
template <int DT, int OP, int P, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void k_reduce_scatter_vec(ReduceArgs a) {
    constexpr uint64_t kTileVecs = uint64_t(BLOCK) * U;
    const uint64_t chunk = blockIdx.y;
    const uint64_t cnt = chunk + 1 == gridDim.y ? a.last_count : a.count;
    const uint64_t t0 = uint64_t(blockIdx.x) * kTileVecs;       // < a.count by the grid
    if (t0 >= cnt) return;                                      // past the end of a shorter last chunk
    const uint64_t left = cnt - t0;
    const uint32_t bytes = uint32_t((left < kTileVecs ? left : kTileVecs) * 16);
    const uint64_t in_off = (chunk * a.chunk_stride + t0) * 16;  // bytes into every rank's input
    const uint32_t lane = threadIdx.x * 16;
    u32x4 x[U][P];
#pragma unroll
    for (int r = 0; r < P; r++) {
        const rsrc_t in = make_rsrc(static_cast<const char*>(a.src[r]) + in_off, bytes);
#pragma unroll
        for (int u = 0; u < U; u++) x[u][r] = bload16<kPolNT>(in, lane + u * (BLOCK * 16));
    }
    const rsrc_t out = make_rsrc(static_cast<char*>(a.dst[chunk]) + t0 * 16, bytes);
#pragma unroll
    for (int u = 0; u < U; u++) bstore16<kPolDevice>(out, lane + u * (BLOCK * 16), fold_vec<DT, OP, P>(x[u], P));
}

// Element-wise path for ragged tails and unaligned buffers.  Elements
// [a.first, a.first + a.count) and [a.first2, a.first2 + a.count2) of chunk
// blockIdx.y.
template <int DT, int OP, int P>
__global__ __launch_bounds__(kBlock) void k_reduce_elems(ReduceArgs a) {
    const uint64_t chunk = a.rs ? blockIdx.y : 0;
    const uint64_t in_base = chunk * a.chunk_elems;
    const uint64_t total = a.count + a.count2;
    for (uint64_t i = uint64_t(blockIdx.x) * kBlock + threadIdx.x; i < total;
         i += uint64_t(gridDim.x) * kBlock) {
        const uint64_t e = i < a.count ? a.first + i : a.first2 + (i - a.count);
        if (a.rs) {
            fold_elem<DT, OP, P>(a.src, in_base + e, a.dst[chunk], e);
        } else {
            const uint32_t bits = fold_elem_bits<DT, OP, P>(a.src, e);
#pragma unroll
            for (int q = 0; q < P; q++) store_elem<DT>(a.dst[q], e, bits);
        }
    }
}

// ReduceScatter over each output chunk's line grid (GridFoldArgs), for
// buffers that share no offset.  Tile t of chunk c covers bytes
// [t * 2 KiB, (t + 1) * 2 KiB) of the grid that starts at the line holding
// the chunk's first output byte, lead bytes before it; grid.y = chunk; two
// waves per workgroup, one output vector per lane, so every store is an
// aligned vector and each wave writes whole lines.
//
// A tile whose bytes all lie inside the chunk (every tile but the first and
// last of a chunk) is staged: each input's bytes for the tile start d bytes
// into one of its lines, and the workgroup loads those whole lines, d = 0
// exactly the tile's 16 lines and else 17, one aligned vector per lane plus
// eight, non-temporal, every load of every input issued before any use.
// Each line loaded holds at least one byte of the tile's input, so nothing
// beyond the pages that hold the buffer is touched.  The lines go to LDS;
// after one barrier each lane takes its 16 bytes of every input from there
// (the two aligned LDS vectors around byte d + 16 * lane, joined by a byte
// shift that is uniform per input), folds and stores.  Against the earlier
// form, which loaded the two aligned vectors around each lane's bytes from
// memory directly (every wave's loads then straddle 9 lines for 8 lines of
// data), in-process A/B at P=8 bf16, 128 MiB per rank: ReduceScatter with
// the outputs 2 bytes off 216 -> 192 us (0.70 -> 0.78 of peak), with the
// inputs 2 bytes off 218 -> 192 us, with every input at an offset of its own
// 217 -> 190 us; the two-shot AllReduce over it 388 -> 344 us.  The
// input-line grid that the shared-input-offset cases took before (one
// aligned load per lane, the result shifted across lanes onto the outputs)
// ran 216-219 us and is gone.
//
// The first and last tile of a chunk go lane by lane: a full vector from
// two plain aligned loads per input joined by the same shift, a partial one
// (at either end of the chunk) through windows over the input's chunk
// (load_window: nothing outside the chunk's aligned vectors is read), its
// elements inside the chunk stored one by one.
constexpr int kGridOutBlock = 128;
constexpr int64_t kGridTile = int64_t(kGridOutBlock) * 16;
template <int DT, int OP, int P>
__global__ __launch_bounds__(kGridOutBlock) void k_reduce_scatter_grid(GridFoldArgs a) {
    constexpr int64_t ES = DT == kBF16 ? 2 : 4;
    constexpr int kV = int(kGridTile / 16);  // vectors per tile, one per lane
    const uint32_t c = blockIdx.y;
    const int64_t n = int64_t(c + 1 == uint32_t(a.nchunks) ? a.last_count : a.count) * ES;  // chunk bytes
    const int64_t lead = int64_t(a.lead[c]);
    const int64_t g0 = int64_t(blockIdx.x) * kGridTile - lead;  // chunk byte at the tile's grid start
    if (g0 >= n) return;                                        // past the end of this chunk
    const uint64_t in_off = uint64_t(c) * a.in_stride * uint64_t(ES);
    const int tid = int(threadIdx.x);
    if (g0 >= 0 && g0 + kGridTile <= n) {  // uniform per workgroup: every lane reaches the barrier
        __shared__ u32x4 stage[P][kV + 8];
        uint32_t d[P];
        u32x4 v[P], w[P];
#pragma unroll
        for (int r = 0; r < P; r++) {
            const char* base = static_cast<const char*>(a.src[r]) + in_off + g0;
            d[r] = uint32_t(reinterpret_cast<uintptr_t>(base) & uint64_t(kGridAlign - 1));
            const char* line0 = base - d[r];
            v[r] = load16(line0 + tid * 16);
            if (tid < 8 && d[r] != 0) w[r] = load16(line0 + kGridTile + tid * 16);
        }
#pragma unroll
        for (int r = 0; r < P; r++) {
            stage[r][tid] = v[r];
            if (tid < 8 && d[r] != 0) stage[r][kV + tid] = w[r];
        }
        __syncthreads();
        u32x4 x[P];
#pragma unroll
        for (int r = 0; r < P; r++) {
            const uint32_t q = d[r] + uint32_t(tid) * 16;  // at most 127 + 16 * 127: vectors 0 .. kV + 7
            const uint32_t s = q & 15u;
            const u32x4 l = stage[r][q >> 4];
            // the shift's word choice branches once per input (uniform); a
            // branch-free choice by selects ran 10% slower
            x[r] = s != 0 ? funnel16(l, stage[r][(q >> 4) + 1], s) : l;
        }
        const rsrc_t out = make_rsrc(static_cast<char*>(a.dst[c]) + g0, uint32_t(kGridTile));
        bstore16<kPolDevice>(out, uint32_t(tid) * 16, fold_vec<DT, OP, P>(x, P));
        return;
    }
    const int64_t p0 = g0 + int64_t(tid) * 16;
    if (p0 + 16 <= 0 || p0 >= n) return;  // a lane before the chunk's first grid vector or past its last
    uint32_t sm[P];
#pragma unroll
    for (int r = 0; r < P; r++)
        sm[r] = uint32_t((reinterpret_cast<uintptr_t>(a.src[r]) + in_off - uint64_t(lead)) & 15u);
    u32x4 lo[P], hi[P];
    if (p0 >= 0 && p0 + 16 <= n) {
        // both aligned vectors of every input before any is shifted; an
        // input at the grid's own offset (shift 0) loads its one vector
        // twice rather than the next one, which may lie past the buffer
#pragma unroll
        for (int r = 0; r < P; r++) {
            const char* at = static_cast<const char*>(a.src[r]) + in_off + p0 - sm[r];
            lo[r] = load16_h<false>(at);
            hi[r] = load16_h<false>(at + (sm[r] != 0 ? 16 : 0));
        }
        u32x4 x[P];
#pragma unroll
        for (int r = 0; r < P; r++) x[r] = sm[r] != 0 ? funnel16(lo[r], hi[r], sm[r]) : lo[r];
        const rsrc_t out = make_rsrc(static_cast<char*>(a.dst[c]) + g0, uint32_t(kGridTile));
        bstore16<kPolDevice>(out, uint32_t(tid) * 16, fold_vec<DT, OP, P>(x, P));
    } else {
#pragma unroll
        for (int r = 0; r < P; r++) {
            const char* s = static_cast<const char*>(a.src[r]) + in_off;
            const LoadWindow w = load_window(s, n, g0 - int64_t(sm[r]), kGridTile + 16);
            const int64_t o = p0 - int64_t(sm[r]);
            lo[r] = window_load<0>(w, o);
            hi[r] = window_load<0>(w, o + (sm[r] != 0 ? 16 : 0));
        }
        u32x4 x[P];
#pragma unroll
        for (int r = 0; r < P; r++) x[r] = sm[r] != 0 ? funnel16(lo[r], hi[r], sm[r]) : lo[r];
        store_vec_elems<int(ES)>(static_cast<char*>(a.dst[c]), p0, fold_vec<DT, OP, P>(x, P), 0, 16, n);
    }
}

// ------------------------------------------------------ bucket pieces ----
// Piece tables come in two sizes: PieceArgs (32 pieces, 3.3 KiB of kernel
// arguments, for buckets of a few large tensors) and CoalescedArgs (512
// pieces, for many small tensors).  The kernels are shared.
// Piece of tile b in the small table: the last k with tile_start[k] <= b.
// The launchers pad the entries past the last piece with UINT32_MAX, so no
// comparison needs a bound, and the lookup takes two rounds of independent
// scalar loads (the group starts tile_start[8g], then the group's other
// seven) instead of a chain of dependent ones: 1.1% faster for the
// data-parallel bucket workload (in-process A/B).
__device__ __forceinline__ int find_piece(const PieceArgs& a, uint32_t b) {
    constexpr int G = 8;
    static_assert(kMaxPieces % G == 0, "whole groups");
    int g = 0;
#pragma unroll
    for (int i = 1; i < kMaxPieces / G; i++) g += a.tile_start[i * G] <= b ? 1 : 0;
    int k = g * G;
#pragma unroll
    for (int j = 1; j < G; j++) k += a.tile_start[g * G + j] <= b ? 1 : 0;
    return k;
}
__device__ __forceinline__ int find_piece(const CoalescedArgs& a, uint32_t b) {
    int lo = 0, hi = a.npieces;  // largest k with tile_start[k] <= b
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_start[mid] <= b) lo = mid;
        else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ bool piece_aligned(const PieceArgs& a, int k) { return (a.aligned >> k) & 1u; }
__device__ __forceinline__ bool piece_aligned(const CoalescedArgs& a, int k) {
    return (a.aligned[k >> 5] >> (k & 31)) & 1u;
}

// One launch reduces every piece of its table in place: piece k's rank r
// part starts at a.ptr[k*P + r].  grid.x = tiles over all pieces.
template <typename Args, int DT, int OP, int P>
__global__ __launch_bounds__(kBlock) void k_reduce_pieces(Args a) {
    constexpr int V = Elems<DT>::value;
    const uint32_t b = blockIdx.x;
    const int k = find_piece(a, b);
    constexpr int nr = P;
    void* const* ptr = a.ptr + k * nr;
    const uint64_t len = a.len[k];
    const uint64_t e0 = uint64_t(b - a.tile_start[k]) * kPieceTileVecs * V;
    const uint64_t e1 = min(len, e0 + kPieceTileVecs * V);
    if (piece_aligned(a, k)) {
        constexpr int U = int(kPieceTileVecs / kBlock);
        const uint64_t v0 = e0 / V, v1 = e1 / V;  // e0 is a whole number of vectors
        if (v1 > v0) {  // the tile holds whole vectors (not only a ragged end)
            // branch-free loads, as in k_reduce_vec: a lane past the tile's last
            // vector re-reads it (not stored)
            u32x4 x[U][P];
#pragma unroll
            for (int r = 0; r < P; r++) {
                const char* src = static_cast<const char*>(ptr[r]);
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const uint64_t v = v0 + threadIdx.x + uint64_t(u) * kBlock;
                    x[u][r] = load16(src + (v < v1 ? v : v1 - 1) * 16);
                }
            }
            u32x4 y[U];
#pragma unroll
            for (int u = 0; u < U; u++) y[u] = fold_vec<DT, OP, P>(x[u], P);
#pragma unroll
            for (int q = 0; q < P; q++) {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const uint64_t v = v0 + threadIdx.x + uint64_t(u) * kBlock;
                    if (v < v1) store16(static_cast<char*>(ptr[q]) + v * 16, y[u]);
                }
            }
        }
        const uint64_t t = v1 * V + threadIdx.x;  // ragged end of the piece
        if (t < e1) {
            const uint32_t bits = fold_elem_bits<DT, OP, P>(ptr, t);
            for (int q = 0; q < nr; q++) store_elem<DT>(ptr[q], t, bits);
        }
    } else {
        // EU elements per thread and pass, their loads all issued before the
        // folds: an element past the piece's end is clamped to its last one
        // and not stored (one element per pass waited for every pass's loads)
        constexpr int EU = 4;
        for (uint64_t e = e0 + threadIdx.x; e < e1; e += uint64_t(kBlock) * EU) {
            uint32_t bits[EU];
#pragma unroll
            for (int u = 0; u < EU; u++) {
                const uint64_t eu = e + uint64_t(u) * kBlock;
                bits[u] = fold_elem_bits<DT, OP, P>(ptr, eu < e1 ? eu : e1 - 1);
            }
#pragma unroll
            for (int u = 0; u < EU; u++) {
                const uint64_t eu = e + uint64_t(u) * kBlock;
                if (eu < e1)
                    for (int q = 0; q < nr; q++) store_elem<DT>(ptr[q], eu, bits[u]);
            }
        }
    }
}

// ------------------------------------------------ segmented ReduceScatter --
// Many ReduceScatters (e.g. every tensor of one layer, in every shard group)
// in one launch, so the chip never drains between small collectives.  A tile
// is U*kSegBlock output vectors of one chunk j of one segment k; the
// workgroup folds member 0..P-1's vectors of that chunk in rank order.
// Single-wave workgroups with one vector per thread (1 KiB of every member
// per tile): the 32-layer gradient pipeline ran 4% faster than with 256
// threads x 4 vectors (in-process A/B), where 256 threads with 2 or 1
// vectors had been 0.5-1.3% slower.
constexpr int kSegBlock = 64;
template <int DT, int OP, int P, int U>
__global__ __launch_bounds__(kSegBlock) void k_reduce_scatter_segs(SegReduceScatterArgs a) {
    constexpr int V = Elems<DT>::value;
    const uint32_t b = blockIdx.x;
    int k = 0;
    while (k + 1 < a.nsegs && a.tile_start[k + 1] <= b) k++;
    constexpr int nr = P;
    const uint32_t t = b - a.tile_start[k];
    const uint32_t j = t / a.tiles_per_chunk[k];   // output chunk = member
    const uint32_t tt = t - j * a.tiles_per_chunk[k];
    const uint64_t m = a.m[k];
    const void* const* src = a.src + k * nr;
    void* dst = a.dst[k * nr + j];
    if ((a.aligned >> k) & 1u) {
        constexpr uint64_t kTileVecs = uint64_t(kSegBlock) * U;
        const uint64_t mv = m / V;
        const uint64_t t0 = uint64_t(tt) * kTileVecs;            // < mv by the tile count
        const uint64_t left = mv - t0;
        const uint32_t bytes = uint32_t((left < kTileVecs ? left : kTileVecs) * 16);
        const uint64_t in_off = (uint64_t(j) * mv + t0) * 16;
        const uint32_t lane = threadIdx.x * 16;
        u32x4 x[U][P];
#pragma unroll
        for (int r = 0; r < P; r++) {
            const rsrc_t in = make_rsrc(static_cast<const char*>(src[r]) + in_off, bytes);
#pragma unroll
            for (int u = 0; u < U; u++) x[u][r] = bload16<kPolNT>(in, lane + u * (kSegBlock * 16));
        }
        const rsrc_t out = make_rsrc(static_cast<char*>(dst) + t0 * 16, bytes);
#pragma unroll
        for (int u = 0; u < U; u++) bstore16<kPolDevice>(out, lane + u * (kSegBlock * 16), fold_vec<DT, OP, P>(x[u], P));
    } else {
        const uint64_t per_tile = uint64_t(kSegBlock) * U * V;
        const uint64_t e0 = uint64_t(tt) * per_tile;
        const uint64_t e1 = min(m, e0 + per_tile);
        // EU elements per thread and pass, loads before folds (as for the
        // unaligned bucket pieces)
        constexpr int EU = 4;
        for (uint64_t e = e0 + threadIdx.x; e < e1; e += uint64_t(kSegBlock) * EU) {
            uint32_t bits[EU];
#pragma unroll
            for (int u = 0; u < EU; u++) {
                const uint64_t eu = e + uint64_t(u) * kSegBlock;
                bits[u] = fold_elem_bits<DT, OP, P>(src, uint64_t(j) * m + (eu < e1 ? eu : e1 - 1));
            }
#pragma unroll
            for (int u = 0; u < EU; u++) {
                const uint64_t eu = e + uint64_t(u) * kSegBlock;
                if (eu < e1) store_elem<DT>(dst, eu, bits[u]);
            }
        }
    }
}

// Flatten (to_ws = 1) or unflatten (to_ws = 0) the pieces of one bucket for
// rank blockIdx.y: a byte copy between the tensors and the bucket buffer.
template <typename Args>
__global__ __launch_bounds__(kBlock) void k_copy_pieces(Args a, int esize, int to_ws) {
    const uint32_t b = blockIdx.x;
    const int r = blockIdx.y;
    const int k = find_piece(a, b);
    char* tensor = static_cast<char*>(a.ptr[k * a.nranks + r]);
    char* bucket = static_cast<char*>(a.ws[r]) + a.wpos[k] * uint64_t(esize);
    const char* from = to_ws ? tensor : bucket;
    char* to = to_ws ? bucket : tensor;
    const uint64_t bytes = a.len[k] * uint64_t(esize);
    const uint64_t tile_bytes = kPieceTileVecs * 16;
    const uint64_t b0 = uint64_t(b - a.tile_start[k]) * tile_bytes;
    const uint64_t b1 = min(bytes, b0 + tile_bytes);
    if (piece_aligned(a, k)) {
        const uint64_t v1 = b1 / 16;
        for (uint64_t v = b0 / 16 + threadIdx.x; v < v1; v += kBlock) store16(to + v * 16, load16(from + v * 16));
        const uint64_t t = v1 * 16 + threadIdx.x;
        if (t < b1) to[t] = from[t];
    } else {
        // Unaligned: each lane takes 16-byte slices of the tile, every slice
        // one shifted vector loaded through a window over the piece (all of
        // them before any store), stored in the widest words the
        // destination's alignment allows.  (A byte loop here waited for
        // each byte's load in turn.)
        constexpr int U = int(kPieceTileVecs / kBlock);
        const uint32_t sm = uint32_t(reinterpret_cast<uintptr_t>(from) & 15u);
        const LoadWindow w = load_window(from, int64_t(bytes), int64_t(b0) - sm, int64_t(tile_bytes) + 16);
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = b0 + (threadIdx.x + uint64_t(u) * kBlock) * 16;
            if (v < b1) x[u] = window_load_shifted<kPolNT>(w, int64_t(v) - sm, sm);
        }
        const uint32_t ta = uint32_t(reinterpret_cast<uintptr_t>(to) & 3u);  // the same at every slice
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = b0 + (threadIdx.x + uint64_t(u) * kBlock) * 16;
            if (v >= b1) continue;
            const int m = int(b1 - v < 16 ? b1 - v : 16);
            if (ta == 0 && (m & 3) == 0) {
                for (int j = 0; j < m; j += 4) *reinterpret_cast<uint32_t*>(to + v + j) = x[u][j >> 2];
            } else if ((ta & 1) == 0 && (m & 1) == 0) {
                for (int j = 0; j < m; j += 2)
                    *reinterpret_cast<uint16_t*>(to + v + j) = uint16_t(x[u][j >> 2] >> ((j & 2) * 8));
            } else {
                for (int j = 0; j < m; j++) to[v + j] = vec_byte(x[u], j);
            }
        }
    }
}

// ---------------------------------------------------------- dispatchers --
namespace {

// Calls fn(std::integral_constant<int, P>{}) for the run-time rank count
// 1 <= nranks <= 16: every fold kernel is instantiated for each P.
template <typename Fn>
hipError_t with_ranks(int nranks, Fn&& fn) {
    switch (nranks) {
        case 1: return fn(std::integral_constant<int, 1>{});
        case 2: return fn(std::integral_constant<int, 2>{});
        case 3: return fn(std::integral_constant<int, 3>{});
        case 4: return fn(std::integral_constant<int, 4>{});
        case 5: return fn(std::integral_constant<int, 5>{});
        case 6: return fn(std::integral_constant<int, 6>{});
        case 7: return fn(std::integral_constant<int, 7>{});
        case 8: return fn(std::integral_constant<int, 8>{});
        case 9: return fn(std::integral_constant<int, 9>{});
        case 10: return fn(std::integral_constant<int, 10>{});
        case 11: return fn(std::integral_constant<int, 11>{});
        case 12: return fn(std::integral_constant<int, 12>{});
        case 13: return fn(std::integral_constant<int, 13>{});
        case 14: return fn(std::integral_constant<int, 14>{});
        case 15: return fn(std::integral_constant<int, 15>{});
        case 16: return fn(std::integral_constant<int, 16>{});
        default: return hipErrorInvalidValue;
    }
}

// One-shot AllReduce with P >= 2 up to this many bytes per rank: buffer stores
// (for P > 8 only below it: P=16 at exactly 8 MiB measured up to 8% slower).
constexpr uint64_t kBufferStoreAllReduceBytes = 8ull << 20;

// Vectors per thread of the one-shot AllReduce in kBlock-thread tiles,
// measured on the MI355X for 25-256 MiB per rank: two, four for the plain
// copy of P = 1.
template <int P>
constexpr int ar_unroll() { return P == 1 ? 4 : 2; }

template <int DT, int OP, int P>
void reduce_vec_launch(const ReduceArgs& a, uint64_t blocks, hipStream_t s) {
    if (a.rs) {
        const dim3 grid{unsigned(blocks), unsigned(P), 1u};
        k_reduce_scatter_vec<DT, OP, P, kWaveBlock, 1><<<grid, kWaveBlock, 0, s>>>(a);
        return;
    }
    if constexpr (P >= 2) {
        const uint64_t bytes = a.count * 16;
        if (P > 8 ? bytes < kBufferStoreAllReduceBytes : bytes <= kBufferStoreAllReduceBytes) {
            k_reduce_vec<DT, OP, P, ar_unroll<P>(), kBlock, true><<<unsigned(blocks), kBlock, 0, s>>>(a);
            return;
        }
    }
    k_reduce_vec<DT, OP, P, ar_unroll<P>(), kBlock><<<unsigned(blocks), kBlock, 0, s>>>(a);
}

template <int DT, int OP, int P>
hipError_t reduce_vec_p(const ReduceArgs& a, hipStream_t s) {
    // the ReduceScatter runs one-wave tiles; the one-shot AllReduce kBlock threads x ar_unroll vectors
    const uint64_t per_block = a.rs ? uint64_t(kWaveBlock) : uint64_t(kBlock) * ar_unroll<P>();
    const uint64_t blocks = (a.count + per_block - 1) / per_block;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    reduce_vec_launch<DT, OP, P>(a, blocks, s);
    return hipGetLastError();
}

template <int DT, int OP>
hipError_t reduce_vec_op(const ReduceArgs& a, hipStream_t s) {
    return with_ranks(a.nranks, [&](auto p) { return reduce_vec_p<DT, OP, decltype(p)::value>(a, s); });
}

template <int DT>
hipError_t reduce_vec_dt(const ReduceArgs& a, int op, hipStream_t s) {
    switch (op) {
        case kSum: return reduce_vec_op<DT, kSum>(a, s);
        case kMax: return reduce_vec_op<DT, kMax>(a, s);
        case kMin: return reduce_vec_op<DT, kMin>(a, s);
        default: return reduce_vec_op<DT, kAvg>(a, s);
    }
}

template <int DT, int OP, int P>
hipError_t reduce_elems_p(const ReduceArgs& a, hipStream_t s) {
    const uint64_t total = a.count + a.count2;
    if (total == 0) return hipSuccess;
    uint64_t blocks = (total + kBlock - 1) / kBlock;
    if (blocks > 8192) blocks = 8192;
    dim3 grid(unsigned(blocks), a.rs ? unsigned(a.nranks) : 1u);
    k_reduce_elems<DT, OP, P><<<grid, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, int OP>
hipError_t reduce_elems_op(const ReduceArgs& a, hipStream_t s) {
    return with_ranks(a.nranks, [&](auto p) { return reduce_elems_p<DT, OP, decltype(p)::value>(a, s); });
}

template <int DT>
hipError_t reduce_elems_dt(const ReduceArgs& a, int op, hipStream_t s) {
    switch (op) {
        case kSum: return reduce_elems_op<DT, kSum>(a, s);
        case kMax: return reduce_elems_op<DT, kMax>(a, s);
        case kMin: return reduce_elems_op<DT, kMin>(a, s);
        default: return reduce_elems_op<DT, kAvg>(a, s);
    }
}

template <int DT, int OP, int P>
hipError_t reduce_scatter_grid_p(const GridFoldArgs& a, hipStream_t s) {
    constexpr uint64_t tile = uint64_t(kGridTile);
    uint64_t tiles = 0;
    for (int c = 0; c < a.nchunks; c++) {
        const uint64_t n = (c + 1 == a.nchunks ? a.last_count : a.count) * (DT == kBF16 ? 2 : 4);
        const uint64_t t = (a.lead[c] + n + tile - 1) / tile;
        tiles = t > tiles ? t : tiles;
    }
    if (tiles == 0) return hipSuccess;
    if (tiles > 0x7FFFFFFFull) return hipErrorInvalidValue;
    k_reduce_scatter_grid<DT, OP, P><<<dim3(unsigned(tiles), unsigned(a.nchunks)), kGridOutBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, int OP>
hipError_t reduce_scatter_grid_op(const GridFoldArgs& a, hipStream_t s) {
    return with_ranks(a.nranks, [&](auto p) { return reduce_scatter_grid_p<DT, OP, decltype(p)::value>(a, s); });
}

template <int DT>
hipError_t reduce_scatter_grid_dt(const GridFoldArgs& a, int op, hipStream_t s) {
    switch (op) {
        case kSum: return reduce_scatter_grid_op<DT, kSum>(a, s);
        case kMax: return reduce_scatter_grid_op<DT, kMax>(a, s);
        case kMin: return reduce_scatter_grid_op<DT, kMin>(a, s);
        default: return reduce_scatter_grid_op<DT, kAvg>(a, s);
    }
}

template <typename Args, int DT, int OP, int P>
hipError_t reduce_pieces_p(const Args& a, hipStream_t s) {
    const uint32_t tiles = a.tile_start[a.npieces];
    if (tiles == 0) return hipSuccess;
    k_reduce_pieces<Args, DT, OP, P><<<tiles, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename Args, int DT, int OP>
hipError_t reduce_pieces_op(const Args& a, hipStream_t s) {
    return with_ranks(a.nranks, [&](auto p) { return reduce_pieces_p<Args, DT, OP, decltype(p)::value>(a, s); });
}

template <typename Args, int DT>
hipError_t reduce_pieces_dt(const Args& a, int op, hipStream_t s) {
    switch (op) {
        case kSum: return reduce_pieces_op<Args, DT, kSum>(a, s);
        case kMax: return reduce_pieces_op<Args, DT, kMax>(a, s);
        case kMin: return reduce_pieces_op<Args, DT, kMin>(a, s);
        default: return reduce_pieces_op<Args, DT, kAvg>(a, s);
    }
}

template <typename Args>
hipError_t reduce_pieces_any(const Args& a, int dtype, int op, hipStream_t s) {
    switch (dtype) {
        case kF32: return reduce_pieces_dt<Args, kF32>(a, op, s);
        case kBF16: return reduce_pieces_dt<Args, kBF16>(a, op, s);
        default: return reduce_pieces_dt<Args, kI32>(a, op, s);
    }
}

template <typename Args>
hipError_t copy_pieces_any(const Args& a, int esize, int to_ws, hipStream_t s) {
    const uint32_t tiles = a.tile_start[a.npieces];
    if (tiles == 0) return hipSuccess;
    dim3 grid(tiles, unsigned(a.nranks));
    k_copy_pieces<Args><<<grid, kBlock, 0, s>>>(a, esize, to_ws);
    return hipGetLastError();
}

template <int DT, int OP, int P>
hipError_t reduce_scatter_segs_p(const SegReduceScatterArgs& a, hipStream_t s) {
    constexpr int U = 1;
    const uint32_t tiles = a.tile_start[a.nsegs];
    if (tiles == 0) return hipSuccess;
    k_reduce_scatter_segs<DT, OP, P, U><<<tiles, kSegBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, int OP>
hipError_t reduce_scatter_segs_op(const SegReduceScatterArgs& a, hipStream_t s) {
    return with_ranks(a.nranks, [&](auto p) { return reduce_scatter_segs_p<DT, OP, decltype(p)::value>(a, s); });
}

template <int DT>
hipError_t reduce_scatter_segs_dt(const SegReduceScatterArgs& a, int op, hipStream_t s) {
    switch (op) {
        case kSum: return reduce_scatter_segs_op<DT, kSum>(a, s);
        case kMax: return reduce_scatter_segs_op<DT, kMax>(a, s);
        case kMin: return reduce_scatter_segs_op<DT, kMin>(a, s);
        default: return reduce_scatter_segs_op<DT, kAvg>(a, s);
    }
}

}  // namespace

uint64_t seg_rs_tile_vecs(int) { return kSegBlock; }  // U = 1 for every rank count

hipError_t launch_reduce_scatter_segs(const SegReduceScatterArgs& a, int dtype, int op, hipStream_t s) {
    switch (dtype) {
        case kF32: return reduce_scatter_segs_dt<kF32>(a, op, s);
        case kBF16: return reduce_scatter_segs_dt<kBF16>(a, op, s);
        default: return reduce_scatter_segs_dt<kI32>(a, op, s);
    }
}

hipError_t launch_reduce_vec(const ReduceArgs& a, int dtype, int op, hipStream_t s) {
    switch (dtype) {
        case kF32: return reduce_vec_dt<kF32>(a, op, s);
        case kBF16: return reduce_vec_dt<kBF16>(a, op, s);
        default: return reduce_vec_dt<kI32>(a, op, s);
    }
}

hipError_t launch_reduce_elems(const ReduceArgs& a, int dtype, int op, hipStream_t s) {
    switch (dtype) {
        case kF32: return reduce_elems_dt<kF32>(a, op, s);
        case kBF16: return reduce_elems_dt<kBF16>(a, op, s);
        default: return reduce_elems_dt<kI32>(a, op, s);
    }
}

hipError_t launch_reduce_scatter_grid(const GridFoldArgs& a, int dtype, int op, hipStream_t s) {
    if (a.nranks < 1 || a.nranks > kMaxRanksHost || a.nchunks < 1 || a.nchunks > kMaxRanksHost)
        return hipErrorInvalidValue;
    for (int c = 0; c < a.nchunks; c++)
        if (a.lead[c] >= kGridAlign) return hipErrorInvalidValue;
    switch (dtype) {
        case kF32: return reduce_scatter_grid_dt<kF32>(a, op, s);
        case kBF16: return reduce_scatter_grid_dt<kBF16>(a, op, s);
        default: return reduce_scatter_grid_dt<kI32>(a, op, s);
    }
}

// Copy of a small piece table with the entries past its last piece set to
// UINT32_MAX, as find_piece expects.
PieceArgs padded(const PieceArgs& a) {
    PieceArgs p = a;
    for (int k = p.npieces + 1; k <= kMaxPieces; k++) p.tile_start[k] = UINT32_MAX;
    return p;
}

hipError_t launch_reduce_pieces(const PieceArgs& a, int dtype, int op, hipStream_t s) {
    if (a.npieces < 1) return hipSuccess;
    if (a.npieces > kMaxPieces) return hipErrorInvalidValue;
    return reduce_pieces_any(padded(a), dtype, op, s);
}

hipError_t launch_reduce_coalesced(const CoalescedArgs& a, int dtype, int op, hipStream_t s) {
    return reduce_pieces_any(a, dtype, op, s);
}

hipError_t launch_copy_pieces(const PieceArgs& a, int esize, int to_ws, hipStream_t s) {
    if (a.npieces < 1) return hipSuccess;
    if (a.npieces > kMaxPieces) return hipErrorInvalidValue;
    return copy_pieces_any(padded(a), esize, to_ws, s);
}

hipError_t launch_copy_coalesced(const CoalescedArgs& a, int esize, int to_ws, hipStream_t s) {
    return copy_pieces_any(a, esize, to_ws, s);
}

}  // namespace dt
