// copy.hip -- the gather and all-to-all copy engines.
//
// Both are byte copies driven by an offset table carried in the kernel
// arguments (no device-side tables).  The work is cut into 4-16 KiB tiles of
// source data; one workgroup copies one tile, so uneven pieces (1 row or
// 16384 rows, an empty all-to-all block or a 4096-row one) balance across the
// whole chip.  A workgroup finds its piece from an exclusive prefix sum of
// tile counts: a linear scan over at most 16 ranks for the gather, a binary
// search over the P*P blocks for the all-to-all.
//
// AllGather fans out: each source tile is read once and written to every
// rank's output, (1 + P) bytes of HBM traffic per gathered byte.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

constexpr int kCopyU = int(kCopyTileBytes / 16 / kBlock);  // 16-byte vectors per thread per tile

// PMAX bounds the rank count; EXACT (P == PMAX) unrolls the P destination
// stores.  A tile is U * 4 KiB of one rank's source (U = kGatherU).
template <int PMAX, bool EXACT, int U>
__global__ __launch_bounds__(kBlock) void k_gather(GatherArgs a) {
    constexpr uint64_t kTile = uint64_t(U) * kBlock * 16;
    const uint32_t b = blockIdx.x;
    const int nr = EXACT ? PMAX : a.nranks;
    int r = 0;
    while (r + 1 < nr && a.tile_start[r + 1] <= b) r++;
    const char* src = static_cast<const char*>(a.src[r]);
    const uint64_t off = a.offset[r];
    const uint64_t b0 = uint64_t(b - a.tile_start[r]) * kTile;
    const uint64_t b1 = min(a.bytes[r], b0 + kTile);
    if ((a.aligned >> r) & 1u) {
        const uint64_t v1 = b1 / 16;
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kBlock;
            if (v < v1) x[u] = load16_h<false>(src + v * 16);  // writes dominate 1:P
        }
#pragma unroll
        for (int q = 0; q < PMAX; q++) {
            if (q < nr) {
                char* dst = static_cast<char*>(a.dst[q]) + off;
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kBlock;
                    if (v < v1) store16_h<true>(dst + v * 16, x[u]);
                }
            }
        }
        const uint64_t t = v1 * 16 + threadIdx.x;  // ragged end: fewer than 16 bytes
        if (t < b1) {
            const char c = src[t];
            for (int q = 0; q < nr; q++) static_cast<char*>(a.dst[q])[off + t] = c;
        }
    } else {
        for (uint64_t t = b0 + threadIdx.x; t < b1; t += kBlock) {
            const char c = src[t];
            for (int q = 0; q < nr; q++) static_cast<char*>(a.dst[q])[off + t] = c;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_all_to_all(AllToAllArgs a) {
    const uint32_t b = blockIdx.x;
    const int nr = a.nranks;
    // largest block index s with tile_start[s] <= b; that block is non-empty
    int lo = 0, hi = nr * nr;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_start[mid] <= b)
            lo = mid;
        else
            hi = mid;
    }
    const int s = lo, i = s / nr, j = s - i * nr;
    uint64_t send_off = 0;  // blocks i -> 0..j-1 precede i -> j in rank i's input
    for (int jj = 0; jj < j; jj++) send_off += a.split[i * nr + jj];
    uint64_t recv_off = 0;  // blocks 0..i-1 -> j precede i -> j in rank j's output
    for (int ii = 0; ii < i; ii++) recv_off += a.split[ii * nr + j];
    const char* src = static_cast<const char*>(a.src[i]) + send_off;
    char* dst = static_cast<char*>(a.dst[j]) + recv_off;
    const uint64_t b0 = uint64_t(b - a.tile_start[s]) * kCopyTileBytes;
    const uint64_t b1 = min(a.split[s], b0 + kCopyTileBytes);
    if ((a.aligned[s >> 5] >> (s & 31)) & 1u) {
        const uint64_t v1 = b1 / 16;
        u32x4 x[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kBlock;
            if (v < v1) x[u] = load16(src + v * 16);
        }
#pragma unroll
        for (int u = 0; u < kCopyU; u++) {
            const uint64_t v = b0 / 16 + threadIdx.x + uint64_t(u) * kBlock;
            if (v < v1) store16(dst + v * 16, x[u]);
        }
        const uint64_t t = v1 * 16 + threadIdx.x;
        if (t < b1) dst[t] = src[t];
    } else {
        for (uint64_t t = b0 + threadIdx.x; t < b1; t += kBlock) dst[t] = src[t];
    }
}

namespace {
template <int PMAX, int U>
hipError_t gather_pu(const GatherArgs& a, uint32_t tiles, hipStream_t s) {
    if (a.nranks == PMAX)
        k_gather<PMAX, true, U><<<tiles, kBlock, 0, s>>>(a);
    else
        k_gather<PMAX, false, U><<<tiles, kBlock, 0, s>>>(a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gather(const GatherArgs& a, uint32_t tiles, hipStream_t s) {
    if (tiles == 0) return hipSuccess;
    const int p = a.nranks;
    return p <= 1 ? gather_pu<1, kGatherU>(a, tiles, s) : p <= 2 ? gather_pu<2, kGatherU>(a, tiles, s)
           : p <= 4 ? gather_pu<4, kGatherU>(a, tiles, s) : p <= 8 ? gather_pu<8, kGatherU>(a, tiles, s)
           : gather_pu<16, kGatherU>(a, tiles, s);
}

hipError_t launch_all_to_all(const AllToAllArgs& a, uint32_t tiles, hipStream_t s) {
    if (tiles == 0) return hipSuccess;
    k_all_to_all<<<tiles, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace dt
