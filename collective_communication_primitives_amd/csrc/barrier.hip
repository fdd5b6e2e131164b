// barrier.hip -- the HBM signal-window barrier.
//
// pypto page "Barrier：仅信号（Signals Only）": every rank owns a window of P
// int32 cells; cell s of rank r's window has exactly one writer, rank s.
// Notify is an atomic add of 1 into the peer's window at the notifier's own
// row; wait is "cell >= threshold".  Windows are reused by raising the
// threshold by one per generation (the page's edge-case table), so nothing
// has to be reset between calls.
//
// Each rank is one 64-wide wave: lane p notifies peer p and lane s watches
// cell s, so the P-1 notifies and P-1 waits of the page's cost card run in
// parallel.  Two layouts:
//   packed (default): all P waves in ONE workgroup (P <= 16 -> <= 1024
//     threads).  A workgroup is always resident as a whole, so the spin-waits
//     cannot starve, and the launch is an ordinary one.
//   spread: one workgroup per rank, launched cooperatively so all P are
//     resident at once; the ranks then sit on different CUs and XCDs.
// Notifies are atomic adds and waits atomic loads at the narrowest scope
// that holds every rank: device scope for the spread layout (the MI355X's
// eight XCDs each have their own L2; device-scope atomics go past it, so the
// window is coherent across them), workgroup scope for the packed layout,
// whose ranks all share one CU.  The signals themselves are relaxed: a
// standalone barrier launch touches no other memory, and the exchange, which
// does, orders its data with a release fence before the notifies and an
// acquire fence after the waits (fence-to-fence synchronization through the
// window cells), so no notify or poll has to write back or invalidate a
// cache.  The packed layout polls with workgroup-scope acquire loads, which
// skip the CU's L1 copy of the cell (1.5 us per generation at P=16, against
// 2.4 us for relaxed loads that keep hitting it).  Every wait is bounded by a wall-clock budget; on expiry the wave
// records DT_ERR_TIMEOUT (4) and leaves, so no launch can hang.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

constexpr int kTimeoutStatus = 4;

// One generation for rank r, executed by one full wave (lane = 0..63), with
// the notifies and waits at memory scope SCOPE; POLL is the memory order of
// the polling loads.  Returns false on timeout (wave-uniform).
template <int SCOPE, int POLL>
__device__ bool barrier_round(const BarrierArgs& a, int r, int g, int lane) {
    const bool peer = lane < a.nranks && lane != r;
    if (peer) __hip_atomic_fetch_add(a.win[lane] + r, 1, __ATOMIC_RELAXED, SCOPE);
    const uint64_t start = wall_clock64();
    while (true) {
        const bool ok = !peer || __hip_atomic_load(a.win[r] + lane, POLL, SCOPE) >= g;
        if (__all(ok)) return true;
        if (wall_clock64() - start > a.timeout_ticks) {
            if (lane == 0) __hip_atomic_store(a.status, kTimeoutStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// spread: blockIdx.x = rank, one wave per workgroup
__global__ __launch_bounds__(64) void k_barrier_spread(BarrierArgs a) {
    const int r = blockIdx.x;
    for (int k = 0; k < a.generations; k++)
        if (!barrier_round<__HIP_MEMORY_SCOPE_AGENT, __ATOMIC_RELAXED>(a, r, a.first_generation + k, threadIdx.x)) return;
}

// packed: one workgroup, wave w = rank w
__global__ __launch_bounds__(1024) void k_barrier_packed(BarrierArgs a) {
    const int r = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    for (int k = 0; k < a.generations; k++)
        if (!barrier_round<__HIP_MEMORY_SCOPE_WORKGROUP, __ATOMIC_ACQUIRE>(a, r, a.first_generation + k, lane)) return;
}

// Byte copy by `n_threads` cooperating threads (index `tid`).
__device__ void copy_bytes(char* to, const char* from, uint64_t n, uint32_t tid, uint32_t n_threads) {
    const bool vec = ((reinterpret_cast<uintptr_t>(to) | reinterpret_cast<uintptr_t>(from)) & 15) == 0;
    uint64_t done = 0;
    if (vec) {
        const uint64_t nv = n / 16;
        for (uint64_t v = tid; v < nv; v += n_threads)
            *reinterpret_cast<u32x4*>(to + v * 16) = *reinterpret_cast<const u32x4*>(from + v * 16);
        done = nv * 16;
    }
    for (uint64_t t = done + tid; t < n; t += n_threads) to[t] = from[t];
}

// spread exchange: workgroup r stages src[r], meets the barrier, then reads
// the next rank's stage: dst[r] = src[(r+1) % P].
__global__ __launch_bounds__(kBlock) void k_exchange_spread(ExchangeArgs a) {
    __shared__ int passed;
    const int r = blockIdx.x;
    copy_bytes(static_cast<char*>(a.stage[r]), static_cast<const char*>(a.src[r]), a.nbytes, threadIdx.x, blockDim.x);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // every thread's staged bytes before the notifies
    __syncthreads();
    if (threadIdx.x < 64) {
        const bool ok = barrier_round<__HIP_MEMORY_SCOPE_AGENT, __ATOMIC_RELAXED>(a.bar, r, a.bar.first_generation, threadIdx.x);
        if (threadIdx.x == 0) passed = ok ? 1 : 0;
    }
    __syncthreads();
    if (!passed) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // peers' staged bytes are visible
    const int peer = (r + 1) % a.bar.nranks;
    copy_bytes(static_cast<char*>(a.dst[r]), static_cast<const char*>(a.stage[peer]), a.nbytes, threadIdx.x,
               blockDim.x);
}

// packed exchange: wave r of the single workgroup does rank r's part.
__global__ __launch_bounds__(1024) void k_exchange_packed(ExchangeArgs a) {
    const int r = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    copy_bytes(static_cast<char*>(a.stage[r]), static_cast<const char*>(a.src[r]), a.nbytes, lane, 64);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the wave's staged bytes before its notifies
    if (!barrier_round<__HIP_MEMORY_SCOPE_WORKGROUP, __ATOMIC_ACQUIRE>(a.bar, r, a.bar.first_generation, lane)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // peers' staged bytes are visible
    const int peer = (r + 1) % a.bar.nranks;
    copy_bytes(static_cast<char*>(a.dst[r]), static_cast<const char*>(a.stage[peer]), a.nbytes, lane, 64);
}

hipError_t launch_barrier(const BarrierArgs& a, int spread, hipStream_t s) {
    if (!spread) {
        k_barrier_packed<<<1, a.nranks * 64, 0, s>>>(a);
        return hipGetLastError();
    }
    BarrierArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_barrier_spread), dim3(a.nranks), dim3(64),
                                      params, 0, s);
}

hipError_t launch_exchange(const ExchangeArgs& a, int spread, hipStream_t s) {
    if (!spread) {
        k_exchange_packed<<<1, a.bar.nranks * 64, 0, s>>>(a);
        return hipGetLastError();
    }
    ExchangeArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_exchange_spread), dim3(a.bar.nranks),
                                      dim3(kBlock), params, 0, s);
}

}  // namespace dt
