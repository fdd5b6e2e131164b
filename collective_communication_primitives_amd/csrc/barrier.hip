// barrier.hip -- the HBM signal-window barrier.
//
// pypto page "Barrier：仅信号（Signals Only）": every rank owns a window of P
// int32 cells; cell s of rank r's window has exactly one writer, rank s.
// Notify is an atomic add of 1 into the peer's window at the notifier's own
// row; wait is "cell >= threshold".  Windows are reused by raising the
// threshold by one per generation (the page's edge-case table), so nothing
// has to be reset between calls.
//
// One workgroup per rank, launched cooperatively so that all P workgroups are
// resident at once (a spin-wait across workgroups that were not co-resident
// could never finish).  Within the rank's first wave, lane p notifies peer p
// and lane s watches cell s, so the P-1 notifies and P-1 waits of the page's
// cost card run in parallel.  The MI355X has eight XCDs, each with its own
// L2: notifies are device-scope release atomics and waits device-scope
// acquire loads, which make the signalling (and the data it guards) coherent
// across XCDs.  Every wait is bounded by a wall-clock budget; on expiry the
// workgroup records DT_ERR_TIMEOUT (4) and leaves, so no launch can hang.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

constexpr int kTimeoutStatus = 4;

// One generation for rank r, executed by one full wave.  Returns false on
// timeout (wave-uniform).
__device__ bool barrier_round(const BarrierArgs& a, int r, int g) {
    const int lane = threadIdx.x;
    const bool peer = lane < a.nranks && lane != r;
    if (peer) __hip_atomic_fetch_add(a.win[lane] + r, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t start = wall_clock64();
    while (true) {
        const bool ok = !peer || __hip_atomic_load(a.win[r] + lane, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) >= g;
        if (__all(ok)) return true;
        if (wall_clock64() - start > a.timeout_ticks) {
            if (lane == 0) __hip_atomic_store(a.status, kTimeoutStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

__global__ __launch_bounds__(64) void k_barrier(BarrierArgs a) {
    const int r = blockIdx.x;
    for (int k = 0; k < a.generations; k++)
        if (!barrier_round(a, r, a.first_generation + k)) return;
}

__device__ void copy_bytes(char* to, const char* from, uint64_t n) {
    const bool vec = ((reinterpret_cast<uintptr_t>(to) | reinterpret_cast<uintptr_t>(from)) & 15) == 0;
    uint64_t done = 0;
    if (vec) {
        const uint64_t nv = n / 16;
        for (uint64_t v = threadIdx.x; v < nv; v += blockDim.x)
            *reinterpret_cast<u32x4*>(to + v * 16) = *reinterpret_cast<const u32x4*>(from + v * 16);
        done = nv * 16;
    }
    for (uint64_t t = done + threadIdx.x; t < n; t += blockDim.x) to[t] = from[t];
}

// Stage, barrier, then read the next rank's stage: dst[r] = src[(r+1) % P].
__global__ __launch_bounds__(kBlock) void k_exchange(ExchangeArgs a) {
    __shared__ int passed;
    const int r = blockIdx.x;
    copy_bytes(static_cast<char*>(a.stage[r]), static_cast<const char*>(a.src[r]), a.nbytes);
    __threadfence();  // this workgroup's staged bytes before its notifies
    __syncthreads();
    if (threadIdx.x < 64) {
        const bool ok = barrier_round(a.bar, r, a.bar.first_generation);
        if (threadIdx.x == 0) passed = ok ? 1 : 0;
    }
    __syncthreads();
    if (!passed) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // peers' staged bytes are visible
    const int peer = (r + 1) % a.bar.nranks;
    copy_bytes(static_cast<char*>(a.dst[r]), static_cast<const char*>(a.stage[peer]), a.nbytes);
}

hipError_t launch_barrier(const BarrierArgs& a, hipStream_t s) {
    BarrierArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_barrier), dim3(a.nranks), dim3(64), params,
                                      0, s);
}

hipError_t launch_exchange(const ExchangeArgs& a, hipStream_t s) {
    ExchangeArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_exchange), dim3(a.bar.nranks),
                                      dim3(kBlock), params, 0, s);
}

}  // namespace dt
