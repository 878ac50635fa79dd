// Measurement program (not part of libmoe.so): what a device-wide barrier inside one persistent
// kernel costs on this GPU, against the boundary between two kernels of a HIP graph, which is what
// the decode path pays between its dependent stages.
//
// The decode step on the pages runs as a single CUDA graph (648news 07-nano-cuda-moe-qwen38-release,
// section on asynchronous CPU/GPU compute and speculative decoding); the alternative, one persistent
// kernel walking the layers with grid-wide barriers between dependent stages, only pays if such a
// barrier is cheaper than a kernel boundary. Printed, one JSON object per line:
//   barrier_release_acquire: each block publishes 64 words and a flag with an agent-scope release
//       store; every block polls all flags with acquire loads (the fences write back and invalidate
//       the L2 of each XCD, whose caches are not coherent with each other);
//   barrier_system_relaxed: the same with relaxed system-scope atomics (write-through stores,
//       L2-bypassing loads), no fences;
//   barrier_counter: one relaxed system-scope counter that every block increments and polls;
//   kernel_eager / kernel_graph: an empty kernel of the same grid launched back to back, eagerly or
//       as the nodes of one HIP graph (each node waits for the previous one).
// Every barrier spin is bounded (kSpin polls); a block that runs out counts a timeout and leaves, so
// the grid always drains. After each barrier every block checks the words of its neighbour block
// ("stale" counts reads older than the barrier).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

constexpr int kSpin = 1 << 20;
constexpr int kThreads = 256;

#define CHECK(x)                                                                             \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
            std::exit(1);                                                                    \
        }                                                                                    \
    } while (0)

template <int MODE>
__device__ __forceinline__ void store_flag(unsigned* p, unsigned v) {
    if (MODE == 0) __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <int MODE>
__device__ __forceinline__ unsigned load_flag(unsigned* p) {
    if (MODE == 0) return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// MODE 0, 1: per-block flags; MODE 2: one counter. data[b][64] is block b's payload.
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_barriers(unsigned* flags, unsigned* data, int nbar, unsigned* err,
                                                       unsigned* stale) {
    const int nb = gridDim.x, b = blockIdx.x, lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    __shared__ int failed;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    for (int i = 0; i < nbar; ++i) {
        const unsigned tok = (unsigned)i + 1u;
        if (wave == 0) {
            if (MODE == 0) data[b * 64 + lane] = tok * 1000u + b;
            else __hip_atomic_store(&data[b * 64 + lane], tok * 1000u + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            int ok = 0;
            if (MODE == 2) {
                if (lane == 0) {
                    __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    const unsigned target = tok * (unsigned)nb;
                    for (int s = 0; s < kSpin; ++s)
                        if (__hip_atomic_load(flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) >= target) {
                            ok = 1;
                            break;
                        }
                }
                ok = __shfl(ok, 0, 64);
            } else {
                if (lane == 0) store_flag<MODE>(&flags[b], tok);
                for (int s = 0; s < kSpin; ++s) {
                    int all = 1;
                    for (int j = lane; j < nb; j += 64) all &= (load_flag<MODE>(&flags[j]) >= tok);
                    if (__all(all)) {
                        ok = 1;
                        break;
                    }
                }
            }
            if (!ok) {
                if (lane == 0) {
                    atomicAdd(err, 1u);
                    failed = 1;
                }
            } else {
                const int src = (b + 1) % nb;
                const unsigned v = MODE == 0 ? data[src * 64 + lane]
                                             : __hip_atomic_load(&data[src * 64 + lane], __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_SYSTEM);
                if (v < tok * 1000u + src) atomicAdd(stale, 1u);
            }
        }
        __syncthreads();
        if (failed) break;
    }
}

__global__ __launch_bounds__(kThreads) void k_empty(unsigned* p) {
    if (p != nullptr && threadIdx.x == kThreads) p[0] = 1;   // never taken (threadIdx.x < kThreads)
}

}  // namespace

int main() {
    int dev = 0, ncu = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    if (ncu <= 0 || ncu > 4096) return 1;
    unsigned *flags, *data, *err, *stale;
    CHECK(hipMalloc(&flags, 4096 * 4));
    CHECK(hipMalloc(&data, 4096 * 64 * 4));
    CHECK(hipMalloc(&err, 4));
    CHECK(hipMalloc(&stale, 4));
    hipStream_t st;
    CHECK(hipStreamCreate(&st));
    hipEvent_t a, z;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&z));
    const char* names[3] = {"barrier_release_acquire", "barrier_system_relaxed", "barrier_counter"};
    for (int mode = 0; mode < 3; ++mode) {
        for (int nbar : {1, 200}) {
            CHECK(hipMemsetAsync(flags, 0, 4096 * 4, st));
            CHECK(hipMemsetAsync(data, 0, 4096 * 64 * 4, st));
            CHECK(hipMemsetAsync(err, 0, 4, st));
            CHECK(hipMemsetAsync(stale, 0, 4, st));
            CHECK(hipStreamSynchronize(st));
            CHECK(hipEventRecord(a, st));
            if (mode == 0) hipLaunchKernelGGL(k_barriers<0>, dim3(ncu), dim3(kThreads), 0, st, flags, data, nbar, err, stale);
            else if (mode == 1) hipLaunchKernelGGL(k_barriers<1>, dim3(ncu), dim3(kThreads), 0, st, flags, data, nbar, err, stale);
            else hipLaunchKernelGGL(k_barriers<2>, dim3(ncu), dim3(kThreads), 0, st, flags, data, nbar, err, stale);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(z, st));
            CHECK(hipEventSynchronize(z));
            float ms = 0;
            CHECK(hipEventElapsedTime(&ms, a, z));
            unsigned e = 0, sv = 0;
            CHECK(hipMemcpy(&e, err, 4, hipMemcpyDeviceToHost));
            CHECK(hipMemcpy(&sv, stale, 4, hipMemcpyDeviceToHost));
            std::printf("{\"probe\": \"%s\", \"blocks\": %d, \"barriers\": %d, \"us_total\": %.2f, \"us_per_barrier\": %.3f, "
                        "\"timeouts\": %u, \"stale\": %u}\n",
                        names[mode], ncu, nbar, ms * 1e3, ms * 1e3 / nbar, e, sv);
        }
    }
    constexpr int kLaunches = 200;
    for (int rep = 0; rep < 2; ++rep) {
        CHECK(hipEventRecord(a, st));
        for (int i = 0; i < kLaunches; ++i) hipLaunchKernelGGL(k_empty, dim3(ncu), dim3(kThreads), 0, st, nullptr);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(z, st));
        CHECK(hipEventSynchronize(z));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, a, z));
        if (rep) std::printf("{\"probe\": \"kernel_eager\", \"blocks\": %d, \"launches\": %d, \"us_per_kernel\": %.3f}\n", ncu,
                             kLaunches, ms * 1e3 / kLaunches);
    }
    hipGraph_t g;
    hipGraphExec_t ge;
    CHECK(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < kLaunches; ++i) hipLaunchKernelGGL(k_empty, dim3(ncu), dim3(kThreads), 0, st, nullptr);
    CHECK(hipStreamEndCapture(st, &g));
    CHECK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
    for (int rep = 0; rep < 3; ++rep) {
        CHECK(hipEventRecord(a, st));
        CHECK(hipGraphLaunch(ge, st));
        CHECK(hipEventRecord(z, st));
        CHECK(hipEventSynchronize(z));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, a, z));
        if (rep) std::printf("{\"probe\": \"kernel_graph\", \"blocks\": %d, \"launches\": %d, \"us_per_kernel\": %.3f}\n", ncu,
                             kLaunches, ms * 1e3 / kLaunches);
    }
    CHECK(hipGraphExecDestroy(ge));
    CHECK(hipGraphDestroy(g));
    CHECK(hipStreamDestroy(st));
    return 0;
}
