// Measurement program (not part of libmoe.so): how fast this GPU streams the bytes of one decode
// expert stage when nothing but the read is done, under the protocol the decode benchmark uses:
// 48 distinct buffers resident in HBM (more than the Infinity Cache holds), read back to back as the
// nodes of one HIP graph, each node waiting for the previous one.
//
// The decode pages price a token by the expert bytes it reads (648news
// 10-cyber-on-strata-moe-local-inference, section on bitwise validation and the speed bottleneck);
// this is the ceiling such a stage meets on this GPU at this size, with and without a kernel boundary
// in the middle. Printed, one JSON object per line:
//   one_kernel: one read kernel per buffer of B bytes, for the expert stages of the decode shapes:
//       15,925,248 (one token, 256 experts top-8 + a shared expert, 4-bit codes), 56,819,712 (four
//       tokens of the same layer with 8-bit codes: 16 distinct experts + the shared one) and
//       14,745,600 (one token, 512 experts top-10, 2-bit codes);
//   two_kernels: the same bytes as two dependent kernels per buffer (2/3 then 1/3, the split of the
//       gate/up and down weights);
//   for grids of 256, 512 and 1024 blocks of 256 threads (every thread keeps 8 16-byte loads in
//   flight per step).
// Each kernel folds what it reads into one word per block, written out, so nothing is optimised away.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

#define CHECK(x)                                                                             \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
            std::exit(1);                                                                    \
        }                                                                                    \
    } while (0)

constexpr int kThreads = 256;
constexpr int kInFlight = 8;       // 16-byte loads per thread and step
constexpr int kBuffers = 48;
constexpr size_t kSizes[] = {15925248, 56819712, 14745600};
constexpr int kReps = 20;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Reads n 16-byte words; every thread issues kInFlight loads before folding them.
__global__ __launch_bounds__(kThreads) void k_read(const u32x4* __restrict__ src, size_t n,
                                                   unsigned* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    unsigned acc = 0;
    for (size_t i0 = (size_t)blockIdx.x * kThreads + threadIdx.x; i0 < n; i0 += stride * kInFlight) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const size_t i = i0 + (size_t)j * stride;
            v[j] = src[i < n ? i : n - 1];   // unconditional, so that all of them are in flight
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) acc ^= v[j].x + v[j].y + v[j].z + v[j].w;
    }
    __shared__ unsigned red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned s = 0;
        for (int i = 0; i < kThreads; ++i) s ^= red[i];
        out[blockIdx.x] = s;
    }
}

float time_graph(hipStream_t s, const std::vector<u32x4*>& bufs, size_t bytes, unsigned* out, int blocks,
                 bool split) {
    const size_t n = bytes / 16;
    const size_t n1 = split ? (n * 2) / 3 : n;
    hipGraph_t g;
    hipGraphExec_t ge;
    CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
    for (u32x4* b : bufs) {
        hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kThreads), 0, s, b, n1, out);
        if (split) hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kThreads), 0, s, b + n1, n - n1, out);
    }
    CHECK(hipStreamEndCapture(s, &g));
    CHECK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
    for (int i = 0; i < 3; ++i) CHECK(hipGraphLaunch(ge, s));
    CHECK(hipStreamSynchronize(s));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    CHECK(hipEventRecord(a, s));
    for (int i = 0; i < kReps; ++i) CHECK(hipGraphLaunch(ge, s));
    CHECK(hipEventRecord(b, s));
    CHECK(hipEventSynchronize(b));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, a, b));
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(b));
    CHECK(hipGraphExecDestroy(ge));
    CHECK(hipGraphDestroy(g));
    return ms * 1000.f / (kReps * kBuffers);   // us per buffer
}

}  // namespace

int main() {
    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    unsigned* out = nullptr;
    CHECK(hipMalloc(&out, 4096 * sizeof(unsigned)));
    for (size_t bytes : kSizes) {
        std::vector<u32x4*> bufs(kBuffers);
        for (auto& b : bufs) {
            CHECK(hipMalloc(&b, bytes));
            CHECK(hipMemset(b, 0x5a, bytes));
        }
        CHECK(hipDeviceSynchronize());
        for (int blocks : {256, 512, 1024}) {
            for (bool split : {false, true}) {
                const float us = time_graph(s, bufs, bytes, out, blocks, split);
                std::printf("{\"probe\": \"%s\", \"blocks\": %d, \"bytes\": %zu, \"us_per_buffer\": %.2f, "
                            "\"GB_per_s\": %.1f}\n",
                            split ? "two_kernels" : "one_kernel", blocks, bytes, us, bytes / (us * 1e3));
                std::fflush(stdout);
            }
        }
        for (auto& b : bufs) CHECK(hipFree(b));
    }
    CHECK(hipFree(out));
    CHECK(hipStreamDestroy(s));
    return 0;
}
