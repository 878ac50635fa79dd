// Token-to-expert permutation: a stable counting sort of the (token, slot) pairs by expert.
//
// Prompt chunks run as grouped expert GEMMs (648news 07-nano-cuda-moe-qwen38-release, section
// "speed comparison and accuracy check", 8K-token chunks), which need the pairs of each expert
// contiguous. Deterministic and atomic-free on the order:
//   1. per chunk of 64 tokens, per-expert counts (LDS histogram; counts do not depend on order);
//   2. one block scans counts expert-major, chunk-minor -> offsets[e] and each chunk's base[c][e];
//   3. per chunk, a pair's rank inside its expert is the number of earlier tokens of the chunk
//      that chose the same expert: a 64-bit LDS mask of tokens per expert, popcount below the lane.
// Token t's k choices are distinct (top-k output), so each token adds at most one pair per expert.
#include "kernels.h"

namespace moe {

constexpr int kChunk = 64;

int perm_chunks(int T) { return (T + kChunk - 1) / kChunk; }

__global__ __launch_bounds__(64) void k_perm_hist(const int32_t* __restrict__ ids, int T, int k, int E,
                                                  int32_t* __restrict__ counts) {
    extern __shared__ int32_t cnt[];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    __syncthreads();
    const int t = c * kChunk + lane;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicAdd(&cnt[ids[(size_t)t * k + j]], 1);
    __syncthreads();
    for (int e = lane; e < E; e += kWave) counts[(size_t)c * E + e] = cnt[e];
}

// One block of 1024 threads, one thread per expert.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ counts, int nchunks, int E, int total,
                                                    int32_t* __restrict__ offsets) {
    __shared__ int32_t part[1024];
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
        for (int c = 0; c < nchunks; ++c) tot += counts[(size_t)c * E + e];
    part[e] = e < E ? tot : 0;
    __syncthreads();
    // inclusive Hillis-Steele scan over 1024 entries
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = e >= d ? part[e - d] : 0;
        __syncthreads();
        part[e] += v;
        __syncthreads();
    }
    if (e < E) {
        int base = part[e] - tot;  // exclusive
        offsets[e] = base;
        for (int c = 0; c < nchunks; ++c) {
            const int v = counts[(size_t)c * E + e];
            counts[(size_t)c * E + e] = base;
            base += v;
        }
    }
    if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t* __restrict__ ids, int T, int k, int E,
                                                     const int32_t* __restrict__ base, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
    extern __shared__ unsigned long long tokmask[];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) tokmask[e] = 0ull;
    __syncthreads();
    const int t = c * kChunk + lane;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicOr(&tokmask[ids[(size_t)t * k + j]], 1ull << lane);
    __syncthreads();
    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int j = 0; j < k; ++j) {
            const int q = t * k + j;
            const int e = ids[q];
            const int pos = base[(size_t)c * E + e] + __popcll(tokmask[e] & below);
            perm[pos] = q;
            inv[q] = pos;
        }
    }
}

moe_status launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* perm, int32_t* inv,
                          int32_t* scratch, hipStream_t s) {
    const int nc = perm_chunks(T);
    hipLaunchKernelGGL(k_perm_hist, dim3(nc), dim3(64), E * sizeof(int32_t), s, ids, T, k, E, scratch);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, scratch, nc, E, T * k, offsets);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_perm_scatter, dim3(nc), dim3(64), E * sizeof(unsigned long long), s, ids, T, k, E,
                       scratch, perm, inv);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
