// Token-to-expert permutation: a stable counting sort of the (token, slot) pairs by expert.
//
// Prompt chunks run as grouped expert GEMMs (648news 07-nano-cuda-moe-qwen38-release, section
// "speed comparison and accuracy check", 8K-token chunks), which need the pairs of each expert
// contiguous. Deterministic and atomic-free on the order:
//   1. per chunk of 64 tokens, per-expert counts (LDS histogram; counts do not depend on order),
//      stored expert-major: counts[e][c];
//   2. one block turns counts[e][c] into its exclusive prefix sum in that (expert, chunk) order,
//      which is at once offsets[e] (the value at c = 0) and each chunk's first slot base[e][c];
//   3. per chunk, a pair's rank inside its expert is the number of earlier tokens of the chunk
//      that chose the same expert: a 64-bit LDS mask of tokens per expert, popcount below the lane.
// Token t's k choices are distinct (top-k output), so each token adds at most one pair per expert.
// A pair whose id lies outside [0, E) is dropped: no slot, inv = -1, and offsets[E] counts only
// the kept pairs. Small batches run all three steps in one block (k_perm_small).
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
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
        }
    __syncthreads();
    const int nc = gridDim.x;
    for (int e = lane; e < E; e += kWave) counts[(size_t)e * nc + c] = cnt[e];
}

// One block of 1024 threads: thread i owns the contiguous segment [i * per, (i + 1) * per) of the
// n = E * nchunks counts (per a multiple of 16), sums it, a block scan of the 1024 sums gives each
// segment's start, and a second pass writes the exclusive prefix in place. Counts move 16 per step
// with four independent 16-byte accesses; segments of up to 32 are read once and kept in registers.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ counts, int nchunks, int E,
                                                    int32_t* __restrict__ offsets) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int n = E * nchunks;
    const int per = ((n + 1023) / 1024 + 15) & ~15;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    auto load16 = [&](int i, int (&v)[16]) {
        if (i + 16 <= hi) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int4 w = reinterpret_cast<const int4*>(counts + i)[q];
                v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = i + j < hi ? counts[i + j] : 0;
        }
    };
    // up to 32 counts per thread stay in registers between the two passes (one read of the counts)
    const bool held = per <= 32;
    int h0[16], h1[16];
    int sum = 0;
    if (held) {
        if (lo < hi) load16(lo, h0);
        else
#pragma unroll
            for (int j = 0; j < 16; ++j) h0[j] = 0;
        if (lo + 16 < hi) load16(lo + 16, h1);
        else
#pragma unroll
            for (int j = 0; j < 16; ++j) h1[j] = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) sum += h0[j] + h1[j];
    } else {
        for (int i = lo; i < hi; i += 16) {
            int v[16];
            load16(i, v);
#pragma unroll
            for (int j = 0; j < 16; ++j) sum += v[j];
        }
    }
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;
    int e = lo / nchunks, c = lo - e * nchunks;
    for (int i = lo; i < hi; i += 16) {
        int v[16], o[16];
        if (held) {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = i == lo ? h0[j] : h1[j];
        } else {
            load16(i, v);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            o[j] = run;
            if (c == 0 && i + j < hi) offsets[e] = run;
            run += v[j];
            if (++c == nchunks) { c = 0; ++e; }
        }
        if (i + 16 <= hi) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                reinterpret_cast<int4*>(counts + i)[q] = make_int4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (i + j < hi) counts[i + j] = o[j];
        }
    }
    if (tid == 1023) offsets[E] = run;   // = total when every id is in range
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
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            if ((unsigned)e < (unsigned)E) atomicOr(&tokmask[e], 1ull << lane);
        }
    __syncthreads();
    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int j = 0; j < k; ++j) {
            const int q = t * k + j;
            const int e = ids[q];
            if ((unsigned)e >= (unsigned)E) {
                inv[q] = -1;
                continue;
            }
            const int pos = base[(size_t)e * gridDim.x + c] + __popcll(tokmask[e] & below);
            perm[pos] = q;
            inv[q] = pos;
        }
    }
}

// The same three steps in one block of 1024 threads when the per-(expert, chunk) counts and the
// per-chunk token masks fit in LDS (small batches: one launch instead of three). Wave w takes the
// chunks w, w + 16, ...; thread e takes expert e in the scan (E <= 1024).
__global__ __launch_bounds__(1024) void k_perm_small(const int32_t* __restrict__ ids, int T, int k, int E,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int nc = (T + kChunk - 1) / kChunk;
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);        // [nc][E]
    int32_t* cnt = reinterpret_cast<int32_t*>(mask + (size_t)nc * E);             // [E][nc]
    int32_t* part = cnt + (size_t)E * nc;                                          // [1024]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    constexpr int kWaves = 1024 / kWave;
    for (int i = tid; i < E * nc; i += 1024) {
        cnt[i] = 0;
        mask[i] = 0ull;
    }
    __syncthreads();
    for (int c = wave; c < nc; c += kWaves) {
        const int t = c * kChunk + lane;
        if (t < T)
            for (int j = 0; j < k; ++j) {
                const int e = ids[(size_t)t * k + j];
                if ((unsigned)e < (unsigned)E) {
                    atomicAdd(&cnt[e * nc + c], 1);
                    atomicOr(&mask[(size_t)c * E + e], 1ull << lane);
                }
            }
    }
    __syncthreads();
    int tot = 0;
    if (tid < E)
        for (int c = 0; c < nc; ++c) tot += cnt[tid * nc + c];
    part[tid] = tot;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        int run = part[tid] - tot;
        offsets[tid] = run;
        for (int c = 0; c < nc; ++c) {
            const int v = cnt[tid * nc + c];
            cnt[tid * nc + c] = run;
            run += v;
        }
    }
    if (tid == 1023) offsets[E] = part[1023];   // = kept pairs
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int c = wave; c < nc; c += kWaves) {
        const int t = c * kChunk + lane;
        if (t >= T) continue;
        for (int j = 0; j < k; ++j) {
            const int q = t * k + j;
            const int e = ids[q];
            if ((unsigned)e >= (unsigned)E) {
                inv[q] = -1;
                continue;
            }
            const int pos = cnt[e * nc + c] + __popcll(mask[(size_t)c * E + e] & below);
            perm[pos] = q;
            inv[q] = pos;
        }
    }
}

static size_t perm_small_lds(int T, int E) {
    const size_t nc = (size_t)perm_chunks(T);
    return nc * E * 8 + nc * E * 4 + 1024 * 4;
}

moe_status launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* perm, int32_t* inv,
                          int32_t* scratch, hipStream_t s) {
    const size_t small = perm_small_lds(T, E);
    if (small <= 65536) {
        hipLaunchKernelGGL(k_perm_small, dim3(1), dim3(1024), small, s, ids, T, k, E, offsets, perm, inv);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    }
    const int nc = perm_chunks(T);
    hipLaunchKernelGGL(k_perm_hist, dim3(nc), dim3(64), E * sizeof(int32_t), s, ids, T, k, E, scratch);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, scratch, nc, E, offsets);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_perm_scatter, dim3(nc), dim3(64), E * sizeof(unsigned long long), s, ids, T, k, E,
                       scratch, perm, inv);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
