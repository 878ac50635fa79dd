// Token-to-expert permutation: a stable counting sort of the (token, slot) pairs by expert.
//
// Prompt chunks run as grouped expert GEMMs (648news 07-nano-cuda-moe-qwen38-release, section
// "speed comparison and accuracy check", 8K-token chunks), which need the pairs of each expert
// contiguous. Deterministic and atomic-free on the order:
//   1. per chunk of 64 tokens, per-expert counts (LDS histogram; counts do not depend on order),
//      stored expert-major: counts[e][c];
//   2. one wave per expert turns its counts[e][c] into their exclusive prefix (the chunk's base
//      inside the expert) and writes the expert's total; the offsets are the exclusive prefix of
//      the totals, which every step-3 block derives itself (block 0 writes them out);
//   3. per chunk, a pair's rank inside its expert is the number of earlier tokens of the chunk
//      that chose the same expert: a 64-bit LDS mask of tokens per expert, popcount below the lane.
// Token t's k choices are distinct (top-k output), so each token adds at most one pair per expert.
// A pair whose id lies outside [0, E) is dropped: no slot, inv = -1, and offsets[E] counts only
// the kept pairs. Small batches run all three steps in one block (k_perm_small).
#include "kernels.h"
#include "small_batch.h"

namespace moe {

int perm_chunks(int T) { return (T + kChunk - 1) / kChunk; }
size_t perm_scratch_ints(int T, int E) { return (size_t)(perm_chunks(T) + 1) * E; }

// A token's k <= kMaxTopK expert ids, loaded together (unconditional, clamped loads: one round trip,
// not k); ids past k read as -1.
__device__ __forceinline__ void token_ids(const int32_t* __restrict__ ids, int T, int k, int t, int (&ev)[kMaxTopK]) {
    const size_t row = (size_t)min(t, T - 1) * k;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) ev[j] = ids[row + min(j, k - 1)];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j >= k) ev[j] = -1;
}

__global__ __launch_bounds__(64) void k_perm_hist(const int32_t* __restrict__ ids, int T, int k, int E,
                                                  int32_t* __restrict__ counts) {
    extern __shared__ int32_t cnt[];
    const int c = blockIdx.x, lane = threadIdx.x;
    const int t = c * kChunk + lane;
    int ev[kMaxTopK];
    token_ids(ids, T, k, t, ev);
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    __syncthreads();
    if (t < T) {
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if ((unsigned)ev[j] < (unsigned)E) atomicAdd(&cnt[ev[j]], 1);
    }
    __syncthreads();
    const int nc = gridDim.x;
    for (int e = lane; e < E; e += kWave) counts[(size_t)e * nc + c] = cnt[e];
}

// Exclusive prefix of a wave's per-lane values (every lane also gets the total).
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
    const int lane = threadIdx.x % kWave;
    int incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += u;
    }
    total = __shfl(incl, kWave - 1, kWave);
    return incl - v;
}

// One wave per expert: the counts of its chunks (contiguous, expert-major) become their exclusive
// prefix in place, and the expert's total goes to totals[e].
__global__ __launch_bounds__(64) void k_perm_scan_expert(int32_t* __restrict__ counts, int nchunks,
                                                         int32_t* __restrict__ totals) {
    const int e = blockIdx.x, lane = threadIdx.x;
    int32_t* row = counts + (size_t)e * nchunks;
    const int per = (nchunks + kWave - 1) / kWave;
    const int lo = min(lane * per, nchunks), hi = min(lo + per, nchunks);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += row[i];
    int total;
    int run = wave_excl_scan(sum, total);
    for (int i = lo; i < hi; ++i) {
        const int v = row[i];
        row[i] = run;
        run += v;
    }
    if (lane == 0) totals[e] = total;
}

// Per chunk: the experts' offsets are the exclusive prefix of their totals (every block derives
// them from the E totals itself; block 0 also writes them out), a pair's slot is its expert's
// offset + the chunk's base inside the expert + its rank among the chunk's tokens of that expert.
__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t* __restrict__ ids, int T, int k, int E,
                                                     const int32_t* __restrict__ base,
                                                     const int32_t* __restrict__ totals,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
    extern __shared__ unsigned long long tokmask[];
    int32_t* offs = reinterpret_cast<int32_t*>(tokmask + E);   // [E + 1]
    const int c = blockIdx.x, lane = threadIdx.x;
    const int t = c * kChunk + lane;
    // the token's ids and this lane's E / 64 <= 16 expert totals, each group loaded together
    int ev[kMaxTopK];
    token_ids(ids, T, k, t, ev);
    const int per = (E + kWave - 1) / kWave;
    const int lo = min(lane * per, E), hi = min(lo + per, E);
    int tv[kMaxTopK];
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) tv[i] = totals[min(lo + i, E - 1)];
    for (int e = lane; e < E; e += kWave) tokmask[e] = 0ull;
    {
        int sum = 0;
#pragma unroll
        for (int i = 0; i < kMaxTopK; ++i)
            if (lo + i < hi) sum += tv[i];
        int total;
        int run = wave_excl_scan(sum, total);
#pragma unroll
        for (int i = 0; i < kMaxTopK; ++i)
            if (lo + i < hi) {
                offs[lo + i] = run;
                run += tv[i];
            }
        if (lane == 0) offs[E] = total;   // = kept pairs
    }
    __syncthreads();
    if (c == 0)
        for (int e = lane; e <= E; e += kWave) offsets[e] = offs[e];
    if (t < T) {
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if ((unsigned)ev[j] < (unsigned)E) atomicOr(&tokmask[ev[j]], 1ull << lane);
    }
    __syncthreads();
    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
        // the chunk's base inside each chosen expert, all k loaded together
        int bv[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            bv[j] = base[(size_t)min(max(ev[j], 0), E - 1) * gridDim.x + c];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j >= k) break;
            const int q = t * k + j;
            const int e = ev[j];
            if ((unsigned)e >= (unsigned)E) {
                inv[q] = -1;
                continue;
            }
            const int pos = offs[e] + bv[j] + __popcll(tokmask[e] & below);
            perm[pos] = q;
            inv[q] = pos;
        }
    }
}

// The same three steps in one block of 1024 threads when the per-(expert, chunk) counts and the
// per-chunk token masks fit in LDS (small batches: one launch instead of three).
__global__ __launch_bounds__(1024) void k_perm_small(const int32_t* __restrict__ ids, int T, int k, int E,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    perm_small_block(ids, T, k, E, offsets, perm, inv, smem, nullptr);
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
    int32_t* totals = scratch + (size_t)nc * E;
    hipLaunchKernelGGL(k_perm_hist, dim3(nc), dim3(64), E * sizeof(int32_t), s, ids, T, k, E, scratch);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_perm_scan_expert, dim3(E), dim3(64), 0, s, scratch, nc, totals);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_perm_scatter, dim3(nc), dim3(64), E * sizeof(unsigned long long) + (E + 1) * sizeof(int32_t),
                       s, ids, T, k, E, scratch, totals, offsets, perm, inv);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
