// Device steps shared between kernels of the small and mid-size batch paths: the per-token reduction
// of the router GEMM's split-K partial sums (k_router_reduce_topk), and the token-to-expert
// permutation of a batch done by one block (k_perm_small, k_route_small).
#pragma once

#include "common.h"

namespace moe {

constexpr int kChunk = 64;   // tokens per permutation chunk (one 64-bit token mask per expert)

// Logits of token t from the split-K partial sums part[s][T][E] of the router GEMM: the splits are
// added in split order (the loads of 64 / KPL splits in flight at a time, clamped so that they are
// unconditional: one round trip for the usual 16 splits of 256 experts), then the bias; lane + 64 i
// holds expert e. The values written to logits are the values returned.
template <int KPL>
__device__ __forceinline__ void router_reduce_token(const float* __restrict__ part, int splits, int T, int E, int t,
                                                    const float* __restrict__ bias, float* __restrict__ logits,
                                                    float (&lv)[KPL]) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int i = 0; i < KPL; ++i) lv[i] = 0.f;
    const int64_t stride = (int64_t)T * E;
    constexpr int NB = KPL >= 16 ? 4 : 64 / KPL;   // splits per batch of loads
    for (int sp0 = 0; sp0 < splits; sp0 += NB) {
        float v[NB][KPL];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float* ps = part + min(sp0 + j, splits - 1) * stride + (int64_t)t * E;
#pragma unroll
            for (int i = 0; i < KPL; ++i) v[j][i] = ps[min(lane + kWave * i, E - 1)];
        }
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (sp0 + j < splits) {
#pragma unroll
                for (int i = 0; i < KPL; ++i) lv[i] += v[j][i];
            }
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + kWave * i;
        lv[i] += bias ? bias[min(e, E - 1)] : 0.f;
        if (e < E) logits[(int64_t)t * E + e] = lv[i];
    }
}

// LDS bytes of perm_small_block (the last 4 KB hold the 16 wave totals of the expert scan).
__host__ __device__ inline size_t perm_small_lds(int T, int E) {
    const size_t nc = (size_t)((T + kChunk - 1) / kChunk);
    return nc * E * 8 + nc * E * 4 + 1024 * 4;
}

// The stable counting sort of the pairs q = t k + j by expert, all three steps in one block of 1024
// threads (per-chunk counts and token masks in LDS, smem of perm_small_lds bytes): thread i takes
// the pairs i, i + 1024, ... in the counting and placing steps (a token's experts are distinct, so
// its bit in an expert's chunk mask ranks its pair there); thread e takes expert e in the scan
// (E <= 1024). ids may be global or LDS.
// offsets[E + 1] (global) and, when offs_lds is given, a copy of them in LDS for the same block.
// A pair whose id lies outside [0, E) is dropped: inv = -1, offsets[E] counts the kept pairs.
__device__ inline void perm_small_block(const int32_t* ids, int T, int k, int E, int32_t* __restrict__ offsets,
                                        int32_t* __restrict__ perm, int32_t* __restrict__ inv, char* smem,
                                        int32_t* offs_lds) {
    const int nc = (T + kChunk - 1) / kChunk;
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);        // [nc][E]
    int32_t* cnt = reinterpret_cast<int32_t*>(mask + (size_t)nc * E);             // [E][nc]
    int32_t* wsum = cnt + (size_t)E * nc;                                          // [16]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    constexpr int kWaves = 1024 / kWave;
    for (int i = tid; i < E * nc; i += 1024) {
        cnt[i] = 0;
        mask[i] = 0ull;
    }
    __syncthreads();
    for (int q = tid; q < T * k; q += 1024) {
        const int t = q / k, c = t / kChunk;
        const int e = ids[q];
        if ((unsigned)e < (unsigned)E) {
            atomicAdd(&cnt[e * nc + c], 1);
            atomicOr(&mask[(size_t)c * E + e], 1ull << (t % kChunk));
        }
    }
    __syncthreads();
    // exclusive prefix over the experts' totals: a scan inside each wave, then the wave totals
    int tot = 0;
    if (tid < E)
        for (int c = 0; c < nc; ++c) tot += cnt[tid * nc + c];
    int incl = tot;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += u;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? wsum[w] : 0;
        all += wsum[w];
    }
    if (tid < E) {
        int run = before + incl - tot;
        offsets[tid] = run;
        if (offs_lds) offs_lds[tid] = run;
        for (int c = 0; c < nc; ++c) {
            const int v = cnt[tid * nc + c];
            cnt[tid * nc + c] = run;
            run += v;
        }
    }
    if (tid == 0) {   // = kept pairs
        offsets[E] = all;
        if (offs_lds) offs_lds[E] = all;
    }
    __syncthreads();
    for (int q = tid; q < T * k; q += 1024) {
        const int t = q / k, c = t / kChunk;
        const int e = ids[q];
        if ((unsigned)e >= (unsigned)E) {
            inv[q] = -1;
            continue;
        }
        const unsigned long long below = (1ull << (t % kChunk)) - 1ull;
        const int pos = cnt[e * nc + c] + __popcll(mask[(size_t)c * E + e] & below);
        perm[pos] = q;
        inv[q] = pos;
    }
}

}  // namespace moe
