// Router logits and top-k selection with softmax over the chosen k.
//
// The router is resident and cheap next to the experts; its scores pick a few experts per token
// (648news 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute"; 8 of 256 in
// 648news 10-cyber-on-strata-moe-local-inference, section "tiered VRAM/RAM inference").
#include "kernels.h"

namespace moe {

// ----------------------------------------------------------------------------- prefill GEMM
// logits[T][E] = x[T][H] * W_r[E][H]^T + b, fp32 FMA tiles of 64 tokens x 64 experts.
constexpr int kRgTile = 64, kRgK = 32;

__global__ __launch_bounds__(256) void k_router_gemm(const float* __restrict__ w_r, const float* __restrict__ bias,
                                                     const uint16_t* __restrict__ x, int T, int H, int E,
                                                     float* __restrict__ logits) {
    __shared__ float xs[kRgK][kRgTile + 4];
    __shared__ float ws[kRgK][kRgTile + 4];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kRgTile, e0 = blockIdx.y * kRgTile;
    const int ty = tid / 16, tx = tid % 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < H; k0 += kRgK) {
        // 64 rows x 32 k of each operand: 8 elements per thread
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / kRgK, kk = idx % kRgK;
            const int t = t0 + r, e = e0 + r;
            xs[kk][r] = t < T ? bf16_to_f32(x[(size_t)t * H + k0 + kk]) : 0.f;
            ws[kk][r] = e < E ? w_r[(size_t)e * H + k0 + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kRgK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
        }
    }
}

// ----------------------------------------------------------------------------- top-k + softmax
// One wave per token (topk_wave): k rounds of a DPP wave max over order-preserving keys, ties to the
// lower expert index, then the softmax over the chosen k.
template <int KPL>
__global__ __launch_bounds__(256) void k_topk_softmax(const float* __restrict__ logits, int T, int E, int k,
                                                      int32_t* __restrict__ ids, float* __restrict__ p) {
    const int t = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (t >= T) return;
    int id;
    float pr;
    topk_wave<KPL>(logits + (size_t)t * E, E, k, id, pr);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        p[(size_t)t * k + lane] = pr;
    }
}

// ----------------------------------------------------------------------------- launchers

moe_status launch_router(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                         float* logits, hipStream_t s) {
    dim3 grid((T + kRgTile - 1) / kRgTile, (E + kRgTile - 1) / kRgTile);
    hipLaunchKernelGGL(k_router_gemm, grid, dim3(256), 0, s, w_r, bias, x, T, H, E, logits);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* p, hipStream_t s) {
    const dim3 grid((T + 3) / 4), block(256);
    if (E <= 64) hipLaunchKernelGGL(k_topk_softmax<1>, grid, block, 0, s, logits, T, E, k, ids, p);
    else if (E <= 128) hipLaunchKernelGGL(k_topk_softmax<2>, grid, block, 0, s, logits, T, E, k, ids, p);
    else if (E <= 256) hipLaunchKernelGGL(k_topk_softmax<4>, grid, block, 0, s, logits, T, E, k, ids, p);
    else if (E <= 512) hipLaunchKernelGGL(k_topk_softmax<8>, grid, block, 0, s, logits, T, E, k, ids, p);
    else hipLaunchKernelGGL(k_topk_softmax<16>, grid, block, 0, s, logits, T, E, k, ids, p);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
