// Router logits and top-k selection with softmax over the chosen k.
//
// The router is resident and cheap next to the experts; its scores pick a few experts per token
// (648news 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute"; 8 of 256 in
// 648news 10-cyber-on-strata-moe-local-inference, section "tiered VRAM/RAM inference").
#include "kernels.h"

namespace moe {

// ----------------------------------------------------------------------------- decode GEMV
// One wave per expert row: W_r row streamed with 16-byte loads, x (T <= 4 tokens) re-read from
// L1/L2, fp32 accumulation, wave reduction.
template <int T>
__global__ __launch_bounds__(64) void k_router_gemv(const float* __restrict__ w_r, const float* __restrict__ bias,
                                                    const uint16_t* __restrict__ x, int H, int E,
                                                    float* __restrict__ logits) {
    const int e = blockIdx.x;
    const int lane = threadIdx.x;
    const float4* wr = reinterpret_cast<const float4*>(w_r + (size_t)e * H);
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    for (int c = lane; c < H / 4; c += kWave) {
        const float4 wv = wr[c];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint2 xv = reinterpret_cast<const uint2*>(x + (size_t)t * H)[c];
            acc[t] += wv.x * bf16_lo(xv.x) + wv.y * bf16_hi(xv.x) + wv.z * bf16_lo(xv.y) + wv.w * bf16_hi(xv.y);
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float s = group_sum<kWave>(acc[t]);
        if (lane == 0) logits[(size_t)t * E + e] = s + (bias ? bias[e] : 0.f);
    }
}

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
// One wave per token. Each lane holds up to 16 logits as 64-bit keys (ordered value, ~index) so
// that one unsigned max picks the larger value and, on equal values, the lower index. k rounds of
// a wave-wide max, then the softmax over the chosen k in fp32 with the first (largest) logit
// subtracted.
__global__ __launch_bounds__(256) void k_topk_softmax(const float* __restrict__ logits, int T, int E, int k,
                                                      int32_t* __restrict__ ids, float* __restrict__ p) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float* l = logits + (size_t)t * E;
    uint64_t keys[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = lane + kWave * i;
        keys[i] = e < E ? ((uint64_t)ordered_key(l[e]) << 32) | (uint32_t)(~(uint32_t)e) : 0ull;
    }
    int mine = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) best = keys[i] > best ? keys[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (keys[i] == best) keys[i] = 0ull;
        if (lane == j) mine = e;
    }
    const float v = lane < k ? l[mine] : 0.f;
    const float vmax = __shfl(v, 0, kWave);
    const float ex = lane < k ? expf(v - vmax) : 0.f;
    const float s = group_sum<kWave>(ex);
    if (lane < k) {
        ids[(size_t)t * k + lane] = mine;
        p[(size_t)t * k + lane] = ex / s;
    }
}

// ----------------------------------------------------------------------------- launchers

moe_status launch_router(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                         float* logits, hipStream_t s) {
    if (T <= 4) {
        switch (T) {
            case 1: hipLaunchKernelGGL(k_router_gemv<1>, dim3(E), dim3(64), 0, s, w_r, bias, x, H, E, logits); break;
            case 2: hipLaunchKernelGGL(k_router_gemv<2>, dim3(E), dim3(64), 0, s, w_r, bias, x, H, E, logits); break;
            case 3: hipLaunchKernelGGL(k_router_gemv<3>, dim3(E), dim3(64), 0, s, w_r, bias, x, H, E, logits); break;
            default: hipLaunchKernelGGL(k_router_gemv<4>, dim3(E), dim3(64), 0, s, w_r, bias, x, H, E, logits); break;
        }
    } else {
        dim3 grid((T + kRgTile - 1) / kRgTile, (E + kRgTile - 1) / kRgTile);
        hipLaunchKernelGGL(k_router_gemm, grid, dim3(256), 0, s, w_r, bias, x, T, H, E, logits);
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* p, hipStream_t s) {
    hipLaunchKernelGGL(k_topk_softmax, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, p);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
