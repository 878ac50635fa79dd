// Router logits and top-k selection with softmax over the chosen k.
//
// The router is resident and cheap next to the experts; its scores pick a few experts per token
// (648news 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute"; 8 of 256 in
// 648news 10-cyber-on-strata-moe-local-inference, section "tiered VRAM/RAM inference").
#include <algorithm>

#include "kernels.h"
#include "small_batch.h"

namespace moe {

// ----------------------------------------------------------------------------- prefill GEMM
// logits[T][E] = x[T][H] * W_r[E][H]^T + b on the bf16 matrix cores at fp32 accuracy: x is bf16
// already, and each fp32 weight is split into three bf16 terms w = w1 + w2 + w3 (w1 = bf16(w),
// w2 = bf16(w - w1), w3 = bf16(w - w1 - w2); 3 x 8 significant bits hold all 24 of the fp32
// value). Every product x * wi is exact in fp32, so the three MFMAs per fragment pair give the
// fp32 dot product up to the order of the fp32 additions.
//
// Tiles of MT tokens x 64 experts, four waves of MT/2 x 32 (v_mfma_f32_32x32x16_bf16: MT/64 per
// K half-step and weight term; the 16 x 16 x 32 form runs at a far lower rate on this chip), K
// steps of 32 through double-buffered LDS (rows padded to 80 bytes), loads kept two steps ahead in
// registers. MT = 128 for large batches: the three weight terms are most of what a wave reads from
// LDS, and a wave of 64 tokens reads them once for twice the outputs; MT = 64 below, where taller
// tiles would mostly hold padding. Blocks that share token rows are placed on one XCD so that x is
// read once into that XCD's L2.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRtN = 64, kRtK = 32, kRtLds = kRtK + 8, kRtXcds = 8;
constexpr int kRtBigT = 1024;   // tokens from which the tiles are 128 tokens tall
__host__ __device__ constexpr int router_tile_m(int T) { return T >= kRtBigT ? 128 : 64; }

template <int MT> struct RouterSlot {
    u32x4 a[MT / 64];   // 8 MT / 64 bf16 of x
    floatx4 b0, b1;     // 8 fp32 of W_r
};

// Split K (blockIdx.y = split s of `splits`): with more than one split every block writes fp32 partial
// sums of its K range to part[s][T][E] and k_router_reduce (or k_router_reduce_topk) adds them in
// split order plus the bias (deterministic); with one split the block writes logits + bias directly.
template <int MT>
__global__ __launch_bounds__(256, 2) void k_router_mfma(const float* __restrict__ w_r, const float* __restrict__ bias,
                                                        const uint16_t* __restrict__ x, int T, int H, int E,
                                                        float* __restrict__ logits, int splits,
                                                        float* __restrict__ part) {
    constexpr int NI = MT / 64;   // 32-row MFMA tiles per wave (and x vectors per loader thread)
    __shared__ __attribute__((aligned(16))) __bf16 As[2][MT * kRtLds];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][3][kRtN * kRtLds];
    const int mt = (T + MT - 1) / MT, nt = (E + kRtN - 1) / kRtN;
    const int total = mt * nt, per_xcd = (total + kRtXcds - 1) / kRtXcds;
    const int idx = (int)(blockIdx.x / kRtXcds);
    if (idx >= per_xcd) return;
    const int w = (int)(blockIdx.x % kRtXcds) * per_xcd + idx;
    if (w >= total) return;
    const int t0 = (w / nt) * MT, e0 = (w % nt) * kRtN;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / 2, wn = wave % 2;

    // loaders: W_r thread -> row tid / 4, K chunk 8 * (tid % 4); x thread -> row tid / (4 / NI),
    // K chunk 8 NI * (tid % (4 / NI)); rows past T or E are clamped (their outputs are never stored)
    const int lr = tid >> 2, lc = 8 * (tid & 3);
    const int ar = tid / (4 / NI), ac = 8 * NI * (tid % (4 / NI));
    const int nk_all = H / kRtK;
    const int kbeg = (int)(((int64_t)nk_all * blockIdx.y) / splits);
    const int nk = (int)(((int64_t)nk_all * (blockIdx.y + 1)) / splits) - kbeg;
    const uint16_t* ap = x + (size_t)min(t0 + ar, T - 1) * H + ac + (size_t)kbeg * kRtK;
    const float* bp = w_r + (size_t)min(e0 + lr, E - 1) * H + lc + (size_t)kbeg * kRtK;
    auto gload = [&](RouterSlot<MT>& sl, int ks) __attribute__((always_inline)) {
        ks = min(ks, nk - 1);
#pragma unroll
        for (int i = 0; i < NI; ++i) sl.a[i] = *reinterpret_cast<const u32x4*>(ap + ks * kRtK + 8 * i);
        sl.b0 = *reinterpret_cast<const floatx4*>(bp + ks * kRtK);
        sl.b1 = *reinterpret_cast<const floatx4*>(bp + ks * kRtK + 4);
    };
    auto lstore = [&](const RouterSlot<MT>& sl, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(&As[st][ar * kRtLds + ac + 8 * i]) = sl.a[i];
        const float v[8] = {sl.b0.x, sl.b0.y, sl.b0.z, sl.b0.w, sl.b1.x, sl.b1.y, sl.b1.z, sl.b1.w};
        bf16x8 p1, p2, p3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const __bf16 h1 = (__bf16)v[i];
            const float r1 = v[i] - (float)h1;
            const __bf16 h2 = (__bf16)r1;
            const float r2 = r1 - (float)h2;
            p1[i] = h1;
            p2[i] = h2;
            p3[i] = (__bf16)r2;
        }
        *reinterpret_cast<bf16x8*>(&Bs[st][0][lr * kRtLds + lc]) = p1;
        *reinterpret_cast<bf16x8*>(&Bs[st][1][lr * kRtLds + lc]) = p2;
        *reinterpret_cast<bf16x8*>(&Bs[st][2][lr * kRtLds + lc]) = p3;
    };

    floatx16 acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    const int kofs = 8 * (lane / 32);
    auto kstep = [&](int ks, const RouterSlot<MT>& next_sl, RouterSlot<MT>& refill) __attribute__((always_inline)) {
        const int cur = ks & 1;
        bf16x8 a[NI][2], b[3][2];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                a[i][h] = *reinterpret_cast<const bf16x8*>(
                    &As[cur][(wm * (MT / 2) + 32 * i + lane % 32) * kRtLds + 16 * h + kofs]);
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                b[p][h] = *reinterpret_cast<const bf16x8*>(&Bs[cur][p][(wn * 32 + lane % 32) * kRtLds + 16 * h + kofs]);
        // each half of the step: smallest terms first
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 2; p >= 0; --p)
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][h], b[p][h], acc[i], 0, 0, 0);
        lstore(next_sl, cur ^ 1);
        gload(refill, ks + 3);
        __syncthreads();
    };
    // two register slots: s0 holds even steps, s1 odd steps
    RouterSlot<MT> s0, s1;
    gload(s0, 0);
    gload(s1, 1);
    lstore(s0, 0);
    gload(s0, 2);
    __syncthreads();
    int ks = 0;
    for (; ks + 2 <= nk; ks += 2) {
        kstep(ks, s1, s1);       // writes step ks + 1 (odd), refills s1 with ks + 3
        kstep(ks + 1, s0, s0);   // writes step ks + 2 (even), refills s0 with ks + 4
    }
    if (ks < nk) kstep(ks, s1, s1);

    {
        const int e = e0 + wn * 32 + lane % 32;
        if (e < E) {
            const float b = splits == 1 && bias ? bias[e] : 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = t0 + wm * (MT / 2) + 32 * i + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                    if (t >= T) continue;
                    if (splits == 1) logits[(size_t)t * E + e] = acc[i][r] + b;
                    else part[((size_t)blockIdx.y * T + t) * E + e] = acc[i][r];
                }
        }
    }
}

__global__ __launch_bounds__(256) void k_router_reduce(const float* __restrict__ part, int splits, int T, int E,
                                                       const float* __restrict__ bias, float* __restrict__ logits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * E) return;
    float acc = 0.f;
    const int64_t stride = (int64_t)T * E;
    for (int sp0 = 0; sp0 < splits; sp0 += 4) {   // four loads in flight, added in split order
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = part[min(sp0 + j, splits - 1) * stride + i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (sp0 + j < splits) acc += v[j];
    }
    logits[i] = acc + (bias ? bias[i % E] : 0.f);
}

// ----------------------------------------------------------------------------- top-k + softmax
// One wave per token (topk_wave): k rounds of a DPP wave max over order-preserving keys, ties to the
// lower expert index, then the softmax over the chosen k.
template <int KPL>
__global__ __launch_bounds__(256) void k_topk_softmax(const float* __restrict__ logits, int T, int E, int k,
                                                      int32_t* __restrict__ ids, float* __restrict__ p) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    int id;
    float pr;
    topk_wave<KPL>(logits + (size_t)t * E, E, k, id, pr);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        p[(size_t)t * k + lane] = pr;
    }
}

// Split-K reduction fused with the top-k: one wave per token adds the partial sums of its experts
// in split order plus the bias (the logits written are the values the top-k sees), then selects.
template <int KPL>
__global__ __launch_bounds__(256) void k_router_reduce_topk(const float* __restrict__ part, int splits, int T,
                                                            int E, int k, const float* __restrict__ bias,
                                                            float* __restrict__ logits, int32_t* __restrict__ ids,
                                                            float* __restrict__ p) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    float lv[KPL];
    router_reduce_token<KPL>(part, splits, T, E, t, bias, logits, lv);
    int id;
    float pr;
    topk_wave_regs<KPL>(lv, E, k, id, pr);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        p[(size_t)t * k + lane] = pr;
    }
}

// ----------------------------------------------------------------------------- launchers

// Splits of K for the router GEMM: more blocks when the tiles alone would not fill the GPU (at most
// 128 of them: one per two CUs), at least four K steps of 32 per split.
static int router_blocks(int T, int E) {
    const int m = router_tile_m(T);
    return ((T + m - 1) / m) * ((E + kRtN - 1) / kRtN);
}

int router_splits(int T, int H, int E) {
    const int blocks = router_blocks(T, E);
    int sp = blocks > 128 ? 1 : 256 / blocks;
    sp = std::min(sp, 16);
    sp = std::min(sp, (H / kRtK) / 4);
    return std::max(sp, 1);
}

size_t router_scratch_bytes(int T, int H, int E) {
    const int sp = router_splits(T, H, E);
    return sp > 1 ? (size_t)sp * T * E * sizeof(float) : 0;
}

moe_status launch_router(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                         float* logits, float* scratch, hipStream_t s) {
    const int sp = router_splits(T, H, E);
    if (sp > 1 && !scratch) return MOE_ERR_WORKSPACE;
    const int grid = ((router_blocks(T, E) + kRtXcds - 1) / kRtXcds) * kRtXcds;
    if (router_tile_m(T) == 128)
        hipLaunchKernelGGL(k_router_mfma<128>, dim3(grid, sp), dim3(256), 0, s, w_r, bias, x, T, H, E, logits, sp, scratch);
    else
        hipLaunchKernelGGL(k_router_mfma<64>, dim3(grid, sp), dim3(256), 0, s, w_r, bias, x, T, H, E, logits, sp, scratch);
    MOE_LAUNCH_CHECK();
    if (sp > 1) {
        const int64_t n = (int64_t)T * E;
        hipLaunchKernelGGL(k_router_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, scratch, sp, T, E,
                           bias, logits);
        MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
}

// The router GEMM alone: with router_splits() > 1 it writes the split-K partial sums to scratch (to
// be reduced by k_router_reduce_topk), else logits + bias.
static moe_status launch_router_partials(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                                         float* logits, float* scratch, hipStream_t s) {
    const int sp = router_splits(T, H, E);
    if (sp > 1 && !scratch) return MOE_ERR_WORKSPACE;
    const int grid = ((router_blocks(T, E) + kRtXcds - 1) / kRtXcds) * kRtXcds;
    if (router_tile_m(T) == 128)
        hipLaunchKernelGGL(k_router_mfma<128>, dim3(grid, sp), dim3(256), 0, s, w_r, bias, x, T, H, E, logits, sp, scratch);
    else
        hipLaunchKernelGGL(k_router_mfma<64>, dim3(grid, sp), dim3(256), 0, s, w_r, bias, x, T, H, E, logits, sp, scratch);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_route_topk(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E, int k,
                             float* logits, int32_t* ids, float* p, float* scratch, hipStream_t s) {
    const int sp = router_splits(T, H, E);
    if (sp == 1) {
        const moe_status st = launch_router(w_r, bias, x, T, H, E, logits, scratch, s);
        return st != MOE_OK ? st : launch_topk(logits, T, E, k, ids, p, s);
    }
    const moe_status st = launch_router_partials(w_r, bias, x, T, H, E, logits, scratch, s);
    if (st != MOE_OK) return st;
    const dim3 g2((T + 3) / 4), b2(256);
    if (E <= 64) hipLaunchKernelGGL(k_router_reduce_topk<1>, g2, b2, 0, s, scratch, sp, T, E, k, bias, logits, ids, p);
    else if (E <= 128) hipLaunchKernelGGL(k_router_reduce_topk<2>, g2, b2, 0, s, scratch, sp, T, E, k, bias, logits, ids, p);
    else if (E <= 256) hipLaunchKernelGGL(k_router_reduce_topk<4>, g2, b2, 0, s, scratch, sp, T, E, k, bias, logits, ids, p);
    else if (E <= 512) hipLaunchKernelGGL(k_router_reduce_topk<8>, g2, b2, 0, s, scratch, sp, T, E, k, bias, logits, ids, p);
    else hipLaunchKernelGGL(k_router_reduce_topk<16>, g2, b2, 0, s, scratch, sp, T, E, k, bias, logits, ids, p);
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
