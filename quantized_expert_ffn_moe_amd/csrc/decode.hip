// Decode-regime experts (1 <= T <= 4 tokens): fused dequantise + GEMV, HBM-bound.
//
// Decode on the pages runs the selected experts' weights on the GPU and prices each token by the
// expert bytes it reads (648news 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU
// compute"; 648news 10-cyber-on-strata-moe-local-inference, section "bitwise validation and speed
// bottleneck", about 117 MB of weights per token). Here every expert is resident in HBM, so the
// kernels stream exactly the packed bytes of the distinct chosen experts plus the shared expert.
//
// Phase 1 (gate/up): one wave per (expert slot, row n); lane l owns 32-element blocks l, l+64, ...
//   g_t = sum G[n][:] x_t, u_t = sum U[n][:] x_t, h[slot][t][n] = silu(g_t) * u_t.
// Phase 2 (down): a 16-lane group per (expert slot, output row m), y = D[m][:] h[slot][t][:].
// Tokens that share an expert share one read of its weights (the union of the T*k choices).
#include "kernels.h"

namespace moe {

// Union of the chosen experts of T tokens, built by wave 0 of every block from ids (T*k <= 64).
struct DecodeRouting {
    int nU;                  // distinct routed experts
    int expert[64];          // slot -> expert id (slots in order of first appearance)
    uint32_t tokmask[64];    // slot -> bitmask of tokens that chose it
    int pair_of[64][4];      // slot, token -> pair index q (or -1)
};

__device__ void build_routing(const int32_t* __restrict__ ids, int T, int k, DecodeRouting& r) {
    const int lane = threadIdx.x;  // wave 0 only
    const int P = T * k;
    const int q = lane;
    const int e = q < P ? ids[q] : -1;
    int first_q = q;
    for (int q2 = 0; q2 < 64; ++q2) {
        const int e2 = __shfl(e, q2, kWave);
        if (q2 < q && e2 == e && first_q == q) first_q = q2;
    }
    const uint64_t firsts = __ballot(q < P && first_q == q);
    const int slot = __popcll(firsts & ((1ull << first_q) - 1ull));
    r.tokmask[lane] = 0u;
    for (int t = 0; t < 4; ++t) r.pair_of[lane][t] = -1;
    __builtin_amdgcn_wave_barrier();
    if (q < P) {
        if (first_q == q) r.expert[slot] = e;
        atomicOr(&r.tokmask[slot], 1u << (q / k));
        r.pair_of[slot][q / k] = q;
    }
    if (lane == 0) r.nU = __popcll(firsts);
}

template <int FMT, int T>
__global__ __launch_bounds__(256) void k_decode_gateup(LayerView L, const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ ids, float* __restrict__ h) {
    __shared__ DecodeRouting R;
    if (threadIdx.x < kWave) build_routing(ids, T, L.k, R);
    __syncthreads();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int P = T * L.k;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    int slot, n, e;
    uint32_t mask;
    const uint8_t *gc, *uc;
    const uint16_t *gs, *us;
    const int64_t rb = row_bytes(FMT, L.H);
    const int nb = L.H / 32;
    if (r < (int64_t)P * L.I) {
        slot = (int)(r / L.I);
        n = (int)(r % L.I);
        if (slot >= R.nU) return;
        e = R.expert[slot];
        mask = R.tokmask[slot];
        const int64_t row = (int64_t)e * L.I + n;
        gc = L.g_codes + row * rb; uc = L.u_codes + row * rb;
        gs = L.g_scales + row * nb; us = L.u_scales + row * nb;
    } else {
        n = (int)(r - (int64_t)P * L.I);
        if (L.Is == 0 || n >= L.Is) return;
        slot = P;
        mask = (1u << T) - 1u;
        gc = L.sg_codes + (int64_t)n * rb; uc = L.su_codes + (int64_t)n * rb;
        gs = L.sg_scales + (int64_t)n * nb; us = L.su_scales + (int64_t)n * nb;
    }
    float g[T], u[T];
#pragma unroll
    for (int t = 0; t < T; ++t) g[t] = u[t] = 0.f;
    for (int b = lane; b < nb; b += kWave) {
        Block32 bg, bu;
        load_block<FMT>(gc + (int64_t)b * block_bytes(FMT), bg);
        load_block<FMT>(uc + (int64_t)b * block_bytes(FMT), bu);
        const float sg = f16_to_f32(gs[b]), su = f16_to_f32(us[b]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)t * L.H + (size_t)b * 32);
            float dg = 0.f, du = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 xv = xp[c];
                const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int el = c * 8 + 2 * i;
                    const float x0 = bf16_lo(xw[i]), x1 = bf16_hi(xw[i]);
                    dg += block_level<FMT>(bg, el) * x0 + block_level<FMT>(bg, el + 1) * x1;
                    du += block_level<FMT>(bu, el) * x0 + block_level<FMT>(bu, el + 1) * x1;
                }
            }
            g[t] += sg * dg;
            u[t] += su * du;
        }
    }
    const int Imax = L.Imax();
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float gs_ = group_sum<kWave>(g[t]);
        const float us_ = group_sum<kWave>(u[t]);
        if (lane == 0 && (mask >> t) & 1u) h[((size_t)slot * T + t) * Imax + n] = silu_mul(gs_, us_);
    }
}

template <int FMT, int T>
__global__ __launch_bounds__(256) void k_decode_down(LayerView L, const int32_t* __restrict__ ids,
                                                     const float* __restrict__ h, float* __restrict__ y_pairs,
                                                     float* __restrict__ y_shared) {
    __shared__ DecodeRouting R;
    if (threadIdx.x < kWave) build_routing(ids, T, L.k, R);
    __syncthreads();
    const int sub = threadIdx.x % 16;
    const int64_t grp = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
    const int P = T * L.k;
    const int64_t slot64 = grp / L.H;
    const int m = (int)(grp % L.H);
    const int slot = (int)slot64;
    const int Imax = L.Imax();
    int Kin;
    uint32_t mask;
    const uint8_t* dc;
    const uint16_t* ds;
    bool active = true;
    if (slot < P) {
        active = slot < R.nU;
        const int e = active ? R.expert[slot] : 0;
        mask = active ? R.tokmask[slot] : 0u;
        Kin = L.I;
        const int64_t row = (int64_t)e * L.H + m;
        dc = L.d_codes + row * row_bytes(FMT, L.I);
        ds = L.d_scales + row * (L.I / 32);
    } else {
        active = slot == P && L.Is > 0;
        mask = (1u << T) - 1u;
        Kin = L.Is;
        dc = L.sd_codes + (int64_t)m * row_bytes(FMT, L.Is);
        ds = L.sd_scales + (int64_t)m * (L.Is / 32);
    }
    // every lane of a 16-lane group takes the same branch; whole groups may idle
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    if (active) {
        const int nb = Kin / 32;
        for (int b = sub; b < nb; b += 16) {
            Block32 bd;
            load_block<FMT>(dc + (int64_t)b * block_bytes(FMT), bd);
            const float sd = f16_to_f32(ds[b]);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if (!((mask >> t) & 1u)) continue;
                const float4* hp = reinterpret_cast<const float4*>(h + ((size_t)slot * T + t) * Imax + (size_t)b * 32);
                float d = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float4 hv = hp[c];
                    d += block_level<FMT>(bd, 4 * c) * hv.x + block_level<FMT>(bd, 4 * c + 1) * hv.y +
                         block_level<FMT>(bd, 4 * c + 2) * hv.z + block_level<FMT>(bd, 4 * c + 3) * hv.w;
                }
                acc[t] += sd * d;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float v = group_sum<16>(acc[t]);
        if (active && sub == 0 && ((mask >> t) & 1u)) {
            if (slot < P) {
                const int q = R.pair_of[slot][t];
                y_pairs[(size_t)q * L.H + m] = v;
            } else {
                y_shared[(size_t)t * L.H + m] = v;
            }
        }
    }
}

size_t decode_scratch_floats(const LayerView& L, int T) { return (size_t)(T * L.k + 1) * T * L.Imax(); }

template <int FMT, int T>
static moe_status launch_decode_t(const LayerView& L, const uint16_t* x, const int32_t* ids, float* y_pairs,
                                  float* y_shared, float* h, hipStream_t s) {
    const int64_t P = (int64_t)T * L.k;
    const int64_t rows1 = P * L.I + L.Is;
    hipLaunchKernelGGL((k_decode_gateup<FMT, T>), dim3((unsigned)((rows1 + 3) / 4)), dim3(256), 0, s, L, x, ids, h);
    MOE_LAUNCH_CHECK();
    const int64_t rows2 = (P + (L.Is > 0 ? 1 : 0)) * L.H;
    hipLaunchKernelGGL((k_decode_down<FMT, T>), dim3((unsigned)((rows2 + 15) / 16)), dim3(256), 0, s, L, ids, h,
                       y_pairs, y_shared);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

template <int FMT>
static moe_status launch_decode_f(const LayerView& L, const uint16_t* x, int T, const int32_t* ids, float* y_pairs,
                                  float* y_shared, float* h, hipStream_t s) {
    switch (T) {
        case 1: return launch_decode_t<FMT, 1>(L, x, ids, y_pairs, y_shared, h, s);
        case 2: return launch_decode_t<FMT, 2>(L, x, ids, y_pairs, y_shared, h, s);
        case 3: return launch_decode_t<FMT, 3>(L, x, ids, y_pairs, y_shared, h, s);
        case 4: return launch_decode_t<FMT, 4>(L, x, ids, y_pairs, y_shared, h, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

moe_status launch_decode_experts(const LayerView& L, const uint16_t* x, int T, const int32_t* ids, float* y_pairs,
                                 float* y_shared, float* h, hipStream_t s) {
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_decode_f<MOE_Q8_B32>(L, x, T, ids, y_pairs, y_shared, h, s);
        case MOE_Q4_B32: return launch_decode_f<MOE_Q4_B32>(L, x, T, ids, y_pairs, y_shared, h, s);
        case MOE_Q2_B32: return launch_decode_f<MOE_Q2_B32>(L, x, T, ids, y_pairs, y_shared, h, s);
        default: return MOE_ERR_INVALID_ARG;
    }
}

}  // namespace moe
