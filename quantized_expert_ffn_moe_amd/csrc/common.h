// Internal helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxTopK = 16;   // the largest top_k the library accepts

// ------------------------------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Order-preserving map of a float to uint32 with -0 folded onto +0 (NaN excluded by contract).
__device__ __forceinline__ uint32_t ordered_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------------------------- activation range
// The 16-bit operands (x and the SwiGLU activation h in fp16 on the dot-product and matrix-core
// paths) are kept inside the fp16 range whatever the scale of a token: each token t gets an exact
// power of two sigma_t = 2^e_t chosen from its largest |x| so that max |x_t| * sigma_t lies in
// [2, 4), with e_t clamped to [-kExpClamp, kExpClamp] so that sigma_t^2 and its inverse are normal
// fp32 numbers. x is staged as x * sigma_t; gate and up then come out as g * sigma_t and
// u * sigma_t, the activation is kept as h * sigma_t^2 (silu(g) * u is bounded by |g| |u|, so it
// scales like x^2 in both the small and the large regime), and the expert outputs, linear in h,
// are multiplied by sigma_t^-2 in fp32. For activations of ordinary size (max |x| in [2, 4))
// sigma_t = 1 and nothing changes.
constexpr int kExpClamp = 60;

// e_t from the largest |x| of the token given as bf16 magnitude bits (sign cleared): with the
// biased exponent b of that value, 2^(b - 127) <= max < 2^(b - 126), and e = 128 - b puts the scaled
// maximum in [2, 4). An all-zero (or subnormal-only) token takes the upper clamp.
__host__ __device__ inline int token_exp_from_bits(uint32_t max_abs_bf16_bits) {
    const int b = (int)((max_abs_bf16_bits >> 7) & 0xFFu);
    int e = 128 - b;
    e = e < -kExpClamp ? -kExpClamp : e;
    e = e > kExpClamp ? kExpClamp : e;
    return e;
}

// 2^e as an fp32 (e inside the normal range)
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// largest bf16 magnitude (bits, sign cleared) among the 8 values of a uint4
__device__ __forceinline__ uint32_t bf16_absmax_bits(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7FFFu);
        m = max(m, (w[i] >> 16) & 0x7FFFu);
    }
    return m;
}

// Largest finite fp16; 16-bit activations and outputs saturate there instead of becoming inf.
constexpr float kF16Max = 65504.0f;
__device__ __forceinline__ float sat_f16(float v) { return __builtin_amdgcn_fmed3f(v, -kF16Max, kF16Max); }

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// The SwiGLU activation of scaled accumulators: with gs = g * sigma and us = u * sigma (inv_sigma =
// 1 / sigma), silu(g) * u * sigma^2 = gs * us / (1 + exp(-gs * inv_sigma)).
__device__ __forceinline__ float silu_mul_scaled(float gs, float us, float inv_sigma) {
    return gs * us / (1.0f + expf(-gs * inv_sigma));
}

// The same from the hardware exp2 and reciprocal (each within about 1 ulp of fp32), for results
// that are rounded to fp16 right away. Large negative g gives an infinite exponential and a zero
// reciprocal, i.e. the limit 0.
__device__ __forceinline__ float silu_mul_scaled_fast(float gs, float us, float inv_sigma) {
    const float e = __builtin_amdgcn_exp2f(gs * (inv_sigma * -1.4426950408889634f));
    return gs * us * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------------------------------------- reductions

template <int kWidth>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = kWidth / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// ------------------------------------------------------------------------------------- formats

// Bits per code and the byte size of one 32-element block.
__host__ __device__ constexpr int fmt_bits(int fmt) { return fmt == MOE_Q8_B32 ? 8 : fmt == MOE_Q4_B32 ? 4 : 2; }
__host__ __device__ constexpr int block_bytes(int fmt) { return 32 * fmt_bits(fmt) / 8; }
__host__ __device__ inline int64_t row_bytes(int fmt, int64_t K) { return K * fmt_bits(fmt) / 8; }

// Raw bytes of one 32-element block (8 dwords; Q4 uses 4, Q2 uses 2).
struct Block32 {
    uint32_t w[8];
};

template <int FMT>
__device__ __forceinline__ void load_block(const uint8_t* p, Block32& b) {
    if constexpr (FMT == MOE_Q8_B32) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        const uint4 c = reinterpret_cast<const uint4*>(p)[1];
        b.w[0] = a.x; b.w[1] = a.y; b.w[2] = a.z; b.w[3] = a.w;
        b.w[4] = c.x; b.w[5] = c.y; b.w[6] = c.z; b.w[7] = c.w;
    } else if constexpr (FMT == MOE_Q4_B32) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        b.w[0] = a.x; b.w[1] = a.y; b.w[2] = a.z; b.w[3] = a.w;
    } else {
        const uint2 a = reinterpret_cast<const uint2*>(p)[0];
        b.w[0] = a.x; b.w[1] = a.y;
    }
}

// Level of element i (0..31) of a block, as an exact float (before the scale).
template <int FMT>
__device__ __forceinline__ float block_level(const Block32& b, int i) {
    if constexpr (FMT == MOE_Q8_B32) {
        return (float)(int32_t)(int8_t)(b.w[i >> 2] >> (8 * (i & 3)));
    } else if constexpr (FMT == MOE_Q4_B32) {
        // element i sits in nibble i of the little-endian block
        int32_t v = (int32_t)(b.w[i >> 3] << (28 - 4 * (i & 7))) >> 28;
        return (float)v;
    } else {
        uint32_t c = (b.w[i >> 4] >> (2 * (i & 15))) & 3u;
        return (float)c - 1.5f;
    }
}

// ------------------------------------------------------------------------------------- launch checks

#define MOE_LAUNCH_CHECK()                                  \
    do {                                                    \
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Sequential carve-out of a caller workspace with 256-byte alignment.
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t n) {
        off = align_up(off, 256);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
    size_t bytes() const { return align_up(off, 256); }
};

}  // namespace moe

// ------------------------------------------------------------------------------------- DPP wave ops
// DPP row/bank controls of GFX9: quad_perm, row_half_mirror, row_mirror, row_bcast:15, row_bcast:31.
namespace moe {

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Sum over the 64 lanes; the result is returned to every lane (via lane 63).
__device__ __forceinline__ float wave_sum(float v) {
    v += __uint_as_float(dpp_u32<0xb1>(__float_as_uint(v)));    // quad_perm [1,0,3,2]
    v += __uint_as_float(dpp_u32<0x4e>(__float_as_uint(v)));    // quad_perm [2,3,0,1]
    v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));   // row_half_mirror
    v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));   // row_mirror
    v += __uint_as_float(dpp_u32<0x142, 0xa>(__float_as_uint(v)));  // row_bcast:15
    v += __uint_as_float(dpp_u32<0x143, 0xc>(__float_as_uint(v)));  // row_bcast:31
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Max over the 64 lanes of an unsigned value, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xb1>(v));
    v = max(v, dpp_u32<0x4e>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    v = max(v, dpp_u32<0x142, 0xa>(v));
    v = max(v, dpp_u32<0x143, 0xc>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// Inverse of ordered_key (the -0 that ordered_key folds onto +0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Top-k of one token by one wave: KPL keys per lane (expert e = lane + 64 i) held in registers,
// k rounds of a DPP wave max of the order-preserving key, ties resolved to the lowest index with
// ballots; lane j < k ends with the j-th expert and its softmax weight over the chosen k (the
// first chosen, i.e. largest, logit is subtracted before exp).
// topk_wave_rounds takes the logits already in registers (lv[i] = logit of expert lane + 64 i).
template <int KPL>
__device__ __forceinline__ void topk_wave_rounds(const float (&lv)[KPL], int E, int k, int& my_id, float& my_p) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) key[i] = lane + kWave * i < E ? ordered_key(lv[i]) : 0u;
    int mine = 0;
    uint32_t mykey = 0u;
    for (int j = 0; j < k; ++j) {
        uint32_t lb = key[0];
#pragma unroll
        for (int i = 1; i < KPL; ++i) lb = max(lb, key[i]);
        const uint32_t vmax = wave_max_u32(lb);
        int sel = 0;
#pragma unroll
        for (int i = KPL - 1; i >= 0; --i) {   // the lowest i holding the maximum wins
            const uint64_t b = __ballot(key[i] == vmax);
            if (b) sel = kWave * i + __ffsll((unsigned long long)b) - 1;
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (lane + kWave * i == sel) key[i] = 0u;
        if (lane == j) { mine = sel; mykey = vmax; }
    }
    const float v = lane < k ? key_value(mykey) : 0.f;
    const float vmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
    const float ex = lane < k ? expf(v - vmax) : 0.f;
    const float s = wave_sum(ex);
    my_id = mine;
    my_p = ex / s;
}

// Min over the 64 lanes of an unsigned value, returned to every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp_u32<0xb1>(v));
    v = min(v, dpp_u32<0x4e>(v));
    v = min(v, dpp_u32<0x141>(v));
    v = min(v, dpp_u32<0x140>(v));
    v = min(v, dpp_u32<0x142, 0xa>(v));
    v = min(v, dpp_u32<0x143, 0xc>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// The same selection as a tournament over sorted lanes: each lane first orders its KPL keys by
// (value descending, expert index ascending) with a stable insertion network; round j then takes
// the wave max of the lanes' first keys, the lane holding it (the lowest expert index among equal
// first keys, found with a wave min only when several lanes tie) gives up its first key. A round
// is one wave max and one ballot instead of a max over KPL keys and KPL ballots.
template <int KPL>
__device__ __forceinline__ void topk_wave_sorted(const float (&lv)[KPL], int E, int k, int& my_id, float& my_p) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[KPL];
    int idx[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        idx[i] = lane + kWave * i;
        key[i] = idx[i] < E ? ordered_key(lv[i]) : 0u;
    }
#pragma unroll
    for (int a = 1; a < KPL; ++a)
#pragma unroll
        for (int b = a; b > 0; --b) {
            const bool sw = key[b] > key[b - 1];   // strictly greater: equal keys keep the lower index first
            const uint32_t k0 = key[b - 1], k1 = key[b];
            const int i0 = idx[b - 1], i1 = idx[b];
            key[b - 1] = sw ? k1 : k0;
            key[b] = sw ? k0 : k1;
            idx[b - 1] = sw ? i1 : i0;
            idx[b] = sw ? i0 : i1;
        }
    int mine = 0;
    uint32_t mykey = 0u;
    for (int j = 0; j < k; ++j) {
        const uint32_t vmax = wave_max_u32(key[0]);
        const uint64_t b = __ballot(key[0] == vmax);
        int win = __ffsll((unsigned long long)b) - 1;
        if (__builtin_expect(__popcll(b) != 1, 0)) {
            const uint32_t mi = wave_min_u32(key[0] == vmax ? (uint32_t)idx[0] : 0xFFFFFFFFu);
            win = (int)(mi % kWave);
        }
        const int wid = __builtin_amdgcn_readlane(idx[0], win);
        if (lane == j) { mine = wid; mykey = vmax; }
        if (lane == win) {
#pragma unroll
            for (int i = 0; i + 1 < KPL; ++i) { key[i] = key[i + 1]; idx[i] = idx[i + 1]; }
            key[KPL - 1] = 0u;
        }
    }
    const float v = lane < k ? key_value(mykey) : 0.f;
    const float vmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
    const float ex = lane < k ? expf(v - vmax) : 0.f;
    const float s = wave_sum(ex);
    my_id = mine;
    my_p = ex / s;
}

// topk_wave_regs: the tournament for 4 or 8 keys per lane (measured 3141 -> 2585 and 6225 -> 3853
// cycles per call for E = 256, k = 8 and E = 512, k = 10); the plain rounds otherwise (fewer keys per
// lane gain nothing from the presort, 16 would spend more on it than they save). Both give the
// same ids and weights.
template <int KPL>
__device__ __forceinline__ void topk_wave_regs(const float (&lv)[KPL], int E, int k, int& my_id, float& my_p) {
    if constexpr (KPL == 4 || KPL == 8) topk_wave_sorted<KPL>(lv, E, k, my_id, my_p);
    else topk_wave_rounds<KPL>(lv, E, k, my_id, my_p);
}

template <int KPL>
__device__ __forceinline__ void topk_wave(const float* __restrict__ l, int E, int k, int& my_id, float& my_p) {
    const int lane = threadIdx.x % kWave;
    // all KPL loads issued unconditionally before any is used (the empty asm pins each value, so the
    // compiler cannot sink a load into the e < E branch and serialise the round trips)
    float lv[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) lv[i] = l[min(lane + kWave * i, E - 1)];
#pragma unroll
    for (int i = 0; i < KPL; ++i) asm volatile("" : "+v"(lv[i]));
    topk_wave_regs<KPL>(lv, E, k, my_id, my_p);
}

}  // namespace moe
