// Decode regime (1 <= T <= 8 tokens, T k <= 64 pairs): router + top-k, then the chosen experts' FFNs streamed
// from HBM.
//
// Decode on the pages runs the selected experts' weights on the GPU and prices each token by the
// expert bytes it reads (648news 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU
// compute"; 648news 10-cyber-on-strata-moe-local-inference, section "bitwise validation and speed
// bottleneck", about 117 MB of weights per token). Every expert is resident in HBM here, so the
// kernels move exactly the packed bytes of the distinct chosen experts plus the shared expert.
//
// Three launches per layer. Each kernel costs about 2 us of fixed overhead on this GPU and a
// device-scope fence (L2 write-back + invalidate) costs several us, so no kernel synchronises with
// other blocks: every cross-block dependency is a kernel boundary, and work that all blocks need
// (top-k, the union of chosen experts) is recomputed per block from data already in HBM.
//   k_route_gemv     router logits, one wave per expert row, all loads issued before use.
//   k_dec_gateup     per block: top-k of every token from the logits (one wave per token, in
//                    registers), the union of the chosen experts in LDS, x staged as fp16 pairs
//                    laid out to match the packed codes; then gate/up rows streamed with every
//                    load of a wave issued up front (one or two tokens: a row per 16 lanes, four
//                    rows per wave; more: three or two rows over all 64 lanes): codes become fp16
//                    by OR-ing them into the mantissa of 1024.0 and multiply into x with
//                    v_dot2_f32_f16 (fp32 accumulation); for one or two tokens the constant 1024
//                    (and the code offset) is removed once per block with a sum over the staged x,
//                    from three tokens on by a packed subtract per code pair. Block 0 publishes
//                    ids and p.
//   k_dec_down       output rows m: every chosen expert's down row m times its h (LDS as fp16
//                    hi/lo pairs for one or two tokens, the fp16 high halves alone from three on,
//                    laid out so that lanes reading consecutive 32-blocks hit consecutive banks),
//                    weighted by the routing probability and summed with the shared expert
//                    (combine fused), or written per pair for moe_experts_decode.
#include <algorithm>

#include <atomic>

#include "kernels.h"

namespace moe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------------------------- routing plan

// Union of the chosen experts of T <= 8 tokens (T*k <= 64 pairs), built in LDS by a whole block.
constexpr int kMaxDecodeT = 8;
struct DecodePlan {
    int nU;                            // distinct routed experts
    int expert[64];                    // slot -> expert id, slots in order of first appearance
    uint32_t tokmask[64];              // slot -> bitmask of the tokens that chose it
    int pair_of[64][kMaxDecodeT];      // slot, token -> pair q = t*k + j, or -1
    float pw[64][kMaxDecodeT];         // slot, token -> routing probability of that pair (0 if none)
    int xexp[kMaxDecodeT];             // token -> e_t of its activation scale 2^e_t (token_exp_from_bits)
};

// Built by one wave (lane q = pair q = t*k + j; T*k <= 64), LDS only, no block barrier: the caller
// publishes P to the other waves with one. first: LDS scratch of E ints. ids outside [0, E) are
// ignored (no memory access with them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ void build_plan_wave(const int32_t* __restrict__ ids, const float* __restrict__ p, int T, int k, int E,
                                DecodePlan& P, int* first) {
    const int lane = threadIdx.x % kWave;
    const int npairs = T * k;
    const int q = lane;
    const int e = q < npairs ? ids[q] : -1;
    const float pq = p && q < npairs ? p[q] : 0.f;
    for (int i = lane; i < E; i += kWave) first[i] = 64;
    P.tokmask[lane] = 0u;
#pragma unroll
    for (int t = 0; t < kMaxDecodeT; ++t) { P.pair_of[lane][t] = -1; P.pw[lane][t] = 0.f; }
    wave_lds_sync();
    const bool valid = q < npairs && e >= 0 && e < E;
    if (valid) atomicMin(&first[e], q);
    wave_lds_sync();
    const int fq = valid ? first[e] : 63;
    const uint64_t firsts = __ballot(valid && fq == q);
    const int slot = __popcll(firsts & ((1ull << fq) - 1ull));
    if (valid) {
        if (fq == q) P.expert[slot] = e;
        atomicOr(&P.tokmask[slot], 1u << (q / k));
        P.pair_of[slot][q / k] = q;
        P.pw[slot][q / k] = pq;
    }
    if (lane == 0) P.nU = __popcll(firsts);
}

// ----------------------------------------------------------------------------------- K1 router

// One block of four waves per expert row: wave w takes the float4 chunks w, w + 4, w + 8, ... of
// the row (every W_r and x chunk of a lane loaded before any is used), the four partial sums meet
// in LDS. One block per expert spreads the 2 MB of W_r over as many CUs as there are experts.
template <int T>
__global__ __launch_bounds__(256) void k_route_gemv(const float* __restrict__ w_r, const float* __restrict__ bias,
                                                    const uint16_t* __restrict__ x, int H, int E,
                                                    float* __restrict__ logits) {
    __shared__ float part[4][T];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int e = blockIdx.x;
    const float4* wr = reinterpret_cast<const float4*>(w_r + (size_t)e * H);
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    const int nch = H / 4;
    for (int c0 = 0; c0 < nch; c0 += 2 * 256) {
        float4 wv[2];
        uint2 xv[T][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = c0 + i * 256 + threadIdx.x;
            wv[i] = c < nch ? wr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int t = 0; t < T; ++t)
                xv[t][i] = c < nch ? reinterpret_cast<const uint2*>(x + (size_t)t * H)[c] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[t] += wv[i].x * bf16_lo(xv[t][i].x) + wv[i].y * bf16_hi(xv[t][i].x) +
                          wv[i].z * bf16_lo(xv[t][i].y) + wv[i].w * bf16_hi(xv[t][i].y);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) part[wave][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        const float b = bias ? bias[e] : 0.f;
        logits[(size_t)t * E + e] = ((part[0][t] + part[1][t]) + (part[2][t] + part[3][t])) + b;
    }
}

// ----------------------------------------------------------------------------------- code pairs

// Per format: pairs of codes per dword (NP), dwords per 32-block (ND), and for pair j of a dword the
// two element indices (e0, e1), the factor f (the code sits f times its level above 1024.0 in each
// fp16 half) and the matching activation scale xs = 1 / f.
template <int FMT> struct Fmt;
template <> struct Fmt<MOE_Q4_B32> {
    static constexpr int NP = 4, ND = 4;
    __device__ static int e0(int d, int j) { return 8 * d + j; }
    __device__ static int e1(int d, int j) { return 8 * d + j + 4; }
    __device__ static float xs(int j) { return (j & 1) ? 0.0625f : 1.f; }
};
template <> struct Fmt<MOE_Q8_B32> {
    static constexpr int NP = 2, ND = 8;
    __device__ static int e0(int d, int j) { return 4 * d + j; }
    __device__ static int e1(int d, int j) { return 4 * d + j + 2; }
    __device__ static float xs(int) { return 1.f; }
};
template <> struct Fmt<MOE_Q2_B32> {
    static constexpr int NP = 8, ND = 2;
    __device__ static int e0(int d, int j) { return 16 * d + j; }
    __device__ static int e1(int d, int j) { return 16 * d + j + 8; }
    // f = 2, 4, 16, 64, 256 for j = 0..4 and 2, 8, 32 for j = 5..7
    __device__ static float xs(int j) {
        return j == 0 ? 0.5f : j == 1 ? 0.25f : j == 2 ? 0.0625f : j == 3 ? 0.015625f : j == 4 ? 0.00390625f
             : j == 5 ? 0.5f : j == 6 ? 0.125f : 0.03125f;
    }
};

constexpr uint32_t kMagic = 0x64006400u;  // (1024.0, 1024.0) as fp16 pair

// Subtract the same constant K from both fp16 halves; exact when K and the results are integers
// below 2048 (all values here are).
template <int K, bool SUB = true>
__device__ __forceinline__ uint32_t sub_k(uint32_t pr) {
    if constexpr (!SUB) return pr;
    half2_t v = __builtin_bit_cast(half2_t, pr);
    v -= half2_t{(_Float16)(float)K, (_Float16)(float)K};
    return __builtin_bit_cast(uint32_t, v);
}

// The constant sub_k takes off code pair p of a block (p = 0 .. 15, in code_pairs' order).
template <int FMT>
__device__ __forceinline__ float pair_offset(int p) {
    if constexpr (FMT == MOE_Q4_B32) return (p & 1) ? 1152.f : 1032.f;
    else if constexpr (FMT == MOE_Q8_B32) return 1152.f;
    else {
        const int j = p & 7;
        return j == 0 ? 1027.f : j == 1 ? 1030.f : j == 2 ? 1048.f : j == 3 ? 1120.f : j == 4 ? 1408.f
             : j == 5 ? 1027.f : j == 6 ? 1036.f : 1072.f;
    }
}

// The 16 fp16 pairs of one 32-element block, each half = f * level exactly: the stored code (offset
// to be unsigned) is OR-ed into the mantissa of 1024.0 at f times its unit, then 1024 + f * offset
// is subtracted (Q4: offset 8, Q8: offset 128, Q2: offset 1.5, the level being c - 1.5). With
// SUB = false the subtraction is left out: each half is pair_offset(p) + f * level, and the caller
// removes pair_offset(p) times the pair's activations once per block.
//
// The sign flip of the two's-complement codes (XOR with the code's top bit) and the OR with 1024.0
// touch disjoint bits, so they merge into one constant: ((w & mask) ^ (flip & mask | 1024.0)) is a
// single three-input bit operation per pair.
template <int FMT, bool SUB = true>
__device__ __forceinline__ void code_pairs(const uint32_t* w, uint32_t (&pr)[16]) {
    if constexpr (FMT == MOE_Q4_B32) {
        constexpr uint32_t kLo = 0x00080008u | kMagic, kHi = 0x00800080u | kMagic;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t u = w[d], v = w[d] >> 8;
            pr[4 * d + 0] = sub_k<1032, SUB>((u & 0x000F000Fu) ^ kLo);
            pr[4 * d + 1] = sub_k<1152, SUB>((u & 0x00F000F0u) ^ kHi);
            pr[4 * d + 2] = sub_k<1032, SUB>((v & 0x000F000Fu) ^ kLo);
            pr[4 * d + 3] = sub_k<1152, SUB>((v & 0x00F000F0u) ^ kHi);
        }
    } else if constexpr (FMT == MOE_Q8_B32) {
        constexpr uint32_t kB = 0x00800080u | kMagic;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            pr[2 * d + 0] = sub_k<1152, SUB>((w[d] & 0x00FF00FFu) ^ kB);
            pr[2 * d + 1] = sub_k<1152, SUB>(((w[d] >> 8) & 0x00FF00FFu) ^ kB);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t u = w[d];
            const uint32_t v = u >> 9;   // elements 5..7 (and 13..15) at bits 1, 3, 5 (17, 19, 21)
            pr[8 * d + 0] = sub_k<1027, SUB>(((u << 1) & 0x00060006u) | kMagic);
            pr[8 * d + 1] = sub_k<1030, SUB>((u & 0x000C000Cu) | kMagic);
            pr[8 * d + 2] = sub_k<1048, SUB>((u & 0x00300030u) | kMagic);
            pr[8 * d + 3] = sub_k<1120, SUB>((u & 0x00C000C0u) | kMagic);
            pr[8 * d + 4] = sub_k<1408, SUB>((u & 0x03000300u) | kMagic);
            pr[8 * d + 5] = sub_k<1027, SUB>((v & 0x00060006u) | kMagic);
            pr[8 * d + 6] = sub_k<1036, SUB>((v & 0x00180018u) | kMagic);
            pr[8 * d + 7] = sub_k<1072, SUB>((v & 0x00600060u) | kMagic);
        }
    }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

template <int FMT>
__device__ __forceinline__ void load_codes(const uint8_t* p, uint32_t (&w)[8]) {
    if constexpr (FMT == MOE_Q8_B32) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (FMT == MOE_Q4_B32) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
        const uint2 a = reinterpret_cast<const uint2*>(p)[0];
        w[0] = a.x; w[1] = a.y;
    }
}

// ----------------------------------------------------------------------------------- staging

// 32 activations (fp32, natural order) -> fp16 pairs in code-pair order, scaled by the pair's xs:
// NH = 1 keeps one fp16 per value, NH = 2 also a second fp16 with the rounding residual (value =
// hi + lo to about 22 bits). Stored as NH * 4 uint4 at dst[c * stride].
template <int FMT, int NH>
__device__ __forceinline__ void stage_pairs(const float (&v)[32], uint4* dst, size_t stride) {
    using F = Fmt<FMT>;
    uint32_t hi[16], lo[16];
#pragma unroll
    for (int d = 0; d < F::ND; ++d)
#pragma unroll
        for (int j = 0; j < F::NP; ++j) {
            const float sc = F::xs(j);
            const float a = v[F::e0(d, j)] * sc, b = v[F::e1(d, j)] * sc;
            const _Float16 ah = (_Float16)a, bh = (_Float16)b;
            half2_t ph = {ah, bh};
            hi[d * F::NP + j] = __builtin_bit_cast(uint32_t, ph);
            if constexpr (NH == 2) {
                half2_t pl = {(_Float16)(a - (float)ah), (_Float16)(b - (float)bh)};
                lo[d * F::NP + j] = __builtin_bit_cast(uint32_t, pl);
            }
        }
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c * stride] = make_uint4(hi[4 * c], hi[4 * c + 1], hi[4 * c + 2], hi[4 * c + 3]);
    if constexpr (NH == 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            dst[(4 + c) * stride] = make_uint4(lo[4 * c], lo[4 * c + 1], lo[4 * c + 2], lo[4 * c + 3]);
    }
}

// sum over the block's code pairs p of pair_offset(p) times the two staged fp16 activations of pair
// p (rounded exactly as stage_pairs<FMT, 1> rounds them): what the dot products of pairs left
// without their offset (code_pairs<FMT, false>) carry in excess, in a fixed order
template <int FMT>
__device__ __forceinline__ float stage_corr(const float (&v)[32]) {
    using F = Fmt<FMT>;
    float c = 0.f;
#pragma unroll
    for (int d = 0; d < F::ND; ++d)
#pragma unroll
        for (int j = 0; j < F::NP; ++j) {
            const float sc = F::xs(j);
            const float a = (float)(_Float16)(v[F::e0(d, j)] * sc), b = (float)(_Float16)(v[F::e1(d, j)] * sc);
            c += pair_offset<FMT>(d * F::NP + j) * (a + b);
        }
    return c;
}

// One activation h[row][n] written straight into the staged layout that stage_pairs<FMT, 2> builds
// for a whole 32-block: row = [8][nbm] uint4 (pairs 0..15 as fp16 hi, then as fp16 lo), pair p of
// block b at uint4 (p / 4) * nbm + b, component p % 4, half 0 for e0 and 1 for e1.
template <int FMT>
__device__ __forceinline__ void put_staged(_Float16* row, int nbm, int n, float v) {
    using F = Fmt<FMT>;
    const int b = n / 32, e = n % 32;
    constexpr int GS = 32 / F::ND;           // elements per dword: 8 (Q4), 4 (Q8), 16 (Q2)
    const int d = e / GS, r = e % GS;
    const int j = r % F::NP, half = r / F::NP;
    const int pidx = d * F::NP + j;
    const float a = sat_f16(v) * F::xs(j);
    const _Float16 hi = (_Float16)a;
    const _Float16 lo = (_Float16)(a - (float)hi);
    row[((size_t)(pidx / 4) * nbm + b) * 8 + 2 * (pidx % 4) + half] = hi;
    row[((size_t)(4 + pidx / 4) * nbm + b) * 8 + 2 * (pidx % 4) + half] = lo;
}

__device__ __forceinline__ void bf16x32_to_f32(const uint4 (&raw)[4], float (&v)[32]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t wv[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[8 * c + 2 * i] = bf16_lo(wv[i]); v[8 * c + 2 * i + 1] = bf16_hi(wv[i]); }
    }
}

// ----------------------------------------------------------------------------------- K2 gate/up

// Sum over each row of 16 lanes (lanes 16r .. 16r + 15), returned to every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += __uint_as_float(dpp_u32<0xb1>(__float_as_uint(v)));    // quad_perm [1,0,3,2]
    v += __uint_as_float(dpp_u32<0x4e>(__float_as_uint(v)));    // quad_perm [2,3,0,1]
    v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));   // row_half_mirror
    v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));   // row_mirror
    return v;
}

// Gate/up rows per K2 wave and waves per K2 block. One or two tokens: 4 rows, one per 16-lane row
// of the wave (each lane 4 of the row's 32-blocks per step), so that a row's dot product ends in a
// 16-lane sum and the four rows share one epilogue; up to 8 waves (256 VGPRs: the 8-bit codes of
// 4 blocks of gate and up stay in registers), 8192 rows per pass over 256 CUs. Three or four tokens: 3 rows
// over all 64 lanes and up to 12 waves (168 VGPRs, so that the 8-bit codes of 3 rows and 4 tokens'
// sums stay in registers), i.e. 9216 rows per pass over 256 CUs: the union of the chosen experts
// (about 16 + the shared one, 8704 rows) then takes one pass instead of two; for five to eight
// tokens 2 rows and up to 8 waves (256 VGPRs: the sums of 8 tokens stay in registers).
__host__ __device__ constexpr int gateup_rows(int T) { return T >= 5 ? 2 : T >= 3 ? 3 : 4; }
__host__ __device__ constexpr bool gateup_row_lanes(int T) { return T <= 2; }
__host__ __device__ constexpr int gateup_max_waves(int T) { return T >= 5 ? 8 : T >= 3 ? 12 : 8; }
constexpr int kDownRows = 1;      // output rows per K3 wave
constexpr int kDownWaves = 8;     // waves per K3 block (two per SIMD hide each other's latency)
constexpr int kDownThreads = kDownWaves * kWave;
// Down items per row whose loads a K3 lane issues together: 4, and 5 from three tokens on (16 + 1
// experts x 16 blocks = 272 items per row of a 4-token batch then take one batch of loads, not two).
__host__ __device__ constexpr int down_batch(int T) { return T >= 3 ? 5 : 4; }

// LDS of k_dec_gateup: plan | first[E] | ids_s[64] | p_s[64] | xq[T][4][nb] uint4
__host__ __device__ inline size_t lds_head(int E) {
    return align_up(sizeof(DecodePlan), 16) + align_up((size_t)E * 4, 16) + 2 * 64 * 4;
}
static size_t gateup_smem_bytes(int T, int H, int E) { return lds_head(E) + (size_t)T * (H / 32) * (64 + 4); }

// Per block: top-k of every token (given logits) or the given ids, the union of the chosen experts,
// x as fp16 pairs; per wave: R consecutive rows of one expert's gate and up, all loads issued before
// use, h = silu(g) * u written for each token that chose the expert, already in the staged fp16
// hi/lo layout the down kernel reads. Block 0 publishes ids, p and the plan (plan_g).
template <int FMT, int T, bool ROUTE, int KPL>
__global__ __launch_bounds__(kWave * gateup_max_waves(T)) void k_dec_gateup(LayerView L, const uint16_t* __restrict__ x,
                                                    const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                    float* __restrict__ p, float* __restrict__ h,
                                                    DecodePlan* __restrict__ plan_g) {
    constexpr int R = gateup_rows(T);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    DecodePlan& P = *reinterpret_cast<DecodePlan*>(smem);
    int* first = reinterpret_cast<int*>(smem + align_up(sizeof(DecodePlan), 16));
    int* ids_s = reinterpret_cast<int*>(smem + align_up(sizeof(DecodePlan), 16) + align_up((size_t)L.E * 4, 16));
    float* p_s = reinterpret_cast<float*>(ids_s + 64);
    uint4* xq = reinterpret_cast<uint4*>(smem + lds_head(L.E));
    float* xc = reinterpret_cast<float*>(xq + (size_t)T * 4 * (L.H / 32));   // [T][nb] pair-offset sums
    // one or two tokens: code pairs keep their offsets and each block's dot product drops the
    // pair-offset sum xc of its activations (one instruction per pair less); three or more tokens
    // subtract per pair (the extra LDS read per token and block costs them more than it saves)
    constexpr bool kSubPairs = T >= 3;   // code_pairs subtracts the offsets itself
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int H = L.H, nb = H / 32;
    const int Imax = L.Imax();
    const int npairs = T * L.k;

    // x is staged by the waves after the first T (the top-k waves; without routing, after wave 0,
    // which builds the plan), one wave per token, so that the staging runs beside the top-k and the
    // plan rather than after them; a block too small for that stages with all its waves after their
    // other work. A token's largest |x| is one wave reduction; its scale 2^e_t (see common.h) is
    // applied before the fp16 rounding. The first chunk of each staging wave's first token is loaded
    // before the top-k (it does not depend on the routing).
    constexpr int kBusyWaves = ROUTE ? T : 1;
    const int nwaves = (int)blockDim.x / kWave;
    const bool spare = nwaves > kBusyWaves;
    const int sw = spare ? wave - kBusyWaves : wave;   // staging wave index (< 0: none)
    const int nsw = spare ? nwaves - kBusyWaves : nwaves;
    auto load_chunk = [&](int t, int c, uint4 (&r)[4]) __attribute__((always_inline)) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H + (size_t)c * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = xr[i];
    };
    uint4 xpre[4];
    if (sw >= 0) load_chunk(min(sw, T - 1), min(lane, nb - 1), xpre);
    const int32_t* ids_src = ids;
    if constexpr (ROUTE) {
        // top-k of every token from the router logits (wave t: token t), recomputed by every block
        if (wave < T) {
            int id;
            float pr;
            topk_wave<KPL>(logits + (size_t)wave * L.E, L.E, L.k, id, pr);
            if (lane < L.k) {
                ids_s[wave * L.k + lane] = id;
                p_s[wave * L.k + lane] = pr;
                if (blockIdx.x == 0) {
                    ids[wave * L.k + lane] = id;
                    p[wave * L.k + lane] = pr;
                }
            }
        }
        ids_src = ids_s;
    }

    // x staging: max |x| of the token (chunks beyond the first 64 are read twice, from L2), then
    // x * 2^e_t as fp16 pairs (and their offset sums)
    for (int t = sw; sw >= 0 && t < T; t += nsw) {   // uniform per wave
        uint4 keep[4];
        if (t == sw) {
#pragma unroll
            for (int i = 0; i < 4; ++i) keep[i] = xpre[i];
        } else {
            load_chunk(t, min(lane, nb - 1), keep);
        }
        uint32_t m = 0u;
        if (lane < nb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) m = max(m, bf16_absmax_bits(keep[i]));
        }
        for (int c = lane + kWave; c < nb; c += kWave) {
            uint4 r[4];
            load_chunk(t, c, r);
#pragma unroll
            for (int i = 0; i < 4; ++i) m = max(m, bf16_absmax_bits(r[i]));
        }
        const int e = token_exp_from_bits(wave_max_u32(m));
        if (lane == 0) P.xexp[t] = e;
        const float sc = pow2f(e);
        auto stage = [&](const uint4 (&r)[4], int c) __attribute__((always_inline)) {
            float v[32];
            bf16x32_to_f32(r, v);
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] *= sc;
            stage_pairs<FMT, 1>(v, xq + (size_t)t * 4 * nb + c, nb);
            if constexpr (!kSubPairs) xc[t * nb + c] = stage_corr<FMT>(v);
        };
        if (lane < nb) stage(keep, lane);
        for (int c = lane + kWave; c < nb; c += kWave) {
            uint4 r[4];
            load_chunk(t, c, r);
            stage(r, c);
        }
    }
    // every token's choices in ids_s before the plan: with one token the wave that chose them is
    // the wave that builds the plan, so its own LDS writes only need to be complete
    if constexpr (ROUTE && T > 1) __syncthreads();
    if (wave == 0) {
        if constexpr (ROUTE && T == 1) wave_lds_sync();
        build_plan_wave(ids_src, ROUTE ? p_s : nullptr, T, L.k, L.E, P, first);
    }
    __syncthreads();                        // the plan and the staged x
    if (blockIdx.x == 0) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(&P);
        uint32_t* dst = reinterpret_cast<uint32_t*>(plan_g);
        for (int i = threadIdx.x; i < (int)(sizeof(DecodePlan) / 4); i += blockDim.x) dst[i] = src[i];
    }

    if constexpr (gateup_row_lanes(T)) {
        // tasks of 4 consecutive rows of one expert (I and Is are multiples of 32), row n0 + g on
        // lanes 16g .. 16g + 15, lane li of a row taking the 32-blocks li, li + 16, ...: those of
        // the distinct chosen experts (slot order) then the shared expert's, one task per wave and
        // step, the grid striding over them
        static_assert(R == 4, "one row per 16 lanes");
        constexpr int JB = 4;                      // 32-blocks per lane whose loads are in flight together
        const int g = lane >> 4, li = lane & 15;
        const int gw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * (int)(blockDim.x / kWave) + wave);
        const int tstride = (int)gridDim.x * (int)(blockDim.x / kWave);
        const int tpeI = L.I / 4, tpeS = L.Is / 4;
        const int nrouted = P.nU * tpeI;
        const int ntasks = nrouted + tpeS;
        const int64_t rb = row_bytes(FMT, H);
        for (int tk = gw; tk < ntasks; tk += tstride) {   // uniform per wave
            int slot, n;
            const uint8_t *gc, *uc;
            const uint16_t *gsp, *usp;
            if (tk < nrouted) {
                slot = tk / tpeI;
                n = (tk - slot * tpeI) * 4 + g;
                const int64_t row = (int64_t)P.expert[slot] * L.I + n;
                gc = L.g_codes + row * rb; uc = L.u_codes + row * rb;
                gsp = L.g_scales + row * nb; usp = L.u_scales + row * nb;
            } else {
                slot = 64;  // shared
                n = (tk - nrouted) * 4 + g;
                gc = L.sg_codes + (int64_t)n * rb; uc = L.su_codes + (int64_t)n * rb;
                gsp = L.sg_scales + (int64_t)n * nb; usp = L.su_scales + (int64_t)n * nb;
            }
            const uint32_t mask = slot < 64 ? P.tokmask[slot] : (1u << T) - 1u;
            float ga[T], ua[T];
#pragma unroll
            for (int t = 0; t < T; ++t) ga[t] = ua[t] = 0.f;
            for (int j0 = 0; j0 * 16 < nb; j0 += JB) {   // uniform
                uint32_t wg[JB][8], wu[JB][8];
                uint16_t sgb[JB], sub[JB];
                int bj[JB];
                // every load of the step issued before any is used (scales first); blocks past the
                // row's end read its last block (result unused)
#pragma unroll
                for (int jj = 0; jj < JB; ++jj) {
                    bj[jj] = li + 16 * (j0 + jj);
                    const int bc = min(bj[jj], nb - 1);
                    sgb[jj] = gsp[bc];
                    sub[jj] = usp[bc];
                }
#pragma unroll
                for (int jj = 0; jj < JB; ++jj) {
                    const int bc = min(bj[jj], nb - 1);
                    load_codes<FMT>(gc + (int64_t)bc * block_bytes(FMT), wg[jj]);
                    load_codes<FMT>(uc + (int64_t)bc * block_bytes(FMT), wu[jj]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // staged x of XB blocks read from LDS together (one round trip), then their dot
                // products: all four blocks for one token, one block at a time for two
                constexpr int XB = T == 1 ? JB : 1;
#pragma unroll
                for (int j1 = 0; j1 < JB; j1 += XB) {
                    uint4 xv[XB][T][4];
                    float xcv[XB][T];
#pragma unroll
                    for (int jx = 0; jx < XB; ++jx) {
                        const int bc = min(bj[j1 + jx], nb - 1);
#pragma unroll
                        for (int t = 0; t < T; ++t) {
#pragma unroll
                            for (int c = 0; c < 4; ++c) xv[jx][t][c] = xq[((size_t)t * 4 + c) * nb + bc];
                            xcv[jx][t] = xc[t * nb + bc];
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    auto blockdot = [&](const uint32_t (&w)[8], uint16_t sc, int jx, float (&acc)[T]) __attribute__((always_inline)) {
                        uint32_t pw[16];
                        code_pairs<FMT, false>(w, pw);
                        const float sf = f16_to_f32(sc);
#pragma unroll
                        for (int t = 0; t < T; ++t) {
                            float d = 0.f;
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                d = dot2(pw[4 * c], xv[jx][t][c].x, d);
                                d = dot2(pw[4 * c + 1], xv[jx][t][c].y, d);
                                d = dot2(pw[4 * c + 2], xv[jx][t][c].z, d);
                                d = dot2(pw[4 * c + 3], xv[jx][t][c].w, d);
                            }
                            acc[t] += sf * (d - xcv[jx][t]);
                        }
                    };
#pragma unroll
                    for (int jx = 0; jx < XB; ++jx) {
                        if (bj[j1 + jx] < nb) {
                            blockdot(wg[j1 + jx], sgb[j1 + jx], jx, ga);
                            blockdot(wu[j1 + jx], sub[j1 + jx], jx, ua);
                        }
                    }
                }
            }
            // every lane of a row holds the row's sums (the same bits: the DPP tree adds the same
            // pairs in every lane); lane li of the row takes token li, one epilogue for all
            float gsel = 0.f, usel = 0.f;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float gs_ = row16_sum(ga[t]);
                const float us_ = row16_sum(ua[t]);
                gsel = li == t ? gs_ : gsel;
                usel = li == t ? us_ : usel;
            }
            if (li < T && ((mask >> li) & 1u)) {
                const int t = li;
                const int row = slot < 64 ? P.pair_of[slot][t] : npairs + t;
                put_staged<FMT>(reinterpret_cast<_Float16*>(h + (size_t)row * Imax), Imax / 32, n,
                                silu_mul_scaled(gsel, usel, pow2f(-P.xexp[t])));
            }
        }
    } else {
    // tasks of R consecutive rows of one expert (the last task of an expert may hold fewer): those
    // of the distinct chosen experts (slot order) then the shared expert's, one task per wave and
    // step, the grid striding over them (a grid of at most one block per CU)
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave;
    const int tpeI = (L.I + R - 1) / R, tpeS = (L.Is + R - 1) / R;
    const int64_t nrouted = (int64_t)P.nU * tpeI;
    const int64_t ntasks = nrouted + tpeS;
    const int64_t tstride = (int64_t)gridDim.x * (blockDim.x / kWave);
    const int64_t rb = row_bytes(FMT, H);
    for (int64_t tk = gw; tk < ntasks; tk += tstride) {   // uniform per wave
        int slot, n0, nv;
        const uint8_t *gc, *uc;
        const uint16_t *gs, *us;
        if (tk < nrouted) {
            slot = (int)(tk / tpeI);
            n0 = (int)(tk % tpeI) * R;
            nv = min(R, L.I - n0);
            const int64_t row = (int64_t)P.expert[slot] * L.I + n0;
            gc = L.g_codes + row * rb; uc = L.u_codes + row * rb;
            gs = L.g_scales + row * nb; us = L.u_scales + row * nb;
        } else {
            slot = 64;  // shared
            n0 = (int)(tk - nrouted) * R;
            nv = min(R, L.Is - n0);
            gc = L.sg_codes + (int64_t)n0 * rb; uc = L.su_codes + (int64_t)n0 * rb;
            gs = L.sg_scales + (int64_t)n0 * nb; us = L.su_scales + (int64_t)n0 * nb;
        }
        // row i of the task, clamped to its last valid row (loads stay in the expert's matrix;
        // the results of clamped rows are not stored)
        int ro[R];
#pragma unroll
        for (int i = 0; i < R; ++i) ro[i] = min(i, nv - 1);

        const uint32_t mask = slot < 64 ? P.tokmask[slot] : (1u << T) - 1u;
        float g[R][T], u[R][T];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int t = 0; t < T; ++t) g[i][t] = u[i][t] = 0.f;
        for (int b = lane; b < nb; b += kWave) {
            uint32_t wg[R][8], wu[R][8];
            uint16_t sgb[R], sub[R];
            // every load of the step issued before any is used (scales first: the compiler would
            // otherwise sink them behind the code arithmetic, costing a second round trip)
#pragma unroll
            for (int i = 0; i < R; ++i) {
                sgb[i] = gs[ro[i] * nb + b];
                sub[i] = us[ro[i] * nb + b];
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                load_codes<FMT>(gc + ro[i] * rb + (int64_t)b * block_bytes(FMT), wg[i]);
                load_codes<FMT>(uc + ro[i] * rb + (int64_t)b * block_bytes(FMT), wu[i]);
            }
            __builtin_amdgcn_sched_barrier(0);
            // matrix- and row-outer: each row's codes become fp16 pairs once, and the staged x of
            // every token is read from LDS per row (few registers live at a time, so nothing spills
            // at 4 tokens)
            auto rowdot = [&](const uint32_t (&w)[8], uint16_t sc, float (&acc)[T]) __attribute__((always_inline)) {
                uint32_t pw[16];
                code_pairs<FMT, kSubPairs>(w, pw);
                const float sf = f16_to_f32(sc);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    uint32_t xr[16];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint4 v = xq[((size_t)t * 4 + c) * nb + b];
                        xr[4 * c] = v.x; xr[4 * c + 1] = v.y; xr[4 * c + 2] = v.z; xr[4 * c + 3] = v.w;
                    }
                    float d = 0.f;
#pragma unroll
                    for (int j = 0; j < 16; ++j) d = dot2(pw[j], xr[j], d);
                    if constexpr (kSubPairs) acc[t] += sf * d;
                    else acc[t] += sf * (d - xc[t * nb + b]);
                }
            };
#pragma unroll
            for (int i = 0; i < R; ++i) {
                rowdot(wg[i], sgb[i], g[i]);
                rowdot(wu[i], sub[i], u[i]);
            }
        }
        // the R T sums of gate and up moved into lanes 0 .. R T - 1 (row i, token t at lane i T + t),
        // so that one epilogue (SiLU, h in its staged layout) serves them all instead of R T
        // epilogues of a single active lane
        static_assert(R * T <= kWave, "one lane per output");
        float gl = 0.f, ul = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float gs_ = wave_sum(g[i][t]), us_ = wave_sum(u[i][t]);
                const bool mine = lane == i * T + t;
                gl = mine ? gs_ : gl;
                ul = mine ? us_ : ul;
            }
        {
            const int i = lane / T, t = lane - i * T;
            if (lane < R * T && i < nv && ((mask >> t) & 1u)) {
                const int row = slot < 64 ? P.pair_of[slot][t] : npairs + t;
                put_staged<FMT>(reinterpret_cast<_Float16*>(h + (size_t)row * Imax), Imax / 32, n0 + i,
                                silu_mul_scaled(gl, ul, pow2f(-P.xexp[t])));
            }
        }
    }
    }
}

// ----------------------------------------------------------------------------------- K3 down

// LDS of k_dec_down: plan | (unused, E ints) | eoff[64] int64 | hq[rows][8][nbm] uint4 (fp16 hi/lo
// pairs; lanes reading consecutive 32-blocks hit consecutive banks) | partials
// [waves][RPW][T][items_cap] (per-pair outputs only). The layout up to hq is the gate/up kernel's
// (lds_head), whose ids/p arrays (512 bytes) hold eoff here.
static size_t down_smem_bytes(int T, int k, int E, int Imax, int items_cap, bool combine) {
    size_t b = lds_head(E) + (size_t)(T * k + T) * (Imax / 32) * 128;
    if (!combine) b += (size_t)kDownWaves * kDownRows * T * items_cap * 4;
    return b;
}

// Each wave owns RPW output rows m; lane items are (slot, 32-block) pairs of those rows; a lane
// issues the loads of up to MAXJ items of every row before using any of them. The plan and h (fp16
// hi + lo pairs, about 22 bits, already in the LDS layout) come from the gate/up kernel and are
// copied into LDS first, so the dot products run on v_dot2_f32_f16 with fp32 accumulation.
// Per-pair outputs (no combine) keep each item's partial sum in LDS until its slot is complete; the
// slots are taken in chunks of spc (items_cap partials per wave, row and token), the shared
// expert's blocks last, so that any shape fits: each chunk is reduced in block order before the
// next one reuses the partials.
template <int FMT, int T, bool COMBINE>
__global__ __launch_bounds__(kDownThreads) void k_dec_down(LayerView L, const DecodePlan* __restrict__ plan_g,
                                                  const float* __restrict__ h, float* __restrict__ out,
                                                  float* __restrict__ y_pairs, float* __restrict__ y_shared,
                                                  int items_cap, int spc) {
    constexpr int RPW = kDownRows, MAXJ = down_batch(T);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    DecodePlan& P = *reinterpret_cast<DecodePlan*>(smem);
    // per slot: element offset of the expert's down scales (its codes sit block_bytes times further)
    int64_t* eoff = reinterpret_cast<int64_t*>(smem + align_up(sizeof(DecodePlan), 16) + align_up((size_t)L.E * 4, 16));
    uint4* hq = reinterpret_cast<uint4*>(smem + lds_head(L.E));
    const int Imax = L.Imax();
    const int nbm = Imax / 32;
    const int npairs = T * L.k;
    const int nrows_h = npairs + (L.Is > 0 ? T : 0);
    float* part = reinterpret_cast<float*>(hq + (size_t)(npairs + T) * 8 * nbm);
    // the plan first (the weight addresses depend on it), h (already staged) in flight behind it
    constexpr int kPlanWords = (int)(sizeof(DecodePlan) / 4);
    // uint4 of h per thread held in registers across the weight loads (2048, or 2560 from three
    // tokens on: the h loads past the batch go out behind the weights and wait for them; threads
    // past the end load the last piece again)
    constexpr int kHBatch = T >= 3 ? 5 : 4;
    const uint4* hs = reinterpret_cast<const uint4*>(h);
    // From three tokens on only the fp16 high halves of h are copied and multiplied (h at fp16, as
    // on the grouped-GEMM path): the staged activations are read from LDS once per output row, and
    // at four tokens those reads, not the weights, bound the kernel. One and two tokens keep hi +
    // lo (about 22 bits).
    constexpr bool kHiOnly = T >= 3;
    constexpr int NC = kHiOnly ? 4 : 8;          // uint4 per 32-block of an h row that are used
    const int hstride = NC * nbm;                // uint4 copied per h row
    const int n4 = nrows_h * hstride;            // uint4 copied
    // copied element i -> its uint4 in the staged rows (the same index in global memory and LDS)
    auto hidx = [&](int i) __attribute__((always_inline)) {
        if constexpr (kHiOnly) {
            const int row = i / hstride;
            return row * 8 * nbm + (i - row * hstride);
        } else {
            return i;
        }
    };
    const int hrot = (int)((blockIdx.x / 8) * 320u % (unsigned)n4);
    const uint32_t* ps = reinterpret_cast<const uint32_t*>(plan_g);
    uint32_t pw[(kPlanWords + kDownThreads - 1) / kDownThreads];
#pragma unroll
    for (int i = 0; i < (kPlanWords + kDownThreads - 1) / kDownThreads; ++i) {
        const int w = (int)threadIdx.x + kDownThreads * i;
        pw[i] = ps[min(w, kPlanWords - 1)];   // unconditional loads stay in flight together
    }
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // (a HIP uint4 array would live in scratch)
    const u32x4_t* hs4 = reinterpret_cast<const u32x4_t*>(h);
    u32x4_t hv0[kHBatch];
#pragma unroll
    for (int b = 0; b < kHBatch; ++b) {
        // every block reads all of h; each starts at its own offset, so that the blocks of an XCD do
        // not all ask for the same lines at once
        const int i = min((int)threadIdx.x + kDownThreads * b, n4 - 1) + hrot;
        hv0[b] = hs4[hidx(i < n4 ? i : i - n4)];
    }
    __builtin_amdgcn_sched_barrier(0);   // h loads are issued before the wait on the plan words
    {
        uint32_t* pd = reinterpret_cast<uint32_t*>(&P);
#pragma unroll
        for (int i = 0; i < (kPlanWords + kDownThreads - 1) / kDownThreads; ++i) {
            // unconditional (threads past the end write the last word again, with its own value):
            // a conditional store would let the compiler sink the load behind the h loads
            const int w = (int)threadIdx.x + kDownThreads * i;
            pd[min(w, kPlanWords - 1)] = pw[i];
        }
        // plan words 1 .. 64 are expert[0 .. 63] (nU comes first): their threads turn them into
        // the slots' matrix offsets once, instead of every lane per item
        static_assert(offsetof(DecodePlan, expert) == 4, "expert[] follows nU");
        const int s = (int)threadIdx.x - 1;
        if (s >= 0 && s < 64) eoff[s] = (int64_t)(int)pw[0] * L.H * (L.I / 32);
    }
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int H = L.H;
    const int nbI = L.I / 32, nbS = L.Is / 32;
    const int nU = P.nU;
    const int m0 = (blockIdx.x * kDownWaves + wave) * RPW;
    // per output row of the wave: element offsets of the row within a routed expert's scales and
    // within the shared expert's (codes: block_bytes times these)
    int offR[RPW], offSh[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int m = min(m0 + r, H - 1);
        offR[r] = m * nbI;
        offSh[r] = m * nbS;
    }
    const int qd = kWave / nbI, rd = kWave - qd * nbI;   // a lane's next item: 64 items further
    float* mypart = part + (size_t)wave * RPW * T * items_cap;
    // every item in one pass when the partials fit (always with the combine fused), else chunks of
    // spc routed slots and then the shared expert's blocks
    const bool one = COMBINE || nU * nbI + nbS <= items_cap;
    const int nrc = one ? 1 : (nU + spc - 1) / spc;   // chunks of routed slots
    const int nch = one ? 1 : nrc + (nbS > 0 ? 1 : 0);

    float acc[RPW][T];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r][t] = 0.f;

    bool h_in = false;   // h staged into LDS (by the first batch of loads; uniform over the block)
    for (int ch = 0; ch < nch; ++ch) {
        // routed slots [s0, s1) and, with has_sh, the shared expert: items [it0, it1)
        int s0, s1;
        bool has_sh;
        if (one) { s0 = 0; s1 = nU; has_sh = nbS > 0; }
        else if (ch < nrc) { s0 = ch * spc; s1 = min(s0 + spc, nU); has_sh = false; }
        else { s0 = s1 = nU; has_sh = true; }
        const int it0 = s0 * nbI, it1 = s1 * nbI + (has_sh ? nbS : 0);
        const int nit = (it1 - it0 + kWave - 1) / kWave;
    for (int j0 = 0; j0 < nit; j0 += MAXJ) {
        uint32_t w[RPW][MAXJ][8];
        uint16_t sdb[RPW][MAXJ];
        int slot_[MAXJ], b_[MAXJ];
        // up to four tokens: the row of h per item and token is looked up with the addresses (-1:
        // the token did not choose the slot) and the item's h is read from LDS in groups (the
        // registers this takes would spill from five tokens on, which keep the lookups in the loop)
        constexpr bool kBatchH = T <= 4;
        int hrow[MAXJ][kBatchH ? T : 1];
        bool ok[RPW][MAXJ];
        const uint8_t* dcp[RPW][MAXJ];
        const uint16_t* dsp[RPW][MAXJ];
        // addresses first; an item past the end reads expert 0's first row (valid memory, result
        // unused), so that every load below is unconditional and all of them stay in flight together.
        // Item it = (slot, block b) of the routed experts for it < nU nbI, then the shared expert's
        // blocks; one division per batch, then 64 items further per step.
        const int nUb = nU * nbI;
        int it = it0 + lane + kWave * j0;
        int slot = it / nbI, b = it - slot * nbI;
#pragma unroll
        for (int jj = 0; jj < MAXJ; ++jj) {
            if (jj > 0) {
                it += kWave;
                slot += qd;
                b += rd;
                if (b >= nbI) { b -= nbI; ++slot; }
            }
            const bool iv = it < it1;
            const bool routed = iv && it < nUb;
            const int bs = it - nUb;   // block of the shared expert
            slot_[jj] = routed ? slot : 64;
            b_[jj] = routed ? b : bs;
            if constexpr (kBatchH) {
#pragma unroll
                for (int t = 0; t < T; ++t) hrow[jj][t] = routed ? P.pair_of[routed ? slot : 0][t] : npairs + t;
            }
            const int64_t eo = eoff[routed ? slot : 0];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                ok[r][jj] = iv && m0 + r < H;
                const int64_t so = routed ? eo + (offR[r] + b) : iv ? (int64_t)(offSh[r] + bs) : (int64_t)0;
                dcp[r][jj] = (routed || !iv ? L.d_codes : L.sd_codes) + so * block_bytes(FMT);
                dsp[r][jj] = (routed || !iv ? L.d_scales : L.sd_scales) + so;
            }
        }
#pragma unroll
        for (int jj = 0; jj < MAXJ; ++jj)
#pragma unroll
            for (int r = 0; r < RPW; ++r) sdb[r][jj] = *dsp[r][jj];
#pragma unroll
        for (int jj = 0; jj < MAXJ; ++jj)
#pragma unroll
            for (int r = 0; r < RPW; ++r) load_codes<FMT>(dcp[r][jj], w[r][jj]);
        __builtin_amdgcn_sched_barrier(0);
        if (!h_in) {
            // h into LDS behind the first weight loads
            u32x4_t* hq4 = reinterpret_cast<u32x4_t*>(hq);
#pragma unroll
            for (int b = 0; b < kHBatch; ++b) {
                const int i = (int)threadIdx.x + kDownThreads * b;
                if (i < n4) hq4[hidx(i + hrot < n4 ? i + hrot : i + hrot - n4)] = hv0[b];
            }
            // the rest (unrolled: each group of loads in flight together, not one round trip each)
#pragma unroll 8
            for (int i = (int)threadIdx.x + kDownThreads * kHBatch; i < n4; i += kDownThreads) {
                const int ir = hidx(i + hrot < n4 ? i + hrot : i + hrot - n4);   // the same rotation
                hq[ir] = hs[ir];
            }
            __syncthreads();
            h_in = true;
        }
#pragma unroll
        for (int jj = 0; jj < MAXJ; ++jj) {
            const int slot = slot_[jj], b = b_[jj];
            const int it = it0 + lane + kWave * (j0 + jj);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                if (!ok[r][jj]) continue;
                uint32_t pd[16];
                float dt[T];   // the item's dot product per token
                if constexpr (kBatchH) {
                    // h (hi and lo) read from LDS TB tokens at a time, the first group before the
                    // codes are needed: the reads of a group are in flight together
                    constexpr int TB = T < 2 ? T : 2;
                    uint4 hv[TB][NC];
                    auto read_h = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) {
                            const int t = min(t0 + tb, T - 1);
                            const uint4* hp = hq + (size_t)max(hrow[jj][t], 0) * 8 * nbm + b;
#pragma unroll
                            for (int c = 0; c < NC; ++c) hv[tb][c] = hp[(size_t)c * nbm];
                        }
                        __builtin_amdgcn_sched_barrier(0);   // (the scheduler would pair them with the dot products)
                    };
                    read_h(0);
                    code_pairs<FMT>(w[r][jj], pd);
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        if (t > 0 && t % TB == 0) read_h(t);
                        float d = 0.f;
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const int j = 4 * (c & 3);
                            d = dot2(pd[j], hv[t % TB][c].x, d);
                            d = dot2(pd[j + 1], hv[t % TB][c].y, d);
                            d = dot2(pd[j + 2], hv[t % TB][c].z, d);
                            d = dot2(pd[j + 3], hv[t % TB][c].w, d);
                        }
                        dt[t] = hrow[jj][t] < 0 ? 0.f : d;
                    }
                } else {
                    code_pairs<FMT>(w[r][jj], pd);
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        const int row = slot < 64 ? P.pair_of[slot][t] : npairs + t;
                        float d = 0.f;
                        if (row >= 0) {
                            const uint4* hp = hq + (size_t)row * 8 * nbm + b;
#pragma unroll
                            for (int c = 0; c < NC; ++c) {
                                const uint4 hv = hp[(size_t)c * nbm];
                                const int j = 4 * (c & 3);
                                d = dot2(pd[j], hv.x, d);
                                d = dot2(pd[j + 1], hv.y, d);
                                d = dot2(pd[j + 2], hv.z, d);
                                d = dot2(pd[j + 3], hv.w, d);
                            }
                        }
                        dt[t] = d;
                    }
                }
                const float sd = f16_to_f32(sdb[r][jj]);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const float d = dt[t];
                    if constexpr (COMBINE) {
                        const float wgt = slot < 64 ? P.pw[slot][t] : 1.f;
                        acc[r][t] += wgt * sd * d;
                    } else {
                        mypart[((size_t)r * T + t) * items_cap + (it - it0)] = sd * d;
                    }
                }
            }
        }
    }
        if constexpr (!COMBINE) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane -> (row, slot of the chunk or the shared expert, token): the slot's block partials
            // summed in block order, read four at a time when the block counts allow (16-byte
            // aligned: the partial arrays then hold multiples of four); one path for routed slots
            // and the shared expert
            const int nr = s1 - s0, ns = nr + (has_sh ? 1 : 0);
            const bool vec4 = ((nbI | nbS) & 3) == 0;
            for (int st = lane; st < RPW * ns * T; st += kWave) {
                const int r = RPW == 1 ? 0 : st / (ns * T);
                const int rem = st - r * ns * T;
                const int sl = rem / T, t = rem - sl * T;
                const int m = m0 + r;
                const bool sh = sl >= nr;
                const int q = sh ? t : P.pair_of[s0 + sl][t];   // y_shared row (token) or y_pairs row
                const float sc = pow2f(-2 * P.xexp[t]);
                const int cnt = sh ? nbS : nbI;
                const float* pr = mypart + ((size_t)r * T + t) * items_cap + (size_t)(sh ? nr : sl) * nbI;
                float sum = 0.f;
                if (vec4) {
#pragma unroll 4
                    for (int b = 0; b < cnt; b += 4) {
                        const float4 v = *reinterpret_cast<const float4*>(pr + b);
                        sum += v.x;
                        sum += v.y;
                        sum += v.z;
                        sum += v.w;
                    }
                } else {
#pragma unroll 8
                    for (int b = 0; b < cnt; ++b) sum += pr[b];
                }
                if (m < H && q >= 0) (sh ? y_shared : y_pairs)[(size_t)q * H + m] = sum * sc;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    if constexpr (COMBINE) {
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float sm = wave_sum(acc[r][t]);
                if (lane == 0 && m0 + r < H) out[(size_t)t * H + m0 + r] = sm * pow2f(-2 * P.xexp[t]);
            }
    }
}

// ----------------------------------------------------------------------------------- launchers

moe_status launch_route_gemv(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                             float* logits, hipStream_t s) {
    const dim3 grid(E), block(256);
    switch (T) {
        case 1: hipLaunchKernelGGL(k_route_gemv<1>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 2: hipLaunchKernelGGL(k_route_gemv<2>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 3: hipLaunchKernelGGL(k_route_gemv<3>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 4: hipLaunchKernelGGL(k_route_gemv<4>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 5: hipLaunchKernelGGL(k_route_gemv<5>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 6: hipLaunchKernelGGL(k_route_gemv<6>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 7: hipLaunchKernelGGL(k_route_gemv<7>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 8: hipLaunchKernelGGL(k_route_gemv<8>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 9: hipLaunchKernelGGL(k_route_gemv<9>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 10: hipLaunchKernelGGL(k_route_gemv<10>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 11: hipLaunchKernelGGL(k_route_gemv<11>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 12: hipLaunchKernelGGL(k_route_gemv<12>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 13: hipLaunchKernelGGL(k_route_gemv<13>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 14: hipLaunchKernelGGL(k_route_gemv<14>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 15: hipLaunchKernelGGL(k_route_gemv<15>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        case 16: hipLaunchKernelGGL(k_route_gemv<16>, grid, block, 0, s, w_r, bias, x, H, E, logits); break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// h rows (T*k pairs then T shared tokens, Imax floats each, holding the staged fp16 hi/lo pairs),
// then the plan published by the gate/up kernel
static size_t h_floats(const LayerView& L, int T) { return (size_t)(T * L.k + T) * L.Imax(); }
size_t decode_scratch_floats(const LayerView& L, int T) {
    return h_floats(L, T) + align_up(sizeof(DecodePlan), 256) / 4;
}

constexpr size_t kMaxLds = 160 * 1024;   // LDS of a gfx950 workgroup

// LDS plan of the down kernel: for per-pair outputs, partials of items_cap items per wave, row and
// token (all slots at once when they fit, else chunks of spc whole slots).
struct DownFit {
    bool ok;
    int items_cap, spc;
    size_t smem;
};
static DownFit down_fit(const LayerView& L, int T, bool combine) {
    DownFit f{false, 0, 1, 0};
    const size_t base = down_smem_bytes(T, L.k, L.E, L.Imax(), 0, true);
    if (combine) {
        f.smem = base;
        f.ok = base <= kMaxLds;
        return f;
    }
    const int nbI = L.I / 32, nbS = L.Is / 32;
    const int slots = min(T * L.k, L.E);
    const int need = slots * nbI + nbS;               // every slot and the shared expert at once
    const size_t per_item = (size_t)kDownWaves * kDownRows * T * 4;
    const int avail = base < kMaxLds ? (int)((kMaxLds - base) / per_item) : 0;
    if (avail >= need) {
        f.items_cap = need;
        f.spc = slots;
        f.ok = true;
    } else {
        f.spc = avail / nbI;
        f.items_cap = max(f.spc * nbI, nbS);
        f.ok = f.spc >= 1 && f.items_cap <= avail;
    }
    f.smem = down_smem_bytes(T, L.k, L.E, L.Imax(), f.items_cap, false);
    f.ok = f.ok && f.smem <= kMaxLds;
    return f;
}

bool decode_fits(const LayerView& L, int T, bool combine) {
    return T >= 1 && T <= kMaxDecodeT && T * L.k <= 64 && gateup_smem_bytes(T, L.H, L.E) <= kMaxLds &&
           down_fit(L, T, combine).ok;
}

// Kernels asking for more than 64 KB of dynamic LDS must say so (gfx950 has 160 KB per workgroup).
template <typename K>
static bool allow_smem(K kernel, size_t bytes) {
    if (bytes > kMaxLds) return false;
    if (bytes <= 65536) return true;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess;
}

// Compute units of the current device (cached per device; callers on several host threads may
// race to fill an entry, with the same value).
static int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int FMT, int T, bool ROUTE, int KPL>
static moe_status launch_gateup(const LayerView& L, const uint16_t* x, const float* logits, int32_t* ids, float* p,
                                float* h, DecodePlan* plan_g, hipStream_t s) {
    constexpr int R = gateup_rows(T);
    const int64_t waves1 = (int64_t)T * L.k * ((L.I + R - 1) / R) + (L.Is + R - 1) / R;   // tasks, at most
    const size_t sm = gateup_smem_bytes(T, L.H, L.E);
    auto kern = k_dec_gateup<FMT, T, ROUTE, KPL>;
    if (!allow_smem(kern, sm)) return MOE_ERR_UNSUPPORTED;
    // waves per block chosen so that the blocks spread evenly over the CUs (4..16 waves), and at
    // most one block per CU: the waves stride over the rows of the experts actually chosen
    const int cus = cu_count();
    // (with routing, every token's top-k needs a wave of its own: at least T waves)
    const int64_t wpb = std::max<int64_t>(ROUTE ? T : 1, std::min<int64_t>(gateup_max_waves(T),
                                                                          std::max<int64_t>(4, (waves1 + cus - 1) / cus)));
    const int64_t blocks = std::min<int64_t>((waves1 + wpb - 1) / wpb, cus);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3((unsigned)(wpb * kWave)), sm, s, L, x, logits, ids, p, h,
                       plan_g);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

template <int FMT, int T>
static moe_status launch_experts_t(const LayerView& L, const uint16_t* x, const float* logits, int32_t* ids, float* p,
                                   float* h, float* out, float* y_pairs, float* y_shared, hipStream_t s) {
    DecodePlan* plan_g = reinterpret_cast<DecodePlan*>(h + h_floats(L, T));
    // both kernels' LDS is settled before anything is enqueued
    const bool combine = out != nullptr;
    const DownFit fit = down_fit(L, T, combine);
    if (!fit.ok) return MOE_ERR_UNSUPPORTED;
    if (combine ? !allow_smem(k_dec_down<FMT, T, true>, fit.smem) : !allow_smem(k_dec_down<FMT, T, false>, fit.smem))
        return MOE_ERR_UNSUPPORTED;
    moe_status st;
    if (!logits) st = launch_gateup<FMT, T, false, 1>(L, x, nullptr, ids, nullptr, h, plan_g, s);
    else if (L.E <= 64) st = launch_gateup<FMT, T, true, 1>(L, x, logits, ids, p, h, plan_g, s);
    else if (L.E <= 128) st = launch_gateup<FMT, T, true, 2>(L, x, logits, ids, p, h, plan_g, s);
    else if (L.E <= 256) st = launch_gateup<FMT, T, true, 4>(L, x, logits, ids, p, h, plan_g, s);
    else if (L.E <= 512) st = launch_gateup<FMT, T, true, 8>(L, x, logits, ids, p, h, plan_g, s);
    else st = launch_gateup<FMT, T, true, 16>(L, x, logits, ids, p, h, plan_g, s);
    if (st != MOE_OK) return st;
    const int blocks = (L.H + kDownWaves * kDownRows - 1) / (kDownWaves * kDownRows);
    if (combine)
        hipLaunchKernelGGL((k_dec_down<FMT, T, true>), dim3(blocks), dim3(kDownThreads), fit.smem, s, L, plan_g, h, out,
                           nullptr, nullptr, 0, 1);
    else
        hipLaunchKernelGGL((k_dec_down<FMT, T, false>), dim3(blocks), dim3(kDownThreads), fit.smem, s, L, plan_g, h,
                           nullptr, y_pairs, y_shared, fit.items_cap, fit.spc);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

template <int FMT>
static moe_status launch_experts_f(const LayerView& L, const uint16_t* x, int T, const float* logits, int32_t* ids,
                                   float* p, float* h, float* out, float* y_pairs, float* y_shared, hipStream_t s) {
    switch (T) {
        case 1: return launch_experts_t<FMT, 1>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 2: return launch_experts_t<FMT, 2>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 3: return launch_experts_t<FMT, 3>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 4: return launch_experts_t<FMT, 4>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 5: return launch_experts_t<FMT, 5>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 6: return launch_experts_t<FMT, 6>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 7: return launch_experts_t<FMT, 7>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        case 8: return launch_experts_t<FMT, 8>(L, x, logits, ids, p, h, out, y_pairs, y_shared, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

moe_status launch_decode_experts(const LayerView& L, const uint16_t* x, int T, const float* logits, int32_t* ids,
                                 float* p, float* h, float* out, float* y_pairs, float* y_shared, hipStream_t s) {
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_experts_f<MOE_Q8_B32>(L, x, T, logits, ids, p, h, out, y_pairs, y_shared, s);
        case MOE_Q4_B32: return launch_experts_f<MOE_Q4_B32>(L, x, T, logits, ids, p, h, out, y_pairs, y_shared, s);
        case MOE_Q2_B32: return launch_experts_f<MOE_Q2_B32>(L, x, T, logits, ids, p, h, out, y_pairs, y_shared, s);
        default: return MOE_ERR_INVALID_ARG;
    }
}

}  // namespace moe
