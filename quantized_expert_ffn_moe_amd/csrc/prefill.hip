// Prefill-regime experts: grouped GEMM over expert-sorted row tiles on the gfx950 matrix cores.
//
// Prompt processing on the pages runs in 8K-token chunks with GEMMs and grouped expert kernels
// (648news 07-nano-cuda-moe-qwen38-release, section "speed comparison and accuracy check"). Here:
//   - the pairs of each expert are contiguous after the permutation; a tile list of
//     (group, first row) covers every group with 128-row tiles, the shared expert being one more
//     group of all T tokens;
//   - one kernel template, two uses: gate/up (A = x rows gathered through perm, B = 128 gate rows
//     and 128 up rows interleaved in 32-row granules so that g and u of the same (row, n) meet in
//     one lane; SwiGLU epilogue writes h in fp16) and down (A = h rows in sorted order, B = 256
//     down rows; fp32 output rows);
//   - block tile 128 x 256, four waves of 64 x 128, K steps of 32 through double-buffered LDS
//     (rows padded to 80 bytes: the 16-byte fragment reads of 16 lanes hit distinct banks), two
//     v_mfma_f32_32x32x16_f16 per 32 x 32 output tile and K step (on this chip the 32 x 32 form
//     sustains a far higher rate than 16 x 16 x 32);
//   - weights are dequantised in registers: the code is OR-ed into the mantissa of 1024.0, the
//     offset subtracted (an exact fp16 level) and multiplied by the fp16 scale with packed fp16
//     arithmetic, i.e. level * scale rounded once to fp16. The pairs come out in an order that
//     permutes K inside each 4-, 8- or 16-element group; x (converted from bf16) and h are stored
//     with the same permutation so the dot products are unchanged;
//   - blocks are mapped so that consecutive row tiles of one expert (which share a weight panel)
//     run on the same XCD and reuse it from that XCD's L2.
#include <utility>

#include "kernels.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;      // rows (pairs) per tile
constexpr int kBN = 256;      // weight rows per tile
constexpr int kAS = 64 + 8;   // fp16 per A row in LDS: one step of K = 64, padded to 144 bytes
constexpr int kXcds = 8;

struct TileDesc {
    int group;  // expert id, or E for the shared expert
    int row0;   // first row of the tile inside its group
};

// -------------------------------------------------------------------------------- tile list
// One block of 1024 threads: thread e counts the tiles of expert e, a block scan places them,
// the shared group's tiles follow the routed ones. Offsets are clamped to [0, T*k] and the list
// to tiles_max entries, so that inconsistent offsets cannot move any access out of bounds.
__device__ __forceinline__ void group_rows(const int32_t* offsets, int E, int T, int Tk, int g, int& base,
                                           int& count) {
    if (g == E) { base = 0; count = T; return; }
    base = min(max(offsets[g], 0), Tk);
    count = min(max(offsets[g + 1], base), Tk) - base;
}

__global__ __launch_bounds__(1024) void k_build_tiles(const int32_t* __restrict__ offsets, int E, int T, int k,
                                                      int has_shared, int tiles_max, TileDesc* __restrict__ tiles,
                                                      int32_t* __restrict__ ntiles) {
    __shared__ int part[1024];
    const int e = threadIdx.x;
    int base = 0, n = 0;
    if (e < E) group_rows(offsets, E, T, T * k, e, base, n);
    const int nt = (n + kBM - 1) / kBM;
    part[e] = nt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = e >= d ? part[e - d] : 0;
        __syncthreads();
        part[e] += v;
        __syncthreads();
    }
    const int start = part[e] - nt;
    for (int i = 0; i < nt && start + i < tiles_max; ++i) tiles[start + i] = TileDesc{e, i * kBM};
    if (e == 1023) {
        int total = min(part[1023], tiles_max);
        if (has_shared) {
            const int ns = (T + kBM - 1) / kBM;
            for (int i = 0; i < ns && total < tiles_max; ++i) tiles[total++] = TileDesc{E, i * kBM};
        }
        *ntiles = total;
    }
}

int max_tiles(int T, int k, int E) { return (T * k) / kBM + E + (T + kBM - 1) / kBM + 1; }

// -------------------------------------------------------------------------------- K permutation

// Group size of the K permutation of a format's dequantised pairs, and the position of natural
// element e inside its group: pair j of a dword holds elements (j, j + G/2) of the group.
template <int FMT> __host__ __device__ constexpr int perm_group() {
    return FMT == MOE_Q4_B32 ? 8 : FMT == MOE_Q8_B32 ? 4 : 16;
}
__host__ __device__ inline int kperm(int e, int G) {
    const int g = e / G, r = e % G, h = G / 2;
    return g * G + 2 * (r % h) + r / h;
}

// -------------------------------------------------------------------------------- x to fp16
// x (bf16) -> fp16, 16 elements per thread, stored with the format's K permutation.
template <int G>
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, int64_t n16, _Float16* __restrict__ x16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n16) return;
    const uint4* src = reinterpret_cast<const uint4*>(x) + 2 * i;
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    _Float16 o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float v = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
        o[kperm(e, G)] = (_Float16)v;
    }
    half8* dst = reinterpret_cast<half8*>(x16) + 2 * i;
    half8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) { lo[e] = o[e]; hi[e] = o[8 + e]; }
    dst[0] = lo;
    dst[1] = hi;
}

// -------------------------------------------------------------------------------- dequantisation

constexpr uint32_t kMagic16 = 0x64006400u;   // (1024.0, 1024.0) as fp16 pair

__device__ __forceinline__ uint32_t h2bits(half2v v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ half2v bits2h(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// Codes of one 32-element block held by a lane: Q4 16 bytes (c0), Q8 32 bytes (c0, c1), Q2 8 bytes
// (c0.xy).
struct BlockCodes {
    u32x4 c0, c1;
};

template <int FMT>
__device__ __forceinline__ void load_codes(const uint8_t* p, BlockCodes& b) {
    if constexpr (FMT == MOE_Q8_B32) {
        b.c0 = reinterpret_cast<const u32x4*>(p)[0];
        b.c1 = reinterpret_cast<const u32x4*>(p)[1];
    } else if constexpr (FMT == MOE_Q4_B32) {
        b.c0 = reinterpret_cast<const u32x4*>(p)[0];
    } else {
        const u32x2 v = reinterpret_cast<const u32x2*>(p)[0];
        b.c0.x = v.x;
        b.c0.y = v.y;
    }
}

__device__ __forceinline__ uint32_t dword_of(const BlockCodes& b, int d) {
    switch (d) {
        case 0: return b.c0.x;
        case 1: return b.c0.y;
        case 2: return b.c0.z;
        case 3: return b.c0.w;
        case 4: return b.c1.x;
        case 5: return b.c1.y;
        case 6: return b.c1.z;
        default: return b.c1.w;
    }
}

// Pairs 4 kk .. 4 kk + 3 of a block (K-permuted positions 8 kk .. 8 kk + 7) as level * scale,
// each rounded once to fp16. Pair p of a block holds elements (j, j + G/2) of its G-group:
//   Q4: dword d = elements 8d .. 8d+7, pair 4d + j = nibbles (j, j + 4), offset 1032 = 1024 + 8;
//   Q8: dword d = elements 4d .. 4d+3, pairs 2d (bytes 0, 2) and 2d + 1 (bytes 1, 3), offset 1152;
//   Q2: dword d = elements 16d .. 16d+15, pair 8d + j = crumbs (j, j + 8) as 2c + 1024, offset
//       1027 = 1024 + 2 * 1.5, times s / 2.
template <int FMT, int KK>
__device__ __forceinline__ half8 dequant8(const BlockCodes& b, half2v sv) {
    uint32_t o[4];
    if constexpr (FMT == MOE_Q4_B32) {
        const half2v off = {(_Float16)1032.f, (_Float16)1032.f};
        const uint32_t u = dword_of(b, KK) ^ 0x88888888u;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = h2bits((bits2h(((u >> (4 * j)) & 0x000F000Fu) | kMagic16) - off) * sv);
    } else if constexpr (FMT == MOE_Q8_B32) {
        const half2v off = {(_Float16)1152.f, (_Float16)1152.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t u = dword_of(b, 2 * KK + h) ^ 0x80808080u;
            o[2 * h] = h2bits((bits2h((u & 0x00FF00FFu) | kMagic16) - off) * sv);
            o[2 * h + 1] = h2bits((bits2h(((u >> 8) & 0x00FF00FFu) | kMagic16) - off) * sv);
        }
    } else {
        const half2v off = {(_Float16)1027.f, (_Float16)1027.f};
        const half2v s2 = sv * half2v{(_Float16)0.5f, (_Float16)0.5f};
        const uint32_t u = dword_of(b, KK / 2);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            constexpr int j0 = 4 * (KK % 2);
            const int j = j0 + jj;
            const uint32_t t = j == 0 ? (u << 1) : (u >> (2 * j - 1));
            o[jj] = h2bits((bits2h((t & 0x00060006u) | kMagic16) - off) * s2);
        }
    }
    return __builtin_bit_cast(half8, u32x4{o[0], o[1], o[2], o[3]});
}

// -------------------------------------------------------------------------------- grouped GEMM

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One pipeline step of loads (K = 64, two 32-blocks): four 16-byte chunks of A for the LDS stage,
// and for each of the lane's two weight tiles the codes and the scale of the lane's own block.
// Plain members only: a slot must never be indexed at run time, or it would leave the registers.
struct StepSlot {
    u32x4 a0, a1, a2, a3;
    BlockCodes b0, b1;
    uint32_t s0, s1;
};

// YT: type of the down outputs (float, or _Float16 for the fused layer's internal rows).
template <int FMT, bool GATEUP, typename YT = float>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm(LayerView L, int T, const TileDesc* __restrict__ tiles,
                                                         const int32_t* __restrict__ ntiles, int n_ntile,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ perm,
                                                         const _Float16* __restrict__ asrc, _Float16* __restrict__ h16,
                                                         YT* __restrict__ y_sorted, YT* __restrict__ y_shared) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][kBM * kAS];
    constexpr int G = perm_group<FMT>();
    constexpr int BB = FMT == MOE_Q8_B32 ? 32 : FMT == MOE_Q4_B32 ? 16 : 8;   // bytes per block

    // XCD-aware work index: block b runs on XCD b % 8, and consecutive work items go to the same
    // XCD. Work items are ordered tile-major: the weight-row tiles of one row tile (same A rows)
    // run side by side, and so do the row tiles of one expert (same weights). The grid is sized for
    // the largest possible tile count; the split uses the real count so that every XCD gets an
    // equal share.
    const int nt = *ntiles;
    const int total = nt * n_ntile;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int idx = (int)(blockIdx.x / kXcds);
    if (idx >= per_xcd) return;
    const int w = (int)(blockIdx.x % kXcds) * per_xcd + idx;
    if (w >= total) return;
    const int tile = w / n_ntile, ntile = w % n_ntile;
    const TileDesc td = tiles[tile];
    const bool shared = td.group == L.E;
    const int H = L.H, Imax = L.Imax();
    int N, n0, K;
    if constexpr (GATEUP) {
        N = shared ? L.Is : L.I;          // h columns of this group
        n0 = ntile * (kBN / 2);
        K = H;
    } else {
        N = H;
        n0 = ntile * kBN;
        K = shared ? L.Is : L.I;
    }
    if (n0 >= N) return;
    const int Tk = T * L.k;
    int base, count;
    group_rows(offsets, L.E, T, Tk, td.group, base, count);
    const int nrows = min(kBM, count - td.row0);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int frow = lane % 32, g = lane / 32;
    const int nb = K / 32;                    // scale blocks along K
    const int nsteps = (nb + 1) / 2;

    // Operand rows past the tile's valid rows or columns are clamped to a valid row: they only feed
    // output rows or columns that are never stored, and every load stays unconditional (so the
    // compiler can keep several steps of loads in flight).
    // A: thread -> 16-byte chunk c = tid % 8 of rows tid / 8 + 32 q (q = 0..3) of every step
    const int ac = tid & 7;
    const _Float16* arow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = (tid >> 3) + 32 * q;
        const int pos = td.row0 + min(r, nrows - 1);
        if constexpr (GATEUP) {
            const int qq = shared ? pos * L.k : perm[base + pos];
            const int tok = (unsigned)qq < (unsigned)Tk ? qq / L.k : 0;
            arow[q] = asrc + (size_t)tok * H;
        } else {
            const int64_t hrow = shared ? (int64_t)Tk + pos : (int64_t)base + pos;
            arow[q] = asrc + (size_t)hrow * Imax;
        }
    }
    // B: wave w owns weight rows 64 w .. 64 w + 63 of the tile as two 32-row MFMA tiles; lane
    // (frow, g) loads, for each tile, block 2 s + g of its row at step s and dequantises it
    // straight into its MFMA operand (no LDS). Gate/up: tile 0 = gate rows, tile 1 = up rows of
    // the same h columns n0 + 32 w + [0, 32); down: output columns n0 + 64 w + [0, 64).
    const uint8_t* bc[2];
    const uint16_t* bs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if constexpr (GATEUP) {
            const int n = min(n0 + 32 * wave + frow, N - 1);
            const int64_t rb = (int64_t)nb * BB;
            if (shared) {
                bc[j] = (j ? L.su_codes : L.sg_codes) + (int64_t)n * rb;
                bs[j] = (j ? L.su_scales : L.sg_scales) + (int64_t)n * nb;
            } else {
                const int64_t row = (int64_t)td.group * L.I + n;
                bc[j] = (j ? L.u_codes : L.g_codes) + row * rb;
                bs[j] = (j ? L.u_scales : L.g_scales) + row * nb;
            }
        } else {
            const int m = min(n0 + 64 * wave + 32 * j + frow, H - 1);
            const int64_t rb = (int64_t)nb * BB;
            if (shared) {
                bc[j] = L.sd_codes + (int64_t)m * rb;
                bs[j] = L.sd_scales + (int64_t)m * nb;
            } else {
                const int64_t row = (int64_t)td.group * H + m;
                bc[j] = L.d_codes + row * rb;
                bs[j] = L.d_scales + row * nb;
            }
        }
    }

    StepSlot ring0, ring1;
    auto ring = [&](auto rc) __attribute__((always_inline)) -> StepSlot& {
        if constexpr (decltype(rc)::value == 0) return ring0;
        else return ring1;
    };
    auto gload = [&](StepSlot& sl, int s) __attribute__((always_inline)) {
        s = min(s, nsteps - 1);
        const int ka = min(64 * s + 8 * ac, K - 8);   // a chunk past K reloads the last one (zeroed in lstore)
        sl.a0 = *reinterpret_cast<const u32x4*>(arow[0] + ka);
        sl.a1 = *reinterpret_cast<const u32x4*>(arow[1] + ka);
        sl.a2 = *reinterpret_cast<const u32x4*>(arow[2] + ka);
        sl.a3 = *reinterpret_cast<const u32x4*>(arow[3] + ka);
        const int b = min(2 * s + g, nb - 1);
        load_codes<FMT>(bc[0] + (int64_t)b * BB, sl.b0);
        load_codes<FMT>(bc[1] + (int64_t)b * BB, sl.b1);
        sl.s0 = bs[0][b];
        sl.s1 = bs[1][b];
    };
    // A chunk past K (the second half of a last step when K % 64 == 32) is written as zeros
    auto lstore = [&](const StepSlot& sl, int st, int s) __attribute__((always_inline)) {
        const bool live = 64 * s + 8 * ac < K;
        const u32x4 z = {0u, 0u, 0u, 0u};
        _Float16* dst = &As[st][(tid >> 3) * kAS + 8 * ac];
        *reinterpret_cast<u32x4*>(dst) = live ? sl.a0 : z;
        *reinterpret_cast<u32x4*>(dst + 32 * kAS) = live ? sl.a1 : z;
        *reinterpret_cast<u32x4*>(dst + 64 * kAS) = live ? sl.a2 : z;
        *reinterpret_cast<u32x4*>(dst + 96 * kAS) = live ? sl.a3 : z;
    };

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // one step: dequantise this lane's blocks of slot s % 2, MFMAs against LDS stage s & 1
    // (A fragment of lane (frow, g) for sub-step kk: row 32 i + frow, K offset 32 g + 8 kk), then
    // A of step s + 1 into the other stage, refill the slot with step s + 2, barrier
    auto kstep = [&](int s, auto rc) __attribute__((always_inline)) {
        StepSlot& cur_sl = ring(rc);
        StepSlot& nxt_sl = ring(std::integral_constant<int, 1 - decltype(rc)::value>{});
        const int cur = s & 1;
        const bool blive = 2 * s + g < nb;     // a block past K contributes zero
        const _Float16 s0 = blive ? __builtin_bit_cast(_Float16, (uint16_t)cur_sl.s0) : (_Float16)0.f;
        const _Float16 s1 = blive ? __builtin_bit_cast(_Float16, (uint16_t)cur_sl.s1) : (_Float16)0.f;
        const half2v sv0 = {s0, s0}, sv1 = {s1, s1};
        static_for<4>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            const half8 b0 = dequant8<FMT, kk>(cur_sl.b0, sv0);
            const half8 b1 = dequant8<FMT, kk>(cur_sl.b1, sv1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half8 a = *reinterpret_cast<const half8*>(&As[cur][(32 * i + frow) * kAS + 32 * g + 8 * kk]);
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc[i][1], 0, 0, 0);
            }
        });
        gload(cur_sl, s + 2);
        __builtin_amdgcn_sched_barrier(0);   // issue the refill before waiting on the next step's A
        lstore(nxt_sl, cur ^ 1, s + 1);
        __syncthreads();
    };
    gload(ring0, 0);
    gload(ring1, 1);
    lstore(ring0, 0, 0);
    __syncthreads();
    // the slot of step s + 1 (read by lstore) must be complete before its refill: within a step,
    // the refill targets slot s % 2 and lstore reads slot (s + 1) % 2
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        kstep(s, std::integral_constant<int, 0>{});
        kstep(s + 1, std::integral_constant<int, 1>{});
    }
    if (s < nsteps) kstep(s, std::integral_constant<int, 0>{});

    const int rq = 4 * g;
    if constexpr (GATEUP) {
        const int n = n0 + 32 * wave + frow;
        if (n < N) {
            const int np = kperm(n, G);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r / 4) + rq + r % 4;
                    if (row >= nrows) continue;
                    const float hv = silu_mul(acc[i][0][r], acc[i][1][r]);
                    const int64_t hrow = shared ? (int64_t)Tk + td.row0 + row : (int64_t)base + td.row0 + row;
                    h16[hrow * Imax + np] = (_Float16)hv;
                }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = n0 + 64 * wave + 32 * j + frow;
            if (m >= H) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r / 4) + rq + r % 4;
                    if (row >= nrows) continue;
                    if (shared) y_shared[(int64_t)(td.row0 + row) * H + m] = (YT)acc[i][j][r];
                    else y_sorted[((int64_t)base + td.row0 + row) * H + m] = (YT)acc[i][j][r];
                }
        }
    }
}

// -------------------------------------------------------------------------------- launch

struct PrefillScratch {
    TileDesc* tiles;
    int32_t* ntiles;
    _Float16* x16;
    _Float16* h16;
};

static PrefillScratch carve_prefill(const LayerView& L, int T, void* base, size_t* bytes) {
    Carve c(base);
    PrefillScratch s;
    s.tiles = c.take<TileDesc>((size_t)max_tiles(T, L.k, L.E));
    s.ntiles = c.take<int32_t>(1);
    s.x16 = c.take<_Float16>((size_t)T * L.H);
    s.h16 = c.take<_Float16>((size_t)(T * L.k + T) * L.Imax());
    if (bytes) *bytes = c.bytes();
    return s;
}

size_t prefill_scratch_bytes(const LayerView& L, int T) {
    size_t b = 0;
    carve_prefill(L, T, nullptr, &b);
    return b;
}

template <int FMT>
static moe_status launch_prefill_f(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                   const int32_t* perm, void* y_sorted, void* y_shared, bool y16,
                                   const PrefillScratch& s, hipStream_t st) {
    constexpr int G = perm_group<FMT>();
    const int64_t n16 = (int64_t)T * L.H / 16;
    hipLaunchKernelGGL(k_x_to_f16<G>, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, x, n16, s.x16);
    MOE_LAUNCH_CHECK();
    const int mt = max_tiles(T, L.k, L.E);
    const int nt1 = (L.Imax() + kBN / 2 - 1) / (kBN / 2);
    const int g1 = ((mt * nt1 + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL((k_grouped_gemm<FMT, true>), dim3(g1), dim3(256), 0, st, L, T, s.tiles, s.ntiles, nt1,
                       offsets, perm, s.x16, s.h16, (float*)nullptr, (float*)nullptr);
    MOE_LAUNCH_CHECK();
    const int nt2 = (L.H + kBN - 1) / kBN;
    const int g2 = ((mt * nt2 + kXcds - 1) / kXcds) * kXcds;
    if (y16)
        hipLaunchKernelGGL((k_grouped_gemm<FMT, false, _Float16>), dim3(g2), dim3(256), 0, st, L, T, s.tiles,
                           s.ntiles, nt2, offsets, perm, s.h16, nullptr, static_cast<_Float16*>(y_sorted),
                           static_cast<_Float16*>(y_shared));
    else
        hipLaunchKernelGGL((k_grouped_gemm<FMT, false, float>), dim3(g2), dim3(256), 0, st, L, T, s.tiles,
                           s.ntiles, nt2, offsets, perm, s.h16, nullptr, static_cast<float*>(y_sorted),
                           static_cast<float*>(y_shared));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_prefill_experts(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                  const int32_t* perm, void* y_sorted, void* y_shared, bool y16, void* scratch,
                                  hipStream_t st) {
    const PrefillScratch s = carve_prefill(L, T, scratch, nullptr);
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, st, offsets, L.E, T, L.k, L.Is > 0 ? 1 : 0,
                       max_tiles(T, L.k, L.E), s.tiles, s.ntiles);
    MOE_LAUNCH_CHECK();
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_prefill_f<MOE_Q8_B32>(L, x, T, offsets, perm, y_sorted, y_shared, y16, s, st);
        case MOE_Q4_B32: return launch_prefill_f<MOE_Q4_B32>(L, x, T, offsets, perm, y_sorted, y_shared, y16, s, st);
        case MOE_Q2_B32: return launch_prefill_f<MOE_Q2_B32>(L, x, T, offsets, perm, y_sorted, y_shared, y16, s, st);
        default: return MOE_ERR_INVALID_ARG;
    }
}

}  // namespace moe
