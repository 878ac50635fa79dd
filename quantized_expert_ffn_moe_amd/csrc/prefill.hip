// Prefill-regime experts: grouped GEMM over expert-sorted row tiles on the gfx950 matrix cores.
//
// Prompt processing on the pages runs in 8K-token chunks with GEMMs and grouped expert kernels
// (648news 07-nano-cuda-moe-qwen38-release, section "speed comparison and accuracy check"). Here:
//   - the pairs of each expert are contiguous after the permutation; a tile list of
//     (group, first row) covers every group with 128-row tiles, the shared expert being one more
//     group of all T tokens;
//   - one kernel template, two uses: gate/up (A = x rows gathered through perm, B = 128 gate rows
//     and 128 up rows interleaved in 16-row granules so that g and u of the same (row, n) meet in
//     one lane; SwiGLU epilogue writes h in fp16) and down (A = h rows in sorted order, B = 256
//     down rows; fp32 output rows);
//   - block tile 128 x 256, four waves of 64 x 128, K steps of 32 through double-buffered LDS
//     (rows padded to 80 bytes: the 16-byte fragment reads of 16 lanes hit distinct banks), one
//     v_mfma_f32_16x16x32_f16 per 16 x 16 output tile and K step;
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
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;      // rows (pairs) per tile
constexpr int kBN = 256;      // weight rows per tile
constexpr int kBK = 32;       // K per step (one scale block)
constexpr int kLds = kBK + 8; // fp16 per LDS row (80 bytes)
constexpr int kXcds = 8;
constexpr int kPD = 3;        // K steps of global loads in flight

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

// One 32-element block -> 16 fp16 pairs (level * scale, rounded once), in K-permuted order.
template <int FMT>
__device__ __forceinline__ void dequant16(const uint32_t (&w)[8], uint16_t sbits, uint32_t (&o)[16]) {
    const _Float16 s = __builtin_bit_cast(_Float16, sbits);
    const half2v sv = {s, s};
    if constexpr (FMT == MOE_Q4_B32) {
        const half2v off = {(_Float16)1032.f, (_Float16)1032.f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t u = w[d] ^ 0x88888888u;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[4 * d + j] = h2bits((bits2h(((u >> (4 * j)) & 0x000F000Fu) | kMagic16) - off) * sv);
        }
    } else if constexpr (FMT == MOE_Q8_B32) {
        const half2v off = {(_Float16)1152.f, (_Float16)1152.f};
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const uint32_t u = w[d] ^ 0x80808080u;
            o[2 * d] = h2bits((bits2h((u & 0x00FF00FFu) | kMagic16) - off) * sv);
            o[2 * d + 1] = h2bits((bits2h(((u >> 8) & 0x00FF00FFu) | kMagic16) - off) * sv);
        }
    } else {
        // 1024 + 2c - 1027 = 2 (c - 1.5), times s / 2
        const half2v off = {(_Float16)1027.f, (_Float16)1027.f};
        const half2v s2 = sv * half2v{(_Float16)0.5f, (_Float16)0.5f};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t u = w[d];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t t = j == 0 ? (u << 1) : (u >> (2 * j - 1));
                o[8 * d + j] = h2bits((bits2h((t & 0x00060006u) | kMagic16) - off) * s2);
            }
        }
    }
}

template <int FMT>
__device__ __forceinline__ void load_block_codes(const uint8_t* p, uint32_t (&w)[8]) {
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

// -------------------------------------------------------------------------------- grouped GEMM

// Registers holding one K step of global loads: two 16-byte A chunks, one block of codes (16 bytes
// for Q4, 32 for Q8, 8 for Q2) and its scale. Plain members, no arrays: a slot must never be
// indexed at run time, or it would leave the registers.
struct LoadSlot {
    u32x4 a0, a1;
    u32x4 b0, b1;
    uint32_t s;
};

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm(LayerView L, int T, const TileDesc* __restrict__ tiles,
                                                         const int32_t* __restrict__ ntiles, int n_ntile, const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ perm,
                                                         const _Float16* __restrict__ asrc, _Float16* __restrict__ h16,
                                                         float* __restrict__ y_sorted, float* __restrict__ y_shared) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][kBM * kLds];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][kBN * kLds];
    constexpr int G = perm_group<FMT>();

    // XCD-aware work index: block b runs on XCD b % 8, and consecutive work items go to the same
    // XCD. Work items are ordered tile-major: the weight-row tiles of one row tile (same A rows)
    // run side by side, and so do the row tiles of one expert (same weights). The grid is sized for
    // tiles_max tiles; the split uses the real count so that every XCD gets an equal share.
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
    const int wm = wave / 2, wn = wave % 2;

    // Operand rows past the tile's valid rows or columns are clamped to a valid row: they only feed
    // output rows or columns that are never stored, and every load stays unconditional (so the
    // compiler can keep several K steps of loads in flight).
    // A: thread -> two 16-byte chunks (rows tid/4 and tid/4 + 64, quarter tid % 4) of every K step
    const _Float16* aptr[2];
    int arow[2];
    const int aq = tid & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = (tid >> 2) + 64 * i;
        arow[i] = r;
        const int pos = td.row0 + min(r, nrows - 1);
        if constexpr (GATEUP) {
            const int q = shared ? pos * L.k : perm[base + pos];
            const int tok = (unsigned)q < (unsigned)Tk ? q / L.k : 0;
            aptr[i] = asrc + (size_t)tok * H + aq * 8;
        } else {
            const int64_t hrow = shared ? (int64_t)Tk + pos : (int64_t)base + pos;
            aptr[i] = asrc + (size_t)hrow * Imax + aq * 8;
        }
    }
    // B: thread -> LDS row tid (one weight row; one 32-block per K step)
    const uint8_t* bcodes;
    const uint16_t* bscales;
    if constexpr (GATEUP) {
        const int gran = tid / 16;
        const bool is_up = gran & 1;
        const int n = min(n0 + (gran / 2) * 16 + tid % 16, N - 1);
        const int64_t rb = row_bytes(FMT, H);
        if (shared) {
            bcodes = (is_up ? L.su_codes : L.sg_codes) + (int64_t)n * rb;
            bscales = (is_up ? L.su_scales : L.sg_scales) + (int64_t)n * (H / 32);
        } else {
            const int64_t row = (int64_t)td.group * L.I + n;
            bcodes = (is_up ? L.u_codes : L.g_codes) + row * rb;
            bscales = (is_up ? L.u_scales : L.g_scales) + row * (H / 32);
        }
    } else {
        const int m = min(n0 + tid, H - 1);
        const int64_t rb = row_bytes(FMT, K);
        if (shared) {
            bcodes = L.sd_codes + (int64_t)m * rb;
            bscales = L.sd_scales + (int64_t)m * (K / 32);
        } else {
            const int64_t row = (int64_t)td.group * H + m;
            bcodes = L.d_codes + row * rb;
            bscales = L.d_scales + row * (K / 32);
        }
    }

    // Global loads run kPD K steps ahead through a ring of register slots: slot r holds step j
    // with j % kPD == r (steps past the end reload the last one). LDS is double-buffered: stage
    // ks & 1 holds step ks. Slots are only ever named with compile-time indices so that they stay
    // in registers.
    LoadSlot ring0, ring1, ring2;
    auto ring = [&](auto rc) __attribute__((always_inline)) -> LoadSlot& {
        constexpr int i = decltype(rc)::value;
        static_assert(i < 3, "at most three slots");
        if constexpr (i == 0) return ring0;
        else if constexpr (i == 1) return ring1;
        else return ring2;
    };
    const int nk = K / kBK;
    auto gload = [&](LoadSlot& sl, int ks) __attribute__((always_inline)) {
        ks = min(ks, nk - 1);
        sl.a0 = *reinterpret_cast<const u32x4*>(aptr[0] + ks * kBK);
        sl.a1 = *reinterpret_cast<const u32x4*>(aptr[1] + ks * kBK);
        const uint8_t* c = bcodes + (int64_t)ks * block_bytes(FMT);
        if constexpr (FMT == MOE_Q8_B32) {
            sl.b0 = reinterpret_cast<const u32x4*>(c)[0];
            sl.b1 = reinterpret_cast<const u32x4*>(c)[1];
        } else if constexpr (FMT == MOE_Q4_B32) {
            sl.b0 = reinterpret_cast<const u32x4*>(c)[0];
        } else {
            const u32x2 v = reinterpret_cast<const u32x2*>(c)[0];
            sl.b0.x = v.x;
            sl.b0.y = v.y;
        }
        sl.s = bscales[ks];
    };
    auto lstore = [&](const LoadSlot& sl, int st) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4*>(&As[st][arow[0] * kLds + aq * 8]) = sl.a0;
        *reinterpret_cast<u32x4*>(&As[st][arow[1] * kLds + aq * 8]) = sl.a1;
        const uint32_t w[8] = {sl.b0.x, sl.b0.y, sl.b0.z, sl.b0.w, sl.b1.x, sl.b1.y, sl.b1.z, sl.b1.w};
        uint32_t o[16];
        dequant16<FMT>(w, (uint16_t)sl.s, o);
        u32x4* dst = reinterpret_cast<u32x4*>(&Bs[st][tid * kLds]);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
    };

    floatx4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int kofs = 8 * (lane / 16);
    // one K step: MFMAs on LDS stage ks & 1, then step ks + 1 from slot (ks + 1) % kPD into the
    // other stage, refill that slot with step ks + 1 + kPD, barrier
    auto kstep = [&](int ks, auto rc) __attribute__((always_inline)) {
        constexpr int next = (decltype(rc)::value + 1) % kPD;
        const int cur = ks & 1;
        half8 a[4], b[8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const half8*>(&As[cur][(wm * 64 + 16 * i + lane % 16) * kLds + kofs]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            b[j] = *reinterpret_cast<const half8*>(&Bs[cur][(wn * 128 + 16 * j + lane % 16) * kLds + kofs]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        lstore(ring(std::integral_constant<int, next>{}), cur ^ 1);
        gload(ring(std::integral_constant<int, next>{}), ks + 1 + kPD);
        __syncthreads();
    };
    static_for<kPD>([&](auto rc) { gload(ring(rc), decltype(rc)::value); });
    lstore(ring0, 0);
    gload(ring0, kPD);
    __syncthreads();
    int kb = 0;
    for (; kb + kPD <= nk; kb += kPD) static_for<kPD>([&](auto rc) { kstep(kb + decltype(rc)::value, rc); });
    static_for<kPD - 1>([&](auto rc) {
        if (kb + decltype(rc)::value < nk) kstep(kb + decltype(rc)::value, rc);
    });

    if constexpr (GATEUP) {
        // tiles j = 2jj (gate) and 2jj + 1 (up) of a wave cover h columns (4 wn + jj) * 16 + [0, 16)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int n = n0 + (4 * wn + jj) * 16 + lane % 16;
                if (n >= N) continue;
                const int np = kperm(n, G);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * 64 + 16 * i + 4 * (lane / 16) + r;
                    if (row >= nrows) continue;
                    const float hv = silu_mul(acc[i][2 * jj][r], acc[i][2 * jj + 1][r]);
                    const int64_t hrow = shared ? (int64_t)Tk + td.row0 + row : (int64_t)base + td.row0 + row;
                    h16[hrow * Imax + np] = (_Float16)hv;
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int m = n0 + wn * 128 + 16 * j + lane % 16;
                if (m >= H) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * 64 + 16 * i + 4 * (lane / 16) + r;
                    if (row >= nrows) continue;
                    if (shared) y_shared[(int64_t)(td.row0 + row) * H + m] = acc[i][j][r];
                    else y_sorted[((int64_t)base + td.row0 + row) * H + m] = acc[i][j][r];
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
                                   const int32_t* perm, float* y_sorted, float* y_shared, const PrefillScratch& s,
                                   hipStream_t st) {
    constexpr int G = perm_group<FMT>();
    const int64_t n16 = (int64_t)T * L.H / 16;
    hipLaunchKernelGGL(k_x_to_f16<G>, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, x, n16, s.x16);
    MOE_LAUNCH_CHECK();
    const int mt = max_tiles(T, L.k, L.E);
    const int nt1 = (L.Imax() + kBN / 2 - 1) / (kBN / 2);
    const int g1 = ((mt * nt1 + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL((k_grouped_gemm<FMT, true>), dim3(g1), dim3(256), 0, st, L, T, s.tiles, s.ntiles, nt1,
                       offsets, perm, s.x16, s.h16, nullptr, nullptr);
    MOE_LAUNCH_CHECK();
    const int nt2 = (L.H + kBN - 1) / kBN;
    const int g2 = ((mt * nt2 + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL((k_grouped_gemm<FMT, false>), dim3(g2), dim3(256), 0, st, L, T, s.tiles, s.ntiles, nt2,
                       offsets, perm, s.h16, nullptr, y_sorted, y_shared);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_prefill_experts(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                  const int32_t* perm, float* y_sorted, float* y_shared, void* scratch,
                                  hipStream_t st) {
    const PrefillScratch s = carve_prefill(L, T, scratch, nullptr);
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, st, offsets, L.E, T, L.k, L.Is > 0 ? 1 : 0,
                       max_tiles(T, L.k, L.E), s.tiles, s.ntiles);
    MOE_LAUNCH_CHECK();
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_prefill_f<MOE_Q8_B32>(L, x, T, offsets, perm, y_sorted, y_shared, s, st);
        case MOE_Q4_B32: return launch_prefill_f<MOE_Q4_B32>(L, x, T, offsets, perm, y_sorted, y_shared, s, st);
        case MOE_Q2_B32: return launch_prefill_f<MOE_Q2_B32>(L, x, T, offsets, perm, y_sorted, y_shared, s, st);
        default: return MOE_ERR_INVALID_ARG;
    }
}

}  // namespace moe
