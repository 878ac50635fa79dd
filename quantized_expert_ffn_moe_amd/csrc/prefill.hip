// Prefill-regime experts: grouped GEMM over expert-sorted row tiles on the gfx950 matrix cores.
//
// Prompt processing on the pages runs in 8K-token chunks with GEMMs and grouped expert kernels
// (648news 07-nano-cuda-moe-qwen38-release, section "speed comparison and accuracy check"). Here:
//   - the pairs of each expert are contiguous after the permutation; a tile list covers every
//     group (the shared expert being one more group of all T tokens) with 128-row tiles and one
//     last tile of 32, 64 or 128 rows for the remainder, so small groups waste little work;
//   - one kernel template, two uses: gate/up (A = x rows gathered through perm; each wave's two
//     32-row weight tiles are gate and up rows of the same h columns, so SwiGLU pairs them in one
//     lane; h is written in fp16 through LDS with full-row stores) and down (A = h rows in sorted
//     order; fp16 outputs leave through LDS as whole-row pieces, fp32 ones straight from the
//     accumulators);
//   - a block is 4 waves over a tile of up to 128 rows x 256 weight rows, two blocks per CU so that
//     one block's prologue, barriers and stores overlap the other's MFMAs; each wave computes all
//     rows of the tile against its own 64 weight rows with v_mfma_f32_32x32x16_f16 (on this chip
//     the 32 x 32 form sustains a far higher rate than 16 x 16 x 32): every A fragment read from
//     LDS feeds 2 MFMAs and every dequantised weight fragment up to 4;
//   - A goes global -> LDS directly (16 bytes per lane, no registers), in a four-stage ring three K
//     steps ahead, each 128-byte row segment XOR-swizzled in 16-byte slots so that the fragment
//     reads of 16 lanes hit distinct banks; one barrier per K step of 64;
//   - weights never touch LDS: each lane loads the codes and scale of one 32-block of its weight
//     row (three steps ahead, in named register slots, through buffer descriptors) and dequantises
//     them straight into its MFMA operand: the code is placed in the mantissa of an fp16 power of
//     two, the offset subtracted (an exact fp16 level) and multiplied by the fp16 scale with packed
//     fp16 arithmetic, i.e. level * scale rounded once to fp16. The pairs come out in an order that
//     permutes K inside each 4-, 8- or 16-element group; x (converted from bf16) and h are stored
//     with the same permutation so the dot products are unchanged;
//   - blocks are mapped so that consecutive row tiles of one expert (which share a weight panel)
//     run on the same XCD and reuse it from that XCD's L2.
#include <utility>

#include "kernels.h"
#include "small_batch.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTM = 128;                   // rows of a full tile
constexpr int kGW = 4;                     // waves per block (two blocks per CU)
constexpr int kGT = kGW * kWave;           // threads per block
constexpr int kStages = 4;                 // A stages in LDS (a ring of four, loads three steps ahead)
constexpr int kStageBytes = kTM * 128;     // one K step (64 fp16) of 128 rows
constexpr int kHS = 128 + 8;               // fp16 per row of the staged h tile (padded)
constexpr int kScaleBytes = 2 * kGW * 1024; // two groups of 4 K steps of scales, 1 KB per wave each
constexpr int kRowExpBytes = kTM * 4;      // the exponent e of each row's activation scale
constexpr int kXcds = 8;
// Word 3 of a raw buffer descriptor (no stride, no swizzle) with the 32-bit data format; loads past
// num_records bytes return zero.
constexpr int kRawBufferWord3 = 0x00020000;

struct TileDesc {
    int group;  // expert id, or E for the shared expert
    int row0;   // first row of the tile inside its group
    int ni;     // 32-row MFMA tiles: 1, 2 or 4
    int pad;
};

// -------------------------------------------------------------------------------- tile list
// Each expert takes floor(count / 128) full tiles and, for a
// remainder, one tile of 32 * ni rows (ni the power of two at or above ceil(rem / 32)). The list is
// expert-major (each expert's tiles side by side, so that they run on one XCD and share its L2;
// experts of every size end up mixed along the list, which balances the XCDs), the shared group
// last; a block scan places the experts and each thread writes its experts' tiles. Offsets are
// clamped to [0, T*k] and the list to tiles_max entries, so that inconsistent offsets cannot move
// any access out of bounds.
__device__ __forceinline__ void group_rows(const int32_t* offsets, int E, int T, int Tk, int g, int& base,
                                           int& count) {
    if (g == E) { base = 0; count = T; return; }
    base = min(max(offsets[g], 0), Tk);
    count = min(max(offsets[g + 1], base), Tk) - base;
}

__host__ __device__ inline int rem_tile_ni(int rem) {
    const int n = (rem + 31) / 32;
    return n <= 1 ? 1 : n <= 2 ? 2 : 4;
}

// Built by one block of NT threads (block 0 of k_x_to_f16, 256 threads, or of k_route_small, 1024):
// thread i takes experts EPT i .. EPT i + EPT - 1, EPT = 1024 / NT (E <= 1024), and writes their
// first kDirectTiles tiles at its place in the block's exclusive scan of the tile counts (one
// barrier); the shared group's tiles follow all routed ones, spread over the block. Only when some
// expert has more tiles (large batches; block-uniform) do all threads then write the rest, list
// slot i by list slot i, each finding its group by a binary search over the scan in LDS, so that
// no thread writes a hot expert's tiles alone. offsets may be global or LDS.
constexpr int kTileThreads = 256;
constexpr int kDirectTiles = 4;
template <int NT>
__device__ __forceinline__ void build_tiles_block(const int32_t* offsets, int E, int T, int k,
                                                  int has_shared, int tiles_max, TileDesc* __restrict__ tiles,
                                                  int32_t* __restrict__ ntiles) {
    constexpr int EPT = 1024 / NT;
    __shared__ int wsum[NT / kWave];
    __shared__ int wbig[NT / kWave];
    __shared__ int part[1024];   // inclusive prefix of the tile counts (large batches only)
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int rows[EPT], sum = 0;
    bool big = false;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = EPT * tid + q;
        int base = 0;
        rows[q] = 0;
        if (e < E) group_rows(offsets, E, T, T * k, e, base, rows[q]);
        const int nt = (rows[q] + kTM - 1) / kTM;
        sum += nt;
        big |= nt > kDirectTiles;
    }
    // block exclusive scan of the per-thread tile counts: wave scans, then the wave totals
    int incl = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += u;
    }
    const bool wave_big = __ballot(big) != 0ull;
    if (lane == kWave - 1) {
        wsum[wave] = incl;
        wbig[wave] = wave_big ? 1 : 0;
    }
    __syncthreads();
    int run = incl - sum, routed = 0, any_big = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        run += w < wave ? wsum[w] : 0;
        routed += wsum[w];
        any_big |= wbig[w];
    }
    // tiles j0, j0 + js, ... below jmax of group g (n rows) at list position first + j
    auto put = [&](int g, int n, int first, int j0, int js, int jmax) __attribute__((always_inline)) {
        const int nf = n / kTM, nt = min((n + kTM - 1) / kTM, jmax);
        for (int j = j0; j < nt; j += js)
            if (first + j < tiles_max) tiles[first + j] = TileDesc{g, j * kTM, j < nf ? kTM / 32 : rem_tile_ni(n % kTM), 0};
    };
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        put(EPT * tid + q, rows[q], run, 0, 1, kDirectTiles);
        run += (rows[q] + kTM - 1) / kTM;
        if (any_big) part[EPT * tid + q] = run;
    }
    const int nsh = has_shared ? T : 0;
    put(E, nsh, routed, tid, NT, 1 << 30);   // the shared group's tiles (T / 128 of them)
    if (tid == 0) *ntiles = min(routed + (nsh + kTM - 1) / kTM, tiles_max);
    if (!any_big) return;
    __syncthreads();
    // slot i of the routed list belongs to the first expert whose inclusive prefix exceeds it
    for (int i = tid; i < min(routed, tiles_max); i += NT) {
        int lo = 0, hi = 1023;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (part[mid] > i) hi = mid;
            else lo = mid + 1;
        }
        const int first = lo > 0 ? part[lo - 1] : 0;
        const int j = i - first;
        if (j < kDirectTiles) continue;
        int base = 0, n = 0;
        group_rows(offsets, E, T, T * k, lo, base, n);
        tiles[i] = TileDesc{lo, j * kTM, j < n / kTM ? kTM / 32 : rem_tile_ni(n % kTM), 0};
    }
}

int max_tiles(int T, int k, int E) { return (T * k) / kTM + T / kTM + E + 2; }

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
// x (bf16) -> fp16 times the token's power-of-two scale 2^e_t (e_t from its largest |x|, see
// common.h; written to xexp[t]), stored with the format's K permutation. One block of 256 threads
// per token: thread i takes the VPT-element pieces i, i + 256, ... of the row (one 16- or 32-byte
// load each, contiguous over the block; a permutation group never crosses a piece), the block
// maximum comes from a wave reduction and four LDS words, then every piece goes out converted.
// Pieces beyond the first two of a thread (rows longer than 512 VPT) are read again from L2.
// Block 0 builds the tile list instead (the two do not depend on each other; the first block is
// dispatched first, so the longer tile build overlaps the conversion).
// One token's row by a block of NT threads (only the first H / VPT of them hold a piece).
template <int G, int VPT, int NT>
__device__ __forceinline__ void x_token_to_f16(const uint16_t* __restrict__ x, int t, int H, _Float16* __restrict__ x16,
                                               int32_t* __restrict__ xexp) {
    static_assert(VPT % G == 0 && VPT % 8 == 0, "a piece holds whole permutation groups");
    constexpr int NV = VPT / 8;   // 16-byte vectors per piece
    __shared__ uint32_t wmax[NT / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int np = H / VPT;
    const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
    auto load = [&](int c, u32x4 (&r)[NV]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NV; ++i) r[i] = row[NV * c + i];
    };
    auto absmax = [&](const u32x4 (&r)[NV]) __attribute__((always_inline)) {
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < NV; ++i) m = max(m, bf16_absmax_bits(make_uint4(r[i].x, r[i].y, r[i].z, r[i].w)));
        return m;
    };
    u32x4 k0[NV], k1[NV];
    load(min(tid, np - 1), k0);
    load(min(tid + NT, np - 1), k1);
    uint32_t m = tid < np ? absmax(k0) : 0u;
    if (tid + NT < np) m = max(m, absmax(k1));
    for (int c = tid + 2 * NT; c < np; c += NT) {
        u32x4 r[NV];
        load(c, r);
        m = max(m, absmax(r));
    }
    m = wave_max_u32(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) m = max(m, wmax[w]);
    const int e = token_exp_from_bits(m);
    if (tid == 0) xexp[t] = e;
    const float sc = pow2f(e);
    half8* dst = reinterpret_cast<half8*>(x16 + (size_t)t * H);
    auto convert = [&](const u32x4 (&r)[NV], int c) __attribute__((always_inline)) {
        _Float16 o[VPT];
#pragma unroll
        for (int i = 0; i < VPT / 2; ++i) {
            const uint32_t w = r[i / 4][i % 4];
            o[kperm(2 * i, G)] = (_Float16)(bf16_lo(w) * sc);
            o[kperm(2 * i + 1, G)] = (_Float16)(bf16_hi(w) * sc);
        }
#pragma unroll
        for (int h = 0; h < NV; ++h) {
            half8 v;
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = o[8 * h + q];
            dst[NV * c + h] = v;
        }
    };
    if (tid < np) convert(k0, tid);
    if (tid + NT < np) convert(k1, tid + NT);
    for (int c = tid + 2 * NT; c < np; c += NT) {
        u32x4 r[NV];
        load(c, r);
        convert(r, c);
    }
}

template <int G, int VPT>
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, int T, int H, _Float16* __restrict__ x16,
                                                  int32_t* __restrict__ xexp, const int32_t* __restrict__ offsets,
                                                  int E, int k, int has_shared, int tiles_max,
                                                  TileDesc* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    if (blockIdx.x == 0) {
        build_tiles_block<kTileThreads>(offsets, E, T, k, has_shared, tiles_max, tiles, ntiles);
        return;
    }
    x_token_to_f16<G, VPT, kTileThreads>(x, (int)blockIdx.x - 1, H, x16, xexp);
}

// -------------------------------------------------------------------------------- small batches
// The routing front end of a small batch as one kernel of 1024-thread blocks, in place of the top-k,
// the permutation, and the x conversion with the tile list (three launches, each a dependent step of
// a few microseconds at these sizes). Block 0: every token's top-k and softmax from the router
// GEMV's logits (wave w takes tokens w, w + 16, ...), the permutation of the pairs (the one-block
// counting sort) and the tile list; blocks 1 .. T: x of one token to fp16 at its activation scale
// (it does not depend on the routing). Same arithmetic and the same outputs as the separate kernels.
constexpr int kSmallThreads = 1024;
template <int KPL, int G, int VPT>
__global__ __launch_bounds__(kSmallThreads) void k_route_small(const float* __restrict__ logits,
                                                               int T, int E, int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ p, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                               const uint16_t* __restrict__ x, int H,
                                                               _Float16* __restrict__ x16, int32_t* __restrict__ xexp,
                                                               int has_shared, int tiles_max,
                                                               TileDesc* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    if (blockIdx.x > 0) {
        x_token_to_f16<G, VPT, kSmallThreads>(x, (int)blockIdx.x - 1, H, x16, xexp);
        return;
    }
    extern __shared__ __attribute__((aligned(16))) char smem[];
    int32_t* ids_s = reinterpret_cast<int32_t*>(smem);                                    // [T k]
    int32_t* offs_s = ids_s + align_up((size_t)T * k, 4);                                 // [E + 1]
    char* perm_lds = reinterpret_cast<char*>(offs_s + align_up((size_t)E + 1, 4));
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    for (int t = wave; t < T; t += kSmallThreads / kWave) {   // uniform per wave
        float lv[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) lv[i] = logits[(int64_t)t * E + min(lane + kWave * i, E - 1)];
        int id;
        float pr;
        topk_wave_regs<KPL>(lv, E, k, id, pr);
        if (lane < k) {
            ids[(size_t)t * k + lane] = id;
            p[(size_t)t * k + lane] = pr;
            ids_s[t * k + lane] = id;
        }
    }
    __syncthreads();
    perm_small_block(ids_s, T, k, E, offsets, perm, inv, perm_lds, offs_s);
    __syncthreads();
    build_tiles_block<kSmallThreads>(offs_s, E, T, k, has_shared, tiles_max, tiles, ntiles);
}

// -------------------------------------------------------------------------------- dequantisation


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
//   Q4: dword d = elements 8d .. 8d+7, pair 4d + j = nibbles (j, j + 4), each read as offset
//       binary n = code + 8 (its top bit flipped). Nibbles at bits 0-3 (j = 0, and j = 2 after a
//       shift by 8) land in the mantissa of 1024.0 (1024 + n, offset 1032); nibbles at bits 4-7
//       (j = 1, 3) in that of 64.0, whose last mantissa bit is worth 1/16 (64 + n, offset 72): one
//       three-input bit operation per pair (mask, flip, exponent), no shifts.
//   Q8: dword d = elements 4d .. 4d+3, pairs 2d (bytes 0, 2) and 2d + 1 (bytes 1, 3): one byte
//       permute puts two codes under the exponent byte of 1024.0 (1024 + b, offset 1152).
//   Q2: dword d = elements 16d .. 16d+15, pair 8d + j = crumbs (j, j + 8) as 2c + 1024, offset
//       1027 = 1024 + 2 * 1.5, times s / 2.
// The exponent patterns come in as register values (DequantConsts) rather than literals: an
// and-or (or a byte permute) can then take its mask as its one literal and run as one instruction.
struct DequantConsts {
    uint32_t m1024;   // 0x64006400: (1024.0, 1024.0)
    uint32_t q4lo;    // 0x64086408: (1024.0, 1024.0) with the sign flips of nibbles 0 and 4
    uint32_t q4hi;    // 0x54805480: (64.0, 64.0) with the sign flips of nibbles 1 and 5
    uint32_t b64;     // 0x64646464: four copies of the exponent byte of 1024.0
};

__device__ __forceinline__ DequantConsts dequant_consts() {
    DequantConsts c;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(c.m1024));
    asm volatile("v_mov_b32 %0, 0x64086408" : "=v"(c.q4lo));
    asm volatile("v_mov_b32 %0, 0x54805480" : "=v"(c.q4hi));
    asm volatile("v_mov_b32 %0, 0x64646464" : "=v"(c.b64));
    return c;
}

template <int FMT, int KK>
__device__ __forceinline__ half8 dequant8(const BlockCodes& b, half2v sv, const DequantConsts& q) {
    uint32_t o[4];
    if constexpr (FMT == MOE_Q4_B32) {
        const half2v off0 = {(_Float16)1032.f, (_Float16)1032.f}, off1 = {(_Float16)72.f, (_Float16)72.f};
        // (u & mask) ^ pattern: the mantissa bits take the nibbles with their top bit flipped (two's
        // complement -> offset binary), every other bit the exponent pattern
        const uint32_t u = dword_of(b, KK), v = u >> 8;
        o[0] = h2bits((bits2h((u & 0x000F000Fu) ^ q.q4lo) - off0) * sv);
        o[1] = h2bits((bits2h((u & 0x00F000F0u) ^ q.q4hi) - off1) * sv);
        o[2] = h2bits((bits2h((v & 0x000F000Fu) ^ q.q4lo) - off0) * sv);
        o[3] = h2bits((bits2h((v & 0x00F000F0u) ^ q.q4hi) - off1) * sv);
    } else if constexpr (FMT == MOE_Q8_B32) {
        const half2v off = {(_Float16)1152.f, (_Float16)1152.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t u = dword_of(b, 2 * KK + h) ^ 0x80808080u;
            // bytes {u0, 0x64, u2, 0x64} and {u1, 0x64, u3, 0x64}
            o[2 * h] = h2bits((bits2h(__builtin_amdgcn_perm(q.b64, u, 0x04020400u)) - off) * sv);
            o[2 * h + 1] = h2bits((bits2h(__builtin_amdgcn_perm(q.b64, u, 0x04030401u)) - off) * sv);
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
            o[jj] = h2bits((bits2h((t & 0x00060006u) | q.m1024) - off) * s2);
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

// Weight operand of one K step for one lane: the codes and the scale of its 32-block. Plain
// members only: a slot must never be indexed at run time, or it would leave the registers.
struct BSlot {
    BlockCodes b;
    uint32_t sc;
};

template <int FMT> constexpr int code_loads() { return FMT == MOE_Q8_B32 ? 2 : 1; }

// Wait until at most VM vector-memory loads of this wave are in flight (and its LDS operations are
// done), then meet the other waves. Written with the wait visible to the compiler and without a
// memory fence, which would make the barrier wait for every load in flight; the empty asm
// statements keep memory operations from moving across it.
template <int VM> __device__ __forceinline__ void step_barrier() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One tile of 32 * NI rows against the block's 256 weight rows (gate/up: 128 h columns). SD: the
// scales come as groups of four K steps straight into LDS (the scale rows are 16-byte aligned).
// Activation scales (common.h): every A row carries the exponent e of its token's scale 2^e, read
// from rexp (gate/up: by token; down: by h row, as the gate/up epilogue wrote it to hexp). Gate/up
// turns the scaled accumulators into h * 2^(2e); down multiplies its outputs by 2^(-2e) when UNSC
// (fp32 rows, and the fp16 rows of moe_experts_prefill_f16), else leaves them at that scale (the
// fused layer's internal fp16 rows, unscaled by its combine). fp16 values saturate at +-65504.
template <int FMT, bool GATEUP, typename YT, int NI, bool SD, bool UNSC>
__device__ __forceinline__ void gemm_tile(const LayerView& L, int T, const TileDesc& td, int ntile,
                                          const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                                          const _Float16* __restrict__ asrc, const int32_t* __restrict__ rexp,
                                          _Float16* __restrict__ h16, int32_t* __restrict__ hexp,
                                          YT* __restrict__ y_sorted, YT* __restrict__ y_shared, uint8_t* smem) {
    constexpr int G = perm_group<FMT>();
    constexpr int BB = FMT == MOE_Q8_B32 ? 32 : FMT == MOE_Q4_B32 ? 16 : 8;   // bytes per block
    constexpr int QW = NI;                         // 1 KB (8-row) direct loads per wave and step
    // vector-memory instructions per step (with SD, one more in every fourth step's batch)
    constexpr int BATCH = QW + 2 * code_loads<FMT>() + (SD ? 0 : 2);

    const bool shared = td.group == L.E;
    const int H = L.H, Imax = L.Imax();
    int N, n0, K;
    if constexpr (GATEUP) {
        N = shared ? L.Is : L.I;          // h columns of this group
        n0 = ntile * 128;
        K = H;
    } else {
        N = H;
        n0 = ntile * 256;
        K = shared ? L.Is : L.I;
    }
    if (n0 >= N) return;
    const int Tk = T * L.k;
    int base, count;
    group_rows(offsets, L.E, T, Tk, td.group, base, count);
    const int nrows = min(NI * 32, count - td.row0);
    if (nrows <= 0) return;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int frow = lane % 32, g = lane / 32;
    const int nb = K / 32;                    // scale blocks along K
    const int nsteps = (nb + 1) / 2;

    // A: stage row r (0 .. 32 NI - 1) sits at r * 128 bytes, its 16-byte K chunk c in slot
    // c ^ ((r >> 1) & 7). Wave load u fills rows 8 q .. 8 q + 7 (q = wave + 4 u); lane l writes
    // slot l % 8 of row 8 q + l / 8, so it fetches the chunk that belongs there. Rows past the
    // tile are clamped to a valid row: they only feed output rows that are never stored.
    // The exponents of the rows' activation scales are loaded here and written to LDS (row r at
    // rexp_s[r]) after the prologue's wait, which they precede in the load order.
    constexpr bool kRowExp = GATEUP || UNSC;
    int* rexp_s = reinterpret_cast<int*>(smem + kStages * kStageBytes + kScaleBytes);
    const _Float16* arow[QW];
    int ach[QW];
    int rexp_v[QW];
#pragma unroll
    for (int u = 0; u < QW; ++u) {
        const int q = wave + kGW * u;
        const int r = 8 * q + lane / 8;
        ach[u] = 8 * ((lane & 7) ^ ((r >> 1) & 7));
        const int pos = td.row0 + min(r, nrows - 1);
        if constexpr (GATEUP) {
            const int qq = shared ? pos * L.k : perm[base + pos];
            const int tok = (unsigned)qq < (unsigned)Tk ? qq / L.k : 0;
            arow[u] = asrc + (size_t)tok * H;
            rexp_v[u] = rexp[tok];
        } else {
            const int64_t hrow = shared ? (int64_t)Tk + pos : (int64_t)base + pos;
            arow[u] = asrc + (size_t)hrow * Imax;
            if constexpr (kRowExp) rexp_v[u] = rexp[hrow];
        }
    }
    // fragment of lane (frow, g) for K sub-step kk: row 32 i + frow, chunk 4 g + kk
    int aoff[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) aoff[kk] = frow * 128 + 16 * ((4 * g + kk) ^ ((frow >> 1) & 7));

    // B: wave w owns weight rows 64 w .. 64 w + 63 of the tile as two 32-row MFMA tiles; lane
    // (frow, g) loads, for each, block 2 s + g of its row at step s. Gate/up: tile 0 = gate rows,
    // tile 1 = up rows of the same h columns n0 + 32 w + [0, 32); down: output columns
    // n0 + 64 w + [0, 64).
    // Each matrix (one expert's gate, up or down, or the shared expert's) is at most
    // 4096 x 16384 bytes of codes, so 32-bit lane offsets suffice.
    const uint8_t* bmat[2];
    const uint8_t* smat[2];
    const int64_t rb = (int64_t)nb * BB;
    int64_t mrows;   // rows of the matrices
    int wrow[2];     // this lane's row in each
    if constexpr (GATEUP) {
        mrows = N;
        const int n = min(n0 + 32 * wave + frow, N - 1);
        wrow[0] = wrow[1] = n;
        if (shared) {
            bmat[0] = L.sg_codes; bmat[1] = L.su_codes;
            smat[0] = reinterpret_cast<const uint8_t*>(L.sg_scales);
            smat[1] = reinterpret_cast<const uint8_t*>(L.su_scales);
        } else {
            const int64_t e = td.group;
            bmat[0] = L.g_codes + e * N * rb; bmat[1] = L.u_codes + e * N * rb;
            smat[0] = reinterpret_cast<const uint8_t*>(L.g_scales + e * N * nb);
            smat[1] = reinterpret_cast<const uint8_t*>(L.u_scales + e * N * nb);
        }
    } else {
        mrows = H;
#pragma unroll
        for (int j = 0; j < 2; ++j) wrow[j] = min(n0 + 64 * wave + 32 * j + frow, H - 1);
        if (shared) {
            bmat[0] = bmat[1] = L.sd_codes;
            smat[0] = smat[1] = reinterpret_cast<const uint8_t*>(L.sd_scales);
        } else {
            const int64_t e = td.group;
            bmat[0] = bmat[1] = L.d_codes + e * H * rb;
            smat[0] = smat[1] = reinterpret_cast<const uint8_t*>(L.d_scales + e * H * nb);
        }
    }
    int64_t bbytes = mrows * rb;
    const int64_t sbytes = mrows * nb * 2;
    // lane offsets of block g of row wrow (tile 0; tile 1 adds its row difference), and the code
    // bytes the buffer base advances per K step
    int bvo0 = (int)(wrow[0] * rb) + g * BB, bdv = (int)((wrow[1] - wrow[0]) * rb), cstep = 2 * BB;
    // SD: where each lane's 16 bytes of scales start, and how far they move per group of 4 steps
    const char* sgsrc = nullptr;
    int sgstep = 16;
    const int svo0 = (wrow[0] * nb + g) * 2, sdv = (wrow[1] - wrow[0]) * nb * 2;
    if (L.pk) {
        // the packed copy: the piece of (32-row group, step) is 64 BB bytes and lane (frow, g) reads
        // BB bytes at BB (frow + 32 g) of it, so that each load is one contiguous run; a group past
        // the matrix reads its last group (those rows are never stored)
        const PackedOffsets po = packed_offsets(L);
        const int ngrp = (int)((mrows + 31) / 32);
        int grp[2];
        if constexpr (GATEUP) {
            grp[0] = grp[1] = min((n0 + 32 * wave) / 32, ngrp - 1);
            const int64_t e = td.group;
            bmat[0] = L.pk + (shared ? po.sh_gate : po.gate + e * po.pg);
            bmat[1] = L.pk + (shared ? po.sh_up : po.up + e * po.pg);
            bbytes = shared ? po.psg : po.pg;
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) grp[j] = min((n0 + 64 * wave + 32 * j) / 32, ngrp - 1);
            bmat[0] = bmat[1] = L.pk + (shared ? po.sh_down : po.down + (int64_t)td.group * po.pd);
            bbytes = shared ? po.psd : po.pd;
        }
        cstep = 64 * BB;
        bvo0 = grp[0] * nsteps * cstep + BB * (frow + 32 * g);
        bdv = (grp[1] - grp[0]) * nsteps * cstep;
        if constexpr (SD) {
            // packed scales: the piece of (32-row group, 4 steps) is 512 bytes, row r at 16 r
            const int j = lane / 32;
            int64_t sb;
            if constexpr (GATEUP) sb = shared ? (j ? po.s_sh_up : po.s_sh_gate) : (j ? po.s_up : po.s_gate) + (int64_t)td.group * po.qg;
            else sb = shared ? po.s_sh_down : po.s_down + (int64_t)td.group * po.qd;
            sgsrc = reinterpret_cast<const char*>(L.pk) + sb + (int64_t)grp[j] * (nb / 8) * 512 + 16 * (lane % 32);
            sgstep = 512;
        }
    }
    // SD: lane l of wave w loads 16 bytes (the 8 scales of 4 K steps) of row wrow[l / 32] of tile
    // l / 32 for rows 32 w + l % 32 (from the packed copy when there is one); they land at byte
    // 16 l of the wave's 1 KB of the group's buffer
    if constexpr (SD) {
        const int j = lane / 32;
        if (!sgsrc) sgsrc = reinterpret_cast<const char*>(smat[j]) + (int64_t)wrow[j] * nb * 2;
    }
    uint8_t* sbuf = smem + kStages * kStageBytes;

    BSlot slot0[2], slot1[2], slot2[2], slot3[2];   // steps s .. s + 3 live at a time
    auto slot = [&](auto sc) __attribute__((always_inline)) -> BSlot(&)[2] {
        constexpr int v = decltype(sc)::value;
        if constexpr (v == 0) return slot0;
        else if constexpr (v == 1) return slot1;
        else if constexpr (v == 2) return slot2;
        else return slot3;
    };
    // A source of load u at step t: its row + min(128 t + 2 ach, 2 (K - 8)) bytes
    const char* abase[QW];
#pragma unroll
    for (int u = 0; u < QW; ++u) abase[u] = reinterpret_cast<const char*>(arow[u]);
    const int klim = 2 * (K - 8);
    // loads of step t (clamped: steps past the end reload the last one, unused) into B slots and
    // an A stage. Weights come through buffer descriptors whose base moves with the step, so the
    // lane offsets stay fixed; a block past the end of the matrix reads as zero (bounds-checked).
    // A chunk past K (the second half of the last step when K % 64 == 32) reloads the row's last
    // chunk instead (its weights are zero, see below).
    // TAIL: the step may lie past the end of K. Such a step issues no direct-to-LDS load at all: the
    // stages and the scale buffers are reused by the epilogue, and a transfer still landing there
    // after the final wait would overwrite the staged outputs (such late writes were observed). Its
    // register loads still go out (clamped, unused), so every step issues a known number of loads.
    auto issue = [&](BSlot (&sl)[2], int t, int stage, auto group_start, auto tail) __attribute__((always_inline)) {
        const bool live = !decltype(tail)::value || t < nsteps;
        t = min(t, nsteps - 1);
        uint8_t* st = smem + stage * kStageBytes + wave * 1024;
        if (live) {
#pragma unroll
            for (int u = 0; u < QW; ++u)
                __builtin_amdgcn_global_load_lds(abase[u] + min(128 * t + 2 * ach[u], klim),
                                                 (lds_void*)(st + u * kGW * 1024), 16, 0, 0);
            // the scales of steps t .. t + 3 (blocks 2 t .. 2 t + 7), issued by the steps that start a
            // group of four (known at compile time)
            if constexpr (SD && decltype(group_start)::value)
                __builtin_amdgcn_global_load_lds(sgsrc + sgstep * (t >> 2),
                                                 (lds_void*)(sbuf + ((t >> 2) & 1) * (kGW * 1024) + wave * 1024), 16,
                                                 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cofs = cstep * t, sofs = 4 * t;
            const int bvo = bvo0 + j * bdv, svo = svo0 + j * sdv;
            const __amdgpu_buffer_rsrc_t rc =
                __builtin_amdgcn_make_buffer_rsrc((void*)(bmat[j] + cofs), (short)0, (int)(bbytes - cofs), kRawBufferWord3);
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(smat[j] + sofs), (short)0, (int)(sbytes - sofs), kRawBufferWord3);
            if constexpr (FMT == MOE_Q8_B32) {
                sl[j].b.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, bvo, 0, 0));
                sl[j].b.c1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, bvo + 16, 0, 0));
            } else if constexpr (FMT == MOE_Q4_B32) {
                sl[j].b.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, bvo, 0, 0));
            } else {
                const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, bvo, 0, 0));
                sl[j].b.c0.x = v.x;
                sl[j].b.c0.y = v.y;
            }
            if constexpr (!SD) sl[j].sc = __builtin_amdgcn_raw_buffer_load_b16(rs, svo, 0, 0);
        }
    };

    const DequantConsts dq = dequant_consts();
    floatx16 acc[NI][2];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Scales of step t as an fp16 pair per weight tile (zero for a block past K, which then
    // contributes nothing): from the LDS group buffer (t / 4) % 2, element 2 (t % 4) + g of tile
    // j's 16 bytes, or from the B slot itself.
    auto scales = [&](int t, const BSlot (&sl)[2], half2v& v0, half2v& v1) __attribute__((always_inline)) {
        const bool blive = 2 * t + g < nb;
        uint16_t sc0, sc1;
        if constexpr (SD) {
            const uint16_t* sb = reinterpret_cast<const uint16_t*>(sbuf + ((t >> 2) & 1) * (kGW * 1024) + wave * 1024);
            sc0 = sb[frow * 8 + 2 * (t & 3) + g];
            sc1 = sb[(32 + frow) * 8 + 2 * (t & 3) + g];
        } else {
            sc0 = (uint16_t)sl[0].sc;
            sc1 = (uint16_t)sl[1].sc;
        }
        const _Float16 s0 = blive ? __builtin_bit_cast(_Float16, sc0) : (_Float16)0.f;
        const _Float16 s1 = blive ? __builtin_bit_cast(_Float16, sc1) : (_Float16)0.f;
        v0 = half2v{s0, s0};
        v1 = half2v{s1, s1};
    };
    auto frag = [&](const uint8_t* st, auto kc, half8 (&f)[NI]) __attribute__((always_inline)) {
        constexpr int kk = decltype(kc)::value;
#pragma unroll
        for (int i = 0; i < NI; ++i) f[i] = *reinterpret_cast<const half8*>(st + aoff[kk] + i * 4096);
    };
    auto deq = [&](const BSlot (&sl)[2], auto kc, half2v v0, half2v v1, half8 (&b)[2]) __attribute__((always_inline)) {
        constexpr int kk = decltype(kc)::value;
        b[0] = dequant8<FMT, kk>(sl[0].b, v0, dq);
        b[1] = dequant8<FMT, kk>(sl[1].b, v1, dq);
    };
    // A fragments and dequantised weights of the next sub-step are prepared while the MFMAs of the
    // current one run (two named sets of each, so that nothing is indexed at run time); scheduling
    // groups interleave each MFMA with a share of that preparation, so that a wave keeps issuing
    // MFMAs back to back. The operands of sub-step 0 of a step are prepared during sub-step 3 of
    // the step before, so no step starts with an exposed LDS read or dequantisation.
    half8 fa[NI], fb[NI];
    half8 ba[2], bb[2];
    half2v svc0, svc1;   // scales of the current step

    // Step s. Sub-steps 0-2 run on operands prepared one sub-step ahead. Before sub-step 3 the wave
    // waits for the loads of step s + 1 (everything but those of steps s + 2 and s + 3) and for
    // its LDS reads, then meets the other waves: stage s % 4 and the B slot of step s are then
    // free, and step s + 4 is loaded into them while sub-step 3 runs and step s + 1's first
    // operands are prepared. The barrier is written out so that no memory fence makes it wait for
    // the loads still in flight.
    // TAIL: one of the last steps, where steps s + 2 .. s + 4 may lie past the end (the steady-state
    // loop runs only steps whose loads are all live).
    auto kstep = [&](int s, auto sc, auto tail) __attribute__((always_inline)) {
        constexpr int SL = decltype(sc)::value;   // = s % 4
        constexpr bool TAIL = decltype(tail)::value;
        constexpr int SN = (SL + 1) % 4;
        constexpr bool kIssueGroup = SD && SL == 0;                  // step s + 4 starts a scale group
        constexpr int kInFlightGroups = (SD && (SL == 1 || SL == 2)) ? 1 : 0;   // s + 2 or s + 3 does
        const BSlot(&cur)[2] = slot(sc);
        const BSlot(&nxt)[2] = slot(std::integral_constant<int, SN>{});
        const uint8_t* st = smem + SL * kStageBytes;
        const uint8_t* stn = smem + SN * kStageBytes;
        half2v svn0, svn1;
        static_for<4>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            half8 (&cur_a)[NI] = (kk % 2 == 0) ? fa : fb;
            half8 (&nxt_a)[NI] = (kk % 2 == 0) ? fb : fa;
            half8 (&cur_b)[2] = (kk % 2 == 0) ? ba : bb;
            half8 (&nxt_b)[2] = (kk % 2 == 0) ? bb : ba;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kk < 3) {
                frag(st, std::integral_constant<int, kk + 1>{}, nxt_a);
                deq(cur, std::integral_constant<int, kk + 1>{}, svc0, svc1, nxt_b);
            } else {
                // leave in flight exactly the loads of steps s + 2 and s + 3: a full batch (and a scale
                // group) for a live step, only the register loads for a step past the end
                if constexpr (!TAIL) {
                    step_barrier<2 * BATCH + kInFlightGroups>();
                } else {
                    constexpr int kDead = BATCH - QW;                          // loads of a dead step
                    constexpr int kG2 = (SD && SL == 2) ? 1 : 0;               // s + 2 starts a group
                    if (s + 3 < nsteps) step_barrier<2 * BATCH + kInFlightGroups>();
                    else if (s + 2 < nsteps) step_barrier<BATCH + kG2 + kDead>();
                    else step_barrier<2 * kDead>();
                }
                issue(slot(sc), s + 4, SL, std::integral_constant<bool, kIssueGroup>{}, tail);
                scales(s + 1, nxt, svn0, svn1);
                frag(stn, std::integral_constant<int, 0>{}, nxt_a);
                deq(nxt, std::integral_constant<int, 0>{}, svn0, svn1, nxt_b);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur_a[i], cur_b[0], acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur_a[i], cur_b[1], acc[i][1], 0, 0, 0);
            }
            // 2 NI MFMAs; the NI LDS reads of the next sub-step behind the first NI of them (their
            // latency then hides behind the rest), about 26 VALU spread over all of them
            constexpr int kV = (28 + 2 * NI - 1) / (2 * NI);
            static_for<2 * NI>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
                if constexpr (m < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);    // VALU
            });
        });
        __builtin_amdgcn_sched_barrier(0);
        svc0 = svn0;
        svc1 = svn1;
    };

    // prologue: steps 0-3 in flight, then step 0's first operands
    const std::integral_constant<bool, true> kTail{};
    const std::integral_constant<bool, false> kSteady{};
    issue(slot0, 0, 0, std::integral_constant<bool, SD>{}, kTail);
    issue(slot1, 1, 1, std::integral_constant<bool, false>{}, kTail);
    issue(slot2, 2, 2, std::integral_constant<bool, false>{}, kTail);
    issue(slot3, 3, 3, std::integral_constant<bool, false>{}, kTail);
    if (nsteps >= 4) step_barrier<3 * BATCH>();
    else step_barrier<0>();
    if constexpr (kRowExp) {
        if ((lane & 7) == 0) {
#pragma unroll
            for (int u = 0; u < QW; ++u) rexp_s[8 * (wave + kGW * u) + lane / 8] = rexp_v[u];
        }
    }
    scales(0, slot0, svc0, svc1);
    frag(smem, std::integral_constant<int, 0>{}, fa);
    deq(slot0, std::integral_constant<int, 0>{}, svc0, svc1, ba);
    int s = 0;
    for (; s + 8 <= nsteps; s += 4) {   // every load these steps issue is live
        kstep(s, std::integral_constant<int, 0>{}, kSteady);
        kstep(s + 1, std::integral_constant<int, 1>{}, kSteady);
        kstep(s + 2, std::integral_constant<int, 2>{}, kSteady);
        kstep(s + 3, std::integral_constant<int, 3>{}, kSteady);
    }
    if (s + 4 <= nsteps) {
        kstep(s, std::integral_constant<int, 0>{}, kTail);
        kstep(s + 1, std::integral_constant<int, 1>{}, kTail);
        kstep(s + 2, std::integral_constant<int, 2>{}, kTail);
        kstep(s + 3, std::integral_constant<int, 3>{}, kTail);
        s += 4;
    }
    if (s < nsteps) kstep(s, std::integral_constant<int, 0>{}, kTail);
    if (s + 1 < nsteps) kstep(s + 1, std::integral_constant<int, 1>{}, kTail);
    if (s + 2 < nsteps) kstep(s + 2, std::integral_constant<int, 2>{}, kTail);
    // every direct load has landed and every wave is done with the stages: LDS is free
    step_barrier<0>();

    const int rq = 4 * g;
    if constexpr (GATEUP) {
        // SwiGLU of (gate, up) = (tile 0, tile 1) in every lane; h goes to an LDS tile of the
        // block's 128 columns, then out in 16-byte pieces of whole rows
        _Float16* hs = reinterpret_cast<_Float16*>(smem);
        const int pc = kperm(32 * wave + frow, G);   // n0 is a multiple of 128, so of G
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int4 ev = *reinterpret_cast<const int4*>(rexp_s + 32 * i + 8 * r4 + rq);
                const int ee[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
                for (int r1 = 0; r1 < 4; ++r1) {
                    const int r = 4 * r4 + r1;
                    const int row = 32 * i + 8 * r4 + rq + r1;
                    hs[row * kHS + pc] =
                        (_Float16)sat_f16(silu_mul_scaled_fast(acc[i][0][r], acc[i][1][r], pow2f(-ee[r1])));
                }
            }
        // the h rows' exponents for the down GEMM (written once, by the first column tile)
        if (ntile == 0) {
            for (int row = tid; row < nrows; row += kGT) {
                const int64_t hrow = shared ? (int64_t)Tk + td.row0 + row : (int64_t)base + td.row0 + row;
                hexp[hrow] = rexp_s[row];
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 2 * NI; ++it) {
            const int idx = tid + kGT * it;      // NI * 32 rows x 16 pieces
            const int row = idx / 16, ch = idx % 16;
            const int col = n0 + 8 * ch;
            if (row < nrows && col < N) {
                const int64_t hrow = shared ? (int64_t)Tk + td.row0 + row : (int64_t)base + td.row0 + row;
                *reinterpret_cast<u32x4*>(h16 + hrow * Imax + col) =
                    *reinterpret_cast<const u32x4*>(hs + row * kHS + 8 * ch);
            }
        }
    } else if constexpr (sizeof(YT) == 2) {
        // fp16 rows through LDS, one 32-column tile per wave at a time: pass j stages columns
        // n0 + 64 w + 32 j + [0, 32) of every wave (staged column 32 w + frow), then whole rows
        // leave in 16-byte pieces
        _Float16* ys = reinterpret_cast<_Float16*>(smem);
        YT* ybase = shared ? y_shared + (int64_t)td.row0 * H : y_sorted + ((int64_t)base + td.row0) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (j) __syncthreads();
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    int ee[4] = {0, 0, 0, 0};
                    if constexpr (UNSC) {
                        const int4 ev = *reinterpret_cast<const int4*>(rexp_s + 32 * i + 8 * r4 + rq);
                        ee[0] = ev.x; ee[1] = ev.y; ee[2] = ev.z; ee[3] = ev.w;
                    }
#pragma unroll
                    for (int r1 = 0; r1 < 4; ++r1) {
                        const int row = 32 * i + 8 * r4 + rq + r1;
                        const float v = acc[i][j][4 * r4 + r1];
                        ys[row * kHS + 32 * wave + frow] = (_Float16)sat_f16(UNSC ? v * pow2f(-2 * ee[r1]) : v);
                    }
                }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < 2 * NI; ++it) {
                const int idx = tid + kGT * it;      // NI * 32 rows x 16 pieces
                const int row = idx / 16, ch = idx % 16;
                const int col = n0 + 64 * (ch / 4) + 32 * j + 8 * (ch % 4);
                if (row < nrows && col < H)
                    *reinterpret_cast<u32x4*>(ybase + (int64_t)row * H + col) =
                        *reinterpret_cast<const u32x4*>(ys + row * kHS + 8 * ch);
            }
        }
    } else {
        // fp32 rows straight from the accumulators: 32 lanes write one 128-byte row segment
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = n0 + 64 * wave + 32 * j + frow;
            if (m >= H) continue;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int4 ev = *reinterpret_cast<const int4*>(rexp_s + 32 * i + 8 * r4 + rq);
                    const int ee[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
                    for (int r1 = 0; r1 < 4; ++r1) {
                        const int row = 32 * i + 8 * r4 + rq + r1;
                        if (row >= nrows) continue;
                        const float v = acc[i][j][4 * r4 + r1] * pow2f(-2 * ee[r1]);
                        if (shared) y_shared[(int64_t)(td.row0 + row) * H + m] = (YT)v;
                        else y_sorted[((int64_t)base + td.row0 + row) * H + m] = (YT)v;
                    }
                }
        }
    }
}

// YT: type of the down outputs (float, or _Float16); UNSC: down outputs at the true scale (see
// gemm_tile).
template <int FMT, bool GATEUP, typename YT = float, bool UNSC = true>
__global__ __launch_bounds__(kGT, 2) void k_grouped_gemm(LayerView L, int T, const TileDesc* __restrict__ tiles,
                                                         const int32_t* __restrict__ ntiles, int n_ntile,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ perm,
                                                         const _Float16* __restrict__ asrc,
                                                         const int32_t* __restrict__ rexp, _Float16* __restrict__ h16,
                                                         int32_t* __restrict__ hexp, YT* __restrict__ y_sorted,
                                                         YT* __restrict__ y_shared) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes + kScaleBytes + kRowExpBytes];
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
    // scale rows are 16-byte aligned when the scale count per row is a multiple of 8
    const int K = GATEUP ? L.H : (td.group == L.E ? L.Is : L.I);
    const bool sd = (K / 32) % 8 == 0;
#define MOE_GEMM_TILE(NI_, SD_)                                                                              \
    gemm_tile<FMT, GATEUP, YT, NI_, SD_, UNSC>(L, T, td, ntile, offsets, perm, asrc, rexp, h16, hexp, y_sorted, \
                                               y_shared, smem)
    switch (td.ni) {
        case 4: if (sd) MOE_GEMM_TILE(4, true); else MOE_GEMM_TILE(4, false); break;
        case 2: if (sd) MOE_GEMM_TILE(2, true); else MOE_GEMM_TILE(2, false); break;
        default: if (sd) MOE_GEMM_TILE(1, true); else MOE_GEMM_TILE(1, false); break;
    }
#undef MOE_GEMM_TILE
}

// -------------------------------------------------------------------------------- packed codes

// One thread per 4 bytes of the packed copy of `count` matrices of N x K whose row-major codes
// start at src (one after another): byte o of a matrix's copy lies in piece o / (64 BB) = (group r,
// step s); its slot l = (o % (64 BB)) / BB holds block 2s + l / 32 of row 32 r + l % 32, zero past
// the matrix's rows or the row's blocks.
__global__ __launch_bounds__(256) void k_pack_codes(const uint8_t* __restrict__ src, int N, int K, int fmt,
                                                    int64_t pmat, int count, uint8_t* __restrict__ dst) {
    const int64_t units = pmat / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units * count) return;
    const int64_t m = i / units, o = (i % units) * 4;
    const int BB = block_bytes(fmt);
    const int nsteps = (K + 63) / 64, nb = K / 32;
    const int64_t rb = row_bytes(fmt, K);
    const int64_t c = o / (64 * BB);
    const int ob = (int)(o % (64 * BB));
    const int r = (int)(c / nsteps), st = (int)(c % nsteps);
    const int l = ob / BB, bo = ob % BB;
    const int row = 32 * r + l % 32, blk = 2 * st + l / 32;
    uint32_t v = 0u;
    if (row < N && blk < nb)
        v = *reinterpret_cast<const uint32_t*>(src + (m * N + row) * rb + (int64_t)blk * BB + bo);
    *reinterpret_cast<uint32_t*>(dst + m * pmat + o) = v;
}

// One thread per 16 bytes (8 scales) of the packed scales of `count` matrices of N rows and nb
// blocks (row-major [N][nb] each, one after another): piece (group r, blocks 8q .. 8q + 7) holds
// row 32 r + i at 16 i; zero past the rows or blocks.
__global__ __launch_bounds__(256) void k_pack_scales(const uint16_t* __restrict__ src, int N, int nb, int64_t pmat,
                                                     int count, uint8_t* __restrict__ dst) {
    const int64_t units = pmat / 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units * count) return;
    const int64_t m = i / units, u = i % units;
    const int nq = (nb + 7) / 8;
    const int64_t piece = u / 32;
    const int rr = (int)(u % 32);
    const int r = (int)(piece / nq), q = (int)(piece % nq);
    const int row = 32 * r + rr;
    uint16_t v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int blk = 8 * q + b;
        v[b] = (row < N && blk < nb) ? src[(m * N + row) * nb + blk] : (uint16_t)0;
    }
    uint4 o;
    o.x = v[0] | ((uint32_t)v[1] << 16);
    o.y = v[2] | ((uint32_t)v[3] << 16);
    o.z = v[4] | ((uint32_t)v[5] << 16);
    o.w = v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<uint4*>(dst + m * pmat + 16 * u) = o;
}

moe_status launch_pack_codes(const LayerView& L, uint8_t* dst, hipStream_t s) {
    const PackedOffsets po = packed_offsets(L);
    auto pack = [&](const uint8_t* src, int N, int K, int64_t pmat, int count, int64_t at) -> moe_status {
        const int64_t n = pmat / 4 * count;
        hipLaunchKernelGGL(k_pack_codes, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, N, K, L.fmt, pmat,
                           count, dst + at);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    };
    auto pack_s = [&](const uint16_t* src, int N, int K, int64_t pmat, int count, int64_t at) -> moe_status {
        const int64_t n = pmat / 16 * count;
        hipLaunchKernelGGL(k_pack_scales, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, N, K / 32, pmat,
                           count, dst + at);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    };
    moe_status st = pack(L.g_codes, L.I, L.H, po.pg, L.E, po.gate);
    if (st == MOE_OK) st = pack(L.u_codes, L.I, L.H, po.pg, L.E, po.up);
    if (st == MOE_OK) st = pack(L.d_codes, L.H, L.I, po.pd, L.E, po.down);
    if (st == MOE_OK) st = pack_s(L.g_scales, L.I, L.H, po.qg, L.E, po.s_gate);
    if (st == MOE_OK) st = pack_s(L.u_scales, L.I, L.H, po.qg, L.E, po.s_up);
    if (st == MOE_OK) st = pack_s(L.d_scales, L.H, L.I, po.qd, L.E, po.s_down);
    if (st == MOE_OK && L.Is > 0) {
        st = pack(L.sg_codes, L.Is, L.H, po.psg, 1, po.sh_gate);
        if (st == MOE_OK) st = pack(L.su_codes, L.Is, L.H, po.psg, 1, po.sh_up);
        if (st == MOE_OK) st = pack(L.sd_codes, L.H, L.Is, po.psd, 1, po.sh_down);
        if (st == MOE_OK) st = pack_s(L.sg_scales, L.Is, L.H, po.qsg, 1, po.s_sh_gate);
        if (st == MOE_OK) st = pack_s(L.su_scales, L.Is, L.H, po.qsg, 1, po.s_sh_up);
        if (st == MOE_OK) st = pack_s(L.sd_scales, L.H, L.Is, po.qsd, 1, po.s_sh_down);
    }
    return st;
}

// -------------------------------------------------------------------------------- launch

struct PrefillScratch {
    TileDesc* tiles;
    int32_t* ntiles;
    _Float16* x16;
    _Float16* h16;
    int32_t* xexp;   // [T]: e of each token's activation scale
    int32_t* hexp;   // [T*k + T]: e of each h row's token
};

static PrefillScratch carve_prefill(const LayerView& L, int T, void* base, size_t* bytes) {
    Carve c(base);
    PrefillScratch s;
    s.tiles = c.take<TileDesc>((size_t)max_tiles(T, L.k, L.E));
    s.ntiles = c.take<int32_t>(1);
    s.x16 = c.take<_Float16>((size_t)T * L.H);
    s.h16 = c.take<_Float16>((size_t)(T * L.k + T) * L.Imax());
    s.xexp = c.take<int32_t>((size_t)T);
    s.hexp = c.take<int32_t>((size_t)T * L.k + T);
    if (bytes) *bytes = c.bytes();
    return s;
}

size_t prefill_scratch_bytes(const LayerView& L, int T) {
    size_t b = 0;
    carve_prefill(L, T, nullptr, &b);
    return b;
}

const int32_t* prefill_token_exps(const LayerView& L, int T, void* scratch) {
    return carve_prefill(L, T, scratch, nullptr).xexp;
}

template <int FMT>
static moe_status launch_prefill_f(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                   const int32_t* perm, void* y_sorted, void* y_shared, PrefillOut mode,
                                   const PrefillScratch& s, bool prepared, hipStream_t st) {
    constexpr int G = perm_group<FMT>();
    constexpr int VPT = G <= 8 ? 8 : 16;
    if (!prepared) {
        hipLaunchKernelGGL((k_x_to_f16<G, VPT>), dim3((unsigned)(T + 1)), dim3(kTileThreads), 0, st, x, T, L.H, s.x16,
                           s.xexp, offsets, L.E, L.k, L.Is > 0 ? 1 : 0, max_tiles(T, L.k, L.E), s.tiles, s.ntiles);
        MOE_LAUNCH_CHECK();
    }
    const int mt = max_tiles(T, L.k, L.E);
    const int nt1 = (L.Imax() + 127) / 128;
    const int g1 = ((mt * nt1 + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL((k_grouped_gemm<FMT, true>), dim3(g1), dim3(kGT), 0, st, L, T, s.tiles, s.ntiles, nt1,
                       offsets, perm, s.x16, s.xexp, s.h16, s.hexp, (float*)nullptr, (float*)nullptr);
    MOE_LAUNCH_CHECK();
    const int nt2 = (L.H + 255) / 256;
    const int g2 = ((mt * nt2 + kXcds - 1) / kXcds) * kXcds;
    switch (mode) {
        case PrefillOut::kF16Scaled:
            hipLaunchKernelGGL((k_grouped_gemm<FMT, false, _Float16, false>), dim3(g2), dim3(kGT), 0, st, L, T,
                               s.tiles, s.ntiles, nt2, offsets, perm, s.h16, s.hexp, nullptr, nullptr,
                               static_cast<_Float16*>(y_sorted), static_cast<_Float16*>(y_shared));
            break;
        case PrefillOut::kF16:
            hipLaunchKernelGGL((k_grouped_gemm<FMT, false, _Float16, true>), dim3(g2), dim3(kGT), 0, st, L, T,
                               s.tiles, s.ntiles, nt2, offsets, perm, s.h16, s.hexp, nullptr, nullptr,
                               static_cast<_Float16*>(y_sorted), static_cast<_Float16*>(y_shared));
            break;
        default:
            hipLaunchKernelGGL((k_grouped_gemm<FMT, false, float, true>), dim3(g2), dim3(kGT), 0, st, L, T,
                               s.tiles, s.ntiles, nt2, offsets, perm, s.h16, s.hexp, nullptr, nullptr,
                               static_cast<float*>(y_sorted), static_cast<float*>(y_shared));
            break;
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_prefill_experts(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                  const int32_t* perm, void* y_sorted, void* y_shared, PrefillOut mode, void* scratch,
                                  hipStream_t st, bool prepared) {
    const PrefillScratch s = carve_prefill(L, T, scratch, nullptr);
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_prefill_f<MOE_Q8_B32>(L, x, T, offsets, perm, y_sorted, y_shared, mode, s, prepared, st);
        case MOE_Q4_B32: return launch_prefill_f<MOE_Q4_B32>(L, x, T, offsets, perm, y_sorted, y_shared, mode, s, prepared, st);
        case MOE_Q2_B32: return launch_prefill_f<MOE_Q2_B32>(L, x, T, offsets, perm, y_sorted, y_shared, mode, s, prepared, st);
        default: return MOE_ERR_INVALID_ARG;
    }
}

static size_t route_small_lds(const LayerView& L, int T) {
    return align_up((size_t)T * L.k, 4) * 4 + align_up((size_t)L.E + 1, 4) * 4 + perm_small_lds(T, L.E);
}

bool route_small_fits(const LayerView& L, int T) {
    return T >= 2 && T <= kSmallMaxT && L.E <= 1024 && route_small_lds(L, T) <= 65536;
}

template <int KPL, int FMT>
static moe_status launch_route_small_f(const LayerView& L, const uint16_t* x, int T, const float* logits,
                                       int32_t* ids, float* p, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, const PrefillScratch& s, hipStream_t st) {
    constexpr int G = perm_group<FMT>();
    constexpr int VPT = G <= 8 ? 8 : 16;
    auto kern = k_route_small<KPL, G, VPT>;
    const size_t sm = route_small_lds(L, T);
    if (sm > 65536) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(kern, dim3((unsigned)(T + 1)), dim3(kSmallThreads), sm, st, logits, T, L.E,
                       L.k, ids, p, offsets, perm, inv, x, L.H, s.x16, s.xexp, L.Is > 0 ? 1 : 0,
                       max_tiles(T, L.k, L.E), s.tiles, s.ntiles);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

template <int KPL>
static moe_status launch_route_small_k(const LayerView& L, const uint16_t* x, int T, const float* logits,
                                       int32_t* ids, float* p, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, const PrefillScratch& s, hipStream_t st) {
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_route_small_f<KPL, MOE_Q8_B32>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
        case MOE_Q4_B32: return launch_route_small_f<KPL, MOE_Q4_B32>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
        case MOE_Q2_B32: return launch_route_small_f<KPL, MOE_Q2_B32>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
        default: return MOE_ERR_INVALID_ARG;
    }
}

moe_status launch_route_small(const LayerView& L, const uint16_t* x, int T, const float* logits, int32_t* ids,
                              float* p, int32_t* offsets, int32_t* perm, int32_t* inv, void* scratch, hipStream_t st) {
    if (!route_small_fits(L, T)) return MOE_ERR_UNSUPPORTED;
    const PrefillScratch s = carve_prefill(L, T, scratch, nullptr);
    if (L.E <= 64) return launch_route_small_k<1>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
    if (L.E <= 128) return launch_route_small_k<2>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
    if (L.E <= 256) return launch_route_small_k<4>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
    if (L.E <= 512) return launch_route_small_k<8>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
    return launch_route_small_k<16>(L, x, T, logits, ids, p, offsets, perm, inv, s, st);
}

}  // namespace moe
