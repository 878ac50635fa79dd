// Prefill-regime experts: grouped GEMM over expert-sorted row tiles on the gfx950 matrix cores.
//
// Prompt processing on the pages runs in 8K-token chunks with GEMMs and grouped expert kernels
// (648news 07-nano-cuda-moe-qwen38-release, section "speed comparison and accuracy check"). Here:
//   - the pairs of each expert are contiguous after the permutation; a tile list of
//     (group, first row) covers every group with BM-row tiles, the shared expert being one more
//     group of all T tokens;
//   - gate/up: C[BM x 128] = A[BM x H] * B[128 x H]^T where A rows are the tokens gathered through
//     perm (x converted once to fp16) and B rows interleave 16 gate rows and 16 up rows, so the
//     SwiGLU epilogue finds g and u of the same (row, n) in the same lane; h is written in fp16;
//   - down: C[BM x 128] = h[BM x I] * D[128 x I]^T, fp32 output rows in sorted order;
//   - weights are dequantised into LDS as fp16 (level * scale, rounded once), both operands feed
//     v_mfma_f32_16x16x32_f16 with fp32 accumulation.
#include "kernels.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;      // rows (pairs) per tile
constexpr int kBN = 128;      // weight rows per tile
constexpr int kBK = 64;       // K per step (two 32-element scale blocks)
constexpr int kLdsStride = kBK + 8;  // fp16 elements per LDS row (padding against bank conflicts)

struct TileDesc {
    int group;  // expert id, or E for the shared expert
    int row0;   // first row of the tile inside its group
};

// -------------------------------------------------------------------------------- tile list
// One block of 1024 threads: thread e counts the tiles of expert e, a block scan places them,
// the shared group's tiles follow the routed ones.
__global__ __launch_bounds__(1024) void k_build_tiles(const int32_t* __restrict__ offsets, int E, int T, int has_shared,
                                                      TileDesc* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    __shared__ int part[1024];
    const int e = threadIdx.x;
    const int n = e < E ? offsets[e + 1] - offsets[e] : 0;
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
    for (int i = 0; i < nt; ++i) tiles[start + i] = TileDesc{e, i * kBM};
    if (e == 1023) {
        int total = part[1023];
        if (has_shared) {
            const int ns = (T + kBM - 1) / kBM;
            for (int i = 0; i < ns; ++i) tiles[total + i] = TileDesc{E, i * kBM};
            total += ns;
        }
        *ntiles = total;
    }
}

int max_tiles(int T, int k, int E) { return (T * k) / kBM + E + (T + kBM - 1) / kBM + 1; }

// -------------------------------------------------------------------------------- x to fp16
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, int64_t n8, _Float16* __restrict__ x16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    half8 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = (_Float16)bf16_lo(w[j]);
        o[2 * j + 1] = (_Float16)bf16_hi(w[j]);
    }
    reinterpret_cast<half8*>(x16)[i] = o;
}

// -------------------------------------------------------------------------------- shared pieces

// Dequantise one 32-element block into 32 fp16 values in LDS.
template <int FMT>
__device__ __forceinline__ void dequant_block_to_lds(const uint8_t* codes, uint16_t scale_bits, _Float16* dst) {
    Block32 b;
    load_block<FMT>(codes, b);
    const float s = f16_to_f32(scale_bits);
    half8 v[4];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i / 8][i % 8] = (_Float16)(block_level<FMT>(b, i) * s);
#pragma unroll
    for (int c = 0; c < 4; ++c) reinterpret_cast<half8*>(dst)[c] = v[c];
}

__device__ __forceinline__ half8 lds_frag(const _Float16* base, int row, int kofs) {
    return *reinterpret_cast<const half8*>(base + row * kLdsStride + kofs);
}

// 4 waves in a 2 x 2 grid; each wave owns a 64 x 64 sub-tile = 4 x 4 MFMA tiles of 16 x 16.
__device__ __forceinline__ void mma_step(const _Float16* As, const _Float16* Bs, int wm, int wn, int lane,
                                         floatx4 (&acc)[4][4]) {
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
        const int kofs = kk + 8 * (lane / 16);
        half8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = lds_frag(As, wm * 64 + 16 * i + lane % 16, kofs);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = lds_frag(Bs, wn * 64 + 16 * j + lane % 16, kofs);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// Rows of a tile: the group's base (in sorted order, or 0 for the shared group) and its row count.
__device__ __forceinline__ void group_rows(const int32_t* offsets, int E, int T, int g, int& base, int& count) {
    if (g == E) { base = 0; count = T; }
    else { base = offsets[g]; count = offsets[g + 1] - base; }
}

// -------------------------------------------------------------------------------- gate/up
template <int FMT>
__global__ __launch_bounds__(256) void k_prefill_gateup(LayerView L, int T, const TileDesc* __restrict__ tiles,
                                                        const int32_t* __restrict__ ntiles,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm,
                                                        const _Float16* __restrict__ x16, _Float16* __restrict__ h16) {
    __shared__ _Float16 As[kBM * kLdsStride];
    __shared__ _Float16 Bs[kBN * kLdsStride];
    if ((int)blockIdx.x >= *ntiles) return;
    const TileDesc td = tiles[blockIdx.x];
    const bool shared = td.group == L.E;
    const int N = shared ? L.Is : L.I;
    const int n0 = blockIdx.y * (kBN / 2);
    if (n0 >= N) return;
    int base, count;
    group_rows(offsets, L.E, T, td.group, base, count);
    const int nrows = min(kBM, count - td.row0);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int H = L.H;

    // A: 4 16-byte pieces per thread, rows tid/8 + 32 i, piece tid % 8
    int arow_tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid / 8 + 32 * i;
        if (r < nrows) {
            const int pos = td.row0 + r;
            arow_tok[i] = shared ? pos : perm[base + pos] / L.k;
        } else {
            arow_tok[i] = -1;
        }
    }
    // B: thread -> (LDS row j = tid / 2, block tid % 2); LDS rows interleave 16 gate / 16 up rows
    const int bj = tid / 2, bblk = tid % 2;
    const int granule = bj / 16;
    const bool is_up = granule & 1;
    const int bn = n0 + (granule / 2) * 16 + bj % 16;
    const int64_t rb = row_bytes(FMT, H);
    const uint8_t* bcodes;
    const uint16_t* bscales;
    if (shared) {
        bcodes = (is_up ? L.su_codes : L.sg_codes) + (int64_t)bn * rb;
        bscales = (is_up ? L.su_scales : L.sg_scales) + (int64_t)bn * (H / 32);
    } else {
        const int64_t row = (int64_t)td.group * L.I + bn;
        bcodes = (is_up ? L.u_codes : L.g_codes) + row * rb;
        bscales = (is_up ? L.u_scales : L.g_scales) + row * (H / 32);
    }
    const bool bvalid = bn < N;

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < H; k0 += kBK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = tid / 8 + 32 * i, piece = tid % 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (arow_tok[i] >= 0) v = *reinterpret_cast<const uint4*>(x16 + (size_t)arow_tok[i] * H + k0 + piece * 8);
            *reinterpret_cast<uint4*>(As + r * kLdsStride + piece * 8) = v;
        }
        {
            const int kb = k0 / 32 + bblk;
            _Float16* dst = Bs + bj * kLdsStride + bblk * 32;
            if (bvalid) {
                dequant_block_to_lds<FMT>(bcodes + (int64_t)kb * block_bytes(FMT), bscales[kb], dst);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) reinterpret_cast<uint4*>(dst)[c] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        __syncthreads();
        mma_step(As, Bs, wm, wn, lane, acc);
        __syncthreads();
    }

    // epilogue: tiles j = 0,2 are gate, j = 1,3 the matching up
    const int Imax = L.Imax();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
            const int n = n0 + (2 * wn + jp) * 16 + lane % 16;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + 16 * i + 4 * (lane / 16) + r;
                if (row >= nrows) continue;
                const float hv = silu_mul(acc[i][2 * jp][r], acc[i][2 * jp + 1][r]);
                const int64_t hrow = shared ? (int64_t)T * L.k + td.row0 + row : (int64_t)base + td.row0 + row;
                h16[hrow * Imax + n] = (_Float16)hv;
            }
        }
    }
}

// -------------------------------------------------------------------------------- down
template <int FMT>
__global__ __launch_bounds__(256) void k_prefill_down(LayerView L, int T, const TileDesc* __restrict__ tiles,
                                                      const int32_t* __restrict__ ntiles,
                                                      const int32_t* __restrict__ offsets,
                                                      const _Float16* __restrict__ h16, float* __restrict__ y_sorted,
                                                      float* __restrict__ y_shared) {
    __shared__ _Float16 As[kBM * kLdsStride];
    __shared__ _Float16 Bs[kBN * kLdsStride];
    if ((int)blockIdx.x >= *ntiles) return;
    const TileDesc td = tiles[blockIdx.x];
    const bool shared = td.group == L.E;
    const int Kin = shared ? L.Is : L.I;
    const int H = L.H;
    const int m0 = blockIdx.y * kBN;
    int base, count;
    group_rows(offsets, L.E, T, td.group, base, count);
    const int nrows = min(kBM, count - td.row0);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int Imax = L.Imax();
    const int64_t hrow0 = shared ? (int64_t)T * L.k + td.row0 : (int64_t)base + td.row0;

    const int bj = tid / 2, bblk = tid % 2;
    const int bm = m0 + bj;
    const int64_t rb = row_bytes(FMT, Kin);
    const uint8_t* bcodes;
    const uint16_t* bscales;
    if (shared) {
        bcodes = L.sd_codes + (int64_t)bm * rb;
        bscales = L.sd_scales + (int64_t)bm * (Kin / 32);
    } else {
        const int64_t row = (int64_t)td.group * H + bm;
        bcodes = L.d_codes + row * rb;
        bscales = L.d_scales + row * (Kin / 32);
    }
    const bool bvalid = bm < H;

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < Kin; k0 += kBK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = tid / 8 + 32 * i, piece = tid % 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r < nrows) v = *reinterpret_cast<const uint4*>(h16 + (hrow0 + r) * Imax + k0 + piece * 8);
            *reinterpret_cast<uint4*>(As + r * kLdsStride + piece * 8) = v;
        }
        {
            const int kb = k0 / 32 + bblk;
            _Float16* dst = Bs + bj * kLdsStride + bblk * 32;
            if (bvalid) {
                dequant_block_to_lds<FMT>(bcodes + (int64_t)kb * block_bytes(FMT), bscales[kb], dst);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) reinterpret_cast<uint4*>(dst)[c] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        __syncthreads();
        mma_step(As, Bs, wm, wn, lane, acc);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + wn * 64 + 16 * j + lane % 16;
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
    const int mt = max_tiles(T, L.k, L.E);
    const int nmax = L.Imax();
    hipLaunchKernelGGL((k_prefill_gateup<FMT>), dim3(mt, (nmax + kBN / 2 - 1) / (kBN / 2)), dim3(256), 0, st, L, T,
                       s.tiles, s.ntiles, offsets, perm, s.x16, s.h16);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL((k_prefill_down<FMT>), dim3(mt, (L.H + kBN - 1) / kBN), dim3(256), 0, st, L, T, s.tiles,
                       s.ntiles, offsets, s.h16, y_sorted, y_shared);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_prefill_experts(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                  const int32_t* perm, float* y_sorted, float* y_shared, void* scratch,
                                  hipStream_t st) {
    const PrefillScratch s = carve_prefill(L, T, scratch, nullptr);
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, st, offsets, L.E, T, L.Is > 0 ? 1 : 0, s.tiles,
                       s.ntiles);
    MOE_LAUNCH_CHECK();
    const int64_t n8 = (int64_t)T * L.H / 8;
    hipLaunchKernelGGL(k_x_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, x, n8, s.x16);
    MOE_LAUNCH_CHECK();
    switch (L.fmt) {
        case MOE_Q8_B32: return launch_prefill_f<MOE_Q8_B32>(L, x, T, offsets, perm, y_sorted, y_shared, s, st);
        case MOE_Q4_B32: return launch_prefill_f<MOE_Q4_B32>(L, x, T, offsets, perm, y_sorted, y_shared, s, st);
        case MOE_Q2_B32: return launch_prefill_f<MOE_Q2_B32>(L, x, T, offsets, perm, y_sorted, y_shared, s, st);
        default: return MOE_ERR_INVALID_ARG;
    }
}

}  // namespace moe
