// Probability-weighted combine plus the always-used shared expert (648news
// 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute": the shared expert is
// resident next to the router). Gather form, no atomics: every output element is one thread's sum
// in slot order, then the shared term, so repeated calls give identical bits.
#include "kernels.h"

namespace moe {

// Rows are fp32 (the C-ABI call) or fp16 (the fused layer's internal rows); the sum is fp32 either
// way. Thread c of a token owns the 4 columns 4c .. 4c + 3 and the 4 columns H/2 + 4c ..: each of
// its loads and stores is then contiguous over the lanes of a wave (16 or 8 bytes a lane).
template <typename RT>
__device__ __forceinline__ void load8(const RT* row, int c, int half, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* row, int c, int half, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(row)[c];
    const float4 b = reinterpret_cast<const float4*>(row + half)[c];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<_Float16>(const _Float16* row, int c, int half, float (&v)[8]) {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    const half4_t a = reinterpret_cast<const half4_t*>(row)[c];
    const half4_t b = reinterpret_cast<const half4_t*>(row + half)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = (float)a[e];
        v[4 + e] = (float)b[e];
    }
}

// The shared row and the token's exponent do not depend on the routing and are loaded first; the
// pair rows and weights of a token are the same for the whole block (scalar loads, no LDS), and its
// k rows are read eight at a time with every load of a group in flight before any is used (a dropped
// pair reads row 0 and adds nothing). The sum stays in slot order, then the shared row. With texp,
// the rows of token t are at the scale 2^(2 texp[t]) of its activations and the sum is multiplied
// by 2^(-2 texp[t]) (exact in fp32).
template <typename RT>
__global__ __launch_bounds__(256) void k_combine(int T, int k, int H, const float* __restrict__ p,
                                                 const RT* __restrict__ y_rows,
                                                 const int32_t* __restrict__ row_of_pair,
                                                 const RT* __restrict__ y_shared, const int32_t* __restrict__ texp,
                                                 float* __restrict__ out) {
    constexpr int kB = 8;   // rows in flight
    const int t = blockIdx.y;
    const int nc = H / 8;
    const int c8 = blockIdx.x * blockDim.x + threadIdx.x;  // columns 4 c8 .. and H/2 + 4 c8 ..
    const int cc = min(c8, nc - 1);                        // loads stay in the row; only c8 < nc stores
    const int half = H / 2;
    float sh[8];
    if (y_shared) load8<RT>(y_shared + (size_t)t * H, cc, half, sh);
    const int e = texp ? texp[t] : 0;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kB) {
        float v[kB][8], pj[kB];
        bool ok[kB];
#pragma unroll
        for (int jj = 0; jj < kB; ++jj) {
            const int q = t * k + min(j0 + jj, k - 1);
            const int r = row_of_pair ? row_of_pair[q] : q;
            pj[jj] = p[q];
            ok[jj] = j0 + jj < k && (unsigned)r < (unsigned)(T * k);
            load8<RT>(y_rows + (size_t)(ok[jj] ? r : 0) * H, cc, half, v[jj]);
        }
#pragma unroll
        for (int jj = 0; jj < kB; ++jj) {
            if (!ok[jj]) continue;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += pj[jj] * v[jj][i];
        }
    }
    if (y_shared) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sh[i];
    }
    if (texp) {
        const float sc = pow2f(-2 * e);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= sc;
    }
    if (c8 >= nc) return;
    reinterpret_cast<float4*>(out + (size_t)t * H)[c8] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(out + (size_t)t * H + half)[c8] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

moe_status launch_combine(int T, int k, int H, const float* p, const float* y_rows, const int32_t* row_of_pair,
                          const float* y_shared, float* out, hipStream_t s) {
    const int cols = H / 8;
    dim3 grid((cols + 255) / 256, T);
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, s, T, k, H, p, y_rows, row_of_pair, y_shared,
                       (const int32_t*)nullptr, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_combine_f16(int T, int k, int H, const float* p, const _Float16* y_rows,
                              const int32_t* row_of_pair, const _Float16* y_shared, const int32_t* texp, float* out,
                              hipStream_t s) {
    const int cols = H / 8;
    dim3 grid((cols + 255) / 256, T);
    hipLaunchKernelGGL(k_combine<_Float16>, grid, dim3(256), 0, s, T, k, H, p, y_rows, row_of_pair, y_shared, texp,
                       out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
