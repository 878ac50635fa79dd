// Probability-weighted combine plus the always-used shared expert (648news
// 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute": the shared expert is
// resident next to the router). Gather form, no atomics: every output element is one thread's sum
// in slot order, then the shared term, so repeated calls give identical bits.
#include "kernels.h"

namespace moe {

// Rows are fp32 (the C-ABI call) or fp16 (the fused layer's internal rows); the sum is fp32 either way.
template <typename RT>
__device__ __forceinline__ float4 load4(const RT* row, int c);
template <>
__device__ __forceinline__ float4 load4<float>(const float* row, int c) {
    return reinterpret_cast<const float4*>(row)[c];
}
template <>
__device__ __forceinline__ float4 load4<_Float16>(const _Float16* row, int c) {
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const half4 v = reinterpret_cast<const half4*>(row)[c];
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

template <typename RT>
__global__ __launch_bounds__(256) void k_combine(int T, int k, int H, const float* __restrict__ p,
                                                 const RT* __restrict__ y_rows,
                                                 const int32_t* __restrict__ row_of_pair,
                                                 const RT* __restrict__ y_shared, float* __restrict__ out) {
    const int t = blockIdx.y;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;  // float4 column
    __shared__ float ps[16];
    __shared__ int rows[16];
    if (threadIdx.x < k) {
        const int q = t * k + threadIdx.x;
        ps[threadIdx.x] = p[q];
        rows[threadIdx.x] = row_of_pair ? row_of_pair[q] : q;
    }
    __syncthreads();
    if (c >= H / 4) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        if ((unsigned)rows[j] >= (unsigned)(T * k)) continue;  // dropped pair
        const float4 v = load4<RT>(y_rows + (size_t)rows[j] * H, c);
        const float pj = ps[j];
        acc.x += pj * v.x; acc.y += pj * v.y; acc.z += pj * v.z; acc.w += pj * v.w;
    }
    if (y_shared) {
        const float4 v = load4<RT>(y_shared + (size_t)t * H, c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<float4*>(out + (size_t)t * H)[c] = acc;
}

moe_status launch_combine(int T, int k, int H, const float* p, const float* y_rows, const int32_t* row_of_pair,
                          const float* y_shared, float* out, hipStream_t s) {
    const int cols = H / 4;
    dim3 grid((cols + 255) / 256, T);
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, s, T, k, H, p, y_rows, row_of_pair, y_shared, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_combine_f16(int T, int k, int H, const float* p, const _Float16* y_rows,
                              const int32_t* row_of_pair, const _Float16* y_shared, float* out, hipStream_t s) {
    const int cols = H / 4;
    dim3 grid((cols + 255) / 256, T);
    hipLaunchKernelGGL(k_combine<_Float16>, grid, dim3(256), 0, s, T, k, H, p, y_rows, row_of_pair, y_shared, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
