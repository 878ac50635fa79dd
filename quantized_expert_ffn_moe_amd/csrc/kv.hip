// KV cache codec: block-32 int8 with one fp16 scale per block, and a sparse gather of cache rows.
//
// The pages keep the attention KV cache as int8 with one scale per 32 values and select 2048
// positions per query with an indexer (648news 07-nano-cuda-moe-qwen38-release, section "memory
// hierarchy spanning VRAM and RAM"; cache sizes in 648news 10-cyber-on-strata-moe-local-inference,
// section "KV transfer and next update"). Both kernels are HBM-bound streams:
//   k_kv_encode  one thread per 32-value block: 64 bytes of bf16 in, max |v| in fp32 (NaNs left
//                out), s = fp16(max / 127) saturating at 65504, codes rne(v / s) (fp32 division,
//                correctly rounded) clamped to +-127 (a NaN value: code 0), 32 bytes of codes and 2
//                bytes of scale out;
//   k_kv_gather  nb = D / 32 threads per output row, each taking 8 chunks of 4 values strided by
//                nb chunks: all 8 code words and scales of a thread are in flight together, and
//                at each of the 8 steps the row's threads read contiguous code bytes and write
//                contiguous 16-byte pieces of exact fp32 values.
#include "kernels.h"

namespace moe {

typedef uint32_t kv_u32x4 __attribute__((ext_vector_type(4)));
typedef float kv_f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_kv_encode(const uint16_t* __restrict__ src, int64_t nblocks,
                                                   int8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const kv_u32x4* in = reinterpret_cast<const kv_u32x4*>(src + b * 32);
    const kv_u32x4 r0 = in[0], r1 = in[1], r2 = in[2], r3 = in[3];
    const uint32_t w[16] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w,
                            r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w};
    float v[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
    // block maximum by comparison, so that NaNs (quiet or signalling) never enter it: fmaxf follows
    // IEEE maxNum, which returns NaN for a signalling NaN and would drop the earlier elements
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float a = fabsf(v[i]);
        m = a > m ? a : m;
    }
    _Float16 s16 = (_Float16)(m / 127.0f);
    if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;   // scale saturates at the largest finite fp16
    const float sf = (float)s16;
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t packed = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // a NaN value gets code 0 (it took no part in the block maximum either)
            const float xv = v[4 * i + j];
            int c = 0;
            if (sf != 0.f && xv == xv) c = (int)fminf(fmaxf(rintf(xv / sf), -127.f), 127.f);
            packed |= ((uint32_t)c & 0xFFu) << (8 * j);
        }
        out[i] = packed;
    }
    kv_u32x4* dst = reinterpret_cast<kv_u32x4*>(codes + b * 32);
    dst[0] = kv_u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = kv_u32x4{out[4], out[5], out[6], out[7]};
    scales[b] = __builtin_bit_cast(uint16_t, s16);
}

__global__ __launch_bounds__(256) void k_kv_gather(const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                                   int32_t n_rows, int32_t nb, const int32_t* __restrict__ idx,
                                                   int64_t nitems, float* __restrict__ out) {
    const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (it >= nitems) return;
    const int64_t j = it / nb;
    const int l = (int)(it - j * nb);
    const int32_t r = idx[j];
    const int D = 32 * nb;
    float* dst = out + j * D;
    // lane l of the row's nb lanes takes the 4-value chunks l, l + nb, ..., l + 7 nb: for each of
    // its 8 steps the row's lanes read 4 nb contiguous code bytes and write 16 nb contiguous bytes
    if ((uint32_t)r >= (uint32_t)n_rows) {
#pragma unroll
        for (int q = 0; q < 8; ++q) *reinterpret_cast<kv_f32x4*>(dst + 4 * (l + nb * q)) = kv_f32x4{0.f, 0.f, 0.f, 0.f};
        return;
    }
    const int8_t* crow = codes + (int64_t)r * D;
    const uint16_t* srow = scales + (int64_t)r * nb;
    uint32_t w[8];
    uint16_t sc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int e0 = 4 * (l + nb * q);
        w[q] = *reinterpret_cast<const uint32_t*>(crow + e0);
        sc[q] = srow[e0 / 32];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t u = w[q];
        const float s = f16_to_f32(sc[q]);
        *reinterpret_cast<kv_f32x4*>(dst + 4 * (l + nb * q)) =
            kv_f32x4{(float)(int8_t)(u & 0xFFu) * s, (float)(int8_t)((u >> 8) & 0xFFu) * s,
                     (float)(int8_t)((u >> 16) & 0xFFu) * s, (float)(int8_t)(u >> 24) * s};
    }
}

moe_status launch_kv_encode(const uint16_t* src, int32_t rows, int32_t D, int8_t* codes, uint16_t* scales,
                            hipStream_t s) {
    const int64_t nblocks = (int64_t)rows * (D / 32);
    if (nblocks == 0) return MOE_OK;
    hipLaunchKernelGGL(k_kv_encode, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, src, nblocks, codes,
                       scales);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status launch_kv_gather(const int8_t* codes, const uint16_t* scales, int32_t n_rows, int32_t D,
                            const int32_t* idx, int32_t n_idx, float* out, hipStream_t s) {
    const int64_t nitems = (int64_t)n_idx * (D / 32);
    if (nitems == 0) return MOE_OK;
    hipLaunchKernelGGL(k_kv_gather, dim3((unsigned)((nitems + 255) / 256)), dim3(256), 0, s, codes, scales, n_rows,
                       D / 32, idx, nitems, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
