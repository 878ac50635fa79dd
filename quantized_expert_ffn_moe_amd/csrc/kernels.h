// Internal launchers of the gfx950 kernels (host side). Each returns MOE_OK or MOE_ERR_HIP.
#pragma once

#include "common.h"

namespace moe {

// Shapes and weight pointers as the kernels see them (validated by the API layer).
struct LayerView {
    int H, I, E, k, Is, fmt;
    const float* w_router;
    const float* bias;
    const uint8_t *g_codes, *u_codes, *d_codes;
    const uint16_t *g_scales, *u_scales, *d_scales;
    const uint8_t *sg_codes, *su_codes, *sd_codes;
    const uint16_t *sg_scales, *su_scales, *sd_scales;
    const uint8_t* pk;   // the packed copy of the codes for the grouped GEMMs, or NULL
    __host__ __device__ int Imax() const { return I > Is ? I : Is; }
};

// The packed copy (moe_pack_prefill_codes): the codes of a matrix of N rows and K columns in pieces
// of 32 rows x 64 columns (64 BB bytes: block 2s of the 32 rows, then block 2s + 1), group-major;
// its scales in pieces of 32 rows x 8 blocks (512 bytes: row by row, 8 scales each), group-major;
// the code matrices in the order E gates, E ups, E downs, shared gate, up, down, then the scale
// matrices in the same order.
__host__ __device__ inline int64_t packed_mat_bytes(int N, int K, int fmt) {
    return (int64_t)((N + 31) / 32) * ((K + 63) / 64) * 64 * block_bytes(fmt);
}
__host__ __device__ inline int64_t packed_scale_bytes(int N, int K) {
    return (int64_t)((N + 31) / 32) * ((K / 32 + 7) / 8) * 512;
}
struct PackedOffsets {
    int64_t pg, pd, psg, psd;                         // code bytes of one gate/up, down, shared gate/up, shared down
    int64_t gate, up, down, sh_gate, sh_up, sh_down;  // where each code stack starts
    int64_t qg, qd, qsg, qsd;                         // scale bytes of the same matrices
    int64_t s_gate, s_up, s_down, s_sh_gate, s_sh_up, s_sh_down;   // where each scale stack starts
    int64_t total;
};
__host__ __device__ inline PackedOffsets packed_offsets(const LayerView& L) {
    PackedOffsets o;
    o.pg = packed_mat_bytes(L.I, L.H, L.fmt);
    o.pd = packed_mat_bytes(L.H, L.I, L.fmt);
    o.psg = L.Is > 0 ? packed_mat_bytes(L.Is, L.H, L.fmt) : 0;
    o.psd = L.Is > 0 ? packed_mat_bytes(L.H, L.Is, L.fmt) : 0;
    o.gate = 0;
    o.up = o.gate + (int64_t)L.E * o.pg;
    o.down = o.up + (int64_t)L.E * o.pg;
    o.sh_gate = o.down + (int64_t)L.E * o.pd;
    o.sh_up = o.sh_gate + o.psg;
    o.sh_down = o.sh_up + o.psg;
    o.qg = packed_scale_bytes(L.I, L.H);
    o.qd = packed_scale_bytes(L.H, L.I);
    o.qsg = L.Is > 0 ? packed_scale_bytes(L.Is, L.H) : 0;
    o.qsd = L.Is > 0 ? packed_scale_bytes(L.H, L.Is) : 0;
    o.s_gate = o.sh_down + o.psd;
    o.s_up = o.s_gate + (int64_t)L.E * o.qg;
    o.s_down = o.s_up + (int64_t)L.E * o.qg;
    o.s_sh_gate = o.s_down + (int64_t)L.E * o.qd;
    o.s_sh_up = o.s_sh_gate + o.qsg;
    o.s_sh_down = o.s_sh_up + o.qsg;
    o.total = o.s_sh_down + o.qsd;
    return o;
}
// Writes the packed copy of L's codes to dst (16-byte aligned, packed_offsets(L).total bytes).
moe_status launch_pack_codes(const LayerView& L, uint8_t* dst, hipStream_t s);

// Router GEMM (above kGemvMaxT tokens) and the top-k + softmax kernel (one wave per token); the GEMM's
// scratch: router_scratch_bytes() (split-K partial sums; none when 0).
int router_splits(int T, int H, int E);
size_t router_scratch_bytes(int T, int H, int E);
moe_status launch_router(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                         float* logits, float* scratch, hipStream_t s);
moe_status launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* p, hipStream_t s);
// Router GEMM + top-k; with a split K the reduction and the top-k run as one kernel.
moe_status launch_route_topk(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E, int k,
                             float* logits, int32_t* ids, float* p, float* scratch, hipStream_t s);

// permutation: scratch of perm_scratch_ints(T, E) ints (per-chunk counts, then per-expert totals)
int perm_chunks(int T);
size_t perm_scratch_ints(int T, int E);
moe_status launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* perm, int32_t* inv,
                          int32_t* chunk_scratch, hipStream_t s);

// Router GEMV, 1 <= T <= kGemvMaxT (W_r read once for every token; fp32 dot products).
constexpr int kGemvMaxT = 16;
moe_status launch_route_gemv(const float* w_r, const float* bias, const uint16_t* x, int T, int H, int E,
                             float* logits, hipStream_t s);
// decode (T <= 8): gate/up (given logits, every block runs the top-k and block 0 publishes ids/p);
// down(+combine). h scratch: decode_scratch_floats() floats.
size_t decode_scratch_floats(const LayerView& L, int T);
// Whether the decode kernels fit this shape (their LDS holds x, the routing plan and the SwiGLU
// activations of every chosen pair): with the combine fused (combine) or with per-pair outputs.
bool decode_fits(const LayerView& L, int T, bool combine);
// logits != NULL: route inside (ids/p written); else ids given. out != NULL: combined output [T][H]
// (p required); else y_pairs [T*k][H] and y_shared [T][H].
moe_status launch_decode_experts(const LayerView& L, const uint16_t* x, int T, const float* logits, int32_t* ids,
                                 float* p, float* h, float* out, float* y_pairs, float* y_shared, hipStream_t s);

// prefill experts
size_t prefill_scratch_bytes(const LayerView& L, int T);
// Output rows: fp32 or fp16 at the true scale, or fp16 at each token's activation scale 2^(2 e_t)
// (the fused layer's internal rows; its combine multiplies by 2^(-2 e_t)).
enum class PrefillOut { kF32, kF16, kF16Scaled };
// prepared: x in fp16, its exponents and the tile list are already in the scratch (k_route_small).
moe_status launch_prefill_experts(const LayerView& L, const uint16_t* x, int T, const int32_t* offsets,
                                  const int32_t* perm, void* y_sorted, void* y_shared, PrefillOut mode,
                                  void* scratch, hipStream_t s, bool prepared = false);
// Small batches (2 <= T <= kSmallMaxT): from the router GEMV's logits, one kernel runs the top-k, the
// permutation, the tile list and the x conversion (the prefill scratch then holds what
// launch_prefill_experts(..., prepared = true) needs).
constexpr int kSmallMaxT = 16;
static_assert(kSmallMaxT <= kGemvMaxT, "small batches take their logits from the router GEMV");
bool route_small_fits(const LayerView& L, int T);
moe_status launch_route_small(const LayerView& L, const uint16_t* x, int T, const float* logits, int32_t* ids,
                              float* p, int32_t* offsets, int32_t* perm, int32_t* inv, void* scratch, hipStream_t s);
// e_t of every token, in the scratch of the last launch_prefill_experts on it
const int32_t* prefill_token_exps(const LayerView& L, int T, void* scratch);

moe_status launch_combine(int T, int k, int H, const float* p, const float* y_rows, const int32_t* row_of_pair,
                          const float* y_shared, float* out, hipStream_t s);
// fp16 rows at the scale 2^(2 e_t) of their token (texp[t] = e_t); the sum is unscaled in fp32
moe_status launch_combine_f16(int T, int k, int H, const float* p, const _Float16* y_rows,
                              const int32_t* row_of_pair, const _Float16* y_shared, const int32_t* texp, float* out,
                              hipStream_t s);

// KV cache codec
moe_status launch_kv_encode(const uint16_t* src, int32_t rows, int32_t D, int8_t* codes, uint16_t* scales,
                            hipStream_t s);
moe_status launch_kv_gather(const int8_t* codes, const uint16_t* scales, int32_t n_rows, int32_t D,
                            const int32_t* idx, int32_t n_idx, float* out, hipStream_t s);

}  // namespace moe
