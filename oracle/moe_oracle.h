/*
 * Oracle of the routed, block-quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded fp64 CPU implementation of what the layer computes, used to
 * check the HIP library. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header, table or helper with the HIP library; it decodes the
 * same packed bytes with its own readers.
 *
 * The pages describe a layer in which a router picks a few experts per token (8 of 256, about
 * 10 of 24,576; 648news "cyber-on-strata" article, section on tiered VRAM/RAM inference; bagrov.by
 * article, section on MoE and hierarchical caching), the router and an always-used shared expert
 * stay resident on the GPU (648news "nano-cuda-moe" article, section on CPU/GPU asynchronous
 * compute), and weights are integers with one scale per 32 values (same article, section on the
 * VRAM/RAM memory hierarchy). The pages print no formula for any step; the arithmetic below is the
 * plainest reading of that layer, and every such reading is listed with the design notes.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_Q8 = 0, ORC_Q4 = 1, ORC_Q2 = 2 };

/* One quantized matrix stack: codes [E][N][K*bits/8], scales fp16 bits [E][N][K/32]. */
typedef struct {
    const uint8_t* codes;
    const uint16_t* scales;
} orc_qmat;

typedef struct {
    int32_t H, I, E, k, Is, fmt;
    const float* w_router;   /* [E][H] */
    const float* bias;       /* [E] or NULL (= 0) */
    orc_qmat gate, up, down; /* gate/up [E][I][H], down [E][H][I] */
    orc_qmat sh_gate, sh_up, sh_down; /* shared expert, one of each, used iff Is > 0 */
} orc_layer;

double orc_bf16(uint16_t bits);
double orc_f16(uint16_t bits);
/* value of element kappa of a packed row (the code's level, before the scale) */
double orc_code_value(int fmt, const uint8_t* row, int32_t kappa);
/* dense dequantization of one [N][K] matrix: out[n*K + kappa] = value * scale */
void orc_dequant(int fmt, const uint8_t* codes, const uint16_t* scales, int32_t N, int32_t K, double* out);

/* logits[t][e] = sum_h x[t][h] * w_router[e][h] + bias[e] */
void orc_router(const orc_layer* L, const uint16_t* x, int32_t T, double* logits);
/* top-k by (value desc, index asc) and softmax over the chosen k. Returns 0, or -1 on NaN. */
int orc_topk_softmax(const double* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, double* p);
/* stable counting sort of pair ids q = t*k + j by expert: offsets [E+1], perm [T*k], inv [T*k] */
void orc_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* offsets, int32_t* perm,
                 int32_t* inv);
/* one SwiGLU expert on one fp64 activation row: y = D (silu(G x) * (U x)) */
void orc_expert(int fmt, int32_t H, int32_t I, const uint8_t* g_codes, const uint16_t* g_scales,
                const uint8_t* u_codes, const uint16_t* u_scales, const uint8_t* d_codes,
                const uint16_t* d_scales, const double* x, double* h_out /* [I] or NULL */, double* y);
/* routed expert e of the layer, and the shared expert, on one token row */
void orc_routed_expert(const orc_layer* L, int32_t e, const double* x, double* y);
void orc_shared_expert(const orc_layer* L, const double* x, double* y);

/*
 * One token through the whole layer. logits_in (length E) overrides the router when non-NULL.
 * Outputs (any may be NULL): logits [E], ids [k], p [k], y_pairs [k][H], y_shared [H], Y [H].
 */
int orc_token(const orc_layer* L, const uint16_t* x_row, const double* logits_in, double* logits,
              int32_t* ids, double* p, double* y_pairs, double* y_shared, double* Y);
/* All T tokens (loop over orc_token). logits_in is [T][E] or NULL. Same output shapes x T. */
int orc_layer_forward(const orc_layer* L, const uint16_t* x, int32_t T, const double* logits_in,
                      double* logits, int32_t* ids, double* p, double* y_pairs, double* y_shared,
                      double* Y);
/* out[t] = sum_j p[t][j] * y_rows[row_of_pair ? row_of_pair[t*k+j] : t*k+j] + y_shared[t] (NULL = 0) */
void orc_combine(int32_t T, int32_t k, int32_t H, const double* p, const double* y_rows, const int32_t* row_of_pair,
                 const double* y_shared, double* out);
/*
 * Brute force: every expert on every token, weighted by a mask that is the full softmax restricted
 * to the k best experts (by rank counting) and renormalised, summed in expert order, plus shared.
 */
int orc_dense_masked(const orc_layer* L, const uint16_t* x, int32_t T, double* Y);

/*
 * KV cache codec (648news "nano-cuda-moe" article, section on the VRAM/RAM memory hierarchy: the
 * KV cache is int8 with one scale per 32 values, and an indexer picks 2048 positions per query).
 * A row of D values (D a multiple of 32) is cut into blocks of 32; per block, in fp32 as the
 * device does it: m = max |v|, s = fp16(m / 127) (round to nearest even; a result beyond the fp16
 * range saturates at 65504), code = rne(v / s) clamped to [-127, 127], or 0 when s is 0. The
 * quantisation decision is taken in fp32 on both sides (the pages fix no precision for it).
 *   src bf16 [rows][D] -> codes int8 [rows][D], scales fp16 bits [rows][D/32]
 */
uint16_t orc_f32_to_f16(float q);
void orc_kv_encode(const uint16_t* src, int32_t rows, int32_t D, int8_t* codes, uint16_t* scales);
/* out[j][d] = codes[idx[j]][d] * scale of its block, for idx[j] in [0, n_rows); 0 otherwise. */
void orc_kv_gather(const int8_t* codes, const uint16_t* scales, int32_t n_rows, int32_t D, const int32_t* idx,
                   int32_t n_idx, double* out);

#ifdef __cplusplus
}
#endif
#endif
