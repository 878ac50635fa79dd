/*
 * moe.h -- C ABI of the routed, block-quantized MoE expert layer for AMD Instinct MI355X (gfx950).
 *
 * The layer: a router scores every expert for each token, the k best experts are chosen and
 * weighted by a softmax over the chosen k, the (token, expert) pairs are grouped by expert, each
 * chosen expert runs a SwiGLU FFN whose weights are integer codes with one fp16 scale per 32
 * values, and the expert outputs are summed with their weights plus an always-used shared expert.
 *
 * Passages this follows (the pages describe the layer, not its arithmetic):
 *   - only a few experts run per token: 8 of 256 (648news 10-cyber-on-strata-moe-local-inference,
 *     section "tiered VRAM/RAM inference"), about ten of 24,576 over 48 layers (bagrov.by
 *     ierarhicheskaya-pamyat-moe-modelej-strata-maya, section "MoE architecture and hierarchical
 *     caching");
 *   - the router and a shared expert stay resident on the GPU (648news
 *     07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute");
 *   - integer values with one scale per 32 (same page, section "memory hierarchy spanning VRAM and
 *     RAM"); 2-, 3- and 4-bit class expert formats (same page, format table in section "speed
 *     comparison and accuracy check");
 *   - prompts are processed in 8K-token chunks with GEMMs and grouped expert kernels (same page,
 *     same section); decode runs the selected experts on the GPU (same page, section
 *     "asynchronous CPU/GPU compute").
 * Here every expert stays resident in HBM; there is no host offload and no expert cache.
 *
 * ----------------------------------------------------------------------------------------------
 * Conventions for every entry point
 *   - Every pointer is a DEVICE pointer unless stated otherwise; descriptors (moe_layer_desc,
 *     moe_layer_weights) are HOST structs read during the call and not kept.
 *   - The caller owns every buffer. The library allocates nothing and keeps no pointer after it
 *     returns. Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *     call returns without waiting; buffers must stay valid until the stream has passed the work.
 *   - Arguments are checked on the host before anything is enqueued. A failed check returns a
 *     status other than MOE_OK and enqueues nothing. A failed launch returns MOE_ERR_HIP.
 *   - Calls keep no state between them and are reentrant; the only process-wide state is per
 *     device and written once (the compute-unit count, and the device address of
 *     moe_layer_static's array). Two calls that share a workspace must be ordered on one stream.
 *   - Workspaces: size them with moe_workspace_size(), 16-byte aligned, any contents. No kernel
 *     waits on another block of its own grid; every cross-block dependency is a kernel boundary,
 *     so calls may be captured in a HIP graph. Expert ids read from memory are range-checked
 *     before they address weights.
 *   - Preconditions that are not checked: x is finite with |x| < 2^60 and the router logits are
 *     finite (no NaN); ids passed in are in [0, E) and distinct within a token; buffers hold the
 *     documented number of elements.
 *   - Activation range: the expert paths multiply 16-bit operands (fp16) on the dot-product units
 *     and the matrix cores. Each token's activations are taken at an exact power-of-two scale
 *     2^e_t, chosen from the token's largest |x| so that it lands in [2, 4) (e_t clamped to
 *     [-60, 60]); the SwiGLU activation h is kept at the scale 2^(2 e_t) (silu(g) * u is bounded
 *     by |g| |u|, so it grows like x^2) and the expert outputs are multiplied by 2^(-2 e_t) in fp32.
 *     Activations of any size therefore keep fp16's relative precision; 16-bit intermediates that
 *     still leave the fp16 range (weights large enough that |h| 2^(2 e_t) exceeds 65504) saturate at
 *     +-65504 rather than becoming inf.
 *
 * Data layout (row-major, innermost index contiguous)
 *   x            bf16 bits  [T][H]
 *   w_router     fp32       [E][H]        router_bias fp32 [E] or NULL (= 0)
 *   gate, up     codes      [E][I][H*bits/8], scales fp16 bits [E][I][H/32]
 *   down         codes      [E][H][I*bits/8], scales fp16 bits [E][H][I/32]
 *   sh_gate/up   codes      [Is][H*bits/8],   scales [Is][H/32]     (shared expert, if Is > 0)
 *   sh_down      codes      [H][Is*bits/8],   scales [H][Is/32]
 *   Code packing along a row (K = the row length):
 *     MOE_Q8_B32  one int8 per element, value = code * scale
 *     MOE_Q4_B32  element 2i in the low nibble of byte i, 2i+1 in the high nibble; two's
 *                 complement (-8..7); value = code * scale
 *     MOE_Q2_B32  element 4i+m in bits 2m..2m+1 of byte i; unsigned c (0..3);
 *                 value = (c - 1.5) * scale
 *   The scale of element kappa of row n is scales[n][kappa / 32].
 *   logits fp32 [T][E]; ids int32 [T][k]; p fp32 [T][k]; pair q = t*k + j.
 *   offsets int32 [E+1]; perm int32 [T*k] (sorted position -> pair); inv int32 [T*k] (pair ->
 *   sorted position).
 *   Outputs Y, y_pairs, y_sorted, y_shared are fp32 with rows of H.
 *
 * Shape limits (MOE_ERR_INVALID_ARG otherwise): T >= 1; 1 <= k <= min(E, 16); E <= 1024;
 * 0 <= decode_max_tokens <= 8;
 * H, I multiples of 32 and Is = 0 or a multiple of 32; H <= 16384; I, Is <= 4096;
 * pointers to codes, scales, x, outputs and workspace 16-byte aligned.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad shape, misalignment */
    MOE_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement (e.g. T > 8 to decode) */
    MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than moe_workspace_size() */
    MOE_ERR_HIP = 4           /* a HIP launch failed */
};

typedef int32_t moe_qformat;
enum { MOE_Q8_B32 = 0, MOE_Q4_B32 = 1, MOE_Q2_B32 = 2 };

/* Entry-point selector for moe_workspace_size(). */
typedef int32_t moe_call;
enum {
    MOE_CALL_ROUTE = 0,
    MOE_CALL_PERMUTE = 1,
    MOE_CALL_EXPERTS_DECODE = 2,
    MOE_CALL_EXPERTS_PREFILL = 3,
    MOE_CALL_COMBINE = 4,
    MOE_CALL_LAYER = 5
};

/* One stack of quantized matrices (device pointers). */
typedef struct {
    const void* codes;
    const uint16_t* scales;
} moe_qmat;

typedef struct {
    int32_t hidden;        /* H */
    int32_t inter;         /* I, SwiGLU intermediate of a routed expert */
    int32_t num_experts;   /* E */
    int32_t top_k;         /* k */
    int32_t shared_inter;  /* Is, 0 = no shared expert */
    moe_qformat fmt;       /* code format of every expert matrix */
    int32_t decode_max_tokens;  /* moe_layer's regime switch: the decode kernels for T <= this (when
                                   they fit), the grouped GEMMs above; 0 = the default, 6 (measured
                                   crossover at H 2048, 256 experts top-8, 4-bit); at most 8 */
} moe_layer_desc;

typedef struct {
    const float* w_router;     /* [E][H] */
    const float* router_bias;  /* [E] or NULL */
    moe_qmat gate, up, down;   /* routed experts, stacked expert-major */
    moe_qmat sh_gate, sh_up, sh_down;  /* shared expert; ignored when shared_inter == 0 */
    const void* prefill_codes; /* NULL, or the codes of every matrix above repacked by
                                  moe_pack_prefill_codes (16-byte aligned): the grouped GEMMs then
                                  read their weight codes from there (same results, fewer memory
                                  transactions); everything else reads the codes above */
} moe_layer_weights;

/*
 * Router and top-k selection (the router scores every expert and only a few run per token: 648news
 * 10-cyber-on-strata-moe-local-inference, section "tiered VRAM/RAM inference"; the router is
 * resident and finishes early: 648news 07-nano-cuda-moe-qwen38-release, section "asynchronous
 * CPU/GPU compute").
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h] + bias[e]   (fp32 accumulation)
 *   ids[t][j]    = the j-th expert in the order (logit descending, expert index ascending),
 *                  -0.0 and +0.0 being equal
 *   p[t][j]      = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0) over the chosen k (fp32)
 * logits may be NULL (then they live in the workspace). T >= 1. Workspace: MOE_CALL_ROUTE (the logits
 * when logits is NULL and, for T > 16 with few row tiles, the partial sums of the K-split router GEMM,
 * added in a fixed order so that results are deterministic).
 */
moe_status moe_route(const moe_layer_desc* desc, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                     float* logits, int32_t* ids, float* p, void* ws, size_t ws_bytes, void* stream);

/*
 * Grouping of the (token, expert) pairs by expert, so that each chosen expert's weights serve all
 * of its tokens at once (the grouped expert kernels of prompt processing: 648news
 * 07-nano-cuda-moe-qwen38-release, section "speed comparison and accuracy check").
 * Stable counting sort of the pairs q = t*k + j by expert ids[q] (integer, deterministic):
 *   offsets[e] = number of pairs with expert < e (offsets[E] = T*k);
 *   pos(q) = offsets[ids[q]] + number of earlier pairs q' < q with the same expert;
 *   perm[pos(q)] = q, inv[q] = pos(q).
 * A pair whose id lies outside [0, E) is dropped (no slot, inv[q] = -1, offsets[E] counts the
 * kept pairs; perm entries past offsets[E] are left unwritten). Workspace: MOE_CALL_PERMUTE.
 */
moe_status moe_permute(const moe_layer_desc* desc, const int32_t* ids, int32_t T, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* ws, size_t ws_bytes, void* stream);

/*
 * Expert FFNs for a decode step of 1 <= T <= 8 tokens with T k <= 64 pairs (e.g. one token, or a
 * verify pass of a token and its drafts): the selected experts run on the GPU and a
 * token costs the bytes of the experts it reads (648news 07-nano-cuda-moe-qwen38-release, section
 * "asynchronous CPU/GPU compute"; 648news 10-cyber-on-strata-moe-local-inference, section "bitwise
 * validation and speed bottleneck"). Each distinct chosen expert's weights are read once for all
 * tokens that chose it.
 *   y_pairs[q]  = D_e (silu(G_e x_t) * (U_e x_t)), e = ids[q], for every pair q = t*k + j
 *   y_shared[t] = the shared expert on x_t (required iff Is > 0, else ignored)
 * Dequantised weights are exact fp16 values; the dot products accumulate in fp32 over fp16
 * operands: x rounded once to fp16 (at its token scale, see "Activation range"), h as an fp16
 * hi + lo pair (about 22 bits) for one or two tokens and as one fp16 value from three tokens on.
 * Workspace: MOE_CALL_EXPERTS_DECODE.
 * The kernels keep every chosen pair's SwiGLU activations in LDS (160 KB per workgroup):
 * 4 (T k + T) max(I, Is) bytes plus the routing plan and about 4 E bytes must fit; a shape beyond
 * that (or T > 8, or T k > 64) returns MOE_ERR_UNSUPPORTED before anything is enqueued, and so does
 * moe_workspace_size(MOE_CALL_EXPERTS_DECODE).
 */
moe_status moe_experts_decode(const moe_layer_desc* desc, const moe_layer_weights* w, const uint16_t* x,
                              int32_t T, const int32_t* ids, float* y_pairs, float* y_shared, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Expert FFNs for a prefill chunk (any T >= 1; prompts run in 8K-token chunks through GEMMs and
 * grouped expert kernels: 648news 07-nano-cuda-moe-qwen38-release, section "speed comparison and
 * accuracy check"): a grouped GEMM over expert-sorted row tiles
 * (rows in perm order, groups from offsets, as moe_permute returns them), with the shared
 * expert as one more group of all T tokens. Offsets are clamped to [0, T*k] and perm entries
 * outside [0, T*k) read token 0, so inconsistent inputs give wrong rows but no stray access.
 *   y_sorted[i] = expert FFN of pair perm[i] (sorted order), y_shared[t] as above.
 * Operands are fp16 on the matrix cores (x converted from bf16 at its token scale, weights
 * dequantised once to fp16, the SwiGLU activation h kept in fp16 at the token scale squared; see
 * "Activation range") with fp32 accumulation and fp32 outputs at the true scale.
 * Workspace: MOE_CALL_EXPERTS_PREFILL.
 */
moe_status moe_experts_prefill(const moe_layer_desc* desc, const moe_layer_weights* w, const uint16_t* x,
                               int32_t T, const int32_t* offsets, const int32_t* perm, float* y_sorted,
                               float* y_shared, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_experts_prefill with the output rows in fp16 (IEEE binary16 bits, the fp32 row rounded to
 * nearest even, saturating at +-65504): the precision the fused layer keeps between its down GEMM
 * and its combine (half the bytes of the largest stream of the layer; inside the layer the rows
 * stay at the token scale, so they never saturate for ordinary weights). Same kernels, same
 * workspace (MOE_CALL_EXPERTS_PREFILL); y_sorted and y_shared must be 16-byte aligned.
 */
moe_status moe_experts_prefill_f16(const moe_layer_desc* desc, const moe_layer_weights* w, const uint16_t* x,
                                   int32_t T, const int32_t* offsets, const int32_t* perm, uint16_t* y_sorted,
                                   uint16_t* y_shared, void* ws, size_t ws_bytes, void* stream);

/*
 * Weighted combine plus the always-used shared expert (resident beside the router: 648news
 * 07-nano-cuda-moe-qwen38-release, section "asynchronous CPU/GPU compute"), atomic-free and
 * deterministic:
 *   out[t] = sum_{j=0}^{k-1} p[t][j] * y_rows[r(t,j)] + y_shared[t]     (slot order, then shared)
 * with r(t,j) = row_of_pair[t*k+j] (e.g. inv from moe_permute) or t*k+j when row_of_pair is NULL;
 * a row outside [0, T*k) (a dropped pair) contributes nothing. y_shared may be NULL (no shared
 * term). No workspace.
 */
moe_status moe_combine(const moe_layer_desc* desc, int32_t T, const float* p, const float* y_rows,
                       const int32_t* row_of_pair, const float* y_shared, float* out, void* stream);

/*
 * The whole layer: route, permute, experts, combine (the five steps above in one call).
 * T <= decode_max_tokens (default 6; T k <= 64) takes the decode path (three launches: router
 * GEMV; top-k + gate/up; down with the combine fused) when its LDS fits the shape (see
 * moe_experts_decode), else, like larger T, the prefill path (router GEMV up to 16 tokens, GEMM
 * above; top-k, permutation, grouped GEMMs, combine; from 2 to 16 tokens the top-k, the
 * permutation and the x conversion run as one kernel); moe_workspace_size sizes the path that is
 * taken. out [T][H] fp32. logits/ids/p are optional outputs (NULL = kept in the
 * workspace). Workspace: MOE_CALL_LAYER.
 */
moe_status moe_layer(const moe_layer_desc* desc, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                     float* out, float* logits, int32_t* ids, float* p, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * moe_layer for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation, with the workspace taken
 * from a fixed device array inside the library (moe_layer_static_max_bytes() = 16 MiB per GPU, held
 * from load until the process ends) instead of a caller buffer. The caller still passes x, out and
 * the optional logits/ids/p. A shape whose moe_workspace_size(MOE_CALL_LAYER) exceeds the array
 * returns MOE_ERR_UNSUPPORTED before anything is enqueued (every decode shape fits; prefill batches
 * up to a few hundred tokens at H = 2048). Nothing is allocated: the array's device address is
 * looked up once per device, on the first call made with that device current. Every call on a GPU
 * shares that GPU's array, so calls that may overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller; consecutive calls on one stream are safe (the workspace
 * needs no clearing between calls).
 */
moe_status moe_layer_static(const moe_layer_desc* desc, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                            float* out, float* logits, int32_t* ids, float* p, void* stream);

/* Bytes of moe_layer_static's device array (host only). */
size_t moe_layer_static_max_bytes(void);

/*
 * KV cache codec: the same block-32 int8 format as the Q8 weights, for the attention cache (648news
 * 07-nano-cuda-moe-qwen38-release, section "memory hierarchy spanning VRAM and RAM": the KV cache is
 * int8 with one scale per 32 values, and an indexer selects 2048 positions per query). Per block of
 * 32 values of a row, in fp32: m = max |v|, s = fp16(m / 127) rounded to nearest even and
 * saturating at 65504, code = rne(v / s) clamped to [-127, 127], or 0 when s is 0. A NaN value takes
 * no part in m and gets code 0.
 *   src bf16 [rows][D] -> codes int8 [rows][D], scales fp16 bits [rows][D/32]
 * D a multiple of 32, 32 <= D <= 65536; rows >= 0 (0 enqueues nothing). src and codes 16-byte
 * aligned, scales 2-byte aligned. No workspace.
 */
moe_status moe_kv_encode(const uint16_t* src, int32_t rows, int32_t D, int8_t* codes, uint16_t* scales,
                         void* stream);

/*
 * Sparse gather from the int8 cache of n_rows rows: out[j][d] = codes[idx[j]][d] * s(idx[j], d / 32)
 * in fp32 (exact: an int8 times an fp16 fits fp32), for j < n_idx; an index outside [0, n_rows)
 * yields a zero row (no access with it). idx int32 [n_idx] on the device, e.g. the 2048 positions
 * of each of several queries; out fp32 [n_idx][D], 16-byte aligned. No workspace.
 */
moe_status moe_kv_gather(const int8_t* codes, const uint16_t* scales, int32_t n_rows, int32_t D,
                         const int32_t* idx, int32_t n_idx, float* out, void* stream);

/*
 * A copy of the expert codes laid out for the grouped GEMMs' weight loads, made once per set of
 * weights (for example when a model is loaded) and passed as moe_layer_weights.prefill_codes. Each
 * matrix of N rows and K columns (BB = 32, 16 or 8 code bytes per 32-value block for Q8, Q4, Q2) is
 * cut into groups of 32 rows (the last one padded with zero rows) and steps of 64 columns; group r,
 * step s is one piece of 64 BB bytes: block 2s of rows 32r .. 32r + 31 (BB bytes each, in row
 * order), then block 2s + 1 of the same rows (zero bytes past the row's last block). A matrix takes
 * ceil(N / 32) ceil(K / 64) 64 BB bytes, its pieces group-major; the matrices follow one another:
 * the E routed gate matrices (N = I, K = H), the E up matrices, the E down matrices (N = H, K = I),
 * then the shared gate, up and down (N = Is or H, K = H or Is) when shared_inter > 0. The scales of
 * the same matrices follow, in the same order: a matrix's scales in pieces of 32 rows x 8 blocks
 * (512 bytes, row by row, 8 fp16 scales each, zero past the rows or the row's last block), group-
 * major, ceil(N / 32) ceil(K / 256) 512 bytes per matrix. The copy must be made again if the codes
 * or scales change.
 */
/* Bytes of the packed copy of the expert codes (host only; 0 for an invalid descriptor). */
size_t moe_prefill_codes_bytes(const moe_layer_desc* desc);
/* Writes the packed copy of w's expert codes to dst (device, moe_prefill_codes_bytes bytes, 16-byte
 * aligned), stream-ordered. Invalid descriptor or weights, or a NULL or misaligned dst: an error
 * status before anything is enqueued. */
moe_status moe_pack_prefill_codes(const moe_layer_desc* desc, const moe_layer_weights* w, void* dst, void* stream);

/* Bytes of workspace an entry point needs for this shape (host only; no GPU work). */
moe_status moe_workspace_size(const moe_layer_desc* desc, int32_t T, moe_call call, size_t* bytes);

/* Static string for a status code (host only). */
const char* moe_status_string(moe_status status);

/* MOE_ABI_VERSION of the built library (host only). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
