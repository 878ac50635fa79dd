/*
 * Oracle of the routed, block-quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded fp64 C. Only tests, the smoke check and the benchmark's CPU-baseline
 * leg load it; the HIP library never does, and this file shares nothing with it.
 *
 * Pages cited (shape and intent only; they print no formula for the layer):
 *   [P1] 648news 07-nano-cuda-moe-qwen38-release: sections "memory hierarchy spanning VRAM and RAM"
 *        (int8 with one scale per 32 values) and "asynchronous CPU/GPU compute" (router and shared
 *        expert resident on the GPU);
 *   [P3] 648news 10-cyber-on-strata-moe-local-inference: section "tiered VRAM/RAM inference"
 *        (8 of 256 experts per token);
 *   [P4] bagrov.by ierarhicheskaya-pamyat-moe-modelej-strata-maya: section "MoE architecture and
 *        hierarchical caching" (about ten experts of 24,576 per token).
 * The five steps (router, top-k with softmax over the chosen k, permutation, block-quantized
 * SwiGLU expert, weighted combine plus shared expert) are written out here as their plain
 * definitions, in fp64.
 *
 * Parity unpinned: nothing (every function is pinned by the CPU tests: hand-computed worked
 * examples, encoder round-trip bounds, invariants, brute force and library reductions).
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ number formats */

/* bf16 is the top half of an fp32: widen exactly. */
double orc_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16(uint16_t bits) {
    int sign = bits >> 15;
    int ex = (bits >> 10) & 31;
    int frac = bits & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (ex == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), ex - 25);    /* (1 + frac/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

static int32_t bits_of(int fmt) { return fmt == ORC_Q8 ? 8 : fmt == ORC_Q4 ? 4 : 2; }

/* Bytes of one packed row of K elements. */
static int64_t row_bytes(int fmt, int32_t K) { return (int64_t)K * bits_of(fmt) / 8; }

/*
 * The level encoded for element kappa of a row:
 *   Q8: the byte as a signed int8;
 *   Q4: element 2i is the low nibble of byte i, 2i+1 the high nibble; two's complement (-8..7);
 *   Q2: element 4i+m is bits 2m..2m+1 of byte i, an unsigned c in 0..3 meaning c - 1.5.
 */
double orc_code_value(int fmt, const uint8_t* row, int32_t kappa) {
    if (fmt == ORC_Q8) return (double)(int8_t)row[kappa];
    if (fmt == ORC_Q4) {
        uint8_t byte = row[kappa / 2];
        int nib = (kappa % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        return (double)(nib >= 8 ? nib - 16 : nib);
    }
    {
        uint8_t byte = row[kappa / 4];
        int c = (byte >> (2 * (kappa % 4))) & 3;
        return (double)c - 1.5;
    }
}

/* Weight [n][kappa] of one matrix: level times the fp16 scale of its 32-element block. */
static double weight(int fmt, const uint8_t* codes, const uint16_t* scales, int32_t K, int32_t n,
                     int32_t kappa) {
    const uint8_t* row = codes + (int64_t)n * row_bytes(fmt, K);
    double s = orc_f16(scales[(int64_t)n * (K / 32) + kappa / 32]);
    return orc_code_value(fmt, row, kappa) * s;
}

void orc_dequant(int fmt, const uint8_t* codes, const uint16_t* scales, int32_t N, int32_t K, double* out) {
    for (int32_t n = 0; n < N; ++n)
        for (int32_t kappa = 0; kappa < K; ++kappa)
            out[(int64_t)n * K + kappa] = weight(fmt, codes, scales, K, n, kappa);
}

/* ------------------------------------------------------------------ step 1: router */

void orc_router(const orc_layer* L, const uint16_t* x, int32_t T, double* logits) {
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < L->E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < L->H; ++h)
                acc += orc_bf16(x[(int64_t)t * L->H + h]) * (double)L->w_router[(int64_t)e * L->H + h];
            logits[(int64_t)t * L->E + e] = acc + (L->bias ? (double)L->bias[e] : 0.0);
        }
}

/* ------------------------------------------------------------------ step 2: top-k + softmax */

/*
 * Slot j holds the j-th expert in the order (logit descending, expert index ascending): repeated
 * selection of the best remaining expert, where a strictly larger logit wins and an equal logit
 * keeps the lower index (the scan is in ascending index). -0.0 and +0.0 compare equal in C.
 * p[j] = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the chosen k only.
 */
int orc_topk_softmax(const double* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, double* p) {
    char* taken = (char*)malloc((size_t)E);
    if (!taken) return -1;
    for (int32_t t = 0; t < T; ++t) {
        const double* l = logits + (int64_t)t * E;
        for (int32_t e = 0; e < E; ++e)
            if (isnan(l[e])) { free(taken); return -1; }
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        double lmax = l[ids[(int64_t)t * k]];
        double denom = 0.0;
        for (int32_t j = 0; j < k; ++j) denom += exp(l[ids[(int64_t)t * k + j]] - lmax);
        for (int32_t j = 0; j < k; ++j) p[(int64_t)t * k + j] = exp(l[ids[(int64_t)t * k + j]] - lmax) / denom;
    }
    free(taken);
    return 0;
}

/* ------------------------------------------------------------------ step 3: permutation */

/*
 * Stable counting sort of the pair ids q = t*k + j by their expert ids[q]:
 * offsets = exclusive prefix sum of the per-expert counts (offsets[E] = T*k);
 * pos(q) = offsets[e] + (number of earlier pairs q' < q with the same expert);
 * perm[pos(q)] = q and inv[q] = pos(q).
 */
void orc_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* offsets, int32_t* perm,
                 int32_t* inv) {
    int64_t P = (int64_t)T * k;
    int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t q = 0; q < P; ++q) offsets[ids[q] + 1] += 1;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int64_t q = 0; q < P; ++q) {
        int32_t e = ids[q];
        int32_t pos = offsets[e] + seen[e];
        seen[e] += 1;
        perm[pos] = (int32_t)q;
        inv[q] = pos;
    }
    free(seen);
}

/* ------------------------------------------------------------------ step 4: SwiGLU expert */

/*
 * g = G x, u = U x (G, U [I][H]); h = silu(g) * u with silu(g) = g / (1 + e^-g); y = D h (D [H][I]).
 * Every weight is its level times its block scale.
 */
void orc_expert(int fmt, int32_t H, int32_t I, const uint8_t* g_codes, const uint16_t* g_scales,
                const uint8_t* u_codes, const uint16_t* u_scales, const uint8_t* d_codes,
                const uint16_t* d_scales, const double* x, double* h_out, double* y) {
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    for (int32_t n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        for (int32_t kappa = 0; kappa < H; ++kappa) {
            g += weight(fmt, g_codes, g_scales, H, n, kappa) * x[kappa];
            u += weight(fmt, u_codes, u_scales, H, n, kappa) * x[kappa];
        }
        h[n] = g / (1.0 + exp(-g)) * u;
        if (h_out) h_out[n] = h[n];
    }
    for (int32_t m = 0; m < H; ++m) {
        double acc = 0.0;
        for (int32_t n = 0; n < I; ++n) acc += weight(fmt, d_codes, d_scales, I, m, n) * h[n];
        y[m] = acc;
    }
    free(h);
}

/* Expert e of a stack: its matrices start e whole matrices into each array. */
void orc_routed_expert(const orc_layer* L, int32_t e, const double* x, double* y) {
    int64_t gu_codes = (int64_t)L->I * row_bytes(L->fmt, L->H), gu_scales = (int64_t)L->I * (L->H / 32);
    int64_t d_codes = (int64_t)L->H * row_bytes(L->fmt, L->I), d_scales = (int64_t)L->H * (L->I / 32);
    orc_expert(L->fmt, L->H, L->I, L->gate.codes + e * gu_codes, L->gate.scales + e * gu_scales,
               L->up.codes + e * gu_codes, L->up.scales + e * gu_scales, L->down.codes + e * d_codes,
               L->down.scales + e * d_scales, x, NULL, y);
}

void orc_shared_expert(const orc_layer* L, const double* x, double* y) {
    orc_expert(L->fmt, L->H, L->Is, L->sh_gate.codes, L->sh_gate.scales, L->sh_up.codes, L->sh_up.scales,
               L->sh_down.codes, L->sh_down.scales, x, NULL, y);
}

/* ------------------------------------------------------------------ steps 1-5 for one token */

/*
 * Y = sum_{j=0}^{k-1} p[j] * y_(ids[j]) (slot order) + y_shared, the shared expert having weight 1
 * and no gate. Without a shared expert (Is == 0) y_shared is 0.
 */
int orc_token(const orc_layer* L, const uint16_t* x_row, const double* logits_in, double* logits,
              int32_t* ids, double* p, double* y_pairs, double* y_shared, double* Y) {
    const int32_t H = L->H, E = L->E, k = L->k;
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* l = (double*)malloc(sizeof(double) * (size_t)E);
    int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* pr = (double*)malloc(sizeof(double) * (size_t)k);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)calloc((size_t)H, sizeof(double));
    int rc = 0;
    for (int32_t h = 0; h < H; ++h) xd[h] = orc_bf16(x_row[h]);
    if (logits_in)
        memcpy(l, logits_in, sizeof(double) * (size_t)E);
    else
        orc_router(L, x_row, 1, l);
    if (logits) memcpy(logits, l, sizeof(double) * (size_t)E);
    if (orc_topk_softmax(l, 1, E, k, id, pr) != 0) { rc = -1; goto done; }
    for (int32_t j = 0; j < k; ++j) {
        orc_routed_expert(L, id[j], xd, y);
        if (y_pairs) memcpy(y_pairs + (int64_t)j * H, y, sizeof(double) * (size_t)H);
        for (int32_t m = 0; m < H; ++m) acc[m] += pr[j] * y[m];
    }
    if (L->Is > 0) {
        orc_shared_expert(L, xd, y);
    } else {
        for (int32_t m = 0; m < H; ++m) y[m] = 0.0;
    }
    if (y_shared) memcpy(y_shared, y, sizeof(double) * (size_t)H);
    for (int32_t m = 0; m < H; ++m) acc[m] += y[m];
    if (ids) memcpy(ids, id, sizeof(int32_t) * (size_t)k);
    if (p) memcpy(p, pr, sizeof(double) * (size_t)k);
    if (Y) memcpy(Y, acc, sizeof(double) * (size_t)H);
done:
    free(xd); free(l); free(id); free(pr); free(y); free(acc);
    return rc;
}

int orc_layer_forward(const orc_layer* L, const uint16_t* x, int32_t T, const double* logits_in,
                      double* logits, int32_t* ids, double* p, double* y_pairs, double* y_shared,
                      double* Y) {
    const int64_t H = L->H, E = L->E, k = L->k;
    for (int32_t t = 0; t < T; ++t) {
        int rc = orc_token(L, x + t * H, logits_in ? logits_in + t * E : NULL, logits ? logits + t * E : NULL,
                           ids ? ids + t * k : NULL, p ? p + t * k : NULL, y_pairs ? y_pairs + t * k * H : NULL,
                           y_shared ? y_shared + t * H : NULL, Y ? Y + t * H : NULL);
        if (rc) return rc;
    }
    return 0;
}

/*
 * Combine alone, on given expert outputs: out[t] = sum_j p[t][j] * y_rows[r(t,j)] (slot order) +
 * y_shared[t], with r(t,j) = row_of_pair[t*k+j], or t*k+j when row_of_pair is NULL; y_shared may be
 * NULL. The same sum orc_token forms from its own expert outputs.
 */
void orc_combine(int32_t T, int32_t k, int32_t H, const double* p, const double* y_rows, const int32_t* row_of_pair,
                 const double* y_shared, double* out) {
    for (int32_t t = 0; t < T; ++t)
        for (int32_t m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int64_t q = (int64_t)t * k + j;
                int64_t r = row_of_pair ? row_of_pair[q] : q;
                acc += p[q] * y_rows[r * H + m];
            }
            out[(int64_t)t * H + m] = acc + (y_shared ? y_shared[(int64_t)t * H + m] : 0.0);
        }
}

/* ------------------------------------------------------------------ brute force */

int orc_dense_masked(const orc_layer* L, const uint16_t* x, int32_t T, double* Y) {
    const int32_t H = L->H, E = L->E, k = L->k;
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* l = (double*)malloc(sizeof(double) * (size_t)E);
    double* soft = (double*)malloc(sizeof(double) * (size_t)E);
    double* m = (double*)malloc(sizeof(double) * (size_t)E);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t* xr = x + (int64_t)t * H;
        for (int32_t h = 0; h < H; ++h) xd[h] = orc_bf16(xr[h]);
        orc_router(L, xr, 1, l);
        /* softmax over all E experts */
        double lmax = l[0], z = 0.0;
        for (int32_t e = 1; e < E; ++e) if (l[e] > lmax) lmax = l[e];
        for (int32_t e = 0; e < E; ++e) { soft[e] = exp(l[e] - lmax); z += soft[e]; }
        for (int32_t e = 0; e < E; ++e) soft[e] /= z;
        /* e is chosen iff fewer than k experts rank ahead of it */
        double kept = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            int32_t ahead = 0;
            for (int32_t f = 0; f < E; ++f)
                if (l[f] > l[e] || (l[f] == l[e] && f < e)) ahead++;
            m[e] = ahead < k ? soft[e] : 0.0;
            kept += m[e];
        }
        double* Yt = Y + (int64_t)t * H;
        for (int32_t h = 0; h < H; ++h) Yt[h] = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            orc_routed_expert(L, e, xd, y);   /* every expert is evaluated, chosen or not */
            for (int32_t h = 0; h < H; ++h) Yt[h] += (m[e] / kept) * y[h];
        }
        if (L->Is > 0) {
            orc_shared_expert(L, xd, y);
            for (int32_t h = 0; h < H; ++h) Yt[h] += y[h];
        }
    }
    free(xd); free(l); free(soft); free(m); free(y);
    return 0;
}

/* ------------------------------------------------------------------ KV cache codec */

/* fp32 -> fp16 bits, round to nearest, ties to even, from the definition: for |q| in
 * [2^e, 2^(e+1)) with e >= -14 the fp16 step is 2^(e-10) (below 2^-14 it is 2^-24), so the
 * result is the nearest multiple of that step (ties to the even multiple); 65520 and above
 * overflow to infinity. q / step is exact in double, nearbyint rounds it in the default mode. */
uint16_t orc_f32_to_f16(float q) {
    double a = fabs((double)q);
    uint16_t sign = (signbit(q) ? 0x8000u : 0u);
    if (isnan(q)) return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e -= 1;          /* guard against log2 rounding */
    if (ldexp(1.0, e + 1) <= a) e += 1;
    if (e < -14) e = -14;                   /* subnormal range: fixed step 2^-24 */
    double step = ldexp(1.0, e - 10);
    double m = nearbyint(a / step);         /* multiple of the step */
    double r = m * step;
    /* encode r: normal if r >= 2^-14 */
    if (r >= ldexp(1.0, -14)) {
        int er = (int)floor(log2(r));
        if (ldexp(1.0, er) > r) er -= 1;
        if (ldexp(1.0, er + 1) <= r) er += 1;
        if (er > 15) return (uint16_t)(sign | 0x7C00u);
        uint16_t frac = (uint16_t)(r / ldexp(1.0, er - 10) - 1024.0);
        return (uint16_t)(sign | ((uint16_t)(er + 15) << 10) | frac);
    }
    return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
}

void orc_kv_encode(const uint16_t* src, int32_t rows, int32_t D, int8_t* codes, uint16_t* scales) {
    for (int32_t r = 0; r < rows; ++r)
        for (int32_t b = 0; b < D / 32; ++b) {
            const uint16_t* v = src + (int64_t)r * D + 32 * b;
            float m = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf((float)orc_bf16(v[i]));   /* bf16 values are exact in fp32 */
                if (a > m) m = a;
            }
            float q = m / 127.0f;
            uint16_t sb = orc_f32_to_f16(q);
            if (sb == 0x7C00u) sb = 0x7BFFu;   /* scale saturates at the largest finite fp16, 65504 */
            float sf = (float)orc_f16(sb);
            scales[(int64_t)r * (D / 32) + b] = sb;
            for (int i = 0; i < 32; ++i) {
                /* a NaN value gets code 0 (it took no part in the maximum above either) */
                const float xv = (float)orc_bf16(v[i]);
                int c = 0;
                if (sf != 0.0f && !isnan(xv)) {
                    float t = rintf(xv / sf);
                    c = t > 127.0f ? 127 : t < -127.0f ? -127 : (int)t;
                }
                codes[(int64_t)r * D + 32 * b + i] = (int8_t)c;
            }
        }
}

void orc_kv_gather(const int8_t* codes, const uint16_t* scales, int32_t n_rows, int32_t D, const int32_t* idx,
                   int32_t n_idx, double* out) {
    for (int32_t j = 0; j < n_idx; ++j) {
        int32_t r = idx[j];
        for (int32_t d = 0; d < D; ++d) {
            double v = 0.0;
            if (r >= 0 && r < n_rows)
                v = (double)codes[(int64_t)r * D + d] * orc_f16(scales[(int64_t)r * (D / 32) + d / 32]);
            out[(int64_t)j * D + d] = v;
        }
    }
}
