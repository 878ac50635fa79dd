/*
 * Seeded synthetic inputs for the routed, block-quantized MoE expert layer.
 *
 * This module is shared by the tests, the benchmark and the oracle's callers. It holds none of the
 * layer's own arithmetic (no routing, no softmax, no dequantisation, no SwiGLU, no combine). It
 * only provides:
 *   - keyed random streams: SplitMix64 (Steele, Lea & Flood 2014) to derive a key per tensor and
 *     to seed xoshiro256** (Blackman & Vigna 2018);
 *   - standard normals by the Marsaglia polar method (Marsaglia & Bray 1964), drawn in fp64;
 *   - a seeded Fisher-Yates permutation and the Zipf popularity bias b_e = -alpha * ln(rank_e)
 *     that skews the routing, as the pages describe for expert popularity (cache hit rates that
 *     jump with an expert profile, 648news "cyber-on-strata" article, section on fork history
 *     and memory parameters);
 *   - round-to-nearest-even conversion fp32 -> bf16 and fp32 -> fp16 (bit manipulation);
 *   - the data-preparation encoder that turns fp32 weights into block-32 codes with one fp16
 *     scale per 32 consecutive values along K (int8 with one scale per 32 values is the block
 *     shape the pages give for their int8 KV cache, 648news "nano-cuda-moe" article, section on
 *     the VRAM/RAM memory hierarchy).
 *
 * Formats (codes row-major [rows][K], K contiguous; scales [rows][K/32] fp16 bits):
 *   Q8_B32 (fmt 0): one int8 per byte, qmax 127, code = clamp(rne(w/s), -127, 127).
 *   Q4_B32 (fmt 1): two's-complement nibble, element 2i in the low nibble of byte i,
 *                   qmax 7, code = clamp(rne(w/s), -8, 7).
 *   Q2_B32 (fmt 2): unsigned c in 0..3, element 4i+m in bits 2m..2m+1 of byte i, value c-1.5,
 *                   qmax 1.5, c = clamp(rne(w/s + 1.5), 0, 3).
 *   s = fp16_rne(max|w| / qmax) computed in fp32; when s is 0 every code encodes 0
 *   (Q2: c = 2, the level closest to zero from above).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- random streams */

static inline uint64_t splitmix64_next(uint64_t* s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Derive a 64-bit key from a seed and four labels (config, layer, tensor, expert). */
uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    uint64_t s = seed;
    uint64_t h = splitmix64_next(&s);
    uint64_t labels[4] = {a, b, c, d};
    for (int i = 0; i < 4; ++i) {
        s = h ^ (labels[i] + 0x632BE59BD9B4E019ull * (uint64_t)(i + 1));
        h = splitmix64_next(&s);
    }
    return h;
}

typedef struct { uint64_t s[4]; } xoshiro256;

static inline uint64_t rotl64(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static void xo_seed(xoshiro256* r, uint64_t key) {
    uint64_t s = key;
    for (int i = 0; i < 4; ++i) r->s[i] = splitmix64_next(&s);
}

static inline uint64_t xo_next(xoshiro256* r) {
    uint64_t* s = r->s;
    const uint64_t result = rotl64(s[1] * 5, 7) * 9;
    const uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl64(s[3], 45);
    return result;
}

/* Uniform double in (-1, 1) from the top 53 bits. */
static inline double xo_sym_uniform(xoshiro256* r) {
    return (double)(int64_t)(xo_next(r) >> 10) * 0x1p-53 - 1.0;
}

/* Marsaglia polar method: two independent N(0,1) per accepted pair. */
typedef struct { xoshiro256 r; int have; double spare; } normal_stream;

static void ns_init(normal_stream* ns, uint64_t key) { xo_seed(&ns->r, key); ns->have = 0; ns->spare = 0.0; }

static double ns_next(normal_stream* ns) {
    if (ns->have) { ns->have = 0; return ns->spare; }
    double u, v, q;
    do {
        u = xo_sym_uniform(&ns->r);
        v = xo_sym_uniform(&ns->r);
        q = u * u + v * v;
    } while (q >= 1.0 || q == 0.0);
    double f = sqrt(-2.0 * log(q) / q);
    ns->spare = v * f;
    ns->have = 1;
    return u * f;
}

/* ---------------------------------------------------------------- rounding helpers */

static inline uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

uint16_t synth_f32_to_bf16(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

uint16_t synth_f32_to_f16(float f) {
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t absu = u & 0x7FFFFFFFu;
    if (absu >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (absu > 0x7F800000u ? 0x200u : 0u));
    int e = (int)(absu >> 23) - 127;          /* unbiased exponent */
    uint32_t m = (absu & 0x007FFFFFu) | 0x00800000u;
    if (absu < 0x00800000u) return sign;       /* fp32 subnormals are far below fp16's range */
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    if (e >= -14) {
        /* normal fp16: keep 10 fraction bits out of 23 */
        uint32_t mant = m >> 13, rem = m & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (mant & 1u))) mant++;
        uint32_t ex = (uint32_t)(e + 15);
        if (mant == 0x800u) { mant = 0x400u; ex++; }
        if (ex >= 31) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | (ex << 10) | (mant & 0x3FFu));
    }
    /* subnormal fp16: value = mant * 2^-24 */
    int shift = 13 + (-14 - e);
    if (shift > 24) return sign;
    uint32_t mant = m >> shift, rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (mant & 1u))) mant++;
    return (uint16_t)(sign | mant); /* a carry into bit 10 yields the smallest normal, as it should */
}

static float f16_bits_to_f32(uint16_t h) {
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t ex = (h >> 10) & 31u, man = h & 1023u;
    if (ex == 0) {
        float v = (float)man * 0x1p-24f;
        return sign ? -v : v;
    }
    if (ex == 31) return bits_f32(sign | 0x7F800000u | (man << 13));
    return bits_f32(sign | ((ex + 112u) << 23) | (man << 13));
}

/* ---------------------------------------------------------------- draws */

void synth_normal_f32(uint64_t key, double sigma, int64_t n, float* out) {
    normal_stream ns;
    ns_init(&ns, key);
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * ns_next(&ns));
}

void synth_normal_bf16(uint64_t key, double sigma, int64_t n, uint16_t* out) {
    normal_stream ns;
    ns_init(&ns, key);
    for (int64_t i = 0; i < n; ++i) out[i] = synth_f32_to_bf16((float)(sigma * ns_next(&ns)));
}

/* Fisher-Yates shuffle of 0..n-1 (multiply-shift bounded draw). */
void synth_permutation(uint64_t key, int32_t n, int32_t* out) {
    xoshiro256 r;
    xo_seed(&r, key);
    for (int32_t i = 0; i < n; ++i) out[i] = i;
    for (int32_t i = n - 1; i > 0; --i) {
        uint64_t j = (uint64_t)(((unsigned __int128)xo_next(&r) * (uint64_t)(i + 1)) >> 64);
        int32_t t = out[i]; out[i] = out[j]; out[j] = t;
    }
}

/* Zipf popularity bias: expert e has rank 1 + pi(e); b_e = -alpha * ln(rank_e), fp64 -> fp32. */
void synth_zipf_bias(uint64_t key, int32_t n, double alpha, float* out, int32_t* rank_out) {
    int32_t perm[4096];
    if (n > 4096) return;
    synth_permutation(key, n, perm);
    for (int32_t e = 0; e < n; ++e) {
        out[e] = (float)(-alpha * log((double)(1 + perm[e])));
        if (rank_out) rank_out[e] = 1 + perm[e];
    }
}

/* ---------------------------------------------------------------- block-32 encoder */

static int fmt_bits(int fmt) { return fmt == 0 ? 8 : fmt == 1 ? 4 : fmt == 2 ? 2 : 0; }

/* Encode `rows` rows of K fp32 weights. Returns 0 on success, -1 on a bad argument. */
int synth_quantize_rows(int fmt, const float* w, int64_t rows, int32_t K, uint8_t* codes, uint16_t* scales) {
    int bits = fmt_bits(fmt);
    if (!bits || K <= 0 || K % 32 != 0) return -1;
    const float qmax = fmt == 0 ? 127.0f : fmt == 1 ? 7.0f : 1.5f;
    const int64_t row_bytes = (int64_t)K * bits / 8;
    for (int64_t r = 0; r < rows; ++r) {
        const float* wr = w + r * K;
        uint8_t* cr = codes + r * row_bytes;
        memset(cr, 0, (size_t)row_bytes);
        for (int32_t b = 0; b < K / 32; ++b) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) { float a = fabsf(wr[b * 32 + i]); if (a > amax) amax = a; }
            uint16_t s16 = synth_f32_to_f16(amax / qmax);
            scales[r * (K / 32) + b] = s16;
            float s = f16_bits_to_f32(s16);
            for (int i = 0; i < 32; ++i) {
                int kappa = b * 32 + i;
                float v = wr[kappa];
                int q;
                if (fmt == 2) {
                    q = (s == 0.0f) ? 2 : (int)rintf(v / s + 1.5f);
                    if (q < 0) q = 0;
                    if (q > 3) q = 3;
                    cr[kappa / 4] |= (uint8_t)(q << (2 * (kappa % 4)));
                } else {
                    q = (s == 0.0f) ? 0 : (int)rintf(v / s);
                    int lo = fmt == 0 ? -127 : -8, hi = fmt == 0 ? 127 : 7;
                    if (q < lo) q = lo;
                    if (q > hi) q = hi;
                    if (fmt == 0) cr[kappa] = (uint8_t)(int8_t)q;
                    else cr[kappa / 2] |= (uint8_t)((q & 15) << (4 * (kappa % 2)));
                }
            }
        }
    }
    return 0;
}

/*
 * A stack of E expert matrices [N][K], weights N(0, sigma^2) drawn per expert from key
 * synth_key(key, e, ...) so that any expert can be regenerated on its own, then encoded.
 * Experts are independent, so threads only change the speed, never the bytes.
 */
int synth_expert_stack(int fmt, uint64_t key, int32_t E, int32_t N, int32_t K, double sigma,
                       uint8_t* codes, uint16_t* scales, int nthreads) {
    int bits = fmt_bits(fmt);
    if (!bits || K % 32 != 0 || E <= 0 || N <= 0) return -1;
    const int64_t per_codes = (int64_t)N * K * bits / 8;
    const int64_t per_scales = (int64_t)N * (K / 32);
    int rc = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : rc)
    for (int32_t e = 0; e < E; ++e) {
        float* row = (float*)malloc(sizeof(float) * (size_t)K);
        if (!row) { rc |= 1; continue; }
        normal_stream ns;
        ns_init(&ns, synth_key(key, (uint64_t)e, 0x5EED, 0, 0));
        for (int32_t n = 0; n < N; ++n) {
            for (int32_t k = 0; k < K; ++k) row[k] = (float)(sigma * ns_next(&ns));
            rc |= synth_quantize_rows(fmt, row, 1, K, codes + e * per_codes + (int64_t)n * K * bits / 8,
                                      scales + e * per_scales + (int64_t)n * (K / 32)) != 0;
        }
        free(row);
    }
    return rc ? -1 : 0;
}

/* The same draw as synth_expert_stack for a single expert, without encoding (fp32 weights). */
void synth_expert_weights_f32(uint64_t key, int32_t e, int32_t N, int32_t K, double sigma, float* out) {
    synth_normal_f32(synth_key(key, (uint64_t)e, 0x5EED, 0, 0), sigma, (int64_t)N * K, out);
}
