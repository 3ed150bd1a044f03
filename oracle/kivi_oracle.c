/*
 * kivi_oracle.c -- plain, slow CPU reference of KIVI-style KV-cache
 * quantization and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Build: gcc -std=c11 -O2 -fno-fast-math -ffp-contract=off -fopenmp -fPIC -shared
 * (the codec is specified in IEEE fp32 without contraction, so the flags matter).
 *
 * Every function below follows a section of the KIVI explainer page
 * ("ICML 2024論文解説: KIVI — チューニング不要のKVキャッシュ2bit非対称量子化");
 * the section is named at each function. The readings taken where the page is
 * open are listed in kivi_oracle.h.
 */
#include "kivi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal, value = fraction * 2^-24;
 * exponent 31 -> inf / nan; otherwise value = (1024 + fraction) * 2^(exponent - 25). */
float or_half_to_float(uint16_t h) {
    unsigned sign = (h >> 15) & 1u;
    unsigned expo = (h >> 10) & 31u;
    unsigned frac = h & 1023u;
    float mag;
    if (expo == 0)
        mag = ldexpf((float)frac, -24);
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024u + frac), (int)expo - 25);
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of a binary32. */
float or_bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void or_half_to_float_array(const uint16_t* h, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_half_to_float(h[i]);
}

/* ---------------------------------------------------------------- codec */

/* Section 量子化アルゴリズム: Q(X) = clamp(round((X - z) / s), 0, 2^b - 1) with
 * s = (max(X_g) - min(X_g)) / (2^b - 1) and z = min(X_g) over the group X_g.
 * Section アルゴリズム (quantize functions): s is floored at 1e-8, and the
 * rounding is applied before the clamp. All steps in fp32. */
void or_quant_group(const float* x, int n, int bits, uint8_t* codes, float* s_out, float* z_out) {
    const float qmax = (float)((1 << bits) - 1);
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    float s = (mx - mn) / qmax;
    if (!(s >= 1e-8f)) s = 1e-8f;
    float z = mn + 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = (x[i] - z) / s;
        float r = rintf(t); /* round half to even in the default environment */
        if (r < 0.0f) r = 0.0f;
        if (r > qmax) r = qmax;
        codes[i] = (uint8_t)r;
    }
    *s_out = s;
    *z_out = z;
}

/* Section 実装のポイント (bit operations on the 2-bit codes): 32/b codes per
 * 32-bit word, code i of a word at bits [b*i, b*i + b). */
void or_pack_row(const uint8_t* codes, int d, int bits, uint32_t* words) {
    int per = 32 / bits;
    for (int w = 0; w < d / per; ++w) {
        uint32_t word = 0;
        for (int i = 0; i < per; ++i) word |= (uint32_t)codes[w * per + i] << (bits * i);
        words[w] = word;
    }
}

void or_pack_rows(const uint8_t* codes, int64_t rows, int d, int bits, uint32_t* words) {
    for (int64_t r = 0; r < rows; ++r) or_pack_row(codes + r * d, d, bits, words + r * (d * bits / 32));
}

void or_unpack_row(const uint32_t* words, int d, int bits, uint8_t* codes) {
    int per = 32 / bits;
    uint32_t mask = (1u << bits) - 1u;
    for (int c = 0; c < d; ++c) codes[c] = (uint8_t)((words[c / per] >> (bits * (c % per))) & mask);
}

/* ---------------------------------------------------------------- cache */

struct or_cache {
    int B, Hkv, Hq, d, bits, G, vg, R, max_tokens;
    int64_t n_tokens, n_q;
    /* per unit, full history: [unit][max_tokens][d] fp16 bits */
    uint16_t *k_hist, *v_hist;
    /* per unit, quantized part: codes [unit][max_tokens][d], K stats [unit][max_blocks][d],
     * V stats [unit][max_tokens][d/vg] */
    uint8_t *k_codes, *v_codes;
    float *k_s, *k_z, *v_s, *v_z;
    /* SQuat-style key coder: per unit d x d update coefficients, or NULL */
    float* squat_g;
};

static int64_t units(const or_cache* c) { return (int64_t)c->B * c->Hkv; }
static int64_t max_blocks(const or_cache* c) { return c->max_tokens / c->G; }

or_cache* or_cache_new(int batch, int n_kv_heads, int n_q_heads, int head_dim, int bits,
                       int k_block, int v_group, int residual, int max_tokens) {
    or_cache* c = (or_cache*)calloc(1, sizeof *c);
    if (!c) return NULL;
    c->B = batch; c->Hkv = n_kv_heads; c->Hq = n_q_heads; c->d = head_dim; c->bits = bits;
    c->G = k_block; c->vg = v_group; c->R = residual; c->max_tokens = max_tokens;
    int64_t U = units(c), T = max_tokens, d = head_dim;
    c->k_hist = (uint16_t*)calloc((size_t)(U * T * d), sizeof(uint16_t));
    c->v_hist = (uint16_t*)calloc((size_t)(U * T * d), sizeof(uint16_t));
    c->k_codes = (uint8_t*)calloc((size_t)(U * T * d), 1);
    c->v_codes = (uint8_t*)calloc((size_t)(U * T * d), 1);
    c->k_s = (float*)calloc((size_t)(U * max_blocks(c) * d) + 1, sizeof(float));
    c->k_z = (float*)calloc((size_t)(U * max_blocks(c) * d) + 1, sizeof(float));
    c->v_s = (float*)calloc((size_t)(U * T * (d / v_group)) + 1, sizeof(float));
    c->v_z = (float*)calloc((size_t)(U * T * (d / v_group)) + 1, sizeof(float));
    if (!c->k_hist || !c->v_hist || !c->k_codes || !c->v_codes || !c->k_s || !c->k_z ||
        !c->v_s || !c->v_z) {
        or_cache_free(c);
        return NULL;
    }
    return c;
}

void or_cache_free(or_cache* c) {
    if (!c) return;
    free(c->k_hist); free(c->v_hist); free(c->k_codes); free(c->v_codes);
    free(c->k_s); free(c->k_z); free(c->v_s); free(c->v_z);
    free(c->squat_g);
    free(c);
}

/* Section Per-Channel量子化（Key Cache）: key statistics per channel; here over
 * the G tokens of key block j (tokens [jG, jG+G)). */
static void quantize_key_block(or_cache* c, int64_t u, int64_t j) {
    int d = c->d, G = c->G;
    float* x = (float*)malloc(sizeof(float) * (size_t)G);
    uint8_t* q = (uint8_t*)malloc((size_t)G);
    for (int ch = 0; ch < d; ++ch) {
        for (int t = 0; t < G; ++t)
            x[t] = or_half_to_float(c->k_hist[(u * c->max_tokens + j * G + t) * d + ch]);
        float s, z;
        or_quant_group(x, G, c->bits, q, &s, &z);
        for (int t = 0; t < G; ++t) c->k_codes[(u * c->max_tokens + j * G + t) * d + ch] = q[t];
        c->k_s[(u * max_blocks(c) + j) * d + ch] = s;
        c->k_z[(u * max_blocks(c) + j) * d + ch] = z;
    }
    free(x);
    free(q);
    if (c->squat_g) {
        /* SQuat-style codes of the block's tokens, with the statistics just taken */
        float* kf = (float*)malloc(sizeof(float) * (size_t)d);
        for (int t = 0; t < G; ++t) {
            const int64_t tok = j * G + t;
            for (int ch = 0; ch < d; ++ch) kf[ch] = or_half_to_float(c->k_hist[(u * c->max_tokens + tok) * d + ch]);
            or_squat_token(kf, &c->k_s[(u * max_blocks(c) + j) * d], &c->k_z[(u * max_blocks(c) + j) * d],
                           &c->squat_g[(size_t)u * d * d], d, c->bits, &c->k_codes[(u * c->max_tokens + tok) * d]);
        }
        free(kf);
    }
}

/* Section Per-Token量子化（Value Cache）: value statistics per token; here over
 * each group of vg consecutive channels of token t. */
static void quantize_value_token(or_cache* c, int64_t u, int64_t t) {
    int d = c->d, vg = c->vg, ng = d / vg;
    float* x = (float*)malloc(sizeof(float) * (size_t)vg);
    for (int g = 0; g < ng; ++g) {
        for (int i = 0; i < vg; ++i)
            x[i] = or_half_to_float(c->v_hist[(u * c->max_tokens + t) * d + g * vg + i]);
        float s, z;
        or_quant_group(x, vg, c->bits, &c->v_codes[(u * c->max_tokens + t) * d + g * vg], &s, &z);
        c->v_s[(u * c->max_tokens + t) * ng + g] = s;
        c->v_z[(u * c->max_tokens + t) * ng + g] = z;
    }
    free(x);
}

/* Move the oldest k residual tokens (k a multiple of G) into the quantized part. */
static void quantize_oldest(or_cache* c, int64_t k) {
    int64_t U = units(c);
    int64_t j0 = c->n_q / c->G, j1 = (c->n_q + k) / c->G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < U; ++u) {
        for (int64_t j = j0; j < j1; ++j) quantize_key_block(c, u, j);
        for (int64_t t = c->n_q; t < c->n_q + k; ++t) quantize_value_token(c, u, t);
    }
    c->n_q += k;
}

/* Section 残差バッファ（Residual Buffer）and Per-Token量子化: the newest tokens
 * stay fp16; a group of G tokens is quantized once it is no longer among the
 * R most recent. Flush quantizes every whole group of G residual tokens that
 * lies beyond the newest R. */
static int64_t flushable(const or_cache* c) {
    int64_t n_res = c->n_tokens - c->n_q;
    if (n_res < c->R) return 0;
    return ((n_res - c->R) / c->G) * c->G;
}

int64_t or_flush(or_cache* c) {
    int64_t k = flushable(c);
    if (k > 0) quantize_oldest(c, k);
    return k;
}

int or_append(or_cache* c, const uint16_t* k, const uint16_t* v, int ntok) {
    if (ntok < 0 || c->n_tokens + ntok > c->max_tokens) return -1;
    int64_t U = units(c), d = c->d, C = (int64_t)c->R + c->G;
    for (int i = 0; i < ntok; ++i) {
        /* a token arriving at a full ring first makes room */
        if (c->n_tokens - c->n_q == C) or_flush(c);
        for (int64_t u = 0; u < U; ++u) {
            memcpy(&c->k_hist[(u * c->max_tokens + c->n_tokens) * d], &k[(u * ntok + i) * d],
                   sizeof(uint16_t) * (size_t)d);
            memcpy(&c->v_hist[(u * c->max_tokens + c->n_tokens) * d], &v[(u * ntok + i) * d],
                   sizeof(uint16_t) * (size_t)d);
        }
        c->n_tokens += 1;
    }
    return 0;
}

void or_state(const or_cache* c, int64_t* n_tokens, int64_t* n_quant) {
    *n_tokens = c->n_tokens;
    *n_quant = c->n_q;
}

void or_unit_quantized(const or_cache* c, int unit, uint8_t* kcodes, float* ks, float* kz,
                       uint8_t* vcodes, float* vs, float* vz) {
    int64_t d = c->d, nq = c->n_q, ng = c->d / c->vg, nb = c->n_q / c->G, u = unit;
    memcpy(kcodes, &c->k_codes[u * c->max_tokens * d], (size_t)(nq * d));
    memcpy(vcodes, &c->v_codes[u * c->max_tokens * d], (size_t)(nq * d));
    memcpy(ks, &c->k_s[u * max_blocks(c) * d], sizeof(float) * (size_t)(nb * d));
    memcpy(kz, &c->k_z[u * max_blocks(c) * d], sizeof(float) * (size_t)(nb * d));
    memcpy(vs, &c->v_s[u * c->max_tokens * ng], sizeof(float) * (size_t)(nq * ng));
    memcpy(vz, &c->v_z[u * c->max_tokens * ng], sizeof(float) * (size_t)(nq * ng));
}

void or_unit_residual(const or_cache* c, int unit, uint16_t* kres, uint16_t* vres) {
    int64_t d = c->d, u = unit, n_res = c->n_tokens - c->n_q;
    memcpy(kres, &c->k_hist[(u * c->max_tokens + c->n_q) * d], sizeof(uint16_t) * (size_t)(n_res * d));
    memcpy(vres, &c->v_hist[(u * c->max_tokens + c->n_q) * d], sizeof(uint16_t) * (size_t)(n_res * d));
}

/* ---------------------------------------------------------------- attention */

/* Section 量子化アルゴリズム: D(X^) = s * X^ + z, here in fp64. */
static double dequant(double s, double z, uint8_t code) { return s * (double)code + z; }

/* Section 残差バッファ（Residual Buffer）: attention over [D(K_quant); K_res] and
 * [D(V_quant); V_res] concatenated along the tokens, softmax of q.k^T / sqrt(d_k).
 * Query head i reads KV head i / (Hq / Hkv). Plain two-pass softmax in fp64. */
int or_attend(const or_cache* c, const uint16_t* q, int q_is_bf16, double* out) {
    if (c->n_tokens == 0) return -1;
    const int64_t d = c->d, T = c->n_tokens, nq = c->n_q, ng = c->d / c->vg;
    const int group = c->Hq / c->Hkv;
    const int64_t rows = (int64_t)c->B * c->Hq;
#pragma omp parallel
    {
        double* kd = (double*)malloc(sizeof(double) * (size_t)d);
        double* qd = (double*)malloc(sizeof(double) * (size_t)d);
        double* score = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 1)
        for (int64_t row = 0; row < rows; ++row) {
            int64_t b = row / c->Hq, i = row % c->Hq, h = i / group;
            int64_t u = b * c->Hkv + h;
            for (int64_t ch = 0; ch < d; ++ch) {
                uint16_t bitsq = q[row * d + ch];
                qd[ch] = q_is_bf16 ? (double)or_bf16_to_float(bitsq) : (double)or_half_to_float(bitsq);
            }
            const double inv_sqrt_d = 1.0 / sqrt((double)d);
            double m = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                for (int64_t ch = 0; ch < d; ++ch) {
                    if (t < nq) {
                        int64_t j = t / c->G;
                        kd[ch] = dequant(c->k_s[(u * max_blocks(c) + j) * d + ch],
                                         c->k_z[(u * max_blocks(c) + j) * d + ch],
                                         c->k_codes[(u * c->max_tokens + t) * d + ch]);
                    } else {
                        kd[ch] = (double)or_half_to_float(c->k_hist[(u * c->max_tokens + t) * d + ch]);
                    }
                }
                double dot = 0.0;
                for (int64_t ch = 0; ch < d; ++ch) dot += qd[ch] * kd[ch];
                score[t] = dot * inv_sqrt_d;
                if (score[t] > m) m = score[t];
            }
            double denom = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                score[t] = exp(score[t] - m);
                denom += score[t];
            }
            double* o = &out[row * d];
            for (int64_t ch = 0; ch < d; ++ch) o[ch] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                for (int64_t ch = 0; ch < d; ++ch) {
                    double vv;
                    if (t < nq) {
                        int64_t g = ch / c->vg;
                        vv = dequant(c->v_s[(u * c->max_tokens + t) * ng + g],
                                     c->v_z[(u * c->max_tokens + t) * ng + g],
                                     c->v_codes[(u * c->max_tokens + t) * d + ch]);
                    } else {
                        vv = (double)or_half_to_float(c->v_hist[(u * c->max_tokens + t) * d + ch]);
                    }
                    o[ch] += score[t] * vv;
                }
            }
            for (int64_t ch = 0; ch < d; ++ch) o[ch] /= denom;
        }
        free(kd);
        free(qd);
        free(score);
    }
    return 0;
}

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- SQuat-style keys */

/* The SQuat explainer page (aibr.jp, "SQuat": KV cache quantization whose
 * error is kept orthogonal to a query subspace), section 3 中核となる技術的要素:
 * a key is quantized element by element, and after each element the elements
 * not yet quantized are corrected by the closed-form optimal update, so that
 * the error stays (as far as the remaining elements allow) orthogonal to the
 * query subspace; scales and zero points are stored as in plain low-bit
 * quantization.
 *
 * Reading taken here (the page gives no formulas): element c of a key, in
 * channel order, is coded with the KIVI group (s_c, z_c) of its channel and
 * block (section 量子化アルゴリズム of the KIVI page); with delta = x_c -
 * D(code), D(code) = fma(s_c, code, z_c) in fp32, every later element j > c
 * becomes x_j = fma(-delta, g[c][j], x_j) in fp32, where g (d x d, fp32, only
 * j > c used) are the update coefficients of the quadratic objective
 * ||U^T e||^2 + lambda ||e||^2 (U: the query subspace basis), computed by the
 * caller. The code of an element is decided exactly as in or_quant_group:
 * clamp(rint((x - z) / s), 0, 2^b - 1) in fp32. */
static uint8_t squat_code(float x, float s, float z, float qmax) {
    float r = rintf((x - z) / s);
    if (r < 0.0f) r = 0.0f;
    if (r > qmax) r = qmax;
    return (uint8_t)r;
}

void or_squat_token(const float* k, const float* s, const float* z, const float* g, int d, int bits,
                    uint8_t* codes) {
    const float qmax = (float)((1 << bits) - 1);
    float* x = (float*)malloc(sizeof(float) * (size_t)d);
    memcpy(x, k, sizeof(float) * (size_t)d);
    for (int c = 0; c < d; ++c) {
        codes[c] = squat_code(x[c], s[c], z[c], qmax);
        const float delta = x[c] - fmaf(s[c], (float)codes[c], z[c]);
        for (int j = c + 1; j < d; ++j) x[j] = fmaf(-delta, g[(size_t)c * d + j], x[j]);
    }
    free(x);
}

/* The same walk, but following the codes `given` (e.g. another
 * implementation's) instead of its own decisions. For each element it writes
 * the quotient (x_c - z_c) / s_c of its own trajectory (in fp64, from the fp32
 * x_c) to q[c], and its own fp32 decision to own[c]; the caller judges a
 * given code that differs from `own` by the quotient's distance to the
 * rounding boundary between the two. */
void or_squat_replay(const float* k, const float* s, const float* z, const float* g, int d, int bits,
                     const uint8_t* given, uint8_t* own, double* q) {
    const float qmax = (float)((1 << bits) - 1);
    float* x = (float*)malloc(sizeof(float) * (size_t)d);
    memcpy(x, k, sizeof(float) * (size_t)d);
    for (int c = 0; c < d; ++c) {
        own[c] = squat_code(x[c], s[c], z[c], qmax);
        q[c] = ((double)x[c] - (double)z[c]) / (double)s[c];
        const float delta = x[c] - fmaf(s[c], (float)given[c], z[c]);
        for (int j = c + 1; j < d; ++j) x[j] = fmaf(-delta, g[(size_t)c * d + j], x[j]);
    }
    free(x);
}

/* Key coder of the cache: with per-unit coefficients set (or_cache_set_squat),
 * every key block quantized afterwards takes its channel statistics as
 * before and its codes token by token from or_squat_token. */
void or_cache_set_squat(or_cache* c, const float* g) {
    const size_t n = (size_t)(c->B * c->Hkv) * (size_t)c->d * (size_t)c->d;
    if (!c->squat_g) c->squat_g = (float*)malloc(sizeof(float) * n);
    memcpy(c->squat_g, g, sizeof(float) * n);
}

/* Threads the OpenMP loops above use from now on (n >= 1). */
void or_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
