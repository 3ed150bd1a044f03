/*
 * kivi_oracle.h -- plain, slow CPU reference of KIVI-style KV-cache
 * quantization and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library shares
 * no code, header, table or helper with it, and neither includes the other.
 *
 * Source of the arithmetic: the KIVI explainer page ("ICML 2024論文解説: KIVI —
 * チューニング不要のKVキャッシュ2bit非対称量子化"):
 *   - section 量子化アルゴリズム: the quantizer Q, the dequantizer D, and the
 *     per-group scale s = (max - min) / (2^b - 1) and zero-point z = min;
 *   - section Per-Channel量子化（Key Cache）: keys take statistics per channel;
 *   - section Per-Token量子化（Value Cache）: values take statistics per token,
 *     quantized once a group of tokens has accumulated, fp16 until then;
 *   - section 残差バッファ（Residual Buffer）: the most recent tokens stay fp16,
 *     and attention is one softmax over the token-concatenation of the
 *     dequantized part and the fp16 residual, scaled by 1/sqrt(d_k);
 *   - section アルゴリズム (its QuantConfig and quantize functions): defaults
 *     b = 2, group sizes 32, residual 128, and the scale floor of 1e-8.
 *
 * Readings taken where the page leaves a step open (each also listed in the
 * design notes of the repository):
 *   - keys: one (s, z) per channel per block of G consecutive tokens; values:
 *     one (s, z) per token per group of vg consecutive channels;
 *   - the codec runs in IEEE fp32 (round-to-nearest-even division, rintf for
 *     the rounding, no fused multiply-add); s and z are stored as fp32;
 *   - s below 1e-8 (including a constant group) is replaced by 1e-8f;
 *   - z = min + 0.0f, which turns -0 into +0;
 *   - dequantization and attention run in fp64, with no fp16 rounding of the
 *     dequantized values;
 *   - the cache is defined token by token: a ring of R + G fp16 slots, a token
 *     arriving at a full ring first flushes the oldest G tokens, and an explicit
 *     flush quantizes the oldest floor((n_res - R) / G) * G residual tokens.
 */
#ifndef KIVI_ORACLE_H
#define KIVI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE 754 binary16 / bfloat16 bit patterns to float, from the formats' definitions. */
float or_half_to_float(uint16_t h);
float or_bf16_to_float(uint16_t b);
void  or_half_to_float_array(const uint16_t* h, float* out, int64_t n);

/* Quantize one group of n values with b bits: codes[i] in [0, 2^b-1], scale, zero. */
void or_quant_group(const float* x, int n, int bits, uint8_t* codes, float* s, float* z);

/* Pack one row of d codes: word w holds codes [w*per, w*per+per), per = 32/bits,
 * code i of the word at bits [bits*i, bits*i+bits). */
void or_pack_row(const uint8_t* codes, int d, int bits, uint32_t* words);
void or_unpack_row(const uint32_t* words, int d, int bits, uint8_t* codes);
/* or_pack_row over `rows` consecutive rows. */
void or_pack_rows(const uint8_t* codes, int64_t rows, int d, int bits, uint32_t* words);

/* The cache: B sequences x Hkv heads ("units"), each with its full fp16 history. */
typedef struct or_cache or_cache;
/* Key blocks quantized from now on take SQuat-style codes with the per-unit
 * coefficients g ([units][d][d] fp32, copied). */
void or_cache_set_squat(or_cache* c, const float* g);

or_cache* or_cache_new(int batch, int n_kv_heads, int n_q_heads, int head_dim, int bits,
                       int k_block, int v_group, int residual, int max_tokens);
void      or_cache_free(or_cache* c);

/* Append ntok tokens per unit, one token at a time. k, v: fp16 bits [B][Hkv][ntok][d].
 * Returns 0, or -1 when the capacity would be exceeded (nothing appended). */
int     or_append(or_cache* c, const uint16_t* k, const uint16_t* v, int ntok);
/* Explicit flush; returns the number of tokens quantized per unit. */
int64_t or_flush(or_cache* c);
void    or_state(const or_cache* c, int64_t* n_tokens, int64_t* n_quant);

/* Logical quantized contents of one unit (unit = b*Hkv + h):
 *   kcodes [n_q][d], ks/kz [n_q/G][d], vcodes [n_q][d], vs/vz [n_q][d/vg]. */
void or_unit_quantized(const or_cache* c, int unit, uint8_t* kcodes, float* ks, float* kz,
                       uint8_t* vcodes, float* vs, float* vz);
/* Residual tokens [n_q, n_tokens) of one unit, in token order: fp16 bits [n_res][d]. */
void or_unit_residual(const or_cache* c, int unit, uint16_t* kres, uint16_t* vres);

/* Decode attention for every (b, query head): q fp16 or bf16 bits [B][Hq][d];
 * out fp64 [B][Hq][d]. Returns 0, or -1 on an empty cache. */
int or_attend(const or_cache* c, const uint16_t* q, int q_is_bf16, double* out);

/* Number of OpenMP threads or_attend and or_append use (1 without OpenMP). */
int or_num_threads(void);
/* Sets the number of OpenMP threads later calls use (n >= 1). */
void or_set_num_threads(int n);

/* SQuat-style key codes (the SQuat explainer page, section 3 中核となる技術的要素):
 * one key of d fp32 values (widened fp16), coded element by element in channel
 * order with its block's per-channel (s, z); after element c the later
 * elements move by -delta * g[c][j] (fp32 fma), delta = x_c - fma(s_c, code, z_c).
 * g: d x d fp32 row-major (only j > c read). */
void or_squat_token(const float* k, const float* s, const float* z, const float* g, int d, int bits,
                    uint8_t* codes);
/* The walk of or_squat_token along the codes `given`: own[c] its own decision at
 * each element, q[c] its quotient (x_c - z_c) / s_c in fp64. */
void or_squat_replay(const float* k, const float* s, const float* z, const float* g, int d, int bits,
                     const uint8_t* given, uint8_t* own, double* q);

#ifdef __cplusplus
}
#endif

#endif
