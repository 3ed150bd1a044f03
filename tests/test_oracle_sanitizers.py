"""The CPU oracle (oracle/kivi_oracle.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every entry point: groups of
every size the cache uses, packing round trips, caches of several shapes fed
in random chunks with random explicit flushes, the capacity and empty-cache
error paths, attention over the result, and the SQuat-style coder (one key's
walk and its replay, a cache whose key blocks take the walk). Any out-of-bounds access, leak,
signed overflow or misaligned access stops the run."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "kivi_oracle.h"

static unsigned long long st = 88172645463325252ull;
static unsigned rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (unsigned)(st >> 32); }
/* a random finite binary16 bit pattern (exponent field 0..29) */
static uint16_t rnd_half(void) {
    unsigned e = rnd() % 30, f = rnd() % 1024, s = rnd() & 1;
    return (uint16_t)(s << 15 | e << 10 | f);
}

static int run_cache(int B, int Hkv, int Hq, int d, int bits, int R, int T) {
    or_cache* c = or_cache_new(B, Hkv, Hq, d, bits, 32, 32, R, T);
    if (!c) return 10;
    int64_t U = (int64_t)B * Hkv;
    uint16_t* q = malloc(sizeof(uint16_t) * (size_t)(B * Hq * d));
    double* out = malloc(sizeof(double) * (size_t)(B * Hq * d));
    for (int i = 0; i < B * Hq * d; ++i) q[i] = (uint16_t)(rnd_half() & 0x3fff);  /* |q| < 2 */
    if (or_attend(c, q, 0, out) != -1) return 11;  /* empty cache */
    int pos = 0;
    while (pos < T) {
        int n = 1 + (int)(rnd() % 97);
        if (n > T - pos) n = T - pos;
        uint16_t* k = malloc(sizeof(uint16_t) * (size_t)(U * n * d));
        uint16_t* v = malloc(sizeof(uint16_t) * (size_t)(U * n * d));
        for (int64_t i = 0; i < U * n * d; ++i) { k[i] = rnd_half(); v[i] = rnd_half(); }
        if (or_append(c, k, v, n) != 0) return 12;
        free(k);
        free(v);
        pos += n;
        if (rnd() % 3 == 0) or_flush(c);
        if (rnd() % 4 == 0) {
            if (or_attend(c, q, (int)(rnd() & 1), out) != 0) return 13;
            for (int i = 0; i < B * Hq * d; ++i)
                if (!isfinite(out[i])) return 14;
        }
    }
    uint16_t one[1 << 10];
    memset(one, 0, sizeof one);
    if (U * d <= (int64_t)(sizeof one / sizeof one[0]) && or_append(c, one, one, 1) != -1) return 15;  /* full */
    int64_t nt, nq;
    or_state(c, &nt, &nq);
    if (nt != T || nq % 32 != 0 || nq > nt) return 16;
    int ng = d / 32;
    for (int u = 0; u < U; ++u) {
        uint8_t* kc = malloc((size_t)(nq * d) + 1);
        uint8_t* vc = malloc((size_t)(nq * d) + 1);
        float* ks = malloc(sizeof(float) * (size_t)(nq / 32 * d) + 4);
        float* kz = malloc(sizeof(float) * (size_t)(nq / 32 * d) + 4);
        float* vs = malloc(sizeof(float) * (size_t)(nq * ng) + 4);
        float* vz = malloc(sizeof(float) * (size_t)(nq * ng) + 4);
        uint16_t* kr = malloc(sizeof(uint16_t) * (size_t)((nt - nq) * d) + 2);
        uint16_t* vr = malloc(sizeof(uint16_t) * (size_t)((nt - nq) * d) + 2);
        or_unit_quantized(c, u, kc, ks, kz, vc, vs, vz);
        or_unit_residual(c, u, kr, vr);
        for (int64_t i = 0; i < nq * d; ++i)
            if (kc[i] >= (1 << bits) || vc[i] >= (1 << bits)) return 17;
        free(kc); free(vc); free(ks); free(kz); free(vs); free(vz); free(kr); free(vr);
    }
    if (or_attend(c, q, 1, out) != 0) return 18;
    free(q);
    free(out);
    or_cache_free(c);
    return 0;
}

/* the SQuat-style coder: one key walked and replayed along its own codes, and
 * a cache whose key blocks take the walk, fed and read back */
static int run_squat(int d, int bits) {
    float* k = malloc(sizeof(float) * (size_t)d);
    float* s = malloc(sizeof(float) * (size_t)d);
    float* z = malloc(sizeof(float) * (size_t)d);
    float* g = malloc(sizeof(float) * (size_t)d * (size_t)d);
    uint8_t* codes = malloc((size_t)d);
    uint8_t* own = malloc((size_t)d);
    double* qq = malloc(sizeof(double) * (size_t)d);
    for (int c = 0; c < d; ++c) {
        k[c] = or_half_to_float(rnd_half() & 0x43ff);
        s[c] = 0.01f + (float)(rnd() % 1000) / 100.0f;
        z[c] = -(float)(rnd() % 500) / 100.0f;
        for (int j = 0; j < d; ++j) g[c * d + j] = j > c ? ((float)(rnd() % 2001) - 1000.0f) / 10000.0f : 0.0f;
    }
    or_squat_token(k, s, z, g, d, bits, codes);
    or_squat_replay(k, s, z, g, d, bits, codes, own, qq);
    if (memcmp(codes, own, (size_t)d) != 0) return 30;
    for (int c = 0; c < d; ++c)
        if (codes[c] >= (1u << bits) || !isfinite(qq[c])) return 31;
    or_cache* cc = or_cache_new(1, 2, 2, d, bits, 32, 32, 32, 200);
    if (!cc) return 32;
    float* gs = malloc(sizeof(float) * 2 * (size_t)d * (size_t)d);
    for (int u = 0; u < 2; ++u) memcpy(gs + (size_t)u * d * d, g, sizeof(float) * (size_t)d * (size_t)d);
    or_cache_set_squat(cc, gs);
    free(gs);
    uint16_t* kv = malloc(sizeof(uint16_t) * 2 * 150 * (size_t)d);
    uint16_t* vv = malloc(sizeof(uint16_t) * 2 * 150 * (size_t)d);
    for (int i = 0; i < 2 * 150 * d; ++i) { kv[i] = rnd_half(); vv[i] = rnd_half(); }
    if (or_append(cc, kv, vv, 150) != 0) return 33;
    or_flush(cc);
    int64_t nt, nq;
    or_state(cc, &nt, &nq);
    uint8_t* kc = malloc((size_t)nq * d);
    uint8_t* vc = malloc((size_t)nq * d);
    float* ks = malloc(sizeof(float) * (size_t)(nq / 32 + 1) * d);
    float* kz = malloc(sizeof(float) * (size_t)(nq / 32 + 1) * d);
    float* vs = malloc(sizeof(float) * (size_t)nq * (d / 32) + 4);
    float* vz = malloc(sizeof(float) * (size_t)nq * (d / 32) + 4);
    for (int u = 0; u < 2; ++u) or_unit_quantized(cc, u, kc, ks, kz, vc, vs, vz);
    uint16_t q[2 * 256];
    double out[2 * 256];
    for (int i = 0; i < 2 * d; ++i) q[i] = (uint16_t)(rnd_half() & 0x3fff);
    if (or_attend(cc, q, 0, out) != 0) return 34;
    free(kc); free(vc); free(ks); free(kz); free(vs); free(vz); free(kv); free(vv);
    or_cache_free(cc);
    free(k); free(s); free(z); free(g); free(codes); free(own); free(qq);
    return 0;
}

int main(void) {
    /* groups of every size, both widths, with packing round trips */
    for (int trial = 0; trial < 2000; ++trial) {
        int bits = trial % 2 ? 4 : 2, n = 32;
        float x[32];
        uint8_t codes[32], back[32];
        uint32_t words[8];
        for (int i = 0; i < n; ++i) x[i] = or_half_to_float(rnd_half());
        if (trial % 7 == 0) for (int i = 0; i < n; ++i) x[i] = x[0];  /* constant group */
        float s, z;
        or_quant_group(x, n, bits, codes, &s, &z);
        if (!(s >= 1e-8f)) return 1;
        or_pack_row(codes, n, bits, words);
        or_unpack_row(words, n, bits, back);
        if (memcmp(codes, back, (size_t)n) != 0) return 2;
    }
    for (unsigned h = 0; h < 65536; ++h) (void)or_half_to_float((uint16_t)h);
    uint8_t rows[3 * 64];
    uint32_t rw[3 * 8];
    for (int i = 0; i < 3 * 64; ++i) rows[i] = (uint8_t)(rnd() % 4);
    or_pack_rows(rows, 3, 64, 2, rw);
    int rc;
    or_set_num_threads(2);
    if (or_num_threads() < 1) return 40;
    if ((rc = run_squat(64, 2))) return 500 + rc;
    if ((rc = run_squat(128, 4))) return 600 + rc;
    if ((rc = run_cache(2, 2, 4, 64, 2, 32, 300))) return rc;
    if ((rc = run_cache(1, 1, 1, 128, 4, 0, 97))) return 100 + rc;
    if ((rc = run_cache(1, 3, 3, 256, 2, 128, 500))) return 200 + rc;
    if ((rc = run_cache(3, 1, 2, 128, 2, 64, 161))) return 300 + rc;
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.slow
def test_oracle_under_sanitizers(tmp_path):
    src = tmp_path / "driver.c"
    src.write_text(DRIVER)
    exe = tmp_path / "oracle_san"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", ORACLE,
                           os.path.join(ORACLE, "kivi_oracle.c"), str(src), "-o", str(exe), "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip() == "ok"
