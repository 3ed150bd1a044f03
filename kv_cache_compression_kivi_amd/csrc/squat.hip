// squat.hip -- gfx950 kernels of the SQuat-style key coder: the query
// subspace and update coefficients of each unit, and the element-by-element
// key codes.
//
// The SQuat explainer page (aibr.jp, "SQuat"), section 3 中核となる技術的要素:
// the query subspace is spanned by the principal directions of past queries;
// keys are quantized element by element, and after each element the elements
// not yet quantized take the closed-form optimal correction, which keeps the
// error (as far as the remaining elements allow) orthogonal to the subspace;
// scales and zero points are stored as in plain low-bit quantization.
//
// Reading taken (the page gives the steps in prose only):
//   - subspace: the r eigenvectors of C = sum_q q q^T (the queries of the
//     query heads that read the KV head) with the largest eigenvalues;
//   - objective of a key's error e: ||U^T e||^2 + lambda ||e||^2 (U the
//     subspace basis). After fixing element c with error delta, the optimal
//     move of element j > c is -delta * g[c][j], g[c][j] = T[c][j] / T[c][c],
//     T the upper Cholesky factor of (U U^T + lambda I)^-1
//     = (1/lambda) I - (1/lambda - 1/(1 + lambda)) U U^T;
//   - the codes: channel order, each element with its block's KIVI (s_c, z_c)
//     (KIVI page, section 量子化アルゴリズム): code = clamp(rint((x - z) / s),
//     0, 2^b - 1) in IEEE fp32, delta = x - fma(s, code, z), and
//     x_j = fma(-delta, g[c][j], x_j).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "launch.hpp"

namespace kivi {
namespace {

constexpr int kG = 32;  // tokens per key block

// Unit u's d x d fp32 matrix in the coder's region (the Gram matrix until the
// factor kernel replaces it with the update coefficients g).
__device__ __forceinline__ float* squat_matrix(const CacheGeom& g, int64_t u) {
    return reinterpret_cast<float*>(g.base + g.off_squat) + (size_t)u * g.head_dim * g.head_dim;
}

// ------------------------------------------------------------------ Gram matrix

// One work-group of 256 threads per unit: C = sum over the unit's query heads
// and their n_q past queries of q q^T, in fp32. Thread (a, b) of a 16 x 16
// grid accumulates the (D/16) x (D/16) tile of rows a*D/16.., columns b*D/16...
template <int D>
__global__ __launch_bounds__(256) void squat_gram_kernel(const SquatBuildArgs a) {
    constexpr int TS = D / 16;   // tile side
    constexpr int CH = 32;       // queries staged at a time
    __shared__ __align__(16) float sq[CH][D];
    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int64_t u = blockIdx.x;
    const int64_t b = u / g.n_kv_heads, h = u % g.n_kv_heads;
    const int group = g.n_q_heads / g.n_kv_heads;
    const int r0 = (tid / 16) * TS, c0 = (tid % 16) * TS;
    float acc[TS][TS];
#pragma unroll
    for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int k = 0; k < TS; ++k) acc[i][k] = 0.0f;
    const int64_t nvec = (int64_t)group * a.n_q;
    for (int64_t v0 = 0; v0 < nvec; v0 += CH) {
        __syncthreads();
        for (int idx = tid; idx < CH * D; idx += 256) {
            const int vv = idx / D, c = idx % D;
            const int64_t v = v0 + vv;
            float x = 0.0f;
            if (v < nvec) {
                const int64_t head = h * group + v / a.n_q, t = v % a.n_q;
                const uint16_t bits = a.q[((b * g.n_q_heads + head) * a.n_q + t) * D + c];
                x = a.q_bf16 ? __uint_as_float((uint32_t)bits << 16) : __half2float(__ushort_as_half(bits));
            }
            sq[vv][c] = x;
        }
        __syncthreads();
#pragma unroll 4
        for (int vv = 0; vv < CH; ++vv) {
            float ra[TS], rb[TS];
#pragma unroll
            for (int i = 0; i < TS; ++i) {
                ra[i] = sq[vv][r0 + i];
                rb[i] = sq[vv][c0 + i];
            }
#pragma unroll
            for (int i = 0; i < TS; ++i)
#pragma unroll
                for (int k = 0; k < TS; ++k) acc[i][k] = fmaf(ra[i], rb[k], acc[i][k]);
        }
    }
    float* C = squat_matrix(g, u);
#pragma unroll
    for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int k = 0; k < TS; ++k) C[(r0 + i) * D + c0 + k] = acc[i][k];
}

// ------------------------------------------------------------------ coefficients

// A fixed pseudo-random start for the subspace iteration (splitmix of the index).
__device__ __forceinline__ double start_value(uint32_t i) {
    uint64_t x = (uint64_t)i * 0x9E3779B97F4A7C15ull + 0x632BE59BD9B4E019ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    x ^= x >> 31;
    return (double)(x >> 11) * 0x1p-53 * 2.0 - 1.0;
}

// One work-group of 256 threads per unit:
//   1. the top-r subspace of C by subspace iteration in fp64: W = C V, then V
//      = W R^-1 with R the Cholesky factor of W^T W (twice per step), from a
//      fixed pseudo-random start, kSquatIters steps;
//   2. Hinv = (1/lambda) I - (1/lambda - 1/(1 + lambda)) V V^T, its upper
//      Cholesky factor T in place (fp32), and g[c][j] = T[c][j] / T[c][c]
//      for j > c (0 elsewhere), written over C.
constexpr int kSquatIters = 48;

template <int D>
__global__ __launch_bounds__(256) void squat_factor_kernel(const SquatBuildArgs a) {
    constexpr int RM = kSquatMaxRank;
    __shared__ __align__(16) float sa[D][D];     // C, then Hinv and its factor
    __shared__ __align__(16) double sv[D][RM];   // V
    __shared__ __align__(16) double sw[D][RM];   // W
    __shared__ double sm[RM][RM];                // W^T W and its factor
    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int64_t u = blockIdx.x;
    const int r = a.rank;
    float* C = squat_matrix(g, u);
    for (int idx = tid; idx < D * D; idx += 256) sa[idx / D][idx % D] = C[idx];
    for (int idx = tid; idx < D * r; idx += 256) sv[idx / r][idx % r] = start_value((uint32_t)idx);
    __syncthreads();
    // C + eps I has C's eigenvectors; the shift (1e-7 of the mean eigenvalue)
    // keeps W = C V of full rank when the queries span fewer than r directions
    if (tid == 0) {
        double tr = 0.0;
        for (int c = 0; c < D; ++c) tr += sa[c][c];
        sm[0][0] = tr;
    }
    __syncthreads();
    const float eps = (float)(1e-7 * sm[0][0] / D) + 1e-30f;
    __syncthreads();
    for (int c = tid; c < D; c += 256) sa[c][c] += eps;
    __syncthreads();

    // V <- orthonormal basis of the columns of W (Cholesky-QR): M = W^T W,
    // R = chol(M) (upper), V = W R^-1
    auto orthonormalize = [&](double (*src)[RM]) {
        for (int idx = tid; idx < r * r; idx += 256) {
            const int i = idx / r, k = idx % r;
            double s = 0.0;
            for (int c = 0; c < D; ++c) s += src[c][i] * src[c][k];
            sm[i][k] = s;
        }
        __syncthreads();
        // r x r Cholesky, upper, in place (right-looking)
        for (int k = 0; k < r; ++k) {
            if (tid == 0) sm[k][k] = sqrt(sm[k][k] > 0.0 ? sm[k][k] : 1e-300);
            __syncthreads();
            for (int j = k + 1 + tid; j < r; j += 256) sm[k][j] /= sm[k][k];
            __syncthreads();
            const int m = r - 1 - k;
            for (int idx = tid; idx < m * m; idx += 256) {
                const int i = k + 1 + idx / m, j = k + 1 + idx % m;
                if (j >= i) sm[i][j] -= sm[k][i] * sm[k][j];
            }
            __syncthreads();
        }
        // each row of V solves x R = w (forward over the columns)
        for (int c = tid; c < D; c += 256) {
            for (int k = 0; k < r; ++k) {
                double s = src[c][k];
                for (int i = 0; i < k; ++i) s -= sv[c][i] * sm[i][k];
                sv[c][k] = s / sm[k][k];
            }
        }
        __syncthreads();
    };
    orthonormalize(sv);
    for (int it = 0; it < kSquatIters; ++it) {
        for (int idx = tid; idx < D * r; idx += 256) {
            const int c = idx / r, k = idx % r;
            double s = 0.0;
            for (int e = 0; e < D; ++e) s += (double)sa[c][e] * sv[e][k];
            sw[c][k] = s;
        }
        __syncthreads();
        orthonormalize(sw);
        if (it + 1 == kSquatIters) {  // a second pass restores orthogonality to fp64 rounding
            for (int idx = tid; idx < D * r; idx += 256) sw[idx / r][idx % r] = sv[idx / r][idx % r];
            __syncthreads();
            orthonormalize(sw);
        }
    }

    // Hinv = (1/lambda) I - kappa V V^T
    const double lam = (double)a.lambda;
    const double kappa = 1.0 / lam - 1.0 / (1.0 + lam);
    for (int idx = tid; idx < D * D; idx += 256) {
        const int i = idx / D, j = idx % D;
        double p = 0.0;
        for (int k = 0; k < r; ++k) p += sv[i][k] * sv[j][k];
        sa[i][j] = (float)((i == j ? 1.0 / lam : 0.0) - kappa * p);
    }
    __syncthreads();
    // upper Cholesky factor in place (right-looking): after step k, row k holds T[k][k..]
    for (int k = 0; k < D; ++k) {
        if (tid == 0) sa[k][k] = sqrtf(sa[k][k]);
        __syncthreads();
        for (int j = k + 1 + tid; j < D; j += 256) sa[k][j] /= sa[k][k];
        __syncthreads();
        const int m = D - 1 - k;  // trailing (i, j), k < i <= j
        for (int idx = tid; idx < m * m; idx += 256) {
            const int i = k + 1 + idx / m, j = k + 1 + idx % m;
            if (j >= i) sa[i][j] = fmaf(-sa[k][i], sa[k][j], sa[i][j]);
        }
        __syncthreads();
    }
    for (int idx = tid; idx < D * D; idx += 256) {
        const int c = idx / D, j = idx % D;
        C[idx] = j > c ? sa[c][j] / sa[c][c] : 0.0f;
    }
}

// ------------------------------------------------------------------ codes

// One wave per two key blocks of a unit (lane l: token l % 32 of block
// 2 * blockIdx.x + l / 32, with a row table counted from the unit's row's j0).
// The blocks' records already hold the KIVI statistics (written by the
// quantize launch just before, on the same stream); this kernel rewrites their
// key codes. Each lane walks its key in channel order, 16 channels at a time:
// the 16 in registers take the updates among themselves, then every later
// channel (kept in LDS) takes the 16 errors, in the order of the channels that
// made them, so each element receives its updates in channel order.
template <int D, int BITS>
__global__ __launch_bounds__(64) void squat_codes_kernel(const QuantArgs a) {
    constexpr int NB = D / 16;        // channel blocks of 16
    constexpr int W = D * BITS / 32;  // key words per token
    constexpr int PER = 32 / BITS;
    constexpr float kQmax = float((1 << BITS) - 1);
    __shared__ __align__(16) float sx[D / 4][64][4];  // lane's x[4 m .. 4 m + 3] at sx[m][lane]
    __shared__ __align__(16) float2 ssz[2][D];        // (s, z) per channel of the two blocks

    const CacheGeom& g = a.g;
    const int lane = threadIdx.x;
    const int64_t u = blockIdx.y;
    const int brow = (int)((uint32_t)blockIdx.y / (uint32_t)g.n_kv_heads);
    const int64_t jrow0 = a.rows.n ? a.rows.j0[brow] : a.j0;
    const int64_t jrow1 = a.rows.n ? a.rows.j1[brow] : a.j1;
    const int64_t ring_end = a.rows.n ? a.rows.ring_end[brow] : a.ring_end;
    const int half = lane / 32, t = lane % 32;
    const int64_t jb0 = jrow0 + 2 * (int64_t)blockIdx.x;
    if (jb0 >= jrow1) return;  // the whole wave
    const int64_t jb = jb0 + half;
    const bool valid = jb < jrow1;

    // statistics of both blocks (the second may not exist: then the first's again)
    for (int idx = lane; idx < 2 * D; idx += 64) {
        const int hb = idx / D, c = idx % D;
        const int64_t j = jb0 + hb < jrow1 ? jb0 + hb : jb0;
        const uint8_t* rec = g.base + record_offset(g, u, j);
        ssz[hb][c] = reinterpret_cast<const float2*>(rec + g.rec_ksz)[c];
    }
    // this lane's key row, fp16 -> fp32, into its LDS column
    {
        const int64_t tok = (valid ? jb : jb0) * kG + t;
        const uint16_t* row;
        if (tok < ring_end)
            row = reinterpret_cast<const uint16_t*>(g.base + g.off_ring + (size_t)u * g.ring_unit_stride +
                                                    (size_t)((uint32_t)tok % (uint32_t)g.ring_slots) * 4 * D);
        else
            row = a.k + (u * a.ntok + (tok - ring_end)) * D;
#pragma unroll
        for (int m = 0; m < D / 8; ++m) {
            const uint4 x = reinterpret_cast<const uint4*>(row)[m];
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = __half2float(__ushort_as_half((uint16_t)(w[e] & 0xffffu)));
                f[2 * e + 1] = __half2float(__ushort_as_half((uint16_t)(w[e] >> 16)));
            }
            *reinterpret_cast<float4*>(sx[2 * m][lane]) = make_float4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<float4*>(sx[2 * m + 1][lane]) = make_float4(f[4], f[5], f[6], f[7]);
        }
    }
    __syncthreads();

    typedef const __attribute__((address_space(4))) float* const_f32;
    const const_f32 G = (const_f32)squat_matrix(g, u);  // wave-uniform: scalar loads
    uint32_t words[W];
#pragma unroll
    for (int w = 0; w < W; ++w) words[w] = 0;
    for (int kb = 0; kb < NB; ++kb) {
        float xr[16], dl[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 v = *reinterpret_cast<const float4*>(sx[4 * kb + m][lane]);
            xr[4 * m] = v.x;
            xr[4 * m + 1] = v.y;
            xr[4 * m + 2] = v.z;
            xr[4 * m + 3] = v.w;
        }
        uint32_t wd[16 / PER > 0 ? 16 / PER : 1] = {};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = kb * 16 + i;
            const float2 sz = ssz[half][c];
            const float r = __builtin_amdgcn_fmed3f(__builtin_rintf((xr[i] - sz.y) / sz.x), 0.0f, kQmax);
            wd[i / PER] |= (uint32_t)r << (BITS * (i % PER));
            dl[i] = xr[i] - __builtin_fmaf(sz.x, r, sz.y);
#pragma unroll
            for (int i2 = i + 1; i2 < 16; ++i2) xr[i2] = __builtin_fmaf(-dl[i], G[c * D + kb * 16 + i2], xr[i2]);
        }
        // the block's 16 codes are whole words (16 / PER of them) at word kb * 16 / PER
#pragma unroll
        for (int e = 0; e < 16 / PER; ++e)
#pragma unroll
            for (int w = 0; w < W; ++w)
                if (w == kb * (16 / PER) + e) words[w] = wd[e];
        for (int kb2 = kb + 1; kb2 < NB; ++kb2) {
            float xl[16];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 v = *reinterpret_cast<const float4*>(sx[4 * kb2 + m][lane]);
                xl[4 * m] = v.x;
                xl[4 * m + 1] = v.y;
                xl[4 * m + 2] = v.z;
                xl[4 * m + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int i2 = 0; i2 < 16; ++i2)
                    xl[i2] = __builtin_fmaf(-dl[i], G[(kb * 16 + i) * D + kb2 * 16 + i2], xl[i2]);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<float4*>(sx[4 * kb2 + m][lane]) =
                    make_float4(xl[4 * m], xl[4 * m + 1], xl[4 * m + 2], xl[4 * m + 3]);
        }
    }
    if (valid) {
        uint32_t* kw = reinterpret_cast<uint32_t*>(g.base + record_offset(g, u, jb) + g.rec_kcode) + t * W;
#pragma unroll
        for (int w = 0; w < W; w += 4)
            *reinterpret_cast<uint4*>(kw + w) = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
    }
}

template <int D>
hipError_t squat_build_d(const SquatBuildArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
    squat_gram_kernel<D><<<grid, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    squat_factor_kernel<D><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t squat_codes_d(const QuantArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.j1 - a.j0 + 1) / 2), (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
    if (a.g.bits == 2)
        squat_codes_kernel<D, 2><<<grid, 64, 0, s>>>(a);
    else
        squat_codes_kernel<D, 4><<<grid, 64, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_squat_build(const SquatBuildArgs& a, hipStream_t s) {
    return a.g.head_dim == 64 ? squat_build_d<64>(a, s) : squat_build_d<128>(a, s);
}

hipError_t launch_squat_codes(const QuantArgs& a, hipStream_t s) {
    return a.g.head_dim == 64 ? squat_codes_d<64>(a, s) : squat_codes_d<128>(a, s);
}

}  // namespace kivi
