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
//     query heads that read the KV head) with the largest eigenvalues, basis
//     U (rows u_c, one r-vector per channel);
//   - objective of a key's error e: ||U^T e||^2 + lambda ||e||^2. After fixing
//     element c with error delta, the optimal move of every later element j
//     (the optimal-brain-surgeon step on H = U U^T + lambda I restricted to
//     the elements still free) is -delta * g[c][j];
//   - the codes: channel order, each element with its block's KIVI (s_c, z_c)
//     (KIVI page, section 量子化アルゴリズム): code = clamp(rint((x - z) / s),
//     0, 2^b - 1) in IEEE fp32, delta = x - fma(s, code, z).
//
// Computed here in the subspace's own coordinates. With M_c = lambda I +
// sum_{i > c} u_i u_i^T (r x r), the Woodbury identity gives g[c][j] =
// u_j . w_c with w_c = -M_c^-1 u_c, so the correction element c receives from
// all earlier ones is u_c . a, a = sum_{c' < c} delta_c' w_c' (an r-vector per
// key): per element 2 r fused multiply-adds instead of one per later element.
// The w_c come from c = d - 1 down to 0, M_c^-1 kept by Sherman-Morrison
// (M_{c-1}^-1 from M_c^-1 and u_c), in fp64.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "launch.hpp"

namespace kivi {
namespace {

constexpr int kG = 32;  // tokens per key block

// Unit u's coefficients in the coder's region: U [d][r8] then W [d][r8] fp32,
// r8 = the rank rounded up to a multiple of 8 (padding columns are 0).
__device__ __forceinline__ float* squat_coef(const CacheGeom& g, int64_t u) {
    return reinterpret_cast<float*>(g.base + g.off_squat) + (size_t)u * 2 * g.head_dim * g.squat_r8;
}

// A fixed pseudo-random start for the subspace iteration (splitmix of the index).
__device__ __forceinline__ double start_value(uint32_t i) {
    uint64_t x = (uint64_t)i * 0x9E3779B97F4A7C15ull + 0x632BE59BD9B4E019ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    x ^= x >> 31;
    return (double)(x >> 11) * 0x1p-53 * 2.0 - 1.0;
}

constexpr int kSquatIters = 48;
// subspace iteration stops once r - ||V^T V'||_F^2 (the summed squared sines of
// the angles between the subspaces of two steps) falls below this
constexpr double kSquatTol = 1e-12;
// One-sided Jacobi, taken when the subspace iteration has not converged in
// kSquatIters steps (the past queries' spectrum does not fall off after the
// r-th eigenvalue): a pair of columns is rotated unless |m_p . m_q| <=
// kJacobiTol ||m_p|| ||m_q||; the sweeps stop after one with no rotation, or
// after kJacobiSweeps.
constexpr double kJacobiTol = 1.5e-14;
constexpr int kJacobiSweeps = 30;
// M's column stride in doubles: two more than a column, so that the pairs of
// a round spread over the LDS banks
template <int D>
constexpr int jacobi_stride() { return D + 2; }
// Pair i of round k (0 <= k < D - 1) of the circle method: over D - 1 rounds
// the D / 2 disjoint pairs of each round meet every pair of columns once.
template <int D>
__device__ __forceinline__ void jacobi_pair(int k, int i, int& p, int& q) {
    constexpr int m = D - 1;
    if (i == 0) {
        p = k;
        q = D - 1;
    } else {
        p = (k + i) % m;
        q = (k - i + m) % m;
    }
}

// One work-group of 256 threads per unit:
//   1. C = sum over the unit's query heads and their n_q past queries of
//      q q^T in fp32 (thread (a, b) of a 16 x 16 grid owns a (D/16)^2 tile);
//   2. the top-r subspace of C by subspace iteration in fp64: W = C V, then V =
//      W R^-1 with R the Cholesky factor of W^T W, from a fixed pseudo-random
//      start, until the subspace no longer moves (the summed squared sines
//      of the angles between two steps' subspaces below kSquatTol; kSquatIters
//      steps at most), and one more orthonormalisation; when the iteration has
//      not converged by then, the subspace comes from a one-sided Jacobi
//      eigen-decomposition of C + sigma I in fp64 instead (its r columns of
//      largest norm);
//   3. w_c = -M_c^-1 u_c for c = d - 1 .. 0 with M_c^-1 by Sherman-Morrison;
//   4. U and W (fp32, zero-padded to r8 columns) to the unit's coefficients.
template <int D>
__global__ __launch_bounds__(256) void squat_build_kernel(const SquatBuildArgs a) {
    constexpr int RM = kSquatMaxRank;
    constexpr int TS = D / 16;  // Gram tile side
    constexpr int CH = 32;      // queries staged at a time
    constexpr int MS = jacobi_stride<D>();
    // C (fp32), V and W in one pool; the Jacobi fallback's fp64 matrix M
    // (column c at M + c MS) takes the whole pool once the iteration is over
    constexpr int POOL_C = D * D / 2, POOL_VW = POOL_C + 2 * D * RM, POOL_M = D * MS;
    __shared__ __align__(16) double pool[POOL_VW > POOL_M ? POOL_VW : POOL_M];
    float(*const sa)[D] = reinterpret_cast<float(*)[D]>(pool);               // C
    double(*const sv)[RM] = reinterpret_cast<double(*)[RM]>(pool + POOL_C);  // V (the queries' staging buffer before)
    double(*const sw)[RM] = reinterpret_cast<double(*)[RM]>(pool + POOL_C + D * RM);  // W, then the w_c
    __shared__ double sm[RM][RM];                // W^T W and its factor, then M^-1
    __shared__ double st[RM][RM];                // V^T W (the convergence test)
    __shared__ double sz[RM];
    __shared__ double snrm[D];                   // Jacobi: squared column norms
    __shared__ int ssel[RM];                     // Jacobi: the columns of rank 0 .. r - 1
    static_assert(CH * D * sizeof(float) <= D * RM * sizeof(double), "the staged queries fit V's space");
    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int64_t u = blockIdx.x;
    const int r = a.rank;
    const int64_t b = u / g.n_kv_heads, h = u % g.n_kv_heads;
    const int group = g.n_q_heads / g.n_kv_heads;

    // 1. Gram matrix
    {
        float(*sq)[D] = reinterpret_cast<float(*)[D]>(&sv[0][0]);
        const int r0 = (tid / 16) * TS, c0 = (tid % 16) * TS;
        float acc[TS][TS];
#pragma unroll
        for (int i = 0; i < TS; ++i)
#pragma unroll
            for (int k = 0; k < TS; ++k) acc[i][k] = 0.0f;
        const int64_t nvec = (int64_t)group * a.n_q;
        // a chunk of CH queries: 16 bytes (8 values) a lane per load, the next
        // chunk's loads in flight while the current one is computed
        constexpr int NL = CH * D / 8 / 256;
        static_assert(CH * D % (8 * 256) == 0, "a chunk is a whole number of 16-byte loads a thread");
        uint4 nx[NL];
        auto load_chunk = [&](int64_t v0) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int idx = tid + 256 * i;
                const int vv = idx / (D / 8), c8 = idx % (D / 8);
                const int64_t v = v0 + vv;
                if (v < nvec) {
                    const int64_t head = h * group + v / a.n_q, t = v % a.n_q;
                    nx[i] = *reinterpret_cast<const uint4*>(a.q + ((b * g.n_q_heads + head) * a.n_q + t) * D + 8 * c8);
                } else {
                    nx[i] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
        };
        load_chunk(0);
        for (int64_t v0 = 0; v0 < nvec; v0 += CH) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int idx = tid + 256 * i;
                const int vv = idx / (D / 8), c8 = idx % (D / 8);
                const uint32_t w[4] = {nx[i].x, nx[i].y, nx[i].z, nx[i].w};
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t bits = (uint16_t)(w[e / 2] >> (16 * (e & 1)));
                    x[e] = a.q_bf16 ? __uint_as_float((uint32_t)bits << 16) : __half2float(__ushort_as_half(bits));
                }
                reinterpret_cast<float4*>(&sq[vv][8 * c8])[0] = make_float4(x[0], x[1], x[2], x[3]);
                reinterpret_cast<float4*>(&sq[vv][8 * c8])[1] = make_float4(x[4], x[5], x[6], x[7]);
            }
            __syncthreads();
            if (v0 + CH < nvec) load_chunk(v0 + CH);
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
#pragma unroll
        for (int i = 0; i < TS; ++i)
#pragma unroll
            for (int k = 0; k < TS; ++k) sa[r0 + i][c0 + k] = acc[i][k];
        __syncthreads();
    }
    for (int idx = tid; idx < D * r; idx += 256) sv[idx / r][idx % r] = start_value((uint32_t)idx);
    // The iteration runs on C + sigma I, which has C's eigenvectors, with sigma
    // = 1e-5 of C's trace (at least 1e-5 of its largest eigenvalue), added in
    // fp64 to every W = C V: when the queries span fewer than r directions, the
    // columns of W then stay independent to within a condition number of about
    // 1e5, which the fp64 Cholesky factor of W^T W resolves (with sigma at
    // 1e-9 of the largest eigenvalue, a history of three exact directions drove
    // W^T W's smallest eigenvalues below its rounding and the factor to NaN).
    if (tid == 0) {
        double tr = 0.0;
        for (int c = 0; c < D; ++c) tr += sa[c][c];
        sz[0] = tr;
    }
    __syncthreads();
    const double sigma = 1e-5 * sz[0] + 1e-30;
    __syncthreads();

    // 2. V <- orthonormal basis of the columns of src (Cholesky-QR)
    auto orthonormalize = [&](double (*src)[RM]) {
        for (int idx = tid; idx < r * r; idx += 256) {
            const int i = idx / r, k = idx % r;
            double s = 0.0;
            for (int c = 0; c < D; ++c) s += src[c][i] * src[c][k];
            sm[i][k] = s;
        }
        __syncthreads();
        for (int k = 0; k < r; ++k) {  // r x r Cholesky, upper, in place (right-looking)
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
        for (int c = tid; c < D; c += 256) {  // each row of V solves x R = w
            for (int k = 0; k < r; ++k) {
                double s = src[c][k];
                for (int i = 0; i < k; ++i) s -= sv[c][i] * sm[i][k];
                sv[c][k] = s / sm[k][k];
            }
        }
        __syncthreads();
    };
    orthonormalize(sv);
    bool converged = false;
    for (int it = 0; it < kSquatIters; ++it) {
        // W = (C + sigma I) V: a thread takes row c and 8 columns; C is symmetric, so its
        // column c is read (consecutive lanes, consecutive words), and the 8
        // entries of V's row e are the same for the whole wave (broadcasts)
        for (int idx = tid; idx < D * ((r + 7) / 8); idx += 256) {
            const int c = idx % D, k0 = 8 * (idx / D);
            double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int e = 0; e < D; ++e) {
                const double x = (double)sa[e][c];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = fma(x, sv[e][k0 + k], acc[k]);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k0 + k < r) sw[c][k0 + k] = fma(sigma, sv[c][k0 + k], acc[k]);
        }
        __syncthreads();
        // T = V^T W, before V is replaced: with the new V' = W R^-1,
        // ||V^T V'||_F^2 = ||T R^-1||_F^2 is the sum of the squared cosines of
        // the angles between the two subspaces, r when they agree
        for (int idx = tid; idx < r * r; idx += 256) {
            const int i = idx / r, k = idx % r;
            double t = 0.0;
            for (int c = 0; c < D; ++c) t += sv[c][i] * sw[c][k];
            st[i][k] = t;
        }
        __syncthreads();
        orthonormalize(sw);
        if (tid < r) {  // row tid of T R^-1 (R upper, in sm), in place, and its squared norm
            double n2 = 0.0;
            for (int k = 0; k < r; ++k) {
                double t = st[tid][k];
                for (int j = 0; j < k; ++j) t -= st[tid][j] * sm[j][k];
                st[tid][k] = t / sm[k][k];
                n2 += st[tid][k] * st[tid][k];
            }
            sz[tid] = n2;
        }
        __syncthreads();
        double f = 0.0;
        for (int i = 0; i < r; ++i) f += sz[i];
        if ((double)r - f < kSquatTol) {  // the subspace no longer moves (uniform)
            converged = true;
            break;
        }
        __syncthreads();
    }
    __syncthreads();
    if (!converged) {
        // 2b. One-sided Jacobi on C + sigma I, which has C's eigenvectors and
        //     only positive eigenvalues: M = (C + sigma I) J, with J the product
        //     of the rotations, until M's columns are mutually orthogonal; then
        //     column c of M is (lambda_c + sigma) v_c, with v_c an eigenvector
        //     of C, and V takes the r of largest norm, normalised.
        double* const M = pool;
        {
            constexpr int PER = D * D / 256;
            float cr[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = tid + 256 * e;
                cr[e] = sa[idx / D][idx % D];
            }
            __syncthreads();  // C's fp32 entries are in registers; M overwrites them
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = tid + 256 * e, i = idx / D, c = idx % D;
                M[c * MS + i] = (double)cr[e] + (i == c ? sigma : 0.0);
            }
            __syncthreads();
        }
        // a round rotates D / 2 disjoint pairs; TPP consecutive lanes take a
        // pair, lane j of them rows j, j + TPP, ... of both columns
        constexpr int NP = D / 2, TPP = 256 / NP, RPT = D / TPP;
        static_assert(256 % NP == 0 && (TPP & (TPP - 1)) == 0 && TPP <= 64, "a pair's lanes are a power of two in a wave");
        const int pi = tid / TPP, j = tid % TPP;
        for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
            int any = 0;
            for (int k = 0; k < D - 1; ++k) {
                int p, q;
                jacobi_pair<D>(k, pi, p, q);
                double mp[RPT], mq[RPT];
                double aa = 0.0, bb = 0.0, gg = 0.0;
#pragma unroll
                for (int e = 0; e < RPT; ++e) {
                    mp[e] = M[p * MS + j + TPP * e];
                    mq[e] = M[q * MS + j + TPP * e];
                    aa = fma(mp[e], mp[e], aa);
                    bb = fma(mq[e], mq[e], bb);
                    gg = fma(mp[e], mq[e], gg);
                }
#pragma unroll
                for (int o = 1; o < TPP; o <<= 1) {
                    aa += __shfl_xor(aa, o, TPP);
                    bb += __shfl_xor(bb, o, TPP);
                    gg += __shfl_xor(gg, o, TPP);
                }
                const int rot = fabs(gg) > kJacobiTol * sqrt(aa * bb);
                if (rot) {
                    // the rotation that zeroes m_p . m_q (Hestenes)
                    const double zeta = (bb - aa) / (2.0 * gg);
                    const double t = copysign(1.0, zeta) / (fabs(zeta) + sqrt(fma(zeta, zeta, 1.0)));
                    const double cs = 1.0 / sqrt(fma(t, t, 1.0)), sn = cs * t;
#pragma unroll
                    for (int e = 0; e < RPT; ++e) {
                        M[p * MS + j + TPP * e] = cs * mp[e] - sn * mq[e];
                        M[q * MS + j + TPP * e] = sn * mp[e] + cs * mq[e];
                    }
                }
                // orders this round's stores before the next round's loads
                any |= __syncthreads_or(rot);
            }
            if (!any) break;  // a sweep without a rotation: uniform
        }
        // squared column norms; column c's rank by norm (ties by index)
        for (int c = tid; c < D; c += 256) {
            double n2 = 0.0;
            for (int i = 0; i < D; ++i) n2 = fma(M[c * MS + i], M[c * MS + i], n2);
            snrm[c] = n2;
        }
        __syncthreads();
        for (int c = tid; c < D; c += 256) {
            int rk = 0;
            for (int c2 = 0; c2 < D; ++c2) rk += snrm[c2] > snrm[c] || (snrm[c2] == snrm[c] && c2 < c);
            if (rk < r) ssel[rk] = c;
        }
        __syncthreads();
        // V's column k = M's column ssel[k] / its norm (V overlaps M: read first)
        constexpr int PV = D * RM / 256;
        double vr[PV];
#pragma unroll
        for (int e = 0; e < PV; ++e) {
            const int idx = tid + 256 * e, i = idx / RM, k = idx % RM;
            vr[e] = k < r ? M[ssel[k] * MS + i] / sqrt(snrm[ssel[k]]) : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < PV; ++e) {
            const int idx = tid + 256 * e;
            sv[idx / RM][idx % RM] = vr[e];
        }
        __syncthreads();
    }
    // a second pass restores orthogonality to fp64 rounding
    for (int idx = tid; idx < D * r; idx += 256) sw[idx / r][idx % r] = sv[idx / r][idx % r];
    __syncthreads();
    orthonormalize(sw);

    // 3. w_c = -M_c^-1 u_c, M_c = lambda I + sum_{i > c} u_i u_i^T, from c = D - 1 down
    for (int idx = tid; idx < r * r; idx += 256) sm[idx / r][idx % r] = idx / r == idx % r ? 1.0 / (double)a.lambda : 0.0;
    __syncthreads();
    for (int c = D - 1; c >= 0; --c) {
        if (tid < r) {  // z = M_c^-1 u_c
            double s = 0.0;
            for (int k = 0; k < r; ++k) s += sm[tid][k] * sv[c][k];
            sz[tid] = s;
        }
        __syncthreads();
        if (tid < r) sw[c][tid] = -sz[tid];
        double den = 1.0;
        for (int k = 0; k < r; ++k) den += sv[c][k] * sz[k];
        // M_{c-1}^-1 = M_c^-1 - z z^T / (1 + u_c . z)
        for (int idx = tid; idx < r * r; idx += 256) sm[idx / r][idx % r] -= sz[idx / r] * sz[idx % r] / den;
        __syncthreads();
    }

    // 4. U and W, zero-padded to r8 columns
    const int r8 = g.squat_r8;
    float* out = squat_coef(g, u);
    for (int idx = tid; idx < D * r8; idx += 256) {
        const int c = idx / r8, k = idx % r8;
        out[idx] = k < r ? (float)sv[c][k] : 0.0f;
        out[D * r8 + idx] = k < r ? (float)sw[c][k] : 0.0f;
    }
}

// ------------------------------------------------------------------ codes

// One work-group of four waves per 8 TPL key blocks of a unit quantized by the
// launch, TPL tokens per lane: wave w takes blocks 8 TPL blockIdx.x + 2 TPL w
// .. + 2 TPL - 1 (with a row table counted from the unit's row's j0), lane l
// tokens l % L + L p (p < TPL, L = 32 / TPL) of the wave's block l / L. The
// blocks' records already hold the KIVI statistics (written by the quantize
// launch just before, on the same stream); this kernel rewrites their key
// codes. U, W and the blocks' (s, z, rcp s) are staged in LDS once and read as
// broadcasts; each lane walks its fp16 key rows in channel order, 16 channels
// a step with the next step's bytes in flight, keeping -a = -sum_{c' < c}
// delta_c' w_c' (R8 floats) per token.
//
// The broadcasts cost LDS bandwidth per lane, whatever the address: with one
// token per lane they bound the walk (measured). Two tokens per lane halve
// the LDS bytes per element, since each broadcast of u_c, w_c and the
// statistics serves both; a launch of at most two blocks per unit (a flush
// during decode) keeps one token per lane, as there the walk's latency sets
// the time.
//
// The codes are those of the IEEE steps, computed faster, as in the plain
// quantizer: p = (x - z) rcp(s), clamped to [0, 2^b - 1], is within
// (2^b - 1/2) 2^-22 of the IEEE quotient there (rcp within 1 ulp), so rint(p)
// is the IEEE code unless p lies within a margin four times that of a
// half-integer; then the wave takes the IEEE division for that channel.
// -delta is fma(s, code, -(x - z)), one rounding of the same difference.
template <int TPL>
constexpr int squat_blocks_per_wave() { return 64 * TPL / kG; }
template <int TPL>
constexpr int squat_blocks_per_wg() { return 4 * squat_blocks_per_wave<TPL>(); }

// u * a + k with k the fp16 half HI of `pair`, widened exactly inside one
// fused multiply-add (v_fma_mix_f32): fma(u, a, (float)k), one rounding.
template <int HI>
__device__ __forceinline__ float half_fma(float u, float a, uint32_t pair) {
    float r;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(r) : "v"(u), "v"(a), "v"(pair));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,0,1]" : "=v"(r) : "v"(u), "v"(a), "v"(pair));
    return r;
}

template <int D, int BITS, int R8, int TPL>
__global__ __launch_bounds__(256) void squat_codes_kernel(const QuantArgs a) {
    constexpr int LPB = kG / TPL;  // lanes per block
    constexpr int BPW = squat_blocks_per_wave<TPL>();
    constexpr int BPG = squat_blocks_per_wg<TPL>();
    constexpr int W = D * BITS / 32;  // key words per token
    constexpr int H = 16 / BITS;      // codes per 16-bit accumulator
    constexpr float kQmax = float((1 << BITS) - 1);
    constexpr float kMargin = 0.5f - float(1 << BITS) * 0x1p-20f;
    // a block's statistics row, padded where LDS allows: the four blocks a
    // wave reads at once then start 4 banks apart
    constexpr int SQ = 2 * D * R8 * 4 + BPG * (D + 1) * 16 <= 65536 ? D + 1 : D;
    __shared__ __align__(16) float suw[2][D][R8];                // u_c, then w_c
    __shared__ __align__(16) float4 ssz[BPG][SQ];  // (s, z, rcp s) per channel and block
    static_assert(sizeof(suw) + sizeof(ssz) <= 65536, "one work-group's LDS");

    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int64_t u = blockIdx.y;
    const int brow = (int)((uint32_t)blockIdx.y / (uint32_t)g.n_kv_heads);
    const int64_t jrow0 = a.rows.n ? a.rows.j0[brow] : a.j0;
    const int64_t jrow1 = a.rows.n ? a.rows.j1[brow] : a.j1;
    const int64_t ring_end = a.rows.n ? a.rows.ring_end[brow] : a.ring_end;
    const int64_t jw0 = jrow0 + (int64_t)BPG * blockIdx.x;
    if (jw0 >= jrow1) return;  // the whole work-group
    const int bw = lane / LPB, t0 = lane % LPB;
    const int64_t jb = jw0 + BPW * wave + bw;
    const bool valid = jb < jrow1;
    const int64_t jl = valid ? jb : jw0;  // a block that exists, for the loads of a lane past the end

    // this lane's key rows (fp16): 32 bytes (16 channels) of each per step, the next step's in flight
    const uint4* row[TPL];
    uint4 nx[TPL][2];
#pragma unroll
    for (int p = 0; p < TPL; ++p) {
        const int64_t tok = jl * kG + t0 + LPB * p;
        if (tok < ring_end)
            row[p] = reinterpret_cast<const uint4*>(g.base + g.off_ring + (size_t)u * g.ring_unit_stride +
                                                    (size_t)((uint32_t)tok % (uint32_t)g.ring_slots) * 4 * D);
        else
            row[p] = reinterpret_cast<const uint4*>(a.k + (u * a.ntok + (tok - ring_end)) * D);
        nx[p][0] = row[p][0];
        nx[p][1] = row[p][1];
    }
    // the unit's U and W, and the statistics of the work-group's blocks (a
    // block past the end: the first block's again)
    const float* coef = squat_coef(g, u);
    for (int idx = tid; idx < 2 * D * R8 / 4; idx += 256)
        reinterpret_cast<float4*>(&suw[0][0][0])[idx] = reinterpret_cast<const float4*>(coef)[idx];
    for (int idx = tid; idx < BPG * D; idx += 256) {
        const int hb = idx / D, c = idx % D;
        const int64_t j = jw0 + hb < jrow1 ? jw0 + hb : jw0;
        const float2 sz = reinterpret_cast<const float2*>(g.base + record_offset(g, u, j) + g.rec_ksz)[c];
        ssz[hb][c] = make_float4(sz.x, sz.y, __builtin_amdgcn_rcpf(sz.x), 0.0f);
    }
    __syncthreads();

    const float4* sz_mine = ssz[BPW * wave + bw];
    float acc[TPL][R8];  // -a of each token
#pragma unroll
    for (int p = 0; p < TPL; ++p)
#pragma unroll
        for (int k = 0; k < R8; ++k) acc[p][k] = 0.0f;
    uint32_t words[TPL][W];
#pragma unroll
    for (int p = 0; p < TPL; ++p)
#pragma unroll
        for (int w = 0; w < W; ++w) words[p][w] = 0;
#pragma unroll 1
    for (int cb = 0; cb < D / 16; ++cb) {
        uint32_t hw[TPL][8];
#pragma unroll
        for (int p = 0; p < TPL; ++p) {
            const uint4 p0 = nx[p][0], p1 = nx[p][1];
            hw[p][0] = p0.x, hw[p][1] = p0.y, hw[p][2] = p0.z, hw[p][3] = p0.w;
            hw[p][4] = p1.x, hw[p][5] = p1.y, hw[p][6] = p1.z, hw[p][7] = p1.w;
            if (cb + 1 < D / 16) {
                nx[p][0] = row[p][2 * cb + 2];
                nx[p][1] = row[p][2 * cb + 3];
            }
        }
        float hf[TPL][BITS];  // the step's codes, 16 bits per accumulator
#pragma unroll
        for (int p = 0; p < TPL; ++p)
#pragma unroll
            for (int e = 0; e < BITS; ++e) hf[p][e] = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = cb * 16 + i;
            const float* uc = suw[0][c];
            const float* wc = suw[1][c];
            const float4 q = sz_mine[c];  // (s, z, rcp s, -)
            float t[TPL], r[TPL];
            bool tie = false;
#pragma unroll
            for (int p = 0; p < TPL; ++p) {
                // x = k_c + u_c . (-a), the fp16 k_c widened inside the first fma;
                // two chains of R8 / 2 terms
                float x0 = (i & 1) ? half_fma<1>(uc[0], acc[p][0], hw[p][i / 2])
                                   : half_fma<0>(uc[0], acc[p][0], hw[p][i / 2]);
                float x1 = uc[R8 / 2] * acc[p][R8 / 2];
#pragma unroll
                for (int k = 1; k < R8 / 2; ++k) {
                    x0 = __builtin_fmaf(uc[k], acc[p][k], x0);
                    x1 = __builtin_fmaf(uc[R8 / 2 + k], acc[p][R8 / 2 + k], x1);
                }
                t[p] = (x0 + x1) - q.y;
                const float pc = __builtin_amdgcn_fmed3f(t[p] * q.z, 0.0f, kQmax);
                r[p] = __builtin_rintf(pc);
                tie = tie || fabsf(pc - r[p]) > kMargin;
            }
            if (__builtin_amdgcn_ballot_w64(tie)) {
#pragma unroll
                for (int p = 0; p < TPL; ++p) r[p] = __builtin_amdgcn_fmed3f(__builtin_rintf(t[p] / q.x), 0.0f, kQmax);
            }
#pragma unroll
            for (int p = 0; p < TPL; ++p) {
                hf[p][i / H] = __builtin_fmaf(r[p], (float)(1 << (BITS * (i % H))), hf[p][i / H]);
                // -delta = s code - (x - z), then -a += -delta w_c
                const float ndl = __builtin_fmaf(q.x, r[p], -t[p]);
#pragma unroll
                for (int k = 0; k < R8; ++k) acc[p][k] = __builtin_fmaf(ndl, wc[k], acc[p][k]);
            }
        }
        // the step's 16 codes are whole words (BITS / 2 of them) at word cb * BITS / 2
#pragma unroll
        for (int p = 0; p < TPL; ++p)
#pragma unroll
            for (int e = 0; e < BITS / 2; ++e)
#pragma unroll
                for (int w = 0; w < W; ++w)
                    if (w == cb * (BITS / 2) + e)
                        words[p][w] = (uint32_t)hf[p][2 * e] | (uint32_t)hf[p][2 * e + 1] << 16;
    }
    if (valid) {
#pragma unroll
        for (int p = 0; p < TPL; ++p) {
            uint32_t* kw =
                reinterpret_cast<uint32_t*>(g.base + record_offset(g, u, jb) + g.rec_kcode) + (t0 + LPB * p) * W;
#pragma unroll
            for (int w = 0; w < W; w += 4)
                *reinterpret_cast<uint4*>(kw + w) = make_uint4(words[p][w], words[p][w + 1], words[p][w + 2], words[p][w + 3]);
        }
    }
}

template <int D, int BITS, int TPL>
hipError_t squat_codes_dbt(const QuantArgs& a, hipStream_t s) {
    constexpr int BPG = squat_blocks_per_wg<TPL>();
    const dim3 grid((unsigned)((a.j1 - a.j0 + BPG - 1) / BPG), (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
    switch (a.g.squat_r8) {
        case 8: squat_codes_kernel<D, BITS, 8, TPL><<<grid, 256, 0, s>>>(a); break;
        case 16: squat_codes_kernel<D, BITS, 16, TPL><<<grid, 256, 0, s>>>(a); break;
        case 24: squat_codes_kernel<D, BITS, 24, TPL><<<grid, 256, 0, s>>>(a); break;
        default: squat_codes_kernel<D, BITS, 32, TPL><<<grid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <int D, int BITS>
hipError_t squat_codes_db(const QuantArgs& a, hipStream_t s) {
    return a.j1 - a.j0 <= 2 ? squat_codes_dbt<D, BITS, 1>(a, s) : squat_codes_dbt<D, BITS, 2>(a, s);
}

template <int D>
hipError_t squat_codes_d(const QuantArgs& a, hipStream_t s) {
    return a.g.bits == 2 ? squat_codes_db<D, 2>(a, s) : squat_codes_db<D, 4>(a, s);
}

}  // namespace

hipError_t launch_squat_build(const SquatBuildArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
    if (a.g.head_dim == 64)
        squat_build_kernel<64><<<grid, 256, 0, s>>>(a);
    else
        squat_build_kernel<128><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_squat_codes(const QuantArgs& a, hipStream_t s) {
    return a.g.head_dim == 64 ? squat_codes_d<64>(a, s) : squat_codes_d<128>(a, s);
}

}  // namespace kivi
