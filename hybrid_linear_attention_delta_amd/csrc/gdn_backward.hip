// gdn_backward.hip -- gradients of the chunked gated delta rule (gfx950), fp32.
//
// Training evaluates the recurrence of "Long-Context Aware Upcycling: A New
// Frontier for Hybrid LLM Scaling" (arXiv:2604.24715, App. A.3, Eqs. 16-19)
// in chunks (the paragraph after Eq. 21).  This file differentiates that
// chunked (WY) evaluation.  Per chunk of C = 64 tokens of one (sequence, head),
// with chunk-local cumulative log-decay gamma, Gamma_rj = e^{gamma_r - gamma_j}
// (j <= r), D = diag(e^{gamma_L - gamma}) and S the state entering the chunk:
//
//     A = strict_lower(diag(beta) (K K^T) o Gamma),  T = (I + A)^{-1}
//     W = T diag(beta e^gamma) K,   U = T diag(beta) V,   Delta = U - W S^T
//     P = lower(Q K^T o Gamma)
//     O = scale [diag(e^gamma) Q S^T + P Delta],   S' = e^{gamma_L} S + Delta^T D K
//
// (Q, K the L2-normalised queries and keys).  The backward runs in four launches:
//
//   1. bwd_table_kernel   chunk table of the packed batch (one workgroup).
//   2. bwd_local_kernel   per chunk-head: gather and pad the chunk's rows (kept
//                         in the input type, the L2 norms as fp32 row scales),
//                         form Gamma, A, T, P, W, U, D K, scale e^gamma dO and
//                         dDelta_local = scale P^T dO into a workspace, with
//                         the chains' operand fragments.
//   3. bwd_chain_kernel   both directions in one launch.  Forward over the chunks
//                         of each sequence: the state entering every chunk and
//                         its Delta.  Reverse:
//                         the state gradient after every chunk, from
//                             dDelta = dDelta_local + D K dS^T
//                             dS    <- e^{gamma_L} dS + (scale e^gamma dO)^T Q - dDelta^T W.
//                         Both are the same row-split recurrence, so one kernel
//                         serves them with different operands.
//   4. bwd_grad_kernel    per chunk-head: dQ, dK, dV, dg, dbeta of the chunk from
//                         S, dS, Delta and dDelta, then through the L2 norm
//                         (dx = r (dx^ - x^ (x^ . dx^))).
//
// Ragged chunks are padded to C rows with q = k = v = dO = 0, beta = 0 and
// g = 0, which leaves every product of the real rows unchanged.
//
// The arithmetic is fp32.  The per-chunk contractions run on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32 sums) through one
// LDS-tiled 64 x 64 block routine.  The two chains run on the bf16 matrix
// cores with each fp32 operand split into bf16 hi and lo parts (three
// products per fragment pair; a raw bf16 row is its own hi part, one product
// less) and fp32 sums.  Results do not depend on scheduling: no atomics,
// fixed reduction orders.
#include <string.h>

#include <type_traits>

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int BC = kBwdChunk;  // chunk length of the backward
constexpr int LD = 68;   // LDS row pitch of the tile routine (floats)
constexpr int KTL = 32;  // its k block in the local kernel
constexpr int KTG = 32;  // and in the gradient kernel

// acc[i][j] += sum_k A(r, k) B(k, n) for r = 4 tr + i in [0, 64), n = n0 + 16 j + tc
// (tr = threadIdx / 16, tc = threadIdx % 16), with
//   A(r, k) = A[r * lda + k] (AK: rows along k) or A[r + k * lda] (else),
//             times kscale[k] if kscale is given;
//   B(k, n) = B[k * ldb + n] (BN: rows along n) or B[k + n * ldb] (else);
// K a multiple of the k block KT, [n0, n0 + 64) inside B, every operand row
// and n0 a multiple of four floats from a 16-byte aligned base.  All 256 threads
// take part: each k block arrives by 16-byte loads (KT / 16 per operand and
// thread, all in flight together, issued while the previous block's products
// run) into LDS, k-major with row pitch LD (as and bs hold KT x LD floats
// each), two barriers per block.  The products run on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32, exact fp32 products and fp32
// sums): wave w computes rows 16 w .. 16 w + 15 as four 16 x 16 tiles, and its
// accumulator layout (lane l: rows 4 (l / 16) + i, column l % 16 of each tile)
// is the (r, n) map above.
// bf16 bits of eight consecutive values -> widened into LDS at dst[q * stride], q = 0..7
__device__ __forceinline__ void put8_col(float* dst, int stride, u16x8 x)
{
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q * stride] = bf16_bits_to_f32(x[q]);
}

template <int KT, bool AK, bool BN, typename TA = float, typename TB = float>
__device__ void mm64(float acc[4][4], const TA* __restrict__ A, int lda, const float* kscale,
                     const TB* __restrict__ B, int ldb, int K, int n0, float* as, float* bs)
{
    static_assert(KT % 32 == 0, "a k block is a whole number of 16-byte loads per thread");
    static_assert(sizeof(TA) == 4 || AK, "bf16 A operands have rows along k");
    constexpr int NV = KT / 16;   // 16-byte loads per fp32 operand and thread
    constexpr int NB = KT / 32;   // 16-byte loads per bf16 operand and thread (eight values)
    constexpr bool A16 = sizeof(TA) == 2, B16 = sizeof(TB) == 2;
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));  // per-call lane offsets: recomputed here, not hoisted and held across calls
    const int w = t >> 6, l = t & 63, r16 = l & 15, g = l >> 4;
    f32x4 d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = f32x4{acc[0][j], acc[1][j], acc[2][j], acc[3][j]};
    f32x4 xa[NV], xb[NV];
    u16x8 ya[NB], yb[NB];
    auto fetch = [&](int k0) {  // the 64 x KT block of A and the KT x 64 block of B into registers
        if constexpr (A16) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {  // KT / 8 lanes read one row's k block
                const int e = t + 256 * i, r = e / (KT / 8), k8 = e % (KT / 8);
                ya[i] = *reinterpret_cast<const u16x8*>(A + (int64_t)r * lda + k0 + 8 * k8);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = t + 256 * i;
                if constexpr (AK) {  // KT / 4 lanes read one row's k block
                    const int r = e / (KT / 4), kq = e % (KT / 4);
                    xa[i] = *reinterpret_cast<const f32x4*>(A + (int64_t)r * lda + k0 + 4 * kq);
                    if (kscale) {
                        const f32x4 s4 = *reinterpret_cast<const f32x4*>(kscale + k0 + 4 * kq);
                        xa[i] *= s4;
                    }
                } else {  // sixteen lanes read one k row of 64
                    const int kk = e >> 4, rq = e & 15;
                    xa[i] = *reinterpret_cast<const f32x4*>(A + (int64_t)(k0 + kk) * lda + 4 * rq);
                    if (kscale) xa[i] *= kscale[k0 + kk];
                }
            }
        }
        if constexpr (B16) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int e = t + 256 * i;
                if constexpr (BN) {  // eight lanes read one k row of 64
                    const int kk = e >> 3, n8 = e & 7;
                    yb[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)(k0 + kk) * ldb + n0 + 8 * n8);
                } else {
                    const int n = e / (KT / 8), k8 = e % (KT / 8);
                    yb[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)(n0 + n) * ldb + k0 + 8 * k8);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = t + 256 * i;
                if constexpr (BN) {
                    const int kk = e >> 4, nq = e & 15;
                    xb[i] = *reinterpret_cast<const f32x4*>(B + (int64_t)(k0 + kk) * ldb + n0 + 4 * nq);
                } else {
                    const int n = e / (KT / 4), kq = e % (KT / 4);
                    xb[i] = *reinterpret_cast<const f32x4*>(B + (int64_t)(n0 + n) * ldb + k0 + 4 * kq);
                }
            }
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += KT) {
        if constexpr (A16) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int e = t + 256 * i, r = e / (KT / 8), k8 = e % (KT / 8);
                if (kscale) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) as[(8 * k8 + q) * LD + r] = bf16_bits_to_f32(ya[i][q]) * kscale[k0 + 8 * k8 + q];
                } else {
                    put8_col(as + (8 * k8) * LD + r, LD, ya[i]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = t + 256 * i;
                if constexpr (AK) {
                    const int r = e / (KT / 4), kq = e % (KT / 4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) as[(4 * kq + q) * LD + r] = xa[i][q];
                } else {
                    *reinterpret_cast<f32x4*>(as + (e >> 4) * LD + 4 * (e & 15)) = xa[i];
                }
            }
        }
        if constexpr (B16) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int e = t + 256 * i;
                if constexpr (BN) {
                    const int kk = e >> 3, n8 = e & 7;
                    f32x4 lo, hi;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        lo[q] = bf16_bits_to_f32(yb[i][q]);
                        hi[q] = bf16_bits_to_f32(yb[i][4 + q]);
                    }
                    *reinterpret_cast<f32x4*>(bs + kk * LD + 8 * n8) = lo;
                    *reinterpret_cast<f32x4*>(bs + kk * LD + 8 * n8 + 4) = hi;
                } else {
                    const int n = e / (KT / 8), k8 = e % (KT / 8);
                    put8_col(bs + (8 * k8) * LD + n, LD, yb[i]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = t + 256 * i;
                if constexpr (BN) {
                    *reinterpret_cast<f32x4*>(bs + (e >> 4) * LD + 4 * (e & 15)) = xb[i];
                } else {
                    const int n = e / (KT / 4), kq = e % (KT / 4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) bs[(4 * kq + q) * LD + n] = xb[i][q];
                }
            }
        }
        __syncthreads();
        if (k0 + KT < K) fetch(k0 + KT);  // the next block's loads fly during these products
#pragma unroll
        for (int kq = 0; kq < KT / 4; ++kq) {
            const float av = as[(4 * kq + g) * LD + 16 * w + r16];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bs[(4 * kq + g) * LD + 16 * j + r16], d[j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = d[j][i];
}

__device__ __forceinline__ void zero(float acc[4][4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
}

// Three products that share their B operands, in one pass over k:
//   p1 = A1 B1,  p2 = A2 B1,  p3 = A3 B2   (64 x 64 blocks, [n0, n0 + 64) of B),
// A_i[r][k] rows along k (pitch lda), B_i[k][n] rows along n (pitch ldb), and
// dot += sum over the block of B1 o B2, each element counted once over the
// calls for all n0.  The same tiling and 16-byte loads as mm64 (KT = 32),
// with the next k block's loads in flight during the current products; every
// B1 and B2 element crosses from memory once instead of once per product.
// ls holds 5 KT x LD floats (A1, A2, A3, B1, B2).  A1 may be bf16 (eight
// values per 16-byte load).
template <typename TA1>
__device__ void mm64x3(float p1[4][4], float p2[4][4], float p3[4][4], float& dot, const TA1* __restrict__ A1,
                       const float* __restrict__ A2, const float* __restrict__ A3, int lda,
                       const float* __restrict__ B1, const float* __restrict__ B2, int ldb, int K, int n0, float* ls)
{
    constexpr int KT = 32, NV = KT / 16;
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));  // per-call lane offsets: recomputed here, not hoisted and held across calls
    const int w = t >> 6, l = t & 63, r16 = l & 15, g = l >> 4;
    float* const la[3] = {ls, ls + KT * LD, ls + 2 * KT * LD};
    float* const lb[2] = {ls + 3 * KT * LD, ls + 4 * KT * LD};
    f32x4 d[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        d[0][j] = f32x4{p1[0][j], p1[1][j], p1[2][j], p1[3][j]};
        d[1][j] = f32x4{p2[0][j], p2[1][j], p2[2][j], p2[3][j]};
        d[2][j] = f32x4{p3[0][j], p3[1][j], p3[2][j], p3[3][j]};
    }
    constexpr bool A16 = sizeof(TA1) == 2;
    const float* const A[3] = {reinterpret_cast<const float*>(A1), A2, A3};
    const float* const B[2] = {B1, B2};
    f32x4 xa[3][NV], xb[2][NV];
    u16x8 ya;
    auto fetch = [&](int k0) {
        if constexpr (A16) ya = *reinterpret_cast<const u16x8*>(A1 + (int64_t)(t / (KT / 8)) * lda + k0 + 8 * (t % (KT / 8)));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = t + 256 * i;
            const int r = e / (KT / 4), kq = e % (KT / 4);
#pragma unroll
            for (int m = A16 ? 1 : 0; m < 3; ++m)
                xa[m][i] = *reinterpret_cast<const f32x4*>(A[m] + (int64_t)r * lda + k0 + 4 * kq);
            const int kk = e >> 4, nq = e & 15;
#pragma unroll
            for (int m = 0; m < 2; ++m)
                xb[m][i] = *reinterpret_cast<const f32x4*>(B[m] + (int64_t)(k0 + kk) * ldb + n0 + 4 * nq);
        }
    };
    float acc_dot = 0.f;
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += KT) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = t + 256 * i;
            const int r = e / (KT / 4), kq = e % (KT / 4);
#pragma unroll
            for (int m = A16 ? 1 : 0; m < 3; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) la[m][(4 * kq + q) * LD + r] = xa[m][i][q];
#pragma unroll
            for (int m = 0; m < 2; ++m) *reinterpret_cast<f32x4*>(lb[m] + (e >> 4) * LD + 4 * (e & 15)) = xb[m][i];
            acc_dot += xb[0][i].x * xb[1][i].x + xb[0][i].y * xb[1][i].y + xb[0][i].z * xb[1][i].z +
                       xb[0][i].w * xb[1][i].w;
        }
        if constexpr (A16) put8_col(la[0] + (8 * (t % (KT / 8))) * LD + t / (KT / 8), LD, ya);
        __syncthreads();
        if (k0 + KT < K) fetch(k0 + KT);  // the next block's loads fly during these products
#pragma unroll
        for (int kq = 0; kq < KT / 4; ++kq) {
            const int kr = (4 * kq + g) * LD;
            const float a0 = la[0][kr + 16 * w + r16], a1 = la[1][kr + 16 * w + r16], a2 = la[2][kr + 16 * w + r16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float b1 = lb[0][kr + 16 * j + r16], b2 = lb[1][kr + 16 * j + r16];
                d[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, d[0][j], 0, 0, 0);
                d[1][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, d[1][j], 0, 0, 0);
                d[2][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, b2, d[2][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    dot += acc_dot;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p1[i][j] = d[0][j][i];
            p2[i][j] = d[1][j][i];
            p3[i][j] = d[2][j][i];
        }
}

// Per chunk-head slices of the workspace.
struct Slices {
    float *Q, *K, *V, *dO, *rq, *rk, *gam, *bet, *T, *P, *KKG, *U, *E, *dDl, *sck;
    float *S, *Dl, *dS, *dD, *dQ, *dK, *dW, *dPG, *dT, *X1, *Bd;
};

__device__ Slices slices(const BwdArgs& a, int64_t b)
{
    const BwdLayout& L = a.lay;
    unsigned char* ws = a.ws;
    const int64_t cdk = (int64_t)BC * a.dk, cdv = (int64_t)BC * a.dv, cc = BC * BC, dvdk = (int64_t)a.dv * a.dk;
    auto f = [&](size_t off, int64_t per) { return reinterpret_cast<float*>(ws + off) + b * per; };
    Slices s;
    s.Q = f(L.off_Q, cdk);
    s.K = f(L.off_K, cdk);
    s.V = f(L.off_V, cdv);
    s.dO = f(L.off_dO, cdv);
    s.rq = f(L.off_rq, BC);
    s.rk = f(L.off_rk, BC);
    s.gam = f(L.off_gam, BC);
    s.bet = f(L.off_bet, BC);
    s.T = f(L.off_T, cc);
    s.P = f(L.off_P, cc);
    s.KKG = f(L.off_KKG, cc);
    s.U = f(L.off_U, cdv);
    s.E = f(L.off_E, cdv);
    s.sck = f(L.off_sck, BC);
    s.dDl = f(L.off_dDl, cdv);
    s.S = f(L.off_S, dvdk);
    s.Dl = f(L.off_Dl, cdv);
    s.dS = f(L.off_dS, dvdk);
    s.dD = f(L.off_dD, cdv);
    s.dQ = f(L.off_dQ, cdk);
    s.dK = f(L.off_dK, cdk);
    s.dW = f(L.off_dW, cdk);
    s.dPG = f(L.off_dPG, cc);
    s.dT = f(L.off_dT, cc);
    s.X1 = f(L.off_X1, cc);
    s.Bd = f(L.off_Bd, cc);
    return s;
}

// eight consecutive stored elements p[i .. i + 7] (i a multiple of 8), widened
__device__ __forceinline__ void load8(const float* p, int64_t i, f32x4& a, f32x4& b)
{
    a = *reinterpret_cast<const f32x4*>(p + i);
    b = *reinterpret_cast<const f32x4*>(p + i + 4);
}
__device__ __forceinline__ void load8(const uint16_t* p, int64_t i, f32x4& a, f32x4& b)
{
    const u16x8 x = *reinterpret_cast<const u16x8*>(p + i);
    a = f32x4{bf16_bits_to_f32(x[0]), bf16_bits_to_f32(x[1]), bf16_bits_to_f32(x[2]), bf16_bits_to_f32(x[3])};
    b = f32x4{bf16_bits_to_f32(x[4]), bf16_bits_to_f32(x[5]), bf16_bits_to_f32(x[6]), bf16_bits_to_f32(x[7])};
}

// B-operand fragments of a row-major fp32 [BC][d] matrix X for a product
// contracting over the chunk rows, on the bf16 matrix cores with hi/lo
// splits: fragment (ct, ks) gives lane (l16, g) the elements
// X[32 ks + 8 g + e][16 ct + l16], e = 0..7, as bf16 hi and lo parts at
// out + (((ct * 2 + ks) * 2 + part) * 64 + lane) * 8 (HI: the hi parts only,
// for values that bf16 holds exactly).
template <bool HI, typename TX = float>
__device__ void col_frags(const TX* __restrict__ X, int d, uint16_t* __restrict__ out)
{
    for (int task = threadIdx.x; task < (d / 16) * 128; task += 256) {
        const int lane = task & 63, ks = (task >> 6) & 1, ct = task >> 7;
        const int l16 = lane & 15, g = lane >> 4;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = Elem<TX>::load(X, (32 * ks + 8 * g + e) * d + 16 * ct + l16);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) split_bf16x2(x[2 * w], x[2 * w + 1], hi[w], lo[w]);
        uint16_t* p = out + ((size_t)((ct * 2 + ks) * 2) * 64 + lane) * 8;
        *reinterpret_cast<u32x4*>(p) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        if constexpr (!HI) *reinterpret_cast<u32x4*>(p + 512) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
}

// The hi parts of col_frags for bf16 values (exact, so no lo parts), by
// 8 x 8 blocks: a thread loads eight rows of eight consecutive columns (16
// bytes each) and writes the eight lanes' fragments those columns give.
__device__ void col_frags_b16(const uint16_t* __restrict__ X, int d, uint16_t* __restrict__ out)
{
    const int ncg = d / 8;  // groups of eight columns
    for (int task = threadIdx.x; task < 8 * ncg; task += 256) {
        const int cg = task % ncg, rg = task / ncg, ks = rg >> 2, g = rg & 3;
        u16x8 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const u16x8*>(X + (32 * ks + 8 * g + e) * d + 8 * cg);
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int c = 8 * cg + h, ct = c >> 4, lane = (c & 15) + 16 * g;
            u32x4 f;
#pragma unroll
            for (int w = 0; w < 4; ++w) f[w] = (uint32_t)v[2 * w][h] | ((uint32_t)v[2 * w + 1][h] << 16);
            *reinterpret_cast<u32x4*>(out + ((size_t)((ct * 2 + ks) * 2) * 64 + lane) * 8) = f;
        }
    }
}

// col_frags of diag(rscale) X for bf16 X, hi and lo parts, by the same 8 x 8
// blocks (the row scales applied in fp32 before the split).
__device__ void col_frags_b16s(const uint16_t* __restrict__ X, int d, const float* rscale, uint16_t* __restrict__ out)
{
    const int ncg = d / 8;
    for (int task = threadIdx.x; task < 8 * ncg; task += 256) {
        const int cg = task % ncg, rg = task / ncg, ks = rg >> 2, g = rg & 3;
        u16x8 v[8];
        float sc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = *reinterpret_cast<const u16x8*>(X + (32 * ks + 8 * g + e) * d + 8 * cg);
            sc[e] = rscale[32 * ks + 8 * g + e];
        }
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int c = 8 * cg + h, ct = c >> 4, lane = (c & 15) + 16 * g;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int w = 0; w < 4; ++w)
                split_bf16x2(bf16_bits_to_f32(v[2 * w][h]) * sc[2 * w], bf16_bits_to_f32(v[2 * w + 1][h]) * sc[2 * w + 1],
                             hi[w], lo[w]);
            uint16_t* q = out + ((size_t)((ct * 2 + ks) * 2) * 64 + lane) * 8;
            *reinterpret_cast<u32x4*>(q) = u32x4{hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<u32x4*>(q + 512) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
    }
}

// Operand fragments of a row-major fp32 [BC][d] matrix X for a product
// contracting over its columns: fragment (rt, ks) gives lane (l16, g) the
// elements X[16 rt + l16][32 ks + 8 g + e], e = 0..7, as bf16 hi and lo parts
// at out + (((rt * (d / 32) + ks) * 2 + part) * 64 + lane) * 8 (HI: the hi
// parts only).
template <bool HI, typename TX = float>
__device__ void row_frags(const TX* __restrict__ X, int d, uint16_t* __restrict__ out)
{
    const int ksn = d / 32;
    for (int task = threadIdx.x; task < (BC / 16) * ksn * 64; task += 256) {
        const int lane = task & 63, ks = (task >> 6) % ksn, rt = (task >> 6) / ksn;
        const int l16 = lane & 15, g = lane >> 4;
        f32x4 a, b;
        load8(X, (16 * rt + l16) * d + 32 * ks + 8 * g, a, b);
        uint32_t hi[4], lo[4];
        split_bf16x2(a.x, a.y, hi[0], lo[0]);
        split_bf16x2(a.z, a.w, hi[1], lo[1]);
        split_bf16x2(b.x, b.y, hi[2], lo[2]);
        split_bf16x2(b.z, b.w, hi[3], lo[3]);
        uint16_t* p = out + ((size_t)((rt * ksn + ks) * 2) * 64 + lane) * 8;
        *reinterpret_cast<u32x4*>(p) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        if constexpr (!HI) *reinterpret_cast<u32x4*>(p + 512) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
}

__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

// A B with both operands split into bf16 hi + lo: A_hi B_hi + A_lo B_hi + A_hi B_lo
// (the dropped A_lo B_lo is below 2^-16 of the product)
__device__ __forceinline__ f32x4 mma3(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c)
{
    c = mma_bf16(ah, bh, c);
    c = mma_bf16(al, bh, c);
    return mma_bf16(ah, bl, c);
}

// A B with A split into bf16 hi + lo and B exact in bf16: A_hi B + A_lo B
__device__ __forceinline__ f32x4 mma2(u32x4 ah, u32x4 al, u32x4 b, f32x4 c)
{
    c = mma_bf16(ah, b, c);
    return mma_bf16(al, b, c);
}

// eight fp32 values -> bf16 hi and lo operand fragments
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, u32x4& hi, u32x4& lo)
{
    uint32_t h[4], l[4];
    split_bf16x2(a.x, a.y, h[0], l[0]);
    split_bf16x2(a.z, a.w, h[1], l[1]);
    split_bf16x2(b.x, b.y, h[2], l[2]);
    split_bf16x2(b.z, b.w, h[3], l[3]);
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Chunk table: header[0] = 1 if cu_seqlens is invalid (then no chunk is
// processed), header[1] = number of chunks; tab[c] = {first token, length,
// sequence, 0}; seq_first[n] = first chunk of sequence n.
__global__ __launch_bounds__(256) void bwd_table_kernel(const int32_t* __restrict__ cu, int32_t N, int64_t T,
                                                        int64_t max_chunks, int32_t* __restrict__ header,
                                                        int32_t* __restrict__ tab, int32_t* __restrict__ seq_first)
{
    // one workgroup: each thread counts the chunks of a run of sequences, a
    // scan gives their first chunks, then every chunk finds its sequence by a
    // binary search over them
    __shared__ int64_t part[256];
    __shared__ int bad;
    __shared__ int64_t tot_s;
    const int t = threadIdx.x;
    if (t == 0) bad = cu && (cu[0] != 0 || (int64_t)cu[N] != T) ? 1 : 0;
    __syncthreads();
    const int32_t per = (N + 255) / 256, s0 = min(N, t * per), s1 = min(N, s0 + per);
    auto len_of = [&](int32_t n) -> int64_t { return cu ? (int64_t)cu[n + 1] - cu[n] : T; };
    int64_t cnt = 0;
    bool mybad = false;
    for (int32_t n = s0; n < s1; ++n) {
        const int64_t L = len_of(n);
        if (L < 0) mybad = true;
        cnt += (max(L, (int64_t)0) + BC - 1) / BC;
    }
    part[t] = cnt;
    if (mybad) bad = 1;
    __syncthreads();
    if (t == 0) {
        int64_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int64_t c = part[i];
            part[i] = run;
            run += c;
        }
        if (run > max_chunks) bad = 1;  // not for valid input: the chunks number at most T / 64 + N
        tot_s = run;
    }
    __syncthreads();
    const bool ok = !bad;
    const int64_t tot = ok ? tot_s : 0;
    int64_t off = part[t];
    for (int32_t n = s0; n < s1; ++n) {
        seq_first[n] = ok ? (int32_t)off : 0;
        off += (max(len_of(n), (int64_t)0) + BC - 1) / BC;
    }
    if (t == 0) {
        seq_first[N] = (int32_t)tot;
        header[0] = ok ? 0 : 1;
        header[1] = (int32_t)tot;
    }
    __syncthreads();  // seq_first complete
    for (int64_t j = t; j < tot; j += 256) {
        int32_t lo = 0, hi = N - 1;  // the last sequence whose first chunk is <= j (skips empty ones)
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (seq_first[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int64_t p = (cu ? cu[lo] : 0) + (j - seq_first[lo]) * BC, e = cu ? cu[lo + 1] : T;
        tab[4 * j + 0] = (int32_t)p;
        tab[4 * j + 1] = (int32_t)min((int64_t)BC, e - p);
        tab[4 * j + 2] = lo;
        tab[4 * j + 3] = 0;
    }
}

template <typename TIn>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void bwd_local_kernel(BwdArgs a)
{
    const int64_t b = blockIdx.x;
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_header);
    const int32_t* tab = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_tab);
    const int64_t c = b / a.H;
    const int h = (int)(b % a.H);
    if (c >= header[1]) return;
    const int tok0 = tab[4 * c], len = tab[4 * c + 1];
    const int dk = a.dk, dv = a.dv, H = a.H;
    Slices s = slices(a, b);
    // the tile routine's two k-block buffers; A = diag(beta) KKG, from the
    // K K^T product (the last one before the inverse) to the inverse (the
    // first one after it), in the same bytes
    __shared__ __align__(16) float lds_ab[2 * KTL * LD];
    static_assert(BC * (BC + 1) <= 2 * KTL * LD, "A fits the tile buffers");
    float* const as = lds_ab;
    float* const bs = lds_ab + KTL * LD;
    float (*const Am)[BC + 1] = reinterpret_cast<float (*)[BC + 1]>(lds_ab);
    __shared__ float gam[BC], bet[BC], bge[BC], dd[BC], eg[BC], gin[BC], rqs[BC], rks[BC], bgk[BC], esc[BC];
    __shared__ float Ts[BC][BC + 1];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const TIn* q = (const TIn*)a.q;
    const TIn* k = (const TIn*)a.k;
    const TIn* v = (const TIn*)a.v;
    const TIn* dO = (const TIn*)a.dO;

    // chunk-local cumulative log-decay gamma and beta: one row per lane of
    // wave 0 (padded rows add g = 0).  Lane r sums g_0 .. g_r in row order, the
    // running sum's own rounding: a tree scan rounds each gamma_r - gamma_{r-1}
    // differently and measurably loosened the decay gradient.
    if (wv == 0) {
        const bool live = lane < len;
        const int64_t row = (int64_t)(tok0 + (live ? lane : 0)) * H + h;
        gin[lane] = live ? a.g[row] : 0.f;
        const float bt = live ? a.beta[row] : 0.f;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float x = 0.f;
        for (int r = 0; r <= lane; ++r) x += gin[r];
        const float gl = __shfl(x, BC - 1, kWave);
        gam[lane] = x;
        bet[lane] = bt;
        eg[lane] = expf(x);
        dd[lane] = expf(gl - x);
        bge[lane] = bt * expf(x);
        s.gam[lane] = x;
        s.bet[lane] = bt;
    }
    __syncthreads();

    // rows of the chunk, padded with zeros, by 16-byte loads and stores: a row
    // of d elements spreads over d / 8 lanes, eight elements each; wave w takes
    // rows 16 w .. 16 w + 15, up to four rows per lane in flight.  The rows
    // stay raw (in the input type); their L2 norms give the fp32 row scales
    // r_q, r_k and D r_k, which every later product applies in fp32.  With
    // fp32 inputs E = r_q scale e^gamma dO is stored here; with bf16 inputs
    // its fragments come from the bf16 dO copy below.
    const int r_end = 16 * wv + 16;
    {
        const int lpr = dk / 8, rpi = kWave / lpr, sub = lane / lpr, c8 = 8 * (lane % lpr);
        for (int r0 = 16 * wv; r0 < r_end; r0 += 4 * rpi) {
            f32x4 xq[4][2], xk[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i * rpi + sub;
                const bool live = r < len && r0 + i * rpi < r_end;
                const int64_t row = (int64_t)(tok0 + (live ? r : 0)) * H + h;
                if (r0 + i * rpi < r_end) {
                    load8(q, row * dk + c8, xq[i][0], xq[i][1]);
                    load8(k, row * dk + c8, xk[i][0], xk[i][1]);
                }
                if (!live) xq[i][0] = xq[i][1] = xk[i][0] = xk[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (r0 + i * rpi >= r_end) break;
                const int r = r0 + i * rpi + sub;
                float ssq = 0.f, ssk = 0.f;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ssq += xq[i][u][e] * xq[i][u][e];
                        ssk += xk[i][u][e] * xk[i][u][e];
                    }
                for (int m = 1; m < lpr; m <<= 1) {
                    ssq += __shfl_xor(ssq, m, kWave);
                    ssk += __shfl_xor(ssk, m, kWave);
                }
                const float rq = a.l2norm ? 1.0f / sqrtf(ssq + kNormEps) : 1.f;
                const float rk = a.l2norm ? 1.0f / sqrtf(ssk + kNormEps) : 1.f;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int64_t o = (int64_t)r * dk + c8 + 4 * u;
                    if constexpr (sizeof(TIn) != 2) {
                        *reinterpret_cast<f32x4*>(s.Q + o) = xq[i][u];
                        *reinterpret_cast<f32x4*>(s.K + o) = xk[i][u];
                    }
                }
                if constexpr (sizeof(TIn) == 2) {  // the raw rows, exact in bf16
                    const int64_t o = (int64_t)r * dk + c8;
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(s.Q) + o) =
                        u32x4{pack_bf16x2(xq[i][0].x, xq[i][0].y), pack_bf16x2(xq[i][0].z, xq[i][0].w),
                              pack_bf16x2(xq[i][1].x, xq[i][1].y), pack_bf16x2(xq[i][1].z, xq[i][1].w)};
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(s.K) + o) =
                        u32x4{pack_bf16x2(xk[i][0].x, xk[i][0].y), pack_bf16x2(xk[i][0].z, xk[i][0].w),
                              pack_bf16x2(xk[i][1].x, xk[i][1].y), pack_bf16x2(xk[i][1].z, xk[i][1].w)};
                }
                if (c8 == 0) {
                    s.rq[r] = rq;
                    s.rk[r] = rk;
                    s.sck[r] = rk * dd[r];
                    rqs[r] = rq;
                    rks[r] = rk;
                }
            }
        }
    }
    __syncthreads();  // rqs, rks
    if (t < BC) {
        bgk[t] = bge[t] * rks[t];
        esc[t] = a.scale * eg[t] * rqs[t];  // the row scale of E = r_q scale e^gamma dO
    }
    {
        const int lpr = dv / 8, rpi = kWave / lpr, sub = lane / lpr, c8 = 8 * (lane % lpr);
        for (int r0 = 16 * wv; r0 < r_end; r0 += 4 * rpi) {
            f32x4 xv[4][2], xo[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i * rpi + sub;
                const bool live = r < len && r0 + i * rpi < r_end;
                const int64_t row = (int64_t)(tok0 + (live ? r : 0)) * H + h;
                if (r0 + i * rpi < r_end) {
                    load8(v, row * dv + c8, xv[i][0], xv[i][1]);
                    load8(dO, row * dv + c8, xo[i][0], xo[i][1]);
                }
                if (!live) xv[i][0] = xv[i][1] = xo[i][0] = xo[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (r0 + i * rpi >= r_end) break;
                const int r = r0 + i * rpi + sub;
                if constexpr (sizeof(TIn) == 2) {  // V and dO stored as bf16: the values are bf16 inputs, exact
                    const int64_t o = (int64_t)r * dv + c8;
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(s.V) + o) =
                        u32x4{pack_bf16x2(xv[i][0].x, xv[i][0].y), pack_bf16x2(xv[i][0].z, xv[i][0].w),
                              pack_bf16x2(xv[i][1].x, xv[i][1].y), pack_bf16x2(xv[i][1].z, xv[i][1].w)};
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(s.dO) + o) =
                        u32x4{pack_bf16x2(xo[i][0].x, xo[i][0].y), pack_bf16x2(xo[i][0].z, xo[i][0].w),
                              pack_bf16x2(xo[i][1].x, xo[i][1].y), pack_bf16x2(xo[i][1].z, xo[i][1].w)};
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int64_t o = (int64_t)r * dv + c8 + 4 * u;
                    if constexpr (sizeof(TIn) != 2) {
                        *reinterpret_cast<f32x4*>(s.V + o) = xv[i][u];
                        *reinterpret_cast<f32x4*>(s.dO + o) = xo[i][u];
                    }
                    if constexpr (sizeof(TIn) != 2)
                        *reinterpret_cast<f32x4*>(s.E + o) = xo[i][u] * (a.scale * eg[r] * rqs[r]);
                }
            }
        }
    }
    __syncthreads();  // also publishes the rows written above to the whole workgroup

    const int tr = t >> 4, tc = t & 15;
    float acc[4][4];
    // The Q and K slots hold the raw rows (the input type; bf16 exact): the
    // normalised K^ = diag(r_k) k and Q^ = diag(r_q) q take their row scales
    // in fp32, on the products' rows and columns or folded into the k scale.
    const TIn* sQ = reinterpret_cast<const TIn*>(s.Q);
    const TIn* sK = reinterpret_cast<const TIn*>(s.K);
    // Q K^T -> P = lower(Q K^T o Gamma)
    zero(acc);
    mm64<KTL, true, false, TIn, TIn>(acc, sQ, dk, nullptr, sK, dk, dk, 0, as, bs);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * tr + i, n = 16 * j + tc;
            s.P[r * BC + n] = n <= r ? acc[i][j] * (rqs[r] * rks[n]) * expf(gam[r] - gam[n]) : 0.f;
        }
    // K K^T -> KKG = strict_lower(K K^T o Gamma), A = diag(beta) KKG
    zero(acc);
    mm64<KTL, true, false, TIn, TIn>(acc, sK, dk, nullptr, sK, dk, dk, 0, as, bs);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * tr + i, n = 16 * j + tc;
            const float x = n < r ? acc[i][j] * (rks[r] * rks[n]) * expf(gam[r] - gam[n]) : 0.f;
            s.KKG[r * BC + n] = x;
            Am[r][n] = bet[r] * x;
        }
    __syncthreads();
    // T = (I + A)^{-1} by forward substitution.  Column c of T depends only on
    // its own earlier rows, T[r][c] = [r == c] - sum_{j < r} A[r][j] T[j][c],
    // so four lanes of one wave own a column with no barrier: lane q keeps
    // T[4 m + q][c] (m < 16) in registers and sums the terms j = q mod 4; a
    // swap within the quad adds the four sums (the same bits in every lane).
    {
        const int tcol = 16 * wv + (lane >> 2), q = lane & 3;
        float Tq[BC / 4];
#pragma unroll
        for (int m = 0; m < BC / 4; ++m) Tq[m] = 0.f;
#pragma unroll
        for (int r = 0; r < BC; ++r) {
            float part = 0.f;
#pragma unroll
            for (int m = 0; 4 * m < r; ++m)
                if (4 * m + q < r) part += Am[r][4 * m + q] * Tq[m];
            part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0xB1, 0xF, 0xF, false));
            part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0x4E, 0xF, 0xF, false));
            const float x = (r == tcol ? 1.f : 0.f) - part;
            if (q == (r & 3)) Tq[r >> 2] = x;
        }
#pragma unroll
        for (int m = 0; m < BC / 4; ++m) Ts[4 * m + q][tcol] = Tq[m];
    }
    __syncthreads();
    for (int e = t; e < BC * BC; e += 256) s.T[e] = Ts[e >> 6][e & 63];
    __syncthreads();
    // W = T diag(beta e^gamma) K by 64-column blocks, each staged in LDS (Ts is
    // free now) and written out only as the chains' hi/lo fragments: the
    // column fragments (Wf, the reverse chain's Z) and the row fragments (Wr,
    // the forward chain's Y) of its columns, with no fp32 W in the workspace
    const int64_t fper = (int64_t)BC * dk * 2;
    {
        uint16_t* const wf = reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Wf) + b * fper;
        uint16_t* const wr = reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Wr) + b * fper;
        const int ksn = dk / 32;
        for (int n0 = 0; n0 < dk; n0 += 64) {
            zero(acc);
            mm64<KTL, true, true, float, TIn>(acc, s.T, BC, bgk, sK, dk, BC, n0, as, bs);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) Ts[4 * tr + i][16 * j + tc] = acc[i][j];
            __syncthreads();
            // tasks 0..511: column fragment (tile n0/16 + task/128, k-step (task/64)%2);
            // 512..1023: row fragment (row tile (task-512)/128, k-step n0/32 + (task/64)%2)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int task = t + 256 * q, fl = task & 63, kl = (task >> 6) & 1, tl = (task >> 7) & 3;
                const int fl16 = fl & 15, fg = fl >> 4;
                float x[8];
                uint16_t* p;
                if (q < 2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = Ts[32 * kl + 8 * fg + e][16 * tl + fl16];
                    p = wf + ((size_t)(((n0 / 16 + tl) * 2 + kl) * 2) * 64 + fl) * 8;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = Ts[16 * tl + fl16][32 * kl + 8 * fg + e];
                    p = wr + ((size_t)((tl * ksn + n0 / 32 + kl) * 2) * 64 + fl) * 8;
                }
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) split_bf16x2(x[2 * w2], x[2 * w2 + 1], hi[w2], lo[w2]);
                *reinterpret_cast<u32x4*>(p) = u32x4{hi[0], hi[1], hi[2], hi[3]};
                *reinterpret_cast<u32x4*>(p + 512) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            }
            __syncthreads();  // Ts read: free for the next block
        }
    }
    // U = T diag(beta) V
    for (int n0 = 0; n0 < dv; n0 += 64) {
        zero(acc);
        mm64<KTL, true, true, float, TIn>(acc, s.T, BC, bet, reinterpret_cast<const TIn*>(s.V), dv, BC, n0, as, bs);
        float acc2[4][4];
        zero(acc2);
        mm64<KTL, false, true, float, TIn>(acc2, s.P, BC, nullptr, reinterpret_cast<const TIn*>(s.dO), dv, BC, n0, as,
                                           bs);  // P^T dO
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * tr + i, n = n0 + 16 * j + tc;
                s.U[r * dv + n] = acc[i][j];
                s.dDl[r * dv + n] = a.scale * acc2[i][j];
            }
    }
    // the other operands of the chains, as bf16 hi/lo fragments
    __syncthreads();
    constexpr bool RAW_EXACT = sizeof(TIn) == 2;  // bf16 inputs: raw k and q are exact in bf16
    if constexpr (RAW_EXACT) {
        col_frags_b16(reinterpret_cast<const uint16_t*>(sK), dk, reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Kf) + b * fper);
        col_frags_b16(reinterpret_cast<const uint16_t*>(sQ), dk, reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Qf) + b * fper);
    } else {
        col_frags<false>(sK, dk, reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Kf) + b * fper);
        col_frags<false>(sQ, dk, reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Qf) + b * fper);
    }
    if constexpr (RAW_EXACT)  // E from the bf16 dO copy, its row scale applied in fp32
        col_frags_b16s(reinterpret_cast<const uint16_t*>(s.dO), dv, esc,
                       reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Ef) + b * (int64_t)BC * dv * 2);
    else
        col_frags<false>(s.E, dv, reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Ef) + b * (int64_t)BC * dv * 2);
    row_frags<RAW_EXACT>(sK, dk, reinterpret_cast<uint16_t*>(a.ws + a.lay.off_Kr) + b * fper);
}

// One row-split recurrence over the chunks of each sequence (see the header):
//     Delta = X + ysign Y S^T                 (C x 16 rows of this workgroup)
//     S    <- e^{gamma_L} S + zsign Delta^T Z + E^T F
// storing S before each chunk (S_store) and Delta (D_store).  A workgroup owns
// 16 rows of one (sequence, head) state; its four waves run both products on
// the bf16 matrix cores with hi/lo splits of both operands (three products
// per fragment pair, relative error ~2^-16, the fp32 path's level):
//   - S Y^T (16 x 64, K = DK): wave w computes chunk rows 16 w .. 16 w + 15,
//     A = S (the state rows from LDS), B = Y^T (its 16 rows of Y, registers);
//   - Delta^T Z + E^T F (16 x DK, K = 64): wave w owns the DK/4 state columns
//     w DK/4 .. in registers in the accumulator layout (lane l: rows
//     4 (l / 16) + i, column l % 16 of each 16-column tile); A = Delta^T and
//     E^T (both from LDS), B = Z and F as the local kernel's column
//     fragments (registers).
// Every wave loads only its quarter of each operand, straight into registers,
// right after its last use: the next chunk's Y during the update, the next Z,
// F and E during the following products.  E^T is the same for all four waves,
// so each loads a quarter of its fragments and stages it in LDS.  Two
// barriers per chunk (the state rows, Delta and E^T cross the waves through
// LDS).
// The operands of one direction of the chain (workspace byte offsets; E and
// F absent when their offset is 0; Zf and Ff are fragment arrays).
struct ChainOps {
    size_t off_X, off_Yr, off_Zf, off_Ef, off_Ff, off_Sst, off_Dst;
    const float* S_init;  // [N][H][dv][dk] or NULL (zeros)
    float* S_final;       // [N][H][dv][dk] or NULL
    float ysign, zsign;
    int reverse;
};

// The forward and the reverse recurrence need nothing from each other (only
// the gradient kernel reads both), so one launch runs them side by side.
// Workgroup -> (direction and pair, row block): the dv/16 row blocks of one
// (direction, sequence, head) sit 8 workgroups apart, so they share one XCD
// and its L2 copy of the chunk operands (the reverse chains first).
template <int DK, bool EXACT>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdArgs a, ChainOps rev_ops, ChainOps fwd_ops)
{
    constexpr int P = DK + 4;   // LDS pitch of the state rows (floats)
    constexpr int DP = BC + 4;  // LDS pitch of Delta^T
    constexpr int NT = DK / 64;  // 16-column state tiles per wave
    constexpr int DKS = DK / 32;  // k-steps over d_k
    static_assert(BC == 64, "two k-steps over the chunk");
    const int dv = a.dv, H = a.H;
    const int RB = dv / 16;
    const int64_t NP = (int64_t)a.N * H;
    const int xcd = (int)(blockIdx.x & 7);
    const int64_t slot = blockIdx.x >> 3;
    const int64_t sidx = xcd + 8 * (slot / RB);
    const int rb = (int)(slot % RB);
    if (sidx >= 2 * NP) return;
    const bool is_rev = sidx < NP;
    const ChainOps op = is_rev ? rev_ops : fwd_ops;
    const int64_t pair = is_rev ? sidx : sidx - NP;
    const float ysign = op.ysign, zsign = op.zsign;
    const float* __restrict__ S_init = op.S_init;
    float* __restrict__ S_final = op.S_final;
    const int reverse = op.reverse;
    const int n = (int)(pair / H), h = (int)(pair % H);
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, g = lane >> 4;
    const int32_t* seq_first = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_seq_first);
    const float* gamv = reinterpret_cast<const float*>(a.ws + a.lay.off_gam);
    auto wsf = [&](size_t off) { return reinterpret_cast<float*>(a.ws + off); };
    const float* Xb = wsf(op.off_X);
    const uint16_t* Yr = reinterpret_cast<const uint16_t*>(a.ws + op.off_Yr);
    const uint16_t* Zf = reinterpret_cast<const uint16_t*>(a.ws + op.off_Zf);
    const uint16_t* Ef = op.off_Ef ? reinterpret_cast<const uint16_t*>(a.ws + op.off_Ef) : nullptr;
    const uint16_t* Ff = op.off_Ff ? reinterpret_cast<const uint16_t*>(a.ws + op.off_Ff) : nullptr;
    float* Sst = wsf(op.off_Sst);
    float* Dst = wsf(op.off_Dst);
    constexpr int PB = DK + 8;  // LDS pitch of the bf16 state rows (elements)
    __shared__ __align__(16) float Ssh[16 * P];   // state rows before the chunk
    __shared__ __align__(16) uint16_t Sbh[16 * PB], Sbl[16 * PB];  // the same rows, bf16 hi and lo
    __shared__ __align__(16) float dsm[16 * DP];  // Delta^T [state row][chunk row]
    __shared__ __align__(16) uint16_t Esh[4 * 512];  // (reverse) E^T fragments of the chunk: (k-step, hi / lo) x 1 KB

    // this wave's operand quarters, one chunk ahead.  K^ and Q^ enter as raw
    // rows (Y of the reverse direction, Z of the forward one, F): their row
    // scales D r_k are applied in fp32, to the product S Y^T in reverse and to
    // Delta^T forward, and r_q is folded into E.  With bf16 inputs (EXACT) the
    // raw rows are exact in bf16, so only their hi parts are loaded and
    // multiplied: two products per fragment pair instead of three.
    u32x4 yr[DKS][2];     // Y fragments of chunk rows 16 w .., k-step ks, hi / lo
    u32x4 zr[NT][2][2];   // Z fragments of column tiles w NT + tt, k-step ks, hi / lo
    u32x4 fr[NT][2][2];   // F fragments, likewise
    u32x4 eq;             // (reverse) this wave's quarter of the E^T fragments, staged in LDS for all four
    f32x4 xr;             // X[16 w + l16][16 rb + 4 g .. + 3]
    float gl = 0.f;       // gamma_L of the chunk
    float scv = 1.f;      // D r_k of chunk row 16 w + l16
    const float* scb = wsf(a.lay.off_sck);
    const int64_t fper = (int64_t)BC * DK * 2;
    // (REV: the reverse direction, whose Y and F are raw rows; the forward
    // direction's Z is)
    auto load_y = [&](int64_t ch, auto rev_c) {
        constexpr int NPART = decltype(rev_c)::value && EXACT ? 1 : 2;
        const uint16_t* p = Yr + ch * fper + lane * 8;
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks)
#pragma unroll
            for (int part = 0; part < NPART; ++part)
                yr[ks][part] = *reinterpret_cast<const u32x4*>(p + ((w * DKS + ks) * 2 + part) * 512);
        xr = *reinterpret_cast<const f32x4*>(Xb + (ch * BC + 16 * w + l16) * dv + rb * 16 + 4 * g);
        gl = gamv[ch * BC + BC - 1];
        scv = scb[ch * BC + 16 * w + l16];
    };
    auto load_z = [&](int64_t ch, auto rev_c) {
        constexpr int NPART = !decltype(rev_c)::value && EXACT ? 1 : 2;
        const uint16_t* p = Zf + ch * fper + lane * 8;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int part = 0; part < NPART; ++part)
                    zr[tt][ks][part] = *reinterpret_cast<const u32x4*>(p + (((w * NT + tt) * 2 + ks) * 2 + part) * 512);
    };
    auto load_f = [&](int64_t ch) {
        constexpr int NPART = EXACT ? 1 : 2;
        const uint16_t* p = Ff + ch * fper + lane * 8;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int part = 0; part < NPART; ++part)
                    fr[tt][ks][part] = *reinterpret_cast<const u32x4*>(p + (((w * NT + tt) * 2 + ks) * 2 + part) * 512);
        // fragment (k-step, part) = (w / 2, w % 2) of this row block
        eq = *reinterpret_cast<const u32x4*>(Ef + ch * (int64_t)BC * dv * 2 + (rb * 4 + w) * 512 + lane * 8);
    };

    // L2 prefetch two chunks ahead: the operand bytes the chain reads for one
    // chunk (Y, Z, F and E; of a hi-only operand its hi parts, every other
    // 1 KB block), cut into 1 KB pieces, this workgroup's share of the pair's
    // pieces, one 4-byte load per lane at a 16-byte stride (a word of each
    // 16 bytes brings all of the piece's cache lines into L2); the loaded
    // words are folded into a register two chunks later (kept alive to the
    // end), so no wait is added before they arrive.  (16-byte loads of which
    // only two words were folded left the other two registers free at once:
    // the compiler reused them and waited for every load in flight, a full
    // memory round trip on every step.)  A piece beyond this workgroup's
    // share reloads the chunk's first Y piece: every lane loads on every
    // step, with no branch around the loads.
    constexpr int OPB = BC * DK * 4 / 1024;  // 1 KB blocks of one d_k operand (hi and lo)
    const int eb = BC * dv * 4 / 1024;       // of E
    uint32_t pf_acc = 0;
    uint32_t pf[2][4];
    auto prefetch = [&](int64_t ch, uint32_t* dst, auto rev_c) {
        constexpr bool REV = decltype(rev_c)::value;
        constexpr int SY = REV && EXACT ? 2 : 1, SZ = !REV && EXACT ? 2 : 1, SF = EXACT ? 2 : 1;
        constexpr int NY = OPB / SY, NZ = OPB / SZ, NF = REV ? OPB / SF : 0;
        const int npiece = NY + NZ + NF + (REV ? eb : 0);
        const int per_wg = (npiece + RB - 1) / RB, per_wave = (per_wg + 3) / 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q0 = rb * per_wg + w * per_wave + i;
            const bool mine = i < per_wave && q0 < npiece && (w * per_wave + i) < per_wg;
            const int q = mine ? q0 : 0;
            const uint16_t* base = q < NY ? Yr : q < NY + NZ ? Zf : q < NY + NZ + NF ? Ff : Ef;
            const int64_t per = q < NY + NZ + NF ? fper : (int64_t)BC * dv * 2;
            const int blk = q < NY ? q * SY : q < NY + NZ ? (q - NY) * SZ : q < NY + NZ + NF ? (q - NY - NZ) * SF
                                                                                           : q - NY - NZ - NF;
            const unsigned char* src = reinterpret_cast<const unsigned char*>(base + ch * per) + blk * 1024;
            dst[i] = *reinterpret_cast<const uint32_t*>(src + lane * 16);
        }
    };

    // this wave's state columns, accumulator layout
    f32x4 sreg[NT];
    const int64_t sbase = (int64_t)(n * H + h) * dv + rb * 16;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sreg[tt][i] = S_init ? S_init[(sbase + 4 * g + i) * DK + w * (DK / 4) + 16 * tt + l16] : 0.f;
    const int c0 = seq_first[n], c1 = seq_first[n + 1];
    const int steps = c1 - c0;
    auto chunk_of = [&](int it) -> int64_t { return (int64_t)(reverse ? c1 - 1 - it : c0 + it) * H + h; };
    // one chunk; the loop below runs two per iteration, so that each uses a
    // fixed prefetch slot (a slot picked by it & 1 is a dynamic register index,
    // which the compiler serves with a wait for every load in flight)
    auto chunk_step = [&](int it, uint32_t* slot, auto rev_c) __attribute__((always_inline)) {
        constexpr bool REV = decltype(rev_c)::value;
        const int64_t ch = chunk_of(it);
        {
#pragma unroll
            for (int i = 0; i < 4; ++i) pf_acc ^= slot[i];
            prefetch(chunk_of(min(it + 2, steps - 1)), slot, rev_c);
        }
        // the state before the chunk: to LDS in fp32 (for the record) and split
        // into bf16 hi and lo (the A operand of S Y^T), then from its rows to the
        // record, 16 bytes per lane
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int at = (4 * g + i), col = w * (DK / 4) + 16 * tt + l16;
                const float x = sreg[tt][i];
                const uint16_t hb = __builtin_bit_cast(uint16_t, (__bf16)x);
                const float hf = __uint_as_float((uint32_t)hb << 16);
                Ssh[at * P + col] = x;
                Sbh[at * PB + col] = hb;
                Sbl[at * PB + col] = __builtin_bit_cast(uint16_t, (__bf16)(x - hf));
            }
        __syncthreads();  // ---- the state rows in LDS; the previous chunk's Delta readers are done
#pragma unroll
        for (int i = 0; i < 16 * DK / 4 / 256; ++i) {
            const int u = t + 256 * i, row = u / (DK / 4), c4 = u % (DK / 4);
            *reinterpret_cast<f32x4*>(Sst + (ch * dv + rb * 16 + row) * DK + 4 * c4) =
                *reinterpret_cast<const f32x4*>(Ssh + row * P + 4 * c4);
        }
        // (S Y^T)[state row][chunk row 16 w + l16], the three hi/lo products in
        // three accumulators
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) {
            const u32x4 sh = *reinterpret_cast<const u32x4*>(Sbh + l16 * PB + 32 * ks + 8 * g);
            const u32x4 sl = *reinterpret_cast<const u32x4*>(Sbl + l16 * PB + 32 * ks + 8 * g);
            a0 = mma_bf16(sh, yr[ks][0], a0);
            a1 = mma_bf16(sl, yr[ks][0], a1);
            if constexpr (!(REV && EXACT)) a2 = mma_bf16(sh, yr[ks][1], a2);
        }
        const f32x4 acc = a0 + a1 + a2;
        // lane holds state rows 4 g + i of chunk row 16 w + l16; in reverse Y is
        // the raw k rows (the product takes their scale D r_k here), forward
        // Delta^T takes it for the raw k rows of Z
        const f32x4 d = REV ? xr + ysign * (acc * scv) : xr + ysign * acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) dsm[(4 * g + i) * DP + 16 * w + l16] = REV ? d[i] : d[i] * scv;
        *reinterpret_cast<f32x4*>(Dst + (ch * BC + 16 * w + l16) * dv + rb * 16 + 4 * g) = d;
        const float decay = expf(gl);
        if constexpr (REV) *reinterpret_cast<u32x4*>(Esh + w * 512 + lane * 8) = eq;
        load_y(chunk_of(min(it + 1, steps - 1)), rev_c);
        __syncthreads();  // ---- Delta^T and E^T in LDS; the state rows read
        u32x4 er[2][2];
        if constexpr (REV)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int part = 0; part < 2; ++part)
                    er[ks][part] = *reinterpret_cast<const u32x4*>(Esh + (ks * 2 + part) * 512 + lane * 8);
        // S <- e^{gamma_L} S + zsign Delta^T Z (+ E^T F)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) sreg[tt] *= decay;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const float* dp = dsm + l16 * DP + 32 * ks + 8 * g;
            u32x4 dh, dl;
            split8(zsign * *reinterpret_cast<const f32x4*>(dp), zsign * *reinterpret_cast<const f32x4*>(dp + 4), dh, dl);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                sreg[tt] = !REV && EXACT ? mma2(dh, dl, zr[tt][ks][0], sreg[tt])
                                         : mma3(dh, dl, zr[tt][ks][0], zr[tt][ks][1], sreg[tt]);
        }
        load_z(chunk_of(min(it + 1, steps - 1)), rev_c);
        if constexpr (REV) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    sreg[tt] = EXACT ? mma2(er[ks][0], er[ks][1], fr[tt][ks][0], sreg[tt])
                                     : mma3(er[ks][0], er[ks][1], fr[tt][ks][0], fr[tt][ks][1], sreg[tt]);
            load_f(chunk_of(min(it + 1, steps - 1)));
        }
    };
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 4; ++i) pf[b2][i] = 0u;
    // the two directions as separate loops: the E^T F term, the raw-row
    // operands and their loads are compiled in or out, never branched around
    auto run = [&](auto rev_c) __attribute__((always_inline)) {
        if (steps > 0) {
            load_y(chunk_of(0), rev_c);
            load_z(chunk_of(0), rev_c);
            if constexpr (decltype(rev_c)::value) load_f(chunk_of(0));
        }
        for (int it = 0; it < steps; it += 2) {
            chunk_step(it, pf[0], rev_c);
            if (it + 1 < steps) chunk_step(it + 1, pf[1], rev_c);
        }
    };
    if (is_rev)
        run(std::true_type{});
    else
        run(std::false_type{});
    if (S_final)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S_final[(sbase + 4 * g + i) * DK + w * (DK / 4) + 16 * tt + l16] = sreg[tt][i];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 4; ++i) pf_acc ^= pf[b2][i];
    asm volatile("" ::"v"(pf_acc));  // the prefetched words stay live: the loads are kept
}

template <typename TIn>
__global__ __launch_bounds__(256, 3) void bwd_grad_kernel(BwdArgs a)
{
    const int64_t b = blockIdx.x;
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_header);
    const int32_t* tab = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_tab);
    const int64_t c = b / a.H;
    const int h = (int)(b % a.H);
    if (c >= header[1]) return;
    const int tok0 = tab[4 * c], len = tab[4 * c + 1];
    const int dk = a.dk, dv = a.dv, H = a.H;
    const float scale = a.scale;
    Slices s = slices(a, b);
    // V and dO as the local kernel stored them: the input type (bf16 exact)
    const TIn* sV = reinterpret_cast<const TIn*>(s.V);
    const TIn* sdO = reinterpret_cast<const TIn*>(s.dO);
    // and Q, K as the raw rows: Q^ = diag(r_q) q, K^ = diag(r_k) k take their
    // row scales (rqv, rkv) in fp32, folded into the k scale of the products
    // that contract over the chunk rows, on output columns or row sums else
    const TIn* sQ = reinterpret_cast<const TIn*>(s.Q);
    const TIn* sK = reinterpret_cast<const TIn*>(s.K);
    // the fused pass over S and dS stages five tiles; the 64 x 64 tile routine
    // of the other products (never live at the same time) uses two of them
    __shared__ __align__(16) float ls3[5 * 32 * LD];
    float* const as = ls3;
    float* const bs = ls3 + KTG * LD;
    __shared__ float gam[BC], bet[BC], eg[BC], dd[BC], bge[BC], dgam[BC], dbet[BC], rqv[BC], rkv[BC];
    __shared__ float red[4];
    __shared__ float cs[16][BC];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int tr = t >> 4, tc = t & 15;
    if (t < BC) {
        gam[t] = s.gam[t];
        rqv[t] = s.rq[t];
        rkv[t] = s.rk[t];
        bet[t] = s.bet[t];
        dgam[t] = 0.f;
        dbet[t] = 0.f;
    }
    __syncthreads();
    if (t < BC) {
        eg[t] = expf(gam[t]);
        dd[t] = expf(gam[BC - 1] - gam[t]);
        bge[t] = bet[t] * eg[t];
    }
    __syncthreads();
    float acc[4][4];
    float rowp[4];

    // Reductions in a fixed order (the results do not depend on scheduling):
    // a row r = 4 tr + i of a 64 x 64 block belongs to the 16 lanes of one tr,
    // whose lane tc = 0 is its only writer; column sums go through cs.
    auto row_add = [&](float* dst, float sgn) {  // dst[r] += sgn * rowp[i] summed over the 16 lanes of a row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = group_sum<16>(rowp[i]);
            if (tc == 0) dst[4 * tr + i] += sgn * x;
        }
    };
    auto col_sub = [&](float* dst, const float colp[4]) {  // dst[n] -= column n summed over all rows
#pragma unroll
        for (int j = 0; j < 4; ++j) cs[tr][16 * j + tc] = colp[j];
        __syncthreads();
        if (t < BC) {
            float x = 0.f;
            for (int i = 0; i < 16; ++i) x += cs[i][t];
            dst[t] -= x;
        }
        __syncthreads();
    };

    // One pass over the 64-column blocks of S and dS: each block crosses from
    // memory once for the three products that read it,
    //   dO S -> the first term of dQ,  -dDelta S -> dW,  Delta dS -> the first term of dK,
    // and e^{gamma_L} <dS, S> (part of the gradient of gamma_L) from the same
    // registers.  dQ and dK are stored partial here and completed below; the
    // row sums Q_r . (scale e^gamma dO S)_r -> dgamma_r and K_r . (Delta dS)_r ->
    // -D_r dgamma_r and gamma_L are taken now.
    float dgL = 0.f;
    float rq[4] = {0.f, 0.f, 0.f, 0.f}, rk[4] = {0.f, 0.f, 0.f, 0.f}, rt[4] = {0.f, 0.f, 0.f, 0.f};
    {
        float dot = 0.f;
        for (int n0 = 0; n0 < dk; n0 += 64) {
            float pq[4][4], pw[4][4];
            zero(acc);
            zero(pq);
            zero(pw);
            mm64x3(pq, pw, acc, dot, sdO, s.dD, s.Dl, dv, s.S, s.dS, dk, dv, n0, ls3);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * tr + i, n = n0 + 16 * j + tc;
                    const float x = scale * eg[r] * pq[i][j];
                    rq[i] += Elem<TIn>::load(sQ, r * dk + n) * x;
                    s.dQ[r * dk + n] = x;
                    s.dW[r * dk + n] = -pw[i][j];
                    rk[i] += Elem<TIn>::load(sK, r * dk + n) * acc[i][j];
                    s.dK[r * dk + n] = dd[r] * acc[i][j];
                }
        }
        dgL += expf(gam[BC - 1]) * dot;
    }
    // dP = scale lower(dO Delta^T);  dgamma from P;  dPG = dP o Gamma
    zero(acc);
    mm64<KTG, true, false, TIn>(acc, sdO, dv, nullptr, s.Dl, dv, dv, 0, as, bs);
    {
        float colp[4] = {0.f, 0.f, 0.f, 0.f};
        rowp[0] = rowp[1] = rowp[2] = rowp[3] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * tr + i, n = 16 * j + tc;
                const float dp = n <= r ? scale * acc[i][j] : 0.f;
                const float m = dp * s.P[r * BC + n];
                rowp[i] += m;
                colp[j] += m;
                s.dPG[r * BC + n] = n <= r ? dp * expf(gam[r] - gam[n]) : 0.f;
            }
        row_add(dgam, 1.f);
        col_sub(dgam, colp);  // its barriers also complete dPG
    }
    __syncthreads();  // dW complete
    // dT = (dDelta V^T) diag(beta) + (dW K^T) diag(beta e^gamma)
    {
        zero(acc);
        mm64<KTG, true, false, float, TIn>(acc, s.dD, dv, nullptr, sV, dv, dv, 0, as, bs);
        float acc2[4][4];
        zero(acc2);
        mm64<KTG, true, false, float, TIn>(acc2, s.dW, dk, nullptr, sK, dk, dk, 0, as, bs);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * tr + i, n = 16 * j + tc;
                s.dT[r * BC + n] = acc[i][j] * bet[n] + acc2[i][j] * (bge[n] * rkv[n]);
            }
    }
    // dV = diag(beta) T^T dDelta;  dbeta_r += (T^T dDelta)_r . V_r
    rowp[0] = rowp[1] = rowp[2] = rowp[3] = 0.f;
    for (int n0 = 0; n0 < dv; n0 += 64) {
        zero(acc);
        mm64<KTG, false, true>(acc, s.T, BC, nullptr, s.dD, dv, BC, n0, as, bs);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * tr + i, n = n0 + 16 * j + tc;
                rowp[i] += acc[i][j] * Elem<TIn>::load(sV, r * dv + n);
                if (r < len) a.dv_out[((int64_t)(tok0 + r) * H + h) * dv + n] = bet[r] * acc[i][j];
            }
    }
    row_add(dbet, 1.f);
    __syncthreads();  // dT complete
    // X1 = dT T^T
    zero(acc);
    mm64<KTG, true, false>(acc, s.dT, BC, nullptr, s.T, BC, BC, 0, as, bs);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s.X1[(4 * tr + i) * BC + 16 * j + tc] = acc[i][j];
    __syncthreads();
    // dA = -strict_lower(T^T X1);  Bd = diag(beta) (dA o Gamma);  dbeta, dgamma from A
    zero(acc);
    mm64<KTG, false, true>(acc, s.T, BC, nullptr, s.X1, BC, BC, 0, as, bs);
    {
        float colp[4] = {0.f, 0.f, 0.f, 0.f};
        float rowb[4] = {0.f, 0.f, 0.f, 0.f};
        rowp[0] = rowp[1] = rowp[2] = rowp[3] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * tr + i, n = 16 * j + tc;
                const float da = n < r ? -acc[i][j] : 0.f;
                const float kkg = s.KKG[r * BC + n];  // zero unless n < r
                const float m = da * bet[r] * kkg;  // dA o A
                rowb[i] += da * kkg;
                rowp[i] += m;
                colp[j] += m;
                s.Bd[r * BC + n] = n < r ? bet[r] * da * expf(gam[r] - gam[n]) : 0.f;
            }
        row_add(dgam, 1.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) rowp[i] = rowb[i];
        row_add(dbet, 1.f);
        col_sub(dgam, colp);  // its barriers also complete Bd
    }
    // dQ and dK (before the norms) completed one 64-column block at a time,
    // onto the partial blocks of the pass above:
    //   dQ += dPG K
    //   dK += diag(beta e^gamma) T^T dW + dPG^T Q + Bd K + Bd^T K
    // with the row sums (T^T dW)_r . K_r -> dbeta, dgamma.
    for (int n0 = 0; n0 < dk; n0 += 64) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = s.dQ[(4 * tr + i) * dk + n0 + 16 * j + tc];
        mm64<KTG, true, true, float, TIn>(acc, s.dPG, BC, rkv, sK, dk, BC, n0, as, bs);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s.dQ[(4 * tr + i) * dk + n0 + 16 * j + tc] = acc[i][j];

        float acc2[4][4];
        zero(acc2);
        mm64<KTG, false, true>(acc2, s.T, BC, nullptr, s.dW, dk, BC, n0, as, bs);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * tr + i, n = n0 + 16 * j + tc;
                rt[i] += Elem<TIn>::load(sK, r * dk + n) * acc2[i][j];
                acc[i][j] = s.dK[r * dk + n] + bge[r] * acc2[i][j];
            }
        mm64<KTG, false, true, float, TIn>(acc, s.dPG, BC, rqv, sQ, dk, BC, n0, as, bs);
        mm64<KTG, true, true, float, TIn>(acc, s.Bd, BC, rkv, sK, dk, BC, n0, as, bs);
        mm64<KTG, false, true, float, TIn>(acc, s.Bd, BC, rkv, sK, dk, BC, n0, as, bs);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s.dK[(4 * tr + i) * dk + n0 + 16 * j + tc] = acc[i][j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * tr + i;
        const float xq = rqv[r] * group_sum<16>(rq[i]), xk = rkv[r] * group_sum<16>(rk[i]),
                    xt = rkv[r] * group_sum<16>(rt[i]);
        if (tc == 0) {
            dgam[r] += xq - xk * dd[r] + bge[r] * xt;
            dbet[r] += eg[r] * xt;
            dgL += xk * dd[r];
        }
    }
    dgL = group_sum<64>(dgL);
    if (lane == 0) red[wv] = dgL;
    __syncthreads();  // dQ, dK, dgam, dbet complete
    // dg: reverse cumulative sum of dgamma (gamma_L is the last, padded-constant, entry)
    // (lane r of wave 0 adds dgamma_63 .. dgamma_r in that order: the serial
    // sum's own rounding, every row at once)
    if (wv == 0) {
        float run = red[0] + red[1] + red[2] + red[3];
        for (int j = BC - 1; j >= lane; --j) run += dgam[j];
        if (lane < len) {
            const int64_t row = (int64_t)(tok0 + lane) * H + h;
            a.dg[row] = run;
            a.dbeta[row] = dbet[lane];
        }
    }
    // through the L2 norms: dx = r (dx^ - x^ (x^ . dx^)).  A row of d_k values
    // spreads over d_k / 8 lanes, eight each, by 16-byte loads and stores;
    // wave w takes rows 16 w .. 16 w + 15, two rows per lane in flight.
    {
        const int lpr = dk / 8, rpi = kWave / lpr, sub = lane / lpr, c8 = 8 * (lane % lpr);
        const int r_end = 16 * wv + 16;
        for (int r0 = 16 * wv; r0 < r_end; r0 += 2 * rpi) {
            f32x4 xq[2][2], gq[2][2], xk[2][2], gk[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = min(r0 + i * rpi, r_end - rpi) + sub;
                load8(sQ, r * dk + c8, xq[i][0], xq[i][1]);
                load8(sK, r * dk + c8, xk[i][0], xk[i][1]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int o = r * dk + c8 + 4 * u;
                    xq[i][u] *= rqv[r];  // the normalised rows
                    xk[i][u] *= rkv[r];
                    gq[i][u] = *reinterpret_cast<const f32x4*>(s.dQ + o);
                    gk[i][u] = *reinterpret_cast<const f32x4*>(s.dK + o);
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (r0 + i * rpi >= r_end) break;  // wave-uniform
                const int r = r0 + i * rpi + sub;
                float pq = 0.f, pk = 0.f;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pq += xq[i][u][e] * gq[i][u][e];
                        pk += xk[i][u][e] * gk[i][u][e];
                    }
                for (int m = 1; m < lpr; m <<= 1) {
                    pq += __shfl_xor(pq, m, kWave);
                    pk += __shfl_xor(pk, m, kWave);
                }
                if (!a.l2norm) pq = pk = 0.f;
                if (r >= len) continue;
                const int64_t row = (int64_t)(tok0 + r) * H + h;
                const float rq = s.rq[r], rk = s.rk[r];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int64_t o = row * dk + c8 + 4 * u;
                    *reinterpret_cast<f32x4*>(a.dq + o) = rq * (gq[i][u] - xq[i][u] * pq);
                    *reinterpret_cast<f32x4*>(a.dk_out + o) = rk * (gk[i][u] - xk[i][u] * pk);
                }
            }
        }
    }
}

template <int DK>
hipError_t launch_chain(const BwdArgs& a, const ChainOps& rev, const ChainOps& fwd)
{
    const int64_t blocks = (2 * (int64_t)a.N * a.H + 7) / 8 * 8 * (a.dv / 16);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (a.bf16)
        hipLaunchKernelGGL((bwd_chain_kernel<DK, true>), dim3((uint32_t)blocks), dim3(256), 0, a.stream, a, rev, fwd);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<DK, false>), dim3((uint32_t)blocks), dim3(256), 0, a.stream, a, rev, fwd);
    return hipGetLastError();
}

hipError_t chain_dispatch(const BwdArgs& a, const ChainOps& rev, const ChainOps& fwd)
{
    switch (a.dk) {
        case 64: return launch_chain<64>(a, rev, fwd);
        case 128: return launch_chain<128>(a, rev, fwd);
        case 256: return launch_chain<256>(a, rev, fwd);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace


hipError_t launch_backward(const BwdArgs& a)
{
    const BwdLayout& L = a.lay;
    int32_t* header = reinterpret_cast<int32_t*>(a.ws + L.off_header);
    hipLaunchKernelGGL(bwd_table_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, a.N, a.T, L.max_chunks, header,
                       reinterpret_cast<int32_t*>(a.ws + L.off_tab), reinterpret_cast<int32_t*>(a.ws + L.off_seq_first));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t chblocks = L.max_chunks * a.H;
    if (chblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (a.bf16)
        hipLaunchKernelGGL((bwd_local_kernel<uint16_t>), dim3((uint32_t)chblocks), dim3(256), 0, a.stream, a);
    else
        hipLaunchKernelGGL((bwd_local_kernel<float>), dim3((uint32_t)chblocks), dim3(256), 0, a.stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // forward: Delta = U - W S^T,  S <- e^{gamma_L} S + Delta^T (D K); records S and Delta
    ChainOps fwd;
    fwd.off_X = L.off_U; fwd.off_Yr = L.off_Wr; fwd.off_Zf = L.off_Kf; fwd.off_Ef = 0; fwd.off_Ff = 0;
    fwd.off_Sst = L.off_S; fwd.off_Dst = L.off_Dl;
    fwd.S_init = a.init_state; fwd.S_final = nullptr;
    fwd.ysign = -1.f; fwd.zsign = 1.f; fwd.reverse = 0;
    // reverse: dDelta = dDelta_local + (D K) dS^T,  dS <- e^{gamma_L} dS - dDelta^T W + E^T Q
    ChainOps rev;
    rev.off_X = L.off_dDl; rev.off_Yr = L.off_Kr; rev.off_Zf = L.off_Wf; rev.off_Ef = L.off_Ef; rev.off_Ff = L.off_Qf;
    rev.off_Sst = L.off_dS; rev.off_Dst = L.off_dD;
    rev.S_init = a.dstate; rev.S_final = a.dinit;
    rev.ysign = 1.f; rev.zsign = -1.f; rev.reverse = 1;
    e = chain_dispatch(a, rev, fwd);
    if (e != hipSuccess) return e;
    if (a.bf16)
        hipLaunchKernelGGL((bwd_grad_kernel<uint16_t>), dim3((uint32_t)chblocks), dim3(256), 0, a.stream, a);
    else
        hipLaunchKernelGGL((bwd_grad_kernel<float>), dim3((uint32_t)chblocks), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace gdn
