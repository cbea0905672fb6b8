// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// Operation: "Long-Context Aware Upcycling: A New Frontier for Hybrid LLM
// Scaling" (arXiv:2604.24715), App. A.3, Eqs. 16-19, evaluated the way the
// appendix's last paragraph describes: the sequence is cut into chunks of C
// tokens, the delta corrections inside a chunk are batched into matrix
// products through the WY representation, and the state is carried from chunk
// to chunk.  With chunk-local cumulative log-decay gamma_r = sum_{m<=r} g_m,
// normalised rows q^, k^ and the state S (d_v x d_k) at the chunk start:
//
//   A_rj  = beta_r (k^_r . k^_j) e^{gamma_r - gamma_j}        j <  r
//   T     = (I + A)^{-1}                                     (unit lower-triangular)
//   W     = T diag(beta e^{gamma}) K^,    U = T diag(beta) V
//   Delta = U - W S^T                     (row r is beta_r v'_r of Eqs. 17-18)
//   P_rj  = (q^_r . k^_j) e^{gamma_r - gamma_j}               j <= r
//   O     = scale [ diag(e^{gamma}) Q^ S^T + P Delta ]        (Eq. 19, read after write)
//   S'    = e^{gamma_L} S + Delta^T diag(e^{gamma_L - gamma}) K^
//
// Exponents are only formed for j <= r, where they are <= 0 (g <= 0), so
// nothing overflows; e^{gamma} may underflow to 0, which is the exact limit.
//
// Kernels (all on the caller's stream):
//   chunk_table_kernel  varlen only: chunk table from cu_seqlens, on device.
//   intra_kernel        one workgroup per (chunk, head), fully parallel:
//                       norms, gamma, A and P on MFMA, T by forward
//                       substitution in LDS, W and U on MFMA.  Writes an
//                       operand record per chunk-head whose fragments are laid
//                       out exactly in the per-lane order of the MFMA operands
//                       of the chain kernel (one 16-byte load per operand).
//   chain_kernel        one workgroup per (sequence, head, 16*NT state rows):
//                       sequential over the sequence's chunks; state tile in
//                       fp32 MFMA accumulators, a rounded copy in LDS as the
//                       MFMA operand; computes Delta, the outputs, the state
//                       update; writes o and the final state.
//
// MFMA conventions (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32): lane
// l supplies row (l % 16) of A and column (l % 16) of B, with its "k-slots"
// chosen by lane group g = l / 16; the 16x16 result tile gives lane l the
// rows 4g..4g+3 of column l % 16.  Any bijection of the contraction index
// onto (g, element) works as long as A and B agree; two are used:
//   identity: k = g*E + e
//   sigma:    k = 16*(e/4) + 4g + e%4 (bf16), which is what a result tile of
//             the transposed product hands a lane, so results can be stored
//             as next-stage operands without a shuffle.
#include <stdlib.h>

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

// ------------------------------------------------------------------ MFMA policies

template <typename TIn> struct Mma;

template <> struct Mma<uint16_t> {  // bf16 operands, fp32 accumulation
    static constexpr int KS = 32;   // contraction extent per step
    static constexpr int E = 8;     // elements per lane per step
    typedef u16x8 Frag;             // 16 bytes
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t cvt(float x) { return f32_to_bf16_bits(x); }
    static __device__ __forceinline__ float wide(uint16_t x) { return bf16_bits_to_f32(x); }
    static __device__ __forceinline__ int sigma(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }
    // operand slots of lane group g in sigma order, from 32 consecutive elements at p
    static __device__ __forceinline__ Frag ld_sigma(const uint16_t* p, int g)
    {
        const u16x4 lo = *reinterpret_cast<const u16x4*>(p + 4 * g);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(p + 16 + 4 * g);
        Frag f;
        f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
        f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
        return f;
    }
};

template <> struct Mma<float> {  // fp32 operands (4 x 16x16x4 per step)
    static constexpr int KS = 16;
    static constexpr int E = 4;
    typedef f32x4 Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ float cvt(float x) { return x; }
    static __device__ __forceinline__ float wide(float x) { return x; }
    static __device__ __forceinline__ int sigma(int g, int e) { return 4 * g + e; }
    static __device__ __forceinline__ Frag ld_sigma(const float* p, int g)
    {
        return *reinterpret_cast<const f32x4*>(p + 4 * g);
    }
};

template <typename TIn>
__device__ __forceinline__ typename Mma<TIn>::Frag frag_from(const float* x)
{
    typename Mma<TIn>::Frag f;
    if constexpr (sizeof(TIn) == 2) {
        u32x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        f = __builtin_bit_cast(typename Mma<TIn>::Frag, h);
    } else {
#pragma unroll
        for (int e = 0; e < Mma<TIn>::E; ++e) f[e] = x[e];
    }
    return f;
}

template <typename TIn>
__device__ __forceinline__ typename Mma<TIn>::Frag zero_frag()
{
    typename Mma<TIn>::Frag f;
#pragma unroll
    for (int e = 0; e < Mma<TIn>::E; ++e) f[e] = 0;
    return f;
}

template <typename TIn>
__device__ __forceinline__ typename Mma<TIn>::Frag ld_frag(const TIn* p)
{
    return *reinterpret_cast<const typename Mma<TIn>::Frag*>(p);
}

template <typename TIn>
__device__ __forceinline__ void st_frag(TIn* p, typename Mma<TIn>::Frag f)
{
    *reinterpret_cast<typename Mma<TIn>::Frag*>(p) = f;
}

// four consecutive operand elements <-> 4 floats (8 bytes bf16, 16 bytes fp32)
template <typename TIn> struct Quad;
template <> struct Quad<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float* x)
    {
        u16x4 b = *reinterpret_cast<const u16x4*>(p);
        x[0] = bf16_bits_to_f32(b.x); x[1] = bf16_bits_to_f32(b.y);
        x[2] = bf16_bits_to_f32(b.z); x[3] = bf16_bits_to_f32(b.w);
    }
    static __device__ __forceinline__ void store(uint16_t* p, f32x4 v)
    {
        u16x4 b;
        b.x = f32_to_bf16_bits(v.x); b.y = f32_to_bf16_bits(v.y);
        b.z = f32_to_bf16_bits(v.z); b.w = f32_to_bf16_bits(v.w);
        *reinterpret_cast<u16x4*>(p) = b;
    }
};
template <> struct Quad<float> {
    static __device__ __forceinline__ void load(const float* p, float* x)
    {
        f32x4 v = *reinterpret_cast<const f32x4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};

// ------------------------------------------------------------------ record layout

// Per (chunk, head) operand record.  Operand fragments are in the element type
// of TIn; for bf16 a value x that must keep more than 8 significant bits is
// stored as hi = bf16(x), lo = bf16(x - hi), so hi + lo carries ~16 bits and a
// product takes two MFMAs.  K enters as the exact stored input (its per-row
// scale moves to the other operand in fp32); so does Q (read from the input,
// its row scale applied to the fp32 result).
template <typename TIn, int C, int DK, int DV>
struct Rec {
    static constexpr bool SPLIT = sizeof(TIn) == 2;
    static constexpr int KS = Mma<TIn>::KS;
    static constexpr int E = Mma<TIn>::E;
    static constexpr int RT = C / 16;      // chunk row tiles
    static constexpr int DKS = DK / KS;    // k-steps over d_k
    static constexpr int CKS = C / KS;     // k-steps over the chunk (KS <= C)
    static constexpr int MT = DK / 16;     // d_k tiles
    static constexpr int VT = DV / 16;     // d_v tiles
    static constexpr int WH_OFF = 0;                                  // [RT][DKS][64][E] W hi, sigma over d_k
    static constexpr int WL_OFF = WH_OFF + C * DK;                    // [RT][DKS][64][E] W lo (bf16 only)
    static constexpr int Q_OFF = WL_OFF + (SPLIT ? C * DK : 0);       // [RT][DKS][64][E] raw Q, sigma over d_k
    static constexpr int K_OFF = Q_OFF + C * DK;                      // [MT][CKS][64][E] raw K^T, identity over chunk
    static constexpr int PH_OFF = K_OFF + C * DK;                     // [RT][CKS][64][E] P hi
    static constexpr int PL_OFF = PH_OFF + C * C;                     // [RT][CKS][64][E] P lo (bf16 only)
    static constexpr int OPER_ELEMS = PL_OFF + (SPLIT ? C * C : 0);
    static constexpr size_t U_BYTE_OFF = ((size_t)OPER_ELEMS * sizeof(TIn) + 15) / 16 * 16;  // f32 [RT][VT][64][4]
    static constexpr size_t QS_BYTE_OFF = U_BYTE_OFF + (size_t)C * DV * 4;  // f32 [C]: rq_r e^{gamma_r}
    static constexpr size_t KSC_BYTE_OFF = QS_BYTE_OFF + (size_t)C * 4;     // f32 [C]: rk_j e^{gamma_L - gamma_j}
    static constexpr size_t DEC_BYTE_OFF = KSC_BYTE_OFF + (size_t)C * 4;    // f32 [4]: e^{gamma_L}, 0, 0, 0
    static constexpr size_t BYTES = DEC_BYTE_OFF + 16;
    static_assert(C % KS == 0 && DK % KS == 0, "tile shape");
};

// Position of the four consecutive columns 16*tile + 4*g .. +3 inside an LDS
// row stored in sigma order: within each 32-column block (bf16) the columns a
// lane group g needs for one k-step (4g..4g+3 and 16+4g..16+4g+3) sit next to
// each other, so an operand is one 16-byte read.  fp32: natural order.
template <typename TIn>
__device__ __forceinline__ int quad_pos(int tile, int g)
{
    if constexpr (sizeof(TIn) == 2) return (tile >> 1) * 32 + 8 * g + 4 * (tile & 1);
    return tile * 16 + 4 * g;
}

// hi/lo operand fragments from E fp32 values
template <typename TIn>
__device__ __forceinline__ void split_frag(const float* x, typename Mma<TIn>::Frag& hi, typename Mma<TIn>::Frag& lo)
{
    if constexpr (sizeof(TIn) == 2) {
        u32x4 h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t hh, ll;
            split_bf16x2(x[2 * i], x[2 * i + 1], hh, ll);
            h[i] = hh;
            l[i] = ll;
        }
        hi = __builtin_bit_cast(typename Mma<TIn>::Frag, h);
        lo = __builtin_bit_cast(typename Mma<TIn>::Frag, l);
    } else {
#pragma unroll
        for (int e = 0; e < Mma<TIn>::E; ++e) {
            hi[e] = x[e];
            lo[e] = 0.f;
        }
    }
}

// ------------------------------------------------------------------ chunk table

struct ChunkInfo {
    int32_t tok0, len, seq, pad;
};

// One workgroup.  Validates cu_seqlens (0 = c_0 <= ... <= c_N = T), writes the
// first chunk of every sequence and the (tok0, len, seq) of every chunk.  On
// invalid input it raises header[0] and publishes zero chunks, so later
// kernels touch nothing.
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu, int32_t N, int64_t T,
                                                          int32_t C, int64_t max_chunks, int32_t* __restrict__ header,
                                                          ChunkInfo* __restrict__ tab, int32_t* __restrict__ first)
{
    __shared__ int64_t part[256];
    __shared__ int bad;
    const int t = threadIdx.x;
    if (t == 0) bad = (cu[0] != 0 || (int64_t)cu[N] != T) ? 1 : 0;
    const int32_t per = (N + 255) / 256;
    const int32_t s0 = min(N, t * per), s1 = min(N, s0 + per);
    int64_t cnt = 0;
    int mybad = 0;
    for (int32_t i = s0; i < s1; ++i) {
        int32_t L = cu[i + 1] - cu[i];
        if (L < 0) { mybad = 1; L = 0; }
        cnt += (L + C - 1) / C;
    }
    part[t] = cnt;
    __syncthreads();
    if (mybad) bad = 1;
    if (t == 0) {
        int64_t run = 0;
        for (int i = 0; i < 256; ++i) { int64_t c = part[i]; part[i] = run; run += c; }
        if (run > max_chunks) bad = 1;
    }
    __syncthreads();
    const int ok = !bad;
    int64_t off = part[t];
    for (int32_t i = s0; i < s1; ++i) {
        first[i] = ok ? (int32_t)off : 0;
        int32_t L = max(cu[i + 1] - cu[i], 0);
        off += (L + C - 1) / C;
    }
    // thread 255 ends at the total number of chunks
    __shared__ int64_t tot_s;
    if (t == 255) tot_s = ok ? off : 0;
    __syncthreads();
    const int64_t tot = tot_s;
    if (t == 0) {
        first[N] = (int32_t)tot;
        header[0] = ok ? 0 : 1;
        header[1] = (int32_t)tot;
    }
    __syncthreads();
    for (int64_t j = t; j < tot; j += 256) {
        int32_t lo = 0, hi = N - 1;  // last n with first[n] <= j
        while (lo < hi) {
            int32_t mid = (lo + hi + 1) >> 1;
            if (first[mid] <= j) lo = mid; else hi = mid - 1;
        }
        ChunkInfo ci;
        ci.seq = lo;
        ci.tok0 = cu[lo] + (int32_t)(j - first[lo]) * C;
        ci.len = min(C, cu[lo + 1] - ci.tok0);
        ci.pad = 0;
        tab[j] = ci;
    }
}

__device__ __forceinline__ ChunkInfo chunk_info(const ChunkInfo* tab, bool varlen, int64_t c, int32_t C, int64_t T)
{
    if (varlen) return tab[c];
    ChunkInfo ci;
    ci.tok0 = (int32_t)(c * C);
    ci.len = (int32_t)min((int64_t)C, T - c * C);
    ci.seq = 0;
    ci.pad = 0;
    return ci;
}

// ------------------------------------------------------------------ intra-chunk kernel

template <typename TIn, int C, int DK, int DV>
struct IntraCfg {
    static constexpr int VP = DV < DK ? DV : DK;                 // value columns staged per pass
    static constexpr int NVP = DV / VP;                           // passes over d_v
    static constexpr int XR = DK > VP ? DK : VP;                  // rows of the transposed staging buffer
    static constexpr int XP = C + 2 * (16 / (int)sizeof(TIn));    // its pitch (elements), 16-byte rows
    static constexpr int AP = C + 4;                              // fp32 pitch of A and T
    static constexpr int VEC = 16 / (int)sizeof(TIn);             // elements per 16-byte load
};

template <typename TIn, int C, int DK, int DV>
struct IntraSmem {
    using Cf = IntraCfg<TIn, C, DK, DV>;
    TIn xt[Cf::XR * Cf::XP];  // K^T, later V^T (one pass of value columns): xt[col][j]
    float at[C * Cf::AP];     // A, strictly lower
    float tt[C * Cf::AP];     // T = (I + A)^{-1}, unit lower
    float gam[C], beta[C], rk[C], rq[C], sw[C], sb[C];
};

// Rows j < len of a [tokens][H][D] tensor, columns [col0, col0 + NCOL), written
// transposed into dst[col - col0][j]; rows >= len are zero.  Lane = row j, so
// each LDS store instruction of a wave writes 64 consecutive elements (no bank
// conflicts); wave w takes 16-byte column groups w, w + 4, ...  Values are held
// in registers between the (early) global loads and the LDS stores.
template <typename TIn, int C, int NCOL, int XP>
struct TransposeStage {
    static constexpr int VEC = 16 / (int)sizeof(TIn);
    static constexpr int GROUPS = NCOL / VEC;
    static constexpr int ITEMS = (GROUPS + 3) / 4;
    uint4 buf[ITEMS];
    __device__ __forceinline__ void load(const TIn* base, int64_t row_stride, int col0, int len, int lane, int wave)
    {
#pragma unroll
        for (int s = 0; s < ITEMS; ++s) {
            const int cg = wave + 4 * s;
            if (cg < GROUPS && lane < len)
                buf[s] = *reinterpret_cast<const uint4*>(base + (int64_t)lane * row_stride + col0 + cg * VEC);
            else
                buf[s] = uint4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(TIn* dst, int lane, int wave) const
    {
        if (lane >= C) return;
#pragma unroll
        for (int s = 0; s < ITEMS; ++s) {
            const int cg = wave + 4 * s;
            if (cg >= GROUPS) break;
            const TIn* e = reinterpret_cast<const TIn*>(&buf[s]);
#pragma unroll
            for (int u = 0; u < VEC; ++u) dst[(cg * VEC + u) * XP + lane] = e[u];
        }
    }
};

template <typename TIn, int C, int DK, int DV>
__global__ __launch_bounds__(256) void intra_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                    const TIn* __restrict__ v, const float* __restrict__ g,
                                                    const float* __restrict__ beta, const int32_t* __restrict__ header,
                                                    const ChunkInfo* __restrict__ tab, int32_t varlen, int64_t T,
                                                    int32_t H, int32_t l2norm, float* __restrict__ decay_out,
                                                    unsigned char* __restrict__ records, size_t record_bytes)
{
    using M = Mma<TIn>;
    using F = Mma<float>;
    using R = Rec<TIn, C, DK, DV>;
    using Cf = IntraCfg<TIn, C, DK, DV>;
    using Sm = IntraSmem<TIn, C, DK, DV>;
    typedef typename M::Frag Frag;
    constexpr int KS = M::KS, E = M::E;
    constexpr int XP = Cf::XP, AP = Cf::AP;
    constexpr int RT = R::RT;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int64_t c = blockIdx.x;
    const int h = blockIdx.y;
    if (varlen && c >= header[1]) return;
    if (!varlen && c * C >= T) return;
    const ChunkInfo ci = chunk_info(tab, varlen, c, C, T);
    const int len = ci.len;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar branches
    const int g16 = lane >> 4, l16 = lane & 15;

    unsigned char* recb = records + ((size_t)c * H + h) * record_bytes;
    TIn* rec = reinterpret_cast<TIn*>(recb);
    float* recU = reinterpret_cast<float*>(recb + R::U_BYTE_OFF);

    const int64_t row0 = (int64_t)ci.tok0 * H + h;  // row index of token tok0 in [tokens*H]
    auto qk_row = [&](const TIn* base, int r) -> const TIn* { return base + (row0 + (int64_t)r * H) * DK; };

    // ---- global loads first: K (to be transposed), the first pass of V (held in registers)
    TransposeStage<TIn, C, DK, XP> kst;
    kst.load(k + row0 * DK, (int64_t)H * DK, 0, len, lane, wave);
    TransposeStage<TIn, C, Cf::VP, XP> vst;
    vst.load(v + row0 * DV, (int64_t)H * DV, 0, len, lane, wave);

    // ---- gates: gamma (inclusive scan within the chunk), beta; rows >= len: g = 0, beta = 0
    if (wave == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < len) {
            gv = g[row0 + (int64_t)lane * H];
            bv = beta[row0 + (int64_t)lane * H];
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            float y = __shfl_up(gv, off, 64);
            if (lane >= off) gv += y;
        }
        if (lane < C) {
            sm.gam[lane] = gv;
            sm.beta[lane] = bv;
        }
    }
    // ---- inverse norms (4 threads per row)
    {
        const int r = tid >> 2, part = tid & 3;
        float sk = 0.f, sq = 0.f;
        if (r < C && r < len) {
            const TIn* kr = qk_row(k, r);
            const TIn* qr = qk_row(q, r);
#pragma unroll 4
            for (int cc = part * 4; cc < DK; cc += 16) {
                float xk[4], xq[4];
                Quad<TIn>::load(kr + cc, xk);
                Quad<TIn>::load(qr + cc, xq);
#pragma unroll
                for (int e = 0; e < 4; ++e) { sk += xk[e] * xk[e]; sq += xq[e] * xq[e]; }
            }
        }
        sk += __shfl_xor(sk, 1, 64); sk += __shfl_xor(sk, 2, 64);
        sq += __shfl_xor(sq, 1, 64); sq += __shfl_xor(sq, 2, 64);
        if (r < C && part == 0) {
            const bool live = r < len;
            sm.rk[r] = live ? (l2norm ? 1.0f / sqrtf(sk + kNormEps) : 1.0f) : 0.f;
            sm.rq[r] = live ? (l2norm ? 1.0f / sqrtf(sq + kNormEps) : 1.0f) : 0.f;
        }
    }
    kst.store(sm.xt, lane, wave);
    __syncthreads();

    const float gL = sm.gam[C - 1];  // rows >= len carry g = 0, so this is gamma at len-1
    if (tid < C) {
        const int j = tid;
        sm.sw[j] = sm.beta[j] * expf(sm.gam[j]) * sm.rk[j];  // W = T diag(sw) K
        sm.sb[j] = sm.beta[j];                                 // U = T diag(sb) V
        float* qs = reinterpret_cast<float*>(recb + R::QS_BYTE_OFF);
        float* ksc = reinterpret_cast<float*>(recb + R::KSC_BYTE_OFF);
        qs[j] = sm.rq[j] * expf(sm.gam[j]);
        ksc[j] = sm.rk[j] * expf(gL - sm.gam[j]);
    }

    // ---- G = K K^T lower tiles -> A (strict, LDS);  R^T = K Q^T -> P fragments (sigma over j)
    {
        constexpr int NG = RT * (RT + 1) / 2;
        constexpr int UPF = KS / 16;  // j tiles per P fragment
        // P fragment jobs: (rt, ks) with ks*KS <= rt*16 + 15
        constexpr int NP = [] {
            int n = 0;
            for (int rt = 0; rt < RT; ++rt) n += (rt * 16 + 16 + KS - 1) / KS;
            return n;
        }();
        for (int job = wave; job < NG + NP; job += 4) {
            if (job < NG) {
                int tt_ = job, ti = 0;
                while (tt_ > ti) { tt_ -= ti + 1; ++ti; }
                const int tj = tt_;
                const int ra = ti * 16 + l16, rb = tj * 16 + l16;
                const TIn* pa = qk_row(k, ra);
                const TIn* pb = qk_row(k, rb);
                Frag fa[R::DKS], fb[R::DKS];
#pragma unroll
                for (int ks = 0; ks < R::DKS; ++ks) {
                    fa[ks] = ra < len ? ld_frag<TIn>(pa + ks * KS + g16 * E) : zero_frag<TIn>();
                    fb[ks] = rb < len ? ld_frag<TIn>(pb + ks * KS + g16 * E) : zero_frag<TIn>();
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < R::DKS; ++ks) acc = M::mma(fa[ks], fb[ks], acc);
                const int j = tj * 16 + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ti * 16 + 4 * g16 + i;
                    float val = 0.f;
                    if (j < r) val = sm.beta[r] * sm.rk[r] * sm.rk[j] * acc[i] * expf(sm.gam[r] - sm.gam[j]);
                    sm.at[r * AP + j] = val;
                }
            } else {
                int f = job - NG, rt = 0;
                while (f >= (rt * 16 + 16 + KS - 1) / KS) { f -= (rt * 16 + 16 + KS - 1) / KS; ++rt; }
                const int ks = f;
                const int r = rt * 16 + l16;  // fixed per lane: B operand column
                const TIn* pq = qk_row(q, r);
                Frag fq[R::DKS];
#pragma unroll
                for (int dk = 0; dk < R::DKS; ++dk)
                    fq[dk] = r < len ? ld_frag<TIn>(pq + dk * KS + g16 * E) : zero_frag<TIn>();
                float x[E];
#pragma unroll
                for (int u = 0; u < UPF; ++u) {
                    const int tj = ks * UPF + u;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (tj <= rt) {
                        const int rk_row = tj * 16 + l16;
                        const TIn* pk = qk_row(k, rk_row);
#pragma unroll
                        for (int dk = 0; dk < R::DKS; ++dk) {
                            const Frag fk = rk_row < len ? ld_frag<TIn>(pk + dk * KS + g16 * E) : zero_frag<TIn>();
                            acc = M::mma(fk, fq[dk], acc);
                        }
                    }
                    // lane holds R[r][j] for j = tj*16 + 4*g16 + i
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = tj * 16 + 4 * g16 + i;
                        x[u * 4 + i] = (tj <= rt && j <= r)
                                           ? sm.rq[r] * sm.rk[j] * acc[i] * expf(sm.gam[r] - sm.gam[j])
                                           : 0.f;
                    }
                }
                Frag hi, lo;
                split_frag<TIn>(x, hi, lo);
                const size_t fo = ((size_t)(rt * R::CKS + ks) * 64 + lane) * E;
                st_frag<TIn>(rec + R::PH_OFF + fo, hi);
                if constexpr (R::SPLIT) st_frag<TIn>(rec + R::PL_OFF + fo, lo);
            }
        }
        // raw Q fragments in sigma order over d_k (rows >= len are zero)
        for (int f = wave; f < RT * R::DKS; f += 4) {
            const int rt = f / R::DKS, ks = f % R::DKS;
            const int r = rt * 16 + l16;
            Frag fq;
            if (r < len) {
                fq = M::ld_sigma(qk_row(q, r) + ks * KS, g16);
            } else {
                fq = zero_frag<TIn>();
            }
            st_frag<TIn>(rec + R::Q_OFF + ((size_t)f * 64 + lane) * E, fq);
        }
        // raw K^T fragments for the state update (identity over the chunk)
        for (int f = wave; f < R::MT * R::CKS; f += 4) {
            const int mt = f / R::CKS, ks = f % R::CKS;
            const Frag fk = *reinterpret_cast<const Frag*>(sm.xt + (mt * 16 + l16) * XP + ks * KS + g16 * E);
            st_frag<TIn>(rec + R::K_OFF + ((size_t)f * 64 + lane) * E, fk);
        }
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}, blocked by 16: diagonal blocks by substitution, then
    //      T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj on fp32 MFMA, by block distance
    if (wave < RT) {
        const int b0 = wave * 16, col = l16;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
            const float* arow = sm.at + (b0 + r) * AP + b0;
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= arow[j] * t[j];
            t[r] = acc;
        }
        if (lane < 16) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.tt[(b0 + r) * AP + b0 + col] = t[r];
        }
    }
    for (int idx = tid; idx < C * C; idx += 256) {  // strictly upper blocks of T are zero
        const int r = idx / C, j = idx % C;
        if ((j >> 4) > (r >> 4)) sm.tt[r * AP + j] = 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < RT; ++d) {
        for (int jb = wave; jb + d < RT; jb += 4) {
            const int ib = jb + d;
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
            for (int mb = jb; mb < ib; ++mb) {
                const f32x4 fa = *reinterpret_cast<const f32x4*>(sm.at + (ib * 16 + l16) * AP + mb * 16 + 4 * g16);
                f32x4 fb;
#pragma unroll
                for (int e = 0; e < 4; ++e) fb[e] = sm.tt[(mb * 16 + 4 * g16 + e) * AP + jb * 16 + l16];
                X = F::mma(fa, fb, X);
            }
            const f32x4 fd = *reinterpret_cast<const f32x4*>(sm.tt + (ib * 16 + l16) * AP + ib * 16 + 4 * g16);
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
            Y = F::mma(fd, X, Y);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.tt[(ib * 16 + 4 * g16 + e) * AP + jb * 16 + l16] = -Y[e];
        }
        __syncthreads();
    }

    // ---- W^T = K^T (T diag(sw))^T, T diag(sw) split hi/lo, K exact: the result tiles
    //      are the sigma-ordered W fragments of the chain kernel, stored hi/lo
    {
        constexpr int MT_PER = KS / 16;
        for (int f = wave; f < RT * R::DKS; f += 4) {
            const int rt = f / R::DKS, ks = f % R::DKS;
            const int r = rt * 16 + l16;
            const int nks = (rt * 16 + 16 + KS - 1) / KS;  // T[r][j] = 0 for j > r
            f32x4 acc[MT_PER];
#pragma unroll
            for (int u = 0; u < MT_PER; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int jk = 0; jk < nks; ++jk) {
                const int j0 = jk * KS + g16 * E;
                float x[E];
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = sm.tt[r * AP + j0 + e] * sm.sw[j0 + e];
                Frag bh, bl;
                split_frag<TIn>(x, bh, bl);
#pragma unroll
                for (int u = 0; u < MT_PER; ++u) {
                    const Frag fa = *reinterpret_cast<const Frag*>(sm.xt + ((ks * MT_PER + u) * 16 + l16) * XP + j0);
                    acc[u] = M::mma(fa, bh, acc[u]);
                    if constexpr (R::SPLIT) acc[u] = M::mma(fa, bl, acc[u]);
                }
            }
            float x[E];
#pragma unroll
            for (int u = 0; u < MT_PER; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[u * 4 + i] = acc[u][i];
            Frag hi, lo;
            split_frag<TIn>(x, hi, lo);
            st_frag<TIn>(rec + R::WH_OFF + ((size_t)f * 64 + lane) * E, hi);
            if constexpr (R::SPLIT) st_frag<TIn>(rec + R::WL_OFF + ((size_t)f * 64 + lane) * E, lo);
        }
    }

    // ---- U = (T diag(sb)) V, T diag(sb) split hi/lo, V exact, in passes of VP value columns
#pragma unroll 1
    for (int pass = 0; pass < Cf::NVP; ++pass) {
        if (pass > 0) vst.load(v + row0 * DV, (int64_t)H * DV, pass * Cf::VP, len, lane, wave);
        __syncthreads();  // xt free (K^T readers done, or the previous pass done)
        vst.store(sm.xt, lane, wave);
        __syncthreads();
        constexpr int CT = Cf::VP / 16;
        for (int f = wave; f < RT * CT; f += 4) {
            const int rt = f / CT, ctl = f % CT;
            const int r = rt * 16 + l16;
            const int nks = (rt * 16 + 16 + KS - 1) / KS;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int jk = 0; jk < nks; ++jk) {
                const int j0 = jk * KS + g16 * E;
                float xa[E];
#pragma unroll
                for (int e = 0; e < E; ++e) xa[e] = sm.tt[r * AP + j0 + e] * sm.sb[j0 + e];
                Frag ah, al;
                split_frag<TIn>(xa, ah, al);
                const Frag fb = *reinterpret_cast<const Frag*>(sm.xt + (ctl * 16 + l16) * XP + j0);
                acc = M::mma(ah, fb, acc);
                if constexpr (R::SPLIT) acc = M::mma(al, fb, acc);
            }
            const int ct = pass * CT + ctl;
            *reinterpret_cast<f32x4*>(recU + ((size_t)(rt * R::VT + ct) * 64 + lane) * 4) = acc;
        }
    }
    if (tid == 0) {
        decay_out[c * H + h] = expf(gL);
        *reinterpret_cast<f32x4*>(recb + R::DEC_BYTE_OFF) = f32x4{expf(gL), 0.f, 0.f, 0.f};
    }
}

// ------------------------------------------------------------------ chain kernel

// LDS of the chain kernel: the rounded state copy, Delta^T (two layouts), and a
// ring of W and Q operand fragments filled by LDS-DMA (buffer_load ... lds),
// one region per wave and ring stage.  Two stages when they fit (bf16), so the
// fragments of chunk c+1 stream in while chunk c computes.
template <typename TIn, int C, int DK, int NT, bool SPLIT>
struct ChainLds {
    static constexpr int SP = DK + 16 / (int)sizeof(TIn);  // state copy pitch (dwords = 4 mod 32)
    static constexpr int DP = C + 16 / (int)sizeof(TIn);   // Delta^T pitch
    static constexpr int NS = SPLIT ? 2 : 1;
    static constexpr int DKS = DK / Mma<TIn>::KS;
    static constexpr int RING_FRAGS = 2 * DKS;              // W then Q fragments of one chunk row tile
    static constexpr size_t SR_BYTES = (size_t)NS * 16 * NT * SP * sizeof(TIn);
    static constexpr size_t D_BYTES = (size_t)NS * 16 * NT * DP * sizeof(TIn);
    static constexpr size_t FIXED = (SR_BYTES + 2 * D_BYTES + 255) / 256 * 256;
    static constexpr size_t SINK_BYTES = 4 * 1024;           // per-wave 1 KB landing slot of L2 prefetches
    static constexpr size_t STAGE_BYTES = (size_t)4 * RING_FRAGS * 1024;
    static constexpr int STAGES = FIXED + SINK_BYTES + 2 * STAGE_BYTES <= 160 * 1024 ? 2 : 1;
    static constexpr size_t RING_OFF = FIXED + SINK_BYTES;
    static constexpr size_t BYTES = RING_OFF + STAGES * STAGE_BYTES;
    static_assert(BYTES <= 160 * 1024, "chain kernel LDS");
};

// Register operands of one chunk step for one wave, loaded one step ahead.
template <typename TIn, int C, int DK, int DV, int NT, bool SW>
struct ChainOps {
    using R = Rec<TIn, C, DK, DV>;
    typedef typename Mma<TIn>::Frag Frag;
    static constexpr int MT_W = (R::MT + 3) / 4;
    Frag wl[SW ? R::DKS : 1];
    Frag ph[R::CKS];
    Frag pl[R::SPLIT ? R::CKS : 1];
    Frag k[MT_W][R::CKS];
    f32x4 u[NT];
    f32x4 qs, ks;
    float dec;
    int32_t tok0, len;
};

template <typename TIn> struct OStore;
template <> struct OStore<uint16_t> {
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, float x)
    {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(x), r, (int)voff, 0, 0);
    }
};
template <> struct OStore<float> {
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, float x)
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, 0, 0);  // payload is raw bits
    }
};

// Store four fp32 values as operand elements at p (hi) and p2 (lo, bf16 only).
template <typename TIn, bool LO>
__device__ __forceinline__ void store_quad(TIn* p, TIn* p2, f32x4 v)
{
    if constexpr (sizeof(TIn) == 2) {
        uint32_t h0, l0, h1, l1;
        split_bf16x2(v.x, v.y, h0, l0);
        split_bf16x2(v.z, v.w, h1, l1);
        *reinterpret_cast<u32x2*>(p) = u32x2{h0, h1};
        if constexpr (LO) *reinterpret_cast<u32x2*>(p2) = u32x2{l0, l1};
    } else {
        *reinterpret_cast<f32x4*>(p) = v;
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (lgkmcnt) but not for its outstanding global loads or LDS-DMA transfers, which
// the chain kernel tracks itself with counted vmcnt waits.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// SPLIT_S: the state enters W S^T and Q S^T as hi + lo (else hi only).
// SPLIT_W: W enters as hi + lo (else hi only).
// Workgroups are mapped so that all row tiles of one (sequence, head) pair run
// on one XCD (workgroups are dealt to the 8 XCDs round-robin): they read the
// same per-chunk records, which then come from that XCD's L2.
template <typename TIn, int C, int DK, int DV, int NT, bool SPLIT_S, bool SPLIT_W>
__global__ __launch_bounds__(256) void chain_kernel(const int32_t* __restrict__ header,
                                                    const ChunkInfo* __restrict__ tab,
                                                    const int32_t* __restrict__ seq_first, int32_t varlen, int64_t T,
                                                    int32_t H, int32_t pairs, const float* __restrict__ decay,
                                                    const unsigned char* __restrict__ records, size_t record_bytes,
                                                    const float* __restrict__ init_state, float* __restrict__ final_state,
                                                    TIn* __restrict__ o, float scale)
{
    using M = Mma<TIn>;
    using R = Rec<TIn, C, DK, DV>;
    constexpr bool SPL = R::SPLIT;
    constexpr bool SS = SPL && SPLIT_S;
    constexpr bool SW = SPL && SPLIT_W;
    using L = ChainLds<TIn, C, DK, NT, SPL>;
    using Ops = ChainOps<TIn, C, DK, DV, NT, SW>;
    typedef typename M::Frag Frag;
    constexpr int KS = M::KS, E = M::E;
    constexpr int SP = L::SP, DP = L::DP, NS = L::NS;
    constexpr int MT_W = Ops::MT_W;
    constexpr int TILES = DV / (16 * NT);
    constexpr uint32_t FB = 64 * 16;  // bytes of one operand fragment (64 lanes x 16 B)
    constexpr uint32_t EB = sizeof(TIn);

    extern __shared__ __align__(256) unsigned char lds[];
    TIn* sr = reinterpret_cast<TIn*>(lds);                                   // [NS][16 NT][SP]
    TIn* dt = reinterpret_cast<TIn*>(lds + L::SR_BYTES);                     // [NS][16 NT][DP]
    TIn* ds = reinterpret_cast<TIn*>(lds + L::SR_BYTES + L::D_BYTES);        // [NS][16 NT][DP]
    unsigned char* sink = lds + L::FIXED;                                    // [4][1 KB]
    unsigned char* ring = lds + L::RING_OFF;                                 // [STAGES][4][RING_FRAGS][1 KB]
    constexpr int SR_LO = (NS - 1) * 16 * NT * SP;
    constexpr int D_LO = (NS - 1) * 16 * NT * DP;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar branches
    const int g16 = lane >> 4, l16 = lane & 15;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int pair = xcd + 8 * (slot / TILES);
    if (pair >= pairs) return;
    const int n = pair / H, h = pair % H;
    const int row0 = (slot % TILES) * 16 * NT;  // first state row (value index) of this workgroup

    int64_t c_begin, c_end;
    if (varlen) {
        if (header[0] != 0) return;
        c_begin = seq_first[n];
        c_end = seq_first[n + 1];
    } else {
        c_begin = 0;
        c_end = (T + C - 1) / C;
    }

    // state tiles S^T[mt][nt] in result layout: lane holds S[row0 + nt*16 + l16][mt*16 + 4*g16 + i]
    f32x4 S[MT_W][NT];
    const size_t st_base = ((size_t)n * H + h) * DV * DK;
#pragma unroll
    for (int a = 0; a < MT_W; ++a) {
        const int mt = wave + 4 * a;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            S[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (mt < R::MT && init_state)
                S[a][nt] = *reinterpret_cast<const f32x4*>(init_state + st_base +
                                                           (size_t)(row0 + nt * 16 + l16) * DK + mt * 16 + 4 * g16);
            if (mt < R::MT) {
                const int off = (nt * 16 + l16) * SP + quad_pos<TIn>(mt, g16);
                store_quad<TIn, SPL>(sr + off, sr + SR_LO + off, S[a][nt]);
            }
        }
    }
    __syncthreads();

    const bool has_rt = wave < R::RT;
    const int rt = wave;
    const int pks = (rt * 16 + 16 + KS - 1) / KS;  // P k-steps up to the diagonal

    // per-lane byte offsets inside a record (fragments are 64 lanes x 16 B)
    const uint32_t lane_b = (uint32_t)lane * 16;
    const uint32_t offWH = R::WH_OFF * EB + (uint32_t)rt * R::DKS * FB + lane_b;
    const uint32_t offWL = R::WL_OFF * EB + (uint32_t)rt * R::DKS * FB + lane_b;
    const uint32_t offQ = R::Q_OFF * EB + (uint32_t)rt * R::DKS * FB + lane_b;
    const uint32_t offPH = R::PH_OFF * EB + (uint32_t)rt * R::CKS * FB + lane_b;
    const uint32_t offPL = R::PL_OFF * EB + (uint32_t)rt * R::CKS * FB + lane_b;
    const uint32_t offK = R::K_OFF * EB + lane_b;
    const uint32_t offU = (uint32_t)R::U_BYTE_OFF + ((uint32_t)(rt * R::VT + (row0 >> 4)) * 64 + lane) * 16;
    const uint32_t offQS = (uint32_t)R::QS_BYTE_OFF + (uint32_t)(rt * 16 + 4 * g16) * 4;
    const uint32_t offKS = (uint32_t)R::KSC_BYTE_OFF + (uint32_t)(rt * 16 + 4 * g16) * 4;
    const uint32_t rowstride_o = (uint32_t)H * DV * EB;

    auto rec_rsrc = [&](int64_t c) {
        return make_rsrc(records + ((size_t)c * H + h) * record_bytes, (uint32_t)R::BYTES);
    };
    auto ring_frag = [&](int64_t c, int f) -> unsigned char* {
        return ring + ((size_t)((c % L::STAGES) * 4 + wave) * L::RING_FRAGS + f) * 1024;
    };
    // W and Q fragment ks of chunk c -> this wave's ring region (LDS-DMA, no registers)
    auto dma_ks = [&](const __amdgpu_buffer_rsrc_t& rr, int64_t c, int ks) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)ring_frag(c, ks), 16, offWH, ks * FB, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)ring_frag(c, R::DKS + ks), 16, offQ, ks * FB, 0, 0);
    };
    // register operands of chunk c, in NLD independent groups (issued spread over a step)
    constexpr int NLD = 4;
    auto load_part = [&](Ops& op, const __amdgpu_buffer_rsrc_t& rr, int64_t c, int part) {
        if (part == 0) {
            const ChunkInfo ci = chunk_info(tab, varlen, c, C, T);
            op.tok0 = ci.tok0;
            op.len = ci.len;
            op.dec = __builtin_bit_cast(f32x4, buf_load16(rr, (uint32_t)R::DEC_BYTE_OFF, 0)).x;
            if (has_rt) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) op.u[nt] = __builtin_bit_cast(f32x4, buf_load16(rr, offU, nt * FB));
                op.qs = __builtin_bit_cast(f32x4, buf_load16(rr, offQS, 0));
                op.ks = __builtin_bit_cast(f32x4, buf_load16(rr, offKS, 0));
            }
        } else if (part == 1) {
            if (has_rt) {
#pragma unroll
                for (int ks = 0; ks < R::CKS; ++ks) {
                    op.ph[ks] = __builtin_bit_cast(Frag, buf_load16(rr, offPH, ks * FB));
                    if constexpr (SPL) op.pl[ks] = __builtin_bit_cast(Frag, buf_load16(rr, offPL, ks * FB));
                }
                if constexpr (SW) {
#pragma unroll
                    for (int ks = 0; ks < R::DKS; ++ks)
                        op.wl[ks] = __builtin_bit_cast(Frag, buf_load16(rr, offWL, ks * FB));
                }
            }
        } else {
            // K fragments, half of this wave's d_k tiles per part
#pragma unroll
            for (int a = 0; a < MT_W; ++a) {
                if ((a & 1) != (part & 1)) continue;
                const int mt = wave + 4 * a;
                if (mt < R::MT) {
#pragma unroll
                    for (int ks = 0; ks < R::CKS; ++ks)
                        op.k[a][ks] = __builtin_bit_cast(Frag, buf_load16(rr, offK, (mt * R::CKS + ks) * FB));
                }
            }
        }
    };
    // Cooperative L2 prefetch of the shared part of chunk c's record (W, Q, K, P):
    // the TILES workgroups of this (sequence, head) each pull 1/TILES of it into
    // their XCD's L2 (landing in a scratch LDS slot), so the loads one step later hit L2.
    constexpr uint32_t SHARED_BYTES = (uint32_t)R::U_BYTE_OFF;
    constexpr uint32_t PF_INSTR = (SHARED_BYTES / 1024 + TILES * 4 - 1) / (TILES * 4);  // per wave
    const int tile = slot % TILES;
    auto prefetch = [&](int64_t c) {
        const __amdgpu_buffer_rsrc_t rr = rec_rsrc(c);
#pragma unroll
        for (uint32_t i = 0; i < PF_INSTR; ++i) {
            uint32_t blk = (i * TILES + tile) * 4 + wave;  // 1 KB block of the record
            blk = blk < SHARED_BYTES / 1024 ? blk : SHARED_BYTES / 1024 - 1;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)(sink + wave * 1024), 16, lane_b, blk * 1024, 0, 0);
        }
    };
    // VMEM operations a wave with a chunk row tile issues after its last W/Q
    // DMA of a step: the next chunk's U, row scales, P (and W lo), this chunk's
    // outputs, the next chunk's K fragments and one prefetch.  Waiting until at
    // most that many are outstanding means the DMA has landed (the counter
    // retires in issue order).
    constexpr int N_AFTER = (NT + 3 + R::CKS * (SPL ? 2 : 1) + (SW ? R::DKS : 0)) + 4 * NT +
                            MT_W * R::CKS + (int)PF_INSTR;
    static_assert(L::STAGES == 1 || N_AFTER < 64, "vmcnt range");
    constexpr int WAIT_AFTER = (N_AFTER & 15) | ((N_AFTER >> 4) << 14) | (7 << 4) | (15 << 8);

    auto step = [&](const Ops& op, Ops& nxt, int64_t c) {
        const bool more = c + 1 < c_end;
        const __amdgpu_buffer_rsrc_t rn = rec_rsrc(more ? c + 1 : c);
        f32x4 Y[NT];
        if (has_rt) {
            // X = W S^T, Y = Q S^T over all of d_k (two accumulators each); Delta = U - X.
            // The next chunk's W/Q fragments stream into the other ring stage meanwhile.
            f32x4 X[NT], X2[NT], Y2[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) X[nt] = X2[nt] = Y[nt] = Y2[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const unsigned char* rw = ring_frag(c, 0) + lane_b;
            // operands of k-step ks are read from LDS one k-step ahead of their MFMAs
            Frag fwn = *reinterpret_cast<const Frag*>(rw);
            Frag fqn = *reinterpret_cast<const Frag*>(rw + R::DKS * 1024);
            Frag bhn[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bhn[nt] = *reinterpret_cast<const Frag*>(sr + (nt * 16 + l16) * SP + g16 * E);
#pragma unroll
            for (int ks = 0; ks < R::DKS; ++ks) {
                if constexpr (L::STAGES == 2) {
                    if (more) dma_ks(rn, c + 1, ks);
                }
                const Frag fw = fwn, fq = fqn;
                Frag bhc[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bhc[nt] = bhn[nt];
                if (ks + 1 < R::DKS) {
                    fwn = *reinterpret_cast<const Frag*>(rw + (ks + 1) * 1024);
                    fqn = *reinterpret_cast<const Frag*>(rw + (R::DKS + ks + 1) * 1024);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        bhn[nt] = *reinterpret_cast<const Frag*>(sr + (nt * 16 + l16) * SP + (ks + 1) * KS + g16 * E);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int so = (nt * 16 + l16) * SP + ks * KS + g16 * E;
                    const Frag bh = bhc[nt];
                    f32x4& xa = (ks & 1) ? X2[nt] : X[nt];
                    f32x4& ya = (ks & 1) ? Y2[nt] : Y[nt];
                    xa = M::mma(fw, bh, xa);
                    ya = M::mma(fq, bh, ya);
                    if constexpr (SW) xa = M::mma(op.wl[ks], bh, xa);
                    if constexpr (SS) {
                        const Frag bl = *reinterpret_cast<const Frag*>(sr + SR_LO + so);
                        xa = M::mma(fw, bl, xa);
                        ya = M::mma(fq, bl, ya);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // later VMEM stays after the DMA (exact vmcnt wait)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                Y[nt] = (Y[nt] + Y2[nt]) * op.qs;
                const f32x4 d = op.u[nt] - (X[nt] + X2[nt]);
                // Delta^T[r][j] for j = rt*16 + 4*g16 + i: sigma-ordered rows (dt), natural rows (ds)
                const int row = (nt * 16 + l16) * DP;
                const int pd = row + quad_pos<TIn>(rt, g16);
                const int pn = row + rt * 16 + 4 * g16;
                store_quad<TIn, SPL>(dt + pd, dt + D_LO + pd, d);
                store_quad<TIn, SPL>(ds + pn, ds + D_LO + pn, d * op.ks);
            }
        }
        lds_barrier();

        if (has_rt) {
            // O = scale (Y + P Delta); P fragments are sigma-ordered over j
#pragma unroll
            for (int ks = 0; ks < R::CKS; ++ks) {
                if (ks < pks) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int doff = (nt * 16 + l16) * DP + ks * KS + g16 * E;
                        const Frag dh = *reinterpret_cast<const Frag*>(dt + doff);
                        Y[nt] = M::mma(op.ph[ks], dh, Y[nt]);
                        if constexpr (SPL) {
                            const Frag dl = *reinterpret_cast<const Frag*>(dt + D_LO + doff);
                            Y[nt] = M::mma(op.pl[ks], dh, Y[nt]);
                            Y[nt] = M::mma(op.ph[ks], dl, Y[nt]);
                        }
                    }
                }
            }
            // rows >= len lie past the end of this view: the stores are dropped
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + ((int64_t)op.tok0 * H + h) * DV,
                                                        (uint32_t)(((op.len - 1) * H + 1) * DV * EB));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    OStore<TIn>::st(ro, (uint32_t)(rt * 16 + 4 * g16 + i) * rowstride_o +
                                            (uint32_t)(row0 + nt * 16 + l16) * EB, scale * Y[nt][i]);
        }
        if (more) {
            load_part(nxt, rn, c + 1, 0);
            load_part(nxt, rn, c + 1, 1);
        }
        // state update on this wave's d_k tiles: S^T = e^{gamma_L} S^T + K^T (kscale o Delta)
        Frag dsh[R::CKS][NT], dsl[SPL ? R::CKS : 1][NT];
#pragma unroll
        for (int ks = 0; ks < R::CKS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int doff = (nt * 16 + l16) * DP + ks * KS + g16 * E;
                dsh[ks][nt] = *reinterpret_cast<const Frag*>(ds + doff);
                if constexpr (SPL) dsl[ks][nt] = *reinterpret_cast<const Frag*>(ds + D_LO + doff);
            }
#pragma unroll
        for (int a = 0; a < MT_W; ++a) {
            const int mt = wave + 4 * a;
            if (mt >= R::MT) continue;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[a][nt] *= op.dec;
#pragma unroll
            for (int ks = 0; ks < R::CKS; ++ks) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    S[a][nt] = M::mma(op.k[a][ks], dsh[ks][nt], S[a][nt]);
                    if constexpr (SPL) S[a][nt] = M::mma(op.k[a][ks], dsl[ks][nt], S[a][nt]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int off = (nt * 16 + l16) * SP + quad_pos<TIn>(mt, g16);
                store_quad<TIn, SS>(sr + off, sr + SR_LO + off, S[a][nt]);
            }
            if (a == 0 && more) load_part(nxt, rn, c + 1, 2);  // K fragments for the next chunk,
            if (a == 1 && more) load_part(nxt, rn, c + 1, 3);  // issued once this chunk's are used
        }
        if constexpr (L::STAGES == 2) prefetch(c + 2 < c_end ? c + 2 : c);
        lds_barrier();
    };

    // Each iteration first waits for everything issued during the previous step
    // (this chunk's W/Q DMA and register operands, the previous outputs and
    // prefetches), then computes this chunk while issuing the next one's loads.
    auto iter = [&](Ops& cur, Ops& nxt, int64_t c) {
        if constexpr (L::STAGES == 1) {
            const __amdgpu_buffer_rsrc_t rr = rec_rsrc(c);
            if (has_rt) {
#pragma unroll
                for (int ks = 0; ks < R::DKS; ++ks) dma_ks(rr, c, ks);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this chunk's DMA has landed
        } else {
            __builtin_amdgcn_s_waitcnt(WAIT_AFTER);  // this chunk's DMA (issued one step ago) has landed
        }
        __builtin_amdgcn_sched_barrier(0);
        step(cur, nxt, c);
    };
    Ops opA, opB;
    if (c_begin < c_end) {
        const __amdgpu_buffer_rsrc_t rr = rec_rsrc(c_begin);
        if constexpr (L::STAGES == 2) {
            if (has_rt) {
#pragma unroll
                for (int ks = 0; ks < R::DKS; ++ks) dma_ks(rr, c_begin, ks);
            }
        }
#pragma unroll
        for (int p_ = 0; p_ < NLD; ++p_) load_part(opA, rr, c_begin, p_);
        if constexpr (L::STAGES == 2) prefetch(c_begin + 1 < c_end ? c_begin + 1 : c_begin);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): first chunk's operands are in
    }
    for (int64_t c = c_begin; c < c_end; c += 2) {
        iter(opA, opB, c);
        if (c + 1 >= c_end) break;
        iter(opB, opA, c + 1);
    }

    if (final_state) {
#pragma unroll
        for (int a = 0; a < MT_W; ++a) {
            const int mt = wave + 4 * a;
            if (mt >= R::MT) continue;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<f32x4*>(final_state + st_base + (size_t)(row0 + nt * 16 + l16) * DK + mt * 16 +
                                          4 * g16) = S[a][nt];
        }
    }
}

// ------------------------------------------------------------------ dispatch

// Which bf16 hi/lo refinements the chain kernel applies to its two largest
// products (state operand S and W): bit 0 = S, bit 1 = W.  Default none (the
// errors stay well inside the bf16 tolerance); the environment variable
// GDN_CHAIN_SPLIT (0..3) selects a refined variant.
static int chain_split_mode()
{
    static int mode = -1;  // read once; racing initialisers store the same value
    if (mode < 0) {
        const char* e = getenv("GDN_CHAIN_SPLIT");
        mode = (e && e[0] >= '0' && e[0] <= '3') ? e[0] - '0' : 0;
    }
    return mode;
}

template <typename TIn, int C, int DK, int DV>
static hipError_t run_prefill(const PrefillArgs& a)
{
    using R = Rec<TIn, C, DK, DV>;
    if (R::BYTES > a.lay.record_bytes) return hipErrorInvalidValue;
    int32_t* header = reinterpret_cast<int32_t*>(a.ws + a.lay.off_header);
    ChunkInfo* tab = reinterpret_cast<ChunkInfo*>(a.ws + a.lay.off_chunk_tab);
    int32_t* first = reinterpret_cast<int32_t*>(a.ws + a.lay.off_seq_first);
    float* decay = reinterpret_cast<float*>(a.ws + a.lay.off_decay);
    unsigned char* records = a.ws + a.lay.off_records;
    const int varlen = a.cu_seqlens != nullptr;

    if (a.stages & 1) {
        int64_t grid_chunks;
        if (varlen) {
            hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, a.N, a.T, (int32_t)C,
                               a.lay.max_chunks, header, tab, first);
            grid_chunks = a.lay.max_chunks;
        } else {
            grid_chunks = (a.T + C - 1) / C;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (grid_chunks > 0) {
            const size_t smem = sizeof(IntraSmem<TIn, C, DK, DV>);
            static bool attr_set = false;  // idempotent attribute; racing writers store the same value
            if (!attr_set) {
                e = hipFuncSetAttribute((const void*)intra_kernel<TIn, C, DK, DV>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
                if (e != hipSuccess) return e;
                attr_set = true;
            }
            hipLaunchKernelGGL((intra_kernel<TIn, C, DK, DV>), dim3((uint32_t)grid_chunks, a.H), dim3(256), smem,
                               a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.g, a.beta, header, tab,
                               varlen, a.T, a.H, a.l2norm, decay, records, a.lay.record_bytes);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    if (!(a.stages & 2)) return hipSuccess;
    constexpr int NT = 1;
    const int64_t pairs = (int64_t)a.N * a.H;
    const int64_t groups = (pairs + 7) / 8;
    const int64_t blocks = groups * 8 * (DV / (16 * NT));
    if (pairs > 0x7fffffff || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
#define GDN_LAUNCH_CHAIN(SS_, SW_)                                                                                    \
    do {                                                                                                              \
        constexpr size_t lds_bytes = ChainLds<TIn, C, DK, NT, Rec<TIn, C, DK, DV>::SPLIT>::BYTES;                     \
        static bool attr = false; /* idempotent; racing writers store the same value */                               \
        if (!attr) {                                                                                                  \
            hipError_t ea = hipFuncSetAttribute((const void*)chain_kernel<TIn, C, DK, DV, NT, SS_, SW_>,               \
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);          \
            if (ea != hipSuccess) return ea;                                                                          \
            attr = true;                                                                                              \
        }                                                                                                             \
        hipLaunchKernelGGL((chain_kernel<TIn, C, DK, DV, NT, SS_, SW_>), dim3((uint32_t)blocks), dim3(256), lds_bytes, \
                           a.stream, header, tab, first, varlen, a.T, a.H, (int32_t)pairs, decay, records,            \
                           a.lay.record_bytes, a.init_state, a.final_state, (TIn*)a.o, a.scale);                      \
    } while (0)
    if constexpr (sizeof(TIn) == 4) {
        GDN_LAUNCH_CHAIN(false, false);  // fp32 operands: nothing to refine
    } else {
        switch (chain_split_mode()) {
            case 0: GDN_LAUNCH_CHAIN(false, false); break;
            case 1: GDN_LAUNCH_CHAIN(true, false); break;
            case 2: GDN_LAUNCH_CHAIN(false, true); break;
            default: GDN_LAUNCH_CHAIN(true, true); break;
        }
    }
#undef GDN_LAUNCH_CHAIN
    return hipGetLastError();
}

template <typename TIn, int C, int DK>
static hipError_t dispatch_dv(const PrefillArgs& a)
{
    switch (a.dv) {
        case 16: if constexpr (sizeof(TIn) == 4) return run_prefill<TIn, C, DK, 16>(a); break;
        case 32: if constexpr (sizeof(TIn) == 4) return run_prefill<TIn, C, DK, 32>(a); break;
        case 64: return run_prefill<TIn, C, DK, 64>(a);
        case 128: return run_prefill<TIn, C, DK, 128>(a);
        case 256: return run_prefill<TIn, C, DK, 256>(a);
        case 512: if constexpr (sizeof(TIn) == 2) return run_prefill<TIn, C, DK, 512>(a); break;
    }
    return hipErrorInvalidValue;
}

template <int C>
static hipError_t dispatch_f32_dk(const PrefillArgs& a)
{
    switch (a.dk) {
        case 16: return dispatch_dv<float, C, 16>(a);
        case 32: return dispatch_dv<float, C, 32>(a);
        case 64: return dispatch_dv<float, C, 64>(a);
        case 128: return dispatch_dv<float, C, 128>(a);
        case 256: return dispatch_dv<float, C, 256>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a)
{
    if (a.bf16) {
        if (a.chunk != 64) return hipErrorInvalidValue;
        switch (a.dk) {
            case 64: return dispatch_dv<uint16_t, 64, 64>(a);
            case 128: return dispatch_dv<uint16_t, 64, 128>(a);
            case 256: return dispatch_dv<uint16_t, 64, 256>(a);
        }
        return hipErrorInvalidValue;
    }
    switch (a.chunk) {
        case 16: return dispatch_f32_dk<16>(a);
        case 32: return dispatch_f32_dk<32>(a);
        case 64: return dispatch_f32_dk<64>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
