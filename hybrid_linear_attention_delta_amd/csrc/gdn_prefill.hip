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
//                       substitution in LDS, U (and for fp32 W) on MFMA.
//                       Writes an operand record per chunk-head whose
//                       fragments are laid out exactly in the per-lane order
//                       of the MFMA operands of the later kernels (one
//                       16-byte load per operand); for bf16 it holds the raw
//                       K rows and T' = T diag(beta e^{gamma} r_k) in place
//                       of W = T' K.
//   chain_kr_kernel     bf16: one workgroup of 16 waves per (sequence, head,
//                       16 state rows), sequential over the sequence's chunks;
//                       state tile in fp32 MFMA accumulators, a rounded copy in
//                       LDS as the MFMA operand; Delta = U - T' (K S^T) and the
//                       state update from the chunk's K tile in LDS (row reads
//                       and transposing reads); writes the state entering
//                       every chunk, every chunk's Delta and the final state.
//                       Eight compute waves run only LDS and MFMA work between
//                       three barriers per chunk; loader waves bring the
//                       operands two chunks ahead by LDS-DMA and write the
//                       per-chunk outputs.
//   chain_kernel        fp32: the same recurrence as Delta = U - W S^T with W
//                       and K^T fragments read from the record.
//   output_kernel       one workgroup per (chunk, head), fully parallel: the
//                       outputs O of the chunk from Q, P, the state entering
//                       the chunk and Delta.
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
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

// Cache policy of the buffer stores that write data read only by a later
// kernel (the chain's per-chunk states and corrected values, the outputs):
// the non-temporal (nt) bit on gfx950.  Together with non-temporal record
// stores in the intra kernel this keeps the chain's prefetched records in
// L2 while the other kernels stream beside it (64K tokens: chain alone 1.345
// -> 1.304 ms, whole prefill 1.834 -> 1.784 ms).  Non-temporal loads in the
// output kernel measured slower and are not used.
constexpr int kNtAux = 2;

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
    __builtin_nontemporal_store(f, reinterpret_cast<typename Mma<TIn>::Frag*>(p));
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
// its row scale applied to the fp32 result).  This general layout serves the
// fp32 operands; the bf16 record (chunk 64) is the specialisation below.
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
    static constexpr int WH_OFF = 0;                                  // [RT][DKS][64][E] W, sigma over d_k
    static constexpr int K_OFF = WH_OFF + C * DK;                     // [MT][CKS][64][E] raw K^T, identity over chunk
    static constexpr int Q_OFF = K_OFF + C * DK;                      // [RT][DKS][64][E] raw Q, sigma over d_k
    static constexpr int PH_OFF = Q_OFF + C * DK;                     // [RT][CKS][64][E] P hi
    static constexpr int PL_OFF = PH_OFF + C * C;                     // [RT][CKS][64][E] P lo (bf16 only)
    static constexpr int CHAIN_ELEMS = Q_OFF;                         // the state chain's shared operands: W, K^T
    static constexpr int OPER_ELEMS = PL_OFF + (SPLIT ? C * C : 0);
    static constexpr size_t U_BYTE_OFF = ((size_t)OPER_ELEMS * sizeof(TIn) + 15) / 16 * 16;  // f32 [RT][VT][64][4]
    static constexpr size_t QS_BYTE_OFF = U_BYTE_OFF + (size_t)C * DV * 4;  // f32 [C]: rq_r e^{gamma_r}
    static constexpr size_t KSC_BYTE_OFF = QS_BYTE_OFF + (size_t)C * 4;     // f32 [C]: rk_j e^{gamma_L - gamma_j}
    static constexpr size_t DEC_BYTE_OFF = KSC_BYTE_OFF + (size_t)C * 4;    // {e^{gamma_L}, tok0, len, 0} (f32, i32, i32)
    static constexpr size_t BYTES = DEC_BYTE_OFF + 16;
    static_assert(C % KS == 0 && DK % KS == 0, "tile shape");
};

// bf16 (chunk 64): the state chain forms X = W S^T as T' (K^ S^T), with
// T' = T diag(beta e^{gamma} r_k) the 64 x 64 factor of W = T' K^.  The record
// therefore carries the chunk's raw K rows (once, in the LDS tile order of the
// chain, from which the chain reads both K^ and K^T fragments) and T', instead
// of the W and K^T fragments: 40 KB instead of 64 KB of the chain's operands
// per chunk-head at d_k = 256.  The chain's per-chunk operand volume is what
// bounds it (each workgroup streams the chunk's operands from L2 every step).
template <int C, int DK, int DV>
struct Rec<uint16_t, C, DK, DV> {
    static constexpr bool SPLIT = true;
    static constexpr int KS = 32, E = 8;
    static constexpr int RT = C / 16;               // chunk row tiles
    static constexpr int DKS = DK / KS;             // k-steps over d_k
    static constexpr int CKS = C / KS;              // k-steps over the chunk
    static constexpr int MT = DK / 16;              // d_k tiles
    static constexpr int VT = DV / 16;              // d_v tiles
    static constexpr int KR_OFF = 0;                // [C][DK] raw K rows, KTile<DK> layout; rows >= len zero
    static constexpr int TP_OFF = KR_OFF + C * DK;  // [RT][CKS][64][E] T' (bf16), sigma over the chunk
    static constexpr int Q_OFF = TP_OFF + C * C;    // [RT][DKS][64][E] raw Q, sigma over d_k
    static constexpr int PH_OFF = Q_OFF + C * DK;   // [RT][CKS][64][E] P hi
    static constexpr int PL_OFF = PH_OFF + C * C;   // [RT][CKS][64][E] P lo
    static constexpr int CHAIN_ELEMS = Q_OFF;       // the state chain's shared operands: K rows, T'
    static constexpr int OPER_ELEMS = PL_OFF + C * C;
    static constexpr size_t U_BYTE_OFF = ((size_t)OPER_ELEMS * 2 + 15) / 16 * 16;  // f32 [RT][VT][64][4]
    static constexpr size_t QS_BYTE_OFF = U_BYTE_OFF + (size_t)C * DV * 4;
    static constexpr size_t KSC_BYTE_OFF = QS_BYTE_OFF + (size_t)C * 4;
    static constexpr size_t DEC_BYTE_OFF = KSC_BYTE_OFF + (size_t)C * 4;
    static constexpr size_t BYTES = DEC_BYTE_OFF + 16;
    static_assert(C == 64 && DK % KS == 0, "tile shape");
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

// Sequences ranked by length for the state chain's dispatch order up to this
// many sequences (the ranking is quadratic); beyond it, the order of the batch.
constexpr int32_t kSortMax = 2048;

// One workgroup.  Validates cu_seqlens (0 = c_0 <= ... <= c_N = T), writes the
// first chunk of every sequence and the (tok0, len, seq) of every chunk.  On
// invalid input it raises header[0] and publishes zero chunks, so later
// kernels touch nothing.  Also writes order[r] = the sequence of rank r by
// length (longest first, ties by index): the chain hands its workgroups to
// (sequence, head) pairs in this order, so the longest sequential chains are
// dispatched first and the shorter ones fill the CUs around them.
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu, int32_t N, int64_t T,
                                                          int32_t C, int64_t max_chunks, int32_t* __restrict__ header,
                                                          ChunkInfo* __restrict__ tab, int32_t* __restrict__ first,
                                                          int32_t* __restrict__ order)
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
    // the lengths staged in LDS once: the ranking reads each of them N times
    __shared__ int32_t len_s[kSortMax];
    if (N <= kSortMax)
        for (int32_t i = t; i < N; i += 256) len_s[i] = max(cu[i + 1] - cu[i], 0);
    __syncthreads();
    for (int32_t i = t; i < N; i += 256) {
        int32_t r = i;
        if (N <= kSortMax) {
            const int32_t Li = len_s[i];
            r = 0;
            for (int32_t j = 0; j < N; ++j) {
                const int32_t Lj = len_s[j];
                r += (Lj > Li || (Lj == Li && j < i)) ? 1 : 0;
            }
        }
        order[r] = i;  // ranks form a permutation of 0 .. N-1
    }
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
__device__ __forceinline__ void intra_chunk(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                    const TIn* __restrict__ v, const float* __restrict__ g,
                                                    const float* __restrict__ beta, const int32_t* __restrict__ header,
                                                    const ChunkInfo* __restrict__ tab, int32_t varlen, int64_t T,
                                                    int32_t H, int32_t l2norm,
                                                    unsigned char* __restrict__ records, size_t record_bytes,
                                                    int64_t c, int64_t slot)
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

    const int h = blockIdx.y;
    if (varlen && c >= header[1]) return;
    if (!varlen && c * C >= T) return;
    const ChunkInfo ci = chunk_info(tab, varlen, c, C, T);
    const int len = ci.len;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar branches
    const int g16 = lane >> 4, l16 = lane & 15;

    unsigned char* recb = records + ((size_t)slot * H + h) * record_bytes;
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
            st_frag<TIn>(rec + R::WH_OFF + ((size_t)f * 64 + lane) * E, frag_from<TIn>(x));
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
        *reinterpret_cast<f32x4*>(recb + R::DEC_BYTE_OFF) =
            f32x4{expf(gL), __int_as_float(ci.tok0), __int_as_float(ci.len), 0.f};
    }
}

// ---- bf16 form (C = 64)
//
// The chunk's rows are read once, with 16-byte loads along each row: K into
// LDS (row-major), V into registers (written to LDS once K is no longer
// needed), and Q straight into the operand registers of the wave that owns
// its rows.  Wave w owns chunk rows 16w..16w+15: it forms G = K K^T and
// R = K Q^T for those columns against K row tiles 0..w (both products share
// the K operand), the row norms from the operand fragments themselves, and
// writes its rows of A, its P fragments, its Q fragments and its per-row
// scales.  The K^T fragments of the state update are read down the columns
// of the LDS rows.  T, W and U follow as in the general form.

// Row-major bf16 tile in LDS, W elements per row.  The 16-byte chunks of row
// j are stored in the order chunk ^ mask(j), which spreads 16-byte row
// writes, 8-byte reads of one column group over 16 consecutive rows, and
// 2-byte reads down a column at rows 8 apart, over all banks.
template <int W>
struct RowTile {
    static constexpr int CPR = W / 8;  // 16-byte chunks per row
    static __device__ __forceinline__ int chunk(int j, int ch) { return ch ^ ((j ^ (j >> 3)) & (CPR - 1)); }
    static __device__ __forceinline__ int at(int j, int col) { return j * W + (chunk(j, col >> 3) << 3) + (col & 7); }
};

// The state chain's K tile (bf16, chunk 64 x DK, in the record and in the
// chain's LDS): row j holds the chunk's raw K row j in 8-byte units of four
// columns; logical unit 8 kb + 2 g + u holds columns 32 kb + 16 u + 4 g .. + 3
// (so units 2 (4 kb + g) and 2 (4 kb + g) + 1 are the sigma-ordered operand
// slots of lane group g for k-step kb), stored at unit (8 kb + 2 g + u) ^ s(j).
// s(j) places row bits 0, 2, 1, 3 at unit bits 0, 2, 3, 4.  A row fragment
// is two 8-byte reads, and four consecutive columns of a 16-column tile are
// one 8-byte unit, as the transposing read needs.  Both are free of LDS bank
// conflicts: the 32 lanes of one pass touch 32 distinct bank pairs, for a
// row-fragment half (16 consecutive rows x 2 lane groups) as for a
// transposing read (rows 8 g + 4 h + i of 2 lane groups x 4 units).  (A
// 16-byte row read with the halves swapped on odd rows, which the same
// conditions allow, measured slower.)
template <int DK>
struct KTile {
    static constexpr int UPR = DK / 4;  // 8-byte units per row
    static __device__ __forceinline__ int swz(int j)
    {
        return ((j & 1) | (j & 4) | ((j & 2) << 2) | ((j & 8) << 1)) & (UPR - 1);
    }
    // element offset of unit (block kb, lane group g, half u) of row j
    static __device__ __forceinline__ int at(int j, int kb, int g, int u)
    {
        return j * DK + (((8 * kb + 2 * g + u) ^ swz(j)) << 2);
    }
};

template <int DK, int DV>
struct IntraBf {
    static constexpr int C = 64;
    static constexpr int VP = DV < 256 ? DV : 256;  // value columns per pass
    static constexpr int NVP = DV / VP;
    static constexpr int XW = DK > VP ? DK : VP;    // row width of the tile region
    static constexpr int AP = C + 4;                // fp32 pitch of A and T
    static constexpr int KLD = C * (DK / 8) / 256;  // 16-byte loads per thread: K
    static constexpr int VLD = C * (VP / 8) / 256;  //                           V (one pass)
    static constexpr int DKS = DK / 32;             // d_k blocks of one k-step
    static constexpr int DBW = (DKS + 3) / 4;       // d_k blocks per wave
    static constexpr int VTP = VP / 16;             // value tiles per pass
    static constexpr int VTW = (VTP + 3) / 4;       // value tiles per wave and pass
    static_assert(KLD >= 1 && VLD >= 1, "row loads");
};

template <int DK, int DV>
struct IntraBfSmem {
    using Cf = IntraBf<DK, DV>;
    uint16_t x[Cf::C * Cf::XW];  // K rows, later V rows of one pass
    float at[Cf::C * Cf::AP];    // A, strictly lower
    float tt[Cf::C * Cf::AP];    // T = (I + A)^{-1}, lower blocks
    float gam[Cf::C], beta[Cf::C], sw[Cf::C];
};

// The front end folded into the row loads: chunk rows j0 .. j0 + NR - 1 of one
// 8-channel group, each y_t = silu(4-tap causal convolution) of the bf16
// projection x ([tokens][ld], columns col .. col + 7; channels chan .. chan + 7
// of the concatenated conv axis for the taps and the conv state), rounded to
// bf16 exactly as the standalone front end rounds it.  The three inputs before
// a sequence come from its conv state (zeros without one); rows at or past
// len are zero (and nothing past them is read).  The NR + 3 rows are read once
// and the window slides down them in registers.
template <int NR>
__device__ __forceinline__ void conv_strip(const uint16_t* __restrict__ x, int64_t ld, int col, const FrontIn& fe,
                                           int32_t ctot, int32_t chan, int32_t seq, int64_t seq_start, int64_t tok0,
                                           int j0, int len, uint4 (&out)[NR])
{
    float wt[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(fe.w + (int64_t)(chan + e) * 4);
        wt[e][0] = t[0]; wt[e][1] = t[1]; wt[e][2] = t[2]; wt[e][3] = t[3];
    }
    uint4 raw[NR + 3];
#pragma unroll
    for (int m = 0; m < NR + 3; ++m) {
        const int j = j0 - 3 + m;  // chunk row (negative: before the chunk)
        const int64_t p = tok0 + j;
        uint4 r = {0u, 0u, 0u, 0u};
        if (j < len) {
            if (p >= seq_start) {
                r = *reinterpret_cast<const uint4*>(x + p * ld + col);
            } else if (fe.state_in) {
                const int sl = 3 - (int)(seq_start - p);  // slot of the conv state, oldest first
                if (sl >= 0)
                    r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(fe.state_in) +
                                                         ((int64_t)seq * 3 + sl) * ctot + chan);
            }
        }
        raw[m] = r;
    }
    auto widen = [](uint4 r, float (&y)[8]) {
        const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[2 * i] = __uint_as_float(u[i] << 16);
            y[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    };
    float h0[8], h1[8], h2[8];
    widen(raw[0], h0);
    widen(raw[1], h1);
    widen(raw[2], h2);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float xr[8], y[8];
        widen(raw[r + 3], xr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[e] = conv4_silu(wt[e], h0[e], h1[e], h2[e], xr[e]);
            h0[e] = h1[e];
            h1[e] = h2[e];
            h2[e] = xr[e];
        }
        uint4 o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
        out[r] = j0 + r < len ? o : uint4{0u, 0u, 0u, 0u};
    }
}

template <int DK, int DV, bool FE>
__device__ __forceinline__ void intra_chunk_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v, const float* __restrict__ g,
                                                 const float* __restrict__ beta, const int32_t* __restrict__ header,
                                                 const ChunkInfo* __restrict__ tab, int32_t varlen, int64_t T,
                                                 int32_t H, int32_t l2norm, unsigned char* __restrict__ records,
                                                 size_t record_bytes, int64_t c, int64_t slot, const FrontIn& fe)
{
    using M = Mma<uint16_t>;
    using F = Mma<float>;
    using Cf = IntraBf<DK, DV>;
    using R = Rec<uint16_t, 64, DK, DV>;
    using KX = RowTile<DK>;
    using VX = RowTile<Cf::VP>;
    typedef typename M::Frag Frag;
    constexpr int C = 64, AP = Cf::AP, RT = 4, DKS = Cf::DKS, E = 8;
    constexpr int KCPR = DK / 8, VCPR = Cf::VP / 8;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    IntraBfSmem<DK, DV>& sm = *reinterpret_cast<IntraBfSmem<DK, DV>*>(smem_raw);

    const int h = blockIdx.y;
    if (varlen && c >= header[1]) return;
    if (!varlen && c * C >= T) return;
    const ChunkInfo ci = chunk_info(tab, varlen, c, C, T);
    const int len = ci.len;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // = the row tile this wave owns
    const int g16 = lane >> 4, l16 = lane & 15;

    unsigned char* recb = records + ((size_t)slot * H + h) * record_bytes;
    uint16_t* rec = reinterpret_cast<uint16_t*>(recb);
    float* recU = reinterpret_cast<float*>(recb + R::U_BYTE_OFF);
    const int64_t row0 = (int64_t)ci.tok0 * H + h;  // row index of token tok0 in [tokens*H]

    // ---- phase 1: every global read of the chunk, issued up front.  Thread
    // tid owns the 16-byte row pieces (j, ch) of K and V given by kmap / vmap:
    // strided over rows when q, k, v are inputs; with the front end folded in
    // (FE), KLD (VLD) consecutive rows of one 8-channel group, so that the
    // 4-token window slides down them and each projection row is read once,
    // plus three halo rows per strip.
    auto kmap = [&](int s, int& j, int& ch) {
        if constexpr (FE) {
            ch = tid % KCPR;
            j = (tid / KCPR) * Cf::KLD + s;
        } else {
            const int qi = s * 256 + tid;
            j = qi / KCPR;
            ch = qi % KCPR;
        }
    };
    auto vmap = [&](int s, int& j, int& ch) {
        if constexpr (FE) {
            ch = tid % VCPR;
            j = (tid / VCPR) * Cf::VLD + s;
        } else {
            const int qi = s * 256 + tid;
            j = qi / VCPR;
            ch = qi % VCPR;
        }
    };
    const int32_t ctot = H * (2 * DK + DV);                    // FE: channels of the conv axis
    const int64_t seq_start = FE && varlen ? fe.cu[ci.seq] : 0;  // FE: first token of the chunk's sequence
    float gv = 0.f, bv = 0.f;
    if (wave == 0 && lane < len) {
        if constexpr (FE) {
            const int64_t e = row0 + (int64_t)lane * H;
            gv = gate_g(fe.a[e], fe.A_log[h], fe.dt_bias[h]);
            bv = gate_beta(fe.b[e]);
        } else {
            gv = g[row0 + (int64_t)lane * H];
            bv = beta[row0 + (int64_t)lane * H];
        }
    }
    uint4 kr[Cf::KLD];
    if constexpr (FE) {
        int j0, ch;
        kmap(0, j0, ch);
        conv_strip<Cf::KLD>(reinterpret_cast<const uint16_t*>(fe.xk), (int64_t)H * DK, h * DK + ch * 8, fe, ctot,
                            H * DK + h * DK + ch * 8, ci.seq, seq_start, ci.tok0, j0, len, kr);
    } else {
#pragma unroll
        for (int s = 0; s < Cf::KLD; ++s) {
            int j, ch;
            kmap(s, j, ch);
            kr[s] = j < len ? *reinterpret_cast<const uint4*>(k + (row0 + (int64_t)j * H) * DK + ch * 8)
                            : uint4{0u, 0u, 0u, 0u};
        }
    }
    const int r_own = wave * 16 + l16;  // the chunk row (column of the products) this lane owns
    const bool live = r_own < len;
    Frag qf[DKS];  // Q row r_own in sigma order over d_k: operand of R and the stored Q fragments
    if constexpr (FE) {
        // the convolved Q rows pass through the A / T region of LDS (free until phase 2)
        // as a row tile, from which the sigma fragments are read below
        uint4 qr[Cf::KLD];
        int j0, ch;
        kmap(0, j0, ch);
        conv_strip<Cf::KLD>(reinterpret_cast<const uint16_t*>(fe.xq), (int64_t)H * DK, h * DK + ch * 8, fe, ctot,
                            h * DK + ch * 8, ci.seq, seq_start, ci.tok0, j0, len, qr);
        static_assert(sizeof(sm.at) + sizeof(sm.tt) >= sizeof(uint16_t) * C * DK, "Q tile fits the A and T region");
        uint16_t* qt = reinterpret_cast<uint16_t*>(sm.at);
#pragma unroll
        for (int s = 0; s < Cf::KLD; ++s)
            *reinterpret_cast<uint4*>(qt + (j0 + s) * DK + (KX::chunk(j0 + s, ch) << 3)) = qr[s];
    } else {
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks)
            qf[ks] = live ? M::ld_sigma(q + (row0 + (int64_t)r_own * H) * DK + ks * 32, g16) : zero_frag<uint16_t>();
    }
    uint4 vr[Cf::VLD];
    auto load_v = [&](int pass) {
        if constexpr (FE) {
            int j0, ch;
            vmap(0, j0, ch);
            conv_strip<Cf::VLD>(reinterpret_cast<const uint16_t*>(fe.xv), (int64_t)H * DV, h * DV + pass * Cf::VP + ch * 8,
                                fe, ctot, 2 * H * DK + h * DV + pass * Cf::VP + ch * 8, ci.seq, seq_start, ci.tok0,
                                j0, len, vr);
        } else {
#pragma unroll
            for (int s = 0; s < Cf::VLD; ++s) {
                int j, ch;
                vmap(s, j, ch);
                vr[s] = j < len ? *reinterpret_cast<const uint4*>(v + (row0 + (int64_t)j * H) * DV + pass * Cf::VP +
                                                                  ch * 8)
                                : uint4{0u, 0u, 0u, 0u};
            }
        }
    };
    load_v(0);

    // gates: gamma (inclusive scan within the chunk), beta; rows >= len: g = 0, beta = 0
    if (wave == 0) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gv, off, 64);
            if (lane >= off) gv += y;
        }
        sm.gam[lane] = gv;
        sm.beta[lane] = bv;
    }
#pragma unroll
    for (int s = 0; s < Cf::KLD; ++s) {
        int j, ch;
        kmap(s, j, ch);
        *reinterpret_cast<uint4*>(sm.x + j * DK + (KX::chunk(j, ch) << 3)) = kr[s];
    }
    __syncthreads();

    // ---- phase 2: G, R against K row tiles 0..wave; A rows, P, Q fragments, row scales
    auto tile_sigma = [&](const uint16_t* tl, int r, int ks) -> Frag {
        const u16x4 lo = *reinterpret_cast<const u16x4*>(tl + KX::at(r, ks * 32 + 4 * g16));
        const u16x4 hi = *reinterpret_cast<const u16x4*>(tl + KX::at(r, ks * 32 + 16 + 4 * g16));
        Frag f;
        f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
        f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
        return f;
    };
    auto lds_sigma = [&](int r, int ks) -> Frag { return tile_sigma(sm.x, r, ks); };
    if constexpr (FE) {
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) qf[ks] = tile_sigma(reinterpret_cast<const uint16_t*>(sm.at), r_own, ks);
        __syncthreads();  // the Q tile is read; A may be written
    }
    // 1/||x|| of the row whose sigma fragments this lane and its three partner lanes hold
    auto inv_norm = [&](const Frag* f, bool row_live) -> float {
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = bf16_bits_to_f32(f[ks][e]);
                ss += x * x;
            }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        return row_live ? (l2norm ? 1.0f / sqrtf(ss + kNormEps) : 1.0f) : 0.f;
    };
    const float rq = inv_norm(qf, live);
    Frag kw[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) kw[ks] = lds_sigma(r_own, ks);
    const float rk = inv_norm(kw, live);
    const float gam_r = sm.gam[r_own], beta_r = sm.beta[r_own];
    float px[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) px[u][e] = 0.f;
#pragma unroll
    for (int tj = 0; tj < RT; ++tj) {
        if (tj > wave) break;
        Frag kt[DKS];
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) kt[ks] = lds_sigma(tj * 16 + l16, ks);
        const float rkt = inv_norm(kt, tj * 16 + l16 < len);
        f32x4 aG = {0.f, 0.f, 0.f, 0.f}, aR = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) {
            aG = M::mma(kt[ks], kw[ks], aG);
            aR = M::mma(kt[ks], qf[ks], aR);
        }
        // lane holds rows j = 16 tj + 4 g16 + i of column r_own of K K^T and K Q^T
        f32x4 av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = tj * 16 + 4 * g16 + i;
            const float rkj = __shfl(rkt, 4 * g16 + i, 64);
            const float d = expf(gam_r - sm.gam[j]);  // used only for j <= r_own, where the exponent is <= 0
            av[i] = j < r_own ? beta_r * rk * rkj * aG[i] * d : 0.f;
            px[tj >> 1][(tj & 1) * 4 + i] = j <= r_own ? rq * rkj * aR[i] * d : 0.f;
        }
        *reinterpret_cast<f32x4*>(sm.at + r_own * AP + tj * 16 + 4 * g16) = av;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        if (ks > wave / 2) break;  // P row tile `wave` has k-steps up to its diagonal
        Frag hi, lo;
        split_frag<uint16_t>(px[ks], hi, lo);
        const size_t fo = ((size_t)(wave * R::CKS + ks) * 64 + lane) * E;
        st_frag<uint16_t>(rec + R::PH_OFF + fo, hi);
        st_frag<uint16_t>(rec + R::PL_OFF + fo, lo);
    }
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) st_frag<uint16_t>(rec + R::Q_OFF + ((size_t)(wave * DKS + ks) * 64 + lane) * E, qf[ks]);
    if (g16 == 0) {
        const float gL = sm.gam[C - 1];  // rows >= len carry g = 0, so this is gamma at len-1
        const float eg = expf(gam_r);
        sm.sw[r_own] = beta_r * eg * rk;  // W = T diag(sw) K
        reinterpret_cast<float*>(recb + R::QS_BYTE_OFF)[r_own] = rq * eg;
        reinterpret_cast<float*>(recb + R::KSC_BYTE_OFF)[r_own] = rk * expf(gL - gam_r);
    }
    // the raw K rows for the state chain in its tile layout (rows >= len zero):
    // stored units 2 p, 2 p + 1 of row j hold logical units (2 p) ^ s(j) and
    // (2 p + 1) ^ s(j), the two halves of piece (block, lane group) = p ^ (s(j) / 2),
    // swapped when s(j) is odd
#pragma unroll
    for (int s = 0; s < Cf::KLD; ++s) {
        const int pc = s * 256 + tid;  // stored 16-byte chunk
        const int j = pc / KCPR, sw = KTile<DK>::swz(j), lp = (pc % KCPR) ^ (sw >> 1), kb = lp >> 2, gp = lp & 3;
        const u16x4 lo = *reinterpret_cast<const u16x4*>(sm.x + KX::at(j, kb * 32 + 4 * gp));
        const u16x4 hi = *reinterpret_cast<const u16x4*>(sm.x + KX::at(j, kb * 32 + 16 + 4 * gp));
        const u16x8 v = (sw & 1) ? u16x8{hi.x, hi.y, hi.z, hi.w, lo.x, lo.y, lo.z, lo.w}
                                 : u16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(rec + R::KR_OFF + pc * 8));
    }
    __syncthreads();  // K rows no longer read; A complete

    // ---- phase 3: V rows into LDS; T = (I + A)^{-1}
    auto store_v = [&]() {
#pragma unroll
        for (int s = 0; s < Cf::VLD; ++s) {
            int j, ch;
            vmap(s, j, ch);
            *reinterpret_cast<uint4*>(sm.x + j * Cf::VP + (VX::chunk(j, ch) << 3)) = vr[s];
        }
    };
    store_v();
    if constexpr (Cf::NVP > 1) load_v(1);
    if (tid == 0) {
        *reinterpret_cast<f32x4*>(recb + R::DEC_BYTE_OFF) =
            f32x4{expf(sm.gam[C - 1]), __int_as_float(ci.tok0), __int_as_float(ci.len), 0.f};
    }
    {   // diagonal 16x16 blocks by forward substitution, one per wave
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
    __syncthreads();
    // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj on fp32 MFMA, by block distance
#pragma unroll
    for (int dd = 1; dd < RT; ++dd) {
        const int jb = wave, ib = wave + dd;
        if (ib < RT) {
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

    // ---- phase 4: T' = T diag(sw) for the state chain, and U = (T diag(beta)) V with
    // T diag(beta) split hi/lo.  Row r = 16 rt + l16 of T diag(beta) over k-step jk
    // is the A operand of U; entries above the diagonal are zero (masked here, the
    // blocks above the diagonal are never written).
    auto t_frags = [&](int rt, int jk, bool want_w, Frag& swh, Frag& swl, Frag& sbh, Frag& sbl) {
        const int r = rt * 16 + l16, j0 = jk * 32 + g16 * 8;
        const f32x4 t0 = *reinterpret_cast<const f32x4*>(sm.tt + r * AP + j0);
        const f32x4 t1 = *reinterpret_cast<const f32x4*>(sm.tt + r * AP + j0 + 4);
        float xs[E], xb[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float tv = j0 + e <= r ? (e < 4 ? t0[e] : t1[e - 4]) : 0.f;
            xs[e] = tv * sm.sw[j0 + e];
            xb[e] = tv * sm.beta[j0 + e];
        }
        if (want_w) split_frag<uint16_t>(xs, swh, swl);
        split_frag<uint16_t>(xb, sbh, sbl);
    };
    auto v_frags = [&](Frag (&vf)[Cf::VTW][2]) {
#pragma unroll
        for (int t = 0; t < Cf::VTW; ++t) {
            const int vt = wave + 4 * t;
            if (vt >= Cf::VTP) break;
#pragma unroll
            for (int jk = 0; jk < 2; ++jk) {
                Frag f;
#pragma unroll
                for (int e = 0; e < E; ++e) f[e] = sm.x[VX::at(jk * 32 + g16 * 8 + e, vt * 16 + l16)];
                vf[t][jk] = f;
            }
        }
    };
    auto u_tiles = [&](int pass, int rt, int nks, const Frag (&vf)[Cf::VTW][2], const Frag* sbh, const Frag* sbl) {
#pragma unroll
        for (int t = 0; t < Cf::VTW; ++t) {
            const int vt = wave + 4 * t;
            if (vt >= Cf::VTP) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jk = 0; jk < 2; ++jk) {
                if (jk >= nks) break;
                acc = M::mma(sbh[jk], vf[t][jk], acc);
                acc = M::mma(sbl[jk], vf[t][jk], acc);
            }
            const int vg = pass * Cf::VTP + vt;
            __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(recU + ((size_t)(rt * R::VT + vg) * 64 + lane) * 4));
        }
    };
    // T' = T diag(sw): row tile `wave`, both k-steps, sigma order over the chunk
    // (lane group g, element e holds column 32 ks + 16 (e / 4) + 4 g + e % 4);
    // zero above the diagonal
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int r = wave * 16 + l16, j0 = ks * 32 + 4 * g16;
        const f32x4 t0 = *reinterpret_cast<const f32x4*>(sm.tt + r * AP + j0);
        const f32x4 t1 = *reinterpret_cast<const f32x4*>(sm.tt + r * AP + j0 + 16);
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = j0 + 16 * (e >> 2) + (e & 3);
            const float tv = e < 4 ? t0[e & 3] : t1[e & 3];
            x[e] = j <= r ? tv * sm.sw[j] : 0.f;
        }
        st_frag<uint16_t>(rec + R::TP_OFF + ((size_t)(wave * R::CKS + ks) * 64 + lane) * E, frag_from<uint16_t>(x));
    }
    {
        Frag vf[Cf::VTW][2];
        v_frags(vf);
#pragma unroll 1
        for (int rt = 0; rt < RT; ++rt) {
            const int nks = rt / 2 + 1;  // T[r][j] = 0 for j > r
            Frag swh[2], swl[2], sbh[2], sbl[2];
#pragma unroll
            for (int jk = 0; jk < 2; ++jk)
                if (jk < nks) t_frags(rt, jk, false, swh[jk], swl[jk], sbh[jk], sbl[jk]);
            u_tiles(0, rt, nks, vf, sbh, sbl);
        }
    }
#pragma unroll 1
    for (int pass = 1; pass < Cf::NVP; ++pass) {
        __syncthreads();  // the previous pass's value rows are no longer read
        store_v();
        if (pass + 1 < Cf::NVP) load_v(pass + 1);
        __syncthreads();
        Frag vf[Cf::VTW][2];
        v_frags(vf);
#pragma unroll 1
        for (int rt = 0; rt < RT; ++rt) {
            const int nks = rt / 2 + 1;
            Frag swh[2], swl[2], sbh[2], sbl[2];
#pragma unroll
            for (int jk = 0; jk < 2; ++jk)
                if (jk < nks) t_frags(rt, jk, false, swh[jk], swl[jk], sbh[jk], sbl[jk]);
            u_tiles(pass, rt, nks, vf, sbh, sbl);
        }
    }
}

// One workgroup per (chunk, head), for the chunks [c_base, c_end).  With FE
// (bf16, chunk 64 only) the front end is folded into the row loads: fe holds
// the projections and gate inputs, and q, k, v, g, beta are unused.
template <typename TIn, int C, int DK, int DV, bool FE>
__global__ __launch_bounds__(256) void intra_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                    const TIn* __restrict__ v, const float* __restrict__ g,
                                                    const float* __restrict__ beta, const int32_t* __restrict__ header,
                                                    const ChunkInfo* __restrict__ tab, int32_t varlen, int64_t T,
                                                    int32_t H, int32_t l2norm,
                                                    unsigned char* __restrict__ records, size_t record_bytes,
                                                    int64_t c_base, int64_t c_end, int64_t slot0, FrontIn fe)
{
    // chunk c's record is slot c - slot0 of `records` (slot0 = 0 unless the
    // workspace holds a window of the chunks)
    const int64_t c = c_base + blockIdx.x;
    if (c >= c_end) return;
    if constexpr (sizeof(TIn) == 2 && C == 64)
        intra_chunk_bf16<DK, DV, FE>(q, k, v, g, beta, header, tab, varlen, T, H, l2norm, records, record_bytes, c,
                                     c - slot0, fe);
    else if constexpr (!FE)
        intra_chunk<TIn, C, DK, DV>(q, k, v, g, beta, header, tab, varlen, T, H, l2norm, records, record_bytes, c,
                                    c - slot0);
}

// ------------------------------------------------------------------ chain kernel

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

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (lgkmcnt) but not for its outstanding global loads, which are register
// prefetches consumed by this wave alone.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Work split of the fp32 chain kernel over NW compute waves (NW a multiple of 4).
template <typename TIn, int C, int DK, int DV, int NW>
struct ChainSplit {
    using R = Rec<TIn, C, DK, DV>;
    static constexpr int KQ = (NW / 4) < R::DKS ? (NW / 4) : R::DKS;  // d_k split of X = W S^T
    static constexpr int KPW = R::DKS / KQ;                             // k-steps per phase-1 wave
    static constexpr int MTW = (R::MT + NW - 1) / NW;                   // state d_k tiles per wave
    static_assert(R::DKS % KQ == 0, "d_k split");
};

// Per-chunk outputs of the state chain, read by the output kernel.
//   states: [chunk][H][DV][DK] operand type, the state entering the chunk; bf16
//           rows are in sigma order within each 32-column block
//   deltas: [chunk][H][NS][DV][C] operand type, Delta^T (hi, lo for bf16), sigma
//           order over the chunk positions (natural order for fp32)
template <typename TIn, int C, int DK, int DV>
struct ChainOut {
    static constexpr int NS = sizeof(TIn) == 2 ? 2 : 1;
    static constexpr size_t STATE_ELEMS = (size_t)DV * DK;
    static constexpr size_t DELTA_ELEMS = (size_t)NS * DV * C;
};

// LDS of the fp32 chain kernel (its operands are read from the records directly).
template <int C, int DK, int DV, int NW>
struct ChainLds {
    using P = ChainSplit<float, C, DK, DV, NW>;
    static constexpr int SP = DK + 4;  // state copy pitch (dwords = 4 mod 32)
    static constexpr int DP = C + 4;   // (kscale o Delta)^T pitch
    static constexpr int RT = C / 16;
    float sr[16 * SP];                 // state rows S[r][col]
    float ds[16 * DP];                 // (kscale o Delta)^T[r][j]
    f32x4 xp[P::KQ][RT][64];           // partial W S^T per d_k part
};

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Hand-offs of the pipelined prefill through device memory.  The bf16 state
// chain runs as one launch over every chunk while the intra-chunk kernel
// prepares the chunks segment by segment and the output kernel finishes them
// on other CUs.  flags[s] (s < kPipeMaxSeg) is raised by a one-wave kernel that
// follows segment s's intra-chunk kernel on its stream, so the kernel boundary
// has already made the records visible to the whole device; the chain's
// loader waves wait for it before the first transfer of a chunk of segment s.
// flags[kPipeMaxSeg + s] counts the chain's store waves (kPipePublishers per
// workgroup) that have written their part of every state and Delta of segment
// s, each after releasing its stores at agent scope; a one-wave kernel waits
// for all of them in front of segment s's output kernel.  flags[2 kPipeMaxSeg] counts waits that gave up.  Every wait
// is bounded by the device's constant 100 MHz clock (kPipeWaitTicks, about
// 1.3 s), so no wave can spin forever; one that gives up counts itself in
// flags[2 kPipeMaxSeg] and goes on.
constexpr int kPipeMaxSeg = 16;
constexpr int kPipeFlags = 2 * kPipeMaxSeg + 1;
constexpr uint64_t kPipeWaitTicks = (uint64_t)1 << 27;
constexpr uint32_t kPipePublishers = 2;  // store waves of a bf16 chain workgroup
struct PipeSync {
    uint32_t* flags;              // kPipeFlags words in the workspace header; null: no pipeline
    int32_t nseg;                 // segments
    int64_t end[kPipeMaxSeg];     // first chunk after segment s (end[nseg - 1] = every chunk)
};

// Waits until *p >= target (agent-scope loads), then acquires at agent scope.
__device__ __forceinline__ void pipe_wait(const uint32_t* p, uint32_t target, uint32_t* gave_up)
{
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kPipeWaitTicks) {
            if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(gave_up, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Zeroes the hand-off words (a kernel, not a memset, so that the call may be
// captured into a graph).
__global__ __launch_bounds__(64) void pipe_reset_kernel(uint32_t* flags)
{
    for (int i = threadIdx.x; i < kPipeFlags; i += 64) flags[i] = 0u;
}

// Raises flags[s]: every record of segment s, written by the kernels before
// this one on its stream, is visible to the device.
__global__ __launch_bounds__(64) void pipe_signal_kernel(uint32_t* flags, int32_t s)
{
    if (threadIdx.x == 0) __hip_atomic_store(flags + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns once `target` chain workgroups have finished segment s.
__global__ __launch_bounds__(64) void pipe_wait_kernel(uint32_t* flags, int32_t s, uint32_t target)
{
    pipe_wait(flags + kPipeMaxSeg + s, target, flags + 2 * kPipeMaxSeg);
}

// State chain, fp32 operands: one workgroup of NW waves per (sequence, head,
// 16 state rows), sequential over the sequence's chunks, operands read from the
// record.  Per chunk c:
//   phase 1  wave (rt, kq) = (w % 4, w / 4): partial X = W S^T of chunk row
//            tile rt over d_k part kq (partials to LDS)
//   phase 2  wave (rt, 0): Delta = U - X (k-scaled copy to LDS, Delta^T to `deltas`)
//   phase 3  every wave, its state d_k tiles: S^T = e^{gamma_L} S^T + K^T (kscale o Delta)
// separated by the barriers A, B, C; the state entering chunk c goes to
// `states`.  Workgroups are mapped so that all row tiles of one (sequence,
// head) pair run on one XCD (workgroups are dealt to the 8 XCDs
// round-robin): they read the same per-chunk records, which then come from
// that XCD's L2.  Pair indices follow seq_order (longest sequence first) in a
// packed batch, so when there are more workgroups than CUs the longest chains
// are dispatched first.
template <int C, int DK, int DV, int NW, bool SEG>
__global__ __launch_bounds__(NW * 64) void chain_kernel(
    const int32_t* __restrict__ header, const int32_t* __restrict__ seq_first,
    const int32_t* __restrict__ seq_order, int32_t varlen, int64_t T, int32_t H, int32_t pairs,
    const unsigned char* records, size_t record_bytes, const float* init_state, float* final_state,
    float* __restrict__ states, float* __restrict__ deltas, int64_t seg_begin, int64_t seg_end, float* carry,
    int64_t slot0)
{
    using TIn = float;
    using M = Mma<TIn>;
    using R = Rec<TIn, C, DK, DV>;
    using P = ChainSplit<TIn, C, DK, DV, NW>;
    using CO = ChainOut<TIn, C, DK, DV>;
    using L = ChainLds<C, DK, DV, NW>;
    typedef typename M::Frag Frag;
    constexpr int KS = M::KS, E = M::E;
    constexpr int SP = L::SP, DP = L::DP;
    constexpr int TILES = DV / 16;
    constexpr uint32_t FB = 64 * 16;  // bytes of one operand fragment (64 lanes x 16 B)
    constexpr uint32_t EB = sizeof(TIn);

    extern __shared__ __align__(16) unsigned char lds_raw[];
    L& sm = *reinterpret_cast<L*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar branches
    const int g16 = lane >> 4, l16 = lane & 15;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int pair = xcd + 8 * (slot / TILES);
    if (pair >= pairs) return;
    const int n = varlen ? seq_order[pair / H] : pair / H, h = pair % H;  // longest sequences first
    const int tile = slot % TILES;
    const int row0 = tile * 16;  // first state row (value index) of this workgroup

    // SEG: this launch covers the chunks [seg_begin, seg_end) of the global
    // chunk order; a sequence crossing a segment boundary carries its state
    // through `carry` ([N][H][d_v][d_k] fp32).  The state enters from
    // init_state (or zero) at the sequence's first chunk, else from carry, and
    // leaves to final_state after the sequence's last chunk, else to carry.
    // Without SEG the launch covers every chunk.
    int64_t s_first, s_last;  // the sequence's chunk range
    if (varlen) {
        if (header[0] != 0) return;
        s_first = seq_first[n];
        s_last = seq_first[n + 1];
    } else {
        s_first = 0;
        s_last = (T + C - 1) / C;
    }
    const int64_t c_begin = SEG && s_first < seg_begin ? seg_begin : s_first;
    const int64_t c_end = SEG && s_last > seg_end ? seg_end : s_last;
    if (c_begin >= c_end && !(s_first == s_last && s_first >= seg_begin && s_first < seg_end)) return;
    const float* state_in = c_begin == s_first ? init_state : carry;
    float* state_out_ptr = c_end == s_last ? final_state : carry;

    const uint32_t lane_b = (uint32_t)lane * 16;
    // chunk c's record, state and Delta are slot c - slot0 of their regions
    auto rec_ptr = [&](int64_t c) { return records + ((size_t)(c - slot0) * H + h) * record_bytes; };
    auto w_src = [&](int r, int ks) { return R::WH_OFF * EB + (uint32_t)(r * R::DKS + ks) * FB; };
    auto k_src = [&](int mt, int ks) { return R::K_OFF * EB + (uint32_t)(mt * R::CKS + ks) * FB; };
    auto u_src = [&](int r) { return (uint32_t)R::U_BYTE_OFF + (uint32_t)(r * R::VT + tile) * FB; };
    auto state_out = [&](int64_t c) {
        return states + ((size_t)(c - slot0) * H + h) * CO::STATE_ELEMS + (size_t)row0 * DK;
    };
    auto delta_out = [&](int64_t c) {
        return deltas + ((size_t)(c - slot0) * H + h) * CO::DELTA_ELEMS + (size_t)row0 * C;
    };

    // fragment of the current chunk at record byte offset `src`
    __amdgpu_buffer_rsrc_t rcur = make_rsrc(records, 0u);
    auto frag = [&](uint32_t src) -> Frag { return __builtin_bit_cast(Frag, buf_load16(rcur, lane_b, src)); };
    const int rt = wave & 3, kq = wave >> 2;
    const bool p1 = rt < R::RT && kq < P::KQ;  // phase-1 partial products
    const bool fin_d = rt < R::RT && kq == 0;  // Delta finaliser of row tile rt

    // state tiles S^T[mt] in result layout: lane holds S[row0 + l16][mt*16 + 4*g16 + i]
    f32x4 S[P::MTW];
    const size_t st_base = ((size_t)n * H + h) * DV * DK;
#pragma unroll
    for (int a = 0; a < P::MTW; ++a) {
        const int mt = wave + NW * a;
        S[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mt < R::MT) {
            if (state_in)
                S[a] = *reinterpret_cast<const f32x4*>(state_in + st_base + (size_t)(row0 + l16) * DK + mt * 16 +
                                                       4 * g16);
            *reinterpret_cast<f32x4*>(sm.sr + l16 * SP + mt * 16 + 4 * g16) = S[a];
        }
    }
    __syncthreads();

    for (int64_t c = c_begin; c < c_end; ++c) {
        rcur = make_rsrc(rec_ptr(c), (uint32_t)R::BYTES);
        // the state entering chunk c
#pragma unroll
        for (int a = 0; a < P::MTW; ++a) {
            const int mt = wave + NW * a;
            if (mt < R::MT) *reinterpret_cast<f32x4*>(state_out(c) + (size_t)l16 * DK + mt * 16 + 4 * g16) = S[a];
        }
        if (p1) {
            // ---- phase 1: partial X = W S^T over this wave's d_k part
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < P::KPW; ++i) {
                const int ks = kq * P::KPW + i;
                X = M::mma(frag(w_src(rt, ks)), *reinterpret_cast<const Frag*>(sm.sr + l16 * SP + ks * KS + g16 * E), X);
            }
            sm.xp[kq][rt][lane] = X;
        }
        lds_barrier();  // ---- A: partials visible

        if (fin_d) {
            // ---- phase 2: Delta = U - X for row tile rt (natural order, k-scaled in ds)
            const f32x4 ks4 = __builtin_bit_cast(
                f32x4, buf_load16(rcur, (uint32_t)(rt * 16 + 4 * g16) * 4, (uint32_t)R::KSC_BYTE_OFF));
            f32x4 X = sm.xp[0][rt][lane];
#pragma unroll
            for (int qq = 1; qq < P::KQ; ++qq) X += sm.xp[qq][rt][lane];
            const f32x4 d = __builtin_bit_cast(f32x4, frag(u_src(rt))) - X;
            *reinterpret_cast<f32x4*>(sm.ds + l16 * DP + rt * 16 + 4 * g16) = d * ks4;
            *reinterpret_cast<f32x4*>(delta_out(c) + (size_t)l16 * C + rt * 16 + 4 * g16) = d;  // Delta^T rows
        }
        const float decay = __builtin_bit_cast(f32x4, buf_load16(rcur, 0, (uint32_t)R::DEC_BYTE_OFF)).x;
        lds_barrier();  // ---- B: Delta visible

        // ---- phase 3: state update on this wave's d_k tiles
#pragma unroll
        for (int a = 0; a < P::MTW; ++a) {
            const int mt = wave + NW * a;
            if (mt >= R::MT) continue;
            f32x4 acc = S[a] * decay;
#pragma unroll
            for (int ks = 0; ks < R::CKS; ++ks) {
                const int doff = l16 * DP + ks * KS + g16 * E;
                acc = M::mma(frag(k_src(mt, ks)), *reinterpret_cast<const Frag*>(sm.ds + doff), acc);
            }
            S[a] = acc;
            *reinterpret_cast<f32x4*>(sm.sr + l16 * SP + mt * 16 + 4 * g16) = acc;
        }
        lds_barrier();  // ---- C: state copy visible
    }

    if (state_out_ptr) {
#pragma unroll
        for (int a = 0; a < P::MTW; ++a) {
            const int mt = wave + NW * a;
            if (mt < R::MT)
                *reinterpret_cast<f32x4*>(state_out_ptr + st_base + (size_t)(row0 + l16) * DK + mt * 16 + 4 * g16) =
                    S[a];
        }
    }
}

// ---------------------------------------------------------------- bf16 state chain
// LDS transposing read of gfx950 (ds_read_b64_tr_b16): within each group of 16
// lanes, lane j supplies the address of four consecutive 16-bit values, and
// lane i receives value i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4.  When lane j points at row r0 + j / 4, columns c0 + 4 (j % 4)
// .. + 3 of a row-major tile, lane i therefore receives column c0 + i of the
// rows r0 .. r0 + 3: four consecutive elements down one column.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p)
{
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16* lds_v4i16_t;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)p));
}

// LDS of the bf16 chain kernel.  The per-chunk operands are triple-buffered:
// chunk c's sit in buffer c % 3, written by LDS-DMA two chunks ahead.
template <int DK, int DV>
struct ChainKrLds {
    using R = Rec<uint16_t, 64, DK, DV>;
    static constexpr int C = 64, RT = 4, NB = 3;
    static constexpr int SP = DK + 8;              // state copy pitch (dwords = 4 mod 32)
    static constexpr int DP = C + 8;               // Delta^T pitch
    static constexpr int KB = C * DK * 2;          // bytes of the K tile
    static constexpr int NKP = KB / 1024;          // 1 KB transfers of the K tile
    static constexpr int NTP = RT * R::CKS;        // T' fragments
    static constexpr int NDMA = NKP + NTP + RT + 1;  // transfers per chunk: K, T', U tiles, row vectors
    unsigned char kt[NB][KB];                      // K tile, KTile<DK> layout
    unsigned char tp[NB][NTP][1024];               // T' fragments [row tile][k-step], lane order
    unsigned char uf[NB][RT][1024];                // U tiles of this workgroup's 16 value columns
    unsigned char vec[NB][1024];                   // k scales (bytes 0..255), decay and token range (256..271)
    uint16_t sr[16 * SP];                          // state rows S[r][col] rounded to bf16, sigma order
    u32x2 yb[2][2][2][64];                         // Y = K S^T, B operand of T' Y: [k-step][hi, lo][half][lane]
    uint16_t dt[2][16 * DP];                       // Delta^T[r][j], sigma order (hi, lo)
    uint16_t ds[2][16 * DP];                       // (kscale o Delta)^T[r][j], natural order (hi, lo)
};

// State chain, bf16 operands: one workgroup of 16 waves per (sequence, head,
// 16 state rows), sequential over the sequence's chunks.  With the chunk's raw
// K rows in LDS, the corrected values come as Delta = U - T' (K S^T) and the
// state update as S^T = e^{gamma_L} S^T + K^T (kscale o Delta): K is read as
// row fragments for K S^T and, through the transposing read, as column
// fragments for K^T, so each chunk's K crosses from L2 once.  Per chunk c the
// 8 compute waves run
//   phase 1  waves 0..3, row tile w: Y = K S^T (fp32), split hi/lo into LDS
//   phase 2  waves 0..3, row tile w: X = T' (Y_hi + Y_lo), Delta = U - X
//            (sigma-ordered Delta^T and the k-scaled natural-order copy, hi/lo)
//   phase 3  waves 0..7, their state d_k tiles: the state update
// separated by the barriers A, B and C, every operand read from LDS (no global
// memory instruction inside the loop), each phase's reads issued together.
// Loader waves 0..5 (waves 8..13) move chunk c+2's K tile, T', U tiles and row
// vectors into buffer (c+2) % 3 during chunk c (transfer i by loader i mod 6,
// in three bursts, one per phase; the buffer was released by barrier C of
// chunk c-1) and wait before barrier C for chunk c+1's transfers, issued a
// chunk earlier.  Loaders 6 and 7 copy the state rows entering chunk c to
// `states` (before barrier A) and Delta of chunk c to `deltas` (after B); they
// issue no transfer into LDS, so no read of theirs waits for one.  The
// workgroup -> (pair, row tile) mapping and the segment logic are those of
// chain_kernel.  PIPE: the one launch of the pipelined prefill, whose loaders
// and store waves also take the hand-offs of PipeSync.
// At most 120 VGPRs per lane: the 16 waves of a workgroup take 4 x 120 of a
// SIMD's 512, so a chain workgroup still fits on a CU where a one-wave
// hand-off kernel (pipe_wait_kernel, 5 VGPRs) runs.  That wave waits for the
// chain, so a chain workgroup that could not start beside it would never let
// it finish.
template <int DK, int DV, bool SEG, bool PIPE>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(120))) void chain_kr_kernel(
    const int32_t* __restrict__ header, const int32_t* __restrict__ seq_first,
    const int32_t* __restrict__ seq_order, int32_t varlen, int64_t T, int32_t H, int32_t pairs,
    const unsigned char* records, size_t record_bytes, const float* init_state, float* final_state,
    uint16_t* __restrict__ states, uint16_t* __restrict__ deltas, int64_t seg_begin, int64_t seg_end, float* carry,
    int64_t slot0, PipeSync ps)
{
    using M = Mma<uint16_t>;
    using R = Rec<uint16_t, 64, DK, DV>;
    using CO = ChainOut<uint16_t, 64, DK, DV>;
    using L = ChainKrLds<DK, DV>;
    using KT = KTile<DK>;
    typedef M::Frag Frag;
    constexpr int C = 64, RT = 4, KS = 32, E = 8, NW = 8;
    constexpr int SP = L::SP, DP = L::DP, NKP = L::NKP, NTP = L::NTP, NDMA = L::NDMA;
    constexpr int DKS = R::DKS, CKS = R::CKS, MT = R::MT;
    constexpr int MTW = (MT + NW - 1) / NW;      // state d_k tiles per compute wave
    constexpr int TILES = DV / 16;
    constexpr uint32_t FB = 64 * 16;             // bytes of one fragment
    constexpr int ND = 6;                        // transfer loaders
    static_assert(16 - NW - ND == (int)kPipePublishers, "the other loader waves store");
    constexpr int NJ = (NDMA + ND - 1) / ND;     // transfers of the busiest loader
    constexpr int J1 = (NJ + 2) / 3, J2 = (2 * NJ + 2) / 3;  // burst bounds (phase 1 | 2 | 3)
    static_assert(KS == M::KS && E == M::E && CKS == 2 && RT == R::RT, "chunk 64");
    static_assert(sizeof(L) <= 160 * 1024, "chain LDS");

    extern __shared__ __align__(16) unsigned char lds_raw[];
    L& sm = *reinterpret_cast<L*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar branches
    const int g16 = lane >> 4, l16 = lane & 15;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int pair = xcd + 8 * (slot / TILES);
    if (pair >= pairs) return;
    const int n = varlen ? seq_order[pair / H] : pair / H, h = pair % H;  // longest sequences first
    const int tile = slot % TILES;
    const int row0 = tile * 16;  // first state row (value index) of this workgroup

    // this workgroup is done with every segment: nothing of it waits for it
    auto pipe_release_all = [&]() {
        if constexpr (PIPE)
            if (threadIdx.x == 0)
            for (int q = 0; q < ps.nseg; ++q)
                __hip_atomic_fetch_add(ps.flags + kPipeMaxSeg + q, kPipePublishers, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
    };
    int64_t s_first, s_last;  // the sequence's chunk range
    if (varlen) {
        if (header[0] != 0) {
            pipe_release_all();
            return;
        }
        s_first = seq_first[n];
        s_last = seq_first[n + 1];
    } else {
        s_first = 0;
        s_last = (T + C - 1) / C;
    }
    const int64_t c_begin = SEG && s_first < seg_begin ? seg_begin : s_first;
    const int64_t c_end = SEG && s_last > seg_end ? seg_end : s_last;
    if (c_begin >= c_end && !(s_first == s_last && s_first >= seg_begin && s_first < seg_end)) {
        pipe_release_all();
        return;
    }
    const float* state_in = c_begin == s_first ? init_state : carry;
    float* state_out_ptr = c_end == s_last ? final_state : carry;
    const int64_t last = c_end - 1;

    const uint32_t lane_b = (uint32_t)lane * 16;
    auto rec_ptr = [&](int64_t c) { return records + ((size_t)(c - slot0) * H + h) * record_bytes; };
    auto state_out = [&](int64_t c) {
        return states + ((size_t)(c - slot0) * H + h) * CO::STATE_ELEMS + (size_t)row0 * DK;
    };
    auto delta_out = [&](int64_t c, int part) {
        return deltas + ((size_t)(c - slot0) * H + h) * CO::DELTA_ELEMS + ((size_t)part * DV + row0) * C;
    };

    // ------------------------------------------------------------ loader waves
    if (wave >= NW) {
        const int lw = wave - NW;
        if (lw < ND) {
            // transfers j0 .. j1-1 of this loader for chunk cc (transfer i = lw + ND j)
            int64_t ready_below = 0;  // (PIPE) chunks below this are known to be prepared
            int seg = 0;
            auto transfers = [&](int64_t cc, int j0, int j1) {
                if constexpr (PIPE)
                    while (cc >= ready_below) {  // the first chunk of a later segment
                        while (seg + 1 < ps.nseg && ps.end[seg] <= cc) ++seg;
                        pipe_wait(ps.flags + seg, 1u, ps.flags + 2 * kPipeMaxSeg);
                        ready_below = seg + 1 < ps.nseg ? ps.end[seg] : INT64_MAX;
                    }
                const unsigned char* rb = rec_ptr(cc);
                const __amdgpu_buffer_rsrc_t r = make_rsrc(rb, (uint32_t)R::BYTES);
                const __amdgpu_buffer_rsrc_t rv = make_rsrc(rb + R::KSC_BYTE_OFF, C * 4 + 16);  // lanes past: zeros
                const int b = (int)(cc % 3);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int i = lw + ND * j;
                    if (j < j0 || j >= j1 || i >= NDMA) continue;
                    if (i < NKP) {
                        const uint32_t src = (uint32_t)(R::KR_OFF * 2) + (uint32_t)i * FB;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(sm.kt[b] + i * FB), 16, lane_b, src, 0, 0);
                    } else if (i < NKP + NTP) {
                        const uint32_t src = (uint32_t)(R::TP_OFF * 2) + (uint32_t)(i - NKP) * FB;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)sm.tp[b][i - NKP], 16, lane_b, src, 0, 0);
                    } else if (i < NKP + NTP + RT) {
                        const int u = i - NKP - NTP;
                        const uint32_t src = (uint32_t)R::U_BYTE_OFF + (uint32_t)(u * R::VT + tile) * FB;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)sm.uf[b][u], 16, lane_b, src, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)sm.vec[b], 16, lane_b, 0, 0, 0);
                    }
                }
            };
            const bool busiest = lw + ND * (NJ - 1) < NDMA;  // issues NJ transfers per chunk, else NJ - 1
            if (c_begin < c_end) transfers(c_begin, 0, NJ);
            if (c_begin + 1 < c_end) transfers(c_begin + 1, 0, NJ);
            wait_vmcnt<0>();
            __syncthreads();  // the first chunk's operands and the initial state rows are in LDS
            for (int64_t c = c_begin; c < c_end; ++c) {
                const bool more = c + 2 <= last;
                if (more) transfers(c + 2, 0, J1);
                lds_barrier();  // ---- A
                if (more) transfers(c + 2, J1, J2);
                lds_barrier();  // ---- B
                if (more) {
                    transfers(c + 2, J2, NJ);
                    // chunk c+1's transfers (a chunk older than this chunk's) have landed
                    if (busiest)
                        wait_vmcnt<NJ>();
                    else
                        wait_vmcnt<NJ - 1>();
                } else {
                    wait_vmcnt<0>();
                }
                lds_barrier();  // ---- C
            }
            wait_vmcnt<0>();
            return;
        }
        // store loaders 6 and 7: LDS rows -> global rows, 16 bytes per lane
        const int sl = lw - ND;                      // 0 or 1
        constexpr int SROW = DK * 2 / 16;            // 16-byte units per state row
        constexpr int SU = (16 * SROW + 127) / 128;  // units per lane
        auto store_state = [&](int64_t c) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(state_out(c), 16u * DK * 2);
#pragma unroll
            for (int i = 0; i < SU; ++i) {
                int u = (sl * 64 + lane) + 128 * i;
                u = u < 16 * SROW ? u : 16 * SROW;  // past the rows: offset past the view, dropped
                const int row = min(u / SROW, 15), part = u % SROW;
                const u32x4 v = *reinterpret_cast<const u32x4*>(sm.sr + row * SP + part * 8);
                __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)((uint32_t)u * 16), 0, kNtAux);
            }
        };
        constexpr int DROW = C * 2 / 16;  // 16-byte units per Delta row (8)
        static_assert(16 * DROW == 128, "one Delta row-part unit per lane and part");
        auto store_delta = [&](int64_t c) {
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const int u = sl * 64 + lane, row = u / DROW, q = u % DROW;
                const u32x4 v = *reinterpret_cast<const u32x4*>(sm.dt[part] + row * DP + q * 8);
                const __amdgpu_buffer_rsrc_t r = make_rsrc(delta_out(c, part), 16u * C * 2);
                __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)((uint32_t)row * C * 2 + q * 16), 0, kNtAux);
            }
        };
        // segments whose states and Delta this store wave has written its part
        // of: release the stores at agent scope, then count the wave in
        // (the segment index and the next segment end stay wave-uniform, so the
        // loop keeps its addresses and descriptors in scalar registers)
        int sig = 0;
        int64_t next_end = PIPE && ps.nseg > 0 ? ps.end[0] : INT64_MAX;
        auto publish = [&](int64_t done_below) {
            int n = sig;
            while (n < ps.nseg && ps.end[n] <= done_below) ++n;
            n = __builtin_amdgcn_readfirstlane(n);
            if (n == sig) return;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            if (lane == 0)
                for (int q = sig; q < n; ++q)
                    __hip_atomic_fetch_add(ps.flags + kPipeMaxSeg + q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sig = n;
            next_end = n < ps.nseg ? ps.end[n] : INT64_MAX;
        };
        if constexpr (PIPE) publish(c_begin);
        __syncthreads();
        for (int64_t c = c_begin; c < c_end; ++c) {
            store_state(c);  // before phase 3 rewrites the rows
            lds_barrier();  // ---- A
            lds_barrier();  // ---- B
            store_delta(c);  // before phase 2 of c+1 rewrites it
            if constexpr (PIPE)
                if (c + 1 >= next_end) publish(c + 1);
            lds_barrier();  // ---- C
        }
        wait_vmcnt<0>();
        if constexpr (PIPE) publish(INT64_MAX);
        return;
    }

    // ------------------------------------------------------------ compute waves
    // K^T fragment of d_k tile mt, k-step ks (identity order over the chunk):
    // lane (l16, g16) element e = K[32 ks + 8 g16 + e][16 mt + l16], two transposing reads
    auto kt_frag = [&](const uint16_t* kc, int mt, int ks) -> Frag {
        const int r = ks * KS + 8 * g16 + (l16 >> 2);
        const u32x2 a = lds_read_tr16(kc + KT::at(r, mt >> 1, l16 & 3, mt & 1));
        const u32x2 b = lds_read_tr16(kc + KT::at(r + 4, mt >> 1, l16 & 3, mt & 1));
        return __builtin_bit_cast(Frag, u32x4{a.x, a.y, b.x, b.y});
    };
    auto frag_at = [&](const unsigned char* p) -> Frag { return *reinterpret_cast<const Frag*>(p + lane_b); };

    // state tiles S^T[mt] in result layout: lane holds S[row0 + l16][mt*16 + 4*g16 + i]
    f32x4 S[MTW];
    const size_t st_base = ((size_t)n * H + h) * DV * DK;
#pragma unroll
    for (int a = 0; a < MTW; ++a) {
        const int mt = wave + NW * a;
        S[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mt < MT) {
            if (state_in)
                S[a] = *reinterpret_cast<const f32x4*>(state_in + st_base + (size_t)(row0 + l16) * DK + mt * 16 +
                                                       4 * g16);
            store_quad<uint16_t, false>(sm.sr + l16 * SP + quad_pos<uint16_t>(mt, g16), nullptr, S[a]);
        }
    }
    __syncthreads();

    for (int64_t c = c_begin; c < c_end; ++c) {
        const int b = (int)(c % 3);
        const uint16_t* kc = reinterpret_cast<const uint16_t*>(sm.kt[b]);
        if (wave < RT) {
            // ---- phase 1: Y = K S^T for chunk rows 16 wave .. +15, split hi/lo
            Frag kf[DKS], sf[DKS];
#pragma unroll
            for (int ks = 0; ks < DKS; ++ks) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(kc + KT::at(wave * 16 + l16, ks, g16, 0));
                const u32x2 hi = *reinterpret_cast<const u32x2*>(kc + KT::at(wave * 16 + l16, ks, g16, 1));
                kf[ks] = __builtin_bit_cast(Frag, u32x4{lo.x, lo.y, hi.x, hi.y});
                sf[ks] = *reinterpret_cast<const Frag*>(sm.sr + l16 * SP + ks * KS + g16 * E);
            }
            f32x4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DKS; ks += 2) {
                y0 = M::mma(kf[ks], sf[ks], y0);
                if (ks + 1 < DKS) y1 = M::mma(kf[ks + 1], sf[ks + 1], y1);
            }
            const f32x4 y = y0 + y1;
            // lane holds Y[16 wave + 4 g16 + i][row l16]: elements 4 (wave % 2) + i of the
            // sigma-ordered B operand of k-step wave / 2
            uint32_t h0, l0, h1, l1;
            split_bf16x2(y.x, y.y, h0, l0);
            split_bf16x2(y.z, y.w, h1, l1);
            sm.yb[wave >> 1][0][wave & 1][lane] = u32x2{h0, h1};
            sm.yb[wave >> 1][1][wave & 1][lane] = u32x2{l0, l1};
        }
        lds_barrier();  // ---- A: Y visible

        if (wave < RT) {
            // ---- phase 2: Delta = U - T' Y of row tile `wave` (T' is zero above the diagonal)
            const int nks = wave / 2 + 1;
            Frag tf[CKS], yh[CKS], yl[CKS];
#pragma unroll
            for (int ks = 0; ks < CKS; ++ks) {
                if (ks >= nks) break;
                tf[ks] = frag_at(sm.tp[b][wave * CKS + ks]);
                const u32x2 h0 = sm.yb[ks][0][0][lane], h1 = sm.yb[ks][0][1][lane];
                const u32x2 l0 = sm.yb[ks][1][0][lane], l1 = sm.yb[ks][1][1][lane];
                yh[ks] = __builtin_bit_cast(Frag, u32x4{h0.x, h0.y, h1.x, h1.y});
                yl[ks] = __builtin_bit_cast(Frag, u32x4{l0.x, l0.y, l1.x, l1.y});
            }
            const f32x4 ks4 = *reinterpret_cast<const f32x4*>(sm.vec[b] + wave * 64 + 16 * g16);
            const f32x4 u4 = *reinterpret_cast<const f32x4*>(sm.uf[b][wave] + lane_b);
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < CKS; ++ks) {
                if (ks >= nks) break;
                x = M::mma(tf[ks], yh[ks], x);
                x = M::mma(tf[ks], yl[ks], x);
            }
            const f32x4 d = u4 - x;
            const int pd = l16 * DP + quad_pos<uint16_t>(wave, g16);
            const int pn = l16 * DP + wave * 16 + 4 * g16;
            store_quad<uint16_t, true>(sm.dt[0] + pd, sm.dt[1] + pd, d);
            store_quad<uint16_t, true>(sm.ds[0] + pn, sm.ds[1] + pn, d * ks4);
        }
        lds_barrier();  // ---- B: Delta visible

        // ---- phase 3: state update on this wave's d_k tiles
        {
            const float decay = *reinterpret_cast<const float*>(sm.vec[b] + C * 4);
            Frag kf[MTW][CKS], dh[CKS], dl[CKS];
#pragma unroll
            for (int ks = 0; ks < CKS; ++ks) {
                const int doff = l16 * DP + ks * KS + g16 * E;
                dh[ks] = *reinterpret_cast<const Frag*>(sm.ds[0] + doff);
                dl[ks] = *reinterpret_cast<const Frag*>(sm.ds[1] + doff);
#pragma unroll
                for (int a = 0; a < MTW; ++a) {
                    const int mt = wave + NW * a;
                    if (mt < MT) kf[a][ks] = kt_frag(kc, mt, ks);
                }
            }
#pragma unroll
            for (int a = 0; a < MTW; ++a) {
                const int mt = wave + NW * a;
                if (mt >= MT) continue;
                f32x4 acc0 = S[a] * decay, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < CKS; ++ks) {
                    acc0 = M::mma(kf[a][ks], dh[ks], acc0);
                    acc1 = M::mma(kf[a][ks], dl[ks], acc1);
                }
                S[a] = acc0 + acc1;
                store_quad<uint16_t, false>(sm.sr + l16 * SP + quad_pos<uint16_t>(mt, g16), nullptr, S[a]);
            }
        }
        lds_barrier();  // ---- C: state copy visible; buffer c % 3 free
    }

    if (state_out_ptr) {
#pragma unroll
        for (int a = 0; a < MTW; ++a) {
            const int mt = wave + NW * a;
            if (mt < MT)
                *reinterpret_cast<f32x4*>(state_out_ptr + st_base + (size_t)(row0 + l16) * DK + mt * 16 + 4 * g16) =
                    S[a];
        }
    }
}

// Output kernel: one workgroup of 4 waves per (chunk, head), all chunks in
// parallel.  O = scale (qscale o (Q S_c^T) + P Delta_c) for the chunk's rows,
// with S_c the state entering the chunk and Delta_c its corrected values, both
// from the state chain; wave w computes value tiles w, w + 4, ... in groups of
// up to VG tiles.  The output rows are staged in LDS and written 16 bytes per
// lane; rows >= len fall outside the buffer view.
template <typename TIn, int C, int DK, int DV>
struct OutCfg {
    static constexpr int VT = DV / 16;
    static constexpr int VTW = (VT + 3) / 4;               // value tiles per wave
    static constexpr int VG = VTW < 4 ? VTW : 4;           // tiles per accumulation group
    static constexpr int OP = DV + 16 / (int)sizeof(TIn);  // LDS output row pitch (elements)
    static constexpr int OPF = DV + 4;                     // fp32 row pitch with the gated epilogue
    static constexpr size_t lds_bytes(bool gated)
    {
        return gated ? (size_t)C * OPF * 4 : (size_t)C * OP * sizeof(TIn);
    }
};

// With GATED, the epilogue of App. A.3 Eq. 20 follows the read: every output
// row (one token and head, d_v values) is staged in fp32, normalised by its
// root mean square, scaled by the per-channel weight and gated by silu(z).
template <typename TIn, int C, int DK, int DV, bool GATED>
__device__ __forceinline__ void output_chunk(const int32_t* __restrict__ header,
                                                     const ChunkInfo* __restrict__ tab, int32_t varlen, int64_t T,
                                                     int32_t H, const unsigned char* __restrict__ records,
                                                     size_t record_bytes, const TIn* __restrict__ states,
                                                     const TIn* __restrict__ deltas, TIn* __restrict__ o, float scale,
                                                     const TIn* __restrict__ gz, const float* __restrict__ gw,
                                                     float geps, int64_t c, int64_t slot)
{
    using M = Mma<TIn>;
    using R = Rec<TIn, C, DK, DV>;
    using CO = ChainOut<TIn, C, DK, DV>;
    using G = OutCfg<TIn, C, DK, DV>;
    typedef typename M::Frag Frag;
    constexpr int KS = M::KS, E = M::E, RT = R::RT, NS = CO::NS;
    constexpr uint32_t FB = 64 * 16, EB = sizeof(TIn);
    static_assert(G::VTW % G::VG == 0, "value tile groups");

    extern __shared__ __align__(16) unsigned char out_lds[];
    TIn* ot = reinterpret_cast<TIn*>(out_lds);     // [C][OP]   (plain read-out)
    float* otf = reinterpret_cast<float*>(out_lds);  // [C][OPF]  (gated epilogue)

    const int h = blockIdx.y;
    if (varlen && c >= header[1]) return;
    if (!varlen && c * C >= T) return;
    const ChunkInfo ci = chunk_info(tab, varlen, c, C, T);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g16 = lane >> 4, l16 = lane & 15;
    const uint32_t lane_b = (uint32_t)lane * 16;

    const unsigned char* recb = records + ((size_t)slot * H + h) * record_bytes;
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(recb, (uint32_t)R::BYTES);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(states + ((size_t)slot * H + h) * CO::STATE_ELEMS, (uint32_t)(CO::STATE_ELEMS * EB));
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(deltas + ((size_t)slot * H + h) * CO::DELTA_ELEMS, (uint32_t)(CO::DELTA_ELEMS * EB));

    f32x4 qs[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        qs[rt] = __builtin_bit_cast(f32x4, buf_load16(rr, (uint32_t)(rt * 16 + 4 * g16) * 4, (uint32_t)R::QS_BYTE_OFF));

#pragma unroll 1
    for (int grp = 0; grp < G::VTW / G::VG; ++grp) {
        f32x4 acc[RT][G::VG];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < G::VG; ++v) acc[rt][v] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Q S^T over d_k
#pragma unroll 2
        for (int ks = 0; ks < R::DKS; ++ks) {
            Frag fq[RT], fs[G::VG];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                fq[rt] = __builtin_bit_cast(Frag, buf_load16(rr, lane_b, R::Q_OFF * EB + (uint32_t)(rt * R::DKS + ks) * FB));
#pragma unroll
            for (int v = 0; v < G::VG; ++v) {
                const int vt = min(wave + 4 * (grp * G::VG + v), G::VT - 1);  // waves past the last tile recompute it
                fs[v] = __builtin_bit_cast(
                    Frag, buf_load16(rs, (uint32_t)((vt * 16 + l16) * DK + ks * KS + g16 * E) * EB, 0));
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int v = 0; v < G::VG; ++v) acc[rt][v] = M::mma(fq[rt], fs[v], acc[rt][v]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < G::VG; ++v) acc[rt][v] *= qs[rt];
        // + P Delta over the chunk (P is lower triangular: k-steps up to the diagonal)
#pragma unroll
        for (int ks = 0; ks < R::CKS; ++ks) {
            Frag dh[G::VG], dl[G::VG];
#pragma unroll
            for (int v = 0; v < G::VG; ++v) {
                const int vt = min(wave + 4 * (grp * G::VG + v), G::VT - 1);
                const uint32_t off = (uint32_t)((vt * 16 + l16) * C + ks * KS + g16 * E) * EB;
                dh[v] = __builtin_bit_cast(Frag, buf_load16(rd, off, 0));
                if constexpr (NS > 1) dl[v] = __builtin_bit_cast(Frag, buf_load16(rd, off, (uint32_t)(DV * C) * EB));
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (ks * KS > rt * 16 + 15) continue;
                const uint32_t po = (uint32_t)(rt * R::CKS + ks) * FB;
                const Frag ph = __builtin_bit_cast(Frag, buf_load16(rr, lane_b, R::PH_OFF * EB + po));
                Frag pl;
                if constexpr (NS > 1) pl = __builtin_bit_cast(Frag, buf_load16(rr, lane_b, R::PL_OFF * EB + po));
#pragma unroll
                for (int v = 0; v < G::VG; ++v) {
                    acc[rt][v] = M::mma(ph, dh[v], acc[rt][v]);
                    if constexpr (NS > 1) {
                        acc[rt][v] = M::mma(pl, dh[v], acc[rt][v]);
                        acc[rt][v] = M::mma(ph, dl[v], acc[rt][v]);
                    }
                }
            }
        }
        // result layout: lane holds rows rt*16 + 4*g16 + i of column vt*16 + l16
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < G::VG; ++v) {
                const int vt = wave + 4 * (grp * G::VG + v);
                if (vt >= G::VT) continue;  // (only when fewer than 4 value tiles)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (GATED)
                        otf[(rt * 16 + 4 * g16 + i) * G::OPF + vt * 16 + l16] = scale * acc[rt][v][i];
                    else
                        ot[(rt * 16 + 4 * g16 + i) * G::OP + vt * 16 + l16] = M::cvt(scale * acc[rt][v][i]);
                }
            }
    }
    __syncthreads();
    if constexpr (GATED) {
        // 8 values of a row per thread; the DV/8 threads of a row are adjacent lanes
        constexpr int G8 = DV / 8;
        static_assert(G8 >= 2 && G8 <= 64 && (G8 & (G8 - 1)) == 0, "a row's threads are aligned lanes of one wave");
        for (int u = tid; u < C * G8; u += 256) {
            const int row = u / G8, q8 = u % G8;
            const float* src = otf + row * G::OPF + q8 * 8;
            const f32x4 a = *reinterpret_cast<const f32x4*>(src);
            const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
            float ss = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
            ss = group_sum<G8>(ss);
            const float r = 1.0f / sqrtf(ss / (float)DV + geps);
            if (row < ci.len) {
                const int64_t base = ((int64_t)(ci.tok0 + row) * H + h) * DV + q8 * 8;
                float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                float zv[8];
                const f32x4 z0 = Elem<TIn>::load4(gz, base), z1 = Elem<TIn>::load4(gz, base + 4);
                zv[0] = z0.x; zv[1] = z0.y; zv[2] = z0.z; zv[3] = z0.w;
                zv[4] = z1.x; zv[5] = z1.y; zv[6] = z1.z; zv[7] = z1.w;
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float wv = gw ? gw[q8 * 8 + e] : 1.0f;
                    y[e] = x[e] * r * wv * fast_silu(zv[e]);
                }
                Quad<TIn>::store(o + base, f32x4{y[0], y[1], y[2], y[3]});
                Quad<TIn>::store(o + base + 4, f32x4{y[4], y[5], y[6], y[7]});
            }
        }
        return;
    }
    // rows of the output tile -> o, 16 bytes per lane
    constexpr int UROW = DV * (int)EB / 16;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(o + ((int64_t)ci.tok0 * H + h) * DV, (uint32_t)(((ci.len - 1) * H + 1) * DV * EB));
    for (int u = tid; u < C * UROW; u += 256) {
        const int row = u / UROW, q = u % UROW;
        const u32x4 val = *reinterpret_cast<const u32x4*>(ot + row * G::OP + q * (16 / EB));
        __builtin_amdgcn_raw_buffer_store_b128(val, ro, (int)((uint32_t)row * H * DV * EB + q * 16), 0, kNtAux);
    }
}

template <typename TIn, int C, int DK, int DV, bool GATED>
__global__ __launch_bounds__(256) void output_kernel(const int32_t* __restrict__ header,
                                                     const ChunkInfo* __restrict__ tab, int32_t varlen, int64_t T,
                                                     int32_t H, const unsigned char* __restrict__ records,
                                                     size_t record_bytes, const TIn* __restrict__ states,
                                                     const TIn* __restrict__ deltas, TIn* __restrict__ o, float scale,
                                                     const TIn* __restrict__ gz, const float* __restrict__ gw,
                                                     float geps, int64_t c_base, int64_t c_end, int64_t slot0)
{
    const int64_t c = c_base + blockIdx.x;
    if (c >= c_end) return;
    output_chunk<TIn, C, DK, DV, GATED>(header, tab, varlen, T, H, records, record_bytes, states, deltas, o, scale,
                                        gz, gw, geps, c, c - slot0);
}

// ------------------------------------------------------------------ dispatch

}  // namespace gdn

// Streams and events of the pipelined prefill, owned by the caller through
// gdn_context_create / gdn_context_destroy (default priority; the CU-masked
// streams synchronise with the legacy default stream, the unmasked fallback
// streams do not).  The state chain gets a stream of its own, CU-masked to the
// same number of CUs on every XCD (CU mask bit i is CU i / 8 of XCD i % 8: the
// masks number the CUs round-robin over the XCDs), and the per-segment
// intra-chunk and output kernels two more streams, masked to every CU: so each
// stream owns a hardware queue, and the side kernels also use the reserved
// CUs that hold no chain workgroup (at six (sequence, head) pairs, those of
// two XCDs) and every CU before the chain's launch and after its end.  The one
// chain launch of the pipeline holds its CUs from start to end, and nothing
// on the side streams waits while holding a CU except one-wave hand-off
// kernels, beside which a chain workgroup still fits (its VGPR cap).
struct gdn_context {
    static constexpr int MAX_SEG = 16;
    std::mutex use;  // held while one call enqueues its pipeline: the events are reused by every call
    int dev = -1;
    int32_t chain_cus = 0;  // CUs of each XCD reserved for the chain
    bool masked = false;    // the streams are CU-masked, so each has a hardware queue of its own
    hipStream_t chain_s = nullptr, intra_s = nullptr, out_s = nullptr;
    hipEvent_t start = nullptr, intra_end = nullptr, out_end = nullptr;
    hipEvent_t intra_done[MAX_SEG] = {}, chain_done[MAX_SEG] = {};
};

namespace gdn {

// Releases whatever part of the context exists (streams are waited for first).
static hipError_t context_release(gdn_context* r)
{
    hipError_t first = hipSuccess;
    auto keep = [&](hipError_t e) {
        if (first == hipSuccess && e != hipSuccess) first = e;
    };
    for (hipStream_t s : {r->chain_s, r->intra_s, r->out_s})
        if (s) keep(hipStreamSynchronize(s));
    hipEvent_t* evs[] = {&r->start, &r->intra_end, &r->out_end};
    for (hipEvent_t* ev : evs)
        if (*ev) keep(hipEventDestroy(*ev));
    for (int i = 0; i < gdn_context::MAX_SEG; ++i) {
        if (r->intra_done[i]) keep(hipEventDestroy(r->intra_done[i]));
        if (r->chain_done[i]) keep(hipEventDestroy(r->chain_done[i]));
    }
    for (hipStream_t s : {r->chain_s, r->intra_s, r->out_s})
        if (s) keep(hipStreamDestroy(s));
    delete r;
    return first;
}

hipError_t context_create(int32_t chain_cus_per_xcd, gdn_context** out)
{
    *out = nullptr;
    const int32_t per_xcd = chain_cus_per_xcd > 0 ? chain_cus_per_xcd : kDefaultChainCus;
    if (per_xcd > 31) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    gdn_context* r = new (std::nothrow) gdn_context;
    if (!r) return hipErrorOutOfMemory;
    r->dev = dev;
    r->chain_cus = per_xcd;
    auto fail = [&](hipError_t err) {
        (void)context_release(r);  // frees what was created before the failure
        return err;
    };
    if (cus == 256) {
        uint32_t mine[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const uint32_t all[8] = {~0u, ~0u, ~0u, ~0u, ~0u, ~0u, ~0u, ~0u};
        for (int x = 0; x < 8; ++x)
            for (int c = 0; c < per_xcd; ++c) {
                const int bit = x + 8 * c;
                mine[bit >> 5] |= 1u << (bit & 31);
            }
        if ((e = hipExtStreamCreateWithCUMask(&r->chain_s, 8, mine)) != hipSuccess) return fail(e);
        if ((e = hipExtStreamCreateWithCUMask(&r->intra_s, 8, all)) != hipSuccess) return fail(e);
        if ((e = hipExtStreamCreateWithCUMask(&r->out_s, 8, all)) != hipSuccess) return fail(e);
        r->masked = true;
    } else {
        if ((e = hipStreamCreateWithFlags(&r->chain_s, hipStreamNonBlocking)) != hipSuccess) return fail(e);
        if ((e = hipStreamCreateWithFlags(&r->intra_s, hipStreamNonBlocking)) != hipSuccess) return fail(e);
        if ((e = hipStreamCreateWithFlags(&r->out_s, hipStreamNonBlocking)) != hipSuccess) return fail(e);
    }
    hipEvent_t* evs[] = {&r->start, &r->intra_end, &r->out_end};
    for (hipEvent_t* ev : evs)
        if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return fail(e);
    for (int i = 0; i < gdn_context::MAX_SEG; ++i) {
        if ((e = hipEventCreateWithFlags(&r->intra_done[i], hipEventDisableTiming)) != hipSuccess) return fail(e);
        if ((e = hipEventCreateWithFlags(&r->chain_done[i], hipEventDisableTiming)) != hipSuccess) return fail(e);
    }
    *out = r;
    return hipSuccess;
}

hipError_t context_destroy(gdn_context* ctx) { return context_release(ctx); }

}  // namespace gdn

// Workspace of the no-allocation prefill (gdn_chunk_prefill_noalloc): every GPU
// the library runs on holds one copy of this array from the first use of the
// library's code on that device until the process ends.  In host code the name
// stands for a host-side shadow, not a device address: only the address that
// hipGetSymbolAddress returns for the current device may be handed to kernels.
static __device__ __align__(256) unsigned char scratch[gdn::kScratchBytes];

namespace gdn {

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_device_ptr(void** out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

int context_device(const gdn_context* ctx) { return ctx->dev; }

// Raises a kernel's dynamic-LDS limit to what this launch uses.  Set on every
// launch that needs more than the default 64 KB (a host-side attribute of the
// kernel on the current device, idempotent, not a stream operation, so it is
// also legal while the stream is being captured); nothing is cached.
static hipError_t lds_limit(const void* fn, size_t bytes)
{
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename TIn, int C, int DK, int DV>
static hipError_t run_prefill(const PrefillArgs& a)
{
    using R = Rec<TIn, C, DK, DV>;
    if (R::BYTES > a.lay.record_bytes) return hipErrorInvalidValue;
    int32_t* header = reinterpret_cast<int32_t*>(a.ws + a.lay.off_header);
    ChunkInfo* tab = reinterpret_cast<ChunkInfo*>(a.ws + a.lay.off_chunk_tab);
    int32_t* first = reinterpret_cast<int32_t*>(a.ws + a.lay.off_seq_first);
    int32_t* order = reinterpret_cast<int32_t*>(a.ws + a.lay.off_seq_order);
    unsigned char* records = a.ws + a.lay.off_records;
    TIn* states = reinterpret_cast<TIn*>(a.ws + a.lay.off_states);
    TIn* deltas = reinterpret_cast<TIn*>(a.ws + a.lay.off_deltas);
    float* carry = reinterpret_cast<float*>(a.ws + a.lay.off_carry);
    const int varlen = a.cu_seqlens != nullptr;
    const int64_t grid_chunks = varlen ? a.lay.max_chunks : (a.T + C - 1) / C;
    const int64_t pairs = (int64_t)a.N * a.H;
    const int64_t chain_blocks = (pairs + 7) / 8 * 8 * (DV / 16);
    if (pairs > 0x7fffffff || chain_blocks > 0x7fffffff || grid_chunks > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int64_t ALL = INT64_MAX;

    // slot0: the chunk whose per-chunk data sits at slot 0 of the records,
    // states and deltas (0 unless the workspace holds a window of the chunks)
    auto launch_intra = [&](int64_t c0, int64_t c1, hipStream_t st, int64_t slot0 = 0) -> hipError_t {
        if (c1 <= c0) return hipSuccess;
        size_t smem = sizeof(IntraSmem<TIn, C, DK, DV>);
        if constexpr (sizeof(TIn) == 2 && C == 64) smem = sizeof(IntraBfSmem<DK, DV>);
        const dim3 grid((uint32_t)(c1 - c0), a.H);
        if constexpr (sizeof(TIn) == 2 && C == 64) {
            if (a.fused) {
                const hipError_t e = lds_limit((const void*)intra_kernel<TIn, C, DK, DV, true>, smem);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL((intra_kernel<TIn, C, DK, DV, true>), grid, dim3(256), smem, st, (const TIn*)nullptr,
                                   (const TIn*)nullptr, (const TIn*)nullptr, (const float*)nullptr,
                                   (const float*)nullptr, header, tab, varlen, a.T, a.H, a.l2norm, records,
                                   a.lay.record_bytes, c0, c1, slot0, a.fe);
                return hipGetLastError();
            }
        }
        if (a.fused) return hipErrorInvalidValue;
        const hipError_t e = lds_limit((const void*)intra_kernel<TIn, C, DK, DV, false>, smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((intra_kernel<TIn, C, DK, DV, false>), grid, dim3(256), smem, st, (const TIn*)a.q,
                           (const TIn*)a.k, (const TIn*)a.v, a.g, a.beta, header, tab, varlen, a.T, a.H, a.l2norm,
                           records, a.lay.record_bytes, c0, c1, slot0, FrontIn{});
        return hipGetLastError();
    };
    auto launch_chain = [&](int64_t c0, int64_t c1, hipStream_t st, int64_t slot0 = 0,
                            PipeSync pipe = PipeSync{}) -> hipError_t {
        const bool seg = !(c0 == 0 && c1 == ALL);
        if constexpr (sizeof(TIn) == 2) {
            using Lds = ChainKrLds<DK, DV>;
            const bool pipe_on = pipe.flags != nullptr;
            const void* fn = seg ? (const void*)chain_kr_kernel<DK, DV, true, false>
                                 : pipe_on ? (const void*)chain_kr_kernel<DK, DV, false, true>
                                           : (const void*)chain_kr_kernel<DK, DV, false, false>;
            const hipError_t e = lds_limit(fn, sizeof(Lds));
            if (e != hipSuccess) return e;
            const dim3 grid((uint32_t)chain_blocks), block(1024);
            if (seg)
                hipLaunchKernelGGL((chain_kr_kernel<DK, DV, true, false>), grid, block, sizeof(Lds), st, header, first,
                                   order, varlen, a.T, a.H, (int32_t)pairs, records, a.lay.record_bytes, a.init_state,
                                   a.final_state, states, deltas, c0, c1, carry, slot0, pipe);
            else if (pipe_on)
                hipLaunchKernelGGL((chain_kr_kernel<DK, DV, false, true>), grid, block, sizeof(Lds), st, header, first,
                                   order, varlen, a.T, a.H, (int32_t)pairs, records, a.lay.record_bytes, a.init_state,
                                   a.final_state, states, deltas, c0, c1, carry, slot0, pipe);
            else
                hipLaunchKernelGGL((chain_kr_kernel<DK, DV, false, false>), grid, block, sizeof(Lds), st, header, first,
                                   order, varlen, a.T, a.H, (int32_t)pairs, records, a.lay.record_bytes, a.init_state,
                                   a.final_state, states, deltas, c0, c1, carry, slot0, pipe);
            return hipGetLastError();
        } else {
            constexpr int NW = 8;
            using Lds = ChainLds<C, DK, DV, NW>;
            static_assert(sizeof(Lds) <= 160 * 1024, "chain kernel LDS");
            const void* fn = seg ? (const void*)chain_kernel<C, DK, DV, NW, true>
                                 : (const void*)chain_kernel<C, DK, DV, NW, false>;
            const hipError_t e = lds_limit(fn, sizeof(Lds));
            if (e != hipSuccess) return e;
            const dim3 grid((uint32_t)chain_blocks), block(NW * 64);
            if (seg)
                hipLaunchKernelGGL((chain_kernel<C, DK, DV, NW, true>), grid, block, sizeof(Lds), st, header, first,
                                   order, varlen, a.T, a.H, (int32_t)pairs, records, a.lay.record_bytes, a.init_state,
                                   a.final_state, states, deltas, c0, c1, carry, slot0);
            else
                hipLaunchKernelGGL((chain_kernel<C, DK, DV, NW, false>), grid, block, sizeof(Lds), st, header, first,
                                   order, varlen, a.T, a.H, (int32_t)pairs, records, a.lay.record_bytes, a.init_state,
                                   a.final_state, states, deltas, c0, c1, carry, slot0);
            return hipGetLastError();
        }
    };
    auto launch_output = [&](int64_t c0, int64_t c1, hipStream_t st, int64_t slot0 = 0) -> hipError_t {
        if (c1 <= c0) return hipSuccess;
        const bool gated = a.norm.z != nullptr;
        const size_t smem = OutCfg<TIn, C, DK, DV>::lds_bytes(gated);
        const void* fn = gated ? (const void*)output_kernel<TIn, C, DK, DV, true>
                               : (const void*)output_kernel<TIn, C, DK, DV, false>;
        const hipError_t e = lds_limit(fn, smem);
        if (e != hipSuccess) return e;
        const dim3 grid((uint32_t)(c1 - c0), a.H);
        if (gated)
            hipLaunchKernelGGL((output_kernel<TIn, C, DK, DV, true>), grid, dim3(256), smem, st, header, tab, varlen,
                               a.T, a.H, records, a.lay.record_bytes, states, deltas, (TIn*)a.o, a.scale,
                               (const TIn*)a.norm.z, a.norm.w, a.norm.eps, c0, c1, slot0);
        else
            hipLaunchKernelGGL((output_kernel<TIn, C, DK, DV, false>), grid, dim3(256), smem, st, header, tab, varlen,
                               a.T, a.H, records, a.lay.record_bytes, states, deltas, (TIn*)a.o, a.scale,
                               (const TIn*)nullptr, (const float*)nullptr, 0.f, c0, c1, slot0);
        return hipGetLastError();
    };
#define GDN_TRY(x)                       \
    do {                                 \
        hipError_t e_ = (x);             \
        if (e_ != hipSuccess) return e_; \
    } while (0)

    if ((a.stages & 1) && varlen) {
        hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, a.N, a.T, (int32_t)C,
                           a.lay.max_chunks, header, tab, first, order);
        GDN_TRY(hipGetLastError());
    }

    // The state chain keeps only (sequences x heads x d_v/16) workgroups busy.
    // With an execution context whose chain reservation holds them (the
    // pairs p with p % 8 == x, TILES each, on XCD x), when every stage runs in
    // this call, the chunks are cut into segments and pipelined: the chain of
    // segment s runs on the context's CU-masked chain stream while the
    // intra-chunk kernel prepares later segments and the output kernel
    // finishes earlier ones on the other CUs; events order each segment's
    // three kernels.  The kernels and their arguments are the same either way,
    // so the results are too.
    // The hand-offs between the pipeline streams cost about 0.14 ms per call
    // (measured: 8K tokens 0.38 ms pipelined against 0.24 ms stage by stage),
    // which the overlap repays only past about 36K tokens of one sequence
    // (32K: 1.07 against 1.04 ms; 40K: 1.26 against 1.30 ms).
    // A workspace that holds a window of a.window chunks (the no-allocation
    // entry point): the chunks are processed stage by stage, one window at a
    // time, on the caller's stream; each window's chain launch carries the
    // states of the sequences that continue past it through `carry`, exactly as
    // the pipeline's segments do.  The last window is open-ended so that empty
    // sequences after the last chunk still copy their initial state.
    if (a.window > 0) {
        if (a.stages != 7) return hipErrorInvalidValue;
        for (int64_t c0 = 0; c0 == 0 || c0 < grid_chunks; c0 += a.window) {
            const int64_t c1 = std::min(c0 + a.window, grid_chunks);
            GDN_TRY(launch_intra(c0, c1, a.stream, c0));
            GDN_TRY(launch_chain(c0, c1 >= grid_chunks ? ALL : c1, a.stream, c0));
            GDN_TRY(launch_output(c0, c1, a.stream, c0));
        }
        return hipSuccess;
    }

    constexpr int64_t PIPE_MIN_CHUNKS = 576, GEOM_MIN_CHUNKS = 768;
    const int64_t chain_per_xcd = ((pairs + 7) / 8) * (DV / 16);
    gdn_context* pr = a.ctx;
    int nseg = 1;
    // Under stream capture the call runs stage by stage: a graph's executor may
    // run the pipeline's branches in sequence, so the device-memory hand-offs
    // are out, and the event-ordered schedule measured no faster than stage by
    // stage when replayed (1.92 against 1.92 ms at 64K tokens).
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    GDN_TRY(hipStreamIsCapturing(a.stream, &capture));
    if (pr && a.stages == 7 && chain_per_xcd <= pr->chain_cus && grid_chunks >= PIPE_MIN_CHUNKS &&
        capture == hipStreamCaptureStatusNone)
        nseg = (grid_chunks >= GEOM_MIN_CHUNKS && !a.norm.z) ? 6 : 4;
    if (nseg == 1) {
        if (a.stages & 1) GDN_TRY(launch_intra(0, grid_chunks, a.stream));
        if (a.stages & 2) GDN_TRY(launch_chain(0, ALL, a.stream));
        if (a.stages & 4) GDN_TRY(launch_output(0, grid_chunks, a.stream));
        return hipSuccess;
    }
    // One call at a time records and waits on the context's events.
    std::lock_guard<std::mutex> pipe_lock(pr->use);
    // Segment sizes.  From 768 chunks on, six segments in the ratio
    // 1 : 2 : 4 : 4 : 2 : 1: the first preparation and the last outputs, which
    // run alone, are short, and the middle segments overlap the most (1.84 ms
    // against 1.875 ms for four equal segments at 64K tokens; equal at 48K,
    // 3 % slower at 40K, where four equal segments are kept).  The gated
    // read-out keeps four equal segments: its heavier output kernel cannot
    // finish a large middle segment under the next, shorter chain segment
    // (2.01 against 1.93 ms at 64K).
    static constexpr int kGeom[6] = {1, 2, 4, 4, 2, 1};
    int64_t bounds[gdn_context::MAX_SEG + 1];
    {
        const int sum = nseg == 6 ? 14 : nseg;
        int acc = 0;
        bounds[0] = 0;
        for (int i = 0; i < nseg; ++i) {
            acc += nseg == 6 ? kGeom[i] : 1;
            bounds[i + 1] = grid_chunks * acc / sum;
        }
    }
    auto seg_lo = [&](int s) { return bounds[std::min(s, nseg)]; };
    // bf16 on CU-masked streams, outside stream capture: the chain runs as one
    // launch over every chunk and the hand-offs go through device memory
    // (PipeSync), so the chain never stops between segments.  The intra-chunk
    // kernel prepares every segment, in order, on one side stream and raises
    // each segment's flag; the output kernel finishes every segment, in order,
    // on the other, each behind a wait for the chain's store waves.
    // A wait in device memory needs its producer to run beside it: masked
    // streams each own a hardware queue, while streams that share a queue may
    // run the two in sequence.  Unmasked contexts (and the fp32 chain) keep the
    // event-ordered schedule below.
    if (sizeof(TIn) == 2 && pr->masked) {
        PipeSync ps{};
        ps.flags = reinterpret_cast<uint32_t*>(header) + 16;
        ps.nseg = nseg;
        for (int s = 0; s < nseg; ++s) ps.end[s] = s + 1 < nseg ? seg_lo(s + 1) : ALL;
        const uint32_t chain_wgs = (uint32_t)(pairs * (DV / 16)) * kPipePublishers;
        // The caller's stream only forks the three streams and joins them at the
        // end: when it is the legacy default stream, every command on it waits
        // for all work enqueued before on the (blocking) masked streams, and
        // theirs for all enqueued before on it.  The chain stream zeroes the
        // hand-off words and starts the chain, whose loaders then wait for the
        // intra-chunk stream's signals; that stream prepares segment 0 and
        // waits for the zeroing before its first signal.
        GDN_TRY(hipEventRecord(pr->start, a.stream));
        GDN_TRY(hipStreamWaitEvent(pr->chain_s, pr->start, 0));
        GDN_TRY(hipStreamWaitEvent(pr->intra_s, pr->start, 0));
        hipLaunchKernelGGL(pipe_reset_kernel, dim3(1), dim3(64), 0, pr->chain_s, ps.flags);
        GDN_TRY(hipGetLastError());
        GDN_TRY(hipEventRecord(pr->intra_done[0], pr->chain_s));  // the hand-off words are zero
        GDN_TRY(launch_chain(0, ALL, pr->chain_s, 0, ps));
        GDN_TRY(hipEventRecord(pr->chain_done[0], pr->chain_s));
        for (int s = 0; s < nseg; ++s) {
            GDN_TRY(launch_intra(seg_lo(s), seg_lo(s + 1), pr->intra_s));
            if (s == 0) GDN_TRY(hipStreamWaitEvent(pr->intra_s, pr->intra_done[0], 0));
            hipLaunchKernelGGL(pipe_signal_kernel, dim3(1), dim3(64), 0, pr->intra_s, ps.flags, s);
            GDN_TRY(hipGetLastError());
        }
        GDN_TRY(hipEventRecord(pr->intra_end, pr->intra_s));
        GDN_TRY(hipStreamWaitEvent(pr->out_s, pr->intra_done[0], 0));
        for (int s = 0; s < nseg; ++s) {
            hipLaunchKernelGGL(pipe_wait_kernel, dim3(1), dim3(64), 0, pr->out_s, ps.flags, s, chain_wgs);
            GDN_TRY(hipGetLastError());
            GDN_TRY(launch_output(seg_lo(s), seg_lo(s + 1), pr->out_s));
        }
        GDN_TRY(hipEventRecord(pr->out_end, pr->out_s));
        GDN_TRY(hipStreamWaitEvent(a.stream, pr->intra_end, 0));
        GDN_TRY(hipStreamWaitEvent(a.stream, pr->chain_done[0], 0));
        GDN_TRY(hipStreamWaitEvent(a.stream, pr->out_end, 0));
        return hipSuccess;
    }
    // One chain launch per segment, ordered by events.  The first
    // segment's preparation and the last segment's outputs run on the caller's
    // stream over the whole GPU (nothing else runs then); everything in between
    // overlaps on the three pipeline streams.
    GDN_TRY(launch_intra(0, seg_lo(1), a.stream));
    GDN_TRY(hipEventRecord(pr->start, a.stream));
    GDN_TRY(hipStreamWaitEvent(pr->chain_s, pr->start, 0));
    GDN_TRY(hipStreamWaitEvent(pr->intra_s, pr->start, 0));
    GDN_TRY(hipStreamWaitEvent(pr->out_s, pr->start, 0));
    for (int s = 1; s < nseg; ++s) {  // later segments' preparation, in order, on its own stream
        GDN_TRY(launch_intra(seg_lo(s), seg_lo(s + 1), pr->intra_s));
        GDN_TRY(hipEventRecord(pr->intra_done[s], pr->intra_s));
    }
    for (int s = 0; s < nseg; ++s) {
        if (s > 0) GDN_TRY(hipStreamWaitEvent(pr->chain_s, pr->intra_done[s], 0));
        GDN_TRY(launch_chain(seg_lo(s), s + 1 < nseg ? seg_lo(s + 1) : ALL, pr->chain_s));
        GDN_TRY(hipEventRecord(pr->chain_done[s], pr->chain_s));
        if (s + 1 < nseg) {
            GDN_TRY(hipStreamWaitEvent(pr->out_s, pr->chain_done[s], 0));
            GDN_TRY(launch_output(seg_lo(s), seg_lo(s + 1), pr->out_s));
        }
    }
    // the caller's stream resumes after the pipeline streams, then finishes the last segment
    GDN_TRY(hipEventRecord(pr->intra_end, pr->intra_s));
    GDN_TRY(hipEventRecord(pr->out_end, pr->out_s));
    GDN_TRY(hipStreamWaitEvent(a.stream, pr->intra_end, 0));
    GDN_TRY(hipStreamWaitEvent(a.stream, pr->out_end, 0));
    GDN_TRY(hipStreamWaitEvent(a.stream, pr->chain_done[nseg - 1], 0));
    GDN_TRY(launch_output(seg_lo(nseg - 1), seg_lo(nseg), a.stream));
#undef GDN_TRY
    return hipSuccess;
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

static hipError_t launch_prefill_stages(const PrefillArgs& a);

// With the front end folded in, the conv state after the call (the last three
// inputs of every sequence) is written once every preparation kernel has read
// the state it was given (it may be overwritten in place): on `stream`, after
// the prefill's last kernel, which every schedule orders after all the others.
hipError_t launch_prefill(const PrefillArgs& a)
{
    const hipError_t e = launch_prefill_stages(a);
    if (e != hipSuccess || !a.fused || !a.conv_state_out) return e;
    FrontendArgs fa;
    memset(&fa, 0, sizeof fa);
    fa.xq = a.fe.xq; fa.xk = a.fe.xk; fa.xv = a.fe.xv;
    fa.state_in = a.fe.state_in;
    fa.state_out = a.conv_state_out;
    fa.cu = a.cu_seqlens;
    fa.N = a.N; fa.T = a.T; fa.H = a.H; fa.dk = a.dk; fa.dv = a.dv;
    fa.bf16 = a.bf16;
    fa.stream = a.stream;
    return launch_conv_state(fa);
}

static hipError_t launch_prefill_stages(const PrefillArgs& a)
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
