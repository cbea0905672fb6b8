// gdn_frontend.hip -- front end of the gated delta-rule mixer (gfx950): the short
// causal convolution with SiLU on the q, k, v projections and the gate math.
//
// "Long-Context Aware Upcycling: A New Frontier for Hybrid LLM Scaling"
// (arXiv:2604.24715), App. A.3:
//   * the paragraph under Table 8: each of Q, K, V goes through a 1-D
//     convolution of kernel size 4 with SiLU before the recurrence.  Read as
//     causal and depthwise with no bias:
//         y_t[c] = silu(sum_j w[c][j] x_{t-3+j}[c]),  tap 3 on the current token,
//     where the three inputs before a sequence come from its conv state
//     (zeros when none is given) and nothing crosses a sequence boundary;
//   * the paragraph after Eq. 21: g_t = -exp(A_log) softplus(W_alpha x_t + dt_bias)
//     and beta_t = sigmoid(W_beta x_t), one A_log and dt_bias per head.
//
// Channels of q, k and v form one concatenated axis of 2 H d_k + H d_v
// channels (q first, then k, then v); the taps and the conv state use it.
//
// The work is HBM streaming: each input element is read once from HBM and
// each output written once.  A thread owns one 16-byte vector of channels (8
// bf16 or 4 fp32) over a tile of kTile consecutive tokens and slides the
// 4-token window along them in registers, so the only re-reads are the three
// rows before each tile (served from L2: the neighbouring tile's thread reads
// them too).  A wave covers 64 consecutive vectors of one row, i.e. 1 KiB
// contiguous per load instruction for bf16.  All kTile row loads are issued
// before any arithmetic.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kTile = 16;  // tokens per thread (prefill)

// One 16-byte vector of stored elements and its widening / narrowing.
template <typename TIn> struct FVec;
template <> struct FVec<uint16_t> {
    static constexpr int N = 8;
    typedef u32x4 Raw;
    static __device__ __forceinline__ void widen(Raw r, float (&x)[8])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(r[i] << 16);
            x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ Raw narrow(const float (&y)[8])
    {
        Raw r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
        return r;
    }
};
template <> struct FVec<float> {
    static constexpr int N = 4;
    typedef f32x4 Raw;
    static __device__ __forceinline__ void widen(Raw r, float (&x)[4])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = r[i];
    }
    static __device__ __forceinline__ Raw narrow(const float (&y)[4])
    {
        return f32x4{y[0], y[1], y[2], y[3]};
    }
};

// Streaming (non-temporal) 16-byte accesses: every byte is touched once per
// call (measured 3 % faster than plain accesses on the 64K-token workload).
template <typename TIn>
__device__ __forceinline__ typename FVec<TIn>::Raw ld_vec(const TIn* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const typename FVec<TIn>::Raw*>(p));
}
template <typename TIn>
__device__ __forceinline__ void st_vec(TIn* p, typename FVec<TIn>::Raw r)
{
    __builtin_nontemporal_store(r, reinterpret_cast<typename FVec<TIn>::Raw*>(p));
}

// SiLU runs on the hardware exp2 and reciprocal (conv4_silu): the IEEE expf and
// divide made this streaming kernel ALU-bound (0.42 against 0.25 ms at 64K tokens).

__device__ __forceinline__ void gate_one(const float* __restrict__ a, const float* __restrict__ b,
                                         const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                                         float* __restrict__ g, float* __restrict__ beta, int64_t e, int h)
{
    g[e] = gate_g(a[e], A_log[h], dt_bias[h]);
    beta[e] = gate_beta(b[e]);
}

// Which of q, k, v a channel vector belongs to, and its offset inside that tensor.
template <typename TIn>
struct ChanSel {
    const TIn* x;
    TIn* y;
    int32_t col;  // first channel inside the tensor's row
    int32_t ld;   // row length of that tensor (H d_k or H d_v)
};
template <typename TIn>
__device__ __forceinline__ ChanSel<TIn> select_channel(int32_t c, int32_t cq, int32_t cv, const TIn* xq, const TIn* xk,
                                                       const TIn* xv, TIn* q, TIn* k, TIn* v)
{
    if (c < cq) return {xq, q, c, cq};
    if (c < 2 * cq) return {xk, k, c - cq, cq};
    return {xv, v, c - 2 * cq, cv};
}

// Prefill: 1-D grid over (token tile, block of 256 channel vectors), gx channel
// blocks per tile; block 256.  The first channel block of each tile also
// computes the gates of its tokens.
template <typename TIn>
__global__ __launch_bounds__(256) void conv_silu_kernel(const TIn* __restrict__ xq, const TIn* __restrict__ xk,
                                                        const TIn* __restrict__ xv, const float* __restrict__ w,
                                                        const TIn* __restrict__ st_in, const int32_t* __restrict__ cu,
                                                        int32_t N, int32_t T, int32_t cq, int32_t cv,
                                                        TIn* __restrict__ q, TIn* __restrict__ k, TIn* __restrict__ v,
                                                        const float* __restrict__ a, const float* __restrict__ b,
                                                        const float* __restrict__ A_log,
                                                        const float* __restrict__ dt_bias, float* __restrict__ g,
                                                        float* __restrict__ beta, int32_t H, int32_t gx,
                                                        int32_t per_xcd)
{
    using V = FVec<TIn>;
    constexpr int NV = V::N;
    const int32_t ctot = 2 * cq + cv;
    const int32_t groups = ctot / NV;
    // Workgroups are dealt round-robin over the 8 XCDs; give each XCD one
    // contiguous run of (tile, channel block) indices so that the three rows
    // before a tile were just read into the same XCD's L2 by the tile before.
    const int32_t logical = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
    const int32_t tile = logical / gx;
    const int32_t cb = logical % gx;
    const int32_t t0 = tile * kTile;
    if (t0 >= T) return;  // padding of the last XCD's run (whole block)
    const int32_t tend = min(t0 + kTile, T);

    if (cb == 0) {
        const int32_t cnt = (tend - t0) * H;
        for (int32_t i = threadIdx.x; i < cnt; i += blockDim.x) {
            const int64_t e = (int64_t)t0 * H + i;
            gate_one(a, b, A_log, dt_bias, g, beta, e, (int)(e % H));
        }
    }

    // sequence holding t0: the last n with cu[n] <= t0 (an empty sequence
    // starting at t0 is followed by the one that holds t0)
    __shared__ int32_t s_seq;
    if (threadIdx.x == 0) {
        int32_t n = 0;
        if (cu) {
            int32_t lo = 0, hi = N - 1;
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (cu[mid] <= t0) lo = mid;
                else hi = mid - 1;
            }
            n = lo;
        }
        s_seq = n;
    }
    __syncthreads();

    const int32_t gi = cb * (int32_t)blockDim.x + threadIdx.x;
    if (gi >= groups) return;
    const int32_t c = gi * NV;
    const ChanSel<TIn> sel = select_channel<TIn>(c, cq, cv, xq, xk, xv, q, k, v);

    // the tile's rows first (clamped inside [0, T): loads past tend are unused)
    typename V::Raw rows[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i) rows[i] = ld_vec(sel.x + (int64_t)min(t0 + i, T - 1) * sel.ld + sel.col);

    int32_t n = s_seq;
    int32_t nstart = cu ? cu[n] : 0;
    int32_t nend = cu ? cu[n + 1] : T;

    // the three inputs before t0 (oldest first): from x inside the sequence,
    // else from the sequence's conv state, else zero
    float h[3][NV];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int32_t p = t0 - 3 + m;
        typename V::Raw r = {};
        if (p >= nstart && p >= 0) {
            r = ld_vec(sel.x + (int64_t)p * sel.ld + sel.col);
        } else if (st_in) {
            const int32_t j = 3 - (nstart - p);
            if (j >= 0 && j < 3) r = ld_vec(st_in + ((int64_t)n * 3 + j) * ctot + c);
        }
        V::widen(r, h[m]);
    }

    float wt[NV][4];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(w + (int64_t)(c + e) * 4);
        wt[e][0] = t[0];
        wt[e][1] = t[1];
        wt[e][2] = t[2];
        wt[e][3] = t[3];
    }

#pragma unroll
    for (int i = 0; i < kTile; ++i) {
        const int32_t t = t0 + i;
        if (t >= tend) break;
        if (cu && t == nend && n + 1 < N) {  // a new sequence starts here: reset the window from its state
            ++n;
            while (n + 1 < N && cu[n + 1] <= t) ++n;
            nstart = t;
            nend = cu[n + 1];
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                typename V::Raw r = {};
                if (st_in) r = ld_vec(st_in + ((int64_t)n * 3 + m) * ctot + c);
                V::widen(r, h[m]);
            }
        }
        float x[NV], y[NV];
        V::widen(rows[i], x);
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            y[e] = conv4_silu(wt[e], h[0][e], h[1][e], h[2][e], x[e]);
            h[0][e] = h[1][e];
            h[1][e] = h[2][e];
            h[2][e] = x[e];
        }
        st_vec(sel.y + (int64_t)t * sel.ld + sel.col, V::narrow(y));
    }
}

// Conv state after a prefill: the last three inputs of every sequence (reaching
// into the given state for sequences shorter than three tokens).  One thread
// per (sequence, channel vector); it reads its three vectors before writing
// them, so the output may alias the input state.
template <typename TIn>
__global__ __launch_bounds__(256) void conv_state_kernel(const TIn* __restrict__ xq, const TIn* __restrict__ xk,
                                                         const TIn* __restrict__ xv, const TIn* st_in, TIn* st_out,
                                                         const int32_t* __restrict__ cu, int32_t N, int32_t T,
                                                         int32_t cq, int32_t cv)
{
    using V = FVec<TIn>;
    constexpr int NV = V::N;
    const int32_t ctot = 2 * cq + cv;
    const int32_t gi = (int32_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi >= ctot / NV) return;
    const int32_t c = gi * NV;
    const ChanSel<TIn> sel = select_channel<TIn>(c, cq, cv, xq, xk, xv, (TIn*)nullptr, (TIn*)nullptr, (TIn*)nullptr);
    for (int32_t n = blockIdx.y; n < N; n += gridDim.y) {
        const int32_t start = cu ? cu[n] : 0;
        const int32_t end = cu ? cu[n + 1] : T;
        typename V::Raw r[3];
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int32_t p = end - 3 + m;  // token index of slot m
            r[m] = typename V::Raw{};
            if (p >= start && p >= 0 && p < T) r[m] = ld_vec(sel.x + (int64_t)p * sel.ld + sel.col);
            else if (st_in) {
                const int32_t j = 3 - (start - p);
                if (j >= 0 && j < 3) r[m] = ld_vec(st_in + ((int64_t)n * 3 + j) * ctot + c);
            }
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) st_vec(st_out + ((int64_t)n * 3 + m) * ctot + c, r[m]);
    }
}

// Decode: one token per sequence, conv state [N][3][ctot] updated in place.
// grid (ceil(groups / 256), min(N, 65535)); blocks with blockIdx.x == 0 also
// compute the gates of their sequences.
template <typename TIn>
__global__ __launch_bounds__(256) void conv_decode_kernel(const TIn* __restrict__ xq, const TIn* __restrict__ xk,
                                                          const TIn* __restrict__ xv, const float* __restrict__ w,
                                                          TIn* __restrict__ st, int32_t N, int32_t cq, int32_t cv,
                                                          TIn* __restrict__ q, TIn* __restrict__ k,
                                                          TIn* __restrict__ v, const float* __restrict__ a,
                                                          const float* __restrict__ b,
                                                          const float* __restrict__ A_log,
                                                          const float* __restrict__ dt_bias, float* __restrict__ g,
                                                          float* __restrict__ beta, int32_t H)
{
    using V = FVec<TIn>;
    constexpr int NV = V::N;
    const int32_t ctot = 2 * cq + cv;
    const int32_t gi = (int32_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int32_t n = blockIdx.y; n < N; n += gridDim.y) {
        if (blockIdx.x == 0)
            for (int32_t h = threadIdx.x; h < H; h += blockDim.x)
                gate_one(a, b, A_log, dt_bias, g, beta, (int64_t)n * H + h, h);
        if (gi >= ctot / NV) continue;
        const int32_t c = gi * NV;
        const ChanSel<TIn> sel = select_channel<TIn>(c, cq, cv, xq, xk, xv, q, k, v);
        TIn* sp = st + (int64_t)n * 3 * ctot + c;
        const typename V::Raw r0 = ld_vec(sp), r1 = ld_vec(sp + ctot), r2 = ld_vec(sp + 2 * ctot);
        const typename V::Raw rx = ld_vec(sel.x + (int64_t)n * sel.ld + sel.col);
        float h0[NV], h1[NV], h2[NV], x[NV], y[NV];
        V::widen(r0, h0);
        V::widen(r1, h1);
        V::widen(r2, h2);
        V::widen(rx, x);
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(w + (int64_t)(c + e) * 4);
            const float wt[4] = {t[0], t[1], t[2], t[3]};
            y[e] = conv4_silu(wt, h0[e], h1[e], h2[e], x[e]);
        }
        st_vec(sel.y + (int64_t)n * sel.ld + sel.col, V::narrow(y));
        st_vec(sp, r1);
        st_vec(sp + ctot, r2);
        st_vec(sp + 2 * ctot, rx);
    }
}

template <typename TIn>
hipError_t launch_conv_state_t(const FrontendArgs& a);

template <typename TIn>
hipError_t launch_frontend_t(const FrontendArgs& a)
{
    constexpr int NV = FVec<TIn>::N;
    const int32_t cq = a.H * a.dk, cv = a.H * a.dv;
    const int32_t groups = (2 * cq + cv) / NV;
    const uint32_t gx = (uint32_t)((groups + 255) / 256);
    if (a.decode) {
        if (a.N == 0) return hipSuccess;
        const uint32_t gy = (uint32_t)min(a.N, 65535);
        hipLaunchKernelGGL((conv_decode_kernel<TIn>), dim3(gx, gy), dim3(256), 0, a.stream, (const TIn*)a.xq,
                           (const TIn*)a.xk, (const TIn*)a.xv, a.w, (TIn*)a.state_out, a.N, cq, cv, (TIn*)a.q,
                           (TIn*)a.k, (TIn*)a.v, a.a, a.b, a.A_log, a.dt_bias, a.g, a.beta, a.H);
        return hipGetLastError();
    }
    const int32_t T = (int32_t)a.T;
    if (T > 0) {
        const int64_t tiles = (T + kTile - 1) / kTile;
        const int64_t per_xcd = (tiles * gx + 7) / 8;
        if (per_xcd * 8 > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((conv_silu_kernel<TIn>), dim3((uint32_t)(per_xcd * 8)), dim3(256), 0, a.stream,
                           (const TIn*)a.xq, (const TIn*)a.xk, (const TIn*)a.xv, a.w, (const TIn*)a.state_in, a.cu,
                           a.N, T, cq, cv, (TIn*)a.q, (TIn*)a.k, (TIn*)a.v, a.a, a.b, a.A_log, a.dt_bias, a.g,
                           a.beta, a.H, (int32_t)gx, (int32_t)per_xcd);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_conv_state_t<TIn>(a);
}

template <typename TIn>
hipError_t launch_conv_state_t(const FrontendArgs& a)
{
    constexpr int NV = FVec<TIn>::N;
    const int32_t cq = a.H * a.dk, cv = a.H * a.dv;
    const int32_t groups = (2 * cq + cv) / NV;
    const uint32_t gx = (uint32_t)((groups + 255) / 256);
    const int32_t T = (int32_t)a.T;
    if (!a.state_out) return hipSuccess;
    const uint32_t gy = (uint32_t)min(a.N, 65535);
    hipLaunchKernelGGL((conv_state_kernel<TIn>), dim3(gx, gy), dim3(256), 0, a.stream, (const TIn*)a.xq,
                       (const TIn*)a.xk, (const TIn*)a.xv, (const TIn*)a.state_in, (TIn*)a.state_out, a.cu, a.N, T,
                       cq, cv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_frontend(const FrontendArgs& a)
{
    return a.bf16 ? launch_frontend_t<uint16_t>(a) : launch_frontend_t<float>(a);
}

hipError_t launch_conv_state(const FrontendArgs& a)
{
    return a.bf16 ? launch_conv_state_t<uint16_t>(a) : launch_conv_state_t<float>(a);
}

}  // namespace gdn
