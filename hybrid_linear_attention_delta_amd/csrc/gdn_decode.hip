// gdn_decode.hip -- single-token recurrent decode of the gated delta rule (gfx950).
//
// Operation: "Long-Context Aware Upcycling: A New Frontier for Hybrid LLM
// Scaling" (arXiv:2604.24715), App. A.3, Eqs. 16-19, one token per sequence.
// For each (sequence n, head h) and each state row i (value index), with the
// state stored [N][H][d_v][d_k] fp32 (row i = one contiguous d_k vector):
//
//     a   = s_i . k^        retrieval from the old row        (Eq. 17, before decay)
//     b   = s_i . q^        read of the old row
//     c   = beta (v_i - alpha a)                               (Eqs. 16-17, scaled by beta)
//     s_i <- alpha s_i + c k^                                  (Eq. 18)
//     o_i = scale (alpha b + c (k^ . q^))  == scale (s_i_new . q^)   (Eq. 19)
//
// so every state byte is read once and written once, and both dot products
// come out of one pass over the row.
//
// Mapping: a row of d_k fp32 values is split over RL = d_k/16 lanes, each lane
// owning 16 columns as four 16-byte vectors strided by RL*4 columns, so every
// load instruction of a row group touches RL*16 contiguous bytes.  A wave holds
// 64/RL rows per pass (4 rows of 1 KiB at d_k = 256, one pass); q, k and v are
// loaded first, then all state rows, and only then are q and k widened and
// normalised, so that work overlaps the state loads.  Small waves and many of
// them measured faster than deeper per-wave queues (more workgroups in flight
// per CU).  The state is streamed with non-temporal loads and stores: it is
// touched once per step and is larger than the last-level cache in the
// workloads this serves.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK>
struct DecodeShape {
    static_assert(DK % 16 == 0 && DK >= 16 && DK <= 1024, "d_k");
    static constexpr int RL = DK / 16;                         // lanes per row
    static constexpr int ROWS_PER_PASS = kWave / RL;           // rows per wave per pass
    static constexpr int ITERS = ROWS_PER_PASS >= 4 ? 1 : 4 / ROWS_PER_PASS;
    static constexpr int ROWS_PER_WAVE = ROWS_PER_PASS * ITERS;
    static constexpr int WAVES = 4;
    static constexpr int ROWS_PER_BLOCK = ROWS_PER_WAVE * WAVES;
};

template <typename TIn, int DK>
__global__ __launch_bounds__(256) void decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                     const TIn* __restrict__ v, const float* __restrict__ g,
                                                     const float* __restrict__ beta, float* __restrict__ state,
                                                     TIn* __restrict__ o, int32_t H, int32_t dv,
                                                     int32_t blocks_per_head, float scale, int32_t l2norm)
{
    using S = DecodeShape<DK>;
    constexpr int RL = S::RL;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t nh = blockIdx.x / blocks_per_head;  // (n * H + h)
    const int rb = blockIdx.x % blocks_per_head;
    const int j = lane % RL;          // lane within its row group
    const int rsub = lane / RL;       // row group within the wave

    // q, k and v first (raw), then every state row of this wave, then the
    // widening and norm math: vmcnt retires in issue order, so that math waits
    // for q, k, v only while the state rows are in flight.
    const int64_t qk_base = nh * DK;
    typename Elem<TIn>::Raw4 kraw[4], qraw[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int col = 4 * (j + RL * m);  // columns owned by this lane: vector m covers col .. col+3
        kraw[m] = Elem<TIn>::raw4(k, qk_base + col);
        qraw[m] = Elem<TIn>::raw4(q, qk_base + col);
    }
    const int row0 = rb * S::ROWS_PER_BLOCK + wave * S::ROWS_PER_WAVE;
    TIn vraw[S::ITERS];
#pragma unroll
    for (int it = 0; it < S::ITERS; ++it)  // rows past d_v: loaded, not stored
        vraw[it] = v[nh * dv + min(row0 + it * S::ROWS_PER_PASS + rsub, dv - 1)];
    float* srow_base = state + nh * (int64_t)dv * DK;
    f32x4 s[S::ITERS][4];
#pragma unroll
    for (int it = 0; it < S::ITERS; ++it) {
        const int row = min(row0 + it * S::ROWS_PER_PASS + rsub, dv - 1);
        const f32x4* p = reinterpret_cast<const f32x4*>(srow_base + (int64_t)row * DK);
#pragma unroll
        for (int m = 0; m < 4; ++m) s[it][m] = __builtin_nontemporal_load(p + j + RL * m);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the widening below the state loads
    f32x4 kv[4], qv[4];
    float ss_k = 0.f, ss_q = 0.f, qk = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        kv[m] = Elem<TIn>::widen4(kraw[m]);
        qv[m] = Elem<TIn>::widen4(qraw[m]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ss_k += kv[m][e] * kv[m][e];
            ss_q += qv[m][e] * qv[m][e];
            qk += qv[m][e] * kv[m][e];
        }
    }
    ss_k = group_sum<RL>(ss_k);
    ss_q = group_sum<RL>(ss_q);
    qk = group_sum<RL>(qk);
    float rk = 1.f, rq = 1.f;
    if (l2norm) {
        rk = 1.0f / sqrtf(ss_k + kNormEps);
        rq = 1.0f / sqrtf(ss_q + kNormEps);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        kv[m] *= rk;
        qv[m] *= rq;
    }
    const float kq = qk * rk * rq;  // k^ . q^

    const float alpha = expf(g[nh]);
    const float b = beta[nh];

#pragma unroll
    for (int it = 0; it < S::ITERS; ++it) {
        const int row = row0 + it * S::ROWS_PER_PASS + rsub;
        float a = 0.f, bq = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a += s[it][m][e] * kv[m][e];
                bq += s[it][m][e] * qv[m][e];
            }
        a = group_sum<RL>(a);
        bq = group_sum<RL>(bq);
        const float vi = Elem<TIn>::load(vraw, it);
        const float c = b * (vi - alpha * a);
        if (row < dv) {
            f32x4* p = reinterpret_cast<f32x4*>(srow_base + (int64_t)row * DK);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 nv = alpha * s[it][m] + c * kv[m];
                __builtin_nontemporal_store(nv, p + j + RL * m);
            }
            if (j == 0) Elem<TIn>::store(o, nh * dv + row, scale * (alpha * bq + c * kq));
        }
    }
}

// Gated RMSNorm epilogue of a decode step ("Long-Context Aware Upcycling",
// App. A.3, Eq. 20): one wave per (sequence, head) output row of d_v values,
// normalised in place after the step has written it (the step's rows of one
// head are spread over several workgroups, so the mean square over d_v needs
// this second, tiny pass; it reads the row as stored, i.e. bf16-rounded for
// bf16 outputs).
template <typename TIn>
__global__ __launch_bounds__(256) void gated_norm_rows_kernel(TIn* __restrict__ o, const TIn* __restrict__ z,
                                                              const float* __restrict__ w, int64_t rows,
                                                              int32_t dv, float eps)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole waves
    const int lane = threadIdx.x & (kWave - 1);
    TIn* orow = o + row * dv;
    const TIn* zrow = z + row * dv;
    float ss = 0.f;
    for (int c = lane; c < dv; c += kWave) {
        const float x = Elem<TIn>::load(orow, c);
        ss += x * x;
    }
    ss = group_sum<kWave>(ss);
    const float r = 1.0f / sqrtf(ss / (float)dv + eps);
    for (int c = lane; c < dv; c += kWave) {
        const float x = Elem<TIn>::load(orow, c);
        const float zv = Elem<TIn>::load(zrow, c);
        const float wv = w ? w[c] : 1.0f;
        Elem<TIn>::store(orow, c, x * r * wv * fast_silu(zv));
    }
}

template <typename TIn, int DK>
static hipError_t launch_decode_t(const DecodeArgs& a)
{
    using S = DecodeShape<DK>;
    const int32_t bph = (a.dv + S::ROWS_PER_BLOCK - 1) / S::ROWS_PER_BLOCK;
    const int64_t blocks = (int64_t)a.N * a.H * bph;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<TIn, DK>), dim3((uint32_t)blocks), dim3(256), 0, a.stream,
                       (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.g, a.beta, a.state, (TIn*)a.o, a.H,
                       a.dv, bph, a.scale, a.l2norm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.norm.z) return e;
    const int64_t rows = (int64_t)a.N * a.H;
    hipLaunchKernelGGL((gated_norm_rows_kernel<TIn>), dim3((uint32_t)((rows + 3) / 4)), dim3(256), 0, a.stream,
                       (TIn*)a.o, (const TIn*)a.norm.z, a.norm.w, rows, a.dv, a.norm.eps);
    return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_decode_dt(const DecodeArgs& a)
{
    switch (a.dk) {
        case 16: return launch_decode_t<TIn, 16>(a);
        case 32: return launch_decode_t<TIn, 32>(a);
        case 64: return launch_decode_t<TIn, 64>(a);
        case 128: return launch_decode_t<TIn, 128>(a);
        case 256: return launch_decode_t<TIn, 256>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs& a)
{
    return a.bf16 ? launch_decode_dt<uint16_t>(a) : launch_decode_dt<float>(a);
}

}  // namespace gdn
