// gdn_api.cpp -- C-ABI entry points: argument validation, workspace layout,
// dispatch onto the caller's stream (and a caller-owned context's streams).  No device
// allocation, no global state.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "../../include/gdn.h"
#include "gdn_launch.h"

static_assert(gdn::kScratchBytes == GDN_NOALLOC_SCRATCH_BYTES, "scratch size of the no-allocation prefill");

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool debug_sync()
{
    static const bool on = [] {  // read once; function-local static initialisation is thread-safe
        const char* s = getenv("GDN_DEBUG_SYNC");
        return s != nullptr && s[0] == '1';
    }();
    return on;
}

bool in_list(int32_t x, const int32_t* xs, int n)
{
    for (int i = 0; i < n; ++i)
        if (xs[i] == x) return true;
    return false;
}

gdn_status finish(hipError_t e, hipStream_t stream)
{
    if (e != hipSuccess) return GDN_ERR_LAUNCH;
    if (debug_sync()) {
        if (hipStreamSynchronize(stream) != hipSuccess) return GDN_ERR_LAUNCH;
        if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    }
    return GDN_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

namespace gdn {

bool prefill_supported(bool bf16, int32_t dk, int32_t dv, int32_t chunk)
{
    static const int32_t f32_d[] = {16, 32, 64, 128, 256};
    static const int32_t f32_c[] = {16, 32, 64};
    static const int32_t bf_dk[] = {64, 128, 256};
    static const int32_t bf_dv[] = {64, 128, 256, 512};
    if (bf16) return in_list(dk, bf_dk, 3) && in_list(dv, bf_dv, 4) && chunk == 64;
    return in_list(dk, f32_d, 5) && in_list(dv, f32_d, 5) && in_list(chunk, f32_c, 3);
}

PrefillLayout prefill_layout(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t C, bool bf16,
                             int64_t window_chunks)
{
    PrefillLayout L;
    memset(&L, 0, sizeof L);
    L.max_chunks = T / C + N;  // >= sum_n ceil(L_n / C)
    // chunks whose per-chunk data the workspace holds at once
    const int64_t held = window_chunks > 0 && window_chunks < L.max_chunks ? window_chunks : L.max_chunks;
    const size_t el = bf16 ? 2 : 4;
    // record, operand element type: fp32, W fragments (C x dk), raw K^T
    // fragments (dk x C), raw Q fragments (C x dk), P fragments (C x C); bf16,
    // the raw K rows (C x dk), T' = T diag(beta e^gamma r_k) (C x C), raw Q
    // fragments (C x dk), P fragments (C x C, hi and lo).  Then U tiles (C x dv),
    // two per-row scale vectors (C each) and the chunk decay with the chunk's
    // token range in fp32/int32.
    const size_t split = bf16 ? 2 : 1;
    const size_t oper = bf16 ? align_up(((size_t)C * dk * 2 + (size_t)C * C * 3) * el, 16)
                             : align_up(((size_t)C * dk * 3 + (size_t)C * C) * el, 16);
    L.record_bytes = align_up(oper + (size_t)C * dv * 4 + (size_t)C * 8 + 16, 256);
    size_t off = 0;
    L.off_header = off;
    off = align_up(off + 64, 256);
    L.off_chunk_tab = off;
    off = align_up(off + (size_t)L.max_chunks * 16, 256);
    L.off_seq_first = off;
    off = align_up(off + ((size_t)N + 1) * 4, 256);
    L.off_seq_order = off;
    off = align_up(off + (size_t)N * 4, 256);
    L.off_records = off;
    off = align_up(off + (size_t)held * H * L.record_bytes, 256);
    // outputs of the state chain for the output kernel
    L.off_states = off;
    off = align_up(off + (size_t)held * H * dv * dk * el, 256);
    L.off_deltas = off;
    off = align_up(off + (size_t)held * H * split * dv * C * el, 256);
    L.off_carry = off;
    off += (size_t)N * H * dv * dk * 4;
    L.total = off;
    return L;
}

// Workspace of the backward (fp32 per-chunk intermediates, chunk kBwdChunk).
bool backward_supported(int32_t dk, int32_t dv)
{
    return (dk == 64 || dk == 128 || dk == 256) && (dv == 64 || dv == 128 || dv == 256);
}

BwdLayout backward_layout(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv)
{
    BwdLayout L;
    memset(&L, 0, sizeof L);
    L.max_chunks = T / kBwdChunk + N;
    const size_t chs = (size_t)L.max_chunks * H;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = up(off + bytes);
        return o;
    };
    L.off_header = take(64);
    L.off_tab = take((size_t)L.max_chunks * 16);
    L.off_seq_first = take(((size_t)N + 1) * 4);
    const size_t cdk = chs * kBwdChunk * dk * 4, cdv = chs * kBwdChunk * dv * 4;
    const size_t cc = chs * kBwdChunk * kBwdChunk * 4, c1 = chs * kBwdChunk * 4;
    const size_t st = chs * (size_t)dv * dk * 4;
    L.off_Q = take(cdk);
    L.off_K = take(cdk);
    L.off_V = take(cdv);
    L.off_dO = take(cdv);
    L.off_rq = take(c1);
    L.off_rk = take(c1);
    L.off_gam = take(c1);
    L.off_bet = take(c1);
    L.off_T = take(cc);
    L.off_P = take(cc);
    L.off_KKG = take(cc);
    L.off_U = take(cdv);
    L.off_E = take(cdv);
    L.off_dDl = take(cdv);
    L.off_sck = take(c1);
    L.off_S = take(st);
    L.off_Dl = take(cdv);
    L.off_dS = take(st);
    L.off_dD = take(cdv);
    L.off_dQ = take(cdk);
    L.off_dK = take(cdk);
    L.off_dW = take(cdk);
    L.off_dPG = take(cc);
    L.off_dT = take(cc);
    L.off_X1 = take(cc);
    L.off_Bd = take(cc);
    L.off_Wf = take(cdk);
    L.off_Kf = take(cdk);
    L.off_Qf = take(cdk);
    L.off_Ef = take(cdv);
    L.off_Wr = take(cdk);
    L.off_Kr = take(cdk);
    L.total = off;
    return L;
}

}  // namespace gdn

extern "C" {

const char* gdn_status_string(gdn_status s)
{
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_ARG: return "GDN_ERR_NULL_ARG: a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE: invalid or inconsistent sizes";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: dtype/d_k/d_v/chunk combination not built";
        case GDN_ERR_BAD_SEQLENS: return "GDN_ERR_BAD_SEQLENS: cu_seqlens must rise from 0 to total_tokens";
        case GDN_ERR_ALIGNMENT: return "GDN_ERR_ALIGNMENT: tensor pointers must be 16-byte aligned";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: kernel launch or execution failed";
        case GDN_ERR_CONTEXT: return "GDN_ERR_CONTEXT: context creation failed or context of another device";
    }
    return "GDN_ERR_UNKNOWN";
}

int32_t gdn_version(void) { return 200; }

size_t gdn_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                                  int32_t chunk, gdn_dtype dt)
{
    if (total_tokens < 0 || num_seqs < 1 || H < 1) return 0;
    if (dt != GDN_F32 && dt != GDN_BF16) return 0;
    if (!gdn::prefill_supported(dt == GDN_BF16, dk, dv, chunk)) return 0;
    return gdn::prefill_layout(total_tokens, num_seqs, H, dk, dv, chunk, dt == GDN_BF16).total;
}

size_t gdn_prefill_workspace_min_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                                      int32_t chunk, gdn_dtype dt)
{
    if (total_tokens < 0 || num_seqs < 1 || H < 1) return 0;
    if (dt != GDN_F32 && dt != GDN_BF16) return 0;
    if (!gdn::prefill_supported(dt == GDN_BF16, dk, dv, chunk)) return 0;
    const size_t full = gdn::prefill_layout(total_tokens, num_seqs, H, dk, dv, chunk, dt == GDN_BF16).total;
    const size_t one = gdn::prefill_layout(total_tokens, num_seqs, H, dk, dv, chunk, dt == GDN_BF16, 1).total;
    return one < full ? one : full;
}

gdn_status gdn_context_create(int32_t chain_cus_per_xcd, gdn_context_t* ctx)
{
    if (!ctx) return GDN_ERR_NULL_ARG;
    *ctx = nullptr;
    if (chain_cus_per_xcd > 31) return GDN_ERR_BAD_SHAPE;
    return gdn::context_create(chain_cus_per_xcd, ctx) == hipSuccess ? GDN_OK : GDN_ERR_CONTEXT;
}

gdn_status gdn_context_destroy(gdn_context_t ctx)
{
    if (!ctx) return GDN_ERR_NULL_ARG;
    return gdn::context_destroy(ctx) == hipSuccess ? GDN_OK : GDN_ERR_CONTEXT;
}

}  // extern "C"

namespace {

// Checks of the gated-norm epilogue arguments (z has the layout and type of o).
gdn_status check_norm(const gdn::GatedNorm& nm, bool need_z)
{
    if (!nm.z) return need_z ? GDN_ERR_NULL_ARG : GDN_OK;
    if (!aligned16(nm.z)) return GDN_ERR_ALIGNMENT;
    if (nm.w && !aligned4(nm.w)) return GDN_ERR_ALIGNMENT;
    if (!(nm.eps >= 0.f) || !(nm.eps < INFINITY)) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

// Chunks per window of a workspace of `capacity` bytes: 0 when the whole
// layout fits, else the largest window (>= 1 chunk) whose layout fits, or -1
// when not even one chunk does.
int64_t fit_window(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t chunk, bool bf16, size_t capacity)
{
    const gdn::PrefillLayout full = gdn::prefill_layout(T, N, H, dk, dv, chunk, bf16);
    if (full.total <= capacity) return 0;
    if (gdn::prefill_layout(T, N, H, dk, dv, chunk, bf16, 1).total > capacity) return -1;
    int64_t lo = 1, hi = full.max_chunks;  // layout(lo) fits, layout(hi) does not
    while (hi - lo > 1) {
        const int64_t mid = lo + (hi - lo) / 2;
        (gdn::prefill_layout(T, N, H, dk, dv, chunk, bf16, mid).total <= capacity ? lo : hi) = mid;
    }
    return lo;
}

gdn_status prefill_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                        const float* init_state, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                        int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                        gdn_dtype dt, float scale, int32_t qk_l2norm, void* o, float* final_state, void* workspace,
                        size_t workspace_bytes, int32_t stages, const gdn::GatedNorm& norm, gdn_context* ctx,
                        hipStream_t stream, bool use_scratch = false, const gdn::FrontIn* fe = nullptr,
                        void* conv_state_out = nullptr)
{
    if (stages < 1 || stages > GDN_STAGE_ALL) return GDN_ERR_BAD_SHAPE;
    if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (total_tokens < 0 || num_seqs < 1 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return GDN_ERR_BAD_SHAPE;
    if (total_tokens > ((int64_t)1 << 31) - 1) return GDN_ERR_BAD_SHAPE;  // int32 token indices on device
    if (!cu_seqlens && num_seqs != 1) return GDN_ERR_BAD_SHAPE;
    if (!gdn::prefill_supported(dt == GDN_BF16, dk, dv, chunk)) return GDN_ERR_UNSUPPORTED;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL_ARG;
    if (!workspace && !use_scratch) return GDN_ERR_WORKSPACE;
    const bool bf16 = dt == GDN_BF16;
    const void* ptrs[] = {q, k, v, init_state, o, final_state};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGNMENT;
    if (((uintptr_t)workspace & 255u) != 0) return GDN_ERR_ALIGNMENT;
    if (cu_seqlens_host) {
        if (cu_seqlens_host[0] != 0 || cu_seqlens_host[num_seqs] != total_tokens) return GDN_ERR_BAD_SEQLENS;
        for (int32_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return GDN_ERR_BAD_SEQLENS;
    }
    // The workspace (the caller's, or the library's scratch array) holds every
    // chunk's intermediates when it is large enough; else, for a call that runs
    // every stage, the largest window of chunks that fits, processed window by
    // window with the state carried in between (bit-identical results).
    const size_t capacity = use_scratch ? gdn::kScratchBytes : workspace_bytes;
    const int64_t window = fit_window(total_tokens, num_seqs, H, dk, dv, chunk, bf16, capacity);
    if (window < 0 || (window > 0 && stages != GDN_STAGE_ALL)) return GDN_ERR_WORKSPACE;
    const gdn::PrefillLayout lay = gdn::prefill_layout(total_tokens, num_seqs, H, dk, dv, chunk, bf16, window);
    if (use_scratch) {
        if (gdn::scratch_device_ptr(&workspace) != hipSuccess || !workspace) return GDN_ERR_LAUNCH;
        workspace_bytes = gdn::kScratchBytes;
    }
    if (workspace_bytes < lay.total) return GDN_ERR_WORKSPACE;
    if (init_state && final_state && init_state != final_state) {
        // partial overlap would make the in-place carry order-dependent
        const char* a0 = (const char*)init_state;
        const char* b0 = (const char*)final_state;
        size_t bytes = (size_t)num_seqs * H * dv * dk * 4;
        if (a0 < b0 + bytes && b0 < a0 + bytes) return GDN_ERR_BAD_SHAPE;
    }
    if (ctx) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev != gdn::context_device(ctx)) return GDN_ERR_CONTEXT;
    }

    gdn::PrefillArgs a;
    a.fused = fe != nullptr;
    if (fe) {
        a.fe = *fe;
        a.fe.cu = cu_seqlens;
    }
    a.conv_state_out = conv_state_out;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.init_state = init_state;
    a.cu_seqlens = cu_seqlens;
    a.seq_order = nullptr;
    a.N = num_seqs; a.T = total_tokens; a.H = H; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.bf16 = bf16;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)dk);
    a.l2norm = qk_l2norm ? 1 : 0;
    a.o = o; a.final_state = final_state;
    a.ws = (unsigned char*)workspace;
    a.lay = lay;
    a.stages = stages;
    a.norm = norm;
    a.ctx = ctx;
    a.window = window;
    a.stream = stream;
    return finish(gdn::launch_prefill(a), stream);
}

gdn_status decode_impl(const void* q, const void* k, const void* v, const float* g, const float* beta, float* state,
                       int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, float scale, int32_t qk_l2norm,
                       void* o, const gdn::GatedNorm& norm, hipStream_t stream)
{
    static const int32_t ds[] = {16, 32, 64, 128, 256};
    static const int32_t dvs[] = {16, 32, 64, 128, 256, 512};
    if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (N < 0 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_BAD_SHAPE;
    if (!in_list(dk, ds, 5) || !in_list(dv, dvs, 6)) return GDN_ERR_UNSUPPORTED;
    if (N == 0) return GDN_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_NULL_ARG;
    const void* ptrs[] = {q, k, v, state, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGNMENT;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGNMENT;
    gdn::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.state = state; a.o = o;
    a.N = N; a.H = H; a.dk = dk; a.dv = dv;
    a.bf16 = dt == GDN_BF16;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)dk);
    a.l2norm = qk_l2norm ? 1 : 0;
    a.norm = norm;
    a.stream = stream;
    return finish(gdn::launch_decode(a), stream);
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_prefill_staged(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                    const float* init_state, const int32_t* cu_seqlens,
                                    const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens,
                                    int32_t H, int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                    int32_t qk_l2norm, void* o, float* final_state, void* workspace,
                                    size_t workspace_bytes, int32_t stages, hipStream_t stream)
{
    return prefill_impl(q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H, dk, dv,
                        chunk, dt, scale, qk_l2norm, o, final_state, workspace, workspace_bytes, stages,
                        gdn::GatedNorm{}, nullptr, stream);
}

gdn_status gdn_chunk_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* init_state, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                             int32_t chunk, gdn_dtype dt, float scale, int32_t qk_l2norm, void* o,
                             float* final_state, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return prefill_impl(q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H, dk, dv,
                        chunk, dt, scale, qk_l2norm, o, final_state, workspace, workspace_bytes, GDN_STAGE_ALL,
                        gdn::GatedNorm{}, nullptr, stream);
}

gdn_status gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                     const float* init_state, const int32_t* cu_seqlens,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens,
                                     int32_t H, int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                     int32_t qk_l2norm, void* o, float* final_state, hipStream_t stream)
{
    return prefill_impl(q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H, dk, dv,
                        chunk, dt, scale, qk_l2norm, o, final_state, nullptr, 0, GDN_STAGE_ALL, gdn::GatedNorm{},
                        nullptr, stream, true);
}

gdn_status gdn_chunk_prefill_frontend(gdn_context_t ctx, const void* xq, const void* xk, const void* xv,
                                      const float* conv_weight, const float* a, const float* b, const float* A_log,
                                      const float* dt_bias, const void* conv_state_in, const float* init_state,
                                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                      int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                                      gdn_dtype dt, float scale, int32_t qk_l2norm, void* o, float* final_state,
                                      void* conv_state_out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream)
{
    if (dt != GDN_BF16 && dt != GDN_F32) return GDN_ERR_UNSUPPORTED;
    if (dt != GDN_BF16 || chunk != 64) return GDN_ERR_UNSUPPORTED;  // the folded front end is built for bf16
    if (H < 1 || dk < 1 || dv < 1 || num_seqs < 1 || total_tokens < 0) return GDN_ERR_BAD_SHAPE;
    if (total_tokens > 0 && (!conv_weight || !A_log || !dt_bias)) return GDN_ERR_NULL_ARG;
    const void* p16[] = {conv_weight, conv_state_in, conv_state_out};
    for (const void* p : p16)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    const void* p4[] = {A_log, dt_bias};
    for (const void* p : p4)
        if (!aligned4(p)) return GDN_ERR_ALIGNMENT;
    if (conv_state_in && conv_state_out && conv_state_in != conv_state_out) {
        const size_t bytes = (size_t)num_seqs * 3 * (size_t)H * (2 * (size_t)dk + dv) * 2;
        const char* a0 = (const char*)conv_state_in;
        const char* b0 = (const char*)conv_state_out;
        if (a0 < b0 + bytes && b0 < a0 + bytes) return GDN_ERR_BAD_SHAPE;  // partial overlap
    }
    gdn::FrontIn fe;
    fe.xq = xq; fe.xk = xk; fe.xv = xv; fe.w = conv_weight;
    fe.a = a; fe.b = b; fe.A_log = A_log; fe.dt_bias = dt_bias;
    fe.state_in = conv_state_in;
    // the projections and gate inputs take the places of q, k, v, g and beta in
    // the shared checks (shapes, alignment, null pointers)
    return prefill_impl(xq, xk, xv, a, b, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H, dk, dv,
                        chunk, dt, scale, qk_l2norm, o, final_state, workspace, workspace_bytes, GDN_STAGE_ALL,
                        gdn::GatedNorm{}, ctx, stream, false, &fe, conv_state_out);
}

gdn_status gdn_chunk_prefill_ctx(gdn_context_t ctx, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* init_state, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens, int32_t H,
                                 int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                 int32_t qk_l2norm, void* o, float* final_state, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream)
{
    return prefill_impl(q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H, dk, dv,
                        chunk, dt, scale, qk_l2norm, o, final_state, workspace, workspace_bytes, GDN_STAGE_ALL,
                        gdn::GatedNorm{}, ctx, stream);
}

gdn_status gdn_chunk_prefill_gated_ctx(gdn_context_t ctx, const void* q, const void* k, const void* v,
                                       const float* g, const float* beta, const float* init_state,
                                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                                       gdn_dtype dt, float scale, int32_t qk_l2norm, const void* gate,
                                       const float* norm_weight, float norm_eps, void* o, float* final_state,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    gdn::GatedNorm nm;
    nm.z = gate;
    nm.w = norm_weight;
    nm.eps = norm_eps;
    const gdn_status st = check_norm(nm, total_tokens > 0);
    if (st != GDN_OK) return st;
    if (!nm.z) nm.z = o;  // no tokens: nothing is read
    return prefill_impl(q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H, dk, dv,
                        chunk, dt, scale, qk_l2norm, o, final_state, workspace, workspace_bytes, GDN_STAGE_ALL, nm,
                        ctx, stream);
}

gdn_status gdn_chunk_prefill_gated(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                   const float* init_state, const int32_t* cu_seqlens,
                                   const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens, int32_t H,
                                   int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                   int32_t qk_l2norm, const void* gate, const float* norm_weight, float norm_eps,
                                   void* o, float* final_state, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    return gdn_chunk_prefill_gated_ctx(nullptr, q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs,
                                       total_tokens, H, dk, dv, chunk, dt, scale, qk_l2norm, gate, norm_weight,
                                       norm_eps, o, final_state, workspace, workspace_bytes, stream);
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           float* state, int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, float scale,
                           int32_t qk_l2norm, void* o, hipStream_t stream)
{
    return decode_impl(q, k, v, g, beta, state, N, H, dk, dv, dt, scale, qk_l2norm, o, gdn::GatedNorm{}, stream);
}

gdn_status gdn_decode_step_gated(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 float* state, int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt,
                                 float scale, int32_t qk_l2norm, const void* gate, const float* norm_weight,
                                 float norm_eps, void* o, hipStream_t stream)
{
    gdn::GatedNorm nm;
    nm.z = gate;
    nm.w = norm_weight;
    nm.eps = norm_eps;
    const gdn_status st = check_norm(nm, N > 0);
    if (st != GDN_OK) return st;
    if (!nm.z) nm.z = o;
    return decode_impl(q, k, v, g, beta, state, N, H, dk, dv, dt, scale, qk_l2norm, o, nm, stream);
}

}  // extern "C"

namespace {

// Checks shared by the two front-end entry points.
gdn_status check_frontend(const void* xq, const void* xk, const void* xv, const float* w, const float* a,
                          const float* b, const float* A_log, const float* dt_bias, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, int32_t H, int32_t dk, int32_t dv,
                          gdn_dtype dt)
{
    if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (H < 1 || dk < 1 || dv < 1) return GDN_ERR_BAD_SHAPE;
    if (dk % 8 != 0 || dv % 8 != 0) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)H * (2 * (int64_t)dk + dv) > (1 << 24)) return GDN_ERR_BAD_SHAPE;
    if (!xq || !xk || !xv || !w || !a || !b || !A_log || !dt_bias || !q || !k || !v || !g || !beta)
        return GDN_ERR_NULL_ARG;
    const void* p16[] = {xq, xk, xv, w, q, k, v};
    for (const void* p : p16)
        if (!aligned16(p)) return GDN_ERR_ALIGNMENT;
    const void* p4[] = {a, b, A_log, dt_bias, g, beta};
    for (const void* p : p4)
        if (!aligned4(p)) return GDN_ERR_ALIGNMENT;
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_frontend_prefill(const void* xq, const void* xk, const void* xv, const float* conv_weight,
                                const float* a, const float* b, const float* A_log, const float* dt_bias,
                                const void* conv_state_in, const int32_t* cu_seqlens, int32_t num_seqs,
                                int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, void* q,
                                void* k, void* v, float* g, float* beta, void* conv_state_out, hipStream_t stream)
{
    if (total_tokens < 0 || num_seqs < 1) return GDN_ERR_BAD_SHAPE;
    if (total_tokens > ((int64_t)1 << 31) - 1) return GDN_ERR_BAD_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return GDN_ERR_BAD_SHAPE;
    if (total_tokens == 0 && !conv_state_out) return GDN_OK;
    if (total_tokens > 0) {
        const gdn_status st = check_frontend(xq, xk, xv, conv_weight, a, b, A_log, dt_bias, q, k, v, g, beta, H,
                                             dk, dv, dt);
        if (st != GDN_OK) return st;
    } else {
        if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
        if (H < 1 || dk < 1 || dv < 1) return GDN_ERR_BAD_SHAPE;
        if (dk % 8 != 0 || dv % 8 != 0) return GDN_ERR_UNSUPPORTED;
    }
    if ((conv_state_in && !aligned16(conv_state_in)) || (conv_state_out && !aligned16(conv_state_out)))
        return GDN_ERR_ALIGNMENT;
    if (conv_state_in && conv_state_out && conv_state_in != conv_state_out) {
        const size_t bytes = (size_t)num_seqs * 3 * (size_t)H * (2 * (size_t)dk + dv) * (dt == GDN_BF16 ? 2 : 4);
        const char* a0 = (const char*)conv_state_in;
        const char* b0 = (const char*)conv_state_out;
        if (a0 < b0 + bytes && b0 < a0 + bytes) return GDN_ERR_BAD_SHAPE;  // partial overlap
    }
    gdn::FrontendArgs fa;
    fa.xq = xq; fa.xk = xk; fa.xv = xv; fa.w = conv_weight;
    fa.a = a; fa.b = b; fa.A_log = A_log; fa.dt_bias = dt_bias;
    fa.state_in = conv_state_in; fa.state_out = conv_state_out;
    fa.cu = cu_seqlens; fa.N = num_seqs; fa.T = total_tokens;
    fa.H = H; fa.dk = dk; fa.dv = dv; fa.bf16 = dt == GDN_BF16; fa.decode = false;
    fa.q = q; fa.k = k; fa.v = v; fa.g = g; fa.beta = beta;
    fa.stream = stream;
    return finish(gdn::launch_frontend(fa), stream);
}

gdn_status gdn_frontend_decode(const void* xq, const void* xk, const void* xv, const float* conv_weight,
                               const float* a, const float* b, const float* A_log, const float* dt_bias,
                               void* conv_state, int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, void* q,
                               void* k, void* v, float* g, float* beta, hipStream_t stream)
{
    if (N < 0) return GDN_ERR_BAD_SHAPE;
    if (N == 0) {
        if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
        return (H < 1 || dk < 1 || dv < 1) ? GDN_ERR_BAD_SHAPE : GDN_OK;
    }
    const gdn_status st = check_frontend(xq, xk, xv, conv_weight, a, b, A_log, dt_bias, q, k, v, g, beta, H, dk,
                                         dv, dt);
    if (st != GDN_OK) return st;
    if (!conv_state) return GDN_ERR_NULL_ARG;
    if (!aligned16(conv_state)) return GDN_ERR_ALIGNMENT;
    gdn::FrontendArgs fa;
    fa.xq = xq; fa.xk = xk; fa.xv = xv; fa.w = conv_weight;
    fa.a = a; fa.b = b; fa.A_log = A_log; fa.dt_bias = dt_bias;
    fa.state_in = conv_state; fa.state_out = conv_state;
    fa.cu = nullptr; fa.N = N; fa.T = N;
    fa.H = H; fa.dk = dk; fa.dv = dv; fa.bf16 = dt == GDN_BF16; fa.decode = true;
    fa.q = q; fa.k = k; fa.v = v; fa.g = g; fa.beta = beta;
    fa.stream = stream;
    return finish(gdn::launch_frontend(fa), stream);
}

}  // extern "C"

extern "C" {

size_t gdn_prefill_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv)
{
    if (total_tokens < 0 || num_seqs < 1 || H < 1) return 0;
    if (!gdn::backward_supported(dk, dv)) return 0;
    return gdn::backward_layout(total_tokens, num_seqs, H, dk, dv).total;
}

gdn_status gdn_chunk_prefill_backward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                      const float* init_state, const void* d_o, const float* d_final_state,
                                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                      int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt,
                                      float scale, int32_t qk_l2norm, float* grad_q, float* grad_k, float* grad_v,
                                      float* grad_g, float* grad_beta, float* grad_init_state, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream)
{
    if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (total_tokens < 0 || num_seqs < 1 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_BAD_SHAPE;
    if (total_tokens > ((int64_t)1 << 31) - 1) return GDN_ERR_BAD_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return GDN_ERR_BAD_SHAPE;
    if (!gdn::backward_supported(dk, dv)) return GDN_ERR_UNSUPPORTED;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !d_o || !grad_q || !grad_k || !grad_v || !grad_g ||
                             !grad_beta))
        return GDN_ERR_NULL_ARG;
    if (!workspace) return GDN_ERR_WORKSPACE;
    const void* p16[] = {q, k, v, d_o, init_state, d_final_state, grad_q, grad_k, grad_v, grad_init_state};
    for (const void* p : p16)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    const void* p4[] = {g, beta, grad_g, grad_beta};
    for (const void* p : p4)
        if (!aligned4(p)) return GDN_ERR_ALIGNMENT;
    if (((uintptr_t)workspace & 255u) != 0) return GDN_ERR_ALIGNMENT;
    if (cu_seqlens_host) {
        if (cu_seqlens_host[0] != 0 || cu_seqlens_host[num_seqs] != total_tokens) return GDN_ERR_BAD_SEQLENS;
        for (int32_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return GDN_ERR_BAD_SEQLENS;
    }
    const gdn::BwdLayout lay = gdn::backward_layout(total_tokens, num_seqs, H, dk, dv);
    if (workspace_bytes < lay.total) return GDN_ERR_WORKSPACE;
    if (grad_init_state) {
        // the two chains run side by side: the initial-state gradient, written at
        // the end of the reverse chain, must not share memory with either state input
        const size_t bytes = (size_t)num_seqs * H * dv * dk * 4;
        const char* o0 = (const char*)grad_init_state;
        const char* ins[] = {(const char*)init_state, (const char*)d_final_state};
        for (const char* p : ins)
            if (p && p < o0 + bytes && o0 < p + bytes) return GDN_ERR_BAD_SHAPE;
    }
    gdn::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dO = d_o; a.g = g; a.beta = beta;
    a.init_state = init_state; a.dstate = d_final_state;
    a.cu_seqlens = cu_seqlens;
    a.N = num_seqs; a.T = total_tokens; a.H = H; a.dk = dk; a.dv = dv;
    a.bf16 = dt == GDN_BF16;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)dk);
    a.l2norm = qk_l2norm ? 1 : 0;
    a.dq = grad_q; a.dk_out = grad_k; a.dv_out = grad_v; a.dg = grad_g; a.dbeta = grad_beta;
    a.dinit = grad_init_state;
    a.ws = (unsigned char*)workspace;
    a.lay = lay;
    a.stream = stream;
    return finish(gdn::launch_backward(a), stream);
}

}  // extern "C"
