// api_driver.cpp -- the C-ABI host code (gdn_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU.
//
// Linked with gdn_api.cpp only: the kernel launchers, the context and scratch
// functions of the HIP translation units and the three HIP runtime calls the
// host code makes are replaced by the stubs below, so every argument check,
// workspace layout and dispatch decision runs on the host.  Device buffers are
// host allocations of exactly the size the library asks for; the launcher
// stubs touch the first and last byte of every region the layout hands a
// kernel, so a layout that overruns its buffer is an ASan report.
#include <assert.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/gdn.h"
#include "../../hybrid_linear_attention_delta_amd/csrc/gdn_launch.h"

// ---------------------------------------------------------------- HIP stubs
extern "C" hipError_t hipGetDevice(int* d)
{
    *d = 0;
    return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

// ---------------------------------------------------------------- library stubs
struct gdn_context {
    int dev;
};

static int g_launches = 0;
static int64_t g_last_window = -1;  // window of the last prefill launch (0: the whole workspace)
static volatile unsigned char g_sink = 0;

static void touch(const void* base, size_t off, size_t bytes)
{
    if (bytes == 0) return;
    const unsigned char* p = static_cast<const unsigned char*>(base) + off;
    g_sink = g_sink + p[0] + p[bytes - 1];
}

namespace gdn {

hipError_t context_create(int32_t, gdn_context** out)
{
    *out = new gdn_context{0};
    return hipSuccess;
}
hipError_t context_destroy(gdn_context* c)
{
    delete c;
    return hipSuccess;
}
int context_device(const gdn_context* c) { return c->dev; }

static unsigned char* g_scratch = nullptr;
hipError_t scratch_device_ptr(void** out)
{
    if (!g_scratch) g_scratch = static_cast<unsigned char*>(malloc(kScratchBytes));
    *out = g_scratch;
    return g_scratch ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t launch_prefill(const PrefillArgs& a)
{
    ++g_launches;
    const PrefillLayout& L = a.lay;
    assert(L.total > 0 && L.off_header == 0);
    const size_t offs[] = {L.off_chunk_tab, L.off_seq_first, L.off_seq_order, L.off_records, L.off_states,
                           L.off_deltas, L.off_carry};
    size_t prev = 0;
    for (size_t o : offs) {
        assert(o % 256 == 0 && o >= prev);
        prev = o;
    }
    touch(a.ws, 0, L.total);  // the whole workspace belongs to the caller's buffer
    touch(a.ws, L.off_carry, (size_t)a.N * a.H * a.dv * a.dk * 4);
    assert(a.window >= 0);
    if (a.window > 0) assert(a.stages == 7);  // windows only for calls that run every stage
    g_last_window = a.window;
    return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs&)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_frontend(const FrontendArgs&)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_conv_state(const FrontendArgs&) { return hipSuccess; }
hipError_t launch_backward(const BwdArgs& a)
{
    ++g_launches;
    assert(a.lay.total > 0);
    touch(a.ws, 0, a.lay.total);
    return hipSuccess;
}

}  // namespace gdn

// ---------------------------------------------------------------- cases
static int g_fail = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

struct Buf {
    std::vector<unsigned char> v;
    explicit Buf(size_t n) : v(n + 256) {}
    void* p() { return reinterpret_cast<void*>(((uintptr_t)v.data() + 255) & ~(uintptr_t)255); }
};

static gdn_status prefill(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t C, gdn_dtype dt,
                          const int32_t* cu_host, size_t ws_bytes, gdn_context_t ctx = nullptr, bool noalloc = false)
{
    const size_t el = dt == GDN_BF16 ? 2 : 4;
    Buf q(T * H * dk * el + 16), k(T * H * dk * el + 16), v(T * H * dv * el + 16), o(T * H * dv * el + 16);
    Buf g(T * H * 4 + 4), b(T * H * 4 + 4), st(N * H * dv * dk * 4 + 16), ws(ws_bytes), cu((N + 1) * 4);
    const int32_t* cu_dev = cu_host ? static_cast<const int32_t*>(cu.p()) : nullptr;
    if (noalloc)
        return gdn_chunk_prefill_noalloc(q.p(), k.p(), v.p(), (float*)g.p(), (float*)b.p(), (float*)st.p(), cu_dev,
                                         cu_host, N, T, H, dk, dv, C, dt, -1.f, 1, o.p(), (float*)st.p(), nullptr);
    return gdn_chunk_prefill_ctx(ctx, q.p(), k.p(), v.p(), (float*)g.p(), (float*)b.p(), (float*)st.p(), cu_dev,
                                 cu_host, N, T, H, dk, dv, C, dt, -1.f, 1, o.p(), (float*)st.p(), ws.p(), ws_bytes,
                                 nullptr);
}

int main()
{
    // workspace sizes: positive, monotone in T, zero for unsupported shapes
    size_t prev = 0;
    for (int64_t T : {0, 1, 63, 64, 65, 4096, 65536, 2097152}) {
        const size_t w = gdn_prefill_workspace_size(T, 1, 6, 256, 256, 64, GDN_BF16);
        CHECK(w > 0 && w >= prev);
        prev = w;
    }
    CHECK(gdn_prefill_workspace_size(100, 1, 6, 48, 48, 64, GDN_BF16) == 0);
    CHECK(gdn_prefill_workspace_size(100, 0, 6, 256, 256, 64, GDN_BF16) == 0);
    CHECK(gdn_prefill_backward_workspace_size(100, 2, 2, 64, 64) > 0);
    CHECK(gdn_prefill_backward_workspace_size(100, 2, 2, 32, 64) == 0);
    for (int s = 0; s <= 9; ++s) CHECK(gdn_status_string((gdn_status)s) != nullptr);

    // valid prefills of every supported shape reach the launcher with an in-bounds layout
    const int32_t dks_bf[] = {64, 128, 256}, dvs_bf[] = {64, 128, 256, 512};
    for (int32_t dk : dks_bf)
        for (int32_t dv : dvs_bf) {
            const int64_t T = 300;
            const size_t ws = gdn_prefill_workspace_size(T, 1, 2, dk, dv, 64, GDN_BF16);
            CHECK(prefill(T, 1, 2, dk, dv, 64, GDN_BF16, nullptr, ws) == GDN_OK);
        }
    const int32_t ds_f32[] = {16, 32, 64, 128, 256}, cs_f32[] = {16, 32, 64};
    for (int32_t d : ds_f32)
        for (int32_t c : cs_f32) {
            const size_t ws = gdn_prefill_workspace_size(100, 1, 2, d, d, c, GDN_F32);
            CHECK(prefill(100, 1, 2, d, d, c, GDN_F32, nullptr, ws) == GDN_OK);
        }
    // packed sequences (with empty ones), host-validated
    {
        const int32_t cu[] = {0, 70, 70, 200, 201};
        const size_t ws = gdn_prefill_workspace_size(201, 4, 2, 64, 64, 64, GDN_BF16);
        CHECK(prefill(201, 4, 2, 64, 64, 64, GDN_BF16, cu, ws) == GDN_OK);
        // below the full size: windows of chunks (the whole buffer still in bounds), down to the minimum
        CHECK(prefill(201, 4, 2, 64, 64, 64, GDN_BF16, cu, ws - 1) == GDN_OK && g_last_window > 0);
        const size_t mn = gdn_prefill_workspace_min_size(201, 4, 2, 64, 64, 64, GDN_BF16);
        CHECK(mn > 0 && mn < ws);
        CHECK(prefill(201, 4, 2, 64, 64, 64, GDN_BF16, cu, mn) == GDN_OK && g_last_window == 1);
        CHECK(prefill(201, 4, 2, 64, 64, 64, GDN_BF16, cu, mn - 1) == GDN_ERR_WORKSPACE);
        CHECK(prefill(201, 4, 2, 64, 64, 64, GDN_BF16, cu, ws) == GDN_OK && g_last_window == 0);
        const int32_t bad[] = {0, 70, 60, 200, 201};
        CHECK(prefill(201, 4, 2, 64, 64, 64, GDN_BF16, bad, ws) == GDN_ERR_BAD_SEQLENS);
    }
    // with a context
    {
        gdn_context_t ctx = nullptr;
        CHECK(gdn_context_create(0, &ctx) == GDN_OK && ctx);
        const size_t ws = gdn_prefill_workspace_size(5000, 1, 2, 256, 256, 64, GDN_BF16);
        CHECK(prefill(5000, 1, 2, 256, 256, 64, GDN_BF16, nullptr, ws, ctx) == GDN_OK);
        CHECK(gdn_context_destroy(ctx) == GDN_OK);
        CHECK(gdn_context_create(32, &ctx) == GDN_ERR_BAD_SHAPE && !ctx);
        CHECK(gdn_context_create(0, nullptr) == GDN_ERR_NULL_ARG);
    }
    // the no-allocation path: whole workspace, windows, and a refusal
    CHECK(prefill(1000, 1, 6, 256, 256, 64, GDN_BF16, nullptr, 0, nullptr, true) == GDN_OK);
    CHECK(prefill(40000, 1, 6, 256, 256, 64, GDN_BF16, nullptr, 0, nullptr, true) == GDN_OK);
    {
        std::vector<int32_t> cu(201, 0);
        CHECK(prefill(0, 200, 6, 256, 256, 64, GDN_BF16, cu.data(), 0, nullptr, true) == GDN_ERR_WORKSPACE);
    }
    // host validation errors
    const size_t ws = gdn_prefill_workspace_size(128, 1, 2, 64, 64, 64, GDN_BF16);
    CHECK(prefill(128, 1, 2, 48, 64, 64, GDN_BF16, nullptr, ws) == GDN_ERR_UNSUPPORTED);
    CHECK(prefill(128, 1, 2, 64, 64, 32, GDN_BF16, nullptr, ws) == GDN_ERR_UNSUPPORTED);
    CHECK(prefill(128, 1, 2, 64, 64, 64, GDN_BF16, nullptr,
                  gdn_prefill_workspace_min_size(128, 1, 2, 64, 64, 64, GDN_BF16) - 1) == GDN_ERR_WORKSPACE);
    {  // a stage subset needs the full size
        Buf x(1 << 16), w(ws);
        CHECK(gdn_chunk_prefill_staged(x.p(), x.p(), x.p(), (float*)x.p(), (float*)x.p(), nullptr, nullptr, nullptr, 1,
                                       128, 2, 64, 64, 64, GDN_BF16, -1.f, 1, x.p(), nullptr, w.p(), ws - 1,
                                       GDN_STAGE_PREPARE, nullptr) == GDN_ERR_WORKSPACE);
    }
    CHECK(prefill(128, 2, 2, 64, 64, 64, GDN_BF16, nullptr, ws) == GDN_ERR_BAD_SHAPE);
    CHECK(prefill(-1, 1, 2, 64, 64, 64, GDN_BF16, nullptr, ws) == GDN_ERR_BAD_SHAPE);

    // decode, front end and backward reach their launchers; bad arguments do not
    {
        Buf x(4096), st(1 << 20), o(4096);
        CHECK(gdn_decode_step(x.p(), x.p(), x.p(), (float*)x.p(), (float*)x.p(), (float*)st.p(), 2, 2, 64, 64,
                              GDN_BF16, -1.f, 1, o.p(), nullptr) == GDN_OK);
        CHECK(gdn_decode_step(x.p(), x.p(), x.p(), (float*)x.p(), (float*)x.p(), (float*)st.p(), 2, 2, 48, 64,
                              GDN_BF16, -1.f, 1, o.p(), nullptr) == GDN_ERR_UNSUPPORTED);
        CHECK(gdn_frontend_decode(x.p(), x.p(), x.p(), (float*)x.p(), (float*)x.p(), (float*)x.p(), (float*)x.p(),
                                  (float*)x.p(), st.p(), 2, 2, 64, 64, GDN_BF16, x.p(), x.p(), x.p(), (float*)x.p(),
                                  (float*)x.p(), nullptr) == GDN_OK);
        const size_t bws = gdn_prefill_backward_workspace_size(100, 1, 2, 64, 64);
        Buf bw(bws), big(1 << 20);
        CHECK(gdn_chunk_prefill_backward(big.p(), big.p(), big.p(), (float*)big.p(), (float*)big.p(), nullptr,
                                         big.p(), nullptr, nullptr, nullptr, 1, 100, 2, 64, 64, GDN_BF16, -1.f, 1,
                                         (float*)big.p(), (float*)big.p(), (float*)big.p(), (float*)big.p(),
                                         (float*)big.p(), nullptr, bw.p(), bws, nullptr) == GDN_OK);
        CHECK(gdn_chunk_prefill_backward(big.p(), big.p(), big.p(), (float*)big.p(), (float*)big.p(), nullptr,
                                         big.p(), nullptr, nullptr, nullptr, 1, 100, 2, 64, 64, GDN_BF16, -1.f, 1,
                                         (float*)big.p(), (float*)big.p(), (float*)big.p(), (float*)big.p(),
                                         (float*)big.p(), nullptr, bw.p(), bws - 1, nullptr) == GDN_ERR_WORKSPACE);
    }
    // the fused front end and the gated read-out reach the launcher; fp32 is refused by the fused path
    {
        const int64_t T = 200;
        const size_t wsf = gdn_prefill_workspace_size(T, 1, 2, 64, 64, 64, GDN_BF16);
        Buf x(T * 2 * 64 * 2 + 64), a(T * 2 * 4), w(2 * 192 * 16), hh(64), st(3 * 2 * 192 * 2 + 64), o(T * 2 * 64 * 2),
            fs(2 * 64 * 64 * 4), wsb(wsf);
        CHECK(gdn_chunk_prefill_frontend(nullptr, x.p(), x.p(), x.p(), (float*)w.p(), (float*)a.p(), (float*)a.p(),
                                         (float*)hh.p(), (float*)hh.p(), st.p(), nullptr, nullptr, nullptr, 1, T, 2,
                                         64, 64, 64, GDN_BF16, -1.f, 1, o.p(), (float*)fs.p(), st.p(), wsb.p(), wsf,
                                         nullptr) == GDN_OK);
        CHECK(gdn_chunk_prefill_frontend(nullptr, x.p(), x.p(), x.p(), (float*)w.p(), (float*)a.p(), (float*)a.p(),
                                         (float*)hh.p(), (float*)hh.p(), st.p(), nullptr, nullptr, nullptr, 1, T, 2,
                                         64, 64, 64, GDN_F32, -1.f, 1, o.p(), (float*)fs.p(), st.p(), wsb.p(), wsf,
                                         nullptr) == GDN_ERR_UNSUPPORTED);
        CHECK(gdn_chunk_prefill_gated(x.p(), x.p(), x.p(), (float*)a.p(), (float*)a.p(), nullptr, nullptr, nullptr, 1,
                                      T, 2, 64, 64, 64, GDN_BF16, -1.f, 1, o.p(), nullptr, 1e-6f, o.p(),
                                      (float*)fs.p(), wsb.p(), wsf, nullptr) == GDN_OK);
        CHECK(gdn_chunk_prefill_gated(x.p(), x.p(), x.p(), (float*)a.p(), (float*)a.p(), nullptr, nullptr, nullptr, 1,
                                      T, 2, 64, 64, 64, GDN_BF16, -1.f, 1, nullptr, nullptr, 1e-6f, o.p(),
                                      (float*)fs.p(), wsb.p(), wsf, nullptr) == GDN_ERR_NULL_ARG);
    }
    free(gdn::g_scratch);
    printf("api driver: %d launches, %d failed checks\n", g_launches, g_fail);
    return g_fail == 0 ? 0 : 1;
}
