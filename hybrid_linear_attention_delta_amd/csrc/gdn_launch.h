// gdn_launch.h -- internal launch interface between the C-ABI host code and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

// Execution context of the pipelined prefill (the opaque gdn_context_t of the
// C ABI): the streams and events one prefill call uses to overlap its stages.
struct gdn_context;

namespace gdn {

// Context management (gdn_prefill.hip).  context_create makes the streams and
// events on the current device; context_destroy waits for them and frees them.
hipError_t context_create(int32_t chain_cus_per_xcd, gdn_context** out);
hipError_t context_destroy(gdn_context* ctx);
int context_device(const gdn_context* ctx);
constexpr int32_t kDefaultChainCus = 16;  // chain CUs per XCD of the B=1, H=6, d=256 workload

// Gated RMSNorm of the read-out (optional epilogue): o <- o / sqrt(mean_v o^2 + eps) * w * silu(z)
// per (token, head) over the d_v values.  z has the layout and type of o; w is [d_v] fp32 or NULL.
struct GatedNorm {
    const void* z = nullptr;  // NULL: no epilogue
    const float* w = nullptr;
    float eps = 0.f;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float* state;
    void* o;
    int32_t N, H, dk, dv;
    bool bf16;
    float scale;
    int32_t l2norm;
    GatedNorm norm;
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);

// Chunked prefill.  The workspace is carved into the regions described by
// PrefillLayout (computed on the host, identically for size queries and calls).
struct PrefillLayout {
    int64_t max_chunks;     // upper bound on sum_n ceil(L_n / C)
    size_t off_header;      // int32[16]: [0] error flag, [1] number of chunks
    size_t off_chunk_tab;   // int32[max_chunks][4]: tok0, len, seq, 0
    size_t off_seq_first;   // int32[N + 1]: first chunk of each sequence
    size_t off_seq_order;   // int32[N]: sequences by descending length (the chain's dispatch order)
    size_t off_records;     // per chunk-head operand records
    size_t record_bytes;    // bytes of one record
    size_t off_states;      // per chunk-head state entering the chunk [dv][dk], operand type
    size_t off_deltas;      // per chunk-head Delta^T [hi, lo][dv][C], operand type
    size_t off_carry;       // fp32 [N][H][dv][dk]: state carried between pipeline segments
    size_t total;
};

bool prefill_supported(bool bf16, int32_t dk, int32_t dv, int32_t chunk);
// window_chunks > 0: the per-chunk regions (records, states, deltas) hold that
// many chunks instead of every chunk of the call
PrefillLayout prefill_layout(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                             int32_t chunk, bool bf16, int64_t window_chunks = 0);

// The front end folded into the prefill's row loads (gdn_chunk_prefill_frontend):
// the projections xq, xk, xv [T][H][dk|dv] and the gate inputs a, b [T][H]
// replace q, k, v, g and beta; taps w [ctot][4] fp32 and the conv state
// [N][3][ctot] as in FrontendArgs.  cu: the device cu_seqlens (or NULL).
struct FrontIn {
    const void *xq = nullptr, *xk = nullptr, *xv = nullptr;
    const float* w = nullptr;
    const float *a = nullptr, *b = nullptr, *A_log = nullptr, *dt_bias = nullptr;
    const void* state_in = nullptr;
    const int32_t* cu = nullptr;
};

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float* init_state;
    const int32_t* cu_seqlens;       // device, may be NULL (single sequence)
    const int32_t* seq_order;        // unused for now (NULL)
    int32_t N;
    int64_t T;
    int32_t H, dk, dv, chunk;
    bool bf16;
    float scale;
    int32_t l2norm;
    void* o;
    float* final_state;
    unsigned char* ws;
    PrefillLayout lay;
    int32_t stages;  // bit 0: prepare (chunk table + intra-chunk), bit 1: propagate (state chain), bit 2: outputs
    GatedNorm norm;  // epilogue of the output stage
    gdn_context* ctx;  // NULL: every kernel on `stream`
    int64_t window;    // > 0: the workspace holds `window` chunks of per-chunk data (stage by stage per window)
    bool fused;        // the front end is folded into the preparation (fe replaces q, k, v, g, beta)
    FrontIn fe;
    void* conv_state_out;  // fused: [N][3][ctot] or NULL (may alias fe.state_in)
    hipStream_t stream;
};

hipError_t launch_prefill(const PrefillArgs& a);

// The no-allocation prefill's workspace: a device array of kScratchBytes per
// GPU inside the library.  scratch_device_ptr returns its address on the
// current device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kScratchBytes = (size_t)256 << 20;
hipError_t scratch_device_ptr(void** out);

// Front end: short causal conv + SiLU on the q, k, v projections and the gate
// math.  Channels of q, k, v form one axis of 2 H dk + H dv (q, k, v in order)
// for the taps w [ctot][4] fp32 and the conv state [N][3][ctot] (type of x).
struct FrontendArgs {
    const void *xq, *xk, *xv;  // [T (or N)][H dk | H dv]
    const float* w;
    const float *a, *b, *A_log, *dt_bias;
    const void* state_in;      // prefill: [N][3][ctot] or NULL (zeros)
    void* state_out;           // prefill: may be NULL or alias state_in; decode: the state, in place
    const int32_t* cu;         // prefill: device [N + 1] or NULL (one sequence)
    int32_t N;
    int64_t T;
    int32_t H, dk, dv;
    bool bf16;
    bool decode;
    void *q, *k, *v;
    float *g, *beta;
    hipStream_t stream;
};

hipError_t launch_frontend(const FrontendArgs& a);
// Only the conv-state update of a prefill front end (state_in -> state_out from
// the last three inputs of every sequence); the q, k, v and gate outputs are not made.
hipError_t launch_conv_state(const FrontendArgs& a);

// Backward of the chunked prefill (fp32 workspace, chunk 64).  Offsets are
// bytes into the workspace; per chunk-head arrays hold max_chunks * H slices.
struct BwdLayout {
    int64_t max_chunks;  // upper bound on sum_n ceil(L_n / 64)
    size_t off_header, off_tab, off_seq_first;
    size_t off_Q, off_K, off_V, off_dO, off_rq, off_rk, off_gam, off_bet;
    size_t off_T, off_P, off_KKG, off_U, off_E, off_dDl, off_sck;
    size_t off_S, off_Dl, off_dS, off_dD;
    size_t off_dQ, off_dK, off_dW, off_dPG, off_dT, off_X1, off_Bd;
    // the state chains' operands as bf16 hi/lo fragments (hi parts only for the
    // raw k and q of bf16 inputs, which bf16 holds exactly): W, raw k, raw q and
    // r_q E over the chunk rows; W and raw k over d_k
    size_t off_Wf, off_Kf, off_Qf, off_Ef;
    size_t off_Wr, off_Kr;
    size_t total;
};

constexpr int kBwdChunk = 64;  // chunk length of the backward
bool backward_supported(int32_t dk, int32_t dv);
BwdLayout backward_layout(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv);

struct BwdArgs {
    const void *q, *k, *v, *dO;           // [T][H][d], bf16 or fp32 (one type)
    const float *g, *beta;                // [T][H]
    const float *init_state, *dstate;     // [N][H][dv][dk] or NULL (zeros)
    const int32_t* cu_seqlens;            // device [N + 1] or NULL (one sequence)
    int32_t N;
    int64_t T;
    int32_t H, dk, dv;
    bool bf16;
    float scale;
    int32_t l2norm;
    float *dq, *dk_out, *dv_out, *dg, *dbeta;  // fp32, shapes of the inputs
    float* dinit;                              // [N][H][dv][dk] or NULL
    unsigned char* ws;
    BwdLayout lay;
    hipStream_t stream;
};

hipError_t launch_backward(const BwdArgs& a);

}  // namespace gdn
