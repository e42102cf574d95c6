// Internal interface between the C ABI (gdn_api.cpp) and the gfx950 kernels
// (gdn_kernels.hip).  Not installed; the public surface is include/gdn_stream.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum KernelKind { KPREP = 0, KSCAN = 1, KSEQ = 2, KBWD = 3, KCOUNT = 4 };

// Everything one launch needs.  Directions: 0 = forward (t ascending, starts
// from S_in), 1 = reverse (t descending, starts from zero).
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o[2];            // output per direction
    const float* a;
    const float* beta;
    int64_t qs[3], ks[3], vs[3], os[3], gs[3];   // (b, t, h) strides, elements
    int64_t T;
    int B, H, Dk, Dv;
    int io_f32;            // 0 = bf16, 1 = fp32 for q, k, v, o
    int l2norm;
    float eps, scale;
    const float* S_in;     // forward start state [B, H, Dv, Dk], or null (zero)
    float* S_out[2];       // final state per direction, or null
    int dir0, ndirs;       // directions dir0 .. dir0 + ndirs - 1
    // chunked path workspace: one item per (dir, b, h, sub-chunk)
    char* ws;
    int64_t ws_item_bytes;
    int nsub_max;
    int C;                 // sub-chunk length
    __bf16* conv;          // fp32 I/O only: bf16 copies of q, k, v ([3][B][T][H][D])
    // K and Q rows as MFMA operand fragments, by 16-token tile in token order (shared by
    // both directions): [2 (K, Q)][B][H][ntile_max][(D/16 + 1)/2 k-steps][64 lanes][16 B]
    char* frag;
    int ntile_max;
};

// Bytes of one workspace item for sub-chunk C (multiple of 16, 16..64).
int64_t chunk_item_bytes(int C, int D);
// Bytes of the fragment area for B streams, H heads and up to max_tokens tokens.
int64_t chunk_frag_bytes(int D, int64_t max_tokens, int B, int H);

// Gradient of one token-sequential scan (fp32).  Workspace (owned by the handle):
// states [B][H][Dv/16][T+1][16][Dk] and partial sums [B][T][H][Dv/16][2 Dk + 2].
struct BwdParams {
    const void* d_o;       // dL/do, io dtype, o's strides (Params::os)
    const float* d_state;  // dL/d(final state) [B, H, Dv, Dk], or null
    const float* state0;   // start state of the scan [B, H, Dv, Dk], or null (zero)
    float* dq;             // [B, T, H, Dk]
    float* dk;             // [B, T, H, Dk]
    float* dv;             // [B, T, H, Dv]
    float* da;             // [B, T, H]
    float* dbeta;          // [B, T, H]
    float* d_state0;       // [B, H, Dv, Dk], or null
    float* states;
    float* partials;
    int reverse;           // 0: the forward scan (t ascending), 1: the reverse scan
};
// Bytes of the backward workspace for max_tokens tokens.
int64_t backward_ws_bytes(int B, int H, int Dk, int Dv, int64_t max_tokens);

// Which (C, D) pairs the chunked kernels are built for.
bool chunked_supported(int C, int Dk, int Dv, int io_f32);

// Optional per-kernel timing: when `ev` is non-null, ev[2*i] / ev[2*i+1] are
// recorded around launch i and *nlaunch receives the count (<= 4).
struct Timing {
    hipEvent_t* ev;
    int* kinds;
    int cap;
    int n;
};

// Softmax attention of a chunk over the sink + window cache (gdn_attention.hip).  Cache
// buffers are [B][H][capacity][D] bf16; n_sink / n_win of their slots are valid.
struct AttnParams {
    const void *q, *k, *v;
    void* o;
    int64_t qs[3], ks[3], vs[3], os[3];
    const void *k_sink, *v_sink, *k_win, *v_win;
    int sink_cap, win_cap, n_sink, n_win;
    int T, B, H, D;
    float scale_log2;   // logit scale times log2(e)
};
// Cache append after a committed call: the first `taken` tokens fill sink slots from
// sink_fill on, the rest go to the window ring from slot win_base, the first `skip` of them
// (already older than the window) not at all.
struct AppendParams {
    const void *k, *v;
    int64_t ks[3], vs[3];
    void *k_sink, *v_sink, *k_win, *v_win;
    int sink_cap, win_cap, T, B, H, D;
    int sink_fill, taken, skip, win_base;
};
bool attn_dim_supported(int d);
hipError_t launch_attention(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_append(const AppendParams& p, hipStream_t s);

hipError_t launch_zero(float* x, int64_t n, hipStream_t s);
hipError_t launch_sequential(const Params& p, hipStream_t s, Timing* tm);
hipError_t launch_chunked(const Params& p, hipStream_t s, Timing* tm);
hipError_t launch_backward(const Params& p, const BwdParams& g, hipStream_t s, Timing* tm);

}  // namespace gdn
