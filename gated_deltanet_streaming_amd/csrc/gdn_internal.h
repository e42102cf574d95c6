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
    int gate_log;          // a holds log a_t instead of a_t
    int spin_limit;        // polls before a wavefront gives up waiting for another
    int* err;              // error word (host memory): set to 1 when a wait gives up
    // Time split of the forward scan (dir0 = 0, ndirs = 1): nseg segments of seg_steps steps (the
    // last one shorter), states [B, H, Dv, Dk] per entry.
    //   seg_mode 0: the plain scan (the fields below unused)
    //   seg_mode 1: every segment twice, from a zero state (variant 0) and from the identity with
    //               v read as zero (variant 1); outputs dropped; final states to
    //               seg_out[2 sigma + variant]
    //   seg_mode 2: segment sigma from S_in (sigma = 0) or seg_in[sigma]; outputs written; the last
    //               segment's final state to S_out[0]
    int seg_mode, nseg, seg_steps;
    const float* seg_in;
    float* seg_out;
};
// Scan workgroups per (stream-head, row slice): directions, or the segments (and variants) of a
// time split.
inline int scan_variants(const Params& p) {
    return p.seg_mode == 1 ? 2 * p.nseg : p.seg_mode == 2 ? p.nseg : p.ndirs;
}

// Bytes of one workspace item for sub-chunk C (multiple of 16, 16..64).
int64_t chunk_item_bytes(int C, int D);

// Gradient of one token-sequential scan (fp32).  Workspace (owned by the handle): state
// checkpoints [B][H][Dv/4][ck_per][4][Dk] (the state before every staged block of tokens)
// and partial sums [B][T][H][Dv/16][2 Dk + 4].
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
    float* states;         // checkpoints
    float* gck;            // adjoint checkpoints [B][H][Dv/4][gck_per][4][Dk]: dL/dS at the end of every segment
    float* partials;
    int64_t ck_per;        // checkpoints per (b, h, row block) in `states`
    int64_t gck_per;       // adjoint checkpoints per (b, h, row block) in `gck`
    int reverse;           // 0: the forward scan (t ascending), 1: the reverse scan
};
// Bytes of the backward workspace for max_tokens tokens, or -1 if the size overflows int64.
int64_t backward_ws_bytes(int B, int H, int Dk, int Dv, int64_t max_tokens);
// Checkpoints per (b, h, row block) for max_tokens tokens, and the floats they take in all
// (where the partial sums start in the workspace).
int64_t backward_ckpt_per(int64_t max_tokens);
int64_t backward_gck_per(int64_t max_tokens);
int64_t backward_state_ckpt_floats(int B, int H, int Dk, int Dv, int64_t max_tokens);
int64_t backward_ckpt_floats(int B, int H, int Dk, int Dv, int64_t max_tokens);

// Which (C, D) pairs the chunked kernels are built for.
bool chunked_supported(int C, int Dk, int Dv, int io_f32);

// Static workspace of the allocation-free entry point: a file-scope device array in
// gdn_kernels.hip, one copy per device, loaded with the library's code object and kept until
// the process ends.  scratch_address gives its device address on `device`, which must be the
// current device; the address is looked up once per device (hipGetSymbolAddress) and kept.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
hipError_t scratch_address(int device, char** out);

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

// Low-precision projection GEMMs (gdn_lowp.hip).  Per-row E4M3 quantisation of x [rows][cols] (bf16 or
// fp32, row stride in elements) into codes [rows][codes_stride] and fp32 scales [rows].
struct QuantParams {
    const void* x;
    int64_t rows, cols, x_stride;
    int x_f32;
    unsigned char* codes;
    int64_t codes_stride;
    float* scales;
};
// y[m][n] (bf16, row stride y_stride elements) = x_scales[m] w_scales[n] sum_k x[m][k] w[n][k] over E4M3 codes
// (row strides in bytes); K a multiple of 16, N a multiple of 4.
struct GemmParams {
    const unsigned char* x;
    int64_t x_stride;
    const float* x_scales;
    const unsigned char* w;
    int64_t w_stride;
    const float* w_scales;
    int64_t M, N, K;
    void* y;
    int64_t y_stride;
};
hipError_t launch_quantize_rows(const QuantParams& p, hipStream_t s);
hipError_t launch_gemm_e4m3(const GemmParams& p, hipStream_t s);
// index of the workgroup tile configuration that launch_gemm_e4m3 picks for M x N on cus compute units
int gemm_e4m3_tile_features(int64_t M, int64_t N, int cus);

hipError_t launch_zero(float* x, int64_t n, hipStream_t s);
hipError_t launch_sequential(const Params& p, hipStream_t s, Timing* tm);
hipError_t launch_chunked(const Params& p, hipStream_t s, Timing* tm);
// The forward scan as a time split (p.seg_mode 0, p.nseg segments of p.seg_steps steps, p.seg_out
// set; seg_in: [nseg][B][H][D][D] for the segments' start states).
hipError_t launch_split(const Params& p, float* seg_in, hipStream_t s, Timing* tm);
// Gradient of g0's scan, and of g1's as well in the same launches when g1 is not null (each with
// its own workspace).
hipError_t launch_backward(const Params& p, const BwdParams& g0, const BwdParams* g1, hipStream_t s, Timing* tm);

}  // namespace gdn
