// gdn_api.cpp -- C ABI of the Gated DeltaNet streaming core (include/gdn_stream.h).
//
// Owns the per-handle state cache (one d_v x d_k fp32 state per stream and
// head: the pages' compact recurrent state, Chinese summary "Core method") and
// a workspace fixed at init, so memory stays constant however long the stream
// runs (the pages' constant-memory streaming, Chinese summary "Prerequisites",
// "Streaming generation").  Every argument is validated before anything is
// enqueued; on error the cache is untouched and nothing runs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "gdn_internal.h"
#include "gdn_attn.h"
#include "gdn_lowp.h"
#include "gdn_stream.h"

struct gdn_stream {
    gdn_config cfg;
    int device;
    int C;                // sub-chunk of the chunked kernels
    bool chunked_ok;      // chunked kernels exist for this shape and dtype
    float* state;         // [B, H, d_v, d_k]
    int64_t state_elems;
    char* ws;             // chunked workspace: [2 directions][B][H][nsub_max] items
    __bf16* conv;         // fp32 I/O with the chunked kernels: bf16 staging of q, k, v
    int64_t item_bytes;
    int nsub_max;
    int64_t items_total;  // bytes of the items
    int* err;             // error word in pinned host memory: a kernel wait gave up
    int spin_limit;       // polls before a wait gives up
    float* bwd_ws;        // backward workspace (states, partial sums), allocated on first use
    float* bwd_ws2;       // the reverse scan's backward workspace of a bidirectional gradient call
    float* seg_ws;        // time-split workspace (segment states), allocated on first use, grown on demand
    int64_t seg_elems;
    // optional per-kernel timing
    bool profile;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pend;
    std::vector<int> pend_kind;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> spare;
    double acc_ms[gdn::KCOUNT];
    int64_t acc_n[gdn::KCOUNT];
};

// Softmax-block attention handle: the sink and window cache of every (stream, head), with
// the fill counters kept on the host (they follow from the sequence of committed calls).
struct gdn_attn {
    gdn_attn_config cfg;
    int device;
    float scale;
    __bf16* cache;        // k_sink | v_sink | k_win | v_win, each [B][H][capacity][d]
    int64_t sink_fill;    // tokens in the sink
    int64_t win_total;    // tokens ever written to the window (the ring head is win_total mod window)
    bool profile;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pend, spare;
    double acc_ms;
    int64_t acc_n;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return GDN_OK;
}

// A wait inside an earlier call's kernels gave up: its outputs are not valid.  Reported once.
int check_err_word(gdn_stream* s) {
    if (s->err && __atomic_load_n(s->err, __ATOMIC_ACQUIRE) != 0) {
        __atomic_store_n(s->err, 0, __ATOMIC_RELEASE);
        return fail(GDN_E_HIP, "a wait inside an earlier call's kernels gave up (spin limit %d): that call's "
                               "outputs and state are not valid", s->spin_limit);
    }
    return GDN_OK;
}

// Makes the handle's device current for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            changed = err == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

bool is_mult16(int x) { return x >= 16 && x <= 128 && x % 16 == 0; }

int elem_size(const gdn_config& c) { return c.io_dtype == GDN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The product of non-negative sizes in int64; false if a factor is negative or it overflows.
bool size_product(std::initializer_list<int64_t> factors, int64_t* out) {
    int64_t r = 1;
    for (const int64_t x : factors)
        if (x < 0 || __builtin_mul_overflow(r, x, &r)) return false;
    *out = r;
    return true;
}

constexpr int64_t kMaxTokens = (int64_t)1 << 30;   // the kernels count tokens in 32-bit integers
constexpr int64_t kMaxStride = (int64_t)1 << 40;   // elements; larger strides cannot address a real tensor

// Rows of one (stream, head) are addressed with 32-bit byte offsets from a
// per-(b, h) base, and rows past the end of the sequence must not overlap real
// rows (they read as zero): token stride >= row width, extent < 2 GiB.
int check_tensor(const char* name, const void* ptr, const int64_t* st, int esz, int width, int64_t T) {
    if (!ptr) return fail(GDN_E_INVAL, "%s is NULL", name);
    if (!aligned16(ptr)) return fail(GDN_E_INVAL, "%s is not 16-byte aligned", name);
    for (int i = 0; i < 3; ++i) {
        if (st[i] < 0) return fail(GDN_E_INVAL, "%s stride %d is negative", name, i);
        if (st[i] > kMaxStride) return fail(GDN_E_SHAPE, "%s stride %d (%lld elements) is too large", name, i, (long long)st[i]);
        if ((st[i] * esz) % 16 != 0)
            return fail(GDN_E_INVAL, "%s stride %d (%lld elements) is not a multiple of 16 bytes", name, i,
                        (long long)st[i]);
    }
    if (st[1] < width)
        return fail(GDN_E_INVAL, "%s token stride %lld is smaller than the row width %d", name, (long long)st[1], width);
    // (T + 64) st[1] esz < 2^31, with T <= kMaxTokens checked by every caller
    if (st[1] > (((int64_t)1 << 31) - 1) / ((T + 64) * esz))
        return fail(GDN_E_SHAPE, "%s: T * token stride exceeds the 2 GiB per-(stream, head) extent", name);
    return GDN_OK;
}

// Validation of a configuration shared by gdn_stream_init and gdn_chunk_bidir_noalloc; on success
// *C receives the sub-chunk length.
int check_config(const gdn_config& c, uint32_t allowed_flags, int* C) {
    if (c.batch < 1 || c.heads < 1) return fail(GDN_E_SHAPE, "batch and heads must be >= 1");
    if (!is_mult16(c.d_k) || !is_mult16(c.d_v))
        return fail(GDN_E_SHAPE, "d_k=%d d_v=%d must be multiples of 16 in [16, 128]", c.d_k, c.d_v);
    if (c.max_tokens < 1 || c.max_tokens > kMaxTokens) return fail(GDN_E_SHAPE, "max_tokens must be in [1, 2^30]");
    *C = c.subchunk == 0 ? 64 : c.subchunk;
    if (!(*C == 16 || *C == 32 || *C == 64)) return fail(GDN_E_SHAPE, "subchunk %d not in {0, 16, 32, 64}", c.subchunk);
    if (c.io_dtype != GDN_BF16 && c.io_dtype != GDN_F32) return fail(GDN_E_DTYPE, "unknown io_dtype %d", c.io_dtype);
    if (c.flags & ~allowed_flags) return fail(GDN_E_INVAL, "unknown config flag bits 0x%x", c.flags & ~allowed_flags);
    if (!std::isfinite(c.l2_eps) || c.l2_eps < 0.f) return fail(GDN_E_INVAL, "l2_eps must be finite and >= 0");
    if (!std::isfinite(c.scale)) return fail(GDN_E_INVAL, "scale must be finite");
    return GDN_OK;
}

// q, k, v, o (and o_rev when given), a and beta of a call of T > 0 tokens.
int check_io(const gdn_config& c, const gdn_io* io, int64_t T, const void* o_rev, bool need_rev) {
    const int esz = elem_size(c);
    int rc;
    const int dk = c.d_k, dv = c.d_v;
    if ((rc = check_tensor("q", io->q, io->q_strides, esz, dk, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("k", io->k, io->k_strides, esz, dk, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("v", io->v, io->v_strides, esz, dv, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("o", io->o, io->o_strides, esz, dv, T)) != GDN_OK) return rc;
    if (need_rev && (rc = check_tensor("o_rev", o_rev, io->o_strides, esz, dv, T)) != GDN_OK) return rc;
    if (!io->a) return fail(GDN_E_INVAL, "a is NULL");
    if (!io->beta) return fail(GDN_E_INVAL, "beta is NULL");
    for (int i = 0; i < 3; ++i)
        if (io->g_strides[i] < 0) return fail(GDN_E_INVAL, "gate stride %d is negative", i);
    return GDN_OK;
}

int check_call(gdn_stream* s, const gdn_io* io, int64_t T, uint32_t flags, const void* o_rev, bool need_rev) {
    if (!s) return fail(GDN_E_INVAL, "handle is NULL");
    if (!io) return fail(GDN_E_INVAL, "io is NULL");
    if (check_err_word(s) != GDN_OK) return GDN_E_HIP;
    if (flags & ~(uint32_t)(GDN_NO_COMMIT | GDN_SEQUENTIAL)) return fail(GDN_E_INVAL, "unknown flag bits 0x%x", flags);
    if (T < 0 || T > s->cfg.max_tokens)
        return fail(GDN_E_SHAPE, "T = %lld outside [0, max_tokens = %lld]", (long long)T, (long long)s->cfg.max_tokens);
    if (T == 0) return GDN_OK;
    const int rc = check_io(s->cfg, io, T, o_rev, need_rev);
    if (rc != GDN_OK) return rc;
    if (!(flags & GDN_SEQUENTIAL) && !s->chunked_ok)
        return fail(GDN_E_SHAPE,
                    "no chunked kernel for d_k=%d d_v=%d subchunk=%d io_dtype=%d; pass GDN_SEQUENTIAL",
                    s->cfg.d_k, s->cfg.d_v, s->C, s->cfg.io_dtype);
    return GDN_OK;
}

// The parts of a launch's parameters that follow from the configuration and the call.
gdn::Params call_params(const gdn_config& c, int C, const gdn_io* io, int64_t T) {
    gdn::Params p;
    std::memset(&p, 0, sizeof p);
    p.q = io->q;
    p.k = io->k;
    p.v = io->v;
    p.o[0] = p.o[1] = io->o;
    p.a = io->a;
    p.beta = io->beta;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = io->q_strides[i];
        p.ks[i] = io->k_strides[i];
        p.vs[i] = io->v_strides[i];
        p.os[i] = io->o_strides[i];
        p.gs[i] = io->g_strides[i];
    }
    p.T = T;
    p.B = c.batch;
    p.H = c.heads;
    p.Dk = c.d_k;
    p.Dv = c.d_v;
    p.io_f32 = c.io_dtype == GDN_F32;
    p.l2norm = (c.flags & GDN_L2NORM_QK) != 0;
    p.eps = c.l2_eps;
    p.scale = c.scale;
    p.C = C;
    p.gate_log = (c.flags & GDN_GATE_IS_LOG) != 0;
    return p;
}

gdn::Params base_params(gdn_stream* s, const gdn_io* io, int64_t T) {
    gdn::Params p = call_params(s->cfg, s->C, io, T);
    p.ws = s->ws;
    p.ws_item_bytes = s->item_bytes;
    p.nsub_max = s->nsub_max;
    p.conv = s->conv;
    p.spin_limit = s->spin_limit;
    p.err = s->err;
    return p;
}

// Polls before a kernel wait gives up: 2^22, or GDN_SPIN_LIMIT from the environment.
int env_spin_limit() {
    int lim = 1 << 22;
    if (const char* sl = std::getenv("GDN_SPIN_LIMIT")) {
        const long v = std::strtol(sl, nullptr, 10);
        if (v >= 1 && v <= INT_MAX) lim = (int)v;
    }
    return lim;
}

// Fold finished timing events into the per-kernel totals.
void drain_profile(gdn_stream* s) {
    for (size_t i = 0; i < s->pend.size(); ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(s->pend[i].second) == hipSuccess &&
            hipEventElapsedTime(&ms, s->pend[i].first, s->pend[i].second) == hipSuccess) {
            s->acc_ms[s->pend_kind[i]] += ms;
            s->acc_n[s->pend_kind[i]] += 1;
        }
        s->spare.push_back(s->pend[i]);
    }
    s->pend.clear();
    s->pend_kind.clear();
}

int run(gdn_stream* s, gdn::Params& p, uint32_t flags, hipStream_t st, float* split_in = nullptr) {
    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", s->device, hipGetErrorString(dg.err));
    hipError_t prior = hipPeekAtLastError();
    if (prior != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_E_HIP, "earlier HIP error: %s", hipGetErrorString(prior));
    }
    hipEvent_t evs[8];
    int kinds[4];
    gdn::Timing tm{nullptr, kinds, 4, 0};
    if (s->profile) {
        for (int i = 0; i < 4; ++i) {
            std::pair<hipEvent_t, hipEvent_t> pr;
            if (!s->spare.empty()) {
                pr = s->spare.back();
                s->spare.pop_back();
            } else if (hipEventCreate(&pr.first) != hipSuccess || hipEventCreate(&pr.second) != hipSuccess) {
                return fail(GDN_E_HIP, "hipEventCreate failed");
            }
            evs[2 * i] = pr.first;
            evs[2 * i + 1] = pr.second;
        }
        tm.ev = evs;
    }
    hipError_t e = split_in                   ? gdn::launch_split(p, split_in, st, &tm)
                   : (flags & GDN_SEQUENTIAL) ? gdn::launch_sequential(p, st, &tm)
                                              : gdn::launch_chunked(p, st, &tm);
    if (s->profile) {
        for (int i = 0; i < 4; ++i) {
            auto pr = std::make_pair(evs[2 * i], evs[2 * i + 1]);
            if (i < tm.n) {
                s->pend.push_back(pr);
                s->pend_kind.push_back(kinds[i]);
            } else {
                s->spare.push_back(pr);
            }
        }
    }
    if (e != hipSuccess) return fail(GDN_E_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

GDN_API int gdn_stream_init(const gdn_config* cfg, int device, gdn_stream** out) {
    if (!cfg || !out) return fail(GDN_E_INVAL, "cfg and out must be non-NULL");
    *out = nullptr;
    const gdn_config c = *cfg;
    int C = 0;
    const int rc = check_config(c, GDN_L2NORM_QK | GDN_GATE_IS_LOG | GDN_POISON_WS, &C);
    if (rc != GDN_OK) return rc;
    // every size the handle allocates, checked for overflow before anything is allocated
    const bool chunked = gdn::chunked_supported(C, c.d_k, c.d_v, c.io_dtype == GDN_F32);
    const int64_t item_bytes = chunked ? gdn::chunk_item_bytes(C, c.d_k) : 0;
    const int64_t nsub_max = (c.max_tokens + C - 1) / C;
    int64_t state_elems = 0, items_total = 0, conv_bytes = 0;
    if (!size_product({c.batch, c.heads, c.d_v, c.d_k, (int64_t)sizeof(float)}, &state_elems) ||
        !size_product({2, c.batch, c.heads, nsub_max, item_bytes}, &items_total) ||
        !size_product({3, c.batch, c.max_tokens, c.heads, c.d_k, 2}, &conv_bytes))
        return fail(GDN_E_SHAPE, "batch %d x heads %d x max_tokens %lld: the state or workspace size overflows",
                    c.batch, c.heads, (long long)c.max_tokens);
    state_elems /= (int64_t)sizeof(float);

    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess) return fail(GDN_E_HIP, "hipGetDeviceCount: %s", hipGetErrorString(e));
    if (device < 0 || device >= ndev) return fail(GDN_E_HIP, "device %d not present (%d devices)", device, ndev);
    DeviceGuard dg(device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", device, hipGetErrorString(dg.err));

    gdn_stream* s = new (std::nothrow) gdn_stream();
    if (!s) return fail(GDN_E_NOMEM, "host allocation failed");
    s->cfg = c;
    s->device = device;
    s->C = C;
    s->chunked_ok = chunked;
    s->state_elems = state_elems;
    s->profile = false;
    for (int i = 0; i < gdn::KCOUNT; ++i) {
        s->acc_ms[i] = 0.0;
        s->acc_n[i] = 0;
    }
    e = hipMalloc(&s->state, s->state_elems * sizeof(float));
    if (e != hipSuccess) {
        delete s;
        return fail(GDN_E_NOMEM, "state cache allocation: %s", hipGetErrorString(e));
    }
    e = hipMemset(s->state, 0, s->state_elems * sizeof(float));
    s->ws = nullptr;
    s->conv = nullptr;
    s->bwd_ws = nullptr;
    s->bwd_ws2 = nullptr;
    s->seg_ws = nullptr;
    s->seg_elems = 0;
    s->item_bytes = 0;
    s->nsub_max = 0;
    s->items_total = 0;
    s->err = nullptr;
    s->spin_limit = env_spin_limit();
    if (e == hipSuccess) {
        e = hipHostMalloc(reinterpret_cast<void**>(&s->err), sizeof(int), hipHostMallocCoherent | hipHostMallocMapped);
        if (e != hipSuccess) {
            s->err = nullptr;
            (void)hipFree(s->state);
            delete s;
            return fail(GDN_E_NOMEM, "error word allocation: %s", hipGetErrorString(e));
        }
        *s->err = 0;
    }
    if (e == hipSuccess && s->chunked_ok) {
        s->item_bytes = item_bytes;
        s->nsub_max = (int)nsub_max;
        s->items_total = items_total;
        const int64_t bytes = s->items_total;
        e = hipMalloc(&s->ws, bytes);
        if (e != hipSuccess) {
            (void)hipFree(s->state);
            (void)hipHostFree(s->err);
            delete s;
            return fail(GDN_E_NOMEM, "workspace allocation (%lld bytes): %s", (long long)bytes, hipGetErrorString(e));
        }
        if (c.flags & GDN_POISON_WS) e = hipMemset(s->ws, 0xff, bytes);
        if (c.io_dtype == GDN_F32) {
            const int64_t cb = conv_bytes;
            e = hipMalloc(&s->conv, cb);
            if (e != hipSuccess) {
                (void)hipFree(s->state);
                (void)hipFree(s->ws);
                (void)hipHostFree(s->err);
                delete s;
                return fail(GDN_E_NOMEM, "bf16 staging allocation (%lld bytes): %s", (long long)cb,
                            hipGetErrorString(e));
            }
        }
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(s->state);
        if (s->ws) (void)hipFree(s->ws);
        if (s->conv) (void)hipFree(s->conv);
        if (s->err) (void)hipHostFree(s->err);
        delete s;
        return fail(GDN_E_HIP, "init: %s", hipGetErrorString(e));
    }
    *out = s;
    return ok();
}

GDN_API int gdn_stream_destroy(gdn_stream* s) {
    if (!s) return ok();
    DeviceGuard dg(s->device);
    hipError_t e = hipDeviceSynchronize();
    for (auto& pr : s->pend) {
        (void)hipEventDestroy(pr.first);
        (void)hipEventDestroy(pr.second);
    }
    for (auto& pr : s->spare) {
        (void)hipEventDestroy(pr.first);
        (void)hipEventDestroy(pr.second);
    }
    (void)hipFree(s->state);
    if (s->ws) (void)hipFree(s->ws);
    if (s->conv) (void)hipFree(s->conv);
    if (s->bwd_ws) (void)hipFree(s->bwd_ws);
    if (s->bwd_ws2) (void)hipFree(s->bwd_ws2);
    if (s->seg_ws) (void)hipFree(s->seg_ws);
    if (s->err) (void)hipHostFree(s->err);
    delete s;
    if (e != hipSuccess) return fail(GDN_E_HIP, "destroy: %s", hipGetErrorString(e));
    return ok();
}

GDN_API int gdn_chunk_forward(gdn_stream* s, const gdn_io* io, int64_t T, uint32_t flags, float* state_out,
                              void* hip_stream) {
    int rc = check_call(s, io, T, flags, nullptr, false);
    if (rc != GDN_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const bool commit = !(flags & GDN_NO_COMMIT);
    if (T == 0) {
        if (!commit && state_out) {
            DeviceGuard dg(s->device);
            hipError_t e = hipMemcpyAsync(state_out, s->state, s->state_elems * sizeof(float),
                                          hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return fail(GDN_E_HIP, "state copy: %s", hipGetErrorString(e));
        }
        return ok();
    }
    gdn::Params p = base_params(s, io, T);
    p.S_in = s->state;
    p.S_out[0] = commit ? s->state : state_out;
    p.dir0 = 0;
    p.ndirs = 1;
    return run(s, p, flags, st);
}

GDN_API int gdn_chunk_forward_split(gdn_stream* s, const gdn_io* io, int64_t T, int segments, uint32_t flags,
                                    float* state_out, void* hip_stream) {
    int rc = check_call(s, io, T, flags, nullptr, false);
    if (rc != GDN_OK) return rc;
    if (flags & GDN_SEQUENTIAL) return fail(GDN_E_INVAL, "the time split runs on the chunked kernels only");
    if (segments < 1) return fail(GDN_E_INVAL, "segments = %d, must be >= 1", segments);
    const int64_t N = (T + s->C - 1) / s->C;
    if (segments == 1 || N < 2) return gdn_chunk_forward(s, io, T, flags, state_out, hip_stream);
    int nseg = (int)std::min<int64_t>(segments, N);
    const int seg_steps = (int)((N + nseg - 1) / nseg);
    nseg = (int)((N + seg_steps - 1) / seg_steps);   // no empty segment
    int64_t need = 0;
    if (__builtin_mul_overflow((int64_t)3 * nseg, s->state_elems, &need))
        return fail(GDN_E_SHAPE, "time-split workspace size overflows");
    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", s->device, hipGetErrorString(dg.err));
    if (s->seg_elems < need) {
        // a larger split than before: the old workspace may still be in use by enqueued work
        hipError_t e = hipDeviceSynchronize();
        if (e == hipSuccess && s->seg_ws) e = hipFree(s->seg_ws);
        s->seg_ws = nullptr;
        s->seg_elems = 0;
        if (e != hipSuccess) return fail(GDN_E_HIP, "time-split workspace release: %s", hipGetErrorString(e));
        e = hipMalloc(&s->seg_ws, need * sizeof(float));
        if (e != hipSuccess) {
            s->seg_ws = nullptr;
            return fail(GDN_E_NOMEM, "time-split workspace (%lld bytes): %s", (long long)(need * 4), hipGetErrorString(e));
        }
        s->seg_elems = need;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const bool commit = !(flags & GDN_NO_COMMIT);
    gdn::Params p = base_params(s, io, T);
    p.S_in = s->state;
    p.S_out[0] = commit ? s->state : state_out;
    p.dir0 = 0;
    p.ndirs = 1;
    p.nseg = nseg;
    p.seg_steps = seg_steps;
    p.seg_out = s->seg_ws + (int64_t)nseg * s->state_elems;
    return run(s, p, flags, st, s->seg_ws);
}

GDN_API int gdn_chunk_reverse(gdn_stream* s, const gdn_io* io, int64_t T, uint32_t flags, float* state_out,
                              void* hip_stream) {
    int rc = check_call(s, io, T, flags, nullptr, false);
    if (rc != GDN_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (T == 0) {
        if (state_out) {
            DeviceGuard dg(s->device);
            hipError_t e = gdn::launch_zero(state_out, s->state_elems, st);
            if (e != hipSuccess) return fail(GDN_E_HIP, "state zero: %s", hipGetErrorString(e));
        }
        return ok();
    }
    gdn::Params p = base_params(s, io, T);
    p.S_in = nullptr;
    p.S_out[1] = state_out;
    p.dir0 = 1;
    p.ndirs = 1;
    return run(s, p, flags, st);
}

GDN_API int gdn_chunk_bidir(gdn_stream* s, const gdn_io* io, void* o_rev, int64_t T, uint32_t flags,
                            float* state_out, void* hip_stream) {
    int rc = check_call(s, io, T, flags, o_rev, T > 0);
    if (rc != GDN_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const bool commit = !(flags & GDN_NO_COMMIT);
    if (T == 0) {
        if (!commit && state_out) {
            DeviceGuard dg(s->device);
            hipError_t e = hipMemcpyAsync(state_out, s->state, s->state_elems * sizeof(float),
                                          hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return fail(GDN_E_HIP, "state copy: %s", hipGetErrorString(e));
        }
        return ok();
    }
    gdn::Params p = base_params(s, io, T);
    p.o[1] = o_rev;
    p.S_in = s->state;
    p.S_out[0] = commit ? s->state : state_out;
    p.S_out[1] = nullptr;
    p.dir0 = 0;
    p.ndirs = 2;
    return run(s, p, flags, st);
}

GDN_API int gdn_chunk_bidir_noalloc(const gdn_config* cfg, const gdn_io* io, void* o_rev, int64_t T,
                                    const float* state_in, float* state_out, int* status, void* hip_stream) {
    static_assert(gdn::kScratchBytes == GDN_NOALLOC_SCRATCH_BYTES, "scratch size");
    if (!cfg || !io) return fail(GDN_E_INVAL, "cfg and io must be non-NULL");
    if (!status) return fail(GDN_E_INVAL, "status is NULL");
    gdn_config c = *cfg;
    c.max_tokens = 1;   // not used by this call
    int C = 0;
    int rc = check_config(c, GDN_L2NORM_QK | GDN_GATE_IS_LOG, &C);
    if (rc != GDN_OK) return rc;
    if (c.io_dtype != GDN_BF16) return fail(GDN_E_DTYPE, "the allocation-free call takes bf16 q, k, v, o only");
    if (!gdn::chunked_supported(C, c.d_k, c.d_v, 0))
        return fail(GDN_E_SHAPE, "no chunked kernel for d_k=%d d_v=%d subchunk=%d", c.d_k, c.d_v, C);
    if (T < 0 || T > kMaxTokens) return fail(GDN_E_SHAPE, "T = %lld outside [0, 2^30]", (long long)T);
    const int64_t item = gdn::chunk_item_bytes(C, c.d_k);
    const int64_t nsub = (T + C - 1) / C;
    int64_t need = 0;
    if (!size_product({2, c.batch, c.heads, nsub, item}, &need) || need > gdn::kScratchBytes)
        return fail(GDN_E_SHAPE, "B=%d H=%d T=%lld needs %lld bytes of workspace, more than the %lld of the static scratch",
                    c.batch, c.heads, (long long)T, (long long)need, (long long)gdn::kScratchBytes);
    if (T > 0 && (rc = check_io(c, io, T, o_rev, true)) != GDN_OK) return rc;

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    char* ws = nullptr;
    e = gdn::scratch_address(dev, &ws);
    if (e != hipSuccess) return fail(GDN_E_HIP, "static scratch on device %d: %s", dev, hipGetErrorString(e));
    hipError_t prior = hipPeekAtLastError();
    if (prior != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_E_HIP, "earlier HIP error: %s", hipGetErrorString(prior));
    }
    const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (T == 0) {
        if (!state_out || state_out == state_in) return ok();
        const int64_t n = (int64_t)c.batch * c.heads * c.d_v * c.d_k;
        e = state_in ? hipMemcpyAsync(state_out, state_in, n * sizeof(float), hipMemcpyDeviceToDevice, st)
                     : gdn::launch_zero(state_out, n, st);
        return e == hipSuccess ? ok() : fail(GDN_E_HIP, "state copy: %s", hipGetErrorString(e));
    }
    static const int spin_limit = env_spin_limit();
    gdn::Params p = call_params(c, C, io, T);
    p.ws = ws;
    p.ws_item_bytes = item;
    p.nsub_max = (int)nsub;
    p.conv = nullptr;
    p.spin_limit = spin_limit;
    p.err = status;
    p.o[1] = o_rev;
    p.S_in = state_in;
    p.S_out[0] = state_out;
    p.S_out[1] = nullptr;
    p.dir0 = 0;
    p.ndirs = 2;
    gdn::Timing tm{nullptr, nullptr, 0, 0};
    e = gdn::launch_chunked(p, st, &tm);
    if (e != hipSuccess) return fail(GDN_E_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

GDN_API int gdn_state_get(gdn_stream* s, float* dst, void* hip_stream) {
    if (!s || !dst) return fail(GDN_E_INVAL, "handle and dst must be non-NULL");
    if (check_err_word(s) != GDN_OK) return GDN_E_HIP;
    DeviceGuard dg(s->device);
    hipError_t e = hipMemcpyAsync(dst, s->state, s->state_elems * sizeof(float), hipMemcpyDeviceToDevice,
                                  reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDN_E_HIP, "state_get: %s", hipGetErrorString(e));
    return ok();
}

GDN_API int gdn_state_set(gdn_stream* s, const float* src, void* hip_stream) {
    if (!s) return fail(GDN_E_INVAL, "handle is NULL");
    if (check_err_word(s) != GDN_OK) return GDN_E_HIP;
    DeviceGuard dg(s->device);
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t e = src ? hipMemcpyAsync(s->state, src, s->state_elems * sizeof(float), hipMemcpyDeviceToDevice, st)
                       : gdn::launch_zero(s->state, s->state_elems, st);
    if (e != hipSuccess) return fail(GDN_E_HIP, "state_set: %s", hipGetErrorString(e));
    return ok();
}

GDN_API int gdn_profile(gdn_stream* s, int enable) {
    if (!s) return fail(GDN_E_INVAL, "handle is NULL");
    s->profile = enable != 0;
    return ok();
}

GDN_API int gdn_profile_read(gdn_stream* s, double* ms, int64_t* launches, int reset) {
    if (!s) return fail(GDN_E_INVAL, "handle is NULL");
    DeviceGuard dg(s->device);
    drain_profile(s);
    for (int i = 0; i < gdn::KCOUNT; ++i) {
        if (ms) ms[i] = s->acc_ms[i];
        if (launches) launches[i] = s->acc_n[i];
        if (reset) {
            s->acc_ms[i] = 0.0;
            s->acc_n[i] = 0;
        }
    }
    return ok();
}

// Checks of one scan's gradient arguments (nothing is enqueued here).
static int check_grad(const gdn_stream* s, const gdn_io* io, const gdn_grad* g, int64_t T, int reverse, const char* which) {
    if (!g) return fail(GDN_E_INVAL, "%s is NULL", which);
    if (reverse && g->state0) return fail(GDN_E_INVAL, "the reverse scan starts from zero: %s->state0 must be NULL", which);
    if (T == 0) return GDN_OK;
    int rc;
    if ((rc = check_tensor("d_o", g->d_o, io->o_strides, elem_size(s->cfg), s->cfg.d_v, T)) != GDN_OK) return rc;
    if (!g->dq || !g->dk || !g->dv || !g->da || !g->dbeta) return fail(GDN_E_INVAL, "a gradient output of %s is NULL", which);
    return GDN_OK;
}

// A backward workspace, allocated on first use and kept until gdn_stream_destroy.
static int ensure_bwd_ws(gdn_stream* s, float** ws) {
    if (*ws) return GDN_OK;
    const int64_t bytes = gdn::backward_ws_bytes(s->cfg.batch, s->cfg.heads, s->cfg.d_k, s->cfg.d_v, s->cfg.max_tokens);
    if (bytes < 0) return fail(GDN_E_SHAPE, "the backward workspace size overflows");
    hipError_t e = hipMalloc(ws, bytes);
    if (e != hipSuccess) {
        *ws = nullptr;
        (void)hipGetLastError();
        return fail(GDN_E_NOMEM, "backward workspace (%lld bytes): %s", (long long)bytes, hipGetErrorString(e));
    }
    if (s->cfg.flags & GDN_POISON_WS) {
        // NaN bytes: a checkpoint or partial sum that the kernels read without writing shows up
        e = hipMemset(*ws, 0xff, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(*ws);
            *ws = nullptr;
            return fail(GDN_E_HIP, "poisoning the backward workspace: %s", hipGetErrorString(e));
        }
    }
    return GDN_OK;
}

static gdn::BwdParams bwd_params(const gdn_stream* s, const gdn_grad* g, float* ws, int reverse) {
    gdn::BwdParams b;
    b.d_o = g->d_o;
    b.d_state = g->d_state;
    b.state0 = g->state0;
    b.dq = g->dq;
    b.dk = g->dk;
    b.dv = g->dv;
    b.da = g->da;
    b.dbeta = g->dbeta;
    b.d_state0 = g->d_state0;
    b.states = ws;
    b.gck = ws + gdn::backward_state_ckpt_floats(s->cfg.batch, s->cfg.heads, s->cfg.d_k, s->cfg.d_v, s->cfg.max_tokens);
    b.partials = ws + gdn::backward_ckpt_floats(s->cfg.batch, s->cfg.heads, s->cfg.d_k, s->cfg.d_v, s->cfg.max_tokens);
    b.ck_per = gdn::backward_ckpt_per(s->cfg.max_tokens);
    b.gck_per = gdn::backward_gck_per(s->cfg.max_tokens);
    b.reverse = reverse;
    return b;
}

// The gradient of one scan (g1 null: g0's scan is the forward scan when reverse0 = 0, the
// reverse scan when reverse0 = 1) or of both scans of a bidirectional call (g0: the forward
// scan, g1: the reverse scan), each with its own workspace, in one launch pair.
static int backward_impl(gdn_stream* s, const gdn_io* io, const gdn_grad* g0, const gdn_grad* g1, int64_t T,
                         int reverse0, void* hip_stream) {
    if (!s) return fail(GDN_E_INVAL, "handle is NULL");
    if (!io) return fail(GDN_E_INVAL, "io is NULL");
    if (check_err_word(s) != GDN_OK) return GDN_E_HIP;
    if (reverse0 != 0 && reverse0 != 1) return fail(GDN_E_INVAL, "reverse must be 0 or 1");
    const bool both = g1 != nullptr;
    int rc;
    if (T < 0 || T > s->cfg.max_tokens)
        return fail(GDN_E_SHAPE, "T = %lld outside [0, max_tokens = %lld]", (long long)T, (long long)s->cfg.max_tokens);
    if ((rc = check_grad(s, io, g0, T, reverse0, both ? "g_fwd" : "grad")) != GDN_OK) return rc;
    if (both && (rc = check_grad(s, io, g1, T, 1, "g_rev")) != GDN_OK) return rc;
    const int64_t sbytes = s->state_elems * (int64_t)sizeof(float);
    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", s->device, hipGetErrorString(dg.err));
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (T == 0) {
        for (const gdn_grad* g : {g0, g1}) {
            if (!g || !g->d_state0) continue;
            hipError_t e = g->d_state ? hipMemcpyAsync(g->d_state0, g->d_state, sbytes, hipMemcpyDeviceToDevice, st)
                                      : gdn::launch_zero(g->d_state0, s->state_elems, st);
            if (e != hipSuccess) return fail(GDN_E_HIP, "d_state0: %s", hipGetErrorString(e));
        }
        return ok();
    }
    const int esz = elem_size(s->cfg);
    const int dk = s->cfg.d_k, dv = s->cfg.d_v;
    if ((rc = check_tensor("q", io->q, io->q_strides, esz, dk, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("k", io->k, io->k_strides, esz, dk, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("v", io->v, io->v_strides, esz, dv, T)) != GDN_OK) return rc;
    if (!io->a) return fail(GDN_E_INVAL, "a is NULL");
    if (!io->beta) return fail(GDN_E_INVAL, "beta is NULL");
    for (int i = 0; i < 3; ++i)
        if (io->g_strides[i] < 0) return fail(GDN_E_INVAL, "gate stride %d is negative", i);
    if ((rc = ensure_bwd_ws(s, &s->bwd_ws)) != GDN_OK) return rc;
    if (both && (rc = ensure_bwd_ws(s, &s->bwd_ws2)) != GDN_OK) return rc;
    gdn::Params p = base_params(s, io, T);
    p.dir0 = reverse0;
    p.ndirs = 1;
    const gdn::BwdParams b0 = bwd_params(s, g0, s->bwd_ws, reverse0);
    const gdn::BwdParams b1 = both ? bwd_params(s, g1, s->bwd_ws2, 1) : b0;
    hipError_t prior = hipPeekAtLastError();
    if (prior != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_E_HIP, "earlier HIP error: %s", hipGetErrorString(prior));
    }
    hipEvent_t evs[2];
    int kinds[1];
    gdn::Timing tm{nullptr, kinds, 1, 0};
    std::pair<hipEvent_t, hipEvent_t> pr;
    if (s->profile) {
        if (!s->spare.empty()) {
            pr = s->spare.back();
            s->spare.pop_back();
        } else if (hipEventCreate(&pr.first) != hipSuccess || hipEventCreate(&pr.second) != hipSuccess) {
            return fail(GDN_E_HIP, "hipEventCreate failed");
        }
        evs[0] = pr.first;
        evs[1] = pr.second;
        tm.ev = evs;
    }
    hipError_t e = gdn::launch_backward(p, b0, both ? &b1 : nullptr, st, &tm);
    if (s->profile) {
        if (tm.n > 0) {
            s->pend.push_back(pr);
            s->pend_kind.push_back(kinds[0]);
        } else {
            s->spare.push_back(pr);
        }
    }
    if (e != hipSuccess) return fail(GDN_E_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

GDN_API int gdn_chunk_backward(gdn_stream* s, const gdn_io* io, const gdn_grad* g, int64_t T, int reverse,
                               void* hip_stream) {
    return backward_impl(s, io, g, nullptr, T, reverse, hip_stream);
}

GDN_API int gdn_chunk_backward_bidir(gdn_stream* s, const gdn_io* io, const gdn_grad* g_fwd, const gdn_grad* g_rev,
                                     int64_t T, void* hip_stream) {
    if (s && io && g_fwd && !g_rev) return fail(GDN_E_INVAL, "g_rev is NULL");
    return backward_impl(s, io, g_fwd, g_rev, T, 0, hip_stream);
}

// ---- softmax-block attention over the sink + window cache (gdn_attn.h) ----------------------

GDN_API int gdn_attn_init(const gdn_attn_config* cfg, int device, gdn_attn** out) {
    if (!cfg || !out) return fail(GDN_E_INVAL, "cfg or out is NULL");
    *out = nullptr;
    const gdn_attn_config& c = *cfg;
    if (c.batch < 1 || c.heads < 1) return fail(GDN_E_SHAPE, "batch and heads must be >= 1");
    if (!gdn::attn_dim_supported(c.head_dim)) return fail(GDN_E_SHAPE, "head_dim %d: 64, 112 or 128", c.head_dim);
    if (c.sink_tokens < 0 || c.window_tokens < 0) return fail(GDN_E_SHAPE, "negative cache size");
    if (c.max_tokens < 1 || c.max_tokens > (1 << 30)) return fail(GDN_E_SHAPE, "max_tokens must be in [1, 2^30]");
    if (!(c.scale >= 0.f) || !std::isfinite(c.scale)) return fail(GDN_E_INVAL, "scale must be finite and >= 0");
    int64_t slots = 0;
    if (!size_product({c.batch, c.heads, (int64_t)c.sink_tokens + c.window_tokens, c.head_dim, 4}, &slots))
        return fail(GDN_E_SHAPE, "batch %d x heads %d x (sink + window) %lld: the cache size overflows", c.batch,
                    c.heads, (long long)c.sink_tokens + c.window_tokens);
    slots /= 4;
    // the kernels address a (stream, head)'s sink or window, and a chunk, with 32-bit byte offsets
    if ((int64_t)std::max(std::max(c.sink_tokens, c.window_tokens), (int32_t)std::min<int64_t>(c.max_tokens, 1 << 30)) *
            c.head_dim * 2 >= ((int64_t)1 << 31))
        return fail(GDN_E_SHAPE, "sink, window or max_tokens too large: %d x %d bf16 values exceed 2 GiB per (stream, head)",
                    std::max(c.sink_tokens, c.window_tokens), c.head_dim);
    DeviceGuard dg(device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", device, hipGetErrorString(dg.err));
    gdn_attn* a = new (std::nothrow) gdn_attn();
    if (!a) return fail(GDN_E_NOMEM, "host allocation failed");
    a->cfg = c;
    a->device = device;
    a->scale = c.scale > 0.f ? c.scale : 1.0f / std::sqrt((float)c.head_dim);
    a->cache = nullptr;
    if (slots > 0) {
        hipError_t e = hipMalloc(&a->cache, 2 * slots * sizeof(__bf16));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            delete a;
            return fail(GDN_E_NOMEM, "cache (%lld bytes): %s", (long long)(4 * slots), hipGetErrorString(e));
        }
    }
    a->sink_fill = a->win_total = 0;
    a->profile = false;
    a->acc_ms = 0.0;
    a->acc_n = 0;
    *out = a;
    return ok();
}

GDN_API int gdn_attn_destroy(gdn_attn* a) {
    if (!a) return ok();
    DeviceGuard dg(a->device);
    (void)hipDeviceSynchronize();
    if (a->cache) (void)hipFree(a->cache);
    for (auto& pr : a->pend) { (void)hipEventDestroy(pr.first); (void)hipEventDestroy(pr.second); }
    for (auto& pr : a->spare) { (void)hipEventDestroy(pr.first); (void)hipEventDestroy(pr.second); }
    delete a;
    return ok();
}

GDN_API int gdn_attn_chunk(gdn_attn* a, const gdn_attn_io* io, int64_t T, uint32_t flags, void* hip_stream) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    if (!io) return fail(GDN_E_INVAL, "io is NULL");
    if (flags & ~(uint32_t)GDN_NO_COMMIT) return fail(GDN_E_INVAL, "unknown flag bits 0x%x", flags);
    if (T < 0 || T > a->cfg.max_tokens)
        return fail(GDN_E_SHAPE, "T = %lld outside [0, max_tokens = %lld]", (long long)T, (long long)a->cfg.max_tokens);
    if (T == 0) return ok();
    const int d = a->cfg.head_dim;
    int rc;
    if ((rc = check_tensor("q", io->q, io->q_strides, 2, d, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("k", io->k, io->k_strides, 2, d, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("v", io->v, io->v_strides, 2, d, T)) != GDN_OK) return rc;
    if ((rc = check_tensor("o", io->o, io->o_strides, 2, d, T)) != GDN_OK) return rc;
    DeviceGuard dg(a->device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", a->device, hipGetErrorString(dg.err));
    hipError_t prior = hipPeekAtLastError();
    if (prior != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_E_HIP, "earlier HIP error: %s", hipGetErrorString(prior));
    }
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const gdn_attn_config& c = a->cfg;
    const int64_t per = (int64_t)c.batch * c.heads * d;
    __bf16* k_sink = a->cache;
    __bf16* v_sink = k_sink + per * c.sink_tokens;
    __bf16* k_win = v_sink + per * c.sink_tokens;
    __bf16* v_win = k_win + per * c.window_tokens;

    gdn::AttnParams p;
    std::memset(&p, 0, sizeof p);
    p.q = io->q;
    p.k = io->k;
    p.v = io->v;
    p.o = io->o;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = io->q_strides[i];
        p.ks[i] = io->k_strides[i];
        p.vs[i] = io->v_strides[i];
        p.os[i] = io->o_strides[i];
    }
    p.k_sink = k_sink;
    p.v_sink = v_sink;
    p.k_win = k_win;
    p.v_win = v_win;
    p.sink_cap = c.sink_tokens;
    p.win_cap = c.window_tokens;
    p.n_sink = (int)a->sink_fill;
    p.n_win = (int)std::min<int64_t>(a->win_total, c.window_tokens);
    p.T = (int)T;
    p.B = c.batch;
    p.H = c.heads;
    p.D = d;
    p.scale_log2 = a->scale * 1.4426950408889634f;

    std::pair<hipEvent_t, hipEvent_t> pr;
    if (a->profile) {
        if (!a->spare.empty()) {
            pr = a->spare.back();
            a->spare.pop_back();
        } else if (hipEventCreate(&pr.first) != hipSuccess || hipEventCreate(&pr.second) != hipSuccess) {
            return fail(GDN_E_HIP, "hipEventCreate failed");
        }
        (void)hipEventRecord(pr.first, st);
    }
    hipError_t e = gdn::launch_attention(p, st);
    if (a->profile) {
        (void)hipEventRecord(pr.second, st);
        a->pend.push_back(pr);
    }
    if (e != hipSuccess) return fail(GDN_E_HIP, "attention launch: %s", hipGetErrorString(e));

    if (!(flags & GDN_NO_COMMIT)) {
        const int64_t taken = std::min<int64_t>(T, c.sink_tokens - a->sink_fill);
        const int64_t rest = T - taken;
        const int64_t skip = c.window_tokens > 0 ? std::max<int64_t>(0, rest - c.window_tokens) : rest;
        if (taken + (rest - skip) > 0) {
            gdn::AppendParams ap;
            std::memset(&ap, 0, sizeof ap);
            ap.k = io->k;
            ap.v = io->v;
            for (int i = 0; i < 3; ++i) {
                ap.ks[i] = io->k_strides[i];
                ap.vs[i] = io->v_strides[i];
            }
            ap.k_sink = k_sink;
            ap.v_sink = v_sink;
            ap.k_win = k_win;
            ap.v_win = v_win;
            ap.sink_cap = c.sink_tokens;
            ap.win_cap = c.window_tokens;
            ap.T = (int)T;
            ap.B = c.batch;
            ap.H = c.heads;
            ap.D = d;
            ap.sink_fill = (int)a->sink_fill;
            ap.taken = (int)taken;
            ap.skip = (int)skip;
            ap.win_base = c.window_tokens > 0 ? (int)(a->win_total % c.window_tokens) : 0;
            e = gdn::launch_attn_append(ap, st);
            if (e != hipSuccess) return fail(GDN_E_HIP, "cache append launch: %s", hipGetErrorString(e));
        }
        a->sink_fill += taken;
        a->win_total += rest;
    }
    return ok();
}

GDN_API int gdn_attn_reset(gdn_attn* a) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    a->sink_fill = a->win_total = 0;
    return ok();
}

GDN_API int gdn_attn_cache_len(const gdn_attn* a, int64_t* sink, int64_t* window) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    if (sink) *sink = a->sink_fill;
    if (window) *window = std::min<int64_t>(a->win_total, a->cfg.window_tokens);
    return ok();
}

GDN_API int gdn_attn_cache_bytes(const gdn_attn* a, int64_t* bytes) {
    if (!a || !bytes) return fail(GDN_E_INVAL, "handle or bytes is NULL");
    *bytes = 4 * (int64_t)a->cfg.batch * a->cfg.heads * ((int64_t)a->cfg.sink_tokens + a->cfg.window_tokens) *
             a->cfg.head_dim;
    return ok();
}

GDN_API int gdn_attn_cache_get(gdn_attn* a, void* dst, int64_t* sink_len, int64_t* window_total, void* hip_stream) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    int64_t bytes = 0;
    (void)gdn_attn_cache_bytes(a, &bytes);
    if (bytes > 0 && (!dst || !aligned16(dst))) return fail(GDN_E_INVAL, "dst is NULL or not 16-byte aligned");
    DeviceGuard dg(a->device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", a->device, hipGetErrorString(dg.err));
    if (bytes > 0) {
        hipError_t e = hipMemcpyAsync(dst, a->cache, bytes, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return fail(GDN_E_HIP, "cache copy: %s", hipGetErrorString(e));
    }
    if (sink_len) *sink_len = a->sink_fill;
    if (window_total) *window_total = a->win_total;
    return ok();
}

GDN_API int gdn_attn_cache_set(gdn_attn* a, const void* src, int64_t sink_len, int64_t window_total,
                               void* hip_stream) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    if (sink_len < 0 || sink_len > a->cfg.sink_tokens || window_total < 0 ||
        (window_total > 0 && sink_len < a->cfg.sink_tokens))
        return fail(GDN_E_INVAL, "counters (sink %lld, window %lld) do not describe a cache of sink %d", (long long)sink_len,
                    (long long)window_total, a->cfg.sink_tokens);
    int64_t bytes = 0;
    (void)gdn_attn_cache_bytes(a, &bytes);
    if (bytes > 0 && (!src || !aligned16(src))) return fail(GDN_E_INVAL, "src is NULL or not 16-byte aligned");
    DeviceGuard dg(a->device);
    if (dg.err != hipSuccess) return fail(GDN_E_HIP, "hipSetDevice(%d): %s", a->device, hipGetErrorString(dg.err));
    if (bytes > 0) {
        hipError_t e = hipMemcpyAsync(a->cache, src, bytes, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return fail(GDN_E_HIP, "cache copy: %s", hipGetErrorString(e));
    }
    a->sink_fill = sink_len;
    a->win_total = window_total;
    return ok();
}

GDN_API int gdn_attn_profile(gdn_attn* a, int enable) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    a->profile = enable != 0;
    return ok();
}

GDN_API int gdn_attn_profile_read(gdn_attn* a, double* ms, int64_t* launches, int reset) {
    if (!a) return fail(GDN_E_INVAL, "handle is NULL");
    DeviceGuard dg(a->device);
    for (auto& pr : a->pend) {
        float t = 0.f;
        if (hipEventSynchronize(pr.second) == hipSuccess && hipEventElapsedTime(&t, pr.first, pr.second) == hipSuccess) {
            a->acc_ms += t;
            a->acc_n += 1;
        }
        a->spare.push_back(pr);
    }
    a->pend.clear();
    if (ms) *ms = a->acc_ms;
    if (launches) *launches = a->acc_n;
    if (reset) {
        a->acc_ms = 0.0;
        a->acc_n = 0;
    }
    return ok();
}

// ---- FP8 projection GEMMs (gdn_lowp.h) -------------------------------------------------------------

GDN_API int gdn_quantize_rows_e4m3(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t x_stride,
                                   uint8_t* codes, int64_t codes_stride, float* scales, void* hip_stream) {
    if (x_dtype != GDN_BF16 && x_dtype != GDN_F32) return fail(GDN_E_DTYPE, "x_dtype %d: GDN_BF16 or GDN_F32", x_dtype);
    if (rows < 0 || cols < 0) return fail(GDN_E_SHAPE, "negative rows or cols");
    if (rows == 0) return ok();
    if (!x || !codes || !scales) return fail(GDN_E_INVAL, "x, codes and scales must be non-NULL");
    if (x_stride < cols || codes_stride < cols) return fail(GDN_E_INVAL, "a row stride is below cols");
    const int esz = x_dtype == GDN_F32 ? 4 : 2;
    int64_t ext = 0;
    if (!size_product({rows, std::max<int64_t>(x_stride, codes_stride), esz}, &ext) || ext >= ((int64_t)1 << 40))
        return fail(GDN_E_SHAPE, "rows x stride reaches 2^40 bytes");
    gdn::QuantParams p;
    p.x = x;
    p.rows = rows;
    p.cols = cols;
    p.x_stride = x_stride;
    p.x_f32 = x_dtype == GDN_F32;
    p.codes = codes;
    p.codes_stride = codes_stride;
    p.scales = scales;
    hipError_t prior = hipPeekAtLastError();
    if (prior != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_E_HIP, "earlier HIP error: %s", hipGetErrorString(prior));
    }
    const hipError_t e = gdn::launch_quantize_rows(p, reinterpret_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : fail(GDN_E_HIP, "kernel launch: %s", hipGetErrorString(e));
}

GDN_API int gdn_gemm_e4m3(const uint8_t* x, int64_t x_stride, const float* x_scales, const uint8_t* w,
                          int64_t w_stride, const float* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                          int64_t y_stride, void* hip_stream) {
    if (M < 0 || N < 0 || K < 0) return fail(GDN_E_SHAPE, "negative M, N or K");
    if (K % 16 != 0) return fail(GDN_E_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
    if (N % 4 != 0) return fail(GDN_E_SHAPE, "N = %lld is not a multiple of 4", (long long)N);
    if (M == 0 || N == 0) return ok();
    // with K = 0 nothing of x or w is read (an empty view may carry no address)
    if ((K > 0 && (!x || !w)) || !x_scales || !w_scales || !y) return fail(GDN_E_INVAL, "a pointer is NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(w_scales) || reinterpret_cast<uintptr_t>(y) % 8)
        return fail(GDN_E_INVAL, "x, w and w_scales must be 16-byte aligned, y 8-byte aligned");
    if (x_stride < K || w_stride < K || x_stride % 16 || w_stride % 16)
        return fail(GDN_E_INVAL, "x_stride and w_stride must be multiples of 16 and >= K");
    if (y_stride < N || y_stride % 4) return fail(GDN_E_INVAL, "y_stride must be a multiple of 4 and >= N");
    const int64_t lim = (int64_t)1 << 31;
    if (M > lim || N > lim || K > lim || (M - 1) * x_stride + K >= lim || (N - 1) * w_stride + K >= lim ||
        M * y_stride >= ((int64_t)1 << 40))
        return fail(GDN_E_SHAPE, "an operand reaches the 2 GiB extent of its 32-bit offsets");
    gdn::GemmParams p;
    p.x = x;
    p.x_stride = x_stride;
    p.x_scales = x_scales;
    p.w = w;
    p.w_stride = w_stride;
    p.w_scales = w_scales;
    p.M = M;
    p.N = N;
    p.K = K;
    p.y = y;
    p.y_stride = y_stride;
    hipError_t prior = hipPeekAtLastError();
    if (prior != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_E_HIP, "earlier HIP error: %s", hipGetErrorString(prior));
    }
    const hipError_t e = gdn::launch_gemm_e4m3(p, reinterpret_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : fail(GDN_E_HIP, "kernel launch: %s", hipGetErrorString(e));
}

GDN_API const char* gdn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
