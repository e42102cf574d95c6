// Drives the C ABI's argument validation with no GPU present, for a build of the library's host
// code under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize_cpu.py).
// Every call here must be refused before any device work; the device pointers are fake and
// never dereferenced.  Exits 0 when every call returned the expected code.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "gdn_attn.h"
#include "gdn_lowp.h"
#include "gdn_stream.h"

static int failures = 0;

static void expect(const char* what, int rc, int want) {
    if (rc != want) {
        std::printf("FAIL %s: returned %d, expected %d (%s)\n", what, rc, want, gdn_last_error());
        ++failures;
    } else if (rc != GDN_OK && std::strlen(gdn_last_error()) == 0) {
        std::printf("FAIL %s: no error message\n", what);
        ++failures;
    }
}

static gdn_config config() {
    gdn_config c;
    std::memset(&c, 0, sizeof c);
    c.batch = 1;
    c.heads = 2;
    c.d_k = c.d_v = 112;
    c.max_tokens = 2640;
    c.subchunk = 0;
    c.io_dtype = GDN_BF16;
    c.flags = GDN_L2NORM_QK;
    c.l2_eps = 1e-6f;
    c.scale = 1.0f;
    return c;
}

// q, k, v, o of [1, T, 2, 112] bf16 at fake 16-byte aligned addresses
static gdn_io io_for(int64_t T) {
    gdn_io io;
    std::memset(&io, 0, sizeof io);
    const uintptr_t base = (uintptr_t)1 << 40;
    io.q = (const void*)(base);
    io.k = (const void*)(base + (1 << 24));
    io.v = (const void*)(base + (2 << 24));
    io.o = (void*)(base + (3 << 24));
    io.a = (const float*)(base + (4 << 24));
    io.beta = (const float*)(base + (5 << 24));
    const int64_t st[3] = {T * 2 * 112, 2 * 112, 112};
    const int64_t gs[3] = {T * 2, 2, 1};
    for (int i = 0; i < 3; ++i) {
        io.q_strides[i] = io.k_strides[i] = io.v_strides[i] = io.o_strides[i] = st[i];
        io.g_strides[i] = gs[i];
    }
    return io;
}

static int noalloc(const gdn_config& c, const gdn_io& io, int64_t T, const void* o_rev) {
    static int status_word = 0;
    return gdn_chunk_bidir_noalloc(&c, &io, const_cast<void*>(o_rev), T, nullptr, nullptr, &status_word, nullptr);
}

static void run_all() {
    gdn_stream* s = nullptr;
    gdn_config c = config();

    // configurations refused at init, including sizes whose products overflow int64
    gdn_config bad = c;
    bad.batch = 0;
    expect("init batch 0", gdn_stream_init(&bad, 0, &s), GDN_E_SHAPE);
    bad = c; bad.d_k = 100;
    expect("init d_k 100", gdn_stream_init(&bad, 0, &s), GDN_E_SHAPE);
    bad = c; bad.max_tokens = ((int64_t)1 << 30) + 1;
    expect("init max_tokens 2^30 + 1", gdn_stream_init(&bad, 0, &s), GDN_E_SHAPE);
    bad = c; bad.max_tokens = INT64_MAX;
    expect("init max_tokens INT64_MAX", gdn_stream_init(&bad, 0, &s), GDN_E_SHAPE);
    bad = c; bad.batch = INT32_MAX; bad.heads = INT32_MAX; bad.max_tokens = (int64_t)1 << 30;
    expect("init batch x heads overflow", gdn_stream_init(&bad, 0, &s), GDN_E_SHAPE);
    bad = c; bad.io_dtype = 9;
    expect("init io_dtype", gdn_stream_init(&bad, 0, &s), GDN_E_DTYPE);
    bad = c; bad.flags = 1u << 31;
    expect("init flags", gdn_stream_init(&bad, 0, &s), GDN_E_INVAL);
    bad = c; bad.l2_eps = -0.f - 1.f;
    expect("init eps", gdn_stream_init(&bad, 0, &s), GDN_E_INVAL);
    expect("init NULL", gdn_stream_init(nullptr, 0, &s), GDN_E_INVAL);
    // a valid configuration reaches the device query; no device here
    const int rc = gdn_stream_init(&c, 0, &s);
    if (rc == GDN_OK) {
        gdn_stream_destroy(s);
    } else {
        expect("init without a device", rc, GDN_E_HIP);
    }

    // calls on a NULL handle
    gdn_io io = io_for(64);
    expect("forward NULL handle", gdn_chunk_forward(nullptr, &io, 64, 0, nullptr, nullptr), GDN_E_INVAL);
    expect("reverse NULL handle", gdn_chunk_reverse(nullptr, &io, 64, 0, nullptr, nullptr), GDN_E_INVAL);
    expect("bidir NULL handle", gdn_chunk_bidir(nullptr, &io, nullptr, 64, 0, nullptr, nullptr), GDN_E_INVAL);
    expect("backward NULL handle", gdn_chunk_backward(nullptr, &io, nullptr, 64, 0, nullptr), GDN_E_INVAL);
    expect("backward_bidir NULL handle", gdn_chunk_backward_bidir(nullptr, &io, nullptr, nullptr, 64, nullptr), GDN_E_INVAL);
    expect("state_get NULL", gdn_state_get(nullptr, nullptr, nullptr), GDN_E_INVAL);
    expect("state_set NULL", gdn_state_set(nullptr, nullptr, nullptr), GDN_E_INVAL);
    expect("profile NULL", gdn_profile(nullptr, 1), GDN_E_INVAL);
    expect("destroy NULL", gdn_stream_destroy(nullptr), GDN_OK);

    // the allocation-free call validates everything before touching a device
    const int64_t T = 64;
    const void* o_rev = (const void*)(((uintptr_t)1 << 40) + (6 << 24));
    expect("noalloc NULL status", gdn_chunk_bidir_noalloc(&c, &io, nullptr, T, nullptr, nullptr, nullptr, nullptr),
           GDN_E_INVAL);
    expect("noalloc T > 2^30", noalloc(c, io, ((int64_t)1 << 30) + 1, o_rev), GDN_E_SHAPE);
    expect("noalloc T INT64_MAX", noalloc(c, io, INT64_MAX, o_rev), GDN_E_SHAPE);
    bad = c; bad.batch = INT32_MAX; bad.heads = INT32_MAX;
    expect("noalloc scratch overflow", noalloc(bad, io, 1 << 20, o_rev), GDN_E_SHAPE);
    bad = c; bad.io_dtype = GDN_F32;
    expect("noalloc f32", noalloc(bad, io, T, o_rev), GDN_E_DTYPE);
    gdn_io x = io;
    x.o = (void*)((uintptr_t)io.o + 2);
    expect("noalloc misaligned o", noalloc(c, x, T, o_rev), GDN_E_INVAL);
    expect("noalloc NULL o_rev", noalloc(c, io, T, nullptr), GDN_E_INVAL);
    x = io; x.k_strides[1] = -224;
    expect("noalloc negative stride", noalloc(c, x, T, o_rev), GDN_E_INVAL);
    x = io; x.q_strides[1] = 2 * 112 + 4;
    expect("noalloc stride not 16 B", noalloc(c, x, T, o_rev), GDN_E_INVAL);
    x = io; x.v_strides[1] = 64;
    expect("noalloc stride below width", noalloc(c, x, T, o_rev), GDN_E_INVAL);
    x = io; x.q_strides[1] = (int64_t)1 << 24;
    expect("noalloc extent beyond 2 GiB", noalloc(c, x, T, o_rev), GDN_E_SHAPE);
    x = io; x.q_strides[1] = INT64_MAX - 7;
    expect("noalloc stride INT64_MAX", noalloc(c, x, T, o_rev), GDN_E_SHAPE);
    x = io; x.q_strides[0] = (int64_t)1 << 62;
    expect("noalloc batch stride 2^62", noalloc(c, x, T, o_rev), GDN_E_SHAPE);
    x = io; x.g_strides[2] = -1;
    expect("noalloc negative gate stride", noalloc(c, x, T, o_rev), GDN_E_INVAL);
    x = io; x.beta = nullptr;
    expect("noalloc NULL beta", noalloc(c, x, T, o_rev), GDN_E_INVAL);

    // attention handle configurations
    gdn_attn_config ac;
    std::memset(&ac, 0, sizeof ac);
    ac.batch = 1; ac.heads = 2; ac.head_dim = 112; ac.sink_tokens = 880; ac.window_tokens = 2640;
    ac.max_tokens = 2640; ac.scale = 0.f;
    gdn_attn* a = nullptr;
    gdn_attn_config abad = ac;
    abad.head_dim = 96;
    expect("attn head_dim", gdn_attn_init(&abad, 0, &a), GDN_E_SHAPE);
    abad = ac; abad.batch = INT32_MAX; abad.heads = INT32_MAX; abad.sink_tokens = INT32_MAX;
    expect("attn cache overflow", gdn_attn_init(&abad, 0, &a), GDN_E_SHAPE);
    abad = ac; abad.sink_tokens = INT32_MAX;
    expect("attn sink extent", gdn_attn_init(&abad, 0, &a), GDN_E_SHAPE);
    abad = ac; abad.max_tokens = INT64_MAX;
    expect("attn max_tokens", gdn_attn_init(&abad, 0, &a), GDN_E_SHAPE);
    expect("attn NULL", gdn_attn_init(nullptr, 0, &a), GDN_E_INVAL);
    expect("attn chunk NULL", gdn_attn_chunk(nullptr, nullptr, 1, 0, nullptr), GDN_E_INVAL);

    // FP8 GEMM and quantisation: refused before any device work
    const uint8_t* fx = reinterpret_cast<const uint8_t*>((uintptr_t)1 << 40);
    const float* fs = reinterpret_cast<const float*>(((uintptr_t)1 << 40) + (1 << 24));
    void* fy = reinterpret_cast<void*>(((uintptr_t)1 << 40) + (2 << 24));
    expect("gemm K not a multiple of 16", gdn_gemm_e4m3(fx, 64, fs, fx, 64, fs, 8, 8, 40, fy, 8, nullptr), GDN_E_SHAPE);
    expect("gemm N not a multiple of 4", gdn_gemm_e4m3(fx, 64, fs, fx, 64, fs, 8, 6, 64, fy, 8, nullptr), GDN_E_SHAPE);
    expect("gemm NULL w", gdn_gemm_e4m3(fx, 64, fs, nullptr, 64, fs, 8, 8, 64, fy, 8, nullptr), GDN_E_INVAL);
    expect("gemm misaligned y", gdn_gemm_e4m3(fx, 64, fs, fx, 64, fs, 8, 8, 64, (char*)fy + 2, 8, nullptr), GDN_E_INVAL);
    expect("gemm stride below K", gdn_gemm_e4m3(fx, 48, fs, fx, 64, fs, 8, 8, 64, fy, 8, nullptr), GDN_E_INVAL);
    expect("gemm extent", gdn_gemm_e4m3(fx, (int64_t)1 << 20, fs, fx, 64, fs, 1 << 12, 8, 64, fy, 8, nullptr), GDN_E_SHAPE);
    expect("gemm huge sizes", gdn_gemm_e4m3(fx, 64, fs, fx, 64, fs, INT64_MAX, 8, 64, fy, 8, nullptr), GDN_E_SHAPE);
    expect("gemm y_stride not a multiple of 4", gdn_gemm_e4m3(fx, 64, fs, fx, 64, fs, 8, 8, 64, fy, 10, nullptr), GDN_E_INVAL);
    expect("gemm NULL x with K > 0", gdn_gemm_e4m3(nullptr, 64, fs, fx, 64, fs, 8, 8, 64, fy, 8, nullptr), GDN_E_INVAL);
    expect("gemm empty", gdn_gemm_e4m3(nullptr, 0, nullptr, nullptr, 0, nullptr, 0, 8, 64, nullptr, 8, nullptr), GDN_OK);
    expect("quantize dtype", gdn_quantize_rows_e4m3(fx, 7, 4, 64, 64, (uint8_t*)fy, 64, (float*)fs, nullptr), GDN_E_DTYPE);
    expect("quantize NULL", gdn_quantize_rows_e4m3(nullptr, GDN_BF16, 4, 64, 64, (uint8_t*)fy, 64, (float*)fs, nullptr), GDN_E_INVAL);
    expect("quantize stride", gdn_quantize_rows_e4m3(fx, GDN_BF16, 4, 64, 32, (uint8_t*)fy, 64, (float*)fs, nullptr), GDN_E_INVAL);
    expect("quantize overflow", gdn_quantize_rows_e4m3(fx, GDN_BF16, INT64_MAX / 2, 64, 64, (uint8_t*)fy, 64, (float*)fs, nullptr), GDN_E_SHAPE);
}

int main() {
    run_all();
    // the error message is per thread: run the same checks on several threads at once
    std::vector<std::thread> th;
    for (int i = 0; i < 4; ++i) th.emplace_back(run_all);
    for (auto& t : th) t.join();
    std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
