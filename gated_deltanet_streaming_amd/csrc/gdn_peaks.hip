// Measured machine peaks for the roofline of the GDN kernels on MI355X (gfx950):
// a device-to-device copy (HBM read + write bandwidth), dense bf16 and fp8 MFMA loops, and the
// LDS read rate of 16-byte reads.
// The vendor figures (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16) are what the roofline
// fractions are quoted against; these probes state what this machine reaches with
// plain kernels, beside them.  Measurement support only: no part of the GDN path
// calls into this library.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte vectors.  Two forms: a grid-stride loop over a fixed grid, and one vector per thread.
__global__ __launch_bounds__(256) void copy_stride_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}
__global__ __launch_bounds__(256) void copy_flat_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// Every wavefront keeps 8 independent accumulation chains of 16x16x32 bf16 MFMAs busy.
constexpr int MFMA_CHAINS = 8;
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* out) {
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
        b[e] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + e) & 7));
    }
    f32x4 acc[MFMA_CHAINS];
    for (int c = 0; c < MFMA_CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < MFMA_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
    for (int c = 0; c < MFMA_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Dense fp8 (E4M3) MFMA: every wavefront keeps 8 independent chains of 16x16x128 MFMAs busy.
typedef int v8i __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256) void mfma_fp8_kernel(int iters, float* out) {
    v8i a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = 0x30303030 + ((threadIdx.x + e) & 7);   // small E4M3 values
        b[e] = 0x28282828 + ((threadIdx.x * 3 + e) & 7);
    }
    f32x4 acc[MFMA_CHAINS];
    for (int c = 0; c < MFMA_CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < MFMA_CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
    float s = 0.f;
    for (int c = 0; c < MFMA_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS read rate: 8 wavefronts per workgroup, each issuing 16-byte reads whose 64 lanes cover 1 KB contiguous
// (free of bank conflicts), 16 per iteration over 16 slices of 2 KB.
typedef int v4i __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(512) void lds_read_kernel(int iters, int* out) {
    __shared__ __align__(16) v4i lds[2048];   // 32 KB
    for (int i = threadIdx.x; i < 2048; i += 512) lds[i] = v4i{i, (int)threadIdx.x, 1, 2};
    __syncthreads();
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    int acc = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const v4i v = lds[128 * ((u + w + it) & 15) + l];   // the address changes with it: no load is hoisted
            acc ^= v.x ^ v.w;
        }
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

int timed(hipStream_t s, int reps, float* ms, void (*launch)(hipStream_t, void*), void* arg) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -1;
    if (hipEventCreate(&e1) != hipSuccess) return -1;
    launch(s, arg);   // warm-up
    hipEventRecord(e0, s);
    for (int r = 0; r < reps; ++r) launch(s, arg);
    hipEventRecord(e1, s);
    const hipError_t err = hipEventSynchronize(e1);
    float t = 0.f;
    hipEventElapsedTime(&t, e0, e1);
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    *ms = t / (float)reps;
    return err == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

struct CopyArgs { const uint4* src; uint4* dst; int64_t n; int form; };
struct MfmaArgs { int blocks, iters; float* out; };
struct LdsArgs { int blocks, iters; int* out; };

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16, 16-byte aligned device buffers, at most 2^40 bytes)
// `reps` times on `stream` and returns the average milliseconds per copy in *ms.  form 0: a
// grid-stride loop over 8192 workgroups; form 1: one 16-byte vector per thread.  0 on success,
// -1 on bad arguments or a HIP error.
__attribute__((visibility("default"))) int gdn_peak_copy(const void* src, void* dst, int64_t bytes, int reps, int form,
                                                         void* stream, float* ms) {
    if (!src || !dst || !ms || bytes <= 0 || bytes % 16 || bytes > ((int64_t)1 << 40) || reps <= 0) return -1;
    if (form != 0 && form != 1) return -1;
    CopyArgs a{static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16, form};
    return timed(static_cast<hipStream_t>(stream), reps, ms, [](hipStream_t s, void* p) {
        const CopyArgs& c = *static_cast<CopyArgs*>(p);
        if (c.form == 0)
            hipLaunchKernelGGL(copy_stride_kernel, dim3(8192), dim3(256), 0, s, c.src, c.dst, c.n);
        else
            hipLaunchKernelGGL(copy_flat_kernel, dim3((unsigned)((c.n + 255) / 256)), dim3(256), 0, s, c.src, c.dst, c.n);
    }, &a);
}

// Runs `blocks` workgroups of 4 wavefronts, each wavefront issuing `iters` x 8 dependent-free
// 16x16x32 bf16 MFMAs, `reps` times; returns the average milliseconds per launch in *ms and
// the flops of one launch in *flops.  `out` is device scratch of blocks * 256 floats.
__attribute__((visibility("default"))) int gdn_peak_mfma_bf16(int blocks, int iters, int reps, float* out, void* stream,
                                                              float* ms, double* flops) {
    if (blocks <= 0 || iters <= 0 || reps <= 0 || !out || !ms || !flops) return -1;
    MfmaArgs a{blocks, iters, out};
    *flops = (double)blocks * 4 * iters * MFMA_CHAINS * (2.0 * 16 * 16 * 32);
    return timed(static_cast<hipStream_t>(stream), reps, ms, [](hipStream_t s, void* p) {
        const MfmaArgs& m = *static_cast<MfmaArgs*>(p);
        hipLaunchKernelGGL(mfma_kernel, dim3(m.blocks), dim3(256), 0, s, m.iters, m.out);
    }, &a);
}

// As gdn_peak_mfma_bf16 with 16x16x128 fp8 (E4M3) MFMAs (unit scales).
__attribute__((visibility("default"))) int gdn_peak_mfma_fp8(int blocks, int iters, int reps, float* out, void* stream,
                                                             float* ms, double* flops) {
    if (blocks <= 0 || iters <= 0 || reps <= 0 || !out || !ms || !flops) return -1;
    MfmaArgs a{blocks, iters, out};
    *flops = (double)blocks * 4 * iters * MFMA_CHAINS * (2.0 * 16 * 16 * 128);
    return timed(static_cast<hipStream_t>(stream), reps, ms, [](hipStream_t s, void* p) {
        const MfmaArgs& m = *static_cast<MfmaArgs*>(p);
        hipLaunchKernelGGL(mfma_fp8_kernel, dim3(m.blocks), dim3(256), 0, s, m.iters, m.out);
    }, &a);
}

// Runs `blocks` workgroups of 8 wavefronts, each wavefront issuing `iters` x 16 LDS reads of 16 bytes per lane,
// `reps` times; returns the average milliseconds per launch in *ms and the bytes read from LDS in one launch in
// *bytes.  `out` is device scratch of blocks * 512 ints.
__attribute__((visibility("default"))) int gdn_peak_lds_read(int blocks, int iters, int reps, int* out, void* stream,
                                                             float* ms, double* bytes) {
    if (blocks <= 0 || iters <= 0 || reps <= 0 || !out || !ms || !bytes) return -1;
    LdsArgs a{blocks, iters, out};
    *bytes = (double)blocks * 8 * iters * 16 * 64 * 16;
    return timed(static_cast<hipStream_t>(stream), reps, ms, [](hipStream_t s, void* p) {
        const LdsArgs& m = *static_cast<LdsArgs*>(p);
        hipLaunchKernelGGL(lds_read_kernel, dim3(m.blocks), dim3(512), 0, s, m.iters, m.out);
    }, &a);
}

}  // extern "C"
