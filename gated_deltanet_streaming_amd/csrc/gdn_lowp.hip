// FP8 (OCP E4M3) projection GEMMs of the GDN block on gfx950: per-row quantisation and a GEMM on the
// v_mfma_scale_f32_16x16x128_f8f6f4 matrix cores.  Behind include/gdn_lowp.h.
//
// The pages run the block's projections in mixed precision (the Chinese summary, "Results", Table 2 and
// Figure 6; the Korean review, section 1 "Key Terms", MPQ) without printing the formats or the scaling
// policy.  Here: E4M3 codes with one float32 scale per row of the activations (per token) and per row of
// the weights (per output feature), s = amax / 448, code = E4M3(x * (448 / amax)) rounded to nearest even and
// saturated at 448; C[m][n] = s_x[m] s_w[n] sum_k E4M3^-1(X[m][k]) E4M3^-1(W[n][k]), accumulated in fp32
// (every product of two E4M3 values is exact in fp32), stored as bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// raw buffer resource over [base, base + bytes); loads beyond it return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// E4M3 code of a float32 value, rounding to nearest with ties to even and saturating at +-448.  Magnitudes
// below 2^-6 are e4m3 subnormals m 2^-9 (m = the integer nearest to |y| 2^9, which is exact in fp32); above,
// the fp32 mantissa is rounded to 3 bits in integer arithmetic, a carry moving to the next binade.
__device__ __forceinline__ unsigned e4m3_code(float y) {
    const unsigned u = __float_as_uint(y);
    const unsigned sign = (u >> 24) & 0x80u;
    const float a = fabsf(y);
    unsigned code;
    if (!(a < 448.f)) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {   // 2^-6
        code = (unsigned)__builtin_rintf(a * 512.f);   // 0 .. 8 (8 is the smallest normal, code 0x08)
    } else {
        const unsigned au = __float_as_uint(a);
        const int e = (int)((au >> 23) & 0xFFu) - 127;   // -6 .. 8
        const unsigned m23 = au & 0x7FFFFFu;
        unsigned q = m23 >> 20;
        const unsigned rem = m23 & 0xFFFFFu;
        q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
        code = ((unsigned)(e + 7) << 3) + q;   // q == 8 carries into the exponent field
    }
    return code == 0 ? 0u : (code | sign);
}

// sum and max over the 64 lanes
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// One wavefront per row: amax, scale, codes.  General form (any alignment and width): the row is read twice
// (the second pass from L2), one element per lane per load.
template <bool F32>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;
    const char* xr = static_cast<const char*>(p.x) + row * p.x_stride * (F32 ? 4 : 2);
    auto elem = [&](int64_t c) -> float {
        if constexpr (F32) return reinterpret_cast<const float*>(xr)[c];
        else return __uint_as_float((unsigned)reinterpret_cast<const unsigned short*>(xr)[c] << 16);
    };
    float amax = 0.f;
    for (int64_t c = lane; c < p.cols; c += 64) amax = fmaxf(amax, fabsf(elem(c)));
    amax = wave_max(amax);
    if (lane == 0) p.scales[row] = amax / 448.f;
    const float r = amax > 0.f ? 448.f / amax : 0.f;   // codes of a zero row: e4m3_code(0) = 0
    unsigned char* qr = p.codes + row * p.codes_stride;
    for (int64_t c = lane; c < p.cols; c += 64) qr[c] = (unsigned char)e4m3_code(elem(c) * r);
}

// Vector form for rows of at most 64 x 8 x QV elements in groups of 8 (16-byte aligned input rows, 8-byte
// aligned code rows): lane l holds groups l, l + 64, ... in registers, so the row is read from memory once;
// each group of 8 codes leaves as one 8-byte store.  The same e4m3_code of the same float32 quotient as the
// general form, so the two produce identical codes.
constexpr int QV = 8;
template <bool F32>
__global__ __launch_bounds__(256) void quantize_rows_vec_kernel(QuantParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;
    const int ng = (int)(p.cols >> 3);
    float v[QV][8];
    const char* xr = static_cast<const char*>(p.x) + row * p.x_stride * (F32 ? 4 : 2);
#pragma unroll
    for (int j = 0; j < QV; ++j) {
        const int g = lane + 64 * j;
        if (g < ng) {
            if constexpr (F32) {
                const float4 a = reinterpret_cast<const float4*>(xr)[2 * g];
                const float4 b = reinterpret_cast<const float4*>(xr)[2 * g + 1];
                v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
                v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
            } else {
                const uint4 a = reinterpret_cast<const uint4*>(xr)[g];
                const unsigned w4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[j][2 * i] = __uint_as_float(w4[i] << 16);
                    v[j][2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < QV; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
    amax = wave_max(amax);
    if (lane == 0) p.scales[row] = amax / 448.f;
    const float r = amax > 0.f ? 448.f / amax : 0.f;
    uint2* qr = reinterpret_cast<uint2*>(p.codes + row * p.codes_stride);
#pragma unroll
    for (int j = 0; j < QV; ++j) {
        const int g = lane + 64 * j;
        if (g < ng) {
            unsigned c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = e4m3_code(v[j][i] * r);
            qr[g] = uint2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM.  Workgroup tile: TN output features (rows of W) x TM tokens (rows of X); NW wavefronts (8: two per
// SIMD) in an NW / 2 x 2 grid, each TN / (NW / 2) features x TM / 2 tokens.  K steps of 128 bytes.  Operands
// travel through staging registers (16-byte buffer loads issued one step ahead) into a double-buffered LDS
// tile, and from LDS into the MFMA operand registers.  (The buffer loads that write LDS directly move about 16
// bytes per clock per CU on this chip, a quarter of what ordinary loads reach, so the data takes the register
// path.)  Loads past the end of a row or of K read zero through the buffer resource's range check.
// MFMA operands (16x16x128, E4M3, unit scales): lane l holds row l % 16 of the 16-row block and the 32
// consecutive k values 32 (l / 16) .. +31 (W as the A operand, X as the B operand); the output lane l holds
// D[feature 4 (l / 16) + i][token l % 16], four consecutive features of one token (one 8-byte bf16 store).
// Loads: lane l of a load instruction takes 16-byte chunk l % 8 (k bytes 16 (l % 8) .. +15 of the step) of row
// l / 8 of the instruction's 8 rows, so that 8 lanes read one row's 128 contiguous bytes.
// LDS layout, k-major within blocks of 16 rows with the row index XOR-ed by the chunk: chunk c of row r sits at
// byte (r / 16) 2048 + c 256 + ((r % 16) ^ c) 16.  Measured on this chip, a 16-byte LDS read is free of bank
// conflicts when each group of 16 consecutive lanes covers one aligned 256-byte run (in any order), and a
// 16-byte write when the 8 lanes of each group of 8 fall on 8 different 16-byte bank groups modulo 128 bytes.
// An MFMA operand read (16 rows, one chunk) covers the aligned run of its chunk, and the 8 lanes writing one
// row's 8 chunks land on bank groups (r % 8) ^ c, all different.  The step loop is unrolled only over the
// register groups (compile-time indices into the register array); the stage is a run-time offset.
// Tile order: workgroup id % 8 is its XCD, and XCD x takes a contiguous range of the tile sequence, which runs
// in bands of BH token tiles (band outer, feature tile, token tile in the band inner).  The 32 workgroups that
// an XCD runs at once then share a few W tiles and one band of X, and the band stays in the XCD's L2 while
// the XCD moves along the feature tiles.
// ---------------------------------------------------------------------------
constexpr int GK = 128;                  // k per step, bytes
constexpr int OUT = (int)0x80000000;     // an offset beyond every buffer resource: the load reads zero

typedef int v4i __attribute__((ext_vector_type(4)));

template <int TN, int TM, int NW>
struct GemmShape {
    static constexpr int WN = NW / 2;                        // wavefronts along the features (2 along the tokens)
    static constexpr int FN = TN / WN;                       // features per wavefront
    static constexpr int FA = FN / 16;                       // 16-feature blocks per wavefront
    static constexpr int TB = TM / 32;                       // 16-token blocks per wavefront
    static constexpr int ROWS = TN + TM;                     // LDS rows of one stage: W rows, then X rows
    static constexpr int STAGE = ROWS * GK;                  // bytes
    static constexpr int NJ = ROWS / 8 / NW;                 // 16-byte loads per lane and step
    static_assert((NW == 4 || NW == 8) && FN % 16 == 0 && TM % 32 == 0 && (ROWS / 8) % NW == 0, "tile shape");
};

// Workgroup barrier for LDS hand-offs: this wavefront's LDS writes complete (lgkmcnt(0)), then s_barrier
// without the memory fence of __syncthreads (which would also wait for the loads in flight); the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}



template <int TN, int TM, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_e4m3_kernel(GemmParams p, int bh) {
    using G = GemmShape<TN, TM, NW>;
    constexpr int NJ = G::NJ;
    __shared__ __align__(16) unsigned char lds[2 * G::STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int ntn = (int)((p.N + TN - 1) / TN), ntm = (int)((p.M + TM - 1) / TM);
    const int ntiles = ntn * ntm;
    const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
    const int per = (ntiles + 7) / 8;
    const int seq = xcd * per + k8;
    if (k8 >= per || seq >= ntiles) return;
    const int band = seq / (ntn * bh);
    const int hb = min(bh, ntm - band * bh);
    const int r = seq - band * ntn * bh;
    const int tn = r / hb, tm = band * bh + (r - (r / hb) * hb);
    const int64_t n0 = (int64_t)tn * TN, m0 = (int64_t)tm * TM;

    const auto wrs = rsrc(p.w, (p.N - 1) * p.w_stride + p.K);
    const auto xrs = rsrc(p.x, (p.M - 1) * p.x_stride + p.K);
    // load j of a lane: stage row 8 i + lane / 8 with i = NJ wave + j (rows 0 .. TN - 1 are W, the rest X; all
    // rows of one i are in the same operand since TN is a multiple of 8), chunk lane % 8 of the step's k slice
    int src_off[NJ], lds_off[NJ];
    const int chunk = lane & 7, pos16 = 16 * chunk;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int i = NJ * wave + j;
        const int row = 8 * i + (lane >> 3);
        const bool isw = 8 * i < TN;
        const int64_t grow = isw ? n0 + row : m0 + (row - TN);
        src_off[j] = grow < (isw ? p.N : p.M) ? (int)(grow * (isw ? p.w_stride : p.x_stride)) : OUT;
        lds_off[j] = (row >> 4) * 2048 + chunk * 256 + (((row & 15) ^ chunk) * 16);
    }
    const int ksz = (int)p.K;
    const int nk = (ksz + GK - 1) / GK;
    v4i rg[NJ];
    auto load = [&](int ks) {
        const int kk = ks * GK + pos16;   // K is a multiple of 16: a 16-byte piece is all in or all out
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int voff = (src_off[j] == OUT || kk >= ksz) ? OUT : src_off[j] + kk;
            rg[j] = __builtin_amdgcn_raw_buffer_load_b128(8 * (NJ * wave + j) < TN ? wrs : xrs, voff, 0, 0);
        }
    };
    auto stage = [&](int ks) { return lds + (ks & 1) * G::STAGE; };
    auto store = [&](unsigned char* st) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) *reinterpret_cast<v4i*>(st + lds_off[j]) = rg[j];
    };

    f32x4 acc[G::FA][G::TB];
#pragma unroll
    for (int a = 0; a < G::FA; ++a)
#pragma unroll
        for (int b = 0; b < G::TB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wn = wave % G::WN, wm = wave / G::WN;
    // operand reads: row block (first row / 16), chunks 2 grp and 2 grp + 1, row r16 within the block
    const int c0 = (2 * grp) * 256 + 16 * (r16 ^ (2 * grp)), c1 = (2 * grp + 1) * 256 + 16 * (r16 ^ (2 * grp + 1));
    const int arow = (wn * G::FN / 16) * 2048, brow = ((TN + (TM / 2) * wm) / 16) * 2048;

    // Step ks reads stage ks % 2.  On entry the staging registers hold step ks + 1 (loaded during step ks - 1);
    // the step writes them to the other stage, whose previous contents every wavefront has read (the barrier),
    // and loads step ks + 2 into them.  Past the last step the loads read zero and are never read from LDS.
    // (Measured alternatives: two staging groups, and a second set of operand registers so that the LDS reads
    // of step ks + 1 overlap the MFMAs of step ks, were not faster.)
    auto step = [&](int ks) {
        lds_barrier();                    // stage ks % 2 is written by every wavefront; the other is read by none
        const unsigned char* cur = stage(ks);
        v8i af[G::FA], bf[G::TB];
#pragma unroll
        for (int f = 0; f < G::FA; ++f) {
            const uint4 lo = *reinterpret_cast<const uint4*>(cur + arow + 2048 * f + c0);
            const uint4 hi = *reinterpret_cast<const uint4*>(cur + arow + 2048 * f + c1);
            af[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int t = 0; t < G::TB; ++t) {
            const uint4 lo = *reinterpret_cast<const uint4*>(cur + brow + 2048 * t + c0);
            const uint4 hi = *reinterpret_cast<const uint4*>(cur + brow + 2048 * t + c1);
            bf[t] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        store(stage(ks + 1));             // step ks + 1 into the other stage
        load(ks + 2);                     // step ks + 2 into the registers just written out
#pragma unroll
        for (int f = 0; f < G::FA; ++f)
#pragma unroll
            for (int t = 0; t < G::TB; ++t)
                acc[f][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[f], bf[t], acc[f][t], 0, 0, 0, 127, 0, 127);
    };
    if (nk > 0) {
        load(0);
        store(stage(0));
        load(1);
        for (int ks = 0; ks < nk; ++ks) step(ks);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loads past the last step have returned
    }

    // epilogue: C[token][features 4 grp + i] = s_x s_w acc, bf16, 8 bytes per lane and tile
#pragma unroll
    for (int t = 0; t < G::TB; ++t) {
        const int64_t m = m0 + (TM / 2) * wm + 16 * t + r16;
        if (m >= p.M) continue;
        const float sx = p.x_scales[m];
        unsigned short* yr = static_cast<unsigned short*>(p.y) + m * p.y_stride;
#pragma unroll
        for (int f = 0; f < G::FA; ++f) {
            const int64_t n = n0 + wn * G::FN + 16 * f + 4 * grp;
            if (n >= p.N) continue;
            const f32x4 ws = *reinterpret_cast<const f32x4*>(p.w_scales + n);
            unsigned short h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned u = __float_as_uint(acc[f][t][i] * sx * ws[i]);
                h[i] = (unsigned short)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // round to nearest even
            }
            *reinterpret_cast<uint2*>(yr + n) = uint2{(unsigned)h[0] | ((unsigned)h[1] << 16), (unsigned)h[2] | ((unsigned)h[3] << 16)};
        }
    }
}

}  // namespace

hipError_t launch_quantize_rows(const QuantParams& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((p.rows + 3) / 4);
    const int es = p.x_f32 ? 4 : 2;
    const bool vec = p.cols % 8 == 0 && p.cols <= 64 * 8 * QV && reinterpret_cast<uintptr_t>(p.x) % 16 == 0 &&
                     (p.x_stride * es) % 16 == 0 && reinterpret_cast<uintptr_t>(p.codes) % 8 == 0 &&
                     p.codes_stride % 8 == 0;
    if (vec) {
        if (p.x_f32) hipLaunchKernelGGL(quantize_rows_vec_kernel<true>, dim3(grid), dim3(256), 0, s, p);
        else hipLaunchKernelGGL(quantize_rows_vec_kernel<false>, dim3(grid), dim3(256), 0, s, p);
    } else {
        if (p.x_f32) hipLaunchKernelGGL(quantize_rows_kernel<true>, dim3(grid), dim3(256), 0, s, p);
        else hipLaunchKernelGGL(quantize_rows_kernel<false>, dim3(grid), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

namespace {
int compute_units() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int TN, int TM, int NW>
void launch_cfg(const GemmParams& p, int bh, hipStream_t s) {
    const int64_t ntiles = ((p.N + TN - 1) / TN) * ((p.M + TM - 1) / TM);
    const int64_t per = (ntiles + 7) / 8;
    hipLaunchKernelGGL((gemm_e4m3_kernel<TN, TM, NW>), dim3((unsigned)(8 * per)), dim3(64 * NW), 0, s, p, bh);
}

// The tiles the host chooses from, all with 8 wavefronts (measured at the 720p
// projection, 2640 x 6720 x 2240: 192 x 128 55-60 us, 192 x 192 57-63 us, 256 x 128 74 us; 4 wavefronts of
// 96 x 96 at 192 x 192 79 us).
struct GemmCfg { int tn, tm; };
constexpr GemmCfg kGemmCfgs[] = {{192, 128}, {192, 192}, {256, 128}, {128, 128}};
}  // namespace

int gemm_e4m3_tile_features(int64_t M, int64_t N, int cus) {
    // one workgroup per CU: the tile whose rounds of cus workgroups cost the least, rounds x TN x TM, the
    // earlier (larger) tile of the list on a tie
    int best = 0;
    int64_t best_cost = INT64_MAX;
    for (int c = 0; c < (int)(sizeof(kGemmCfgs) / sizeof(kGemmCfgs[0])); ++c) {
        const int64_t tiles = ((N + kGemmCfgs[c].tn - 1) / kGemmCfgs[c].tn) * ((M + kGemmCfgs[c].tm - 1) / kGemmCfgs[c].tm);
        const int64_t cost = (tiles + cus - 1) / cus * kGemmCfgs[c].tn * kGemmCfgs[c].tm;
        if (cost < best_cost) best = c, best_cost = cost;
    }
    return best;
}

hipError_t launch_gemm_e4m3(const GemmParams& p, hipStream_t s) {
    if (p.M <= 0 || p.N <= 0) return hipSuccess;
    const int c = gemm_e4m3_tile_features(p.M, p.N, compute_units());
    const int bh = 8;   // token tiles per band
    switch (c) {
        case 0: launch_cfg<192, 128, 8>(p, bh, s); break;
        case 1: launch_cfg<192, 192, 8>(p, bh, s); break;
        case 2: launch_cfg<256, 128, 8>(p, bh, s); break;
        default: launch_cfg<128, 128, 8>(p, bh, s); break;
    }
    return hipGetLastError();
}

}  // namespace gdn
