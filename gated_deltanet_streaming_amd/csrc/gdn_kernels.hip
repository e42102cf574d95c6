// gdn_kernels.hip -- gfx950 (CDNA4) kernels of the Gated DeltaNet streaming core.
//
// Per stream b and head h the state S (d_v x d_k, fp32) follows the gated delta
// rule S_t = a_t S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T and
// o_t = scale * S_t q^_t (Gated DeltaNet, named on the SANA-Streaming pages:
// Korean review section 1; the streaming forward scan with a carried cache plus
// the backward scan inside a chunk: Chinese summary, "Method steps" step 2).
//
// Two paths:
//  * gdn_seq_kernel -- token-sequential fp32 recurrence, one 64-lane workgroup
//    per (direction, stream, head, 16 state rows).  Plain and exact; the anchor.
//  * chunked path -- the pages' fused kernel works in stages (frame summaries,
//    recurrent scan, apply state; Chinese summary "Method steps" step 4).  Here:
//      gdn_prep_kernel  (parallel over sub-chunks of C tokens): per-token L2
//        norms, in-chunk log-gate prefix g, the Gram products K K^T and Q K^T on
//        bf16 MFMA, the decay-masked in-chunk attention A, and the UT transform
//        T = (I + L)^{-1} with L[t,s] = beta_t e^{g_t-g_s} k^_t.k^_s (s < t).
//      gdn_scan_kernel  (serial over sub-chunks): one wavefront owns 16 rows of
//        one head's state, kept in MFMA accumulators for the whole call, and per
//        sub-chunk computes  X = K S^T, U = T (diag(beta) V - diag(beta e^g) X),
//        O = diag(e^g) Q S^T + A U,  S <- e^{g_C} S + U^T diag(e^{g_C-g}) K^.
//    The raw bf16 q/k enter the MFMAs unrounded (norms are applied as row
//    scales); the bounded in-chunk operands T, A, R, U, K^ use fp16 (11-bit
//    significand), the state enters its two products as bf16, everything
//    accumulates in fp32.
//
// MFMA lane layouts (16x16 output tiles, 64 lanes, l = lane, g = l / 16):
//   A operand: lane l holds row l % 16 and the k-slots of group g;
//   B operand: lane l holds column l % 16 and the k-slots of group g;
//   output:    lane l holds column l % 16, rows 4g .. 4g+3.
// An output tile is therefore directly a B operand of the next product when
// its row index becomes the contraction index: slot i of group g stands for
// k = 16 * (i / 4) + 4g + (i % 4) within a 32-wide step (two output tiles), and
// every operand built from memory uses the same slot -> k assignment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// decays below e^-80 are treated as e^-80 (the state is forgotten either way)
#define GDN_MIN_LOG_DECAY (-80.0f)

__device__ __forceinline__ f32x4 mma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A trailing 16-wide k-step is issued as a 32-wide MFMA with zero upper slots in
// both operands (same result).  The 16x16x16 variants are avoided on gfx950:
// with them, accumulator reads that follow after the compiler's wait states
// returned incomplete rows (rows 4g and 4g+1 of the tile).
__device__ __forceinline__ f32x4 mma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8{a[0], a[1], a[2], a[3], z[0], z[1], z[2], z[3]},
                                                   bf16x8{b[0], b[1], b[2], b[3], z[0], z[1], z[2], z[3]}, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
    const f16 z = (f16)0.f;
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(f16x8{a[0], a[1], a[2], a[3], z, z, z, z},
                                                  f16x8{b[0], b[1], b[2], b[3], z, z, z, z}, c, 0, 0, 0);
}

// Keeps a value in its registers up to this point.  An MFMA may start executing
// well after it is issued (behind earlier MFMAs), so the registers holding its
// A/B operands must not be refilled by a short-latency load (LDS) until the
// MFMA has finished; operands loaded from LDS are therefore kept alive until
// the results that depend on them have been consumed.
template <typename T>
__device__ __forceinline__ void keep_alive(const T& x) {
    asm volatile("" ::"v"(x));
}

__device__ __forceinline__ bf16x4 ld_bf16x4(const bf16* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Sub-chunk block bookkeeping for the lower-triangular C x C operands (T, A)
// stored as MFMA A-operand fragments: row tile mt needs the 32-wide k-steps that
// reach its diagonal, plus the trailing 16-wide step when C is an odd multiple of 16.
template <int NB>
struct Blocks {
    static constexpr int NFULL = NB / 2;
    static constexpr bool HALF = (NB % 2) != 0;
    __host__ __device__ static constexpr int nfull_for(int mt) {
        return (mt / 2 + 1) < NFULL ? (mt / 2 + 1) : NFULL;
    }
    __host__ __device__ static constexpr int count(int mt) {
        return nfull_for(mt) + ((HALF && mt == NB - 1) ? 1 : 0);
    }
    __host__ __device__ static constexpr int offset(int mt) {
        int s = 0;
        for (int m = 0; m < mt; ++m) s += count(m);
        return s;
    }
    static constexpr int TOTAL = offset(NB);
};

// workspace item: [T fragments][A fragments][scalars 5*C][gamma_C], 1 KB per fragment block
template <int NB>
__host__ __device__ constexpr int64_t item_bytes_t() {
    int64_t b = 2 * 1024 * (int64_t)Blocks<NB>::TOTAL + 4 * (5 * 16 * NB + 4);
    return (b + 255) / 256 * 256;
}

int64_t chunk_item_bytes(int C) {
    switch (C) {
        case 16: return item_bytes_t<1>();
        case 32: return item_bytes_t<2>();
        case 64: return item_bytes_t<4>();
        default: return -1;
    }
}

// ---------------------------------------------------------------------------
// Token-sequential fp32 kernel.  Lane l owns state row 16*rb + l/4 and the
// columns c = l%4 + 4i; row sums are reduced across the 4 lanes of a row.
// ---------------------------------------------------------------------------
template <bool F32>
__device__ __forceinline__ float ld_elem(const void* base, int64_t idx) {
    if constexpr (F32) return reinterpret_cast<const float*>(base)[idx];
    else return (float)reinterpret_cast<const bf16*>(base)[idx];
}
template <bool F32>
__device__ __forceinline__ void st_elem(void* base, int64_t idx, float v) {
    if constexpr (F32) reinterpret_cast<float*>(base)[idx] = v;
    else reinterpret_cast<bf16*>(base)[idx] = (bf16)v;
}

__device__ __forceinline__ float sum4(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x;
}

template <bool F32>
__global__ __launch_bounds__(64) void gdn_seq_kernel(Params p) {
    constexpr int MAXC = 32;  // d_k <= 128
    const int lane = threadIdx.x, part = lane & 3;
    const int nrb = p.Dv / 16;
    int id = blockIdx.x;
    const int rb = id % nrb; id /= nrb;
    const int h = id % p.H; id /= p.H;
    const int b = id % p.B; id /= p.B;
    const int dir = p.dir0 + id;
    const int row = 16 * rb + (lane >> 2);
    const int nc = p.Dk / 4;
    const int64_t T = p.T;

    float S[MAXC];
    const float* Sin = (dir == 0) ? p.S_in : nullptr;
    const int64_t srow = (((int64_t)b * p.H + h) * p.Dv + row) * p.Dk;
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
        S[i] = (i < nc && Sin) ? Sin[srow + part + 4 * i] : 0.f;

    for (int64_t step = 0; step < T; ++step) {
        const int64_t t = dir ? (T - 1 - step) : step;
        const int64_t kq = (int64_t)b * p.ks[0] + t * p.ks[1] + (int64_t)h * p.ks[2];
        const int64_t qq = (int64_t)b * p.qs[0] + t * p.qs[1] + (int64_t)h * p.qs[2];
        const int64_t vq = (int64_t)b * p.vs[0] + t * p.vs[1] + (int64_t)h * p.vs[2];
        const int64_t oq = (int64_t)b * p.os[0] + t * p.os[1] + (int64_t)h * p.os[2];
        const int64_t gq = (int64_t)b * p.gs[0] + t * p.gs[1] + (int64_t)h * p.gs[2];
        float kv[MAXC], qv[MAXC];
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            kv[i] = (i < nc) ? ld_elem<F32>(p.k, kq + part + 4 * i) : 0.f;
            qv[i] = (i < nc) ? ld_elem<F32>(p.q, qq + part + 4 * i) : 0.f;
            sk += kv[i] * kv[i];
            sq += qv[i] * qv[i];
        }
        const float at = p.a[gq], bt = p.beta[gq];
        const float vr = ld_elem<F32>(p.v, vq + row);
        if (p.l2norm) {
            const float rk = 1.f / sqrtf(sum4(sk) + p.eps);
            const float rq = 1.f / sqrtf(sum4(sq) + p.eps);
#pragma unroll
            for (int i = 0; i < MAXC; ++i) { kv[i] *= rk; qv[i] *= rq; }
        }
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) x += S[i] * kv[i];
        x = sum4(x);
        float ov = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            S[i] = at * (S[i] - bt * x * kv[i]) + bt * vr * kv[i];
            ov += S[i] * qv[i];
        }
        ov = sum4(ov);
        if (part == 0) st_elem<F32>(p.o[dir], oq + row, p.scale * ov);
    }
    if (p.S_out[dir]) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i)
            if (i < nc) p.S_out[dir][srow + part + 4 * i] = S[i];
    }
}

// ---------------------------------------------------------------------------
// Buffer resources: q/k/v/o rows of one (stream, head) are addressed with
// 32-bit byte offsets from a per-(b, h) base.  Loads beyond num_records return
// zero and stores beyond it are dropped, so padded rows of a ragged sub-chunk
// (tokens outside [0, T)) need no branches.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS-only barrier: orders LDS traffic between the wavefronts of a workgroup
// without waiting for global loads that are still in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Token of local row t of processing step n: forward runs 0..N*C-1, reverse
// runs N*C-1 down to 0 (the padding of a ragged sequence then lands beyond
// T-1 in both directions).
struct TokMap {
    int base, sgn;
    __device__ __forceinline__ int operator()(int n, int C, int t) const { return base + sgn * (n * C + t); }
};

__device__ __forceinline__ f16x4 u2_to_f16x4(uint2 u) { return __builtin_bit_cast(f16x4, u); }
__device__ __forceinline__ bf16x4 u2_to_bf16x4(uint2 u) { return __builtin_bit_cast(bf16x4, u); }

// ---------------------------------------------------------------------------
// Chunk preparation: one workgroup (NB wavefronts) per (direction, b, h,
// processing step n).  Rows are stored in processing order.
// ---------------------------------------------------------------------------
template <int NB, int ND>
__global__ __launch_bounds__(64 * NB) void gdn_prep_kernel(Params p) {
    constexpr int C = 16 * NB, D = 16 * ND;
    constexpr int LDR = D + 8;   // bf16 row stride of the staged K and Q rows
    constexpr int LDM = C + 4;   // fp32 row stride of L^T, T, A
    constexpr int NT = 64 * NB;
    constexpr int CH = D / 8;    // 16-byte chunks per row
    using BK = Blocks<NB>;

    // K and Q rows (bf16) share storage with T (fp32), which is built after the Gram products
    constexpr int KQ_BYTES = 2 * C * LDR * 2, T_BYTES = C * LDM * 4;
    __shared__ __align__(16) char KQT[KQ_BYTES > T_BYTES ? KQ_BYTES : T_BYTES];
    __shared__ __align__(16) float Lt[C * LDM];   // L transposed: Lt[s][t] = L[t][s], s < t
    __shared__ __align__(16) float Am[C * LDM];
    __shared__ float sc[4][C];   // 0: log a then g, 1: beta, 2: 1/|k|, 3: 1/|q|
    bf16* Ks = reinterpret_cast<bf16*>(KQT);
    bf16* Qs = Ks + C * LDR;
    float* Tm = reinterpret_cast<float*>(KQT);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int n = blockIdx.x, bh = blockIdx.y, dir = p.dir0 + blockIdx.z;
    const int b = bh / p.H, h = bh - b * p.H;
    const int T = (int)p.T;
    const int N = (T + C - 1) / C;
    const TokMap tok{dir ? N * C - 1 : 0, dir ? -1 : 1};

    {
        const bf16* kb = reinterpret_cast<const bf16*>(p.k) + (int64_t)b * p.ks[0] + (int64_t)h * p.ks[2];
        const bf16* qb = reinterpret_cast<const bf16*>(p.q) + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[2];
        const auto kr = make_rsrc(kb, (uint32_t)(((int64_t)(T - 1) * p.ks[1] + D) * 2));
        const auto qr = make_rsrc(qb, (uint32_t)(((int64_t)(T - 1) * p.qs[1] + D) * 2));
        const int ksb = (int)p.ks[1] * 2, qsb = (int)p.qs[1] * 2;
        for (int idx = tid; idx < C * CH; idx += NT) {
            const int t = idx / CH, c = idx - t * CH;
            const int tk = tok(n, C, t);
            const uint4 kv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, tk * ksb + 16 * c, 0, 0));
            const uint4 qv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, tk * qsb + 16 * c, 0, 0));
            *reinterpret_cast<uint4*>(Ks + t * LDR + 8 * c) = kv;
            *reinterpret_cast<uint4*>(Qs + t * LDR + 8 * c) = qv;
        }
    }
    if (tid < C) {
        const int tk = tok(n, C, tid);
        float la = 0.f, bt = 0.f;
        if (tk >= 0 && tk < T) {
            const int64_t gq = (int64_t)b * p.gs[0] + (int64_t)tk * p.gs[1] + (int64_t)h * p.gs[2];
            la = fmaxf(logf(p.a[gq]), GDN_MIN_LOG_DECAY);
            bt = p.beta[gq];
        }
        sc[0][tid] = la;
        sc[1][tid] = bt;
    }
    __syncthreads();

    // per-token inverse norms: 4 lanes per row, 16 rows per wavefront
    {
        const int t = 16 * w + (lane >> 2), part = lane & 3;
        float sk = 0.f, sq = 0.f;
        for (int c = part; c < CH; c += 4) {
            const bf16x8 kv = ld_bf16x8(Ks + t * LDR + 8 * c);
            const bf16x8 qv = ld_bf16x8(Qs + t * LDR + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kf = (float)kv[e], qf = (float)qv[e];
                sk += kf * kf;
                sq += qf * qf;
            }
        }
        sk = sum4(sk);
        sq = sum4(sq);
        if (part == 0) {
            sc[2][t] = p.l2norm ? 1.f / sqrtf(sk + p.eps) : 1.f;
            sc[3][t] = p.l2norm ? 1.f / sqrtf(sq + p.eps) : 1.f;
        }
    }
    // inclusive prefix of log a along the processing order (C <= 64: one wavefront)
    if (w == 0) {
        float x = (lane < C) ? sc[0][lane] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane < C) sc[0][lane] = x;
    }
    __syncthreads();

    // Gram tiles on MFMA: K K^T -> L (strictly lower), Q K^T -> A (lower incl. diagonal)
    {
        constexpr int NTILE = NB * (NB + 1) / 2;
        for (int tt = w; tt < 2 * NTILE; tt += NB) {
            const bool isq = tt >= NTILE;
            const int ti = isq ? tt - NTILE : tt;
            int mt = 0;
            while ((mt + 1) * (mt + 2) / 2 <= ti) ++mt;
            const int nt = ti - mt * (mt + 1) / 2;
            const bf16* arow = (isq ? Qs : Ks) + (16 * mt + r) * LDR;
            const bf16* brow = Ks + (16 * nt + r) * LDR;
            bf16x8 aop[ND / 2 > 0 ? ND / 2 : 1], bop[ND / 2 > 0 ? ND / 2 : 1];
            bf16x4 aoh, boh;
#pragma unroll
            for (int ks = 0; ks < ND / 2; ++ks) {
                aop[ks] = ld_bf16x8(arow + 32 * ks + 8 * g);
                bop[ks] = ld_bf16x8(brow + 32 * ks + 8 * g);
            }
            if constexpr (ND % 2) {
                aoh = ld_bf16x4(arow + 32 * (ND / 2) + 4 * g);
                boh = ld_bf16x4(brow + 32 * (ND / 2) + 4 * g);
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < ND / 2; ++ks) acc = mma_bf16_k32(aop[ks], bop[ks], acc);
            if constexpr (ND % 2) acc = mma_bf16_k16(aoh, boh, acc);
            const int s = 16 * nt + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * g + i;
                const float dec = (s <= t) ? __expf(sc[0][t] - sc[0][s]) : 0.f;
                if (!isq)
                    Lt[s * LDM + t] = (s < t) ? sc[1][t] * dec * sc[2][t] * sc[2][s] * acc[i] : 0.f;
                else
                    Am[t * LDM + s] = (s <= t) ? p.scale * dec * sc[3][t] * sc[2][s] * acc[i] : 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < ND / 2; ++ks) {
                keep_alive(aop[ks]);
                keep_alive(bop[ks]);
            }
            if constexpr (ND % 2) {
                keep_alive(aoh);
                keep_alive(boh);
            }
        }
    }
    __syncthreads();

    // T = (I + L)^{-1}.  16x16 diagonal blocks: one lane per (block, column),
    // right-looking forward substitution.
    if (tid < C) {
        const int o = 16 * (tid >> 4), j = tid & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int k = 0; k < 15; ++k) {
            const float* lcol = Lt + (o + k) * LDM + o;   // L[o + i][o + k] for i > k
#pragma unroll
            for (int i = k + 1; i < 16; ++i) x[i] -= lcol[i] * x[k];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Tm[(o + i) * LDM + o + j] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks, by distance d from the diagonal, on fp32 MFMA:
    // T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj  (one wavefront per block)
    for (int d = 1; d < NB; ++d) {
        if (w < NB - d) {
            const int ib = w + d, jb = w;
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int kb = jb; kb < ib; ++kb) {
                float la[4], tb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = 16 * kb + 4 * kk + g;
                    la[kk] = Lt[k * LDM + 16 * ib + r];
                    tb[kk] = Tm[k * LDM + 16 * jb + r];
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) z = __builtin_amdgcn_mfma_f32_16x16x4f32(la[kk], tb[kk], z, 0, 0, 0);
                // z is consumed by the next block product or below; keep its operands until then
                const float zs = z[0];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    keep_alive(la[kk]);
                    keep_alive(tb[kk]);
                }
                keep_alive(zs);
            }
            // z: lane (column r, group g) holds Z[4g + e][r]; use it as the B operand with k = 4g + kk
            float ta[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) ta[kk] = Tm[(16 * ib + r) * LDM + 16 * ib + 4 * g + kk];
            f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) t4 = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[kk], z[kk], t4, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[(16 * ib + 4 * g + e) * LDM + 16 * jb + r] = -t4[e];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) keep_alive(ta[kk]);
        }
        __syncthreads();
    }

    // store T and A as fp16 MFMA A-operand fragments, then the per-token scalars
    char* item = p.ws + ((((int64_t)dir * p.B + b) * p.H + h) * p.nsub_max + n) * p.ws_item_bytes;
    f16* Tsw = reinterpret_cast<f16*>(item);
    f16* Asw = Tsw + BK::TOTAL * 512;
    float* scw = reinterpret_cast<float*>(item + 2 * 1024 * BK::TOTAL);
    for (int blk = w; blk < BK::TOTAL; blk += NB) {
        int mt = 0;
        while (BK::offset(mt + 1) <= blk) ++mt;
        const int idx = blk - BK::offset(mt);
        const int row = 16 * mt + r;
        f16x8 tv, av;
        if (idx < BK::nfull_for(mt)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int col = 32 * idx + 16 * (i >> 2) + 4 * g + (i & 3);
                tv[i] = (col <= row) ? (f16)Tm[row * LDM + col] : (f16)0.f;
                av[i] = (col <= row) ? (f16)Am[row * LDM + col] : (f16)0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int col = 32 * BK::NFULL + 4 * g + (i & 3);
                tv[i] = (i < 4 && col <= row) ? (f16)Tm[row * LDM + col] : (f16)0.f;
                av[i] = (i < 4 && col <= row) ? (f16)Am[row * LDM + col] : (f16)0.f;
            }
        }
        *reinterpret_cast<f16x8*>(Tsw + blk * 512 + lane * 8) = tv;
        *reinterpret_cast<f16x8*>(Asw + blk * 512 + lane * 8) = av;
    }
    if (tid < C) {
        const float gt = sc[0][tid], gC = sc[0][C - 1];
        const float gam = __expf(gt), bt = sc[1][tid], rk = sc[2][tid];
        scw[0 * C + tid] = bt;                          // beta
        scw[1 * C + tid] = bt * gam * rk;               // scales K S^T inside R
        scw[2 * C + tid] = p.scale * gam * sc[3][tid];  // scales Q S^T inside O
        scw[3 * C + tid] = __expf(gC - gt) * rk;        // decay to the end of the step, over |k|
        scw[4 * C + tid] = rk;                          // 1/|k|
        if (tid == 0) scw[5 * C] = __expf(gC);          // decay over the whole step
    }
}

// ---------------------------------------------------------------------------
// Chunk scan: one workgroup of two wavefronts per (direction, b, h, 16 state
// rows), serial over the sub-chunks.
//   wave 0 (chain):  X = K S^T, R, U = T R, publishes (S as bf16, U as fp16)
//                    to LDS, then S <- e^{g_C} S + K^T W with
//                    W = diag(e^{g_C-g}/|k|) U carried as a bf16 high/low pair.
//                    The state slice lives in its MFMA accumulators.
//   wave 1 (output): O = diag(scale e^g/|q|) Q S^T + A U from the published
//                    fragments, stored as bf16.
// One LDS barrier per sub-chunk; LDS slots are double-buffered, so wave 1
// works on step n while wave 0 runs the state update of step n and the first
// half of step n+1.  Each wavefront reloads an operand for step n+1 right
// after its last use in step n, so the loads overlap the rest of the step.
//
// Row addressing: the buffer resource of a step starts at the lowest token of
// the step and ends after the last real token, so a row's byte offset is a
// per-lane constant and rows past the end of the sequence read as zero (and
// are not stored).
// ---------------------------------------------------------------------------
template <int NB, int ND>
struct KRows {                                   // K or Q rows (bf16) as MFMA A operands
    uint2 op[NB][ND / 2 > 0 ? ND / 2 : 1][2];    // [mt][ks][low/high 4 elements]
    uint2 h[NB];                                 // trailing 16-wide d-step (odd ND)
};

template <int NB, int ND>
struct ChainIn {
    uint4 tfr[Blocks<NB>::TOTAL];
    uint32_t vv[NB][4];                          // V[t][row]: bf16 bits
    f32x4 bet[NB], c1[NB], w[NB];
    float gC;
};

template <int NB, int ND>
struct OutIn {
    uint4 afr[Blocks<NB>::TOTAL];
    f32x4 c2[NB];
};

// Buffer resource over the rows of processing step n: base at the step's lowest
// token, num_records ending after the last real token.
struct StepRows {
    const char* base;   // row 0 of (b, h)
    int64_t tstride;    // bytes between tokens
    int T, C, N, dir, width_bytes;
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int n) const {
        const int lo = dir ? (N - 1 - n) * C : n * C;   // lowest token of the step
        const int64_t valid = (int64_t)(T - 1 - lo) * tstride + width_bytes;
        return make_rsrc(base + (int64_t)lo * tstride, valid > 0 ? (uint32_t)valid : 0u);
    }
    // offset of local row t (processing order) from the step's lowest token
    __device__ __forceinline__ int row(int t) const { return (dir ? (C - 1 - t) : t) * (int)tstride; }
};

template <int NB, int ND>
__global__ __launch_bounds__(128) void gdn_scan_kernel(Params p, int ngroups) {
    constexpr int C = 16 * NB, D = 16 * ND;
    constexpr int NFK = ND / 2;            // 32-wide steps over d
    constexpr bool HK = (ND % 2) != 0;     // trailing 16-wide step over d
    constexpr int NKD = NFK + (HK ? 1 : 0);
    using BK = Blocks<NB>;
    constexpr int NFT = BK::NFULL;         // 32-wide steps over tokens
    constexpr bool HT = BK::HALF;
    constexpr int NKT = NFT + (HT ? 1 : 0);
    constexpr int LDK = D + 32;            // bf16 row stride of the staged K rows (8-byte aligned rows)
    typedef short s16x4 __attribute__((ext_vector_type(4)));

    __shared__ __align__(16) bf16 Kh[C * LDK];
    __shared__ __align__(16) uint4 pubP[2][NKD][64];
    __shared__ __align__(16) uint4 pubU[2][NKT][64];

    const int lane = threadIdx.x & 63;
    // the role of a wavefront is wave-uniform: keep it in a scalar register so both
    // roles are whole-wavefront branches (each role runs its own barrier sequence)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    // Workgroups are spread over the 8 XCDs round-robin (id % 8); keep the ND
    // row slices of one (direction, b, h) on one XCD so they share its L2.
    const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
    const int group = (slot / ND) * 8 + xcd, j = slot - (slot / ND) * ND;
    if (group >= ngroups) return;
    int gg = group;
    const int h = gg % p.H; gg /= p.H;
    const int b = gg % p.B; gg /= p.B;
    const int dir = p.dir0 + gg;
    const int T = (int)p.T;
    const int N = (T + C - 1) / C;
    const int row0 = 16 * j;
    const char* item0 = p.ws + (((int64_t)dir * p.B + b) * p.H + h) * p.nsub_max * p.ws_item_bytes;
    const int64_t ib = p.ws_item_bytes;

    if (wave == 0) {
        // ------------------------------ chain wavefront ------------------------------
        const StepRows kr{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.k) + (int64_t)b * p.ks[0] +
                                                        (int64_t)h * p.ks[2]),
                          p.ks[1] * 2, T, C, N, dir, 2 * D};
        const StepRows vr{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.v) + (int64_t)b * p.vs[0] +
                                                        (int64_t)h * p.vs[2]),
                          p.vs[1] * 2, T, C, N, dir, 2 * D};
        int koff[NB], voff[NB][4];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            koff[mt] = kr.row(16 * mt + r) + 8 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) voff[mt][i] = vr.row(16 * mt + 4 * g + i) + 2 * (row0 + r);
        }

        ChainIn<NB, ND> in;
        KRows<NB, ND> kA, kB;
        auto load_k = [&](KRows<NB, ND>& kk, int n) {
            const auto rs = kr.rsrc(n);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
                for (int ks = 0; ks < NFK; ++ks) {
                    kk.op[mt][ks][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, koff[mt], 64 * ks, 0));
                    kk.op[mt][ks][1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, koff[mt], 64 * ks + 32, 0));
                }
                if constexpr (HK)
                    kk.h[mt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, koff[mt], 64 * NFK, 0));
            }
        };
        auto load_rest = [&](int n) {
            const char* item = item0 + n * ib;
            const auto rs = vr.rsrc(n);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) in.vv[mt][i] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff[mt][i], 0, 0);
            const uint4* tsw = reinterpret_cast<const uint4*>(item);
#pragma unroll
            for (int blk = 0; blk < BK::TOTAL; ++blk) in.tfr[blk] = tsw[blk * 64 + lane];
            const float* scg = reinterpret_cast<const float*>(item + 2 * 1024 * BK::TOTAL);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) {
                in.bet[mt] = *reinterpret_cast<const f32x4*>(scg + 0 * C + 16 * mt + 4 * g);
                in.c1[mt] = *reinterpret_cast<const f32x4*>(scg + 1 * C + 16 * mt + 4 * g);
                in.w[mt] = *reinterpret_cast<const f32x4*>(scg + 3 * C + 16 * mt + 4 * g);
            }
            in.gC = scg[5 * C];
        };

        // state slice, transposed: P[m][i] = S[row0 + r][16 m + 4 g + i]
        f32x4 P[ND];
        const float* Sin = (dir == 0) ? p.S_in : nullptr;
        const int64_t sbase = ((int64_t)b * p.H + h) * D * D + (int64_t)(row0 + r) * D;
#pragma unroll
        for (int m = 0; m < ND; ++m) {
            if (Sin) P[m] = *reinterpret_cast<const f32x4*>(Sin + sbase + 16 * m + 4 * g);
            else P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        load_k(kA, 0);
        if (N > 1) load_k(kB, 1);
        load_rest(0);
        auto chain_step = [&](KRows<NB, ND>& kc, int n) {
            const int sl = n & 1;
            // state as bf16 B operand: slot i of group g <-> d = 32 ks + 16 (i/4) + 4 g + i%4
            bf16x8 Pb[NKD];
#pragma unroll
            for (int ks = 0; ks < NFK; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Pb[ks][i] = (bf16)P[2 * ks][i];
                    Pb[ks][4 + i] = (bf16)P[2 * ks + 1][i];
                }
            if constexpr (HK) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Pb[NFK][i] = (bf16)P[ND - 1][i];
                    Pb[NFK][4 + i] = (bf16)0.f;
                }
            }
            // X = K S^T (rows: tokens), independent accumulators interleaved; the raw bf16
            // K rows also go to LDS for the state update
            f32x4 X[NB];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) X[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NFK; ++ks)
#pragma unroll
                for (int mt = 0; mt < NB; ++mt)
                    X[mt] = mma_bf16_k32(cat(u2_to_bf16x4(kc.op[mt][ks][0]), u2_to_bf16x4(kc.op[mt][ks][1])), Pb[ks], X[mt]);
            if constexpr (HK) {
                const bf16x4 pbh = {Pb[NFK][0], Pb[NFK][1], Pb[NFK][2], Pb[NFK][3]};
#pragma unroll
                for (int mt = 0; mt < NB; ++mt) X[mt] = mma_bf16_k16(u2_to_bf16x4(kc.h[mt]), pbh, X[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) {
                const int t = 16 * mt + r;
#pragma unroll
                for (int ks = 0; ks < NFK; ++ks) {
                    *reinterpret_cast<uint2*>(Kh + t * LDK + 32 * ks + 4 * g) = kc.op[mt][ks][0];
                    *reinterpret_cast<uint2*>(Kh + t * LDK + 32 * ks + 16 + 4 * g) = kc.op[mt][ks][1];
                }
                if constexpr (HK) *reinterpret_cast<uint2*>(Kh + t * LDK + 32 * NFK + 4 * g) = kc.h[mt];
            }
            // R = diag(beta) V - diag(beta e^g / |k|) X, as fp16 B operand (k = token)
            f16x8 Rb[NKT];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float vv = __builtin_bit_cast(float, in.vv[mt][i] << 16);
                    Rb[mt >> 1][4 * (mt & 1) + i] = (f16)(in.bet[mt][i] * vv - in.c1[mt][i] * X[mt][i]);
                }
            if constexpr (HT) {
#pragma unroll
                for (int i = 4; i < 8; ++i) Rb[NFT][i] = (f16)0.f;
            }
            // X has been consumed (R is formed here), so its operands are free: the K-row
            // registers are refilled for step n + 2
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) keep_alive(Rb[ks]);
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) keep_alive(Pb[ks]);
            __builtin_amdgcn_sched_barrier(0);   // no refill above the consumers of X
            if (n + 2 < N) load_k(kc, n + 2);
            // U = T R (k-step outer, row tiles inner: consecutive MFMAs are independent)
            f32x4 U[NB];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) U[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int idx = 0; idx < NKT; ++idx)
#pragma unroll
                for (int mt = 0; mt < NB; ++mt) {
                    if (idx >= BK::count(mt)) continue;
                    const uint4 tf = in.tfr[BK::offset(mt) + idx];
                    if (idx < BK::nfull_for(mt)) {
                        U[mt] = mma_f16_k32(__builtin_bit_cast(f16x8, tf), Rb[idx], U[mt]);
                    } else {
                        const f16x4 rb = {Rb[NFT][0], Rb[NFT][1], Rb[NFT][2], Rb[NFT][3]};
                        U[mt] = mma_f16_k16(u2_to_f16x4(uint2{tf.x, tf.y}), rb, U[mt]);
                    }
                }
            // publish the state at the start of this step and U for the output wavefront;
            // W = diag(e^{g_C-g}/|k|) U as a bf16 pair (high part + rounded remainder)
            f16x8 Ub[NKT];
            bf16x8 Wh[NKT], Wl[NKT];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int si = 4 * (mt & 1) + i;
                    Ub[mt >> 1][si] = (f16)U[mt][i];
                    const float wv = in.w[mt][i] * U[mt][i];
                    const bf16 hi = (bf16)wv;
                    Wh[mt >> 1][si] = hi;
                    Wl[mt >> 1][si] = (bf16)(wv - (float)hi);
                }
            if constexpr (HT) {
#pragma unroll
                for (int i = 4; i < 8; ++i) {
                    Ub[NFT][i] = (f16)0.f;
                    Wh[NFT][i] = (bf16)0.f;
                    Wl[NFT][i] = (bf16)0.f;
                }
            }
            const float gC = in.gC;
            // U has been consumed (Ub, W are formed here): its operands are free
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) {
                keep_alive(Ub[ks]);
                keep_alive(Wh[ks]);
                keep_alive(Wl[ks]);
                keep_alive(Rb[ks]);
            }
            __builtin_amdgcn_sched_barrier(0);   // no refill above the consumers of U
            if (n + 1 < N) load_rest(n + 1);
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) pubP[sl][ks][lane] = __builtin_bit_cast(uint4, Pb[ks]);
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) pubU[sl][ks][lane] = __builtin_bit_cast(uint4, Ub[ks]);
            lds_barrier();
            // S <- e^{g_C} S + K^T W, computed transposed (rows d, columns r): the A operand
            // (rows d, k = token) comes from the K rows with transposing LDS reads, all issued
            // before the MFMAs; the ND accumulators are interleaved.
            bf16x8 KT[ND][NKT];
#pragma unroll
            for (int m = 0; m < ND; ++m)
#pragma unroll
                for (int ks = 0; ks < NKT; ++ks) {
                    const int t0 = 32 * ks + 4 * g + (r >> 2);
                    const int d0 = 16 * m + 4 * (r & 3);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(Kh + t0 * LDK + d0));
                    s16x4 hi = {0, 0, 0, 0};
                    if (ks < NFT)
                        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4*)(Kh + (t0 + 16) * LDK + d0));
                    KT[m][ks] = cat(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
                }
#pragma unroll
            for (int m = 0; m < ND; ++m) P[m] = P[m] * gC;
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                    for (int m = 0; m < ND; ++m) {
                        const bf16x8 wv = hl ? Wl[ks] : Wh[ks];
                        if (ks < NFT) {
                            P[m] = mma_bf16_k32(KT[m][ks], wv, P[m]);
                        } else {
                            const bf16x4 a = {KT[m][ks][0], KT[m][ks][1], KT[m][ks][2], KT[m][ks][3]};
                            const bf16x4 w4 = {wv[0], wv[1], wv[2], wv[3]};
                            P[m] = mma_bf16_k16(a, w4, P[m]);
                        }
                    }
            // P is read here, so every state-update MFMA has finished before its operands go
#pragma unroll
            for (int m = 0; m < ND; ++m) {
                const float pm = P[m][0];
                keep_alive(pm);
#pragma unroll
                for (int ks = 0; ks < NKT; ++ks) keep_alive(KT[m][ks]);
            }
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) {
                keep_alive(Wh[ks]);
                keep_alive(Wl[ks]);
            }
        };
        for (int n = 0; n < N; n += 2) {
            chain_step(kA, n);
            if (n + 1 < N) chain_step(kB, n + 1);
        }
        float* Sout = p.S_out[dir];
        if (Sout) {
#pragma unroll
            for (int m = 0; m < ND; ++m) *reinterpret_cast<f32x4*>(Sout + sbase + 16 * m + 4 * g) = P[m];
        }
    } else {
        // ------------------------------ output wavefront ------------------------------
        const StepRows qr{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.q) + (int64_t)b * p.qs[0] +
                                                        (int64_t)h * p.qs[2]),
                          p.qs[1] * 2, T, C, N, dir, 2 * D};
        const StepRows orow{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.o[dir]) + (int64_t)b * p.os[0] +
                                                          (int64_t)h * p.os[2]),
                            p.os[1] * 2, T, C, N, dir, 2 * D};
        int qoff[NB], ooff[NB][4];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            qoff[mt] = qr.row(16 * mt + r) + 8 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) ooff[mt][i] = orow.row(16 * mt + 4 * g + i) + 2 * (row0 + r);
        }

        OutIn<NB, ND> in;
        KRows<NB, ND> qA, qB;
        auto load_q = [&](KRows<NB, ND>& qq, int n) {
            const auto rs = qr.rsrc(n);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
                for (int ks = 0; ks < NFK; ++ks) {
                    qq.op[mt][ks][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, qoff[mt], 64 * ks, 0));
                    qq.op[mt][ks][1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, qoff[mt], 64 * ks + 32, 0));
                }
                if constexpr (HK)
                    qq.h[mt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, qoff[mt], 64 * NFK, 0));
            }
        };
        auto load_rest = [&](int n) {
            const char* item = item0 + n * ib;
            const uint4* asw = reinterpret_cast<const uint4*>(item) + BK::TOTAL * 64;
#pragma unroll
            for (int blk = 0; blk < BK::TOTAL; ++blk) in.afr[blk] = asw[blk * 64 + lane];
            const float* scg = reinterpret_cast<const float*>(item + 2 * 1024 * BK::TOTAL);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) in.c2[mt] = *reinterpret_cast<const f32x4*>(scg + 2 * C + 16 * mt + 4 * g);
        };

        load_q(qA, 0);
        if (N > 1) load_q(qB, 1);
        load_rest(0);
        auto out_step = [&](KRows<NB, ND>& qc, int n) {
            const int sl = n & 1;
            const auto ors = orow.rsrc(n);
            lds_barrier();
            bf16x8 Pb[NKD];
            f16x8 Ub[NKT];
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) Pb[ks] = __builtin_bit_cast(bf16x8, pubP[sl][ks][lane]);
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) Ub[ks] = __builtin_bit_cast(f16x8, pubU[sl][ks][lane]);
            f32x4 Y[NB];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) Y[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NFK; ++ks)
#pragma unroll
                for (int mt = 0; mt < NB; ++mt)
                    Y[mt] = mma_bf16_k32(cat(u2_to_bf16x4(qc.op[mt][ks][0]), u2_to_bf16x4(qc.op[mt][ks][1])), Pb[ks], Y[mt]);
            if constexpr (HK) {
                const bf16x4 pbh = {Pb[NFK][0], Pb[NFK][1], Pb[NFK][2], Pb[NFK][3]};
#pragma unroll
                for (int mt = 0; mt < NB; ++mt) Y[mt] = mma_bf16_k16(u2_to_bf16x4(qc.h[mt]), pbh, Y[mt]);
            }
            f32x4 O[NB];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) O[mt] = in.c2[mt] * Y[mt];
            // Y has been consumed (O is started here): the state fragments may go and the Q
            // registers may be refilled
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) keep_alive(O[mt]);
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) keep_alive(Pb[ks]);
            __builtin_amdgcn_sched_barrier(0);   // no refill above the consumers of Y
            if (n + 2 < N) load_q(qc, n + 2);
#pragma unroll
            for (int idx = 0; idx < NKT; ++idx)
#pragma unroll
                for (int mt = 0; mt < NB; ++mt) {
                    if (idx >= BK::count(mt)) continue;
                    const uint4 af = in.afr[BK::offset(mt) + idx];
                    if (idx < BK::nfull_for(mt)) {
                        O[mt] = mma_f16_k32(__builtin_bit_cast(f16x8, af), Ub[idx], O[mt]);
                    } else {
                        const f16x4 ub = {Ub[NFT][0], Ub[NFT][1], Ub[NFT][2], Ub[NFT][3]};
                        O[mt] = mma_f16_k16(u2_to_f16x4(uint2{af.x, af.y}), ub, O[mt]);
                    }
                }
            bf16 ov[NB][4];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[mt][i] = (bf16)O[mt][i];
            // O has been consumed (converted here): the U fragments may go and the A fragments
            // may be refilled
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) keep_alive(ov[mt][i]);
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) keep_alive(Ub[ks]);
            __builtin_amdgcn_sched_barrier(0);   // no refill above the consumers of O
            if (n + 1 < N) load_rest(n + 1);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, ov[mt][i]), ors,
                                                          ooff[mt][i], 0, 0);
        };
        for (int n = 0; n < N; n += 2) {
            out_step(qA, n);
            if (n + 1 < N) out_step(qB, n + 1);
        }
    }
}

// Zero a float buffer (used instead of a memset node so callers may capture it in a graph).
__global__ void gdn_zero_kernel(float* x, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        x[i] = 0.f;
}

hipError_t launch_zero(float* x, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(gdn_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static void tm_begin(Timing* tm, hipStream_t s, int kind) {
    if (tm && tm->ev && tm->n < tm->cap) {
        (void)hipEventRecord(tm->ev[2 * tm->n], s);
        tm->kinds[tm->n] = kind;
    }
}
static void tm_end(Timing* tm, hipStream_t s) {
    if (tm && tm->ev && tm->n < tm->cap) {
        (void)hipEventRecord(tm->ev[2 * tm->n + 1], s);
        tm->n++;
    }
}

hipError_t launch_sequential(const Params& p, hipStream_t s, Timing* tm) {
    const int grid = p.ndirs * p.B * p.H * (p.Dv / 16);
    tm_begin(tm, s, KSEQ);
    if (p.io_f32) hipLaunchKernelGGL(gdn_seq_kernel<true>, dim3(grid), dim3(64), 0, s, p);
    else hipLaunchKernelGGL(gdn_seq_kernel<false>, dim3(grid), dim3(64), 0, s, p);
    tm_end(tm, s);
    return hipGetLastError();
}

template <int NB, int ND>
static hipError_t run_chunked(const Params& p, hipStream_t s, Timing* tm) {
    const int nsub = (int)((p.T + 16 * NB - 1) / (16 * NB));
    tm_begin(tm, s, KPREP);
    hipLaunchKernelGGL((gdn_prep_kernel<NB, ND>), dim3(nsub, p.B * p.H, p.ndirs), dim3(64 * NB), 0, s, p);
    tm_end(tm, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ngroups = p.ndirs * p.B * p.H;
    const int grid = (ngroups + 7) / 8 * 8 * ND;
    tm_begin(tm, s, KSCAN);
    hipLaunchKernelGGL((gdn_scan_kernel<NB, ND>), dim3(grid), dim3(128), 0, s, p, ngroups);
    tm_end(tm, s);
    return hipGetLastError();
}

template <int NB>
static hipError_t run_chunked_d(const Params& p, hipStream_t s, Timing* tm) {
    switch (p.Dk) {
        case 16: return run_chunked<NB, 1>(p, s, tm);
        case 32: return run_chunked<NB, 2>(p, s, tm);
        case 64: return run_chunked<NB, 4>(p, s, tm);
        case 112: return run_chunked<NB, 7>(p, s, tm);
        case 128: return run_chunked<NB, 8>(p, s, tm);
        default: return hipErrorInvalidValue;
    }
}

bool chunked_supported(int C, int Dk, int Dv, int io_f32) {
    if (io_f32) return false;
    if (Dk != Dv) return false;
    if (!(Dk == 16 || Dk == 32 || Dk == 64 || Dk == 112 || Dk == 128)) return false;
    return C == 16 || C == 32 || C == 64;
}

hipError_t launch_chunked(const Params& p, hipStream_t s, Timing* tm) {
    switch (p.C) {
        case 16: return run_chunked_d<1>(p, s, tm);
        case 32: return run_chunked_d<2>(p, s, tm);
        case 64: return run_chunked_d<4>(p, s, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
