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
__device__ __forceinline__ f32x4 mma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
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
// Chunk preparation: one workgroup (NB wavefronts) per (direction, b, h, sub-chunk).
// ---------------------------------------------------------------------------
template <int NB, int ND>
__global__ __launch_bounds__(64 * NB) void gdn_prep_kernel(Params p) {
    constexpr int C = 16 * NB, D = 16 * ND;
    constexpr int LDR = D + 8;   // bf16 row stride of the staged K and Q rows
    constexpr int LDM = C + 1;   // fp32 row stride of L, T, A
    constexpr int NT = 64 * NB;
    constexpr int CH = D / 8;    // 16-byte chunks per row
    using BK = Blocks<NB>;

    // K and Q rows (bf16) share storage with T (fp32), which is only built after the Gram products
    constexpr int KQ_BYTES = 2 * C * LDR * 2, T_BYTES = C * LDM * 4;
    __shared__ __align__(16) char KQT[KQ_BYTES > T_BYTES ? KQ_BYTES : T_BYTES];
    __shared__ float Lm[C * LDM];
    __shared__ float Am[C * LDM];
    __shared__ float Zb[256 * (NB > 1 ? NB - 1 : 1)];
    __shared__ float sc[4][C];   // 0: log a then g, 1: beta, 2: 1/|k|, 3: 1/|q|
    bf16* Ks = reinterpret_cast<bf16*>(KQT);
    bf16* Qs = Ks + C * LDR;
    float* Tm = reinterpret_cast<float*>(KQT);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = blockIdx.x, bh = blockIdx.y, dir = p.dir0 + blockIdx.z;
    const int b = bh / p.H, h = bh - b * p.H;
    const int64_t T = p.T;
    const int64_t m0 = (int64_t)n * C;
    const int nval = (int)((T - m0) < C ? (T - m0) : C);
    auto token = [&](int t) -> int64_t { return dir ? (T - 1 - (m0 + t)) : (m0 + t); };

    // rows of K and Q (zero beyond the end of the sequence)
    for (int idx = tid; idx < C * CH; idx += NT) {
        const int t = idx / CH, c = idx - t * CH;
        uint4 kv = {0, 0, 0, 0}, qv = {0, 0, 0, 0};
        if (t < nval) {
            const int64_t tok = token(t);
            kv = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16*>(p.k) +
                                                  (int64_t)b * p.ks[0] + tok * p.ks[1] + (int64_t)h * p.ks[2] + 8 * c);
            qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16*>(p.q) +
                                                  (int64_t)b * p.qs[0] + tok * p.qs[1] + (int64_t)h * p.qs[2] + 8 * c);
        }
        *reinterpret_cast<uint4*>(Ks + t * LDR + 8 * c) = kv;
        *reinterpret_cast<uint4*>(Qs + t * LDR + 8 * c) = qv;
    }
    if (tid < C) {
        float la = 0.f, bt = 0.f;
        if (tid < nval) {
            const int64_t tok = token(tid);
            const int64_t gq = (int64_t)b * p.gs[0] + tok * p.gs[1] + (int64_t)h * p.gs[2];
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
    // inclusive prefix of log a inside the sub-chunk (C <= 64: one wavefront)
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
        const int g = lane >> 4, r = lane & 15;
        for (int tt = w; tt < 2 * NTILE; tt += NB) {
            const bool isq = tt >= NTILE;
            const int ti = isq ? tt - NTILE : tt;
            int mt = 0;
            while ((mt + 1) * (mt + 2) / 2 <= ti) ++mt;
            const int nt = ti - mt * (mt + 1) / 2;
            const bf16* arow = (isq ? Qs : Ks) + (16 * mt + r) * LDR;
            const bf16* brow = Ks + (16 * nt + r) * LDR;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < ND / 2; ++ks)
                acc = mma_bf16_k32(ld_bf16x8(arow + 32 * ks + 8 * g), ld_bf16x8(brow + 32 * ks + 8 * g), acc);
            if constexpr (ND % 2)
                acc = mma_bf16_k16(ld_bf16x4(arow + 32 * (ND / 2) + 4 * g), ld_bf16x4(brow + 32 * (ND / 2) + 4 * g), acc);
            const int s = 16 * nt + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * g + i;
                const float dec = (s <= t) ? __expf(sc[0][t] - sc[0][s]) : 0.f;
                if (!isq)
                    Lm[t * LDM + s] = (s < t) ? sc[1][t] * dec * sc[2][t] * sc[2][s] * acc[i] : 0.f;
                else
                    Am[t * LDM + s] = (s <= t) ? p.scale * dec * sc[3][t] * sc[2][s] * acc[i] : 0.f;
            }
        }
    }
    __syncthreads();

    // T = (I + L)^{-1}: 16x16 diagonal blocks by forward substitution (one lane per column)
    if (tid < C) {
        const int o = 16 * (tid >> 4), j = tid & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) s -= Lm[(o + i) * LDM + o + kk] * x[kk];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Tm[(o + i) * LDM + o + j] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks, by distance from the diagonal: T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj
    for (int d = 1; d < NB; ++d) {
        const int nblk = NB - d;
        for (int e = tid; e < nblk * 256; e += NT) {
            const int jb = e >> 8, rr = (e >> 4) & 15, cc = e & 15, ib = jb + d;
            float s = 0.f;
            for (int kk = 16 * jb; kk < 16 * ib; ++kk) s += Lm[(16 * ib + rr) * LDM + kk] * Tm[kk * LDM + 16 * jb + cc];
            Zb[e] = s;
        }
        __syncthreads();
        for (int e = tid; e < nblk * 256; e += NT) {
            const int jb = e >> 8, rr = (e >> 4) & 15, cc = e & 15, ib = jb + d;
            float s = 0.f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) s -= Tm[(16 * ib + rr) * LDM + 16 * ib + kk] * Zb[(jb << 8) + (kk << 4) + cc];
            Tm[(16 * ib + rr) * LDM + 16 * jb + cc] = s;
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
        const int row = 16 * mt + (lane & 15), g = lane >> 4;
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
        scw[0 * C + tid] = bt;                       // beta
        scw[1 * C + tid] = bt * gam * rk;            // scales K S^T inside R
        scw[2 * C + tid] = p.scale * gam * sc[3][tid];   // scales Q S^T inside O
        scw[3 * C + tid] = __expf(gC - gt);          // decay from token to chunk end
        scw[4 * C + tid] = rk;                       // 1/|k|
        if (tid == 0) scw[5 * C] = __expf(gC);       // decay over the whole sub-chunk
    }
}

// ---------------------------------------------------------------------------
// Chunk scan: one wavefront per (direction, b, h, 16 state rows), serial over
// the sub-chunks; the state slice lives in MFMA accumulators the whole time.
// ---------------------------------------------------------------------------
template <int NB, int ND>
__global__ __launch_bounds__(64) void gdn_scan_kernel(Params p, int ngroups) {
    constexpr int C = 16 * NB, D = 16 * ND;
    constexpr int NFK = ND / 2;            // 32-wide steps over d
    constexpr bool HK = (ND % 2) != 0;     // trailing 16-wide step over d
    using BK = Blocks<NB>;
    constexpr int NFT = BK::NFULL;         // 32-wide steps over tokens
    constexpr bool HT = BK::HALF;
    constexpr int LDK = D + 4;             // fp16 row stride of K^ in LDS

    __shared__ __align__(16) f16 Kh[C * LDK];
    __shared__ __align__(16) float scl[5 * C + 4];

    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    // Workgroups are spread over the 8 XCDs round-robin (id % 8); keep the ND
    // row slices of one (direction, b, h) on one XCD so they share its L2.
    const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
    const int group = (slot / ND) * 8 + xcd, j = slot - (slot / ND) * ND;
    if (group >= ngroups) return;
    int gg = group;
    const int h = gg % p.H; gg /= p.H;
    const int b = gg % p.B; gg /= p.B;
    const int dir = p.dir0 + gg;
    const int64_t T = p.T;
    const int row0 = 16 * j;

    // state slice, transposed: P[m][i] = S[row0 + r][16 m + 4 g + i]
    f32x4 P[ND];
    const float* Sin = (dir == 0) ? p.S_in : nullptr;
    const int64_t sbase = ((int64_t)b * p.H + h) * D * D + (int64_t)(row0 + r) * D;
#pragma unroll
    for (int m = 0; m < ND; ++m) {
        if (Sin) P[m] = *reinterpret_cast<const f32x4*>(Sin + sbase + 16 * m + 4 * g);
        else P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + (int64_t)b * p.ks[0] + (int64_t)h * p.ks[2];
    const bf16* qbase = reinterpret_cast<const bf16*>(p.q) + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[2];
    const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + (int64_t)b * p.vs[0] + (int64_t)h * p.vs[2] + row0 + r;
    bf16* obase = reinterpret_cast<bf16*>(p.o[dir]) + (int64_t)b * p.os[0] + (int64_t)h * p.os[2] + row0 + r;
    const char* item0 = p.ws + (((int64_t)dir * p.B + b) * p.H + h) * p.nsub_max * p.ws_item_bytes;
    const int nsub = (int)((T + C - 1) / C);

    for (int n = 0; n < nsub; ++n) {
        const char* item = item0 + (int64_t)n * p.ws_item_bytes;
        const f16* Tsw = reinterpret_cast<const f16*>(item);
        const f16* Asw = Tsw + BK::TOTAL * 512;
        const float* scg = reinterpret_cast<const float*>(item + 2 * 1024 * BK::TOTAL);
        const int64_t m0 = (int64_t)n * C;
        const int nval = (int)((T - m0) < C ? (T - m0) : C);
        auto token = [&](int t) -> int64_t { return dir ? (T - 1 - (m0 + t)) : (m0 + t); };

        for (int e = lane; e < 5 * C + 1; e += 64) scl[e] = scg[e];
        __syncthreads();

        // state as bf16 B operand (slot i of group g <-> d = 32 ks + 16 (i/4) + 4 g + i%4)
        bf16x8 Pb[NFK > 0 ? NFK : 1];
        bf16x4 Pbh;
#pragma unroll
        for (int ks = 0; ks < NFK; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Pb[ks][i] = (bf16)P[2 * ks][i];
                Pb[ks][4 + i] = (bf16)P[2 * ks + 1][i];
            }
        if constexpr (HK) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Pbh[i] = (bf16)P[ND - 1][i];
        }

        // X = K S^T and Y = Q S^T (rows: tokens); K^ rows staged to LDS as fp16
        f32x4 X[NB], Y[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            const int t = 16 * mt + r;
            const bool ok = t < nval;
            const int64_t tok = token(t);
            const bf16* kp = kbase + tok * p.ks[1];
            const bf16* qp = qbase + tok * p.qs[1];
            const float rk = scl[4 * C + t];
            const bf16x4 z4 = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NFK; ++ks) {
                const bf16x4 k0 = ok ? ld_bf16x4(kp + 32 * ks + 4 * g) : z4;
                const bf16x4 k1 = ok ? ld_bf16x4(kp + 32 * ks + 16 + 4 * g) : z4;
                const bf16x4 q0 = ok ? ld_bf16x4(qp + 32 * ks + 4 * g) : z4;
                const bf16x4 q1 = ok ? ld_bf16x4(qp + 32 * ks + 16 + 4 * g) : z4;
                x = mma_bf16_k32(cat(k0, k1), Pb[ks], x);
                y = mma_bf16_k32(cat(q0, q1), Pb[ks], y);
                f16x4 h0, h1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h0[e] = (f16)((float)k0[e] * rk);
                    h1[e] = (f16)((float)k1[e] * rk);
                }
                *reinterpret_cast<f16x4*>(Kh + t * LDK + 32 * ks + 4 * g) = h0;
                *reinterpret_cast<f16x4*>(Kh + t * LDK + 32 * ks + 16 + 4 * g) = h1;
            }
            if constexpr (HK) {
                const bf16x4 k0 = ok ? ld_bf16x4(kp + 32 * NFK + 4 * g) : z4;
                const bf16x4 q0 = ok ? ld_bf16x4(qp + 32 * NFK + 4 * g) : z4;
                x = mma_bf16_k16(k0, Pbh, x);
                y = mma_bf16_k16(q0, Pbh, y);
                f16x4 h0;
#pragma unroll
                for (int e = 0; e < 4; ++e) h0[e] = (f16)((float)k0[e] * rk);
                *reinterpret_cast<f16x4*>(Kh + t * LDK + 32 * NFK + 4 * g) = h0;
            }
            X[mt] = x;
            Y[mt] = y;
        }

        // R = diag(beta) V - diag(beta e^g / |k|) X  (rows t = 16 mt + 4 g + i)
        f32x4 R[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * g + i;
                const float vv = (t < nval) ? (float)vbase[token(t) * p.vs[1]] : 0.f;
                R[mt][i] = scl[t] * vv - scl[C + t] * X[mt][i];
            }
        f16x8 Rb[NFT > 0 ? NFT : 1];
        f16x4 Rbh;
#pragma unroll
        for (int ks = 0; ks < NFT; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Rb[ks][i] = (f16)R[2 * ks][i];
                Rb[ks][4 + i] = (f16)R[2 * ks + 1][i];
            }
        if constexpr (HT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Rbh[i] = (f16)R[NB - 1][i];
        }

        // U = T R
        f32x4 U[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int idx = 0; idx < BK::count(mt); ++idx) {
                const int blk = BK::offset(mt) + idx;
                if (idx < BK::nfull_for(mt)) {
                    const f16x8 ta = *reinterpret_cast<const f16x8*>(Tsw + blk * 512 + lane * 8);
                    u = mma_f16_k32(ta, Rb[idx], u);
                } else {
                    const f16x4 ta = *reinterpret_cast<const f16x4*>(Tsw + blk * 512 + lane * 8);
                    u = mma_f16_k16(ta, Rbh, u);
                }
            }
            U[mt] = u;
        }
        f16x8 Ub[NFT > 0 ? NFT : 1], Wb[NFT > 0 ? NFT : 1];
        f16x4 Ubh, Wbh;
#pragma unroll
        for (int ks = 0; ks < NFT; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t0 = 32 * ks + 4 * g + i, t1 = t0 + 16;
                Ub[ks][i] = (f16)U[2 * ks][i];
                Ub[ks][4 + i] = (f16)U[2 * ks + 1][i];
                Wb[ks][i] = (f16)(scl[3 * C + t0] * U[2 * ks][i]);
                Wb[ks][4 + i] = (f16)(scl[3 * C + t1] * U[2 * ks + 1][i]);
            }
        if constexpr (HT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t0 = 32 * NFT + 4 * g + i;
                Ubh[i] = (f16)U[NB - 1][i];
                Wbh[i] = (f16)(scl[3 * C + t0] * U[NB - 1][i]);
            }
        }

        // O = diag(scale e^g / |q|) Y + A U
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = scl[2 * C + 16 * mt + 4 * g + i] * Y[mt][i];
#pragma unroll
            for (int idx = 0; idx < BK::count(mt); ++idx) {
                const int blk = BK::offset(mt) + idx;
                if (idx < BK::nfull_for(mt)) {
                    const f16x8 aa = *reinterpret_cast<const f16x8*>(Asw + blk * 512 + lane * 8);
                    o = mma_f16_k32(aa, Ub[idx], o);
                } else {
                    const f16x4 aa = *reinterpret_cast<const f16x4*>(Asw + blk * 512 + lane * 8);
                    o = mma_f16_k16(aa, Ubh, o);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * g + i;
                if (t < nval) obase[token(t) * p.os[1]] = (bf16)o[i];
            }
        }

        __syncthreads();   // K^ rows visible to every lane
        // S <- e^{g_C} S + U^T diag(e^{g_C - g}) K^   (computed transposed: rows d, columns r)
        const float gC = scl[5 * C];
#pragma unroll
        for (int m = 0; m < ND; ++m) {
            f32x4 acc = P[m] * gC;
            const f16* kcol = Kh + 16 * m + r;
#pragma unroll
            for (int ks = 0; ks < NFT; ++ks) {
                f16x8 ka;
#pragma unroll
                for (int i = 0; i < 8; ++i) ka[i] = kcol[(32 * ks + 16 * (i >> 2) + 4 * g + (i & 3)) * LDK];
                acc = mma_f16_k32(ka, Wb[ks], acc);
            }
            if constexpr (HT) {
                f16x4 ka;
#pragma unroll
                for (int i = 0; i < 4; ++i) ka[i] = kcol[(32 * NFT + 4 * g + i) * LDK];
                acc = mma_f16_k16(ka, Wbh, acc);
            }
            P[m] = acc;
        }
        __syncthreads();   // LDS is rewritten by the next sub-chunk
    }

    float* Sout = p.S_out[dir];
    if (Sout) {
#pragma unroll
        for (int m = 0; m < ND; ++m) *reinterpret_cast<f32x4*>(Sout + sbase + 16 * m + 4 * g) = P[m];
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
    hipLaunchKernelGGL((gdn_scan_kernel<NB, ND>), dim3(grid), dim3(64), 0, s, p, ngroups);
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
