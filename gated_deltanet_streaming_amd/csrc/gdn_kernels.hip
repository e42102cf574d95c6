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
//    recurrent scan, apply state; Chinese summary "Method steps" step 4).  Here
//    a sequence is cut into processing steps of C tokens and:
//      gdn_prep_kernel  (parallel over steps): per-token L2 norms, the in-step
//        log-gate prefix g, the Gram products K K^T and Q K^T on bf16 MFMA, the
//        UT transform T = (I + L)^{-1} with L[t,s] = beta_t e^{g_t-g_s} k^_t.k^_s
//        (s < t), and from them two step operators that do not depend on the
//        state: E = A T (A = decay-masked in-step attention) and
//        Z = T^T diag(e^{g_C-g}) K^.
//      gdn_scan_kernel  (serial over steps): per (direction, stream, head, 16
//        state rows) one wavefront keeps its state slice in MFMA accumulators
//        for the whole call and per step computes X = K S^T,
//        R = diag(beta) V - diag(beta e^g / |k|) X and S^T <- e^{g_C} S^T + Z^T R;
//        a second wavefront forms O = diag(scale e^g / |q|) Q S^T + E R.
//    The raw bf16 q/k enter the MFMAs unrounded (norms are applied as row
//    scales); the bounded in-step operands E, Z, R use fp16 (11-bit
//    significand), the state enters its products as bf16, everything
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

#include <mutex>
#include <utility>

#include "gdn_internal.h"

// Workspace of the allocation-free entry point (gdn_chunk_bidir_noalloc): the prep/scan items of
// both directions, 2 B H ceil(T / C) of them.  Nothing in it has to start at zero: every item the
// scan reads is written by the prep launch before it on the same stream.
static __device__ __align__(256) unsigned char scratch[gdn::kScratchBytes];

namespace gdn {
// a compile-time int as a value (selects a code path of a generic lambda)
template <int V> struct IConst { static constexpr int value = V; };

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// decays below e^-80 are treated as e^-80 (the state is forgotten either way)
#define GDN_MIN_LOG_DECAY (-80.0f)
#define GDN_PREP_BLOCKS 1   // consecutive sub-chunk blocks per prep workgroup

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

// Order of the state index d in the scan.  The scan keeps S^T in MFMA output tiles
// m = 0..ND-1 (rows j = 0..15); row j of tile m holds d = dperm(m, j).  Within each
// 32-wide block, tile 2c takes d = 32c + 8(j/4) + j%4 and tile 2c+1 takes
// d = 32c + 8(j/4) + 4 + j%4, so that the 8 k-slots a lane group contributes to a
// product over d are 8 consecutive d (one 16-byte load of a bf16 row).  A trailing
// single tile (odd ND) keeps d = 16m + j.
template <int ND>
__host__ __device__ constexpr int dperm(int m, int j) {
    return (m < (ND & ~1)) ? 32 * (m >> 1) + 8 * (j >> 2) + 4 * (m & 1) + (j & 3) : 16 * m + j;
}

// workspace item of one processing step (written by the prep, read by the scan): [T~ fragments:
// TOTAL blocks][A^T fragments: TOTAL blocks][scalars c1[C], w[C], c2[C], gamma_C], 1 KB per
// fragment block (64 lanes x 16 bytes), the scalars in a 1 KB block of their own
template <int NB>
__host__ __device__ constexpr int64_t item_bytes_t() {
    return 1024 * (int64_t)(2 * Blocks<NB>::TOTAL + 1);
}

int64_t chunk_item_bytes(int C, int D) {
    if (!(D == 16 || D == 32 || D == 64 || D == 112 || D == 128)) return -1;
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

// Lane exchange within a row of 16 lanes (DPP).  Lanes whose source is out of range, or
// whose row is masked off, read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
// out[n] = x of lane n of the lane's row of 16, n = 0..15 (row broadcasts)
template <int... Is>
__device__ __forceinline__ void row_broadcasts(float x, float* out, std::integer_sequence<int, Is...>) {
    ((out[Is] = dpp<0x150 + Is>(x)), ...);
}
// sum over the 4 lanes of a quad (quad permutations [1,0,3,2] and [2,3,0,1])
__device__ __forceinline__ float sum4(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    return x;
}
// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each row of 16, then
// the last lane of row 0 into row 1 and of row 2 into row 3, then lane 31 into rows 2 and 3
__device__ __forceinline__ float wave_prefix(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    x += dpp<0x142, 0xa>(x);
    x += dpp<0x143, 0xc>(x);
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
        const float at = p.gate_log ? expf(p.a[gq]) : p.a[gq], bt = p.beta[gq];
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

// A 16-byte store through the global address space.  A store through a generic pointer is
// a flat store, which also counts against the LDS wait counter: every later wait for an LDS
// read would then wait for the store to reach memory as well.
__device__ __forceinline__ void gstore16(void* p, uint4 v) {
    *(__attribute__((address_space(1))) u32x4*)p = __builtin_bit_cast(u32x4, v);
}

// LDS-only barrier: orders LDS traffic between the wavefronts of a workgroup
// without waiting for global loads that are still in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Compact LDS storage of the C x C matrices of a step by 16x16 blocks: only the
// blocks on one side of the diagonal are kept (rows padded to 16-byte multiples).
template <int NB>
struct UpperF16 {   // fp16 blocks (a, b) with a <= b (L^T), rows of 16 halves
    static constexpr int COUNT = NB * (NB + 1) / 2, HALVES = COUNT * 256;
    __device__ static int at(int row, int col) {
        const int a = row >> 4, b = col >> 4;
        return (a * NB - (a * (a - 1)) / 2 + (b - a)) * 256 + (row & 15) * 16 + (col & 15);
    }
};
template <int NB>
struct UpperF16S {  // fp16 blocks (a, b) with a <= b (T^T), rows of 16 halves, chunks of rows 8..15 swapped
    static constexpr int COUNT = NB * (NB + 1) / 2, HALVES = COUNT * 256;
    __device__ static int at(int row, int col) {
        const int a = row >> 4, b = col >> 4;
        return (a * NB - (a * (a - 1)) / 2 + (b - a)) * 256 + (row & 15) * 16 + ((((col & 15) >> 3) ^ ((row >> 3) & 1)) << 3) + (col & 7);
    }
};
template <int NB>
struct LowerF16 {   // fp16 blocks (a, b) with a >= b (A), rows of 16 halves; the two 8-half
                    // chunks of rows 8..15 swapped (16-byte row reads free of bank conflicts)
    static constexpr int COUNT = NB * (NB + 1) / 2, HALVES = COUNT * 256;
    __device__ static int at(int row, int col) {
        const int a = row >> 4, b = col >> 4;
        return ((a * (a + 1)) / 2 + b) * 256 + (row & 15) * 16 + ((((col & 15) >> 3) ^ ((row >> 3) & 1)) << 3) + (col & 7);
    }
};

// Stream-heads bh = b H + h are spread over the 8 XCDs in contiguous ranges (workgroup id % 8 is
// the XCD a workgroup runs on): XCD x takes bh in [first(x), first(x + 1)), first(x) =
// ceil(x BH / 8).  Neighbouring heads share the cache lines of a token's row, so a contiguous
// range reads each line into one L2.  Returns the k-th stream-head of XCD x, or -1.
__device__ __forceinline__ int xcd_head(int x, int k, int BH) {
    const int first = (x * BH + 7) / 8, next = ((x + 1) * BH + 7) / 8;
    return k < next - first ? first + k : -1;
}

// ---------------------------------------------------------------------------
// Chunk preparation: one workgroup (2 NB wavefronts) per (b, h, block j of C
// tokens), for every requested direction at once.  The forward direction
// processes block j as its step j, the reverse direction as its step N-1-j
// (the blocks of the two directions coincide; the padding of a ragged sequence
// lies beyond T-1 in both).  Shared by the directions: the K and Q rows, their
// norms, the in-block log-gate prefix and the Gram products K K^T and Q K^T
// (the forward direction takes their lower triangles, the reverse direction
// the upper ones).  Per direction, in its processing order p (token j C + p
// forward, j C + C-1-p reverse), with k^ = k/|k|, q^ = q/|q|, g = prefix of
// log a along p and gamma = e^g:
//   L[t,s] = beta_t e^{g_t-g_s} k^_t.k^_s (s < t),   T = (I + L)^{-1}
//   A[t,s] = scale e^{g_t-g_s} q^_t.k^_s (s <= t)
// and it stores, per direction and step, the step operators the scan needs:
//   T~ = T diag(beta)       (the UT transform: U = T~ R for the step's R)
//   A                        (the decay-masked in-step attention: O += A U)
//   c1 = gamma/|k|, w = e^{g_C-g}/|k|, c2 = scale gamma/|q|, gamma_C.
// L, A and T are held in fp16 (T is built in fp32 arithmetic from fp16 blocks);
// T~ and A leave as fp16 MFMA fragments, the scalars in fp32.
// ---------------------------------------------------------------------------
template <int NB, int ND>
__global__ __launch_bounds__(128 * NB) __attribute__((amdgpu_waves_per_eu(8))) void gdn_prep_kernel(Params p) {
    constexpr int C = 16 * NB, D = 16 * ND;
    using UL = UpperF16<NB>;     // L^T per direction
    using US = UpperF16S<NB>;    // T^T per direction
    using LB = LowerF16<NB>;     // A per direction (over L^T once T is built)
    static_assert(UL::HALVES == LB::HALVES, "A reuses the storage of L^T");
    constexpr int NW = 2 * NB;   // wavefronts
    constexpr int NT = 64 * NW;
    constexpr int CH = D / 8;    // 16-byte chunks per row
    using BK = Blocks<NB>;
    typedef short s16x4 __attribute__((ext_vector_type(4)));

    // K and Q rows (bf16, D per row, token order).  Row t holds its 16-byte chunk c at position
    // c ^ sw(t, c): the chunks of the 32-wide k-steps are permuted within their group of four by
    // (t >> 2) & 3, the two chunks of a trailing 16-wide step swap for rows with bit 3 set.  With
    // this layout the MFMA operand reads (16 consecutive rows at one column, 16- and 8-byte) are
    // free of LDS bank conflicts on gfx950 (measured; a swap by bit 3 alone leaves the 16-byte
    // reads two-way conflicted).  The Q rows are dead after the Gram products; T^T of both
    // directions then takes their storage.
    constexpr int CHF = 4 * (ND / 2);   // chunks of the 32-wide k-steps
    auto kq_tail = [](int t, int d) { return t * D + (((d >> 3) ^ ((t >> 3) & 1)) << 3) + (d & 7); };   // d >= 8 CHF
    auto kq = [](int t, int d) {
        const int c = d >> 3, sw = c < CHF ? ((t >> 2) & 3) : ((t >> 3) & 1);
        return t * D + ((c ^ sw) << 3) + (d & 7);
    };
    constexpr int Q_BYTES = C * D * 2, T2_BYTES = 2 * US::HALVES * 2;
    constexpr int QT_BYTES = Q_BYTES > T2_BYTES ? Q_BYTES : T2_BYTES;
    __shared__ __align__(16) bf16 Ks[C * D];
    __shared__ __align__(16) char QT[QT_BYTES];
    __shared__ __align__(16) f16 LA[2 * UL::HALVES];  // L^T per direction, then A per direction
    __shared__ __align__(16) float sg[2][C];          // by token: forward, reverse inclusive log2-gate prefix
    __shared__ __align__(16) float rk[C], rq[C];      // by token: 1/|k|, 1/|q|
    __shared__ __align__(16) float bp[2][C];          // beta by processing row (forward = token order)
    bf16* Qs = reinterpret_cast<bf16*>(QT);

    // the wavefront index is uniform: in a scalar register, so that everything derived from
    // it (tile and job assignment, addresses) is scalar work
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    // XCD-aware order: the blocks of stream-head bh run on its XCD (xcd_head), where the scan
    // workgroups of both directions of that head run, so that the items land in the L2 they are
    // read from
    const int nsub = (int)((p.T + C - 1) / C);
    const int ngrp = (nsub + GDN_PREP_BLOCKS - 1) / GDN_PREP_BLOCKS;   // block groups per stream-head
    // (for a time split, whose point is to use the whole chip when the stream-heads are few, the
    // blocks are spread over all XCDs instead)
    const int xcd = blockIdx.x & 7, kk = p.seg_mode ? (int)blockIdx.x : (int)(blockIdx.x >> 3);
    const int jg = kk % ngrp;
    const int bh = p.seg_mode ? (kk / ngrp < p.B * p.H ? kk / ngrp : -1) : xcd_head(xcd, kk / ngrp, p.B * p.H);
    if (bh < 0) return;
    const int b = bh / p.H, h = bh - b * p.H;
    const int T = (int)p.T;
    const int N = (T + C - 1) / C;
    const int dlo = p.dir0, dhi = p.dir0 + p.ndirs - 1;
    auto active = [&](int dir) { return dir >= dlo && dir <= dhi; };
    // token row (within the block) of processing row t
    auto mrow = [](int dir, int t) { return dir ? C - 1 - t : t; };
    // The global loads of a block: its gates (threads < C) and its K and Q rows (16-byte chunks,
    // NLD per thread), into registers.  A workgroup takes GDN_PREP_BLOCKS consecutive blocks; the
    // loads of the next block go out before the work on the current one starts, so that their
    // latency hides behind it.
    const bf16* kb = reinterpret_cast<const bf16*>(p.k) + (int64_t)b * p.ks[0] + (int64_t)h * p.ks[2];
    const bf16* qb = reinterpret_cast<const bf16*>(p.q) + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[2];
    const auto kr = make_rsrc(kb, (uint32_t)(((int64_t)(T - 1) * p.ks[1] + D) * 2));
    const auto qr = make_rsrc(qb, (uint32_t)(((int64_t)(T - 1) * p.qs[1] + D) * 2));
    const int ksb = (int)p.ks[1] * 2, qsb = (int)p.qs[1] * 2;
    constexpr int NLD = (C * CH + NT - 1) / NT;
    float av = 1.f, bt = 0.f;
    bool gv = false;
    uint4 kv[NLD], qv[NLD];
    auto load_block = [&](int jb) {
        av = 1.f;
        bt = 0.f;
        gv = false;
        if (tid < C) {
            const int tk = jb * C + tid;
            gv = tk < T;
            if (gv) {
                const int64_t gq = (int64_t)b * p.gs[0] + (int64_t)tk * p.gs[1] + (int64_t)h * p.gs[2];
                av = p.a[gq];
                bt = p.beta[gq];
            }
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int idx = tid + i * NT;
            if (idx < C * CH) {
                const int t = idx / CH, c = idx - t * CH;
                const int tk = jb * C + t;
                kv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, tk * ksb + 16 * c, 0, 0));
                qv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, tk * qsb + 16 * c, 0, 0));
            }
        }
    };
    load_block(jg * GDN_PREP_BLOCKS);

#pragma unroll
    for (int it = 0; it < GDN_PREP_BLOCKS; ++it) {
    const int j = jg * GDN_PREP_BLOCKS + it;
    if (j >= nsub) break;
    if (it > 0) lds_barrier();   // every read of the previous block's LDS data is done
    // this block's item in either direction
    char* const item_f = p.ws + ((((int64_t)0 * p.B + b) * p.H + h) * p.nsub_max + j) * p.ws_item_bytes;
    char* const item_r = p.ws + ((((int64_t)1 * p.B + b) * p.H + h) * p.nsub_max + (N - 1 - j)) * p.ws_item_bytes;
    auto item_of = [&](int dir) { return dir ? item_r : item_f; };

    if (tid < C) {
        sg[0][tid] = gv ? fmaxf(p.gate_log ? av : logf(av), GDN_MIN_LOG_DECAY) : 0.f;   // log a until the prefix
        bp[0][tid] = bt;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int idx = tid + i * NT;
        if (idx < C * CH) {
            const int t = idx / CH, c = idx - t * CH;
            *reinterpret_cast<uint4*>(Ks + kq(t, 8 * c)) = kv[i];
            *reinterpret_cast<uint4*>(Qs + kq(t, 8 * c)) = qv[i];
        }
    }
    if (it + 1 < GDN_PREP_BLOCKS && j + 1 < nsub) load_block(j + 1);
    lds_barrier();

    // per-token inverse norms: 4 lanes per row, 16 rows per wavefront; waves < NB take the
    // K rows, the others the Q rows
    {
        const bool isk = w < NB;
        const int t = 16 * (isk ? w : w - NB) + (lane >> 2), part = lane & 3;
        const bf16* rows = isk ? Ks : Qs;
        float ss = 0.f;
        for (int c = part; c < CH; c += 4) {
            const bf16x8 xv = ld_bf16x8(rows + kq(t, 8 * c));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xf = (float)xv[e];
                ss += xf * xf;
            }
        }
        ss = sum4(ss);
        // rows past the end of the sequence (zero k and q) get zero scales: nothing of them
        // reaches a product, whatever eps is
        const bool tv = j * C + t < T;
        if (part == 0) (isk ? rk : rq)[t] = !tv ? 0.f : p.l2norm ? 1.f / sqrtf(ss + p.eps) : 1.f;
    }
    // inclusive prefixes of log a within the block (C <= 64: one wavefront), in base-2 units
    // (every decay below is an exp2 of a difference of these): forward over tokens <= t,
    // reverse over tokens >= t
    if (w == 0) {
        const float la = (lane < C) ? sg[0][lane] * 1.4426950408889634f : 0.f;
        const float x = wave_prefix(la);
        const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), C - 1));
        if (lane < C) {
            sg[0][lane] = x;
            sg[1][lane] = tot - x + la;
        }
    }
    lds_barrier();

    // per direction and processing row: beta, and the step's scalars c1 = gamma/|k| and
    // w = e^{g_C-g}/|k| (processing order), c2 = scale gamma/|q| (token 16 mt + r at r * NB + mt:
    // one vector load per lane of the scan's output wavefront) and gamma_C
    if (tid < 2 * C) {
        const int dir = tid / C, pr = tid - dir * C;
        if (active(dir)) {
            const int t = mrow(dir, pr);
            const float g2 = sg[dir][t], gtot = sg[0][C - 1];
            const float gam = __builtin_amdgcn_exp2f(g2);
            if (dir) bp[1][pr] = bp[0][t];
            float* scw = reinterpret_cast<float*>(item_of(dir) + 1024 * 2 * BK::TOTAL);
            scw[pr] = gam * rk[t];
            scw[C + pr] = __builtin_amdgcn_exp2f(gtot - g2) * rk[t];
            scw[2 * C + (pr & 15) * NB + (pr >> 4)] = p.scale * gam * rq[t];
            if (pr == 0) scw[3 * C] = __builtin_amdgcn_exp2f(gtot);
        }
    }

    // Gram tiles on MFMA (token-order tiles: rows t = 16 mt + 4 g + i, column s = 16 nt + r).
    //   Q K^T, all tiles a direction needs (forward s <= t, reverse s >= t): scale e^{g_t-g_s}
    //     q^_t.k^_s with the direction's prefix, computed transposed (lane: column t, rows
    //     s = 16 nt + 4 g + i) and kept in registers until L is no longer needed.
    //   K K^T, tiles mt >= nt: forward L[t][s] = beta_t e^{g_t-g_s} k^_t.k^_s (s < t), stored
    //     transposed; the reverse direction takes the mirror entry (processing rows C-1-s >
    //     C-1-t) with its own prefix.
    constexpr int NQ = NB * NB, TPQ = (NQ + NW - 1) / NW;
    constexpr int NKK = NB * (NB + 1) / 2, TPK = (NKK + NW - 1) / NW;
    auto q_needed = [&](int mt, int nt) { return (mt >= nt && active(0)) || (mt <= nt && active(1)); };
    f16x4 qa[TPQ];
    // operands of one Gram tile: A = rows arow of `arows`, B = K rows brow; chunk 4 ks + g of a
    // row sits at 4 ks + (g ^ ((row >> 2) & 3))
    auto gram = [&](int arow, int brow, const bf16* arows, const bf16* brows) {
        bf16x8 aop[ND / 2 > 0 ? ND / 2 : 1], bop[ND / 2 > 0 ? ND / 2 : 1];
        bf16x4 aoh, boh;
        const bf16* ap = arows + arow * D + ((g ^ ((arow >> 2) & 3)) << 3);
        const bf16* bpp = brows + brow * D + ((g ^ ((brow >> 2) & 3)) << 3);
#pragma unroll
        for (int ks = 0; ks < ND / 2; ++ks) {
            aop[ks] = ld_bf16x8(ap + 32 * ks);
            bop[ks] = ld_bf16x8(bpp + 32 * ks);
        }
        if constexpr (ND % 2) {
            aoh = ld_bf16x4(arows + kq_tail(arow, 32 * (ND / 2) + 4 * g));
            boh = ld_bf16x4(brows + kq_tail(brow, 32 * (ND / 2) + 4 * g));
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < ND / 2; ++ks) acc = mma_bf16_k32(aop[ks], bop[ks], acc);
        if constexpr (ND % 2) acc = mma_bf16_k16(aoh, boh, acc);
        return acc;
    };
#pragma unroll
    for (int it = 0; it < TPQ; ++it) {
        const int qi = w + it * NW;
        qa[it] = f16x4{(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
        if (qi < NQ) {
            const int mt = qi / NB, nt = qi - mt * NB;
            if (q_needed(mt, nt)) {
                const f32x4 acc = gram(16 * nt + r, 16 * mt + r, Ks, Qs);
                const int t = 16 * mt + r, s0 = 16 * nt + 4 * g;
                const f32x4 gf = *reinterpret_cast<const f32x4*>(&sg[0][s0]);
                const f32x4 gr = *reinterpret_cast<const f32x4*>(&sg[1][s0]);
                const f32x4 rs = *reinterpret_cast<const f32x4*>(&rk[s0]);
                const float gft = sg[0][t], grt = sg[1][t], rt = rq[t] * p.scale;
                if (mt != nt) {
                    // the whole tile belongs to one direction (forward below the diagonal)
                    const f32x4 gd = mt > nt ? gft - gf : grt - gr;
#pragma unroll
                    for (int i = 0; i < 4; ++i) qa[it][i] = (f16)(acc[i] * (rt * rs[i]) * __builtin_amdgcn_exp2f(gd[i]));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = s0 + i;
                        const bool fw = s <= t;   // forward prefix (on the diagonal both give e^0)
                        const bool ok = s == t || (fw ? active(0) : active(1));
                        const float v = acc[i] * (rt * rs[i]) * __builtin_amdgcn_exp2f(fw ? gft - gf[i] : grt - gr[i]);
                        qa[it][i] = (f16)(ok ? v : 0.f);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int it = 0; it < TPK; ++it) {
        const int kt = (NW - 1 - w) + it * NW;
        if (kt < NKK) {
            int mt = 0;
            while ((mt + 1) * (mt + 2) / 2 <= kt) ++mt;
            const int nt = kt - mt * (mt + 1) / 2;
            const f32x4 acc = gram(16 * mt + r, 16 * nt + r, Ks, Ks);
            const int s = 16 * nt + r, t0 = 16 * mt + 4 * g;
            const f32x4 rt = *reinterpret_cast<const f32x4*>(&rk[t0]);
            const float rs = rk[s];
            if (active(0)) {
                const f32x4 gt = *reinterpret_cast<const f32x4*>(&sg[0][t0]);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&bp[0][t0]);
                const float gs = sg[0][s];
                f16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (f16)((s < t0 + i) ? acc[i] * (rt[i] * rs * bt[i]) * __builtin_amdgcn_exp2f(gt[i] - gs) : 0.f);
                *reinterpret_cast<f16x4*>(LA + UL::at(s, t0)) = v;
            }
            if (active(1)) {
                // entries with s >= t (diagonal tiles only) land at row >= column of the mirrored
                // diagonal block, a part nothing reads: stored without a branch; the mirrored
                // rows C-1-t0-i of one lane are consecutive rows of one 16x16 block
                const f32x4 gt = *reinterpret_cast<const f32x4*>(&sg[1][t0]);
                const float gs = sg[1][s], bs = bp[0][s];
                f16* Lr = LA + UL::HALVES + UL::at(C - 1 - t0, C - 1 - s);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Lr[-16 * i] = (f16)(acc[i] * (rt[i] * rs * bs) * __builtin_amdgcn_exp2f(fminf(gs - gt[i], 0.f)));
            }
        }
    }
    lds_barrier();

    // T = (I + L)^{-1} per direction, built transposed in processing order.  16x16 diagonal
    // blocks: one lane per (direction, block, column j), right-looking forward substitution in
    // fp32; column j of T_bb is row j of T^T.
    if (tid < 2 * C) {
        const int dir = tid / C, tl = tid - dir * C;
        if (active(dir)) {
            const f16* Lt = LA + dir * UL::HALVES;
            f16* T16 = reinterpret_cast<f16*>(QT) + dir * US::HALVES;
            const int o = 16 * (tl >> 4), jc = tl & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == jc) ? 1.f : 0.f;
#pragma unroll
            for (int k = 0; k < 15; ++k) {
                const f16* lcol = Lt + UL::at(o + k, o);   // L[o + i][o + k] for i > k
                float lv[16];
#pragma unroll
                for (int i8 = 0; i8 < 2; ++i8) {
                    const f16x8 v8 = *reinterpret_cast<const f16x8*>(lcol + 8 * i8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) lv[8 * i8 + e] = (float)v8[e];
                }
#pragma unroll
                for (int i = k + 1; i < 16; ++i) x[i] -= lv[i] * x[k];
            }
#pragma unroll
            for (int i8 = 0; i8 < 2; ++i8) {
                f16x8 v8;
#pragma unroll
                for (int e = 0; e < 8; ++e) v8[e] = (f16)x[8 * i8 + e];
                *reinterpret_cast<f16x8*>(T16 + US::at(o + jc, o + 8 * i8)) = v8;
            }
        }
    }
    lds_barrier();
    // off-diagonal blocks, by distance d from the diagonal (one wavefront per direction and
    // block), on fp16 MFMA: z = sum_{k=j}^{i-1} L_ik T_kj with two 16-blocks of k per product,
    // then T_ij = -T_ii z.  L_ik and T_ii are read transposed from their transposed storage
    // (lane r of a group supplies row r/4 and columns 4 (r%4) .. +3 of a 4x16 block and
    // receives column r).
    for (int d = 1; d < NB; ++d) {
        const int dir = w / NB, wl = w - dir * NB;
        if (active(dir) && wl < NB - d) {
            const f16* Lt = LA + dir * UL::HALVES;
            f16* T16 = reinterpret_cast<f16*>(QT) + dir * US::HALVES;
            const int ib = wl + d, jb = wl;
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int kb0 = jb; kb0 < ib; kb0 += 2) {
                // k-slots of group g: block kb0 + g/2, rows 8 (g%2) .. +7
                const int kb = kb0 + (g >> 1), k0 = 16 * kb + 8 * (g & 1);
                f16x8 ao, bo;
                if (kb < ib) {
                    const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(Lt + UL::at(k0 + (r >> 2), 16 * ib + 4 * (r & 3))));
                    const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(Lt + UL::at(k0 + 4 + (r >> 2), 16 * ib + 4 * (r & 3))));
                    const f16x4 a0h = __builtin_bit_cast(f16x4, a0), a1h = __builtin_bit_cast(f16x4, a1);
                    ao = f16x8{a0h[0], a0h[1], a0h[2], a0h[3], a1h[0], a1h[1], a1h[2], a1h[3]};   // L[16 ib + r][k0 ..]
                    bo = *reinterpret_cast<const f16x8*>(T16 + US::at(16 * jb + r, k0));            // T[k0 ..][16 jb + r]
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) ao[e] = bo[e] = (f16)0.f;
                }
                z = mma_f16_k32(ao, bo, z);
            }
            // z: lane (column r, group g) holds z[4g + e][16 jb + r], the B operand of
            // T_ii z with k = 4g + e (upper slots zero); A = T[16 ib + r][16 ib + 4g + e]
            const s16x4 ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(T16 + US::at(16 * ib + 4 * g + (r >> 2), 16 * ib + 4 * (r & 3))));
            const f16x4 tah = __builtin_bit_cast(f16x4, ta);
            const f16 z0 = (f16)0.f;
            const f16x8 a2 = {tah[0], tah[1], tah[2], tah[3], z0, z0, z0, z0};
            const f16x8 b2 = {(f16)z[0], (f16)z[1], (f16)z[2], (f16)z[3], z0, z0, z0, z0};
            const f32x4 t4 = mma_f16_k32(a2, b2, f32x4{0.f, 0.f, 0.f, 0.f});
            // T[16 ib + 4g + e][16 jb + r] -> T^T[16 jb + r][16 ib + 4g + e]
            *reinterpret_cast<f16x4*>(T16 + US::at(16 * jb + r, 16 * ib + 4 * g)) =
                f16x4{(f16)-t4[0], (f16)-t4[1], (f16)-t4[2], (f16)-t4[3]};
        }
        lds_barrier();
    }

    // A per direction in processing order (lower incl. the diagonal) over the dead L^T: the
    // forward direction's entries in place, the reverse direction's mirrored; the diagonal
    // blocks are written whole (zero above the diagonal)
#pragma unroll
    for (int it = 0; it < TPQ; ++it) {
        const int qi = w + it * NW;
        if (qi < NQ) {
            const int mt = qi / NB, nt = qi - mt * NB;
            const int t = 16 * mt + r, s0 = 16 * nt + 4 * g;
            if (mt >= nt && active(0)) {
                f16x4 v = qa[it];
                if (mt == nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (s0 + i <= t) ? v[i] : (f16)0.f;
                }
                *reinterpret_cast<f16x4*>(LA + LB::at(t, s0)) = v;
            }
            if (mt <= nt && active(1)) {
                f16x4 v = {qa[it][3], qa[it][2], qa[it][1], qa[it][0]};   // processing columns C-4-s0 .. C-1-s0
                if (mt == nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (s0 + 3 - i >= t) ? v[i] : (f16)0.f;
                }
                *reinterpret_cast<f16x4*>(LA + LB::HALVES + LB::at(C - 1 - t, C - 4 - s0)) = v;
            }
        }
    }
    lds_barrier();

    // T~ = T diag(beta) (A operand of U = T~ R) and A^T (B operand of O^T += U^T A^T) of each
    // direction as fp16 MFMA fragments.  Fragment (mt, ks) holds in lane r + 16 g row (T~) or
    // column (A^T) t = 16 mt + r and the k-slots e = 0..7 of group g, s = 32 ks + 16 (e / 4) +
    // 4 g + e % 4: the slot order of MFMA output tiles, so that the scan's U tiles meet them
    // without a shuffle.  Blocks of s past the diagonal block of t (or past C) are zero.
    {
        constexpr int NF = BK::TOTAL;
        struct FBlocks { int mt[NF], ks[NF]; };
        constexpr FBlocks fb = [] {
            FBlocks e{};
            int k = 0;
            for (int m = 0; m < NB; ++m)
                for (int s2 = 0; s2 < BK::count(m); ++s2) { e.mt[k] = m; e.ks[k] = s2; ++k; }
            return e;
        }();
        for (int job = w; job < 4 * NF; job += NW) {
            const int dir = job / (2 * NF), kind = (job / NF) & 1, f = job - (job / NF) * NF;
            if (!active(dir)) continue;
            const int mt = fb.mt[f], ks = fb.ks[f];
            const f16* T16 = reinterpret_cast<const f16*>(QT) + dir * US::HALVES;
            const f16* Am = LA + dir * LB::HALVES;
            f16x8 v;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int sb = 2 * ks + hf;   // 16-block of s
                f16x4 x = {(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
                if (sb <= mt) {
                    if (kind == 0) {
                        // T[t][s] for s = 16 sb + 4 g + i: column t of T^T, rows s (transposing read;
                        // lane r of the group supplies row 16 sb + 4 g + r/4, columns 16 mt + 4 (r%4) ..)
                        const s16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4*)(T16 + US::at(16 * sb + 4 * g + (r >> 2), 16 * mt + 4 * (r & 3))));
                        const f16x4 th = __builtin_bit_cast(f16x4, tv);
                        const f32x4 bs = *reinterpret_cast<const f32x4*>(&bp[dir][16 * sb + 4 * g]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] = (f16)((float)th[i] * bs[i]);
                    } else {
                        x = *reinterpret_cast<const f16x4*>(Am + LB::at(16 * mt + r, 16 * sb + 4 * g));
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) v[4 * hf + i] = x[i];
            }
            gstore16(item_of(dir) + (kind * NF + f) * 1024 + 16 * lane, __builtin_bit_cast(uint4, v));
        }
    }
    }   // blocks of the workgroup
}

// ---------------------------------------------------------------------------
// Chunk scan: one workgroup per (direction, b, h, slice of 32 state rows),
// serial over the processing steps.  Rows of S evolve independently, so the
// slices of a head need no exchange.  Per step n with state S (its slice):
//   X = K S^T,  R = V - diag(c1) X,  U = T~ R            (U: the step's u_t rows)
//   O = diag(c2) Q S^T + A U,        S^T <- gamma_C S^T + K^T diag(w) U
// Six wavefronts with fixed roles:
//   chain (2, one per 16-row column tile of the slice): the recurrence; the
//                     state tile lives in MFMA accumulators for the whole call.
//                     Each step's state (bf16) and U (fp16) go to an LDS ring.
//   output (2, one per half of the step's token tiles): O from the ring, the
//                     step's Q rows, and A and c2 (loaded two steps ahead);
//                     bf16 tiles leave through LDS staging.
//   loader (2): copy each step's operands from memory into a 3-slot operand
//                     ring through registers (16-byte buffer loads, then
//                     16-byte LDS stores; two steps in flight):
//                     loader 0 the K rows, the V slice, T~ and the scalars,
//                     loader 1 the Q rows.
// The wavefronts are coupled only through the rings and LDS counters with
// bounded spins.  K and Q rows are stored in processing order with the chunk
// permutation of the prep (conflict-free 16-byte row reads and transposing
// 8-byte reads); the loaders realise it by the source address each lane loads.
// An operand register of an MFMA is refilled only after a result depending on
// that MFMA has been consumed.
//
// Row addressing: the buffer resource of a step starts at the lowest token of
// the step and ends after the last real token, so a row's byte offset is a
// per-lane constant and rows past the end of the sequence read as zero (and
// are not stored).  State rows past d_v (the last slice when d_v is not a
// multiple of 32) are computed from zero inputs and never stored.
// ---------------------------------------------------------------------------
#define GDN_COLS 2       // 16-row column tiles of the state per workgroup
#define GDN_OPS 3        // operand ring slots
#define GDN_RING 2       // output ring slots

template <int NB, int ND>
struct ScanGeom {
    static constexpr int C = 16 * NB, D = 16 * ND;
    static constexpr int CH = 2 * ND;                        // 16-byte chunks of a K or Q row
    static constexpr int CHF = 4 * (ND / 2);                 // chunks of the 32-wide k-steps
    static constexpr int NKD = (ND + 1) / 2, NKF = ND / 2;   // k-steps over d (the last half for odd ND)
    using BK = Blocks<NB>;
    static constexpr int NKT = BK::NFULL + (BK::HALF ? 1 : 0);   // 32-wide k-steps over tokens
    static constexpr int NF = BK::TOTAL;                     // T~ (A) fragments of a step
    static constexpr int NLK = (C * CH + 63) / 64;           // loads of one block of K (Q) rows
    static constexpr int NLV = (C * 4 + 63) / 64;            // loads of one V slice
    static constexpr int ITEM_SC = 2 * NF * 1024;            // scalars in an item: c1[C], w[C], c2[C], gamma_C
    static constexpr int NOUT = NB >= 2 ? 2 : 1;             // output wavefronts
    static constexpr int TPO = NB / NOUT;                    // token tiles per output wavefront
    static constexpr int THREADS = 64 * (GDN_COLS + NOUT + 2);
    static constexpr int NLD0 = NLK + NLV + NF + 1;          // loads per step, loader 0
    static constexpr int NLD1 = NLK;                         // loads per step, loader 1
    // byte offset of (row t, state index d) in a block of K or Q rows: chunk c of row t sits at
    // c ^ sw(t, c) (the prep's permutation)
    __host__ __device__ static constexpr int sw(int t, int c) { return c < CHF ? ((t >> 2) & 3) : ((t >> 3) & 1); }
    __host__ __device__ static constexpr int kq(int t, int d) {
        return t * 2 * D + 16 * ((d >> 3) ^ sw(t, d >> 3)) + 2 * (d & 7);
    }
};

// One step's operands in LDS (16-byte aligned areas; K, Q and V rounded up to whole loads).
template <int NB, int ND>
struct ScanSlot {
    using G = ScanGeom<NB, ND>;
    uint4 k[G::NLK][64];        // K rows
    uint4 q[G::NLK][64];        // Q rows
    uint4 v[G::NLV][64];        // V slice: token t's 64 bytes at 64 t, chunk j at j ^ vswz(t)
    uint4 tt[G::NF][64];        // T~ fragments
    uint4 sc[64];               // c1[C], w[C], c2[C] (lane-major), gamma_C
};

template <int NB, int ND>
struct ScanLds {
    using G = ScanGeom<NB, ND>;
    ScanSlot<NB, ND> ops[GDN_OPS];
    uint4 ringS[GDN_RING][G::NKD][GDN_COLS][64];   // state slice, bf16 A-operand fragments of S Q^T
    uint4 ringU[GDN_RING][G::NKT][GDN_COLS][64];   // U, fp16 A-operand fragments of U^T A^T
    uint4 ostage[G::NOUT][G::TPO][64];             // bf16 output tiles on their way out
};

// Progress counters of the scan's wavefronts (an LDS object of their own).
struct ScanCtr {
    int ready[GDN_COLS];   // steps each chain wavefront has published to the output ring
    int cdone[GDN_COLS];   // steps each chain wavefront has finished reading from the operand ring
    int rdone[2];          // steps each output wavefront has taken from the output ring
    int odone[2];          // steps each output wavefront has finished reading from the operand ring
    int loaded[2];         // steps whose operands loader 0 / loader 1 has landed
};

// A token's 64-byte slice (32 state rows, bf16) in LDS holds its 16-byte chunk j at position
// j ^ vswz(t): tokens 4 apart land on different banks for the chain's transposing reads
// and the output tiles' writes, while each lane quad moves one token's 64 contiguous bytes.
__device__ __forceinline__ int vswz(int t) { return 2 * ((t >> 2) & 1); }
__device__ __forceinline__ int oswz(int t) { return (t >> 2) & 3; }

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

// Wait until an LDS counter written by another wavefront reaches `target`.  Bounded, so a
// wavefront can never hang here: after `limit` polls it records the give-up in the error word
// (host memory the library reads on the handle's next call) and goes on.  The chain wavefronts
// poll without sleeping (a hand-off is seen one LDS round trip after it happens); the others
// sleep ~64 cycles between polls, so that their polls do not take LDS issue slots from a chain
// wavefront on the same SIMD.
template <bool SLEEP>
__device__ __forceinline__ void wait_counter(int* cnt, int target, int limit, int* err) {
    int it = 0;
    for (; it < limit; ++it) {
        if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        if constexpr (SLEEP) __builtin_amdgcn_s_sleep(1);
    }
    if (it == limit && err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Set a counter once this wavefront's earlier LDS reads and writes have taken effect.  The LDS
// performs the operations of one wavefront in the order they were issued, so a counter store
// issued after them is seen by another wavefront only once they are done: the store needs to
// stay behind them in the instruction stream (an instruction of its own with a memory
// clobber), not to wait for them.
__device__ __forceinline__ void signal_counter(int* cnt, int value) {
    const unsigned addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)cnt;
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(value) : "memory");
}
// s_waitcnt on the vector memory counter only (gfx9 encoding: expcnt and lgkmcnt at their maxima)
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
}

// Output wavefront `O`: token tiles out_tile(O, 0 .. TPO-1) of every step.  With two tiles each,
// wavefront O takes tiles O and NB-1-O, so both carry the same number of A fragments (a tile's
// fragments grow with its distance from the start of the step).
template <int NB>
__host__ __device__ constexpr int out_tile(int O, int tt) {
    return ScanGeom<NB, 1>::TPO == 2 ? (tt == 0 ? O : NB - 1 - O) : O * ScanGeom<NB, 1>::TPO + tt;
}

template <int NB, int ND, int O>
__device__ __forceinline__ void scan_output(const Params& p, ScanLds<NB, ND>& L, ScanCtr& K, int lane, int b, int h, int dir, int T,
                                            int N, int row0, const char* item0, int64_t ib, int t0, int To) {
    using G = ScanGeom<NB, ND>;
    constexpr int C = G::C, D = G::D, NKD = G::NKD, NKF = G::NKF, NKT = G::NKT, NF = G::NF, TPO = G::TPO;
    using BK = Blocks<NB>;
    const int r = lane & 15, g = lane >> 4;
    // A fragments of this wavefront's tiles, tile after tile
    constexpr auto aoff = [](int tt) { int o = 0; for (int t2 = 0; t2 < tt; ++t2) o += BK::count(out_tile<NB>(O, t2)); return o; };
    constexpr int AB = aoff(TPO);
    struct OutIn {
        uint4 afr[AB];
        float c2[TPO];
    };
    // o is bf16, or fp32 when the call's I/O is fp32 (its q, k, v were staged as bf16)
    const int oesz = p.io_f32 ? 4 : 2;
    // (To = 0 for the first stage of a time split: a resource of no rows drops every store)
    const StepRows orow{reinterpret_cast<const char*>(p.o[dir]) + ((int64_t)b * p.os[0] + (int64_t)h * p.os[2] + (int64_t)t0 * p.os[1]) * oesz,
                        p.os[1] * oesz, To, C, N, dir, oesz * D};
    int ooff[TPO];
#pragma unroll
    for (int tt = 0; tt < TPO; ++tt) ooff[tt] = orow.row(16 * out_tile<NB>(O, tt) + r) + oesz * (row0 + 4 * g);   // token, state rows row0 + 4g ..
    // bf16: the tiles go out through LDS, lane quad l/4 storing token l/4's 64-byte slice
    // (chunks past d_v are stored outside the resource, i.e. dropped)
    const int st = lane >> 2, sj = (lane & 3) ^ oswz(lane >> 2);
    int soff[TPO];
#pragma unroll
    for (int tt = 0; tt < TPO; ++tt)
        soff[tt] = (row0 + 16 * (sj >> 1) < p.Dv) ? orow.row(16 * out_tile<NB>(O, tt) + st) + 2 * row0 + 16 * sj : (int)0x80000000;
    bool col_ok[GDN_COLS];
#pragma unroll
    for (int c = 0; c < GDN_COLS; ++c) col_ok[c] = row0 + 16 * c < p.Dv;
    // Q operand reads: row 16 tile + r, state indices 32 ks + 8 g .. (a trailing 16-wide step:
    // 16 (ND-1) + 4 g .., 8 bytes)
    int qoff[TPO][NKD];
#pragma unroll
    for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
            qoff[tt][ks] = ks < NKF ? G::kq(16 * out_tile<NB>(O, tt) + r, 32 * ks + 8 * g)
                                    : G::kq(16 * out_tile<NB>(O, tt) + r, 32 * NKF + 4 * g);

    OutIn oA, oB;
    const auto irs = make_rsrc(item0, (uint32_t)(N * ib));
    auto load_out = [&](OutIn& o, int n) {
        const int ioff = n * (int)ib;
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int kt = 0; kt < BK::count(out_tile<NB>(O, tt)); ++kt)
                o.afr[aoff(tt) + kt] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(irs, 16 * lane, ioff + 1024 * (NF + BK::offset(out_tile<NB>(O, tt)) + kt), 0));
        // c2 of tokens 16 mt + r of this wavefront's tiles mt (lane-major scalars)
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
            o.c2[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (NB * r + out_tile<NB>(O, tt)),
                                                                                      ioff + G::ITEM_SC + 8 * C, 0));
    };

    load_out(oA, 0);
    load_out(oB, N > 1 ? 1 : 0);
    auto out_step = [&](OutIn& o, int n) {
        const int sl = n % GDN_RING;
        const ScanSlot<NB, ND>& op = L.ops[n % GDN_OPS];
#pragma unroll
        for (int c = 0; c < GDN_COLS; ++c) wait_counter<true>(&K.ready[c], n + 1, p.spin_limit, p.err);
        bf16x8 Pb[NKD][GDN_COLS];
        f16x8 Ub[NKT][GDN_COLS];
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Pb[ks][c] = __builtin_bit_cast(bf16x8, L.ringS[sl][ks][c][lane]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Ub[kt][c] = __builtin_bit_cast(f16x8, L.ringU[sl][kt][c][lane]);
        // the ring slot is free once its fragments are in registers
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) keep_alive(Pb[ks][c]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) keep_alive(Ub[kt][c]);
        signal_counter(&K.rdone[O], n + 1);
        // the step's Q rows
        wait_counter<true>(&K.loaded[1], n + 1, p.spin_limit, p.err);
        bf16x8 Qf[TPO][NKD];
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) {
                const char* qp = reinterpret_cast<const char*>(&op.q[0][0]) + qoff[tt][ks];
                if (ks < NKF) {
                    Qf[tt][ks] = ld_bf16x8(reinterpret_cast<const bf16*>(qp));
                } else {
                    const bf16x4 h4 = ld_bf16x4(reinterpret_cast<const bf16*>(qp));
                    const bf16 z = (bf16)0.f;
                    Qf[tt][ks] = bf16x8{h4[0], h4[1], h4[2], h4[3], z, z, z, z};
                }
            }
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) keep_alive(Qf[tt][ks]);
        signal_counter(&K.odone[O], n + 1);
        __builtin_amdgcn_sched_barrier(0);
        // Y^T = S Q^T: rows = state rows 16 c + 4 g + i, column = token 16 mt + r
        f32x4 Ot[TPO][GDN_COLS];
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Ot[tt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
                for (int c = 0; c < GDN_COLS; ++c) Ot[tt][c] = mma_bf16_k32(Pb[ks][c], Qf[tt][ks], Ot[tt][c]);
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Ot[tt][c] = Ot[tt][c] * o.c2[tt];
        // + U^T A^T (a trailing 16-token step has zero upper slots in both operands)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int tt = 0; tt < TPO; ++tt) {
                if (kt >= BK::count(out_tile<NB>(O, tt))) continue;
                const f16x8 af = __builtin_bit_cast(f16x8, o.afr[aoff(tt) + kt]);
#pragma unroll
                for (int c = 0; c < GDN_COLS; ++c) Ot[tt][c] = mma_f16_k32(Ub[kt][c], af, Ot[tt][c]);
            }
        uint2 ov[TPO][GDN_COLS];
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) {
                const bf16x4 b4 = {(bf16)Ot[tt][c][0], (bf16)Ot[tt][c][1], (bf16)Ot[tt][c][2], (bf16)Ot[tt][c][3]};
                ov[tt][c] = __builtin_bit_cast(uint2, b4);
            }
        // O is consumed: the operands of step n + 2 may now be loaded into o
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) keep_alive(ov[tt][c]);
        __builtin_amdgcn_sched_barrier(0);
        load_out(o, n + 2 < N ? n + 2 : N - 1);
        const auto ors = orow.rsrc(n);
        if (oesz == 2) {
            // token r's rows 16 c + 4 g .. +3 (8 bytes) to chunk 2 c + g/2, half g%2
#pragma unroll
            for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
                for (int c = 0; c < GDN_COLS; ++c) {
                    char* sp = reinterpret_cast<char*>(&L.ostage[O][tt][0]) + 64 * r + 16 * ((2 * c + (g >> 1)) ^ oswz(r)) + 8 * (g & 1);
                    *reinterpret_cast<uint2*>(sp) = ov[tt][c];
                }
#pragma unroll
            for (int tt = 0; tt < TPO; ++tt) {
                const uint4 v = L.ostage[O][tt][lane];
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ors, soff[tt], 0, 0);
            }
        } else {
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c)
                if (col_ok[c]) {
#pragma unroll
                    for (int tt = 0; tt < TPO; ++tt)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Ot[tt][c]), ors, ooff[tt] + 64 * c, 0, 0);
                }
        }
    };
    // The prefetches are unconditional (the last steps reload step N-1) so that
    // every path through the loop has the same loads in flight.
    int n = 0;
    for (; n + 1 < N; n += 2) {
        out_step(oA, n);
        out_step(oB, n + 1);
    }
    if (n < N) out_step(oA, n);
}

template <int NB, int ND>
__global__ __launch_bounds__((ScanGeom<NB, ND>::THREADS)) void gdn_scan_kernel(Params p, int ngroups) {
    using G = ScanGeom<NB, ND>;
    constexpr int C = G::C, D = G::D;
    constexpr int NKD = G::NKD, NKF = G::NKF, NKT = G::NKT, NF = G::NF;
    constexpr int NS = (ND + GDN_COLS - 1) / GDN_COLS;   // slices per head
    constexpr int NOUT = G::NOUT;
    using BK = Blocks<NB>;
    typedef short s16x4 __attribute__((ext_vector_type(4)));

    __shared__ __align__(16) ScanLds<NB, ND> L;
    __shared__ ScanCtr K;

    const int lane = threadIdx.x & 63;
    // the role of a wavefront is wave-uniform: keep it in a scalar register so every
    // role is a whole-wavefront branch
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    // Workgroup id % 8 is the XCD it runs on.  Both directions and all NS slices of stream-head
    // bh run on its XCD (xcd_head, with the prep workgroups of that head), so that they share
    // its L2.
    // The workgroups of a stream-head: its directions, or the segments (and, for the first stage
    // of a time split, their two variants) of its forward scan.
    // A time split spreads its workgroups over all XCDs instead (its point is to use the whole
    // chip when the stream-heads are few).
    const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
    const int nv = p.seg_mode == 1 ? 2 * p.nseg : p.seg_mode == 2 ? p.nseg : p.ndirs;
    const int j = (p.seg_mode ? id : slot) % NS, rest = (p.seg_mode ? id : slot) / NS;
    const int bh = p.seg_mode ? (rest / nv < ngroups ? rest / nv : -1) : xcd_head(xcd, rest / nv, ngroups);
    if (bh < 0) return;
    const int vi = rest % nv;
    const int dir = p.seg_mode ? 0 : p.dir0 + vi;
    const int sigma = p.seg_mode == 1 ? (vi >> 1) : p.seg_mode == 2 ? vi : 0;
    const int variant = p.seg_mode == 1 ? (vi & 1) : 0;   // 0: from a zero state, 1: from the identity with v = 0
    const int h = bh % p.H, b = bh / p.H;
    // a segment is scanned as a sequence of its own: from its first step n0 (token t0), with the
    // tokens from there on and its own number of steps
    const int n0 = sigma * p.seg_steps, t0 = n0 * C;
    const int T = (int)p.T - t0;
    const int N = p.seg_mode ? min(p.seg_steps, ((int)p.T + C - 1) / C - n0) : (T + C - 1) / C;
    const int row0 = 16 * GDN_COLS * j;
    const int64_t ib = p.ws_item_bytes;
    const char* item0 = p.ws + (((int64_t)dir * p.B + b) * p.H + h) * p.nsub_max * ib + (int64_t)n0 * ib;

    if (threadIdx.x == 0) {
#pragma unroll
        for (int c = 0; c < GDN_COLS; ++c) K.ready[c] = K.cdone[c] = 0;
        K.rdone[0] = K.rdone[1] = K.odone[0] = K.odone[1] = 0;
        K.loaded[0] = K.loaded[1] = 0;
        // a single output wavefront (C = 16) leaves the second pair of counts open
        if (NOUT == 1) K.rdone[1] = K.odone[1] = 1 << 30;
    }
    __syncthreads();

    if (wave >= GDN_COLS + NOUT) {
        // ------------------------------ loader wavefronts ------------------------------
        // Step m goes to operand slot m % GDN_OPS once every wavefront that reads that part of
        // the slot is done with step m - GDN_OPS.  The loads go into registers and from there to
        // LDS with 16-byte stores: the LDS takes them at its full store rate, while loads that write
        // LDS directly held its other traffic back (the scan ran 2 us longer with them).  Two steps
        // are in flight in two register sets: the loads of step m + 1 are issued before those of
        // step m are waited for (the loads of a wavefront complete in order).
        const int part = wave - (GDN_COLS + NOUT);
        const StepRows krow{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.k) + (int64_t)b * p.ks[0] +
                                                          (int64_t)h * p.ks[2] + (int64_t)t0 * p.ks[1]),
                            p.ks[1] * 2, T, C, N, dir, 2 * D};
        const StepRows qrow{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.q) + (int64_t)b * p.qs[0] +
                                                          (int64_t)h * p.qs[2] + (int64_t)t0 * p.qs[1]),
                            p.qs[1] * 2, T, C, N, dir, 2 * D};
        // the identity variant of a split reads v as zero (a resource of no rows)
        const StepRows vrow{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.v) + (int64_t)b * p.vs[0] +
                                                          (int64_t)h * p.vs[2] + (int64_t)t0 * p.vs[1]),
                            p.vs[1] * 2, variant ? 0 : T, C, N, dir, 2 * D};
        const StepRows& rows = part == 0 ? krow : qrow;
        // destination chunk 64 i + lane of a block of rows: row t, position pos; the source chunk
        // is pos ^ sw(t, pos) (the permutation is an involution within its group of chunks)
        int roff[G::NLK];
#pragma unroll
        for (int i = 0; i < G::NLK; ++i) {
            const int pc = 64 * i + lane;
            const int t = pc < C * G::CH ? pc / G::CH : 0, pos = pc < C * G::CH ? pc - t * G::CH : 0;
            roff[i] = rows.row(t) + 16 * (pos ^ G::sw(t, pos));
        }
        // V slice: token t = p / 4 of the step, chunk position p % 4 holds source chunk
        // (p % 4) ^ vswz(t); chunks of column tiles past d_v are read from outside the resource
        int voff[G::NLV];
#pragma unroll
        for (int i = 0; i < G::NLV; ++i) {
            const int pc = 64 * i + lane, t = pc >> 2, jj = (pc & 3) ^ vswz(t);
            voff[i] = (row0 + 16 * (jj >> 1) < p.Dv) ? vrow.row(t) + 2 * row0 + 16 * jj : (int)0x80000000;
        }
        const auto irs = make_rsrc(item0, (uint32_t)(N * ib));
        auto slot_free = [&](int m) {   // readers done with step m - GDN_OPS
            const int need = m + 1 - GDN_OPS;
            if (need <= 0) return;
            if (part == 0) {
#pragma unroll
                for (int c = 0; c < GDN_COLS; ++c) wait_counter<true>(&K.cdone[c], need, p.spin_limit, p.err);
            } else {
                wait_counter<true>(&K.odone[0], need, p.spin_limit, p.err);
                wait_counter<true>(&K.odone[1], need, p.spin_limit, p.err);
            }
        };
        // one code path per loader, so that its register sets have a compile-time size
        auto run = [&](auto PART) __attribute__((always_inline)) {
            constexpr int P = decltype(PART)::value;
            constexpr int NL = P == 0 ? G::NLD0 : G::NLD1;
            auto issue = [&](int m, u32x4 (&R)[NL]) __attribute__((always_inline)) {
                if constexpr (P == 0) {
                    const auto krs = krow.rsrc(m);
#pragma unroll
                    for (int i = 0; i < G::NLK; ++i) R[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, roff[i], 0, 0));
                    const auto vrs = vrow.rsrc(m);
#pragma unroll
                    for (int i = 0; i < G::NLV; ++i) R[G::NLK + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i], 0, 0));
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        R[G::NLK + G::NLV + f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(irs, 1024 * f + 16 * lane, m * (int)ib, 0));
                    R[G::NLK + G::NLV + NF] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(irs, G::ITEM_SC + 16 * lane, m * (int)ib, 0));
                } else {
                    const auto qrs = qrow.rsrc(m);
#pragma unroll
                    for (int i = 0; i < G::NLK; ++i) R[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, roff[i], 0, 0));
                }
            };
            auto step = [&](int m, u32x4 (&R)[NL]) __attribute__((always_inline)) {
                if (m + 1 < N) wait_vmcnt<NL>();
                else wait_vmcnt<0>();
                slot_free(m);
                ScanSlot<NB, ND>& op = L.ops[m % GDN_OPS];
                if constexpr (P == 0) {
#pragma unroll
                    for (int i = 0; i < G::NLK; ++i) *reinterpret_cast<u32x4*>(&op.k[i][lane]) = R[i];
#pragma unroll
                    for (int i = 0; i < G::NLV; ++i) *reinterpret_cast<u32x4*>(&op.v[i][lane]) = R[G::NLK + i];
#pragma unroll
                    for (int f = 0; f < NF; ++f) *reinterpret_cast<u32x4*>(&op.tt[f][lane]) = R[G::NLK + G::NLV + f];
                    *reinterpret_cast<u32x4*>(&op.sc[lane]) = R[G::NLK + G::NLV + NF];
                } else {
#pragma unroll
                    for (int i = 0; i < G::NLK; ++i) *reinterpret_cast<u32x4*>(&op.q[i][lane]) = R[i];
                }
                signal_counter(&K.loaded[P], m + 1);
                if (m + 2 < N) issue(m + 2, R);
            };
            u32x4 ra[NL], rb[NL];
            issue(0, ra);
            if (N > 1) issue(1, rb);
            int m = 0;
            for (; m + 1 < N; m += 2) {
                step(m, ra);
                step(m + 1, rb);
            }
            if (m < N) step(m, ra);
            wait_vmcnt<0>();
        };
        if (part == 0) run(IConst<0>{});
        else run(IConst<1>{});
        return;
    }
    if (wave == GDN_COLS) {
        scan_output<NB, ND, 0>(p, L, K, lane, b, h, dir, T, N, row0, item0, ib, t0, p.seg_mode == 1 ? 0 : T);
        return;
    }
    if constexpr (NOUT > 1) {
        if (wave == GDN_COLS + 1) {
            scan_output<NB, ND, 1>(p, L, K, lane, b, h, dir, T, N, row0, item0, ib, t0, p.seg_mode == 1 ? 0 : T);
            return;
        }
    }

    // ------------------------------ chain wavefronts ------------------------------
    // Chain wavefront cc owns state rows row0 + 16 cc .. +15.  Per step n: wait for the
    // step's operands and a free output-ring slot; Pb = bf16(S) to the ring; X = K S^T on MFMA;
    // R = V - c1 X; U = T~ R (fp16 MFMA) to the ring; S^T <- gamma_C S^T + K^T (w U).
    const int cc = wave;
    const bool tile_ok = row0 + 16 * cc < p.Dv;
    f32x4 P[ND];   // P[m][i] = S[row0 + 16 cc + r][dperm(m, 4 g + i)]
    // start state: the forward scan's S_in, zero for the reverse scan; for a time split, zero or the
    // identity (first stage) or the segment's start state (last stage)
    const int64_t selems = (int64_t)p.B * p.H * D * D;
    const float* Sin = p.seg_mode == 1 ? nullptr
                       : p.seg_mode == 2 ? p.seg_in + sigma * selems
                       : (dir == 0) ? p.S_in : nullptr;
    const int64_t hbase = ((int64_t)b * p.H + h) * D * D;
    const int64_t srow = hbase + (int64_t)(row0 + 16 * cc + r) * D;
#pragma unroll
    for (int m = 0; m < ND; ++m) {
        if (variant) {
            const int srw = row0 + 16 * cc + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) P[m][i] = (tile_ok && srw == dperm<ND>(m, 4 * g + i)) ? 1.f : 0.f;
        } else if (Sin && tile_ok)
            P[m] = *reinterpret_cast<const f32x4*>(Sin + srow + dperm<ND>(m, 4 * g));
        else
            P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // operand read offsets within a slot (bytes):
    //   K rows for X: row 16 mt + r, state indices 32 ks + 8 g .. (trailing half step: 16 (ND-1) + 4 g ..)
    //   K^T for the update (transposing 8-byte reads): lane r of group g supplies row
    //     32 kt + 16 hh + 4 g + r/4 at state indices dperm(m, 4 (r%4)) .. +3, and receives
    //     column dperm(m, r) at rows 32 kt + 16 hh + 4 g .. +3
    int kxo[NB][NKD];
#pragma unroll
    for (int mt = 0; mt < NB; ++mt)
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
            kxo[mt][ks] = ks < NKF ? G::kq(16 * mt + r, 32 * ks + 8 * g) : G::kq(16 * mt + r, 32 * NKF + 4 * g);
    auto kto = [&](int m, int trow) { return G::kq(trow + 4 * g + (r >> 2), dperm<ND>(m, 4 * (r & 3))); };
    // V read back transposed: lane quad q of group g supplies token 16 mt + 4 g + i (i = r/4), columns
    // 16 cc + 4 q .. +3 of the slice; lane (r, g) receives state row 16 cc + r at tokens 16 mt + 4 g ..
    auto vto = [&](int mt) {
        const int q = r & 3, t = 16 * mt + 4 * g + (r >> 2);
        return 64 * t + 16 * ((2 * cc + (q >> 1)) ^ vswz(t)) + 8 * (q & 1);
    };

    int rdone_seen[2] = {0, 0};
    // K rows of a step as X operands; the trailing half k-step's rows are kept as read (kh) and widened
    // with zero slots just before their use, so that no wait for them sits ahead of the update
    constexpr bool HALFK = NKF < NKD;
    constexpr int NKH = HALFK ? NB : 1;
    auto read_kf = [&](const char* kb, bf16x8 (&kf)[NB][NKD], bf16x4 (&kh)[NKH]) {
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) {
                const bf16* kp = reinterpret_cast<const bf16*>(kb + kxo[mt][ks]);
                if (ks < NKF) kf[mt][ks] = ld_bf16x8(kp);
                else kh[mt] = ld_bf16x4(kp);
            }
    };
    bf16x8 kf[NB][NKD];
    bf16x4 kh[NKH];
    wait_counter<false>(&K.loaded[0], 1, p.spin_limit, p.err);
    read_kf(reinterpret_cast<const char*>(&L.ops[0].k[0][0]), kf, kh);
    bf16x8 kT[ND][NKT];
    bf16x8 Ub[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) Ub[kt] = bf16x8{};
#pragma unroll
    for (int m = 0; m < ND; ++m)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) kT[m][kt] = bf16x8{};
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
        const int sl = n % GDN_RING;
        const ScanSlot<NB, ND>& op = L.ops[n % GDN_OPS];
        const char* kb = reinterpret_cast<const char*>(&op.k[0][0]);
        // the output ring slot of this step must have been released by every output wavefront
        // (the counts were read in the previous step; a poll here only when they were short)
#pragma unroll
        for (int o = 0; o < 2; ++o)
            if (rdone_seen[o] < n + 1 - GDN_RING) {
                wait_counter<false>(&K.rdone[o], n + 1 - GDN_RING, p.spin_limit, p.err);
                rdone_seen[o] = n + 1 - GDN_RING;
            }
        // The step's other operands do not depend on the state: they are read now, so that they have
        // arrived by the time X does.  c1 and w of tokens 16 mt + 4 g .. +3, gamma_C, V (transposed)
        // and the T~ fragments.
        const float* scf = reinterpret_cast<const float*>(&op.sc[0]);
        f32x4 c1v[NB], wv[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            c1v[mt] = *reinterpret_cast<const f32x4*>(scf + 16 * mt + 4 * g);
            wv[mt] = *reinterpret_cast<const f32x4*>(scf + C + 16 * mt + 4 * g);
        }
        const float gC = scf[3 * C];
        bf16x4 vt[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            vt[mt] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<const char*>(&op.v[0][0]) + vto(mt))));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (HALFK) {
            const bf16 z = (bf16)0.f;
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) kf[mt][NKD - 1] = bf16x8{kh[mt][0], kh[mt][1], kh[mt][2], kh[mt][3], z, z, z, z};
        }
        // state as bf16 operand: k-slot e of lane group g <-> d = dperm(2 ks + e/4, 4 g + e%4)
        bf16x8 Pb[NKD];
#pragma unroll
        for (int ks = 0; ks < NKF; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Pb[ks][i] = (bf16)P[2 * ks][i];
                Pb[ks][4 + i] = (bf16)P[2 * ks + 1][i];
            }
        if constexpr (ND % 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Pb[NKD - 1][i] = (bf16)P[ND - 1][i];
                Pb[NKD - 1][4 + i] = (bf16)0.f;
            }
        }
        // Pb holds the previous update's results: that update's operands may be released now
#pragma unroll
        for (int m = 0; m < ND; ++m)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) keep_alive(kT[m][kt]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) keep_alive(Ub[kt]);
        // publish the state to the output ring right away
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) L.ringS[sl][ks][cc][lane] = __builtin_bit_cast(uint4, Pb[ks]);
        // X = K S^T (rows: tokens 16 mt + 4 g + i, column: state row 16 cc + r); the decay of the state
        // for the update is applied in the shadow of these products
        f32x4 X[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) X[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) X[mt] = mma_bf16_k32(kf[mt][ks], Pb[ks], X[mt]);
#pragma unroll
        for (int m = 0; m < ND; ++m) P[m] = P[m] * gC;
        __builtin_amdgcn_sched_barrier(0);
        // the counters this wavefront checks next, read ahead of its further LDS reads (LDS reads
        // complete in order: a count read after them would wait for all of them)
        const int ld_early = __hip_atomic_load(&K.loaded[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        int rd_early[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) rd_early[o] = __hip_atomic_load(&K.rdone[o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        f16x8 tf[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) tf[f] = __builtin_bit_cast(f16x8, op.tt[f][lane]);
        __builtin_amdgcn_sched_barrier(0);
        // R = V - diag(c1) X, as fp16 B operand (k = token, slot order of the output tiles)
        f16x8 Rb[NKT];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) Rb[mt >> 1][4 * (mt & 1) + i] = (f16)((float)vt[mt][i] - c1v[mt][i] * X[mt][i]);
        if constexpr (BK::HALF) {
#pragma unroll
            for (int i = 4; i < 8; ++i) Rb[NKT - 1][i] = (f16)0.f;
        }
        // X is consumed: its K operands may be released
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks) keep_alive(kf[mt][ks]);
        // the next step's K rows, read while U and the update run
        if (n + 1 < N) {
            if (ld_early < n + 2) wait_counter<false>(&K.loaded[0], n + 2, p.spin_limit, p.err);
            read_kf(reinterpret_cast<const char*>(&L.ops[(n + 1) % GDN_OPS].k[0][0]), kf, kh);
        }
        // K^T fragments for the update (state index rows, token k-slots)
#pragma unroll
        for (int m = 0; m < ND; ++m)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                s16x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
                if (32 * kt < C)
                    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(kb + kto(m, 32 * kt)));
                if (32 * kt + 16 < C)
                    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(kb + kto(m, 32 * kt + 16)));
                const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
                kT[m][kt] = bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
            }
        // U = T~ R (rows: tokens 16 mt + 4 g + i, column: state row 16 cc + r)
        f32x4 U[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            U[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < BK::count(mt); ++kt) U[mt] = mma_f16_k32(tf[BK::offset(mt) + kt], Rb[kt], U[mt]);
        }
        // U to the output ring (fp16, A operand of U^T A^T) and w U as bf16 B operand of the update
        f16x8 Uh[NKT];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Uh[mt >> 1][4 * (mt & 1) + i] = (f16)U[mt][i];
                Ub[mt >> 1][4 * (mt & 1) + i] = (bf16)(wv[mt][i] * U[mt][i]);
            }
        if constexpr (BK::HALF) {
#pragma unroll
            for (int i = 4; i < 8; ++i) {
                Uh[NKT - 1][i] = (f16)0.f;
                Ub[NKT - 1][i] = (bf16)0.f;
            }
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) keep_alive(tf[f]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) keep_alive(Rb[kt]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) L.ringU[sl][kt][cc][lane] = __builtin_bit_cast(uint4, Uh[kt]);
        signal_counter(&K.ready[cc], n + 1);
#pragma unroll
        for (int o = 0; o < 2; ++o) rdone_seen[o] = rd_early[o] > rdone_seen[o] ? rd_early[o] : rdone_seen[o];
        // S^T <- gamma_C S^T + K^T (w U)  (rows d, columns: state rows); a trailing 16-token
        // step has zero upper slots in both operands
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int m = 0; m < ND; ++m) P[m] = mma_bf16_k32(kT[m][kt], Ub[kt], P[m]);
        __builtin_amdgcn_sched_barrier(0);
        // every read of the operand slot of step n has been issued (and, the LDS being in order,
        // takes effect before this count)
        signal_counter(&K.cdone[cc], n + 1);
    }
    float* Sout = p.seg_mode == 1 ? p.seg_out + (2 * sigma + variant) * selems
                  : p.seg_mode == 2 ? (sigma == p.nseg - 1 ? p.S_out[0] : nullptr)
                  : p.S_out[dir];
    if (Sout && tile_ok) {
#pragma unroll
        for (int m = 0; m < ND; ++m) *reinterpret_cast<f32x4*>(Sout + srow + dperm<ND>(m, 4 * g)) = P[m];
    }
}

// fp32 q, k, v (caller strides) -> bf16 copies in `dst` ([3][B][T][H][D], contiguous), rounded to
// nearest even: the chunked kernels take their MFMA operands in bf16.
__global__ void gdn_to_bf16_kernel(Params p, bf16* dst) {
    const int64_t D = p.Dk, rows = (int64_t)p.B * p.T * p.H, per = rows * D;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 3 * per; i += (int64_t)gridDim.x * blockDim.x) {
        const int w = (int)(i / per);
        const int64_t j = i - w * per, row = j / D, d = j - row * D;
        const int64_t hh = row % p.H, tt = (row / p.H) % p.T, bb = row / ((int64_t)p.H * p.T);
        const float* src = static_cast<const float*>(w == 0 ? p.q : w == 1 ? p.k : p.v);
        const int64_t* st = w == 0 ? p.qs : w == 1 ? p.ks : p.vs;
        dst[i] = (bf16)src[bb * st[0] + tt * st[1] + hh * st[2] + d];
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

// Second stage of a time split: per (stream-head, 16 state rows), serially over the segments,
// S_{s+1} = S_s P_s + D_s in fp32 (rows of S evolve independently), from S_0 = S_in (zero if
// null).  (D_s, P_s) = seg_out[2 s], seg_out[2 s + 1]; S_s goes to seg_in[s] (S_0 too, so that the
// last stage never reads S_in, which its last segment may overwrite).  P_s is staged in LDS (the
// next segment's P loaded into registers while this one is applied); thread t owns column t % 128
// of rows 8 (t / 128) .. +7; the k-sum runs in index order.
constexpr int SPLIT_PLD = (128 * 128 / 4 + 255) / 256;   // float4 loads of a P per thread (D <= 128)
__global__ __launch_bounds__(256) void gdn_split_combine_kernel(Params p, float* seg_in) {
    const int D = p.Dk, nrb = D / 16;
    const int rb = blockIdx.x % nrb, bh = blockIdx.x / nrb;
    const int64_t selems = (int64_t)p.B * p.H * D * D, hbase = (int64_t)bh * D * D;
    __shared__ float srows[16][128];
    __shared__ __align__(16) float ps[128 * 128];
    const int tid = threadIdx.x, col = tid & 127, rg = tid >> 7;
    const int nq = D * D / 4;   // float4 of a P
    for (int e = tid; e < 16 * D; e += 256) {
        const int i = e / D, c = e - i * D;
        const float v = p.S_in ? p.S_in[hbase + (int64_t)(16 * rb + i) * D + c] : 0.f;
        srows[i][c] = v;
        seg_in[hbase + (int64_t)(16 * rb + i) * D + c] = v;
    }
    float4 pr[SPLIT_PLD];
    auto load_p = [&](int sg) {
        const float4* src = reinterpret_cast<const float4*>(p.seg_out + (2 * sg + 1) * selems + hbase);
#pragma unroll
        for (int i = 0; i < SPLIT_PLD; ++i) {
            const int e = tid + 256 * i;
            pr[i] = e < nq ? src[e] : float4{0.f, 0.f, 0.f, 0.f};
        }
    };
    if (p.nseg > 1) load_p(0);
    for (int sg = 0; sg + 1 < p.nseg; ++sg) {
#pragma unroll
        for (int i = 0; i < SPLIT_PLD; ++i) {
            const int e = tid + 256 * i;
            if (e < nq) reinterpret_cast<float4*>(ps)[e] = pr[i];
        }
        __syncthreads();   // P_s and S_s in LDS
        if (sg + 2 < p.nseg) load_p(sg + 1);
        const float* Dm = p.seg_out + (2 * sg) * selems + hbase;
        float acc[8];
        if (col < D) {
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) acc[ii] = Dm[(int64_t)(16 * rb + 8 * rg + ii) * D + col];
            for (int k = 0; k < D; ++k) {
                const float pk = ps[k * D + col];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) acc[ii] = fmaf(srows[8 * rg + ii][k], pk, acc[ii]);
            }
        }
        __syncthreads();   // every read of S_s and P_s is done
        if (col < D) {
            float* out = seg_in + (sg + 1) * selems + hbase;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                srows[8 * rg + ii][col] = acc[ii];
                out[(int64_t)(16 * rb + 8 * rg + ii) * D + col] = acc[ii];
            }
        }
    }
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
static hipError_t run_prep(const Params& p, hipStream_t s, Timing* tm) {
    const int nsub = (int)((p.T + 16 * NB - 1) / (16 * NB));
    tm_begin(tm, s, KPREP);
    const int ngrp = nsub;
    const int grid = p.seg_mode ? p.B * p.H * ngrp : 8 * ((p.B * p.H + 7) / 8) * ngrp;
    hipLaunchKernelGGL((gdn_prep_kernel<NB, ND>), dim3(grid), dim3(128 * NB), 0, s, p);
    tm_end(tm, s);
    return hipGetLastError();
}

template <int NB, int ND>
static hipError_t run_scan(const Params& p, hipStream_t s, Timing* tm) {
    const int ngroups = p.B * p.H;   // stream-heads; each has scan_variants(p) workgroups per row slice
    const int ns = (ND + GDN_COLS - 1) / GDN_COLS;
    const int grid = p.seg_mode ? ngroups * scan_variants(p) * ns : (ngroups + 7) / 8 * 8 * scan_variants(p) * ns;
    tm_begin(tm, s, KSCAN);
    hipLaunchKernelGGL((gdn_scan_kernel<NB, ND>), dim3(grid), dim3(ScanGeom<NB, ND>::THREADS), 0, s, p, ngroups);
    tm_end(tm, s);
    return hipGetLastError();
}

template <int NB, int ND>
static hipError_t run_chunked(const Params& p, hipStream_t s, Timing* tm) {
    hipError_t e = run_prep<NB, ND>(p, s, tm);
    if (e != hipSuccess) return e;
    return run_scan<NB, ND>(p, s, tm);
}

// The forward scan in p.nseg segments (p.seg_steps steps each): every segment from a zero state and
// from the identity (v = 0) at once, the segments' start states by the serial combine, then every
// segment again from its start state, writing o.  seg_in: [nseg][B][H][D][D] (entry 0 unused),
// p.seg_out: [2 nseg][B][H][D][D].
template <int NB, int ND>
static hipError_t run_split(const Params& p, float* seg_in, hipStream_t s, Timing* tm) {
    Params pa = p;
    pa.seg_mode = 1;
    hipError_t e = run_prep<NB, ND>(pa, s, tm);
    if (e != hipSuccess) return e;
    e = run_scan<NB, ND>(pa, s, tm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gdn_split_combine_kernel, dim3((unsigned)(p.B * p.H * (p.Dk / 16))), dim3(256), 0, s, p, seg_in);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    Params pc = p;
    pc.seg_mode = 2;
    pc.seg_in = seg_in;
    return run_scan<NB, ND>(pc, s, tm);
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
    (void)io_f32;   // fp32 q, k, v are staged as bf16 (gdn_to_bf16_kernel), o is stored in fp32
    if (Dk != Dv) return false;
    if (!(Dk == 16 || Dk == 32 || Dk == 64 || Dk == 112 || Dk == 128)) return false;
    return C == 16 || C == 32 || C == 64;
}

// Device address of the static workspace on `device` (current), looked up on the first call for
// that device.  Host code never passes the array's own name to a kernel: on the host that name
// stands for a host-side shadow, not for device memory.
hipError_t scratch_address(int device, char** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static char* addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[device] = static_cast<char*>(ptr);
    }
    *out = addr[device];
    return hipSuccess;
}

template <int NB>
static hipError_t run_split_d(const Params& p, float* seg_in, hipStream_t s, Timing* tm) {
    switch (p.Dk) {
        case 16: return run_split<NB, 1>(p, seg_in, s, tm);
        case 32: return run_split<NB, 2>(p, seg_in, s, tm);
        case 64: return run_split<NB, 4>(p, seg_in, s, tm);
        case 112: return run_split<NB, 7>(p, seg_in, s, tm);
        case 128: return run_split<NB, 8>(p, seg_in, s, tm);
        default: return hipErrorInvalidValue;
    }
}

// bf16 staging copies of fp32 q, k, v; p then points at them
static hipError_t stage_f32(Params& p, const Params& p0, hipStream_t s) {
    if (!p.conv) return hipErrorInvalidValue;
    const int64_t per = (int64_t)p.B * p.T * p.H * p.Dk;
    int64_t blocks = (3 * per + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gdn_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p0, p.conv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.q = p.conv;
    p.k = p.conv + per;
    p.v = p.conv + 2 * per;
    const int64_t st[3] = {p.T * p.H * p.Dk, (int64_t)p.H * p.Dk, p.Dk};
    for (int i = 0; i < 3; ++i) p.qs[i] = p.ks[i] = p.vs[i] = st[i];
    return hipSuccess;
}

hipError_t launch_split(const Params& p0, float* seg_in, hipStream_t s, Timing* tm) {
    Params p = p0;
    if (p.io_f32) {
        const hipError_t e = stage_f32(p, p0, s);
        if (e != hipSuccess) return e;
    }
    switch (p.C) {
        case 16: return run_split_d<1>(p, seg_in, s, tm);
        case 32: return run_split_d<2>(p, seg_in, s, tm);
        case 64: return run_split_d<4>(p, seg_in, s, tm);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunked(const Params& p0, hipStream_t s, Timing* tm) {
    Params p = p0;
    if (p.io_f32) {
        const hipError_t e = stage_f32(p, p0, s);
        if (e != hipSuccess) return e;
    }
    switch (p.C) {
        case 16: return run_chunked_d<1>(p, s, tm);
        case 32: return run_chunked_d<2>(p, s, tm);
        case 64: return run_chunked_d<4>(p, s, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
