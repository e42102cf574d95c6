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

#include <utility>

#include "gdn_internal.h"

namespace gdn {

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

// workspace item of one processing step: [E fragments: TOTAL blocks][Z^T fragments:
// ND x NKT blocks][scalars: c1, c2 (C floats each), gamma_C], 1 KB per fragment
// block (64 lanes x 16 bytes)
template <int NB, int ND>
__host__ __device__ constexpr int64_t item_bytes_t() {
    constexpr int NKT = Blocks<NB>::NFULL + (Blocks<NB>::HALF ? 1 : 0);
    int64_t b = 1024 * (int64_t)(Blocks<NB>::TOTAL + ND * NKT) + 4 * (2 * 16 * NB + 4);
    return (b + 255) / 256 * 256;
}

template <int NB>
static int64_t item_bytes_d(int D) {
    switch (D) {
        case 16: return item_bytes_t<NB, 1>();
        case 32: return item_bytes_t<NB, 2>();
        case 64: return item_bytes_t<NB, 4>();
        case 112: return item_bytes_t<NB, 7>();
        case 128: return item_bytes_t<NB, 8>();
        default: return -1;
    }
}

int64_t chunk_item_bytes(int C, int D) {
    switch (C) {
        case 16: return item_bytes_d<1>(D);
        case 32: return item_bytes_d<2>(D);
        case 64: return item_bytes_d<4>(D);
        default: return -1;
    }
}

int64_t chunk_frag_bytes(int D, int64_t max_tokens, int B, int H) {
    const int64_t nkd = (D / 16 + 1) / 2;
    return 2 * (int64_t)B * H * ((max_tokens + 15) / 16) * nkd * 1024;
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

// K and Q operand fragments by 16-token tile (token order).  Block (tile, ks) holds, for
// lane r + 16 g, row 16 tile + r at d = 32 ks + 8 g .. +7 (16 bytes); a trailing single
// tile of d (odd D/16) holds d = 16 (ND-1) + 4 g .. +3 and 8 zero bytes.  Processing tile mt
// of step n is token tile frag_tile(); the reverse direction takes the tile's rows in
// reverse order (processing row r is the tile's row 15 - r).
__device__ __forceinline__ int frag_tile(int dir, int N, int NB, int n, int mt) {
    return dir ? N * NB - 1 - NB * n - mt : NB * n + mt;
}
// fragments of (kind 0 = K / 1 = Q, b, h): base and bytes of the tiles that hold tokens
__device__ __forceinline__ const char* frag_base(const Params& p, int kind, int b, int h, int nkd) {
    return p.frag + (((int64_t)kind * p.B + b) * p.H + h) * p.ntile_max * nkd * 1024;
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
//   E = A T diag(beta)                  (output:  O = diag(c2) Q S^T + E R)
//   Z = diag(beta) T^T diag(e^{g_C-g}/|k|) K  (state: S^T <- gamma_C S^T + Z^T R)
// with R = V - diag(c1) K S^T, c1 = gamma/|k|, c2 = scale gamma/|q|.  (The gate
// beta is folded into E and Z, so the serial scan needs one scale per token.)
// L, A and T are held in fp16 (T is built in fp32 arithmetic from fp16 blocks);
// E and Z^T are stored as fp16 MFMA fragments for the scan, the state dimension
// d of Z^T in the scan's state order (see dperm).
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
    constexpr int NKT = BK::NFULL + (BK::HALF ? 1 : 0);
    typedef short s16x4 __attribute__((ext_vector_type(4)));

    // K and Q rows (bf16, D per row, token order).  Row t holds its 16-byte chunk c at position
    // c ^ sw(t, c): the chunks of the 32-wide k-steps are permuted within their group of four by
    // (t >> 2) & 3, the two chunks of a trailing 16-wide step swap for rows with bit 3 set.  With
    // this layout the MFMA operand reads (16 consecutive rows at one column, 16- and 8-byte) are
    // free of LDS bank conflicts on gfx950 (measured; a swap by bit 3 alone leaves the 16-byte
    // reads two-way conflicted).  The Q rows are dead after the Gram products; T^T of both
    // directions then takes their storage.
    constexpr int CHF = 4 * (ND / 2);   // chunks of the 32-wide k-steps
    auto kq_full = [](int t, int d) { return t * D + (((d >> 3) ^ ((t >> 2) & 3)) << 3) + (d & 7); };   // d < 8 CHF
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
    __shared__ __align__(16) f16 w16[2][C];           // e^{g_C-g}/|k| by processing row
    __shared__ int jobctr;                            // next E/Z job
    bf16* Qs = reinterpret_cast<bf16*>(QT);

    // the wavefront index is uniform: in a scalar register, so that everything derived from
    // it (tile and job assignment, addresses) is scalar work
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int j = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.H, h = bh - b * p.H;
    const int T = (int)p.T;
    const int N = (T + C - 1) / C;
    const int dlo = p.dir0, dhi = p.dir0 + p.ndirs - 1;
    auto active = [&](int dir) { return dir >= dlo && dir <= dhi; };
    // token row (within the block) of processing row t
    auto mrow = [](int dir, int t) { return dir ? C - 1 - t : t; };
    auto item_addr = [&](int dir) {
        const int n = dir ? N - 1 - j : j;
        return p.ws + ((((int64_t)dir * p.B + b) * p.H + h) * p.nsub_max + n) * p.ws_item_bytes;
    };
    char* const items[2] = {item_addr(0), item_addr(1)};   // this block's item in either direction
    auto item_of = [&](int dir) { return items[dir]; };

    {
        // every global load of the block goes out before the first is used: the gates,
        // then the K and Q rows (16-byte chunks, NLD per thread)
        float av = 1.f, bt = 0.f;
        bool gv = false;
        if (tid < C) {
            const int tk = j * C + tid;
            gv = tk < T;
            if (gv) {
                const int64_t gq = (int64_t)b * p.gs[0] + (int64_t)tk * p.gs[1] + (int64_t)h * p.gs[2];
                av = p.a[gq];
                bt = p.beta[gq];
            }
        }
        const bf16* kb = reinterpret_cast<const bf16*>(p.k) + (int64_t)b * p.ks[0] + (int64_t)h * p.ks[2];
        const bf16* qb = reinterpret_cast<const bf16*>(p.q) + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[2];
        const auto kr = make_rsrc(kb, (uint32_t)(((int64_t)(T - 1) * p.ks[1] + D) * 2));
        const auto qr = make_rsrc(qb, (uint32_t)(((int64_t)(T - 1) * p.qs[1] + D) * 2));
        const int ksb = (int)p.ks[1] * 2, qsb = (int)p.qs[1] * 2;
        constexpr int NLD = (C * CH + NT - 1) / NT;
        uint4 kv[NLD], qv[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int idx = tid + i * NT;
            if (idx < C * CH) {
                const int t = idx / CH, c = idx - t * CH;
                const int tk = j * C + t;
                kv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, tk * ksb + 16 * c, 0, 0));
                qv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, tk * qsb + 16 * c, 0, 0));
            }
        }
        if (tid < C) {
            sg[0][tid] = gv ? fmaxf(logf(av), GDN_MIN_LOG_DECAY) : 0.f;   // log a until the prefix
            bp[0][tid] = bt;
        }
        if (tid == 0) jobctr = 0;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int idx = tid + i * NT;
            if (idx < C * CH) {
                const int t = idx / CH, c = idx - t * CH;
                *reinterpret_cast<uint4*>(Ks + kq(t, 8 * c)) = kv[i];
                *reinterpret_cast<uint4*>(Qs + kq(t, 8 * c)) = qv[i];
            }
        }
    }
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
        if (part == 0) (isk ? rk : rq)[t] = p.l2norm ? 1.f / sqrtf(ss + p.eps) : 1.f;
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

    // per direction and processing row: beta, e^{g_C-g}/|k|, and the step's scalars c1 (token
    // order), c2 (token 16 mt + r at r * NB + mt: one vector load per lane of the scan's output
    // wavefront) and gamma_C
    if (tid < 2 * C) {
        const int dir = tid / C, pr = tid - dir * C;
        if (active(dir)) {
            const int t = mrow(dir, pr);
            const float g2 = sg[dir][t], gtot = sg[0][C - 1];
            const float gam = __builtin_amdgcn_exp2f(g2);
            if (dir) bp[1][pr] = bp[0][t];
            w16[dir][pr] = (f16)(__builtin_amdgcn_exp2f(gtot - g2) * rk[t]);
            float* scw = reinterpret_cast<float*>(item_of(dir) + 1024 * (BK::TOTAL + ND * NKT));
            scw[pr] = gam * rk[t];
            scw[C + (pr & 15) * NB + (pr >> 4)] = p.scale * gam * rq[t];
            if (pr == 0) scw[2 * C] = __builtin_amdgcn_exp2f(gtot);
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
    // the K and Q operand fragments of the block's token tiles (shared by both directions)
    {
        constexpr int NKD = (ND + 1) / 2, NKF = ND / 2;
        const int ntile = (T + 15) / 16;
        char* const fragb[2] = {const_cast<char*>(frag_base(p, 0, b, h, NKD)) + (int64_t)NB * j * NKD * 1024,
                                const_cast<char*>(frag_base(p, 1, b, h, NKD)) + (int64_t)NB * j * NKD * 1024};
        for (int job = w; job < 2 * NB * NKD; job += NW) {
            const int kind = job / (NB * NKD), mt = (job / NKD) % NB, ks = job % NKD;
            if (NB * j + mt >= ntile) continue;
            const bf16* rows = kind ? Qs : Ks;
            const int rr = 16 * mt + r;
            uint4 v;
            if (ks < NKF) {
                v = *reinterpret_cast<const uint4*>(rows + kq_full(rr, 32 * ks + 8 * g));
            } else {
                const uint2 hv = *reinterpret_cast<const uint2*>(rows + kq_tail(rr, 16 * (ND - 1) + 4 * g));
                v = uint4{hv.x, hv.y, 0u, 0u};
            }
            gstore16(fragb[kind] + (mt * NKD + ks) * 1024 + 16 * lane, v);
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
    } else {
        // the other wavefronts turn the K rows into fp16 in place (the operand form Z takes;
        // exact for |k| entries in fp16's normal range)
        for (int idx = tid - 2 * C; idx < C * CH; idx += NT - 2 * C) {
            const int t = idx / CH, c = idx - t * CH;
            uint4* pp = reinterpret_cast<uint4*>(Ks + kq(t, 8 * c));
            const bf16x8 xv = __builtin_bit_cast(bf16x8, *pp);
            f16x8 hv;
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = (f16)(float)xv[e];
            *pp = __builtin_bit_cast(uint4, hv);
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

    // E and Z per direction, as independent jobs that the wavefronts take in turn from an LDS
    // counter (the longer Z jobs first, then the E blocks of the lower rows first)
    constexpr int MG = NW / NKT > 0 ? NW / NKT : 1;     // groups of d tiles in a Z job
    constexpr int MPG = (ND + MG - 1) / MG;             // d tiles per group
    constexpr int NEJ = BK::TOTAL, NZJ = NKT * MG;
    // E block -> (row tile, 32-wide step)
    struct EBlocks { int mt[NEJ], ks[NEJ]; };
    constexpr EBlocks eblk = [] {
        EBlocks e{};
        int k = 0;
        for (int m = 0; m < NB; ++m)
            for (int s2 = 0; s2 < BK::count(m); ++s2) { e.mt[k] = m; e.ks[k] = s2; ++k; }
        return e;
    }();
    const int dsh = p.ndirs - 1;   // 0 or 1: job index -> direction by a shift, not a division
    const int nz = NZJ << dsh;
    for (;;) {
        int q = 0;
        if (lane == 0) q = atomicAdd(&jobctr, 1);
        q = __builtin_amdgcn_readfirstlane(q);
        if (q >= ((NEJ + NZJ) << dsh)) break;
        const int dir = dlo + ((q < nz ? q : q - nz) & dsh);
        const int jj = q < nz ? NEJ + (q >> dsh) : NEJ - 1 - ((q - nz) >> dsh);
        const f16* T16 = reinterpret_cast<const f16*>(QT) + dir * US::HALVES;
        const f16* Am = LA + dir * LB::HALVES;
        // the item: BK::TOTAL E blocks, then ND x NKT Z blocks (1 KB each)
        char* const itm = item_of(dir);
        if (jj < NEJ) {
            // E^T = T^T A^T, tile (ut, tt) = sum_s T^T[u][s] A[t][s] over s in [16 ut, 16 tt + 16);
            // the output tiles (2ks, mt) and (2ks + 1, mt) form the O-product A fragment (mt, ks).
            const int blk = jj;
            const int mt = eblk.mt[blk], ks = eblk.ks[blk];
            f32x4 et[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ut = 2 * ks + hh;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (ut <= mt) {
                    // contraction over s in 32-wide steps (zero outside the triangle)
                    for (int ss = (16 * ut) / 32; ss * 32 < 16 * (mt + 1); ++ss) {
                        f16x8 ao, bo;
                        const int sb = 2 * ss + (g >> 1);   // 16-wide block of this lane's s
                        if (32 * ss + 8 * g < C && sb >= ut && sb <= mt) {
                            ao = *reinterpret_cast<const f16x8*>(T16 + US::at(16 * ut + r, 32 * ss + 8 * g));
                            bo = *reinterpret_cast<const f16x8*>(Am + LB::at(16 * mt + r, 32 * ss + 8 * g));
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) ao[e] = bo[e] = (f16)0.f;
                        }
                        acc = mma_f16_k32(ao, bo, acc);
                    }
                }
                // column beta_u of T diag(beta): rows u = 16 ut + 4 g + i of this E^T tile
                const f32x4 bu = (ut < NB) ? *reinterpret_cast<const f32x4*>(&bp[dir][16 * ut + 4 * g])
                                           : f32x4{0.f, 0.f, 0.f, 0.f};
                et[hh] = acc * bu;
            }
            f16x8 fr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fr[e] = (f16)et[0][e];
                fr[4 + e] = (f16)et[1][e];
            }
            gstore16(itm + blk * 1024 + 16 * lane, __builtin_bit_cast(uint4, fr));
        } else {
            // Z = diag(beta) T^T diag(w) K on fp16 MFMA, w = e^{g_C-g}/|k|: A operand T[s][t] w_s
            // (row t, k = s in slots 16 (i/4) + 4 g + i%4 of each 32-wide step), B operand the fp16 K
            // rows read transposed (token row of processing row s; column r of tile m is state
            // index dperm(m, r)).  A job takes the row tiles mt = 2 ks, 2 ks + 1 and a group of d
            // tiles; output tiles (2ks, m) and (2ks + 1, m) form the state-update fragment
            // (m, ks), written whole.
            const int zj = jj - NEJ, mg = zj % MG, ks = zj / MG;
            // K (fp16) read transposed: lane r of group g supplies processing row t + 4 g + r/4 at
            // state indices dperm(m, 4 (r%4)) .. +3.  Its address is kq(mrow(dir, row), d): the
            // row part is a lane constant plus a scalar step (a multiple of 16 rows), so the chunk
            // permutation of the row ((row >> 2) & 3, and bit 3 for a trailing step) depends on
            // the lane only.
            const int u = 4 * g + (r >> 2);
            const int xs = dir ? 1 - ((u >> 3) & 1) : ((u >> 3) & 1);
            const int s4 = dir ? 3 - g : g;   // ((row >> 2) & 3) of token row mrow(dir, 16 k + u)
            const int kl = (dir ? C - 1 - u : u) * D;
            const int rstep = dir ? -D : D;
            const int cb = 8 * ((r & 3) ^ s4), cbs = 8 * (((r & 3) >> 1) ^ xs) + 4 * (r & 1);
            auto kaddr = [&](int trow, int m) {
                const int col = (m < (ND & ~1)) ? 32 * (m >> 1) + 4 * (m & 1) + cb : 16 * m + cbs;
                return Ks + kl + trow * rstep + col;
            };
            f32x4 acc[2][MPG];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int mi = 0; mi < MPG; ++mi) acc[hh][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int ss = ks; ss < NKT; ++ss) {
                f16x8 aw[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int mt = 2 * ks + hh;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int s0 = 32 * ss + 16 * hf + 4 * g;
                        f16x4 tv = {(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
                        if (mt < NB && s0 < C && 2 * ss + hf >= mt) {   // T[s][t] = 0 for s < t
                            tv = *reinterpret_cast<const f16x4*>(T16 + US::at(16 * mt + r, s0));
                            tv = tv * *reinterpret_cast<const f16x4*>(&w16[dir][s0]);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) aw[hh][4 * hf + e] = tv[e];
                    }
                }
#pragma unroll
                for (int mi = 0; mi < MPG; ++mi) {
                    const int m = mg * MPG + mi;
                    if (m < ND) {
                        s16x4 lo = {0, 0, 0, 0}, hi4 = {0, 0, 0, 0};
                        if (32 * ss < C)
                            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)kaddr(32 * ss, m));
                        if (32 * ss + 16 < C)
                            hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)kaddr(32 * ss + 16, m));
                        const f16x4 lh = __builtin_bit_cast(f16x4, lo), hh4 = __builtin_bit_cast(f16x4, hi4);
                        const f16x8 bh16 = {lh[0], lh[1], lh[2], lh[3], hh4[0], hh4[1], hh4[2], hh4[3]};
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            if (2 * ks + hh < NB) acc[hh][mi] = mma_f16_k32(aw[hh], bh16, acc[hh][mi]);
                    }
                }
            }
            f32x4 bt4[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int mt = 2 * ks + hh;
                bt4[hh] = (mt < NB) ? *reinterpret_cast<const f32x4*>(&bp[dir][16 * mt + 4 * g]) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int mi = 0; mi < MPG; ++mi) {
                const int m = mg * MPG + mi;
                if (m < ND) {
                    const f32x4 z0 = acc[0][mi] * bt4[0], z1 = acc[1][mi] * bt4[1];
                    const f16x8 fr = {(f16)z0[0], (f16)z0[1], (f16)z0[2], (f16)z0[3], (f16)z1[0], (f16)z1[1], (f16)z1[2], (f16)z1[3]};
                    gstore16(itm + (BK::TOTAL + m * NKT + ks) * 1024 + 16 * lane, __builtin_bit_cast(uint4, fr));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk scan: one workgroup per (direction, b, h, slice of 32 state rows),
// serial over the processing steps.  Rows of S evolve independently, so the
// slices of a head need no exchange.  Six wavefronts with fixed roles:
//   chain (2, one per 16-row column tile of the slice): per step X = K S^T,
//                     R = V - diag(c1) X; the step's state (bf16) and R (fp16)
//                     go to an LDS ring, then S^T <- gamma_C S^T + Z^T R.  The
//                     state tile lives in MFMA accumulators for the whole call.
//   output (2, one per half of the step's token tiles): O^T = S Q^T diag(c2) +
//                     R^T E^T from the ring and their own Q, E and c2 (loaded
//                     two steps ahead); bf16 tiles leave through LDS staging.
//   loader (2): deposit each step's K, scalars (loader 0) and Z, V (loader 1)
//                     in a 3-slot operand ring, loaded into registers two steps
//                     before.
// The wavefronts are coupled only through the rings and LDS counters with
// bounded spins: the output wavefronts may trail the chain by up to
// ring_slots() - 1 steps, the loaders run ahead of it by up to two slots.  An
// operand register of an MFMA is refilled only after a result depending on
// that MFMA has been consumed.
//
// Row addressing: the buffer resource of a step starts at the lowest token of
// the step and ends after the last real token, so a row's byte offset is a
// per-lane constant and rows past the end of the sequence read as zero (and
// are not stored).  State rows past d_v (the last slice when d_v is not a
// multiple of 32) are computed from zero inputs and never stored.
// ---------------------------------------------------------------------------
#define GDN_COLS 2       // 16-row column tiles of the state per workgroup
// output ring slots
template <int ND>
__host__ __device__ constexpr int ring_slots() { return 3; }
#define GDN_OPS 3         // operand ring slots
#define GDN_STAGES 2      // register stages of each loader (its loads run up to GDN_STAGES steps ahead of the ring)
#define GDN_SPIN_LIMIT (1 << 22)

template <int NT, int ND>
struct Rows {                    // NT row tiles of Q (lane = row) as MFMA operands
    uint4 op[NT][(ND + 1) / 2];  // [tile][ks]: 8 consecutive d; a trailing single tile holds 4 and zeros
};

template <int NB>
struct VIn {                     // chain operands of one step used right after X
    uint4 v[GDN_COLS][2];        // V row of one token, columns row0 + 16c .. +15 (bf16)
    f32x4 c1[NB];
    float gC;
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

// Wait until an LDS counter written by another wavefront reaches `target`.
// Bounded, so a wavefront can never hang here.  The poll does not sleep between
// reads: a hand-off is seen one LDS round trip after it happens (with a 64-cycle
// sleep per poll the scan measured 0.6 us slower per 720p call).
__device__ __forceinline__ void wait_counter(int* cnt, int target) {
    for (int it = 0; it < GDN_SPIN_LIMIT; ++it) {
        if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Set a counter once this wavefront's earlier LDS writes (or reads) are done.  The LDS
// performs the operations of one wavefront in the order they were issued, so a counter
// store issued after them is seen by another wavefront only once they have taken effect:
// the store needs to stay behind them in the instruction stream (an instruction of its own
// with a memory clobber), not to wait for them.
__device__ __forceinline__ void signal_counter(int* cnt, int value) {
    const unsigned addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)cnt;
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(value) : "memory");
}

template <int NB>
struct ScanShape {
    static constexpr int NOUT = NB >= 2 ? 2 : 1;   // output wavefronts
    static constexpr int TPO = NB / NOUT;          // token tiles per output wavefront
    static constexpr int THREADS = 64 * (GDN_COLS + NOUT + 2);   // + chain wavefronts + two loaders
};

// One step's chain operands as the loader wavefronts deposit them (lane l's 16 bytes of a
// block at byte 16 l), so each block is one MFMA operand fragment read back with one
// 16-byte LDS read.
template <int NB, int ND>
struct ScanOps {
    static constexpr int NKD = (ND + 1) / 2;   // 32-wide k-steps over d (the last half-filled for odd ND)
    static constexpr int NKT = Blocks<NB>::NFULL + (Blocks<NB>::HALF ? 1 : 0);
    uint4 k[NB][NKD][64];                // K fragments of processing tile mt (as stored by the prep)
    uint4 z[ND][NKT][64];                // state-update fragments of the item
    uint4 v[NB][64];                     // V row slices, [token][4 chunks of 16 bytes] (see vslot)
    uint4 sc[64];                        // lanes 0..15: c1 (64 floats); lane 16: gamma_C
};

template <int NB, int ND>
struct ScanLds {
    static constexpr int NKD = (ND + 1) / 2;
    static constexpr int NKT = Blocks<NB>::NFULL + (Blocks<NB>::HALF ? 1 : 0);
    uint4 ringP[ring_slots<ND>()][NKD][GDN_COLS][64];
    uint4 ringR[ring_slots<ND>()][NKT][GDN_COLS][64];
    ScanOps<NB, ND> ops[GDN_OPS];
    uint4 ostage[ScanShape<NB>::NOUT][ScanShape<NB>::TPO][64];   // bf16 output tiles on their way out
};

// A token's 64-byte slice (32 state rows, bf16) in LDS holds its 16-byte chunk j at position
// j ^ vswz(t): tokens 4 apart land on different banks for the chain's transposing reads
// and the output tiles' writes, while each lane quad moves one token's 64 contiguous bytes.
__device__ __forceinline__ int vswz(int t) { return 2 * ((t >> 2) & 1); }
__device__ __forceinline__ int oswz(int t) { return (t >> 2) & 3; }

// Progress counters of the scan's wavefronts (an LDS object of their own).
template <int NB>
struct ScanCtr {
    int ready[GDN_COLS];                 // steps each chain wavefront has published to the output
                                         // ring (and so finished reading from the operand slots)
    int done[ScanShape<NB>::NOUT];       // steps each output wavefront has taken from the ring
    int loaded[2];                       // steps whose operands loader 0 / loader 1 has landed
};

// Store a progress counter to LDS as an instruction of its own: it takes effect after the
// wavefront's earlier LDS stores (one wavefront's LDS operations complete in issue order),
// and the memory clobber keeps the compiler from moving those stores past it.
__device__ __forceinline__ void publish_loaded(int* cnt, int value) {
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
// wavefront O takes tiles O and NB-1-O, so both carry the same number of E blocks (a tile's
// E blocks grow with its distance from the start of the step).
template <int NB>
__host__ __device__ constexpr int out_tile(int O, int tt) {
    return ScanShape<NB>::TPO == 2 ? (tt == 0 ? O : NB - 1 - O) : O * ScanShape<NB>::TPO + tt;
}
template <int NB, int ND, int O>
__device__ __forceinline__ void scan_output(const Params& p, ScanLds<NB, ND>& L, ScanCtr<NB>& K, int lane, int b, int h, int dir, int T,
                                            int N, int row0, const char* item0, int64_t ib) {
    constexpr int C = 16 * NB, D = 16 * ND;
    constexpr int NKD = (ND + 1) / 2;
    using BK = Blocks<NB>;
    constexpr int NKT = BK::NFULL + (BK::HALF ? 1 : 0);
    constexpr int TPO = ScanShape<NB>::TPO;
    // E blocks of this wavefront's tiles, tile after tile
    constexpr auto eoff = [](int tt) { int o = 0; for (int t2 = 0; t2 < tt; ++t2) o += BK::count(out_tile<NB>(O, t2)); return o; };
    constexpr int EB = eoff(TPO);
    constexpr int SCAL_OFF = 1024 * (BK::TOTAL + ND * NKT);
    const int r = lane & 15, g = lane >> 4;
    struct OutIn {
        Rows<TPO, ND> q;
        uint4 efr[EB];
        float c2[TPO];
    };

    // Q fragments (16 bytes per lane, the rows of a tile reversed for the reverse direction)
    const auto qfr = make_rsrc(frag_base(p, 1, b, h, NKD), (uint32_t)(((T + 15) / 16) * NKD * 1024));
    const int qfl = 16 * ((dir ? 15 - r : r) + 16 * g);
    // o is bf16, or fp32 when the call's I/O is fp32 (its q, k, v were staged as bf16)
    const int oesz = p.io_f32 ? 4 : 2;
    const StepRows orow{reinterpret_cast<const char*>(p.o[dir]) + ((int64_t)b * p.os[0] + (int64_t)h * p.os[2]) * oesz,
                        p.os[1] * oesz, T, C, N, dir, oesz * D};
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

    OutIn oA, oB;
    const auto irs = make_rsrc(item0, (uint32_t)(N * ib));
    auto load_out = [&](OutIn& o, int n) {
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt) {
            const int tile = frag_tile(dir, N, NB, n, out_tile<NB>(O, tt));   // past the last token: zero
#pragma unroll
            for (int ks = 0; ks < NKD; ++ks)
                o.q.op[tt][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qfr, qfl, (tile * NKD + ks) * 1024, 0));
        }
        const int ioff = n * (int)ib;
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int kt = 0; kt < BK::count(out_tile<NB>(O, tt)); ++kt)
                o.efr[eoff(tt) + kt] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(irs, 16 * lane, ioff + 1024 * (BK::offset(out_tile<NB>(O, tt)) + kt), 0));
        // c2 of tokens 16 mt + r of this wavefront's tiles mt (lane-major scalars)
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
            o.c2[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (NB * r + out_tile<NB>(O, tt)),
                                                                                      ioff + SCAL_OFF + 4 * C, 0));
    };

    load_out(oA, 0);
    load_out(oB, N > 1 ? 1 : 0);
    auto out_step = [&](OutIn& o, int n) {
        const int sl = n % ring_slots<ND>();
#pragma unroll
        for (int c = 0; c < GDN_COLS; ++c) wait_counter(&K.ready[c], n + 1);
        bf16x8 Pb[NKD][GDN_COLS];
        f16x8 Rb[NKT][GDN_COLS];
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Pb[ks][c] = __builtin_bit_cast(bf16x8, L.ringP[sl][ks][c][lane]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Rb[kt][c] = __builtin_bit_cast(f16x8, L.ringR[sl][kt][c][lane]);
        // the slot is free once its fragments are in registers
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) keep_alive(Pb[ks][c]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) keep_alive(Rb[kt][c]);
        signal_counter(&K.done[O], n + 1);
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
                for (int c = 0; c < GDN_COLS; ++c)
                    Ot[tt][c] = mma_bf16_k32(Pb[ks][c], __builtin_bit_cast(bf16x8, o.q.op[tt][ks]), Ot[tt][c]);
#pragma unroll
        for (int tt = 0; tt < TPO; ++tt)
#pragma unroll
            for (int c = 0; c < GDN_COLS; ++c) Ot[tt][c] = Ot[tt][c] * o.c2[tt];
        // + R^T E^T (a trailing 16-token step has zero upper slots in both operands)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int tt = 0; tt < TPO; ++tt) {
                if (kt >= BK::count(out_tile<NB>(O, tt))) continue;
                const f16x8 ef = __builtin_bit_cast(f16x8, o.efr[eoff(tt) + kt]);
#pragma unroll
                for (int c = 0; c < GDN_COLS; ++c) Ot[tt][c] = mma_f16_k32(Rb[kt][c], ef, Ot[tt][c]);
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
__global__ __launch_bounds__(ScanShape<NB>::THREADS) void gdn_scan_kernel(Params p, int ngroups) {
    constexpr int C = 16 * NB, D = 16 * ND;
    constexpr int NKD = (ND + 1) / 2;      // k-steps over d (the last one half-filled for odd ND)
    constexpr int NKF = ND / 2;            // full k-steps over d
    constexpr int NS = (ND + GDN_COLS - 1) / GDN_COLS;   // slices per head
    using BK = Blocks<NB>;
    constexpr int NFT = BK::NFULL;         // 32-wide steps over tokens
    constexpr bool HT = BK::HALF;
    constexpr int NKT = NFT + (HT ? 1 : 0);
    constexpr int SCAL_OFF = 1024 * (BK::TOTAL + ND * NKT);   // scalars of an item
    constexpr int NOUT = ScanShape<NB>::NOUT;
    // loads the loader wavefronts issue per step: K and the scales; Z and V
    constexpr int NDMA0 = NB * NKD + 1;
    constexpr int NDMA1 = ND * NKT + NB;
    typedef short s16x4 __attribute__((ext_vector_type(4)));

    __shared__ __align__(16) ScanLds<NB, ND> L;
    __shared__ ScanCtr<NB> K;

    const int lane = threadIdx.x & 63;
    // the role of a wavefront is wave-uniform: keep it in a scalar register so every
    // role is a whole-wavefront branch
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    // Workgroups are spread over the 8 XCDs round-robin (id % 8); keep the NS
    // slices of one (direction, b, h) on one XCD so they share its L2.
    const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
    const int group = (slot / NS) * 8 + xcd, j = slot - (slot / NS) * NS;
    if (group >= ngroups) return;
    int gg = group;
    const int h = gg % p.H; gg /= p.H;
    const int b = gg % p.B; gg /= p.B;
    const int dir = p.dir0 + gg;
    const int T = (int)p.T;
    const int N = (T + C - 1) / C;
    const int row0 = 16 * GDN_COLS * j;
    const char* item0 = p.ws + (((int64_t)dir * p.B + b) * p.H + h) * p.nsub_max * p.ws_item_bytes;
    const int64_t ib = p.ws_item_bytes;
    bool col_ok[GDN_COLS];
#pragma unroll
    for (int c = 0; c < GDN_COLS; ++c) col_ok[c] = row0 + 16 * c < p.Dv;

    if (threadIdx.x == 0) {
#pragma unroll
        for (int c = 0; c < GDN_COLS; ++c) K.ready[c] = 0;
#pragma unroll
        for (int o = 0; o < NOUT; ++o) K.done[o] = 0;
        K.loaded[0] = K.loaded[1] = 0;
    }
    __syncthreads();

    const StepRows vr{reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.v) + (int64_t)b * p.vs[0] +
                                                    (int64_t)h * p.vs[2]),
                      p.vs[1] * 2, T, C, N, dir, 2 * D};
    // the items of this (direction, b, h), addressed with lane-constant offsets
    const auto irs = make_rsrc(item0, (uint32_t)(N * ib));

    // roles: waves 0 .. GDN_COLS-1 chain, then the output wavefronts, then the two
    // loaders (which share SIMDs with the chain wavefronts and move data without VGPRs)
    if (wave >= GDN_COLS + NOUT) {
        // ------------------------------ loader wavefronts ------------------------------
        // Deposit the chain's operands of step n in slot n % GDN_OPS once both chain
        // wavefronts are done with that slot, and publish the step.  The operands are
        // loaded into registers GDN_STAGES steps before they are deposited, so each step's
        // loads are in flight while the chain works ~GDN_STAGES + 2 steps behind them.
        // Loader 0 moves K and the scales, loader 1 the state-update fragments Z and V;
        // each publishes its own count.
        const int part = wave - (GDN_COLS + NOUT);
        // K fragments: 16 bytes per lane, the rows of a tile reversed for the reverse direction
        const auto kfr = make_rsrc(frag_base(p, 0, b, h, NKD), (uint32_t)(((T + 15) / 16) * NKD * 1024));
        const int kfl = 16 * ((dir ? 15 - r : r) + 16 * g);
        // V: lane quad l/4 moves token 16 jj + l/4's slice, lane l%4 its chunk at position l%4;
        // chunks of column tiles past d_v are read from outside the resource (zero)
        static_assert(GDN_COLS == 2, "V slices are 64 bytes");
        int voff[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const int t = 16 * jj + (lane >> 2), j = (lane & 3) ^ vswz(t);
            voff[jj] = (row0 + 16 * (j >> 1) < p.Dv) ? vr.row(t) + 2 * row0 + 16 * j : (int)0x80000000;
        }
        const int scoff = lane < 16 ? 16 * lane : (lane == 16 ? 8 * C : 0);
        static_assert(GDN_STAGES * NDMA0 <= 63 && GDN_STAGES * NDMA1 <= 63, "loads in flight per loader");
        auto ld16 = [](__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
        };
        // loader 0: K fragments (NB x NKD blocks), then the scalars; loader 1: Z (ND x NKT), then V (NB)
        auto load0 = [&](uint4* st, int n) {
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) {
                // tiles past the last token read as zero (outside the resource)
                const int tile = frag_tile(dir, N, NB, n, mt);
#pragma unroll
                for (int ks = 0; ks < NKD; ++ks) st[mt * NKD + ks] = ld16(kfr, kfl, (tile * NKD + ks) * 1024);
            }
            st[NB * NKD] = ld16(irs, scoff, n * (int)ib + SCAL_OFF);
        };
        auto put0 = [&](const uint4* st, int n) {
            ScanOps<NB, ND>& op = L.ops[n % GDN_OPS];
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                for (int ks = 0; ks < NKD; ++ks) op.k[mt][ks][lane] = st[mt * NKD + ks];
            op.sc[lane] = st[NB * NKD];
        };
        auto load1 = [&](uint4* st, int n) {
            const int ioff = n * (int)ib;
#pragma unroll
            for (int m = 0; m < ND; ++m)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) st[m * NKT + kt] = ld16(irs, 16 * lane, ioff + 1024 * (BK::TOTAL + m * NKT + kt));
            const auto vrs = vr.rsrc(n);
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) st[ND * NKT + jj] = ld16(vrs, voff[jj], 0);
        };
        auto put1 = [&](const uint4* st, int n) {
            ScanOps<NB, ND>& op = L.ops[n % GDN_OPS];
#pragma unroll
            for (int m = 0; m < ND; ++m)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) op.z[m][kt][lane] = st[m * NKT + kt];
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) op.v[jj][lane] = st[ND * NKT + jj];
        };
        // Per step n: wait for slot n % GDN_OPS, wait for stage n % GDN_STAGES (the loads of the
        // other stages may still be in flight: the loads of a wavefront complete in order), write
        // it to the slot, publish, and reload the stage with step n + GDN_STAGES.
        auto run = [&](auto load, auto put, auto wait_stage) {
            constexpr int NL = NDMA1 > NDMA0 ? NDMA1 : NDMA0;
            uint4 st[GDN_STAGES][NL];
#pragma unroll
            for (int i = 0; i < GDN_STAGES; ++i) load(st[i], i < N ? i : N - 1);
            for (int n = 0; n < N; n += GDN_STAGES) {
#pragma unroll
                for (int i = 0; i < GDN_STAGES; ++i) {
                    const int m = n + i;
                    if (m >= N) break;
#pragma unroll
                    for (int c = 0; c < GDN_COLS; ++c) wait_counter(&K.ready[c], m + 1 - GDN_OPS);
                    wait_stage();
                    put(st[i], m);
                    publish_loaded(&K.loaded[part], m + 1);
                    load(st[i], m + GDN_STAGES < N ? m + GDN_STAGES : N - 1);
                }
            }
            wait_vmcnt<0>();
        };
        // the other stages' loads may still be in flight
        if (part == 0) run(load0, put0, [] { wait_vmcnt<(GDN_STAGES - 1) * NDMA0>(); });
        else run(load1, put1, [] { wait_vmcnt<(GDN_STAGES - 1) * NDMA1>(); });
        return;
    }
    if (wave == GDN_COLS) {
        scan_output<NB, ND, 0>(p, L, K, lane, b, h, dir, T, N, row0, item0, ib);
        return;
    }
    if constexpr (NOUT > 1) {
        if (wave == GDN_COLS + 1) {
            scan_output<NB, ND, 1>(p, L, K, lane, b, h, dir, T, N, row0, item0, ib);
            return;
        }
    }

    // ------------------------------ chain wavefronts ------------------------------
    // Chain wavefront cc owns state rows row0 + 16 cc .. +15.  Per step n: wait for the
    // step's operands; Pb = bf16(S); read K, the scales and Z from the operand slot;
    // X = K S^T on MFMA while the VALU decays the state and reads V back transposed;
    // R = V - c1 X; release the slot; publish the state and R to the output ring;
    // S^T += Z^T R on MFMA.
    const int cc = wave;
    const bool tile_ok = row0 + 16 * cc < p.Dv;
    f32x4 P[ND];   // P[m][i] = S[row0 + 16 cc + r][dperm(m, 4 g + i)]
    const float* Sin = (dir == 0) ? p.S_in : nullptr;
    const int64_t hbase = ((int64_t)b * p.H + h) * D * D;
    const int64_t srow = hbase + (int64_t)(row0 + 16 * cc + r) * D;
#pragma unroll
    for (int m = 0; m < ND; ++m) {
        if (Sin && tile_ok)
            P[m] = *reinterpret_cast<const f32x4*>(Sin + srow + dperm<ND>(m, 4 * g));
        else
            P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int done_seen[NOUT];
#pragma unroll
    for (int o = 0; o < NOUT; ++o) done_seen[o] = 0;
    // K fragments of a step, read one step ahead (while the state update runs); a trailing
    // half k-step (odd ND) has zero upper slots
    uint4 kf[NB][NKD];
    auto read_k = [&](const ScanOps<NB, ND>& op, int dep) {
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) kf[mt][ks] = op.k[mt][ks][lane + dep];
    };
    wait_counter(&K.loaded[0], 1);
    wait_counter(&K.loaded[1], 1);
    read_k(L.ops[0], 0);
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
        const int sl = n % ring_slots<ND>();
        const ScanOps<NB, ND>& op = L.ops[n % GDN_OPS];
        // the loaders' counts, read now so that they are back before the next step's K is read
        const int ld0 = __hip_atomic_load(&K.loaded[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int ld1 = __hip_atomic_load(&K.loaded[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int ldc = ld0 < ld1 ? ld0 : ld1;
        // the output ring slot of this step must have been released by every output
        // wavefront (the last counts seen are kept, so the counters are read only when needed)
#pragma unroll
        for (int o = 0; o < NOUT; ++o)
            if (done_seen[o] < n + 1 - ring_slots<ND>()) {
                wait_counter(&K.done[o], n + 1 - ring_slots<ND>());
                done_seen[o] = __hip_atomic_load(&K.done[o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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
        // The Z fragments are read into the registers the previous state update took its
        // operands from: their LDS addresses depend on Pb (through an empty asm), and Pb
        // on every result of that update, so the reads issue only once it has finished.
        int zdep = 0;
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) asm volatile("" : "+v"(zdep) : "v"(Pb[ks]));
        // publish the state to the output ring right away
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) L.ringP[sl][ks][cc][lane] = __builtin_bit_cast(uint4, Pb[ks]);
        // the step's remaining operands, in order of use: the scales and V (read back
        // transposed: lane quad q of group g supplies row 16 mt + 4 g + i, columns
        // 16 cc + 4 q .. +3 of the deposited rows), then Z.  c1 of the tokens 16 mt + 4 g + i
        // this lane scales is read once per row of 16 lanes (lane 4 mt + i holds it) and
        // handed round the row by broadcasts.
        const float c1l = reinterpret_cast<const float*>(&op.sc[0])[16 * (r >> 2) + 4 * g + (r & 3)];
        const float gC = reinterpret_cast<const float*>(&op.sc[16])[0];
        bf16x4 vt[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            const int q = r & 3, t = 16 * mt + 4 * g + (r >> 2);
            const char* vp = reinterpret_cast<const char*>(&op.v[0][0]) + 64 * t + 16 * ((2 * cc + (q >> 1)) ^ vswz(t)) + 8 * (q & 1);
            vt[mt] = __builtin_bit_cast(
                bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)vp));
        }
        uint4 zfr[ND][NKT];
#pragma unroll
        for (int m = 0; m < ND; ++m)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) zfr[m][kt] = op.z[m][kt][lane + zdep];
        // X = K S^T (rows: tokens 16 mt + 4 g + i, column: state row 16 cc + r)
        f32x4 X[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) X[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) X[mt] = mma_bf16_k32(__builtin_bit_cast(bf16x8, kf[mt][ks]), Pb[ks], X[mt]);
        // meanwhile: decay the state
#pragma unroll
        for (int m = 0; m < ND; ++m) P[m] = P[m] * gC;
        // R = V - diag(e^g / |k|) X, as fp16 B operand (k = token)
        float c1[16];
        row_broadcasts(c1l, c1, std::make_integer_sequence<int, 16>{});
        f16x8 Rb[NKT];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) Rb[mt >> 1][4 * (mt & 1) + i] = (f16)((float)vt[mt][i] - c1[4 * mt + i] * X[mt][i]);
        if constexpr (HT) {
#pragma unroll
            for (int i = 4; i < 8; ++i) Rb[NFT][i] = (f16)0.f;
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) L.ringR[sl][kt][cc][lane] = __builtin_bit_cast(uint4, Rb[kt]);
        // issue order of the step: the conversions and ring writes of Pb, then each X
        // MFMA followed by two of the operand reads, then the arithmetic of R
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * NKD, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, NKD, 0);
#pragma unroll
        for (int i = 0; i < NB * NKD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        signal_counter(&K.ready[cc], n + 1);
        // the next step's operands must have landed before its K is read (the addresses of
        // the reads depend on the count, through an empty asm, so they follow it)
        if (n + 1 < N) {
            int kdep = 0;
            if (ldc < n + 2) {
                wait_counter(&K.loaded[0], n + 2);
                wait_counter(&K.loaded[1], n + 2);
            }
            asm volatile("" : "+v"(kdep) : "v"(ldc));
            read_k(L.ops[(n + 1) % GDN_OPS], kdep);
        }
        // S^T <- gamma_C S^T + Z^T R  (rows d, columns: state rows); a trailing 16-token
        // step has zero upper slots in both operands
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int m = 0; m < ND; ++m) P[m] = mma_f16_k32(__builtin_bit_cast(f16x8, zfr[m][kt]), Rb[kt], P[m]);
    }
    float* Sout = p.S_out[dir];
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
    hipLaunchKernelGGL((gdn_prep_kernel<NB, ND>), dim3(nsub, p.B * p.H), dim3(128 * NB), 0, s, p);
    tm_end(tm, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ngroups = p.ndirs * p.B * p.H;
    const int grid = (ngroups + 7) / 8 * 8 * ((ND + GDN_COLS - 1) / GDN_COLS);
    tm_begin(tm, s, KSCAN);
    hipLaunchKernelGGL((gdn_scan_kernel<NB, ND>), dim3(grid), dim3(ScanShape<NB>::THREADS), 0, s, p, ngroups);
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
    (void)io_f32;   // fp32 q, k, v are staged as bf16 (gdn_to_bf16_kernel), o is stored in fp32
    if (Dk != Dv) return false;
    if (!(Dk == 16 || Dk == 32 || Dk == 64 || Dk == 112 || Dk == 128)) return false;
    return C == 16 || C == 32 || C == 64;
}

hipError_t launch_chunked(const Params& p0, hipStream_t s, Timing* tm) {
    Params p = p0;
    if (p.io_f32) {
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
    }
    switch (p.C) {
        case 16: return run_chunked_d<1>(p, s, tm);
        case 32: return run_chunked_d<2>(p, s, tm);
        case 64: return run_chunked_d<4>(p, s, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
