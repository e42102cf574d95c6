// gdn_attention.hip -- softmax attention of a streaming chunk over a sink + sliding-window
// cache: the hybrid DiT's softmax block (SANA-Streaming pages, Chinese summary "Core method":
// sliding window plus persistent sink, fixed memory, token-level correspondence across chunk
// boundaries).  Per (stream, head) every query of the chunk attends over the cached sink
// tokens, the cached window tokens and all tokens of the chunk:
//
//     o_t = sum_j softmax_j(scale q_t . k_j) v_j
//
// One workgroup of NWAVE wavefronts takes QT consecutive queries of one (stream, head); each
// wavefront keeps its QB x 16 queries' Q fragments in registers for the whole call.  Keys and
// values stream through LDS in tiles of KT keys (four buffers, one barrier per pair of tiles),
// tile after tile over the three segments (sink, window, chunk); a segment's last tile is masked.
// Products run on 16x16x32 bf16 MFMAs in transposed form:
//
//     S^T = K Q^T      (A = K rows from LDS, B = Q fragments in registers)
//     O^T += V^T P^T   (A = V^T rows from LDS, B = P^T built from S^T in registers)
//
// The output tile of S^T (lane l: query l % 16, keys 4g..4g+3, g = l / 16) is the B operand
// of the second product once its key index becomes the contraction index: slot i of group g
// in a 32-key step c stands for key 32c + 4g + i (i < 4) or 32c + 16 + 4g + (i - 4) (i >= 4).
// V is written to LDS transposed, in exactly that key order, so that each A operand is one
// 16-byte LDS read.  Both LDS tiles are k-major in blocks of 16 rows (key rows of K, d rows of
// V^T), with the row index XOR-ed by the 16-byte chunk: chunk u of row r at block + 256 u +
// 16 ((r % 16) ^ u).  A 16-byte operand read (16 rows, one chunk per 16-lane group) then covers
// one aligned 256-byte run of LDS, which this chip serves without bank conflicts, and the
// deposits of a row's consecutive chunks fall on different bank groups.  The softmax is online in the log2 domain (reference maximum m and partial
// sum l per lane; O^T and l rescaled by 2^(m_old - m_new) when m moves); p enters the second
// product rounded to bf16, l sums the fp32 values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 64;                 // keys per tile
constexpr int QB = 2;                  // 16-query blocks per wavefront
constexpr int NWAVE = 7;               // wavefronts per workgroup (224 queries: 240 workgroups at the
                                       // 720p layer, one per CU, against 220 with 8)
constexpr int NTHR = NWAVE * 64;
constexpr int QT = NWAVE * QB * 16;    // queries per workgroup

template <int D>
struct Tile {
    static constexpr int KBLK = (D / 8) * 256;    // one 16-key block of the K tile (D / 8 chunks)
    static constexpr int K_BYTES = (KT / 16) * KBLK;
    static constexpr int V_BYTES = (D / 16) * 2048;   // D / 16 blocks of 16 d rows x 8 chunks (64 keys)
    static constexpr int BUF = K_BYTES + V_BYTES;
    static constexpr int NS = D / 32;             // full 32-wide steps over d
    static constexpr bool TAIL = (D % 32) != 0;   // plus one 16-wide step
    static constexpr int ND = D / 16;             // 16-row blocks of d in O^T
    static constexpr int KCH = D / 8;             // 16-byte chunks per row
    static constexpr int KLOADS = (KT * KCH + NTHR - 1) / NTHR;
    static_assert(16 * KCH <= NTHR && KCH <= 16, "one V task per thread; chunk index within a 16-row block");
};
// byte offset of 16-byte chunk u of row r in a k-major XOR-ed tile whose 16-row blocks are blk bytes
__device__ __forceinline__ int kmaj(int r, int u, int blk) { return (r >> 4) * blk + 256 * u + 16 * ((r & 15) ^ u); }

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A 16-wide step as a 32-wide MFMA with zero upper slots in both operands.
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16 z = (bf16)0.f;
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8{a[0], a[1], a[2], a[3], z, z, z, z},
                                                   bf16x8{b[0], b[1], b[2], b[3], z, z, z, z}, c, 0, 0, 0);
}

// loads through the global address space (flat loads would also hold the LDS counter)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload16(const void* p) {
    return __builtin_bit_cast(uint4, *(__attribute__((address_space(1))) const u32x4*)p);
}
__device__ __forceinline__ uint2 gload8(const void* p) {
    return __builtin_bit_cast(uint2, *(__attribute__((address_space(1))) const u32x2*)p);
}
// Reductions over the 4 lanes that share a query (lanes l, l ^ 16, l ^ 32, l ^ 48) with the
// gfx950 lane swaps: with both operands the same value, the pair returned by
// permlane16_swap holds, in every lane, its own and its l ^ 16 partner's value (in some
// order), and permlane32_swap likewise for l ^ 32.
__device__ __forceinline__ float max4q(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(x);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4q(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(x);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// raw buffer resource over [base, base + bytes); loads beyond it return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D>
__global__ __launch_bounds__(NTHR, 2) void attn_kernel(AttnParams p) {
    using TL = Tile<D>;
    __shared__ __align__(16) char lds[4 * TL::BUF];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    // Work item of this workgroup.  Consecutive workgroups are dispatched to the 8 XCDs in
    // turn, and each XCD has its own L2: the k-th workgroup of XCD x takes item
    // start(x) + k, so that an XCD works through a contiguous band of items, i.e. through the
    // query tiles of a few heads, whose keys and values then stay in its L2.
    const int nwg = gridDim.x, xcd = blockIdx.x % 8, k8 = blockIdx.x / 8;
    const int item = xcd * (nwg / 8) + min(xcd, nwg % 8) + k8;
    const int nqt = (p.T + QT - 1) / QT;
    const int qtile = item % nqt, h = (item / nqt) % p.H, b = item / (nqt * p.H);
    const int64_t bh = (int64_t)b * p.H + h;
    const int64_t q0 = (int64_t)qtile * QT + wave * (QB * 16);
    // launch arguments as plain locals (the lambdas below must not take the argument block's address)
    const int T = p.T, n_sink = p.n_sink, n_win = p.n_win;
    const int64_t ks_chunk = p.ks[1], vs_chunk = p.vs[1];
    const float scale_log2 = p.scale_log2;

    // Q fragments: lane holds query q0 + 16 qb + r, d = 32 s + 8 g .. +7 (tail: d = 32 NS + 4 g .. +3)
    bf16x8 qf[QB][TL::NS > 0 ? TL::NS : 1];
    bf16x4 qt[QB];
    {
        const bf16* qbase = static_cast<const bf16*>(p.q) + b * p.qs[0] + h * p.qs[2];
        for (int qb = 0; qb < QB; ++qb) {
            const int64_t t = q0 + 16 * qb + r;
            const bool in = t < T;
            const bf16* row = qbase + (in ? t : 0) * p.qs[1];
#pragma unroll
            for (int s = 0; s < TL::NS; ++s) {
                uint4 x = in ? gload16(row + 32 * s + 8 * g) : uint4{0, 0, 0, 0};
                qf[qb][s] = __builtin_bit_cast(bf16x8, x);
            }
            if constexpr (TL::TAIL) {
                uint2 x = in ? gload8(row + 32 * TL::NS + 4 * g) : uint2{0, 0};
                qt[qb] = __builtin_bit_cast(bf16x4, x);
            }
        }
    }

    // the three key/value segments: sink, window (cache, [B][H][capacity][D]) and the chunk
    const bf16* k0 = static_cast<const bf16*>(p.k_sink) + bh * p.sink_cap * D;
    const bf16* v0 = static_cast<const bf16*>(p.v_sink) + bh * p.sink_cap * D;
    const bf16* k1 = static_cast<const bf16*>(p.k_win) + bh * p.win_cap * D;
    const bf16* v1 = static_cast<const bf16*>(p.v_win) + bh * p.win_cap * D;
    const bf16* k2 = static_cast<const bf16*>(p.k) + b * p.ks[0] + h * p.ks[2];
    const bf16* v2 = static_cast<const bf16*>(p.v) + b * p.vs[0] + h * p.vs[2];
    const int nt0 = (n_sink + KT - 1) / KT, nt1 = (n_win + KT - 1) / KT, nt2 = (T + KT - 1) / KT;
    const int ntiles = nt0 + nt1 + nt2;

    // valid rows of tile t (uniform)
    auto tile_rows = [&](int t) __attribute__((always_inline)) {
        if (t < nt0) return min(KT, n_sink - t * KT);
        if (t < nt0 + nt1) return min(KT, n_win - (t - nt0) * KT);
        return min(KT, T - (t - nt0 - nt1) * KT);
    };

    // V task of this thread: key quad vq (keys 4 vq .. 4 vq + 3), 16-byte d-chunk vu
    const bool vtask = tid < 16 * TL::KCH;
    const int vq = tid & 15, vu = tid >> 4;
    // position of key 4 vq in the transposed tile (see the slot order above)
    const int vpos = 32 * (vq >> 3) + 8 * (vq & 3) + 4 * ((vq >> 2) & 1);

    uint4 kreg[TL::KLOADS];
    uint4 vreg[4];
    // global -> registers through buffer loads: one resource per segment and tensor, bounded
    // by the segment's valid rows, so rows past the end read as zero without a test; per tile
    // only the scalar offset changes.  Thread offsets: K chunk (row, u) of load i, V chunk vu
    // of rows 4 vq + j.
    const auto rk0 = rsrc(k0, (int64_t)n_sink * D * 2), rv0 = rsrc(v0, (int64_t)n_sink * D * 2);
    const auto rk1 = rsrc(k1, (int64_t)n_win * D * 2), rv1 = rsrc(v1, (int64_t)n_win * D * 2);
    const auto rk2 = rsrc(k2, T > 0 ? ((int64_t)(T - 1) * ks_chunk + D) * 2 : 0);
    const auto rv2 = rsrc(v2, T > 0 ? ((int64_t)(T - 1) * vs_chunk + D) * 2 : 0);
    int krow[TL::KLOADS], kcol[TL::KLOADS];
#pragma unroll
    for (int i = 0; i < TL::KLOADS; ++i) {
        const int idx = min(tid + NTHR * i, KT * TL::KCH - 1);
        krow[i] = idx / TL::KCH;
        kcol[i] = 16 * (idx % TL::KCH);
    }
    const int vcol = vtask ? 16 * vu : 0;
    auto fetch_rows = [&](__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int kstride, int vstride, int tt)
                          __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TL::KLOADS; ++i)
            kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rk, krow[i] * kstride + kcol[i], tt * KT * kstride, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            vreg[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rv, (4 * vq + j) * vstride + vcol, tt * KT * vstride, 0));
    };
    // tile t of the sequence sink, window, chunk
    auto fetch = [&](int t) __attribute__((always_inline)) {
        if (t < nt0)
            fetch_rows(rk0, rv0, 2 * D, 2 * D, t);
        else if (t < nt0 + nt1)
            fetch_rows(rk1, rv1, 2 * D, 2 * D, t - nt0);
        else
            fetch_rows(rk2, rv2, (int)(2 * ks_chunk), (int)(2 * vs_chunk), t - nt0 - nt1);
    };
    auto deposit = [&](int buf) __attribute__((always_inline)) {
        char* kb = lds + buf * TL::BUF;
#pragma unroll
        for (int i = 0; i < TL::KLOADS; ++i) {
            const int idx = tid + NTHR * i;
            if (idx < KT * TL::KCH) {
                const int row = idx / TL::KCH, u = idx % TL::KCH;
                *reinterpret_cast<uint4*>(kb + kmaj(row, u, TL::KBLK)) = kreg[i];
            }
        }
        if (vtask) {
            // keys 4 vq .. 4 vq + 3 sit at positions vpos .. vpos + 3 of a d row: chunk vpos / 8,
            // bytes 2 (vpos % 8) .. of it
            char* vb = kb + TL::K_BYTES + 2 * (vpos & 7);
            const int vj = vpos >> 3;
            const unsigned* w0 = reinterpret_cast<const unsigned*>(&vreg[0]);
            const unsigned* w1 = reinterpret_cast<const unsigned*>(&vreg[1]);
            const unsigned* w2 = reinterpret_cast<const unsigned*>(&vreg[2]);
            const unsigned* w3 = reinterpret_cast<const unsigned*>(&vreg[3]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // d = 8 vu + 2m (low halves) and 8 vu + 2m + 1 (high halves) of the four keys
                const uint2 lo = {(w0[m] & 0xffffu) | (w1[m] << 16), (w2[m] & 0xffffu) | (w3[m] << 16)};
                const uint2 hi = {(w0[m] >> 16) | (w1[m] & 0xffff0000u), (w2[m] >> 16) | (w3[m] & 0xffff0000u)};
                *reinterpret_cast<uint2*>(vb + kmaj(8 * vu + 2 * m, vj, 2048)) = lo;
                *reinterpret_cast<uint2*>(vb + kmaj(8 * vu + 2 * m + 1, vj, 2048)) = hi;
            }
        }
    };

    f32x4 o[TL::ND][QB];
    float m[QB], l[QB];
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -__builtin_inff();
        l[qb] = 0.f;
        for (int db = 0; db < TL::ND; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (ntiles > 0) {
        fetch(0);
        deposit(0);
    }
    // Four LDS buffers and one barrier per pair of tiles: tile t + 2 is fetched before tile t is
    // computed and deposited into buffer (t + 2) mod 4 right after it; that buffer was last read
    // before the previous barrier.
    if (ntiles > 1) {
        fetch(1);
        deposit(1);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();
    for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int t = t0 + half;
            if (t < ntiles) {
                if (t + 2 < ntiles) fetch(t + 2);
                const int cnt = tile_rows(t);
                const char* kb = lds + (t & 3) * TL::BUF;
                const char* vb = kb + TL::K_BYTES;

                // S^T = K Q^T: 4 key blocks x QB query blocks, d-steps outermost so that 4 * QB
                // independent accumulations separate the dependent ones
                f32x4 st[KT / 16][QB];
        #pragma unroll
                for (int kk = 0; kk < KT / 16; ++kk)
        #pragma unroll
                    for (int qb = 0; qb < QB; ++qb) st[kk][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        #pragma unroll
                for (int s = 0; s < TL::NS; ++s) {
                    bf16x8 a[KT / 16];
        #pragma unroll
                    for (int kk = 0; kk < KT / 16; ++kk)
                        a[kk] = *reinterpret_cast<const bf16x8*>(kb + kmaj(16 * kk + r, 4 * s + g, TL::KBLK));
        #pragma unroll
                    for (int kk = 0; kk < KT / 16; ++kk)
        #pragma unroll
                        for (int qb = 0; qb < QB; ++qb) st[kk][qb] = mma32(a[kk], qf[qb][s], st[kk][qb]);
                }
                if constexpr (TL::TAIL) {
                    bf16x4 a[KT / 16];
        #pragma unroll
                    for (int kk = 0; kk < KT / 16; ++kk)
                        a[kk] = *reinterpret_cast<const bf16x4*>(kb + kmaj(16 * kk + r, 4 * TL::NS + (g >> 1), TL::KBLK) +
                                                                 8 * (g & 1));
        #pragma unroll
                    for (int kk = 0; kk < KT / 16; ++kk)
        #pragma unroll
                        for (int qb = 0; qb < QB; ++qb) st[kk][qb] = mma16(a[kk], qt[qb], st[kk][qb]);
                }

                // online softmax (log2 domain) and P^T fragments.  Only a segment's last tile is
                // masked.  The reference maximum m of a query moves only when a tile's maximum exceeds
                // it by more than 8 (p then stays below 2^8, exact enough in fp32 and in bf16); the
                // rescale of O^T and l is skipped when no query of the wavefront needs it.
                if (cnt < KT) {
        #pragma unroll
                    for (int kk = 0; kk < KT / 16; ++kk)
        #pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (kk * 16 + 4 * g + i >= cnt)
        #pragma unroll
                                for (int qb = 0; qb < QB; ++qb) st[kk][qb][i] = -__builtin_inff();
                }
                bf16x8 pf[QB][KT / 32];
        #pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float mx = st[0][qb][0];
        #pragma unroll
                    for (int e = 1; e < 4 * (KT / 16); e += 2) {
                        const int e1 = e + 1 < 4 * (KT / 16) ? e + 1 : e;
                        mx = fmaxf(fmaxf(mx, st[e / 4][qb][e % 4]), st[e1 / 4][qb][e1 % 4]);
                    }
                    mx = max4q(mx);
                    const float ms = mx * scale_log2;
                    if (__any(ms > m[qb] + 8.0f)) {
                        const float mnew = fmaxf(m[qb], ms);
                        const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
                        m[qb] = mnew;
                        l[qb] *= alpha;
        #pragma unroll
                        for (int db = 0; db < TL::ND; ++db) o[db][qb] *= alpha;
                    }
                    const float nm = -m[qb];
                    float ls = 0.f;
                    float pv[KT / 16][4];
        #pragma unroll
                    for (int kk = 0; kk < KT / 16; ++kk)
        #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pv[kk][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kk][qb][i], scale_log2, nm));
                            ls += pv[kk][i];
                        }
                    l[qb] += ls;
        #pragma unroll
                    for (int c = 0; c < KT / 32; ++c)
                        pf[qb][c] = bf16x8{(bf16)pv[2 * c][0], (bf16)pv[2 * c][1], (bf16)pv[2 * c][2], (bf16)pv[2 * c][3],
                                           (bf16)pv[2 * c + 1][0], (bf16)pv[2 * c + 1][1], (bf16)pv[2 * c + 1][2],
                                           (bf16)pv[2 * c + 1][3]};
                }

                // O^T += V^T P^T, 32-key steps outermost (2 * ND * QB accumulations in between)
        #pragma unroll
                for (int c = 0; c < KT / 32; ++c)
        #pragma unroll
                    for (int db = 0; db < TL::ND; ++db) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + kmaj(db * 16 + r, 4 * c + g, 2048));
        #pragma unroll
                        for (int qb = 0; qb < QB; ++qb) o[db][qb] = mma32(a, pf[qb][c], o[db][qb]);
                    }
                if (t + 2 < ntiles) deposit((t + 2) & 3);
            }
        }
        __syncthreads();
    }

    // o = O^T / l, rows of the chunk only
    bf16* obase = static_cast<bf16*>(p.o) + b * p.os[0] + h * p.os[2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = sum4q(l[qb]);
        const float inv = 1.0f / lt;
        const int64_t t = q0 + 16 * qb + r;
        if (t < T) {
            bf16* row = obase + t * p.os[1];
#pragma unroll
            for (int db = 0; db < TL::ND; ++db) {
                const bf16x4 x = {(bf16)(o[db][qb][0] * inv), (bf16)(o[db][qb][1] * inv),
                                  (bf16)(o[db][qb][2] * inv), (bf16)(o[db][qb][3] * inv)};
                *reinterpret_cast<uint2*>(row + 16 * db + 4 * g) = __builtin_bit_cast(uint2, x);
            }
        }
    }
}

// Copies the chunk's k, v rows into the cache: token i < taken fills sink slot sink_fill + i;
// the rest go to the window ring (slot (win_base + j) mod win_cap), where the first `skip`
// of them are already older than the window and are not written.  One thread per 16-byte
// chunk of a k or v row; items ordered (token, stream, head, k/v, chunk).
template <int D>
__global__ __launch_bounds__(256) void attn_append_kernel(AppendParams p) {
    constexpr int KCH = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)p.T * p.B * p.H * 2 * KCH) return;
    const int c = (int)(gid % (2 * KCH));
    int64_t rest = gid / (2 * KCH);
    const int h = (int)(rest % p.H);
    rest /= p.H;
    const int b = (int)(rest % p.B);
    const int i = (int)(rest / p.B);
    const int64_t bh = (int64_t)b * p.H + h;
    const bool isv = c >= KCH;
    const int u = isv ? c - KCH : c;
    int64_t slot;
    bf16* dst;
    if (i < p.taken) {
        slot = bh * p.sink_cap + p.sink_fill + i;
        dst = static_cast<bf16*>(isv ? p.v_sink : p.k_sink);
    } else {
        const int j = i - p.taken;
        if (j < p.skip) return;
        slot = bh * p.win_cap + (int)(((int64_t)p.win_base + j) % p.win_cap);
        dst = static_cast<bf16*>(isv ? p.v_win : p.k_win);
    }
    const bf16* src = isv ? static_cast<const bf16*>(p.v) + b * p.vs[0] + (int64_t)i * p.vs[1] + h * p.vs[2]
                          : static_cast<const bf16*>(p.k) + b * p.ks[0] + (int64_t)i * p.ks[1] + h * p.ks[2];
    *reinterpret_cast<uint4*>(dst + slot * D + 8 * u) = gload16(src + 8 * u);
}

template <int D>
hipError_t launch_attn_d(const AttnParams& p, hipStream_t s) {
    const int64_t nwg = (int64_t)((p.T + QT - 1) / QT) * p.H * p.B;
    if (nwg >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_kernel<D>, dim3((unsigned)nwg), dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_append_d(const AppendParams& p, hipStream_t s) {
    const int64_t n = (int64_t)p.T * p.B * p.H * 2 * (D / 8);
    if ((n + 255) / 256 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_append_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool attn_dim_supported(int d) { return d == 64 || d == 112 || d == 128; }

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
    switch (p.D) {
        case 64: return launch_attn_d<64>(p, s);
        case 112: return launch_attn_d<112>(p, s);
        case 128: return launch_attn_d<128>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_append(const AppendParams& p, hipStream_t s) {
    switch (p.D) {
        case 64: return launch_append_d<64>(p, s);
        case 112: return launch_append_d<112>(p, s);
        case 128: return launch_append_d<128>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
