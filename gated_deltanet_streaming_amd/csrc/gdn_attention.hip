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
// values stream through LDS in tiles of KT keys (double-buffered, one barrier per tile), tile
// after tile over the three segments (sink, window, chunk); a segment's last tile is masked.
// Products run on 16x16x32 bf16 MFMAs in transposed form:
//
//     S^T = K Q^T      (A = K rows from LDS, B = Q fragments in registers)
//     O^T += V^T P^T   (A = V^T rows from LDS, B = P^T built from S^T in registers)
//
// The output tile of S^T (lane l: query l % 16, keys 4g..4g+3, g = l / 16) is the B operand
// of the second product once its key index becomes the contraction index: slot i of group g
// in a 32-key step c stands for key 32c + 4g + i (i < 4) or 32c + 16 + 4g + (i - 4) (i >= 4).
// V is written to LDS transposed, in exactly that key order, so that each A operand is one
// 16-byte LDS read.  The softmax is online in the log2 domain (running maximum m and partial
// sum l per lane; O^T rescaled by 2^(m_old - m_new) when the maximum grows); p enters the
// second product rounded to bf16, l sums the fp32 values.
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
constexpr int NWAVE = 4;               // wavefronts per workgroup
constexpr int NTHR = NWAVE * 64;
constexpr int QT = NWAVE * QB * 16;    // queries per workgroup
constexpr int VT_STRIDE = KT * 2 + 16; // bytes per d-row of the transposed V tile

template <int D>
struct Tile {
    static constexpr int KS = (D * 2) % 128 == 0 ? D * 2 + 16 : D * 2;  // bytes per K row
    static constexpr int K_BYTES = KT * KS;
    static constexpr int V_BYTES = D * VT_STRIDE;
    static constexpr int BUF = K_BYTES + V_BYTES;
    static constexpr int NS = D / 32;             // full 32-wide steps over d
    static constexpr bool TAIL = (D % 32) != 0;   // plus one 16-wide step
    static constexpr int ND = D / 16;             // 16-row blocks of d in O^T
    static constexpr int KCH = D / 8;             // 16-byte chunks per row
    static constexpr int KLOADS = (KT * KCH + NTHR - 1) / NTHR;
    static_assert(16 * KCH <= NTHR, "one V task per thread");
};

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A 16-wide step as a 32-wide MFMA with zero upper slots in both operands.
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16 z = (bf16)0.f;
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8{a[0], a[1], a[2], a[3], z, z, z, z},
                                                   bf16x8{b[0], b[1], b[2], b[3], z, z, z, z}, c, 0, 0, 0);
}

struct Seg {
    const bf16* k;
    const bf16* v;
    int64_t ks, vs;  // token strides, elements
    int n;           // tokens
    int nt;          // tiles
};

template <int D>
__global__ __launch_bounds__(NTHR, 2) void attn_kernel(AttnParams p) {
    using TL = Tile<D>;
    __shared__ __align__(16) char lds[2 * TL::BUF];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t bh = (int64_t)b * p.H + h;
    const int64_t q0 = (int64_t)blockIdx.x * QT + wave * (QB * 16);

    // Q fragments: lane holds query q0 + 16 qb + r, d = 32 s + 8 g .. +7 (tail: d = 32 NS + 4 g .. +3)
    bf16x8 qf[QB][TL::NS > 0 ? TL::NS : 1];
    bf16x4 qt[QB];
    {
        const bf16* qbase = static_cast<const bf16*>(p.q) + b * p.qs[0] + h * p.qs[2];
        for (int qb = 0; qb < QB; ++qb) {
            const int64_t t = q0 + 16 * qb + r;
            const bool in = t < p.T;
            const bf16* row = qbase + (in ? t : 0) * p.qs[1];
#pragma unroll
            for (int s = 0; s < TL::NS; ++s) {
                uint4 x = in ? *reinterpret_cast<const uint4*>(row + 32 * s + 8 * g) : uint4{0, 0, 0, 0};
                qf[qb][s] = __builtin_bit_cast(bf16x8, x);
            }
            if constexpr (TL::TAIL) {
                uint2 x = in ? *reinterpret_cast<const uint2*>(row + 32 * TL::NS + 4 * g) : uint2{0, 0};
                qt[qb] = __builtin_bit_cast(bf16x4, x);
            }
        }
    }

    Seg seg[3];
    seg[0] = Seg{static_cast<const bf16*>(p.k_sink) + bh * p.sink_cap * D,
                 static_cast<const bf16*>(p.v_sink) + bh * p.sink_cap * D, D, D, p.n_sink, 0};
    seg[1] = Seg{static_cast<const bf16*>(p.k_win) + bh * p.win_cap * D,
                 static_cast<const bf16*>(p.v_win) + bh * p.win_cap * D, D, D, p.n_win, 0};
    seg[2] = Seg{static_cast<const bf16*>(p.k) + b * p.ks[0] + h * p.ks[2],
                 static_cast<const bf16*>(p.v) + b * p.vs[0] + h * p.vs[2], p.ks[1], p.vs[1], p.T, 0};
    for (int i = 0; i < 3; ++i) seg[i].nt = (seg[i].n + KT - 1) / KT;
    const int ntiles = seg[0].nt + seg[1].nt + seg[2].nt;

    // tile t -> its rows: key pointer, value pointer, strides, valid rows
    auto locate = [&](int t, const bf16*& kp, const bf16*& vp, int64_t& ks, int64_t& vs, int& cnt) {
        int i = 0;
        if (t >= seg[0].nt) { t -= seg[0].nt; i = 1; }
        if (i == 1 && t >= seg[1].nt) { t -= seg[1].nt; i = 2; }
        const Seg& sg = seg[i];
        kp = sg.k + (int64_t)t * KT * sg.ks;
        vp = sg.v + (int64_t)t * KT * sg.vs;
        ks = sg.ks;
        vs = sg.vs;
        cnt = min(KT, sg.n - t * KT);
    };

    // V task of this thread: key quad vq (keys 4 vq .. 4 vq + 3), 16-byte d-chunk vu
    const bool vtask = tid < 16 * TL::KCH;
    const int vq = tid & 15, vu = tid >> 4;
    // position of key 4 vq in the transposed tile (see the slot order above)
    const int vpos = 32 * (vq >> 3) + 8 * (vq & 3) + 4 * ((vq >> 2) & 1);

    uint4 kreg[TL::KLOADS];
    uint4 vreg[4];
    auto fetch = [&](int t) {
        const bf16 *kp, *vp;
        int64_t ks, vs;
        int cnt;
        locate(t, kp, vp, ks, vs, cnt);
#pragma unroll
        for (int i = 0; i < TL::KLOADS; ++i) {
            const int idx = tid + NTHR * i;
            const int row = idx / TL::KCH, u = idx % TL::KCH;
            kreg[i] = (idx < KT * TL::KCH && row < cnt) ? *reinterpret_cast<const uint4*>(kp + row * ks + 8 * u)
                                                        : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * vq + j;
            vreg[j] = (vtask && row < cnt) ? *reinterpret_cast<const uint4*>(vp + row * vs + 8 * vu)
                                           : uint4{0, 0, 0, 0};
        }
    };
    auto deposit = [&](int buf) {
        char* kb = lds + buf * TL::BUF;
#pragma unroll
        for (int i = 0; i < TL::KLOADS; ++i) {
            const int idx = tid + NTHR * i;
            if (idx < KT * TL::KCH) {
                const int row = idx / TL::KCH, u = idx % TL::KCH;
                *reinterpret_cast<uint4*>(kb + row * TL::KS + 16 * u) = kreg[i];
            }
        }
        if (vtask) {
            char* vb = kb + TL::K_BYTES + vpos * 2;
            const unsigned* w0 = reinterpret_cast<const unsigned*>(&vreg[0]);
            const unsigned* w1 = reinterpret_cast<const unsigned*>(&vreg[1]);
            const unsigned* w2 = reinterpret_cast<const unsigned*>(&vreg[2]);
            const unsigned* w3 = reinterpret_cast<const unsigned*>(&vreg[3]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // d = 8 vu + 2m (low halves) and 8 vu + 2m + 1 (high halves) of the four keys
                const uint2 lo = {(w0[m] & 0xffffu) | (w1[m] << 16), (w2[m] & 0xffffu) | (w3[m] << 16)};
                const uint2 hi = {(w0[m] >> 16) | (w1[m] & 0xffff0000u), (w2[m] >> 16) | (w3[m] & 0xffff0000u)};
                *reinterpret_cast<uint2*>(vb + (8 * vu + 2 * m) * VT_STRIDE) = lo;
                *reinterpret_cast<uint2*>(vb + (8 * vu + 2 * m + 1) * VT_STRIDE) = hi;
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
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) fetch(t + 1);
        int cnt;
        {
            const bf16 *kp, *vp;
            int64_t ks, vs;
            locate(t, kp, vp, ks, vs, cnt);
        }
        const char* kb = lds + buf * TL::BUF;
        const char* vb = kb + TL::K_BYTES;

        // S^T = K Q^T: 4 key blocks x QB query blocks
        f32x4 st[KT / 16][QB];
#pragma unroll
        for (int kk = 0; kk < KT / 16; ++kk) {
            for (int qb = 0; qb < QB; ++qb) st[kk][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const char* krow = kb + (kk * 16 + r) * TL::KS;
#pragma unroll
            for (int s = 0; s < TL::NS; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 64 * s + 16 * g);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) st[kk][qb] = mma32(a, qf[qb][s], st[kk][qb]);
            }
            if constexpr (TL::TAIL) {
                const bf16x4 a = *reinterpret_cast<const bf16x4*>(krow + 64 * TL::NS + 8 * g);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) st[kk][qb] = mma16(a, qt[qb], st[kk][qb]);
            }
        }

        // online softmax (log2 domain) and P^T fragments
        bf16x8 pf[QB][KT / 32];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kk = 0; kk < KT / 16; ++kk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = kk * 16 + 4 * g + i < cnt;
                    st[kk][qb][i] = valid ? st[kk][qb][i] * p.scale_log2 : -__builtin_inff();
                    mx = fmaxf(mx, st[kk][qb][i]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[qb], mx);
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
            m[qb] = mnew;
            float ls = 0.f;
            float pv[KT / 16][4];
#pragma unroll
            for (int kk = 0; kk < KT / 16; ++kk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[kk][i] = __builtin_amdgcn_exp2f(st[kk][qb][i] - mnew);
                    ls += pv[kk][i];
                }
            l[qb] = l[qb] * alpha + ls;
#pragma unroll
            for (int db = 0; db < TL::ND; ++db) o[db][qb] *= alpha;
#pragma unroll
            for (int c = 0; c < KT / 32; ++c)
                pf[qb][c] = bf16x8{(bf16)pv[2 * c][0], (bf16)pv[2 * c][1], (bf16)pv[2 * c][2], (bf16)pv[2 * c][3],
                                   (bf16)pv[2 * c + 1][0], (bf16)pv[2 * c + 1][1], (bf16)pv[2 * c + 1][2],
                                   (bf16)pv[2 * c + 1][3]};
        }

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < TL::ND; ++db) {
            const char* vrow = vb + (db * 16 + r) * VT_STRIDE;
#pragma unroll
            for (int c = 0; c < KT / 32; ++c) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 64 * c + 16 * g);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[db][qb] = mma32(a, pf[qb][c], o[db][qb]);
            }
        }

        if (t + 1 < ntiles) deposit(buf ^ 1);
        __syncthreads();
    }

    // o = O^T / l, rows of the chunk only
    bf16* obase = static_cast<bf16*>(p.o) + b * p.os[0] + h * p.os[2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float lt = l[qb];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const float inv = 1.0f / lt;
        const int64_t t = q0 + 16 * qb + r;
        if (t < p.T) {
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
// of them are already older than the window and are not written.  One 64-lane workgroup per
// (token, head, stream).
template <int D>
__global__ __launch_bounds__(64) void attn_append_kernel(AppendParams p) {
    constexpr int KCH = D / 8;
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int64_t bh = (int64_t)b * p.H + h;
    bf16 *kd, *vd;
    if (i < p.taken) {
        const int64_t slot = bh * p.sink_cap + p.sink_fill + i;
        kd = static_cast<bf16*>(p.k_sink) + slot * D;
        vd = static_cast<bf16*>(p.v_sink) + slot * D;
    } else {
        const int j = i - p.taken;
        if (j < p.skip) return;
        const int64_t slot = bh * p.win_cap + (int)(((int64_t)p.win_base + j) % p.win_cap);
        kd = static_cast<bf16*>(p.k_win) + slot * D;
        vd = static_cast<bf16*>(p.v_win) + slot * D;
    }
    if (lane < KCH) {
        const bf16* ks = static_cast<const bf16*>(p.k) + b * p.ks[0] + (int64_t)i * p.ks[1] + h * p.ks[2];
        *reinterpret_cast<uint4*>(kd + 8 * lane) = *reinterpret_cast<const uint4*>(ks + 8 * lane);
    } else if (lane < 2 * KCH) {
        const int u = lane - KCH;
        const bf16* vs = static_cast<const bf16*>(p.v) + b * p.vs[0] + (int64_t)i * p.vs[1] + h * p.vs[2];
        *reinterpret_cast<uint4*>(vd + 8 * u) = *reinterpret_cast<const uint4*>(vs + 8 * u);
    }
}

template <int D>
hipError_t launch_attn_d(const AttnParams& p, hipStream_t s) {
    dim3 grid((unsigned)((p.T + QT - 1) / QT), (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL(attn_kernel<D>, grid, dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_append_d(const AppendParams& p, hipStream_t s) {
    dim3 grid((unsigned)p.T, (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL(attn_append_kernel<D>, grid, dim3(64), 0, s, p);
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
