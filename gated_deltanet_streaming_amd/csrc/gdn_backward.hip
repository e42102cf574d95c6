// Gradient of one scan of the gated delta rule on gfx950: a token-sequential fp32 path
// behind gdn_chunk_backward.  Part of libgdn_stream.so (the forward kernels live in
// gdn_kernels.hip).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {

namespace {

typedef __bf16 bf16;

// element idx of a q/k/v/d_o tensor in the call's io dtype, as fp32
template <bool F32>
__device__ __forceinline__ float ld_elem(const void* base, int64_t idx) {
    if constexpr (F32) return reinterpret_cast<const float*>(base)[idx];
    else return (float)reinterpret_cast<const bf16*>(base)[idx];
}

// lane data movement within rows of 16 lanes (DPP; every source lane is valid for these controls)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

void tm_begin(Timing* tm, hipStream_t s, int kind) {
    if (tm && tm->ev && tm->n < tm->cap) {
        (void)hipEventRecord(tm->ev[2 * tm->n], s);
        tm->kinds[tm->n] = kind;
    }
}
void tm_end(Timing* tm, hipStream_t s) {
    if (tm && tm->ev && tm->n < tm->cap) {
        (void)hipEventRecord(tm->ev[2 * tm->n + 1], s);
        ++tm->n;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Gradient of one scan (reverse-mode through the per-token rule), fp32 and
// token-sequential: a reference-grade path for training over streaming chunks.
// With G = dL/dS, walking the tokens backward (q_t, k_t normalised):
//     G += scale do_t q_t^T,  x = S_{t-1} k_t,  gk = G k_t
//     dv_t = beta_t gk,  da_t = <G, S_{t-1}> - beta_t gk.x,  dbeta_t = gk.(v_t - a_t x)
//     dk_t = beta_t G^T (v_t - a_t x) - a_t beta_t S_{t-1}^T gk,  dq_t = scale S_t^T do_t
//     G <- a_t (G - beta_t gk k_t^T)
// gdn_bwd_rows_kernel: one 64-lane workgroup per (b, h, block of 4 state rows);
// lane l owns row 4 rb + l/16 and the column 16 j + l%16 of every 16-column
// group j.  Tokens are staged through LDS in
// blocks of TB (k and q normalised once per block; a block's global loads go out
// three blocks before it is worked on, into a ring of register sets).  A forward
// pass keeps only the state before every block (a checkpoint) and an adjoint pass
// keeps G at the end of every segment of kSEG tokens; each segment is then walked
// backward on its own, recomputing the states inside each of its blocks from the
// block's checkpoint into LDS, half a block at a time.  dv and the start-state
// gradient are row-local;
// the other gradients sum over all rows: per token the rows' terms go through an
// LDS buffer and each lane adds one float4 column group over the 4 rows in row
// order, then the workgroup writes its rows' partial sums, and gdn_bwd_reduce_kernel
// adds the row blocks in a fixed order and maps the normalised-vector gradients
// back through the L2 normalisation.
// ---------------------------------------------------------------------------
constexpr int kMinTB = 8;    // smallest token block of any instance (sizes the checkpoints)
constexpr int kRB = 4;       // state rows per workgroup
constexpr int kLPR = 64 / kRB;   // lanes per state row

constexpr int kSEG = 64;     // tokens per walk segment (a multiple of every token block)

int64_t backward_ckpt_per(int64_t max_tokens) { return (max_tokens + kMinTB - 1) / kMinTB + 1; }
int64_t backward_gck_per(int64_t max_tokens) { return (max_tokens + kSEG - 1) / kSEG; }

// floats of the state checkpoints
int64_t backward_state_ckpt_floats(int B, int H, int Dk, int Dv, int64_t max_tokens) {
    return (int64_t)B * H * (Dv / kRB) * backward_ckpt_per(max_tokens) * kRB * Dk;
}
// floats of the state checkpoints, then of the adjoint checkpoints (the partial sums follow)
int64_t backward_ckpt_floats(int B, int H, int Dk, int Dv, int64_t max_tokens) {
    return (int64_t)B * H * (Dv / kRB) * (backward_ckpt_per(max_tokens) + backward_gck_per(max_tokens)) * kRB * Dk;
}

int64_t backward_ws_bytes(int B, int H, int Dk, int Dv, int64_t max_tokens) {
    const int64_t nrb = Dv / kRB;
    int64_t states = 0, partials = 0, total = 0;
    if (__builtin_mul_overflow((int64_t)B * H, nrb * kRB * Dk, &states) ||
        __builtin_mul_overflow(states, backward_ckpt_per(max_tokens) + backward_gck_per(max_tokens), &states) ||
        __builtin_mul_overflow((int64_t)B * H, nrb * (2 * Dk + 4), &partials) ||
        __builtin_mul_overflow(partials, max_tokens, &partials) || __builtin_add_overflow(states, partials, &total) ||
        __builtin_mul_overflow(total, (int64_t)4, &total))
        return -1;
    return total;
}

namespace {

// sum over the 16 lanes of one state row (lane bits 0..3): quad permutations [1,0,3,2] and
// [2,3,0,1], then the mirror within each 8-lane half row, then the mirror of the whole row
__device__ __forceinline__ float sum16(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);   // row_half_mirror
    x += dpp<0x140>(x);   // row_mirror
    return x;
}
// sum over the 4 rows of the workgroup (lane bits 4..5): across the four DPP rows with lane swaps
__device__ __forceinline__ float sum_rows(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(x);
    const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

// raw buffer resource over [base, base + bytes); loads beyond it return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Orders LDS accesses of the (single) wavefront around this point in the compiled code: lanes read
// what other lanes wrote before it, and the LDS performs one wavefront's operations in order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

}  // namespace

// Two launches per gradient.  Phase 0: per (b, h, row block) one workgroup runs the forward
// recurrence and stores the state before every token block, and another runs the adjoint
// recurrence alone (it does not involve the state: G <- a (G + scale do q^T)(I - beta k k^T)) and
// stores dL/dS at the end of every segment of kSEG tokens.  Phase 1: per (b, h, row block,
// segment) one workgroup walks the segment's tokens backward from its adjoint checkpoint,
// recomputing each block's states from its state checkpoint; the segments are independent.  The
// adjoint pass and the walks perform the same operations on G in the same order.
// Workgroups [0, nunits) work on g0's scan, [nunits, 2 nunits) on g1's (the bidirectional call).
// The phases are separate instances: phase 0 uses neither the block-state nor the column-sum
// buffer, and with them gone (and phase 1's registers) more of its workgroups share a CU: with bf16
// I/O its registers fit three wavefronts per SIMD, so that the 2 x 2 x (d_v / 4) x H workgroups of a
// bidirectional call run in one round (fp32 I/O stages twice the bytes and would spill).
template <int NG, bool F32, int PHASE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(PHASE == 0 && !F32 ? 3 : 1))) void gdn_bwd_rows_kernel(Params p, BwdParams g0, BwdParams g1, int nunits) {
    constexpr int DK = 16 * NG;               // d_k
    constexpr int TB = 8;                     // tokens per staged block
    static_assert(TB >= kMinTB, "checkpoint sizing");
    const int lane = threadIdx.x, part = lane & (kLPR - 1), rl = lane / kLPR;
    const int nrb = p.Dv / kRB;
    const int nwg = p.B * p.H * nrb;
    const bool second = (int)blockIdx.x >= nunits;
    const BwdParams g = second ? g1 : g0;
    int id = (int)blockIdx.x - (second ? nunits : 0);
    const int unit = id / nwg;   // phase 0: 0 state checkpoints, 1 adjoint checkpoints; phase 1: the segment
    id -= unit * nwg;
    const int rb = id % nrb;
    id /= nrb;
    const int h = id % p.H;
    id /= p.H;
    const int b = id;
    const int row = kRB * rb + rl;
    const int T = (int)p.T;
    const int nblk = (T + TB - 1) / TB;
    const int wid = 2 * DK + 4;

    constexpr int SH = TB / 2;                         // tokens whose states LDS holds at once (phase 1)
    __shared__ __align__(16) float sst[SH][NG][64];    // S_{t-1} of half a block's tokens, lane-major
    __shared__ __align__(16) float skn[TB][DK];        // normalised k of the block's tokens
    __shared__ __align__(16) float sqn[TB][DK];        // normalised q
    __shared__ __align__(16) float scol[2][kRB][DK];   // per-row terms of dq and dk of one token
    __shared__ __align__(16) float sv[TB][kRB], sdo[TB][kRB];
    __shared__ float sx[SH][kRB], sa[TB], sb[TB];

    float* ck = g.states + (((int64_t)b * p.H + h) * nrb + rb) * g.ck_per * kRB * DK;
    float* gk0 = g.gck + (((int64_t)b * p.H + h) * nrb + rb) * g.gck_per * kRB * DK;
    constexpr int BPS = kSEG / TB;   // token blocks per segment
    static_assert(kSEG % TB == 0, "segments of whole blocks");
    auto tok = [&](int pi) { return g.reverse ? T - 1 - pi : pi; };

    // ---- staging: raw loads of a block into registers, then fp32 (normalised) into LDS ----
    // Rows are read in 16-byte chunks through buffer resources over the (b, h) rows; chunks of
    // tokens past the block or past T use an offset beyond the resource and read as zero.
    constexpr int ESZ = F32 ? 4 : 2, EPC = 16 / ESZ;   // bytes per element, elements per chunk
    constexpr int CPR = DK / EPC, NCH = TB * CPR;        // chunks per k/q row, per block
    constexpr int NLC = (NCH + 63) / 64;                 // k (q) chunks per lane
    static_assert(TB <= 64 && kRB == 4, "lane ti < TB loads token ti's 4 v (d_o) values");
    const char* kb = static_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)h * p.ks[2]) * ESZ;
    const char* qb = static_cast<const char*>(p.q) + ((int64_t)b * p.qs[0] + (int64_t)h * p.qs[2]) * ESZ;
    const char* vb = static_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)h * p.vs[2] + kRB * rb) * ESZ;
    const char* ob = static_cast<const char*>(g.d_o) + ((int64_t)b * p.os[0] + (int64_t)h * p.os[2] + kRB * rb) * ESZ;
    const auto krs = make_rsrc(kb, ((int64_t)(T - 1) * p.ks[1] + DK) * ESZ);
    const auto qrs = make_rsrc(qb, ((int64_t)(T - 1) * p.qs[1] + DK) * ESZ);
    const auto vrs = make_rsrc(vb, ((int64_t)(T - 1) * p.vs[1] + kRB) * ESZ);
    const auto ors = make_rsrc(ob, ((int64_t)(T - 1) * p.os[1] + kRB) * ESZ);
    const int ksb = (int)(p.ks[1] * ESZ), qsb = (int)(p.qs[1] * ESZ), vsb = (int)(p.vs[1] * ESZ), osb = (int)(p.os[1] * ESZ);
    constexpr int OUT = (int)0x80000000;   // beyond every resource
    // one block's raw loads (a register set of the staging ring)
    struct Staged {
        uint4 rk[NLC], rq[NLC], rv, rdo;
        float ra, rbt;
        float ck[NG];   // the block's state checkpoint (walk only)
    };
    auto load_block = [&](Staged& st, int blk, bool with_q, bool with_ck) {
        const int pi0 = blk * TB;
        if (with_ck) {
#pragma unroll
            for (int j = 0; j < NG; ++j) st.ck[j] = ck[((int64_t)blk * kRB + rl) * DK + 16 * j + part];
        }
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
            const int e = lane + 64 * i, ti = e / CPR, c = e - ti * CPR;
            const bool ok = e < NCH && pi0 + ti < T;
            const int t = ok ? tok(pi0 + ti) : 0;
            st.rk[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, ok ? t * ksb + 16 * c : OUT, 0, 0));
            if (with_q)
                st.rq[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qrs, ok ? t * qsb + 16 * c : OUT, 0, 0));
        }
        {
            // token ti = lane: its 4 v (d_o) values, 16 bytes (fp32) or 8 bytes as two dwords (bf16)
            const bool ok = lane < TB && pi0 + lane < T;
            const int t = ok ? tok(pi0 + lane) : 0;
            const int vo = ok ? t * vsb : OUT, oo = ok ? t * osb : OUT;
            if constexpr (F32) {
                st.rv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vo, 0, 0));
                if (with_q) st.rdo = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ors, oo, 0, 0));
            } else {
                st.rv.x = __builtin_amdgcn_raw_buffer_load_b32(vrs, vo, 0, 0);
                st.rv.y = __builtin_amdgcn_raw_buffer_load_b32(vrs, ok ? vo + 4 : OUT, 0, 0);
                if (with_q) {
                    st.rdo.x = __builtin_amdgcn_raw_buffer_load_b32(ors, oo, 0, 0);
                    st.rdo.y = __builtin_amdgcn_raw_buffer_load_b32(ors, ok ? oo + 4 : OUT, 0, 0);
                }
            }
        }
        // gates of tokens past T: a = 1 (log a = 0), beta = 0; a given as log a is exponentiated
        // when the block is staged, so that no arithmetic waits for these loads here
        st.ra = p.gate_log ? 0.f : 1.f;
        st.rbt = 0.f;
        if (lane < TB && pi0 + lane < T) {
            const int64_t t = tok(pi0 + lane);
            const int64_t gq = (int64_t)b * p.gs[0] + t * p.gs[1] + (int64_t)h * p.gs[2];
            st.ra = p.a[gq];
            st.rbt = p.beta[gq];
        }
    };
    // a 16-byte chunk of EPC elements as fp32, to dst (16-byte aligned)
    auto put_chunk = [&](float* dst, const uint4& raw) {
        if constexpr (F32) {
            *reinterpret_cast<float4*>(dst) = __builtin_bit_cast(float4, raw);
        } else {
            const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
                *reinterpret_cast<float4*>(dst + 4 * k2) =
                    float4{__uint_as_float(w[2 * k2] << 16), __uint_as_float(w[2 * k2] & 0xffff0000u),
                           __uint_as_float(w[2 * k2 + 1] << 16), __uint_as_float(w[2 * k2 + 1] & 0xffff0000u)};
        }
    };
    // a token's 4 v (d_o) values as fp32 (fp32: the 16 bytes as loaded; bf16: the two dwords)
    auto put4 = [&](float* dst, const uint4& raw) {
        if constexpr (F32) *reinterpret_cast<float4*>(dst) = __builtin_bit_cast(float4, raw);
        else
            *reinterpret_cast<float4*>(dst) = float4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                                                     __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
    };
    auto store_block = [&](const Staged& st, bool with_q) {
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
            const int e = lane + 64 * i, ti = e / CPR, c = e - ti * CPR;
            if (e < NCH) {
                put_chunk(&skn[ti][EPC * c], st.rk[i]);
                if (with_q) put_chunk(&sqn[ti][EPC * c], st.rq[i]);
            }
        }
        if (lane < TB) {
            put4(&sv[lane][0], st.rv);
            if (with_q) put4(&sdo[lane][0], st.rdo);
        }
        if (lane < TB) {
            sa[lane] = p.gate_log ? expf(st.ra) : st.ra;
            sb[lane] = st.rbt;
        }
        lds_order();
        // normalise the rows in place: lane 4 r + u (r < 2 TB = 16) holds quarter u of row r of k
        // (r < TB) or of q (row r - TB): its DK/4 values are read at once, summed, combined over the
        // lane quad, scaled and written back (one LDS round trip per block)
        static_assert(2 * TB * 4 == 64, "four lanes per staged k or q row");
        if (p.l2norm) {
            const int r = lane >> 2, u = lane & 3;
            const bool isq = r >= TB;
            float* rowp = (isq ? &sqn[0][0] : &skn[0][0]) + (isq ? r - TB : r) * DK + u * (DK / 4);
            const bool act = with_q || !isq;
            float4 xs[DK / 16];
            float ss = 0.f;
            if (act) {
#pragma unroll
                for (int c = 0; c < DK / 16; ++c) xs[c] = *reinterpret_cast<const float4*>(rowp + 4 * c);
#pragma unroll
                for (int c = 0; c < DK / 16; ++c) ss += dot4(xs[c], xs[c]);
            }
            ss += dpp<0xB1>(ss);   // quad permutations [1,0,3,2] and [2,3,0,1]
            ss += dpp<0x4E>(ss);
            // rows past the end of the sequence are zero and stay zero
            const float sc = ss + p.eps > 0.f ? 1.f / sqrtf(ss + p.eps) : 0.f;
            if (act) {
#pragma unroll
                for (int c = 0; c < DK / 16; ++c) {
                    float4 x = xs[c];
                    x.x *= sc; x.y *= sc; x.z *= sc; x.w *= sc;
                    *reinterpret_cast<float4*>(rowp + 4 * c) = x;
                }
            }
        }
        lds_order();
    };
    // blocks first, first + dirn, ... (count of them) in turn: each is staged into LDS and handed to
    // body; its loads were issued three blocks earlier, in a ring of three register sets
    // (with_ck: the block's state checkpoint is loaded with it and handed to body in registers)
    auto run_blocks = [&](int first, int count, int dirn, bool with_q, bool with_ck, auto&& body)
                          __attribute__((always_inline)) {
        Staged s0, s1, s2;
        load_block(s0, first, with_q, with_ck);
        if (count > 1) load_block(s1, first + dirn, with_q, with_ck);
        if (count > 2) load_block(s2, first + 2 * dirn, with_q, with_ck);
        auto one = [&](Staged& st, int i) __attribute__((always_inline)) {
            store_block(st, with_q);
            float ckv[NG];
#pragma unroll
            for (int j = 0; j < NG; ++j) ckv[j] = with_ck ? st.ck[j] : 0.f;
            if (i + 3 < count) load_block(st, first + (i + 3) * dirn, with_q, with_ck);
            body(first + i * dirn, ckv);
        };
        for (int i = 0; i < count; i += 3) {
            one(s0, i);
            if (i + 1 < count) one(s1, i + 1);
            if (i + 2 < count) one(s2, i + 2);
        }
    };
    // column of this lane in staged row r: 16 j + part
    auto krow = [&](int r, int j) { return skn[r][16 * j + part]; };
    auto qrow = [&](int r, int j) { return sqn[r][16 * j + part]; };
    auto ckp = [&](int blk, int j) { return ck + ((int64_t)blk * kRB + rl) * DK + 16 * j + part; };
    auto gckp = [&](int seg, int j) { return gk0 + ((int64_t)seg * kRB + rl) * DK + 16 * j + part; };
    // a dot product over the lane's NG columns in two independent chains, then over the row's lanes
    auto rowdot = [&](const float* a, const float* c) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (j & 1) s1 += a[j] * c[j];
            else s0 += a[j] * c[j];
        }
        return sum16(s0 + s1);
    };

    // one token of the forward recurrence on S (row dot and update); returns x = S k
    float S[NG];
    auto fwd_step = [&](const float* kr, float at, float bt, float vr) __attribute__((always_inline)) {
        const float x = rowdot(S, kr);
        // a (S - beta x k^T) + beta v k^T = a S + beta (v - a x) k^T: a multiply and an FMA per column
        const float d = bt * (vr - at * x);
#pragma unroll
        for (int j = 0; j < NG; ++j) S[j] = fmaf(d, kr[j], at * S[j]);
        return x;
    };
    auto fwd_token = [&](int r) {
        float kr[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) kr[j] = krow(r, j);
        return fwd_step(kr, sa[r], sb[r], sv[r][rl]);
    };
    // one token of the adjoint recurrence: G <- a (G + scale do q^T)(I - beta k k^T)
    float G[NG];
    auto adj_step = [&](const float* kr, const float* qr, float dor, float at, float bt) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NG; ++j) G[j] += dor * qr[j];
        const float gk = rowdot(G, kr);
        const float cg = bt * gk;
#pragma unroll
        for (int j = 0; j < NG; ++j) G[j] = at * (G[j] - cg * kr[j]);
    };

    if constexpr (PHASE == 0) {
    if (unit == 0) {
        // ---- forward: checkpoints before every block ----
#pragma unroll
        for (int j = 0; j < NG; ++j)
            S[j] = g.state0 ? g.state0[(((int64_t)b * p.H + h) * p.Dv + row) * DK + 16 * j + part] : 0.f;
        run_blocks(0, nblk, 1, false, false, [&](int blk, const float*) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NG; ++j) *ckp(blk, j) = S[j];
            const int n = min(TB, T - blk * TB);
            if (n == TB) {
                // a full block: half the block's operands into registers at a time, then the chain
                constexpr int HB = TB / 2;
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    float kb[HB][NG], ab[HB], bb[HB], vb[HB];
#pragma unroll
                    for (int i = 0; i < HB; ++i) {
                        const int r = HB * hb + i;
#pragma unroll
                        for (int j = 0; j < NG; ++j) kb[i][j] = krow(r, j);
                        ab[i] = sa[r];
                        bb[i] = sb[r];
                        vb[i] = sv[r][rl];
                    }
#pragma unroll
                    for (int i = 0; i < HB; ++i) (void)fwd_step(kb[i], ab[i], bb[i], vb[i]);
                }
            } else {
                for (int r = 0; r < n; ++r) (void)fwd_token(r);
            }
        });
        return;
    }
    {
        // ---- the adjoint recurrence alone, backward: dL/dS at the end of every segment ----
#pragma unroll
        for (int j = 0; j < NG; ++j) G[j] = g.d_state ? g.d_state[(((int64_t)b * p.H + h) * p.Dv + row) * DK + 16 * j + part] : 0.f;
        run_blocks(nblk - 1, nblk, -1, true, false, [&](int blk, const float*) __attribute__((always_inline)) {
            if (blk == nblk - 1 || (blk + 1) % BPS == 0) {
#pragma unroll
                for (int j = 0; j < NG; ++j) *gckp(blk / BPS, j) = G[j];
            }
            const int n = min(TB, T - blk * TB);
            auto token = [&](int r) __attribute__((always_inline)) {
                float kr[NG], qr[NG];
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    kr[j] = krow(r, j);
                    qr[j] = qrow(r, j);
                }
                adj_step(kr, qr, p.scale * sdo[r][rl], sa[r], sb[r]);
            };
            if (n == TB) {
                // a full block: a quarter of the block's operands into registers at a time, then the chain
                constexpr int HB = TB / 4;
#pragma unroll
                for (int hb = TB / HB - 1; hb >= 0; --hb) {
                    float kb[HB][NG], qb[HB][NG], db[HB], ab[HB], bb[HB];
#pragma unroll
                    for (int i = 0; i < HB; ++i) {
                        const int r = HB * hb + i;
#pragma unroll
                        for (int j = 0; j < NG; ++j) {
                            kb[i][j] = krow(r, j);
                            qb[i][j] = qrow(r, j);
                        }
                        db[i] = p.scale * sdo[r][rl];
                        ab[i] = sa[r];
                        bb[i] = sb[r];
                    }
#pragma unroll
                    for (int i = HB - 1; i >= 0; --i) adj_step(kb[i], qb[i], db[i], ab[i], bb[i]);
                }
            } else {
                for (int r = n - 1; r >= 0; --r) token(r);
            }
        });
        return;
    }
    } else {
    // ---- phase 1: the walk of segment `unit`, its blocks in reverse, from its adjoint checkpoint ----
    const int blo = unit * BPS, bhi = min(nblk, blo + BPS) - 1;
#pragma unroll
    for (int j = 0; j < NG; ++j) G[j] = *gckp(unit, j);
    run_blocks(bhi, bhi - blo + 1, -1, true, true, [&](int blk, const float* ckv) __attribute__((always_inline)) {
        const int n = min(TB, T - blk * TB);
        // The block is walked in two parts of SH tokens, the later part first, so that LDS holds the
        // states of one part (18 KB instead of 25 KB of LDS at d = 112: eight workgroups per CU
        // instead of six).  Each part recomputes the states from the block's checkpoint up to its
        // last token (the same operations in the same order, so the same bits) and keeps S_{t-1} and
        // x of its own tokens [lo, hi).
        int lo = 0;
        auto rec_token = [&](int r) __attribute__((always_inline)) {
            if (r >= lo) {
#pragma unroll
                for (int j = 0; j < NG; ++j) sst[r - lo][j][lane] = S[j];
            }
            const float x = fwd_token(r);
            if (r >= lo && part == 0) sx[r - lo][rl] = x;
        };
        // After the recomputation S is the state after the part's last token; the part's tokens are
        // walked backward.  A token's LDS operands are read while the previous token finishes (after
        // its column-sum reads, so that they do not hold those back), alternating between two
        // register sets.
        struct TokOps {
            float Sp[NG], kr[NG], qr[NG];
            float dor, at, bt, vr, x;
        };
        auto read_ops = [&](TokOps& o, int r) {
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                o.Sp[j] = sst[r - lo][j][lane];
                o.kr[j] = krow(r, j);
                o.qr[j] = qrow(r, j);
            }
            o.dor = p.scale * sdo[r][rl];
            o.at = sa[r];
            o.bt = sb[r];
            o.vr = sv[r][rl];
            o.x = sx[r - lo][rl];
        };
        auto walk = [&](const TokOps& c, TokOps& nx, int r) __attribute__((always_inline)) {
            const int64_t t = tok(blk * TB + r);
            const float dor = c.dor, at = c.at, bt = c.bt, vr = c.vr, x = c.x;
#pragma unroll
            for (int j = 0; j < NG; ++j) G[j] += dor * c.qr[j];
            const float gk = rowdot(G, c.kr), gs = rowdot(G, c.Sp);
            if (part == 0) g.dv[(((int64_t)b * T + t) * p.H + h) * p.Dv + row] = bt * gk;
            // this row's terms of dq_t = scale S_t^T do_t and dk_t = beta G^T (v - a x) - a beta S_{t-1}^T gk
            const float wv = bt * (vr - at * x), ws = at * bt * gk;
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                scol[0][rl][16 * j + part] = dor * S[j];
                scol[1][rl][16 * j + part] = wv * G[j] - ws * c.Sp[j];
            }
            lds_order();
            const float cg = bt * gk;
#pragma unroll
            for (int j = 0; j < NG; ++j) G[j] = at * (G[j] - cg * c.kr[j]);
            // per-row scalars (identical in the 16 lanes of a row; counted once)
            float da = (part == 0) ? gs - bt * gk * x : 0.f;
            float db = (part == 0) ? gk * (vr - at * x) : 0.f;
            da = sum_rows(da);
            db = sum_rows(db);
            float* pw = g.partials + ((((int64_t)b * T + t) * p.H + h) * nrb + rb) * wid;
            // column sums over the 4 rows, in row order: lane l adds float4 group l
            float4 acc = {0.f, 0.f, 0.f, 0.f};
            const int a = lane / (DK / 4), c4 = 4 * (lane - a * (DK / 4));
            if (lane < DK / 2) {
                acc = *reinterpret_cast<const float4*>(&scol[a][0][c4]);
#pragma unroll
                for (int rr = 1; rr < kRB; ++rr) {
                    const float4 v4 = *reinterpret_cast<const float4*>(&scol[a][rr][c4]);
                    acc.x += v4.x;
                    acc.y += v4.y;
                    acc.z += v4.z;
                    acc.w += v4.w;
                }
            }
            // the next token's operands, behind the column-sum reads
            if (r > lo) read_ops(nx, r - 1);
            lds_order();
            if (lane < DK / 2) *reinterpret_cast<float4*>(pw + a * DK + c4) = acc;
            if (lane == 0) {
                pw[2 * DK] = da;
                pw[2 * DK + 1] = db;
            }
#pragma unroll
            for (int j = 0; j < NG; ++j) S[j] = c.Sp[j];
        };
#pragma unroll
        for (int half = 1; half >= 0; --half) {
            lo = half * SH;
            const int hi = half ? n : min(n, SH);
            if (lo >= hi) continue;
#pragma unroll
            for (int j = 0; j < NG; ++j) S[j] = ckv[j];
            if (n == TB) {
#pragma unroll
                for (int r = 0; r < (half ? TB : SH); ++r) rec_token(r);
            } else {
                for (int r = 0; r < hi; ++r) rec_token(r);
            }
            TokOps oa, ob;
            read_ops(oa, hi - 1);
            int r = hi - 1;
            for (; r >= lo + 1; r -= 2) {
                walk(oa, ob, r);
                walk(ob, oa, r - 1);
            }
            if (r == lo) walk(oa, ob, lo);
        }
    });
    if (unit == 0 && g.d_state0) {
#pragma unroll
        for (int j = 0; j < NG; ++j)
            g.d_state0[(((int64_t)b * p.H + h) * p.Dv + row) * DK + 16 * j + part] = G[j];
    }
    }
}

// sum over the 64 lanes
__device__ __forceinline__ float sum_wave(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// One 64-lane workgroup per (b, t, h): add the row blocks' partial sums (in row-block
// order) and map the gradients of the normalised q_t, k_t back to q_t, k_t.
template <bool F32>
__global__ __launch_bounds__(64) void gdn_bwd_reduce_kernel(Params p, BwdParams g0, BwdParams g1, int64_t n0) {
    const int lane = threadIdx.x;
    const bool second = (int64_t)blockIdx.x >= n0;
    const BwdParams g = second ? g1 : g0;
    int64_t id = (int64_t)blockIdx.x - (second ? n0 : 0);
    const int h = (int)(id % p.H); id /= p.H;
    const int64_t t = id % p.T; id /= p.T;
    const int b = (int)id;
    const int Dk = p.Dk, nrb = p.Dv / kRB, wid = 2 * Dk + 4, nq = wid / 4;
    const float* pw = g.partials + (((int64_t)b * p.T + t) * p.H + h) * nrb * wid;
    // lane l adds the 16-byte groups l and l + 64 of every row block's partial row (wid floats, a
    // multiple of 4) in row-block order, unrolled so that several row blocks' loads are in flight;
    // the sums then go through LDS to the per-column layout below
    __shared__ __align__(16) float red[2 * 128 + 4];
    float4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 8
    for (int r = 0; r < nrb; ++r) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int q4 = lane + 64 * j;
            if (q4 < nq) {
                const float4 v4 = *reinterpret_cast<const float4*>(pw + (int64_t)r * wid + 4 * q4);
                acc[j].x += v4.x;
                acc[j].y += v4.y;
                acc[j].z += v4.z;
                acc[j].w += v4.w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        if (lane + 64 * j < nq) *reinterpret_cast<float4*>(&red[4 * (lane + 64 * j)]) = acc[j];
    lds_order();
    float gq[2], gkk[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j;
        gq[j] = (c < Dk) ? red[c] : 0.f;
        gkk[j] = (c < Dk) ? red[Dk + c] : 0.f;
    }
    const float da = red[2 * Dk], db = red[2 * Dk + 1];
    const int64_t kq = (int64_t)b * p.ks[0] + t * p.ks[1] + (int64_t)h * p.ks[2];
    const int64_t qq = (int64_t)b * p.qs[0] + t * p.qs[1] + (int64_t)h * p.qs[2];
    float kx[2], qx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j;
        kx[j] = (c < Dk) ? ld_elem<F32>(p.k, kq + c) : 0.f;
        qx[j] = (c < Dk) ? ld_elem<F32>(p.q, qq + c) : 0.f;
    }
    const int64_t out = ((int64_t)b * p.T + t) * p.H + h;
    if (p.l2norm) {
        // d x = (d xh - xh (xh . d xh)) / n,  xh = x / n,  n = sqrt(sum x^2 + eps)
        const float nk = sqrtf(sum_wave(kx[0] * kx[0] + kx[1] * kx[1]) + p.eps);
        const float nq = sqrtf(sum_wave(qx[0] * qx[0] + qx[1] * qx[1]) + p.eps);
        const float hk = sum_wave((kx[0] * gkk[0] + kx[1] * gkk[1]) / nk);
        const float hq = sum_wave((qx[0] * gq[0] + qx[1] * gq[1]) / nq);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            gkk[j] = (gkk[j] - kx[j] / nk * hk) / nk;
            gq[j] = (gq[j] - qx[j] / nq * hq) / nq;
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j;
        if (c < Dk) {
            g.dq[out * Dk + c] = gq[j];
            g.dk[out * Dk + c] = gkk[j];
        }
    }
    if (lane == 0) {
        // with a given as log a, dL/d(log a) = a dL/da
        const int64_t gq = (int64_t)b * p.gs[0] + t * p.gs[1] + (int64_t)h * p.gs[2];
        g.da[out] = p.gate_log ? da * expf(p.a[gq]) : da;
        g.dbeta[out] = db;
    }
}

template <int NG, int PHASE>
static void launch_rows_ph(const Params& p, const BwdParams& g0, const BwdParams& g1, hipStream_t s, int nunits, int grid) {
    if (p.io_f32) hipLaunchKernelGGL((gdn_bwd_rows_kernel<NG, true, PHASE>), dim3(grid), dim3(64), 0, s, p, g0, g1, nunits);
    else hipLaunchKernelGGL((gdn_bwd_rows_kernel<NG, false, PHASE>), dim3(grid), dim3(64), 0, s, p, g0, g1, nunits);
}
template <int NG>
static void launch_rows_ng(const Params& p, const BwdParams& g0, const BwdParams& g1, hipStream_t s, int nunits, int grid,
                           int phase) {
    if (phase == 0) launch_rows_ph<NG, 0>(p, g0, g1, s, nunits, grid);
    else launch_rows_ph<NG, 1>(p, g0, g1, s, nunits, grid);
}

static hipError_t launch_rows(const Params& p, const BwdParams& g0, const BwdParams& g1, hipStream_t s, int nunits,
                              int grid, int phase) {
    switch (p.Dk) {
        case 16: launch_rows_ng<1>(p, g0, g1, s, nunits, grid, phase); break;
        case 32: launch_rows_ng<2>(p, g0, g1, s, nunits, grid, phase); break;
        case 48: launch_rows_ng<3>(p, g0, g1, s, nunits, grid, phase); break;
        case 64: launch_rows_ng<4>(p, g0, g1, s, nunits, grid, phase); break;
        case 80: launch_rows_ng<5>(p, g0, g1, s, nunits, grid, phase); break;
        case 96: launch_rows_ng<6>(p, g0, g1, s, nunits, grid, phase); break;
        case 112: launch_rows_ng<7>(p, g0, g1, s, nunits, grid, phase); break;
        case 128: launch_rows_ng<8>(p, g0, g1, s, nunits, grid, phase); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_backward(const Params& p, const BwdParams& g0, const BwdParams* g1, hipStream_t s, Timing* tm) {
    const int nscan = g1 ? 2 : 1;
    const int rows0 = p.B * p.H * (p.Dv / kRB);
    const int nseg = (int)((p.T + kSEG - 1) / kSEG);
    const int64_t red0 = (int64_t)p.B * p.T * p.H;
    const BwdParams& gb = g1 ? *g1 : g0;
    tm_begin(tm, s, KBWD);
    hipError_t e = launch_rows(p, g0, gb, s, 2 * rows0, nscan * 2 * rows0, 0);
    if (e == hipSuccess) e = launch_rows(p, g0, gb, s, nseg * rows0, nscan * nseg * rows0, 1);
    if (e == hipSuccess && red0 > 0) {
        const unsigned grid = (unsigned)(nscan * red0);
        if (p.io_f32) hipLaunchKernelGGL(gdn_bwd_reduce_kernel<true>, dim3(grid), dim3(64), 0, s, p, g0, gb, red0);
        else hipLaunchKernelGGL(gdn_bwd_reduce_kernel<false>, dim3(grid), dim3(64), 0, s, p, g0, gb, red0);
        e = hipGetLastError();
    }
    tm_end(tm, s);
    return e;
}

}  // namespace gdn
