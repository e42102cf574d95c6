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
// sum over the 4 lanes of a lane quad (one state row): quad permutations [1,0,3,2] and [2,3,0,1]
__device__ __forceinline__ float sum4(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    return x;
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
// gdn_bwd_rows_kernel: one 64-lane workgroup per (b, h, block of 16 state rows),
// lane l owns row 16 rb + l/4 and columns l%4 + 4i, as in gdn_seq_kernel.  It
// runs the scan forward storing the state before every token, then walks the
// tokens backward with G = dL/dS:
//     G += scale do_t q_t^T,  x = S_{t-1} k_t,  gk = G k_t
//     dv_t = beta_t gk,  da_t = <G, S_{t-1}> - beta_t gk.x,  dbeta_t = gk.(v_t - a_t x)
//     dk_t = beta_t G^T v_t - a_t beta_t (S_{t-1}^T gk + G^T x),  dq_t = scale S_t^T do_t
//     G <- a_t (G - beta_t gk k_t^T)
// (q_t, k_t normalised).  dv and the start-state gradient are row-local; the
// other gradients sum over all rows, so each workgroup writes its rows' partial
// sums, and gdn_bwd_reduce_kernel adds them in a fixed order and maps the
// normalised-vector gradients back through the L2 normalisation.
// ---------------------------------------------------------------------------
int64_t backward_ws_bytes(int B, int H, int Dk, int Dv, int64_t max_tokens) {
    const int64_t nrb = Dv / 16;
    int64_t states = 0, partials = 0, total = 0;
    if (__builtin_mul_overflow((int64_t)B * H, nrb * 16 * Dk, &states) ||
        __builtin_mul_overflow(states, max_tokens + 1, &states) ||
        __builtin_mul_overflow((int64_t)B * H, nrb * (2 * Dk + 2), &partials) ||
        __builtin_mul_overflow(partials, max_tokens, &partials) || __builtin_add_overflow(states, partials, &total) ||
        __builtin_mul_overflow(total, (int64_t)4, &total))
        return -1;
    return total;
}

// sum over the 16 rows of the workgroup (lane bits 2..5): within each row of 16 lanes by two
// rotations (by 4, then by 8: lanes j, j-4, j-8, j-12), then across the four rows
__device__ __forceinline__ float sum_rows(float x) {
    x += dpp<0x124>(x);   // row_ror:4
    x += dpp<0x128>(x);   // row_ror:8
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

template <bool F32>
__global__ __launch_bounds__(64) void gdn_bwd_rows_kernel(Params p, BwdParams g) {
    constexpr int MAXC = 32;  // d_k <= 128
    const int lane = threadIdx.x, part = lane & 3, rl = lane >> 2;
    const int nrb = p.Dv / 16;
    int id = blockIdx.x;
    const int rb = id % nrb; id /= nrb;
    const int h = id % p.H; id /= p.H;
    const int b = id;
    const int row = 16 * rb + rl;
    const int nc = p.Dk / 4;
    const int64_t T = p.T;
    const int Dk = p.Dk;
    float* st = g.states + (((int64_t)b * p.H + h) * nrb + rb) * (T + 1) * 16 * Dk;
    auto sidx = [&](int64_t pi, int i) { return (pi * 16 + rl) * Dk + part + 4 * i; };
    const int64_t srow = (((int64_t)b * p.H + h) * p.Dv + row) * Dk;

    // token loads: the normalised k_t, q_t columns of this lane, a_t, beta_t, v_t[row]
    auto load_token = [&](int64_t t, float* kv, float* qv, float& at, float& bt, float& vr) {
        const int64_t kq = (int64_t)b * p.ks[0] + t * p.ks[1] + (int64_t)h * p.ks[2];
        const int64_t qq = (int64_t)b * p.qs[0] + t * p.qs[1] + (int64_t)h * p.qs[2];
        const int64_t vq = (int64_t)b * p.vs[0] + t * p.vs[1] + (int64_t)h * p.vs[2];
        const int64_t gq = (int64_t)b * p.gs[0] + t * p.gs[1] + (int64_t)h * p.gs[2];
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            kv[i] = (i < nc) ? ld_elem<F32>(p.k, kq + part + 4 * i) : 0.f;
            qv[i] = (i < nc) ? ld_elem<F32>(p.q, qq + part + 4 * i) : 0.f;
            sk += kv[i] * kv[i];
            sq += qv[i] * qv[i];
        }
        if (p.l2norm) {
            const float rk = 1.f / sqrtf(sum4(sk) + p.eps);
            const float rq = 1.f / sqrtf(sum4(sq) + p.eps);
#pragma unroll
            for (int i = 0; i < MAXC; ++i) { kv[i] *= rk; qv[i] *= rq; }
        }
        at = p.gate_log ? expf(p.a[gq]) : p.a[gq];
        bt = p.beta[gq];
        vr = ld_elem<F32>(p.v, vq + row);
    };

    // forward, keeping the state before every step (and the final one)
    float S[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) S[i] = (i < nc && g.state0) ? g.state0[srow + part + 4 * i] : 0.f;
    for (int64_t pi = 0; pi < T; ++pi) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i)
            if (i < nc) st[sidx(pi, i)] = S[i];
        const int64_t t = g.reverse ? (T - 1 - pi) : pi;
        float kv[MAXC], qv[MAXC], at, bt, vr;
        load_token(t, kv, qv, at, bt, vr);
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) x += S[i] * kv[i];
        x = sum4(x);
#pragma unroll
        for (int i = 0; i < MAXC; ++i) S[i] = at * (S[i] - bt * x * kv[i]) + bt * vr * kv[i];
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
        if (i < nc) st[sidx(T, i)] = S[i];

    // backward
    float G[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) G[i] = (i < nc && g.d_state) ? g.d_state[srow + part + 4 * i] : 0.f;
    const int wid = 2 * Dk + 2;
    for (int64_t pi = T - 1; pi >= 0; --pi) {
        const int64_t t = g.reverse ? (T - 1 - pi) : pi;
        float kv[MAXC], qv[MAXC], at, bt, vr;
        load_token(t, kv, qv, at, bt, vr);
        const int64_t oq = (int64_t)b * p.os[0] + t * p.os[1] + (int64_t)h * p.os[2];
        const float dor = p.scale * ld_elem<F32>(g.d_o, oq + row);
        float Sp[MAXC], pq[MAXC], pk[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            Sp[i] = (i < nc) ? st[sidx(pi, i)] : 0.f;
            pq[i] = (i < nc) ? dor * st[sidx(pi + 1, i)] : 0.f;   // scale do_t[row] S_t[row, c]
            G[i] += dor * qv[i];
        }
        float x = 0.f, gk = 0.f, gs = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            x += Sp[i] * kv[i];
            gk += G[i] * kv[i];
            gs += G[i] * Sp[i];
        }
        x = sum4(x);
        gk = sum4(gk);
        gs = sum4(gs);
        if (part == 0) g.dv[(((int64_t)b * T + t) * p.H + h) * p.Dv + row] = bt * gk;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            pk[i] = bt * G[i] * vr - at * bt * (Sp[i] * gk + G[i] * x);
            G[i] = at * (G[i] - bt * gk * kv[i]);
        }
        // per-row scalars: every lane of a row holds them; count each row once
        float da = (part == 0) ? gs - bt * gk * x : 0.f;
        float db = (part == 0) ? gk * (vr - at * x) : 0.f;
        da = sum4(da);
        db = sum4(db);
        da = sum_rows(da);
        db = sum_rows(db);
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            if (i < nc) {
                pq[i] = sum_rows(pq[i]);
                pk[i] = sum_rows(pk[i]);
            }
        }
        float* pw = g.partials + ((((int64_t)b * T + t) * p.H + h) * nrb + rb) * wid;
        if (rl == 0) {
#pragma unroll
            for (int i = 0; i < MAXC; ++i) {
                if (i < nc) {
                    pw[part + 4 * i] = pq[i];
                    pw[Dk + part + 4 * i] = pk[i];
                }
            }
            if (part == 0) {
                pw[2 * Dk] = da;
                pw[2 * Dk + 1] = db;
            }
        }
    }
    if (g.d_state0) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i)
            if (i < nc) g.d_state0[srow + part + 4 * i] = G[i];
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
__global__ __launch_bounds__(64) void gdn_bwd_reduce_kernel(Params p, BwdParams g) {
    const int lane = threadIdx.x;
    int64_t id = blockIdx.x;
    const int h = (int)(id % p.H); id /= p.H;
    const int64_t t = id % p.T; id /= p.T;
    const int b = (int)id;
    const int Dk = p.Dk, nrb = p.Dv / 16, wid = 2 * Dk + 2;
    const float* pw = g.partials + (((int64_t)b * p.T + t) * p.H + h) * nrb * wid;
    float gq[2] = {0.f, 0.f}, gkk[2] = {0.f, 0.f}, da = 0.f, db = 0.f;
    for (int r = 0; r < nrb; ++r) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = lane + 64 * j;
            if (c < Dk) {
                gq[j] += pw[r * wid + c];
                gkk[j] += pw[r * wid + Dk + c];
            }
        }
        da += pw[r * wid + 2 * Dk];
        db += pw[r * wid + 2 * Dk + 1];
    }
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

hipError_t launch_backward(const Params& p, const BwdParams& g, hipStream_t s, Timing* tm) {
    const int rows_grid = p.B * p.H * (p.Dv / 16);
    const int64_t red_grid = (int64_t)p.B * p.T * p.H;
    tm_begin(tm, s, KBWD);
    if (p.io_f32) hipLaunchKernelGGL(gdn_bwd_rows_kernel<true>, dim3(rows_grid), dim3(64), 0, s, p, g);
    else hipLaunchKernelGGL(gdn_bwd_rows_kernel<false>, dim3(rows_grid), dim3(64), 0, s, p, g);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && red_grid > 0) {
        if (p.io_f32) hipLaunchKernelGGL(gdn_bwd_reduce_kernel<true>, dim3((unsigned)red_grid), dim3(64), 0, s, p, g);
        else hipLaunchKernelGGL(gdn_bwd_reduce_kernel<false>, dim3((unsigned)red_grid), dim3(64), 0, s, p, g);
        e = hipGetLastError();
    }
    tm_end(tm, s);
    return e;
}

}  // namespace gdn
