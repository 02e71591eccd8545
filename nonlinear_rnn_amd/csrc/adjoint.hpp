// Adjoint of the converged solve (the backward pass), one streaming kernel.
//
// For L = sum_t <g_t, s_t> (g_t = dL/ds_t from upstream) the adjoint
// lam = dL/ds solves the transposed block-bidiagonal system of
// "Параллельность RNN?" (forpes.ru), §1.3: J(s*)^T lam = g, i.e. the
// reverse-time recurrence lam_t = g_t + A_{t+1}^T lam_{t+1} (lam_{T+1} = 0)
// with A_t = df/ds at (s_{t-1}, u_t).  Writing mu_t = A_t^T lam_t it is the
// affine recurrence
//     mu_t = A_t^T mu_{t+1} + A_t^T g_t,      lam_t = g_t + mu_{t+1},
// whose maps use only step t's own Jacobian, so it is scanned exactly like
// the forward Newton systems, in reverse time: lanes, waves and time blocks
// are laid out so that ascending lane / wave / ticket order is descending
// time and the forward scan machinery applies unchanged.  dL/ds_0 = mu_1.
// Gate gradients follow elementwise from lam_t; dL/da is reduced per
// workgroup and then over batch rows and time blocks in a fixed order.
#pragma once

#include "cells.hpp"
#include "solve.hpp"

namespace pararnn {

struct AdjArgs {
    const void *u[4];
    const float *a;
    const float *s0[2];
    const float *s[2];
    const float *gs[2];
    const float *gend[2];  // [B][D] added to g at the last step, or null
    float *du[4];
    float *da;
    int32_t da_acc;        // 1: da += the new sum, 0: da = the new sum
    float *ds0[2];
    float *lam[2];
    int64_t B, T, D;
    int64_t usb, usd, ssb, ssd;
    int64_t ust, sst;  // time strides (1 = channel-major)
    int64_t channels;
    int32_t nb;
    int32_t u_vec, du_vec, s_vec;
    uint32_t *ticket;
    int32_t *flags;
    float *records;
    float *da_part;
};

// Per-step quantities the reverse sweep needs, computed once from
// (s_{t-1}, u_t); the reverse map is (A_t^T, A_t^T g_t).
struct GruAdj {
    using Cell = GruCell;
    struct F {
        float J, y1, y2, y3, rh, hp, gh;
    };
    static __device__ __forceinline__ F prep(const GruCell::Coef &p, const float (&u)[3],
                                             const Vec1 &sp, const Vec1 &g)
    {
        F x;
        const float hp = sp.x;
        const float z = sigmoid_q(fmaf_(p.qz, hp, u[0]));
        const float r = sigmoid_q(fmaf_(p.qr, hp, u[1]));
        const float rh = r * hp;
        const float c = tanh_q(fmaf_(p.qc, rh, u[2]));
        const float cmh = c - hp;
        const float omz = 1.0f - z;
        const float zz = z * omz;
        const float dr = (r * (1.0f - r)) * p.ar;
        const float y2 = z * fmaf_(-c, c, 1.0f);          // d h' / d p_c
        x.J = fmaf_(cmh, zz * p.az, fmaf_(y2 * p.ac, fmaf_(hp, dr, r), omz));
        x.y1 = cmh * zz;                                  // d h' / d p_z
        x.y2 = y2;
        x.y3 = y2 * p.ac * hp * (r * (1.0f - r));         // d h' / d p_r
        x.rh = rh;
        x.hp = hp;
        x.gh = g.x;
        return x;
    }
    static __device__ __forceinline__ Map1 map(const GruCell::Coef &, const F &x)
    {
        return {x.J, x.J * x.gh};
    }
    // One reverse step: lam = g + mu_{t+1}; gate gradients; returns mu_t.
    static __device__ __forceinline__ Vec1 back(const GruCell::Coef &, const F &x, const Vec1 &mu,
                                                float (&dp)[3], float (&da)[3], Vec1 &lam)
    {
        const float l = x.gh + mu.x;
        lam.x = l;
        dp[0] = l * x.y1;
        dp[1] = l * x.y3;
        dp[2] = l * x.y2;
        da[0] = fmaf_(dp[0], x.hp, da[0]);
        da[1] = fmaf_(dp[1], x.hp, da[1]);
        da[2] = fmaf_(dp[2], x.rh, da[2]);
        return {x.J * l};
    }
};

struct LstmAdj {
    using Cell = LstmCell;
    struct F {
        float f, x1, x2, x3, x4, x5, hp, gc, gh;
    };
    static __device__ __forceinline__ F prep(const LstmCell::Coef &p, const float (&u)[4],
                                             const Vec2 &sp, const Vec2 &g)
    {
        F x;
        const float cp = sp.x0, hp = sp.x1;
        const float i = sigmoid_q(fmaf_(p.qi, hp, u[0]));
        const float f = sigmoid_q(fmaf_(p.qf, hp, u[1]));
        const float gg = tanh_q(fmaf_(p.qg, hp, u[2]));
        const float o = sigmoid_q(fmaf_(p.qo, hp, u[3]));
        const float c = fmaf_(f, cp, i * gg);
        const float tc = tanh_q(c * (-2.0f * kLog2e));
        x.f = f;
        x.x1 = o * fmaf_(-tc, tc, 1.0f);      // d h'/d c' = o (1 - tanh^2 c')
        x.x2 = tc * (o * (1.0f - o));         // d h'/d p_o
        x.x3 = gg * (i * (1.0f - i));         // d c'/d p_i
        x.x4 = cp * (f * (1.0f - f));         // d c'/d p_f
        x.x5 = i * fmaf_(-gg, gg, 1.0f);      // d c'/d p_g
        x.hp = hp;
        x.gc = g.x0;
        x.gh = g.x1;
        return x;
    }
    // A^T with A = [[f, dcdh], [x1 f, x1 dcdh + a_o x2]], state order (c, h).
    static __device__ __forceinline__ Map2 map(const LstmCell::Coef &p, const F &x)
    {
        const float dcdh = fmaf_(p.af, x.x4, fmaf_(p.ai, x.x3, p.ag * x.x5));
        const float dhdh = fmaf_(p.ao, x.x2, x.x1 * dcdh);
        Map2 m;
        m.a00 = x.f;
        m.a01 = x.x1 * x.f;
        m.a10 = dcdh;
        m.a11 = dhdh;
        m.b0 = fmaf_(m.a00, x.gc, m.a01 * x.gh);
        m.b1 = fmaf_(m.a10, x.gc, m.a11 * x.gh);
        return m;
    }
    static __device__ __forceinline__ Vec2 back(const LstmCell::Coef &p, const F &x, const Vec2 &mu,
                                                float (&dp)[4], float (&da)[4], Vec2 &lam)
    {
        const float lc = x.gc + mu.x0, lh = x.gh + mu.x1;
        lam = {lc, lh};
        const float ec = fmaf_(lh, x.x1, lc);  // total dL/dc' at this step
        dp[0] = ec * x.x3;
        dp[1] = ec * x.x4;
        dp[2] = ec * x.x5;
        dp[3] = lh * x.x2;
#pragma unroll
        for (int q = 0; q < 4; ++q) da[q] = fmaf_(dp[q], x.hp, da[q]);
        return {ec * x.f,
                fmaf_(p.ai, dp[0], fmaf_(p.af, dp[1], fmaf_(p.ag, dp[2], p.ao * dp[3])))};
    }
};

template <class Cell>
struct AdjOf;
template <>
struct AdjOf<GruCell> {
    using type = GruAdj;
};
template <>
struct AdjOf<LstmCell> {
    using type = LstmAdj;
};

template <class Cell, int K, int W, bool BF16>
__global__ void __launch_bounds__(W * kWave) adjoint_kernel(AdjArgs A)
{
    using Adj = typename AdjOf<Cell>::type;
    using M = typename Cell::Map;
    using V = typename Cell::Vec;
    using F = typename Adj::F;
    constexpr int G = Cell::G, S = Cell::S;
    constexpr int P = W * kWave * K;
    constexpr int RF = MapRec<M>::kFloats;

    __shared__ M s_agg[W];
    __shared__ float s_da[W][G];
    __shared__ int64_t s_ticket;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    int64_t ch;
    int32_t k;
    if (A.nb > 1) {
        int32_t q;
        take_unit(A.ticket, A.channels, A.nb, s_ticket, ch, q);
        k = A.nb - 1 - q;  // later time blocks take earlier tickets
    } else {
        ch = xcd_channel(blockIdx.x, A.channels);
        k = 0;
    }
    if (ch >= A.channels) return;
    const int64_t unit = ch * A.nb + k;
    const int64_t b = ch / A.D, d = ch - b * A.D;
    const int64_t T = A.T;
    const int64_t tb0 = (int64_t)k * P;
    // ascending lane/wave order = descending time
    const int64_t chunk = (int64_t)(W * kWave - 1) - (wave * kWave + lane);
    const int64_t t0 = tb0 + chunk * K;

    const typename Cell::Coef cf = Cell::coef(A.a, A.D, d);
    const int64_t uoff = b * A.usb + d * A.usd;
    const int64_t soff = b * A.ssb + d * A.ssd;

    F fx[K];
    // A block wholly inside [0, T) on 16-byte vectors issues every load of
    // its inputs before using any (no per-vector bounds tests, which would
    // put each load in a block of its own and make the compiler wait for one
    // before issuing the next); the general path below serves the rest.
    constexpr int EU = BF16 ? 8 : 4;
    bool done = false;
    if constexpr (K % EU == 0 && K % 4 == 0) {
        if (A.u_vec && A.s_vec && tb0 + P <= T) {
            uint4 ru[G][K / EU];
            float4 rs[S][K / 4], rg[S][K / 4];
            float first[S];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint8_t *p =
                    static_cast<const uint8_t *>(A.u[g]) + (uoff + t0) * (BF16 ? 2 : 4);
#pragma unroll
                for (int q = 0; q < K / EU; ++q) ru[g][q] = reinterpret_cast<const uint4 *>(p)[q];
            }
#pragma unroll
            for (int c = 0; c < S; ++c) {
                const float *p = A.s[c] + soff + t0;
#pragma unroll
                for (int q = 0; q < K / 4; ++q) rs[c][q] = reinterpret_cast<const float4 *>(p)[q];
                first[c] = *(t0 == 0 ? A.s0[c] + b * A.D + d : A.s[c] + soff + t0 - 1);
            }
#pragma unroll
            for (int c = 0; c < S; ++c) {
                if (A.gs[c]) {
                    const float *p = A.gs[c] + soff + t0;
#pragma unroll
                    for (int q = 0; q < K / 4; ++q) rg[c][q] = reinterpret_cast<const float4 *>(p)[q];
                } else {
#pragma unroll
                    for (int q = 0; q < K / 4; ++q) rg[c][q] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
            float u[K][G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float sc = Cell::uscale(g);
#pragma unroll
                for (int q = 0; q < K / EU; ++q) {
                    const uint32_t w[4] = {ru[g][q].x, ru[g][q].y, ru[g][q].z, ru[g][q].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (BF16) {
                            u[8 * q + 2 * j][g] = __uint_as_float(w[j] << 16) * sc;
                            u[8 * q + 2 * j + 1][g] = __uint_as_float(w[j] & 0xffff0000u) * sc;
                        } else {
                            u[4 * q + j][g] = __uint_as_float(w[j]) * sc;
                        }
                    }
                }
            }
            V sp[K], gv[K];
#pragma unroll
            for (int c = 0; c < S; ++c) {
                float st[K], gt[K];
#pragma unroll
                for (int q = 0; q < K / 4; ++q) {
                    st[4 * q] = rs[c][q].x;
                    st[4 * q + 1] = rs[c][q].y;
                    st[4 * q + 2] = rs[c][q].z;
                    st[4 * q + 3] = rs[c][q].w;
                    gt[4 * q] = rg[c][q].x;
                    gt[4 * q + 1] = rg[c][q].y;
                    gt[4 * q + 2] = rg[c][q].z;
                    gt[4 * q + 3] = rg[c][q].w;
                }
                // the gradient a continuation of the sequence sends back to s_T
                if (A.gend[c] && t0 + K == T) gt[K - 1] += A.gend[c][b * A.D + d];
                vset(sp[0], c, first[c]);
#pragma unroll
                for (int kk = 1; kk < K; ++kk) vset(sp[kk], c, st[kk - 1]);
#pragma unroll
                for (int kk = 0; kk < K; ++kk) vset(gv[kk], c, gt[kk]);
            }
#pragma unroll
            for (int kk = 0; kk < K; ++kk) fx[kk] = Adj::prep(cf, u[kk], sp[kk], gv[kk]);
            done = true;
        }
    }
    if (!done) {
        float u[K][G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float tmp[K];
            load_steps<K, BF16>(A.u[g], uoff, t0, T, A.ust, A.u_vec != 0, tmp);
            const float sc = Cell::uscale(g);
#pragma unroll
            for (int kk = 0; kk < K; ++kk) u[kk][g] = tmp[kk] * sc;
        }
        V sp[K], gv[K];
#pragma unroll
        for (int c = 0; c < S; ++c) {
            float tmp[K];
            load_steps<K, false>(A.s[c], soff, t0, T, A.sst, A.s_vec != 0, tmp);
            float first = 0.0f;
            if (t0 == 0)
                first = A.s0[c][b * A.D + d];
            else if (t0 - 1 < T)
                first = A.s[c][soff + (t0 - 1) * A.sst];
            vset(sp[0], c, first);
#pragma unroll
            for (int kk = 1; kk < K; ++kk) vset(sp[kk], c, tmp[kk - 1]);
            if (A.gs[c]) {
                load_steps<K, false>(A.gs[c], soff, t0, T, A.sst, A.s_vec != 0, tmp);
            } else {
#pragma unroll
                for (int kk = 0; kk < K; ++kk) tmp[kk] = 0.0f;
            }
            // the gradient a continuation of the sequence sends back to s_T
            if (A.gend[c] && t0 <= T - 1 && T - 1 < t0 + K) {
                const float e = A.gend[c][b * A.D + d];
#pragma unroll
                for (int kk = 0; kk < K; ++kk)
                    if (t0 + kk == T - 1) tmp[kk] += e;
            }
#pragma unroll
            for (int kk = 0; kk < K; ++kk) vset(gv[kk], c, tmp[kk]);
        }
#pragma unroll
        for (int kk = 0; kk < K; ++kk) fx[kk] = Adj::prep(cf, u[kk], sp[kk], gv[kk]);
    }

    // lane aggregate of the reverse maps, latest step applied first
    M agg = identity_map(M{});
#pragma unroll
    for (int kk = K - 1; kk >= 0; --kk) {
        const M mk = (t0 + kk < T) ? Adj::map(cf, fx[kk]) : identity_map(M{});
        agg = kk == K - 1 ? mk : compose(mk, agg);
    }
    const M inc = wave_scan_inclusive(agg);
    const M exc = wave_shift_up(inc);
    if (lane == kWave - 1) s_agg[wave] = inc;
    __syncthreads();
    M blk = s_agg[0];
#pragma unroll
    for (int j = 1; j < W; ++j) blk = compose(s_agg[j], blk);

    // carry from the later time blocks of the channel
    V din = vzero<V>();
    if (A.nb > 1) {
        if (threadIdx.x == 0) {
            rec_store(A.records + unit * RF, blk, 0u);
            publish_flag(A.flags + unit, 1);
        }
        if (k < A.nb - 1) {
            // later blocks k+1..nb-1, one per lane, folded from the last one
            const int lane = threadIdx.x & (kWave - 1);
            const int32_t *flags = A.flags + ch * A.nb;
            for (int32_t hi = A.nb; hi > k + 1; hi -= kWave) {
                const int32_t lo = hi - kWave > k + 1 ? hi - kWave : k + 1;
                const int32_t j = lo + lane;
                const bool mine = j < hi;
                int32_t v = mine ? load_flag(flags + j) : 1;
                while (!__all(!mine || v >= 1)) {
                    __builtin_amdgcn_s_sleep(1);
                    if (mine && v < 1) v = load_flag(flags + j);
                }
                after_flag();
                M mj = identity_map(M{});
                if (mine) rec_load(A.records + (ch * A.nb + j) * RF, mj);
                for (int32_t q = hi - lo - 1; q >= 0; --q) din = apply(readlane_map(mj, q), din);
            }
        }
    }
    V mu = din;
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        if (j < wave) mu = apply(s_agg[j], mu);
    mu = apply(exc, mu);  // mu at step t0 + K, from every later step

    float da[G];
#pragma unroll
    for (int g = 0; g < G; ++g) da[g] = 0.0f;
    float dpo[G][K];
    float lo[S][K];
#pragma unroll
    for (int kk = K - 1; kk >= 0; --kk) {
        float dp[G];
        V lam;
        if (t0 + kk < T) {
            mu = Adj::back(cf, fx[kk], mu, dp, da, lam);
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) dp[g] = 0.0f;
            lam = vzero<V>();
        }
#pragma unroll
        for (int g = 0; g < G; ++g) dpo[g][kk] = dp[g];
#pragma unroll
        for (int c = 0; c < S; ++c) lo[c][kk] = vget(lam, c);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) store_steps<K>(A.du[g] + uoff, t0, T, A.ust, A.du_vec != 0, dpo[g]);
    if (A.lam[0]) {
#pragma unroll
        for (int c = 0; c < S; ++c) store_steps<K>(A.lam[c] + soff, t0, T, A.sst, A.s_vec != 0, lo[c]);
    }
    if (t0 == 0) {
#pragma unroll
        for (int c = 0; c < S; ++c) A.ds0[c][b * A.D + d] = vget(mu, c);
    }

    // dL/da partial of this workgroup, fixed-order reduction
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float w = wave_sum_to_last(da[g]);
        if (lane == kWave - 1) s_da[wave][g] = w;
    }
    __syncthreads();
    if (threadIdx.x < G) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < W; ++j) acc += s_da[j][threadIdx.x];
        A.da_part[unit * G + threadIdx.x] = acc;
    }
}

#ifdef PARARNN_DEFINE_AUX_KERNELS  // compiled once, in the ABI translation unit
__global__ void adjoint_init_kernel(AdjArgs A, int32_t S, int32_t G, int64_t units)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) *A.ticket = 0u;
    if (i < units) {
        A.flags[i] = 0;
        if (A.T == 0) {
            // no steps: every gradient that exists is zero
            for (int g = 0; g < G; ++g) A.da_part[i * G + g] = 0.0f;
            // (s_T is s_0 itself: a continuation's gradient passes through)
            const int64_t ch = i / A.nb;
            if (i - ch * A.nb == 0)
                for (int c = 0; c < S; ++c) A.ds0[c][ch] = A.gend[c] ? A.gend[c][ch] : 0.0f;
        }
    }
}

// da[g][d] = sum over batch rows b and time blocks k of the partials, in
// that fixed order (added to the value already in da when da_acc is set).
__global__ void da_reduce_kernel(AdjArgs A, int32_t G)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)G * A.D) return;
    const int64_t g = i / A.D, d = i - g * A.D;
    float acc = 0.0f;
    for (int64_t b = 0; b < A.B; ++b)
        for (int32_t k = 0; k < A.nb; ++k) acc += A.da_part[((b * A.D + d) * A.nb + k) * G + g];
    A.da[i] = A.da_acc ? A.da[i] + acc : acc;
}

#endif

}  // namespace pararnn
