// ParaGRU / ParaLSTM cells: residual, local Jacobian and adjoint factors.
//
// The cells are the GRU and LSTM with diagonal recurrent matrices of the
// voguetech.ru ParaRNN article ("Что именно сделали технически", item 3):
// their Jacobians are diagonal (ParaGRU) and 2x2 block diagonal
// (ParaLSTM, state (c, h)), so one channel is a 1- or 2-dimensional system.
//   ParaGRU  z = sig(a_z h + u_z), r = sig(a_r h + u_r),
//            c = tanh(a_c (r h) + u_c),  h' = (1 - z) h + z c
//   ParaLSTM i, f, o = sig(a_* h + u_*), g = tanh(a_g h + u_g),
//            c' = f c + i g,  h' = o tanh(c')
// The DEER residual is r_t = s_t - f(s_{t-1}, u_t) ("Параллельность RNN?",
// forpes.ru, §1.1) and the Newton system's sub-diagonal block is
// A_t = df/ds at (s_{t-1}, u_t) (§1.3).  Each element yields the affine map
// ds_t = A_t ds_{t-1} + b_t with b_t = -r_t = f(s_{t-1}) - s_t.
//
// Transcendentals run on pre-scaled arguments: a gate pre-activation
// p = a h + u enters sigmoid as q = -log2(e) p = a' h + u' with
// a' = -log2(e) a and u' = -log2(e) u computed once per solve (tanh uses
// -2 log2(e)), so each gate costs one FMA, one v_exp, one add, one v_rcp.
#pragma once

#include "scan.hpp"

namespace pararnn {

// ------------------------------------------------------------ ParaGRU ----
struct GruCell {
    static constexpr int G = 3;  // z, r, c
    static constexpr int S = 1;  // h
    using Map = Map1;
    using Vec = Vec1;
    struct Coef {
        float qz, qr, qc;  // scaled diagonal weights
        float az, ar, ac;  // raw diagonal weights (Jacobian)
    };
    static __device__ __forceinline__ Coef coef(const float *a, int64_t D, int64_t d)
    {
        Coef c;
        c.az = a[d];
        c.ar = a[D + d];
        c.ac = a[2 * D + d];
        c.qz = -kLog2e * c.az;
        c.qr = -kLog2e * c.ar;
        c.qc = -2.0f * kLog2e * c.ac;
        return c;
    }
    static __device__ __forceinline__ float uscale(int g) { return g == 2 ? -2.0f * kLog2e : -kLog2e; }

    struct Gates {
        float z, r, c;
    };
    static __device__ __forceinline__ Gates gates(const Coef &p, const float (&u)[G], float hp)
    {
        Gates q;
        q.z = sigmoid_q(fmaf_(p.qz, hp, u[0]));
        q.r = sigmoid_q(fmaf_(p.qr, hp, u[1]));
        q.c = tanh_q(fmaf_(p.qc, q.r * hp, u[2]));
        return q;
    }
    // f(h_{t-1} = hp, u_t): one step of the recurrence.
    static __device__ __forceinline__ Vec1 next(const Coef &p, const float (&u)[G], const Vec1 &hp_)
    {
        const float hp = hp_.x;
        const Gates q = gates(p, u, hp);
        return {fmaf_(q.z, q.c - hp, hp)};
    }
    // -r_t = f(h_{t-1} = hp, u_t) - h_t alone (no Jacobian).
    static __device__ __forceinline__ Vec1 step_residual(const Coef &p, const float (&u)[G],
                                                         const Vec1 &hp_, const Vec1 &h_)
    {
        const float hp = hp_.x;
        const Gates q = gates(p, u, hp);
        return {fmaf_(q.z, q.c - hp, hp - h_.x)};
    }
    // Affine map of one step at (h_{t-1} = hp, u_t) for the current iterate
    // h_t = h.  b = -r_t.
    static __device__ __forceinline__ Map1 step_map(const Coef &p, const float (&u)[G],
                                                    const Vec1 &hp_, const Vec1 &h_)
    {
        const float hp = hp_.x;
        const Gates q = gates(p, u, hp);
        const float z = q.z, r = q.r, c = q.c;
        const float cmh = c - hp;
        const float b = fmaf_(z, cmh, hp - h_.x);   // f - h_t = -r_t, f = (1 - z) h + z c
        // df/dh = (1 - z) + z [ (c - h)(1 - z) a_z + (1 - c^2) a_c (r + h a_r r(1 - r)) ]
        const float omz = 1.0f - z;
        const float dcr = (fmaf_(-c, c, 1.0f) * p.ac) * fmaf_(hp * p.ar, fmaf_(-r, r, r), r);
        const float J = fmaf_(z, fmaf_(cmh * omz, p.az, dcr), omz);
        return {J, b};
    }
    // step_map at h_{t-1} = h_t = 0 (every step of the zero Newton start but
    // a lane's first): the terms with h drop out exactly, so the values are
    // those of step_map bit for bit — z = sig(u_z), r = sig(u_r),
    // c = tanh(u_c), b = z c, df/dh = (1 - z) + z [c (1 - z) a_z + (1 - c^2) a_c r].
    static constexpr bool kZeroPass = true;
    static __device__ __forceinline__ Map1 step_map_zero(const Coef &p, const float (&u)[G])
    {
        const float z = sigmoid_q(u[0]), r = sigmoid_q(u[1]), c = tanh_q(u[2]);
        const float omz = 1.0f - z;
        const float dcr = (fmaf_(-c, c, 1.0f) * p.ac) * r;
        const float J = fmaf_(z, fmaf_(c * omz, p.az, dcr), omz);
        return {J, fmaf_(z, c, 0.0f)};
    }
};

// ----------------------------------------------------------- ParaLSTM ----
struct LstmCell {
    static constexpr int G = 4;  // i, f, g, o
    static constexpr int S = 2;  // c, h
    using Map = Map2;
    using Vec = Vec2;
    struct Coef {
        float qi, qf, qg, qo;
        float ai, af, ag, ao;
    };
    static __device__ __forceinline__ Coef coef(const float *a, int64_t D, int64_t d)
    {
        Coef c;
        c.ai = a[d];
        c.af = a[D + d];
        c.ag = a[2 * D + d];
        c.ao = a[3 * D + d];
        c.qi = -kLog2e * c.ai;
        c.qf = -kLog2e * c.af;
        c.qg = -2.0f * kLog2e * c.ag;
        c.qo = -kLog2e * c.ao;
        return c;
    }
    static __device__ __forceinline__ float uscale(int g) { return g == 2 ? -2.0f * kLog2e : -kLog2e; }

    // No zero-start first pass: with every step's gates depending on u alone
    // the scheduler hoists them all and the one-block kernels spill.
    static constexpr bool kZeroPass = false;
    struct Gates {
        float i, f, g, o, c, tc;  // gates, c' and tanh(c')
    };
    static __device__ __forceinline__ Gates gates(const Coef &p, const float (&u)[G], float cp,
                                                  float hp)
    {
        Gates q;
        q.i = sigmoid_q(fmaf_(p.qi, hp, u[0]));
        q.f = sigmoid_q(fmaf_(p.qf, hp, u[1]));
        q.g = tanh_q(fmaf_(p.qg, hp, u[2]));
        q.o = sigmoid_q(fmaf_(p.qo, hp, u[3]));
        q.c = fmaf_(q.f, cp, q.i * q.g);
        q.tc = tanh_q(q.c * (-2.0f * kLog2e));
        return q;
    }
    // f(s_{t-1} = sp, u_t): one step of the recurrence.
    static __device__ __forceinline__ Vec2 next(const Coef &p, const float (&u)[G], const Vec2 &sp)
    {
        const Gates q = gates(p, u, sp.x0, sp.x1);
        return {q.c, q.o * q.tc};
    }
    // -r_t = f(s_{t-1} = sp, u_t) - s_t alone (no Jacobian).
    static __device__ __forceinline__ Vec2 step_residual(const Coef &p, const float (&u)[G],
                                                         const Vec2 &sp, const Vec2 &s)
    {
        const Gates q = gates(p, u, sp.x0, sp.x1);
        return {q.c - s.x0, q.o * q.tc - s.x1};
    }
    static __device__ __forceinline__ Map2 step_map(const Coef &p, const float (&u)[G],
                                                    const Vec2 &sp, const Vec2 &s)
    {
        const float cp = sp.x0;
        const Gates q = gates(p, u, cp, sp.x1);
        const float i = q.i, f = q.f, g = q.g, o = q.o, c = q.c, tc = q.tc;
        const float h = o * tc;
        Map2 m;
        m.b0 = c - s.x0;
        m.b1 = h - s.x1;
        // dc'/dc = f
        // dc'/dh = c f(1-f) a_f + g i(1-i) a_i + i (1-g^2) a_g
        // dh'/dc = o (1 - tanh^2 c') f
        // dh'/dh = tanh(c') o(1-o) a_o + o (1 - tanh^2 c') dc'/dh
        // x(1 - x) as one FMA: fma(-x, x, x)
        const float dcdh = fmaf_(cp * fmaf_(-f, f, f), p.af,
                                 fmaf_(g * fmaf_(-i, i, i), p.ai, (i * fmaf_(-g, g, 1.0f)) * p.ag));
        const float ot = o * fmaf_(-tc, tc, 1.0f);
        m.a00 = f;
        m.a01 = dcdh;
        m.a10 = ot * f;
        m.a11 = fmaf_(tc * fmaf_(-o, o, o), p.ao, ot * dcdh);
        return m;
    }
};

}  // namespace pararnn
