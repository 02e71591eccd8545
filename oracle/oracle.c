/*
 * ORACLE — test infrastructure only.
 *
 * Plain, slow, sequential fp64 reference for the ParaGRU / ParaLSTM cells.
 * Only the test suite, the smoke check and the CPU-baseline leg of the bench
 * may load this library; the product path never calls it.  It shares no code
 * with the HIP path.
 *
 * What it computes
 * ----------------
 * "Параллельность RNN?" (forpes.ru), §1.1: the true trajectory s*_1..s*_T is
 * the unique zero of the DEER residual r_t = s_t - f(s_{t-1}), and it is what
 * one gets by applying the transition step by step from s_0.  Newton's method
 * on r therefore converges to exactly this sequence; the oracle is that plain
 * definition written out: s_t = f(s_{t-1}, u_t), t = 1..T, one channel at a
 * time, in double precision.
 *
 * The cells (the pages fix only their structure — GRU / LSTM whose recurrent
 * matrices are diagonal, so the Jacobian is diagonal, resp. 2x2 block
 * diagonal: voguetech.ru ParaRNN article, "Что именно сделали технически",
 * item 3; the exact per-channel formulas are those of the workload
 * definitions):
 *   ParaGRU  z = sig(a_z h + u_z), r = sig(a_r h + u_r),
 *            c = tanh(a_c (r h) + u_c),  h' = (1 - z) h + z c
 *   ParaLSTM i,f,o = sig(a_* h + u_*), g = tanh(a_g h + u_g),
 *            c' = f c + i g,  h' = o tanh(c')
 * with sig(x) = 1 / (1 + exp(-x)).  u_* are the precomputed input
 * projections of x_t, a_* the diagonal recurrent weights.
 *
 * The backward oracle is ordinary back-propagation through time of the
 * scalar loss L = sum_t <dL/dh_t, h_t> (+ <dL/dc_t, c_t> for the LSTM),
 * through the same sequential loop, chain rule applied step by step.
 *
 * Layout: every per-time-step plane is [B][D][T] contiguous (T fastest);
 * the diagonal weights are [G][D]; initial states are [B][D].  Inputs are
 * float32 (exactly the values the device path consumes); all arithmetic and
 * all outputs are double.  Channels (b, d) are independent, so the only
 * parallelism is an OpenMP loop over channels; every channel is sequential
 * in t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sig(double x) { return 1.0 / (1.0 + exp(-x)); }

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- GRU --- */

/* h: [B][D][T] out.  a: [3][D] (z, r, c). */
int oracle_gru_forward(int64_t B, int64_t T, int64_t D,
                       const float *uz, const float *ur, const float *uc,
                       const float *a, const float *h0, double *h,
                       int nthreads)
{
    if (B < 0 || T < 0 || D < 0) return 1;
    set_threads(nthreads);
    const int64_t nch = B * D;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t ch = 0; ch < nch; ++ch) {
        const int64_t d = ch % D;
        const double az = a[0 * D + d], ar = a[1 * D + d], ac = a[2 * D + d];
        const float *pz = uz + ch * T, *pr = ur + ch * T, *pc = uc + ch * T;
        double *out = h + ch * T;
        double hp = h0[ch];
        for (int64_t t = 0; t < T; ++t) {
            const double z = sig(az * hp + pz[t]);
            const double r = sig(ar * hp + pr[t]);
            const double c = tanh(ac * (r * hp) + pc[t]);
            const double hn = (1.0 - z) * hp + z * c;
            out[t] = hn;
            hp = hn;
        }
    }
    return 0;
}

/* Back-propagation through time for the GRU.
 * dh: [B][D][T] upstream dL/dh_t (float32).
 * Outputs (double): h [B][D][T] (forward states, may be NULL),
 * du_z, du_r, du_c [B][D][T], da [3][D] (summed over batch and time),
 * dh0 [B][D], lam [B][D][T] = total dL/dh_t (may be NULL). */
int oracle_gru_bptt(int64_t B, int64_t T, int64_t D,
                    const float *uz, const float *ur, const float *uc,
                    const float *a, const float *h0, const float *dh,
                    double *h, double *duz, double *dur, double *duc,
                    double *da, double *dh0, double *lam_out, int nthreads)
{
    if (B < 0 || T < 0 || D < 0) return 1;
    set_threads(nthreads);
    const int64_t nch = B * D;
    double *da_ch = (double *)calloc((size_t)(nch > 0 ? nch : 1) * 3, sizeof(double));
    if (!da_ch) return 2;
    int fail = 0;
#pragma omp parallel
    {
        double *hs = (double *)malloc((size_t)(T + 1) * sizeof(double));
        if (!hs) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t ch = 0; ch < nch; ++ch) {
            if (!hs) continue;
            const int64_t d = ch % D;
            const double az = a[0 * D + d], ar = a[1 * D + d], ac = a[2 * D + d];
            const float *pz = uz + ch * T, *pr = ur + ch * T, *pc = uc + ch * T;
            const float *g = dh + ch * T;
            /* forward, keeping every state (hs[t] = h_t, hs[0] = h_0) */
            hs[0] = h0[ch];
            for (int64_t t = 1; t <= T; ++t) {
                const double hp = hs[t - 1];
                const double z = sig(az * hp + pz[t - 1]);
                const double r = sig(ar * hp + pr[t - 1]);
                const double c = tanh(ac * (r * hp) + pc[t - 1]);
                hs[t] = (1.0 - z) * hp + z * c;
            }
            if (h) memcpy(h + ch * T, hs + 1, (size_t)T * sizeof(double));
            /* reverse sweep: lam = dL/dh_t including the path through h_{t+1} */
            double carry = 0.0, gz = 0.0, gr = 0.0, gc = 0.0;
            for (int64_t t = T; t >= 1; --t) {
                const double hp = hs[t - 1];
                const double z = sig(az * hp + pz[t - 1]);
                const double r = sig(ar * hp + pr[t - 1]);
                const double q = r * hp;
                const double c = tanh(ac * q + pc[t - 1]);
                const double lam = (double)g[t - 1] + carry;
                /* h_t = h_{t-1} + z (c - h_{t-1}) */
                const double dz = lam * (c - hp);
                const double dc = lam * z;
                const double dpz = dz * z * (1.0 - z);
                const double dpc = dc * (1.0 - c * c);
                const double dq = dpc * ac;
                const double dr = dq * hp;
                const double dpr = dr * r * (1.0 - r);
                const double dhp = lam * (1.0 - z) + dpz * az + dq * r + dpr * ar;
                const int64_t i = ch * T + (t - 1);
                if (lam_out) lam_out[i] = lam;
                duz[i] = dpz;
                dur[i] = dpr;
                duc[i] = dpc;
                gz += dpz * hp;
                gr += dpr * hp;
                gc += dpc * q;
                carry = dhp;
            }
            dh0[ch] = carry;
            da_ch[3 * ch + 0] = gz;
            da_ch[3 * ch + 1] = gr;
            da_ch[3 * ch + 2] = gc;
        }
        free(hs);
    }
    if (fail) { free(da_ch); return 2; }
    /* fixed-order reduction over the batch */
    for (int64_t k = 0; k < 3 * D; ++k) da[k] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int k = 0; k < 3; ++k) da[k * D + d] += da_ch[3 * (b * D + d) + k];
    free(da_ch);
    return 0;
}

/* --------------------------------------------------------------- LSTM --- */

/* c, h: [B][D][T] out.  a: [4][D] (i, f, g, o). */
int oracle_lstm_forward(int64_t B, int64_t T, int64_t D,
                        const float *ui, const float *uf, const float *ug,
                        const float *uo, const float *a, const float *c0,
                        const float *h0, double *c, double *h, int nthreads)
{
    if (B < 0 || T < 0 || D < 0) return 1;
    set_threads(nthreads);
    const int64_t nch = B * D;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t ch = 0; ch < nch; ++ch) {
        const int64_t d = ch % D;
        const double ai = a[0 * D + d], af = a[1 * D + d];
        const double ag = a[2 * D + d], ao = a[3 * D + d];
        const float *pi = ui + ch * T, *pf = uf + ch * T;
        const float *pg = ug + ch * T, *po = uo + ch * T;
        double cp = c0[ch], hp = h0[ch];
        for (int64_t t = 0; t < T; ++t) {
            const double ig = sig(ai * hp + pi[t]);
            const double fg = sig(af * hp + pf[t]);
            const double gg = tanh(ag * hp + pg[t]);
            const double og = sig(ao * hp + po[t]);
            const double cn = fg * cp + ig * gg;
            const double hn = og * tanh(cn);
            c[ch * T + t] = cn;
            h[ch * T + t] = hn;
            cp = cn;
            hp = hn;
        }
    }
    return 0;
}

/* Back-propagation through time for the LSTM.
 * dh: [B][D][T] upstream dL/dh_t; dc: upstream dL/dc_t or NULL (= 0).
 * Outputs (double): c, h forward states (each may be NULL),
 * du[4] planes [B][D][T] (i, f, g, o), da [4][D], dc0, dh0 [B][D],
 * lam_c, lam_h [B][D][T] = total dL/dc_t, dL/dh_t (each may be NULL). */
int oracle_lstm_bptt(int64_t B, int64_t T, int64_t D,
                     const float *ui, const float *uf, const float *ug,
                     const float *uo, const float *a, const float *c0,
                     const float *h0, const float *dh, const float *dc,
                     double *c, double *h, double *dui, double *duf,
                     double *dug, double *duo, double *da, double *dc0,
                     double *dh0, double *lamc_out, double *lamh_out,
                     int nthreads)
{
    if (B < 0 || T < 0 || D < 0) return 1;
    set_threads(nthreads);
    const int64_t nch = B * D;
    double *da_ch = (double *)calloc((size_t)(nch > 0 ? nch : 1) * 4, sizeof(double));
    if (!da_ch) return 2;
    int fail = 0;
#pragma omp parallel
    {
        double *cs = (double *)malloc((size_t)(T + 1) * sizeof(double));
        double *hs = (double *)malloc((size_t)(T + 1) * sizeof(double));
        if (!cs || !hs) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t ch = 0; ch < nch; ++ch) {
            if (!cs || !hs) continue;
            const int64_t d = ch % D;
            const double ai = a[0 * D + d], af = a[1 * D + d];
            const double ag = a[2 * D + d], ao = a[3 * D + d];
            const float *pi = ui + ch * T, *pf = uf + ch * T;
            const float *pg = ug + ch * T, *po = uo + ch * T;
            cs[0] = c0[ch];
            hs[0] = h0[ch];
            for (int64_t t = 1; t <= T; ++t) {
                const double cp = cs[t - 1], hp = hs[t - 1];
                const double ig = sig(ai * hp + pi[t - 1]);
                const double fg = sig(af * hp + pf[t - 1]);
                const double gg = tanh(ag * hp + pg[t - 1]);
                const double og = sig(ao * hp + po[t - 1]);
                cs[t] = fg * cp + ig * gg;
                hs[t] = og * tanh(cs[t]);
            }
            if (c) memcpy(c + ch * T, cs + 1, (size_t)T * sizeof(double));
            if (h) memcpy(h + ch * T, hs + 1, (size_t)T * sizeof(double));
            double carry_c = 0.0, carry_h = 0.0;
            double gi = 0.0, gf = 0.0, gg_ = 0.0, go = 0.0;
            for (int64_t t = T; t >= 1; --t) {
                const double cp = cs[t - 1], hp = hs[t - 1];
                const double ig = sig(ai * hp + pi[t - 1]);
                const double fg = sig(af * hp + pf[t - 1]);
                const double gg = tanh(ag * hp + pg[t - 1]);
                const double og = sig(ao * hp + po[t - 1]);
                const double cn = fg * cp + ig * gg;
                const double tc = tanh(cn);
                const int64_t idx = ch * T + (t - 1);
                const double lam_h = (double)dh[idx] + carry_h;
                const double lam_c = (dc ? (double)dc[idx] : 0.0) + carry_c;
                if (lamc_out) lamc_out[idx] = lam_c;
                if (lamh_out) lamh_out[idx] = lam_h;
                /* h_t = o tanh(c_t): gradient reaching c_t in total */
                const double ec = lam_c + lam_h * og * (1.0 - tc * tc);
                const double dpo = lam_h * tc * og * (1.0 - og);
                const double dpi = ec * gg * ig * (1.0 - ig);
                const double dpf = ec * cp * fg * (1.0 - fg);
                const double dpg = ec * ig * (1.0 - gg * gg);
                dui[idx] = dpi;
                duf[idx] = dpf;
                dug[idx] = dpg;
                duo[idx] = dpo;
                gi += dpi * hp;
                gf += dpf * hp;
                gg_ += dpg * hp;
                go += dpo * hp;
                carry_c = ec * fg;
                carry_h = dpi * ai + dpf * af + dpg * ag + dpo * ao;
            }
            dc0[ch] = carry_c;
            dh0[ch] = carry_h;
            da_ch[4 * ch + 0] = gi;
            da_ch[4 * ch + 1] = gf;
            da_ch[4 * ch + 2] = gg_;
            da_ch[4 * ch + 3] = go;
        }
        free(cs);
        free(hs);
    }
    if (fail) { free(da_ch); return 2; }
    for (int64_t k = 0; k < 4 * D; ++k) da[k] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int k = 0; k < 4; ++k) da[k * D + d] += da_ch[4 * (b * D + d) + k];
    free(da_ch);
    return 0;
}
