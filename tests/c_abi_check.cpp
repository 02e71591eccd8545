// A consumer of libpararnn.so through its C ABI alone (no Python, no torch):
// device buffers come from the HIP runtime, inputs from a small seeded
// generator, and the results are compared with the CPU oracle's C library
// (liboracle.so, fp64 sequential recurrence and back-propagation through
// time).  Checks:
//   1. ParaGRU solve, one block per channel and forced time blocks, with an
//      info record and the workspace pararnn_workspace_bytes asks for;
//   2. ParaLSTM solve;
//   3. ParaGRU adjoint (du, da, dh0) against the oracle's BPTT.
// Prints one line per check; the exit status is the number of failures.
// Test infrastructure: built in-tree by the package build, run by a GPU test.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pararnn.h"

extern "C" {
int oracle_gru_forward(int64_t B, int64_t T, int64_t D, const float *uz, const float *ur,
                       const float *uc, const float *a, const float *h0, double *h,
                       int nthreads);
int oracle_lstm_forward(int64_t B, int64_t T, int64_t D, const float *ui, const float *uf,
                        const float *ug, const float *uo, const float *a, const float *c0,
                        const float *h0, double *c, double *h, int nthreads);
int oracle_gru_bptt(int64_t B, int64_t T, int64_t D, const float *uz, const float *ur,
                    const float *uc, const float *a, const float *h0, const float *dh,
                    double *h, double *duz, double *dur, double *duc, double *da, double *dh0,
                    double *lam, int nthreads);
}

namespace {

int failures = 0;

#define HIP_OK(x)                                                                          \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            std::exit(100);                                                                \
        }                                                                                  \
    } while (0)

// splitmix64 counter generator; normals by the Box-Muller transform
struct Rng {
    uint64_t s;
    uint64_t next()
    {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
    float normal()
    {
        const double u1 = uniform(), u2 = uniform();
        return (float)(std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2));
    }
};

struct Dev {
    void *p = nullptr;
    explicit Dev(size_t bytes) { HIP_OK(hipMalloc(&p, bytes ? bytes : 1)); }
    ~Dev() { (void)hipFree(p); }
    float *f() const { return static_cast<float *>(p); }
};

void put(const Dev &d, const std::vector<float> &h)
{
    HIP_OK(hipMemcpy(d.p, h.data(), h.size() * sizeof(float), hipMemcpyHostToDevice));
}
std::vector<float> get(const Dev &d, size_t n)
{
    std::vector<float> h(n);
    HIP_OK(hipMemcpy(h.data(), d.p, n * sizeof(float), hipMemcpyDeviceToHost));
    return h;
}

void check(const char *what, double err, double bound)
{
    const bool ok = err <= bound;
    std::printf("%-44s max error %.3e (bound %.1e) %s\n", what, err, bound, ok ? "ok" : "FAIL");
    if (!ok) ++failures;
}

double max_abs_diff(const std::vector<float> &g, const std::vector<double> &r)
{
    double m = 0.0;
    for (size_t i = 0; i < g.size(); ++i) m = std::fmax(m, std::fabs((double)g[i] - r[i]));
    return m;
}

pararnn_shape_t dense_shape(int64_t B, int64_t T, int64_t D)
{
    pararnn_shape_t s;
    std::memset(&s, 0, sizeof(s));
    s.B = B;
    s.T = T;
    s.D = D;
    s.u_stride_b = s.s_stride_b = D * T;
    s.u_stride_d = s.s_stride_d = T;
    s.u_stride_t = s.s_stride_t = 1;
    return s;
}

void gru_solve_case(int64_t B, int64_t T, int64_t D, int K, int W, uint64_t seed)
{
    Rng rng{seed};
    const size_t n = (size_t)(B * D * T);
    std::vector<float> u[3], a(3 * D), h0(B * D);
    for (auto &p : u) {
        p.resize(n);
        for (auto &x : p) x = rng.normal();
    }
    for (auto &x : a) x = (float)(2.0 * rng.uniform() - 1.0);
    for (auto &x : h0) x = 0.3f * rng.normal();

    Dev du0(n * 4), du1(n * 4), du2(n * 4), da(a.size() * 4), dh0(h0.size() * 4), dh(n * 4);
    put(du0, u[0]);
    put(du1, u[1]);
    put(du2, u[2]);
    put(da, a);
    put(dh0, h0);
    const pararnn_shape_t sh = dense_shape(B, T, D);
    pararnn_newton_t opt;
    std::memset(&opt, 0, sizeof(opt));
    opt.tol = 1e-6f;
    opt.max_iters = 30;
    opt.steps_per_lane = K;
    opt.waves_per_block = W;
    const size_t wsb = pararnn_workspace_bytes(PARARNN_GRU, &sh, &opt, 0);
    Dev ws(wsb), info(sizeof(pararnn_info_t));
    const void *uu[3] = {du0.p, du1.p, du2.p};
    const pararnn_status_t st = pararnn_solve_gru(&sh, uu, PARARNN_F32, da.f(), dh0.f(), dh.f(),
                                                  &opt, static_cast<pararnn_info_t *>(info.p),
                                                  ws.p, wsb, nullptr);
    if (st != PARARNN_OK) {
        std::printf("pararnn_solve_gru: %s\n", pararnn_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    pararnn_info_t inf;
    HIP_OK(hipMemcpy(&inf, info.p, sizeof(inf), hipMemcpyDeviceToHost));
    std::vector<double> ref(n);
    oracle_gru_forward(B, T, D, u[0].data(), u[1].data(), u[2].data(), a.data(), h0.data(),
                       ref.data(), 0);
    int32_t K_, W_;
    int64_t nb;
    pararnn_plan(PARARNN_GRU, &sh, &opt, 0, &K_, &W_, &nb);
    char what[96];
    std::snprintf(what, sizeof(what), "GRU solve B=%lld T=%lld D=%lld K=%d W=%d blocks=%lld",
                  (long long)B, (long long)T, (long long)D, K_, W_, (long long)nb);
    check(what, max_abs_diff(get(dh, n), ref), 1e-5);
    if (!inf.converged || !(inf.max_abs_res < opt.tol) || inf.units != B * D * nb) {
        std::printf("  info record: converged %d max|r| %.3e units %lld FAIL\n", inf.converged,
                    inf.max_abs_res, (long long)inf.units);
        ++failures;
    }
}

void lstm_solve_case(int64_t B, int64_t T, int64_t D, uint64_t seed)
{
    Rng rng{seed};
    const size_t n = (size_t)(B * D * T);
    std::vector<float> u[4], a(4 * D), c0(B * D, 0.0f), h0(B * D, 0.0f);
    for (int g = 0; g < 4; ++g) {
        u[g].resize(n);
        for (auto &x : u[g]) x = rng.normal() + (g == 1 ? 1.0f : 0.0f);
    }
    for (auto &x : a) x = (float)(2.0 * rng.uniform() - 1.0);
    Dev dug[4] = {Dev(n * 4), Dev(n * 4), Dev(n * 4), Dev(n * 4)};
    for (int g = 0; g < 4; ++g) put(dug[g], u[g]);
    Dev da(a.size() * 4), dc0(c0.size() * 4), dh0(h0.size() * 4), dc(n * 4), dh(n * 4);
    put(da, a);
    put(dc0, c0);
    put(dh0, h0);
    const pararnn_shape_t sh = dense_shape(B, T, D);
    pararnn_newton_t opt;
    std::memset(&opt, 0, sizeof(opt));
    opt.tol = 1e-6f;
    opt.max_iters = 30;
    const size_t wsb = pararnn_workspace_bytes(PARARNN_LSTM, &sh, &opt, 0);
    Dev ws(wsb);
    const void *uu[4] = {dug[0].p, dug[1].p, dug[2].p, dug[3].p};
    const pararnn_status_t st = pararnn_solve_lstm(&sh, uu, PARARNN_F32, da.f(), dc0.f(),
                                                   dh0.f(), dc.f(), dh.f(), &opt, nullptr,
                                                   ws.p, wsb, nullptr);
    if (st != PARARNN_OK) {
        std::printf("pararnn_solve_lstm: %s\n", pararnn_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    std::vector<double> rc(n), rh(n);
    oracle_lstm_forward(B, T, D, u[0].data(), u[1].data(), u[2].data(), u[3].data(), a.data(),
                        c0.data(), h0.data(), rc.data(), rh.data(), 0);
    const double e = std::fmax(max_abs_diff(get(dc, n), rc), max_abs_diff(get(dh, n), rh));
    char what[96];
    std::snprintf(what, sizeof(what), "LSTM solve B=%lld T=%lld D=%lld", (long long)B,
                  (long long)T, (long long)D);
    check(what, e, 1e-5);
}

void gru_adjoint_case(int64_t B, int64_t T, int64_t D, uint64_t seed)
{
    Rng rng{seed};
    const size_t n = (size_t)(B * D * T);
    std::vector<float> u[3], a(3 * D), h0(B * D), g(n);
    for (auto &p : u) {
        p.resize(n);
        for (auto &x : p) x = rng.normal();
    }
    for (auto &x : a) x = (float)(2.0 * rng.uniform() - 1.0);
    for (auto &x : h0) x = 0.3f * rng.normal();
    for (auto &x : g) x = rng.normal();
    // the oracle's trajectory and gradients
    std::vector<double> h(n), duz(n), dur(n), duc(n), dav(3 * D), dh0(B * D);
    oracle_gru_bptt(B, T, D, u[0].data(), u[1].data(), u[2].data(), a.data(), h0.data(),
                    g.data(), h.data(), duz.data(), dur.data(), duc.data(), dav.data(),
                    dh0.data(), nullptr, 0);
    std::vector<float> hf(h.begin(), h.end());
    Dev du[3] = {Dev(n * 4), Dev(n * 4), Dev(n * 4)}, gu[3] = {Dev(n * 4), Dev(n * 4), Dev(n * 4)};
    for (int k = 0; k < 3; ++k) put(du[k], u[k]);
    Dev da(a.size() * 4), dh0d(h0.size() * 4), dh(n * 4), dg(n * 4), gda(a.size() * 4),
        gdh0(h0.size() * 4);
    put(da, a);
    put(dh0d, h0);
    put(dh, hf);
    put(dg, g);
    const pararnn_shape_t sh = dense_shape(B, T, D);
    const size_t wsb = pararnn_workspace_bytes(PARARNN_GRU, &sh, nullptr, 1);
    Dev ws(wsb);
    const void *uu[3] = {du[0].p, du[1].p, du[2].p};
    const float *s0[1] = {dh0d.f()}, *s[1] = {dh.f()}, *gs[1] = {dg.f()};
    float *duo[3] = {gu[0].f(), gu[1].f(), gu[2].f()}, *ds0[1] = {gdh0.f()};
    const pararnn_status_t st = pararnn_adjoint(PARARNN_GRU, &sh, uu, PARARNN_F32, da.f(), s0,
                                                s, gs, nullptr, duo, gda.f(), 0, ds0, nullptr,
                                                nullptr, ws.p, wsb, nullptr);
    if (st != PARARNN_OK) {
        std::printf("pararnn_adjoint: %s\n", pararnn_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    const std::vector<double> *ref[3] = {&duz, &dur, &duc};
    double rel = 0.0;
    auto rel_err = [](const std::vector<float> &got, const std::vector<double> &r) {
        double scale = 1.0;
        for (double x : r) scale = std::fmax(scale, std::fabs(x));
        return max_abs_diff(got, r) / scale;
    };
    for (int k = 0; k < 3; ++k) rel = std::fmax(rel, rel_err(get(gu[k], n), *ref[k]));
    rel = std::fmax(rel, rel_err(get(gda, a.size()), dav));
    rel = std::fmax(rel, rel_err(get(gdh0, h0.size()), dh0));
    char what[96];
    std::snprintf(what, sizeof(what), "GRU adjoint B=%lld T=%lld D=%lld (relative)",
                  (long long)B, (long long)T, (long long)D);
    check(what, rel, 1e-5);
}

}  // namespace

int main()
{
    gru_solve_case(2, 1000, 24, 0, 0, 11);
    gru_solve_case(2, 3000, 8, 8, 2, 12);  // three time blocks per channel
    gru_solve_case(1, 1, 5, 0, 0, 13);
    lstm_solve_case(2, 2049, 16, 14);
    gru_adjoint_case(2, 1500, 12, 15);
    std::printf("%d failure(s)\n", failures);
    return failures;
}
