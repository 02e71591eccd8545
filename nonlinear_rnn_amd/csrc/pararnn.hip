// libpararnn.so — host side of the C ABI declared in include/pararnn.h:
// argument checks, tiling plan, workspace layout and kernel dispatch.  No
// entry point allocates, frees or synchronises; everything is enqueued on
// the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>

#define PARARNN_DEFINE_AUX_KERNELS
#include "launch.hpp"
#include "pararnn.h"

using namespace pararnn;

namespace {

constexpr int64_t kMaxIters = 1 << 20;  // flag encoding leaves room below kStopBase
constexpr size_t kAlign = 256;
constexpr int64_t kComputeUnits = 256;  // MI355X

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

struct Plan {
    int K = 0, W = 0;
    int64_t P = 0, nb = 1;
    int64_t channels = 0, units = 0;
};

int cell_S(pararnn_cell_t c) { return c == PARARNN_LSTM ? 2 : 1; }
int cell_G(pararnn_cell_t c) { return c == PARARNN_LSTM ? 4 : 3; }
int rec_floats(pararnn_cell_t c) { return c == PARARNN_LSTM ? MapRec<Map2>::kFloats : MapRec<Map1>::kFloats; }

// Elements (b, d, t) of a plane must not overlap: with the dimensions of
// extent > 1 taken in increasing stride, each stride must exceed the largest
// offset the smaller ones reach.  Covers channel-major [B][D][T], time-major
// [B][T][D] and any padded or permuted variant of them.
bool planes_disjoint(int64_t B, int64_t T, int64_t D, int64_t sb, int64_t sd, int64_t st)
{
    if (sb < 0 || sd < 0 || st < 0) return false;
    if (B == 0 || D == 0 || T == 0) return true;  // no elements
    int64_t n[3] = {B, D, T}, str[3] = {sb, sd, st};
    for (int i = 0; i < 3; ++i)  // sort by stride
        for (int j = i + 1; j < 3; ++j)
            if (str[j] < str[i]) {
                std::swap(str[i], str[j]);
                std::swap(n[i], n[j]);
            }
    __int128 reach = 0;  // largest offset of the smaller dimensions
    for (int i = 0; i < 3; ++i) {
        if (n[i] <= 1) continue;
        if ((__int128)str[i] <= reach) return false;
        reach += (__int128)str[i] * (n[i] - 1);
        if (reach > (__int128)INT64_MAX) return false;
    }
    return true;
}

pararnn_status_t check_shape(const pararnn_shape_t *sh)
{
    if (!sh) return PARARNN_ERR_INVALID;
    if (sh->B < 0 || sh->T < 0 || sh->D < 0) return PARARNN_ERR_INVALID;
    if (sh->B > (int64_t(1) << 31) || sh->D > (int64_t(1) << 31) || sh->T > (int64_t(1) << 40))
        return PARARNN_ERR_UNSUPPORTED;
    if (!planes_disjoint(sh->B, sh->T, sh->D, sh->u_stride_b, sh->u_stride_d, sh->u_stride_t))
        return PARARNN_ERR_INVALID;
    if (!planes_disjoint(sh->B, sh->T, sh->D, sh->s_stride_b, sh->s_stride_d, sh->s_stride_t))
        return PARARNN_ERR_INVALID;
    return PARARNN_OK;
}

bool opt_k_w_unset(const pararnn_newton_t *opt)
{
    return !opt || (opt->steps_per_lane == 0 && opt->waves_per_block == 0);
}

// Default tiling: the smallest block capacity P = 64 W K that covers T, from
// a list ordered by preference; past the largest one, several time blocks
// per channel.
// kind: 0 = Newton solve, 1 = adjoint, 2 = standalone scan (cell selects the
// state size: GRU 1, LSTM 2).
pararnn_status_t make_plan(pararnn_cell_t cell, const pararnn_shape_t *sh,
                           const pararnn_newton_t *opt, int kind, Plan &pl)
{
    const bool adjoint = kind != 0;
    pararnn_status_t st = check_shape(sh);
    if (st != PARARNN_OK) return st;
    int K = opt ? opt->steps_per_lane : 0;
    int W = opt ? opt->waves_per_block : 0;
    if ((K != 0 && !pow2_in(K, 1, 32)) || (W != 0 && !pow2_in(W, 1, 8)))
        return PARARNN_ERR_UNSUPPORTED;
    if (K == 0 || W == 0) {
        static const int gru_kw[][2] = {{16, 4}, {16, 2}, {16, 1}, {8, 1}, {4, 1}, {2, 1}, {1, 1}};
        static const int lstm_kw[][2] = {{16, 4}, {16, 2}, {16, 1}, {8, 1}, {4, 1}, {2, 1}, {1, 1}};
        static const int adj_kw[][2] = {{8, 4}, {8, 2}, {8, 1}, {4, 1}, {2, 1}, {1, 1}};
        // One pass and no Newton state: the scan keeps a channel in one
        // workgroup as long as it can (up to 8192 steps), since a time-block
        // hand-off costs more than the rest of the pass.
        static const int scan_kw[][2] = {{16, 8}, {8, 8}, {8, 4}, {8, 2},
                                         {8, 1},  {4, 1}, {2, 1}, {1, 1}};
        const int(*tab)[2] =
            kind == 2 ? scan_kw : adjoint ? adj_kw : (cell == PARARNN_LSTM ? lstm_kw : gru_kw);
        const int n = kind == 2 ? 8 : adjoint ? 6 : 7;
        int pick = 0;
        for (int i = 0; i < n; ++i) {
            const int kk = K ? K : tab[i][0], ww = W ? W : tab[i][1];
            if ((int64_t)kWave * kk * ww >= sh->T) pick = i;
        }
        if (K == 0) K = tab[pick][0];
        if (W == 0) W = tab[pick][1];
        // Few ParaGRU channels on a very long sequence: a channel's blocks run
        // side by side and look back every iteration over all their
        // predecessors, so fewer, longer blocks (8192 steps, K = 16, W = 8)
        // pay off once there are more than 8 of 4096 steps (B=1 D=64:
        // T=65536 0.085 -> 0.075 ms, T=262144 0.297 -> 0.188 ms; at
        // T=16384, and with 1024 channels, 4096-step blocks stay faster).
        if (kind == 0 && cell == PARARNN_GRU && opt_k_w_unset(opt) && K == 16 && W == 4 &&
            sh->T > 8 * (int64_t)kWave * 16 * 4 && sh->B * sh->D < kTicketGroup)
            W = 8;
        // Past 4096 steps a channel takes time blocks of 4096 steps (K = 16,
        // W = 4): a block whose predecessors are done loads all their carries
        // at once, so more, smaller blocks cost little and hide each other's
        // loads better (ParaGRU bf16-u B=4 T=16384 D=4096: 4 blocks of 4096
        // steps 1.36 ms, 2 blocks of 8192 steps 1.46 ms, 8 blocks of 2048
        // steps 1.61 ms).
        // Few channels in one block each: spread every channel over more
        // waves at the same capacity (half the steps per lane, twice the
        // waves) until the solve has about two waves per CU.  Each lane's
        // serial chain per Newton pass shortens; nothing else changes.
        if (kind == 0 && opt_k_w_unset(opt) && sh->T <= (int64_t)kWave * K * W) {
            const int64_t channels = sh->B * sh->D;
            while (K > 4 && W < 8 && channels * W < 2 * kComputeUnits) {
                K /= 2;
                W *= 2;
            }
        }
    }
    const bool lstm = cell == PARARNN_LSTM;
    if (adjoint ? !adjoint_tiling_built(lstm, K, W) : !newton_tiling_built(lstm, K, W))
        return PARARNN_ERR_UNSUPPORTED;
    pl.K = K;
    pl.W = W;
    pl.P = (int64_t)kWave * K * W;
    pl.nb = sh->T > 0 ? (sh->T + pl.P - 1) / pl.P : 1;
    pl.channels = sh->B * sh->D;
    pl.units = pl.channels * pl.nb;
    // dispatch packets count work-items in 32 bits
    const int64_t groups = ((pl.channels + 7) / 8) * 8 * pl.nb;
    if (groups * kWave * W >= (int64_t(1) << 32)) return PARARNN_ERR_UNSUPPORTED;
    if (pl.nb >= kStopBase) return PARARNN_ERR_UNSUPPORTED;
    return PARARNN_OK;
}

// Solve workspace: the time-block hand-off of a multi-block solve (ticket,
// flags, per-iteration block records, warm-start boundary states), then the
// per-unit convergence records the info fold reads (needed only when an info
// record is requested).
struct SolveWs {
    size_t ticket = 0, flags = 0, records = 0, hin0 = 0;
    size_t multi = 0;      // bytes of the hand-off part (0 with one block per channel
                           // and for block-sequential solves)
    size_t unit_info = 0;  // offset of the per-unit records, 8 bytes a unit
    size_t total = 0;
};

// With a full ticket group of channels (more workgroups than the device
// holds at once) every workgroup solves one channel's time blocks one after
// the other, each from its predecessor's converged last state: no
// per-iteration carries, tickets or flags, so no hand-off workspace.  With
// fewer channels a channel's blocks run side by side, in workgroups of their
// own, as one Newton iteration over the whole sequence.
bool block_sequential(const Plan &pl)
{
    return pl.nb > 1 && (pl.channels + 7) / 8 * 8 >= kTicketGroup && newton_seq_built(pl.K, pl.W);
}

SolveWs solve_ws_layout(pararnn_cell_t cell, const Plan &pl, const pararnn_newton_t *opt)
{
    SolveWs w;
    size_t off = 0;
    if (pl.nb > 1 && !block_sequential(pl)) {
        const int64_t cap = opt ? opt->max_iters : 0;
        w.ticket = off;
        off += kAlign;
        w.flags = off;
        off = align_up(off + (size_t)pl.units * sizeof(int32_t));
        w.records = off;
        off = align_up(off +
                       (size_t)pl.units * (size_t)(cap + 1) * rec_floats(cell) * sizeof(float));
        if (opt && opt->init_from_output) {
            w.hin0 = off;
            off = align_up(off + (size_t)pl.units * cell_S(cell) * sizeof(float));
        }
        w.multi = off;
    }
    w.unit_info = off;
    if (pl.units > 0) off = align_up(off + (size_t)pl.units * 2 * sizeof(uint32_t));
    w.total = off;
    return w;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pararnn_status_t check_newton(const pararnn_newton_t *opt)
{
    if (!opt) return PARARNN_ERR_INVALID;
    if (!(opt->tol >= 0.0f) || std::isinf(opt->tol)) return PARARNN_ERR_INVALID;
    if (opt->max_iters < 0 || opt->max_iters > kMaxIters) return PARARNN_ERR_INVALID;
    if (opt->init_from_output != 0 && opt->init_from_output != 1) return PARARNN_ERR_INVALID;
    return PARARNN_OK;
}

pararnn_status_t solve_core(pararnn_cell_t cell, const pararnn_shape_t *sh, const void *const *u,
                            pararnn_dtype_t dt, const float *a, const float *const *s0,
                            float *const *s, const pararnn_newton_t *opt, pararnn_info_t *info,
                            void *ws, size_t ws_bytes, void *stream)
{
    pararnn_status_t st = check_newton(opt);
    if (st != PARARNN_OK) return st;
    Plan pl;
    st = make_plan(cell, sh, opt, 0, pl);
    if (st != PARARNN_OK) return st;
    if (dt != PARARNN_F32 && dt != PARARNN_BF16) return PARARNN_ERR_UNSUPPORTED;
    const int G = cell_G(cell), S = cell_S(cell);
    const bool work = pl.channels > 0 && sh->T > 0;
    if (work) {
        if (!u || !a || !s0 || !s) return PARARNN_ERR_INVALID;
        for (int g = 0; g < G; ++g)
            if (!u[g]) return PARARNN_ERR_INVALID;
        for (int c = 0; c < S; ++c)
            if (!s0[c] || !s[c]) return PARARNN_ERR_INVALID;
    }
    const SolveWs wl = solve_ws_layout(cell, pl, opt);
    const size_t need = info ? wl.total : wl.multi;
    if (work && need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return PARARNN_ERR_WORKSPACE;
    hipStream_t strm = static_cast<hipStream_t>(stream);

    SolveArgs A;
    std::memset(&A, 0, sizeof(A));
    for (int g = 0; g < G && work; ++g) A.u[g] = u[g];
    A.a = a;
    for (int c = 0; c < S && work; ++c) {
        A.s0[c] = s0[c];
        A.s[c] = s[c];
    }
    A.B = sh->B;
    A.T = sh->T;
    A.D = sh->D;
    A.usb = sh->u_stride_b;
    A.usd = sh->u_stride_d;
    A.ssb = sh->s_stride_b;
    A.ssd = sh->s_stride_d;
    A.ust = sh->u_stride_t;
    A.sst = sh->s_stride_t;
    A.channels = pl.channels;
    A.tol = opt->tol;
    A.guess_tol = std::sqrt(opt->tol);
    A.cap = opt->max_iters;
    A.nb = (int32_t)pl.nb;
    A.init_from_output = opt->init_from_output;
    const int ve = dt == PARARNN_BF16 ? 8 : 4;
    bool uv = sh->u_stride_t == 1 && (sh->T % ve == 0) && (sh->u_stride_b % ve == 0) &&
              (sh->u_stride_d % ve == 0);
    for (int g = 0; g < G && work; ++g) uv = uv && aligned16(u[g]);
    bool sv = sh->s_stride_t == 1 && (sh->T % 4 == 0) && (sh->s_stride_b % 4 == 0) &&
              (sh->s_stride_d % 4 == 0);
    for (int c = 0; c < S && work; ++c) sv = sv && aligned16(s[c]);
    A.u_vec = uv ? 1 : 0;
    A.s_vec = sv ? 1 : 0;
    char *base = static_cast<char *>(ws);
    if (work && wl.multi > 0) {
        A.ticket = reinterpret_cast<uint32_t *>(base + wl.ticket);
        A.flags = reinterpret_cast<int32_t *>(base + wl.flags);
        A.records = reinterpret_cast<float *>(base + wl.records);
        A.hin0 = opt->init_from_output ? reinterpret_cast<float *>(base + wl.hin0) : nullptr;
    }
    if (work && info) A.unit_info = reinterpret_cast<uint32_t *>(base + wl.unit_info);
    uint32_t tolb;
    std::memcpy(&tolb, &opt->tol, sizeof(tolb));
    const auto fold_info = [&]() -> pararnn_status_t {
        if (!info) return PARARNN_OK;
        hipLaunchKernelGGL(info_fold_kernel, dim3(1), dim3(kFoldThreads), 0, strm,
                           A.unit_info, work ? pl.units : (int64_t)0, tolb, info);
        return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
    };
    if (!work) return fold_info();

    const bool seq = block_sequential(pl);
    if (pl.nb > 1 && !seq) {
        const int tpb = 256;
        hipLaunchKernelGGL(solve_init_kernel, dim3((unsigned)((pl.units + tpb - 1) / tpb)),
                           dim3(tpb), 0, strm, A, S, pl.units, (int32_t)pl.P);
        if (hipGetLastError() != hipSuccess) return PARARNN_ERR_HIP;
    }
    const int64_t groups = ((pl.channels + 7) / 8) * 8 * (seq ? 1 : pl.nb);
    const int variant = sh->T % pl.P != 0 ? (seq ? kNewtonAnySeq : kNewtonAny)
                        : pl.nb == 1      ? kNewtonFullSingle
                                          : (seq ? kNewtonFullSeq : kNewtonFull);
    hipError_t e;
    if (cell == PARARNN_GRU)
        e = dt == PARARNN_BF16 ? launch_newton_gru_bf16(pl.K, pl.W, variant, groups, strm, A)
                               : launch_newton_gru_f32(pl.K, pl.W, variant, groups, strm, A);
    else
        e = dt == PARARNN_BF16 ? launch_newton_lstm_bf16(pl.K, pl.W, variant, groups, strm, A)
                               : launch_newton_lstm_f32(pl.K, pl.W, variant, groups, strm, A);
    if (e != hipSuccess) return PARARNN_ERR_HIP;
    return fold_info();
}

// ------------------------------------------------- time-major staging ---
// Planes that are not time-contiguous (time-major [B][T][D] and the like)
// are read by the solve with one 4-byte load per step.  With room in the
// workspace they are staged instead: copied into channel-major scratch by
// plane_transpose_kernel, solved there, and the states copied back.
struct Stage {
    bool u = false, s = false;
    size_t u_off = 0, u_plane = 0, s_off = 0, s_plane = 0, total = 0;
};

Stage stage_layout(pararnn_cell_t cell, const pararnn_shape_t *sh, size_t u_esize, size_t base)
{
    Stage g;
    if (!sh || sh->B <= 0 || sh->D <= 0 || sh->T <= 1) return g;
    const int64_t n = sh->B * sh->D;
    if (n > (int64_t(1) << 40) / sh->T) return g;  // no staging for absurd sizes
    const int64_t e = n * sh->T;
    g.u = sh->u_stride_t != 1;
    g.s = sh->s_stride_t != 1;
    if (!g.u && !g.s) return g;
    size_t off = align_up(base);
    if (g.u) {
        g.u_off = off;
        g.u_plane = align_up((size_t)e * u_esize);
        off += (size_t)cell_G(cell) * g.u_plane;
    }
    if (g.s) {
        g.s_off = off;
        g.s_plane = align_up((size_t)e * sizeof(float));
        off += (size_t)cell_S(cell) * g.s_plane;
    }
    g.total = off;
    return g;
}

// Staging room of the adjoint for planes that are not time-contiguous:
// u-family (u in, du out) and s-family (s and dL/ds in, lambda out).
struct AdjStage {
    bool u = false, s = false;
    size_t u_off = 0, u_plane = 0, du_off = 0, f_plane = 0, s_off = 0, gs_off = 0, lam_off = 0,
           total = 0;
};

AdjStage adj_stage_layout(pararnn_cell_t cell, const pararnn_shape_t *sh, size_t u_esize,
                          size_t base)
{
    AdjStage g;
    if (!sh || sh->B <= 0 || sh->D <= 0 || sh->T <= 1) return g;
    const int64_t n = sh->B * sh->D;
    if (n > (int64_t(1) << 40) / sh->T) return g;
    const int64_t e = n * sh->T;
    g.u = sh->u_stride_t != 1;
    g.s = sh->s_stride_t != 1;
    if (!g.u && !g.s) return g;
    const size_t G = cell_G(cell), S = cell_S(cell);
    g.f_plane = align_up((size_t)e * sizeof(float));
    size_t off = align_up(base);
    if (g.u) {
        g.u_plane = align_up((size_t)e * u_esize);
        g.u_off = off;
        off += G * g.u_plane;
        g.du_off = off;
        off += G * g.f_plane;
    }
    if (g.s) {
        g.s_off = off;
        off += S * g.f_plane;
        g.gs_off = off;
        off += S * g.f_plane;
        g.lam_off = off;
        off += S * g.f_plane;
    }
    g.total = off;
    return g;
}

// Whether a plane with strides (sd, st) is walked faster along t than d.
int32_t t_fast(int64_t sd, int64_t st) { return st == 1 ? 1 : sd == 1 ? 0 : (st <= sd ? 1 : 0); }

hipError_t launch_transpose(int esize, const TransArgs &t, hipStream_t st)
{
    const int64_t groups = transpose_groups(t.B, t.T, t.D);
    if (groups == 0) return hipSuccess;
    if (esize == 2) {
        TransArgs t2 = t;
        t2.vec = 0;
        hipLaunchKernelGGL(plane_transpose_kernel<2>, dim3((unsigned)groups), dim3(256), 0, st, t2);
    } else {
        hipLaunchKernelGGL(plane_transpose_kernel<4>, dim3((unsigned)groups), dim3(256), 0, st, t);
    }
    return hipGetLastError();
}

TransArgs plane_copy(const void *src, const pararnn_shape_t *sh, int64_t sb, int64_t sd, int64_t st,
                     void *dst, int64_t db, int64_t dd, int64_t dt)
{
    TransArgs t;
    t.src = src;
    t.dst = dst;
    t.B = sh->B;
    t.T = sh->T;
    t.D = sh->D;
    t.ssb = sb;
    t.ssd = sd;
    t.sst = st;
    t.dsb = db;
    t.dsd = dd;
    t.dstt = dt;
    t.src_t_fast = t_fast(sd, st);
    t.dst_t_fast = t_fast(dd, dt);
    // 16-byte path: unit stride along each side's fast dimension, the other
    // strides multiples of 4 elements, 16-byte aligned bases (4-byte
    // elements only; the launcher ignores it for 2-byte ones)
    const auto side_ok = [](const void *p, int64_t sb, int64_t sd, int64_t st, int32_t tf) {
        const int64_t unit = tf ? st : sd, other = tf ? sd : st;
        return unit == 1 && other % 4 == 0 && sb % 4 == 0 && aligned16(p);
    };
    t.vec = side_ok(src, sb, sd, st, t.src_t_fast) && side_ok(dst, db, dd, dt, t.dst_t_fast);
    return t;
}

pararnn_status_t solve_common(pararnn_cell_t cell, const pararnn_shape_t *sh, const void *const *u,
                              pararnn_dtype_t dt, const float *a, const float *const *s0,
                              float *const *s, const pararnn_newton_t *opt, pararnn_info_t *info,
                              void *ws, size_t ws_bytes, void *stream)
{
    pararnn_status_t st = check_newton(opt);
    if (st != PARARNN_OK) return st;
    Plan pl;
    st = make_plan(cell, sh, opt, 0, pl);
    if (st != PARARNN_OK) return st;
    if (dt != PARARNN_F32 && dt != PARARNN_BF16) return PARARNN_ERR_UNSUPPORTED;
    const int G = cell_G(cell), S = cell_S(cell);
    const size_t esize = dt == PARARNN_BF16 ? 2 : 4;
    const Stage sg = stage_layout(cell, sh, esize, solve_ws_layout(cell, pl, opt).total);
    const bool staged = sg.total > 0 && ws && ws_bytes >= sg.total && aligned16(ws) && u && s;
    if (!staged) return solve_core(cell, sh, u, dt, a, s0, s, opt, info, ws, ws_bytes, stream);
    for (int g = 0; g < G && sg.u; ++g)
        if (!u[g]) return PARARNN_ERR_INVALID;
    for (int c = 0; c < S; ++c)
        if (!s[c]) return PARARNN_ERR_INVALID;

    hipStream_t strm = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    const int64_t dT = sh->T, dDT = sh->D * sh->T;  // dense channel-major strides
    pararnn_shape_t sh2 = *sh;
    const void *u2[4] = {nullptr, nullptr, nullptr, nullptr};
    float *s2[2] = {nullptr, nullptr};
    for (int g = 0; g < G; ++g) {
        u2[g] = u[g];
        if (!sg.u) continue;
        u2[g] = base + sg.u_off + (size_t)g * sg.u_plane;
        const TransArgs t = plane_copy(u[g], sh, sh->u_stride_b, sh->u_stride_d, sh->u_stride_t,
                                       const_cast<void *>(u2[g]), dDT, dT, 1);
        if (launch_transpose((int)esize, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
    }
    if (sg.u) {
        sh2.u_stride_b = dDT;
        sh2.u_stride_d = dT;
        sh2.u_stride_t = 1;
    }
    for (int c = 0; c < S; ++c) {
        s2[c] = s[c];
        if (!sg.s) continue;
        s2[c] = reinterpret_cast<float *>(base + sg.s_off + (size_t)c * sg.s_plane);
        if (opt->init_from_output) {
            const TransArgs t = plane_copy(s[c], sh, sh->s_stride_b, sh->s_stride_d,
                                           sh->s_stride_t, s2[c], dDT, dT, 1);
            if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
        }
    }
    if (sg.s) {
        sh2.s_stride_b = dDT;
        sh2.s_stride_d = dT;
        sh2.s_stride_t = 1;
    }
    st = solve_core(cell, &sh2, u2, dt, a, s0, s2, opt, info, ws, ws_bytes, stream);
    if (st != PARARNN_OK) return st;
    for (int c = 0; c < S && sg.s; ++c) {
        const TransArgs t = plane_copy(s2[c], sh, dDT, dT, 1, s[c], sh->s_stride_b,
                                       sh->s_stride_d, sh->s_stride_t);
        if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
    }
    return PARARNN_OK;
}

// ------------------------------------------------------------- adjoint ---

struct AdjWs {
    size_t ticket = 0, flags = 0, records = 0, da_part = 0, total = 0;
};

AdjWs adj_ws_layout(pararnn_cell_t cell, const Plan &pl)
{
    AdjWs w;
    size_t off = 0;
    w.ticket = off;
    off += kAlign;
    w.flags = off;
    off = align_up(off + (size_t)pl.units * sizeof(int32_t));
    w.records = off;
    off = align_up(off + (size_t)pl.units * rec_floats(cell) * sizeof(float));
    w.da_part = off;
    off = align_up(off + (size_t)pl.units * cell_G(cell) * sizeof(float));
    w.total = off;
    return w;
}

struct ScanWs {
    size_t ticket = 0, flags = 0, records = 0, total = 0;
};

ScanWs scan_ws_layout(int S, const Plan &pl)
{
    ScanWs w;
    if (pl.nb <= 1) return w;
    size_t off = 0;
    w.ticket = off;
    off += kAlign;
    w.flags = off;
    off = align_up(off + (size_t)pl.units * sizeof(int32_t));
    w.records = off;
    const int rf = S == 2 ? MapRec<Map2>::kFloats : MapRec<Map1>::kFloats;
    off = align_up(off + (size_t)pl.units * rf * sizeof(float));
    w.total = off;
    return w;
}

// The scan is built for the adjoint's tilings (one pass, no Newton state).
pararnn_status_t make_scan_plan(int32_t S, const pararnn_shape_t *sh, const pararnn_newton_t *opt,
                                Plan &pl)
{
    if (S != 1 && S != 2) return PARARNN_ERR_INVALID;
    return make_plan(S == 2 ? PARARNN_LSTM : PARARNN_GRU, sh, opt, 2, pl);
}

// Staging room of the scan: S*S + S input planes (u strides) and S output
// planes (s strides), when they are not time-contiguous.
struct ScanStage {
    bool in = false, out = false;
    size_t in_off = 0, out_off = 0, plane = 0, total = 0;
};

ScanStage scan_stage_layout(int S, const pararnn_shape_t *sh, size_t base)
{
    ScanStage g;
    if (!sh || sh->B <= 0 || sh->D <= 0 || sh->T <= 1) return g;
    const int64_t n = sh->B * sh->D;
    if (n > (int64_t(1) << 40) / sh->T) return g;
    g.in = sh->u_stride_t != 1;
    g.out = sh->s_stride_t != 1;
    if (!g.in && !g.out) return g;
    g.plane = align_up((size_t)(n * sh->T) * sizeof(float));
    size_t off = align_up(base);
    if (g.in) {
        g.in_off = off;
        off += (size_t)(S * S + S) * g.plane;
    }
    if (g.out) {
        g.out_off = off;
        off += (size_t)S * g.plane;
    }
    g.total = off;
    return g;
}

pararnn_status_t scan_core(int32_t state_size, const pararnn_shape_t *shape,
                           const float *const *Am, const float *const *bv, const float *const *x0,
                           float *const *x, int32_t reverse, const pararnn_newton_t *opt, void *ws,
                           size_t ws_bytes, void *stream);

pararnn_status_t adjoint_core(pararnn_cell_t cell, const pararnn_shape_t *shape,
                              const void *const *u, pararnn_dtype_t u_dtype, const float *a,
                              const float *const *s0, const float *const *s,
                              const float *const *gs, const float *const *gs_end,
                              float *const *du, float *da, int32_t da_accumulate,
                              float *const *ds0, float *const *lam, const pararnn_newton_t *opt,
                              void *ws, size_t ws_bytes, void *stream);

}  // namespace

extern "C" {

size_t pararnn_scan_workspace_bytes(int32_t state_size, const pararnn_shape_t *shape,
                                    const pararnn_newton_t *opt)
{
    Plan pl;
    if (make_scan_plan(state_size, shape, opt, pl) != PARARNN_OK) return 0;
    const size_t base = scan_ws_layout(state_size, pl).total;
    const ScanStage sg = scan_stage_layout(state_size, shape, base);
    return sg.total > 0 ? sg.total : base;
}

pararnn_status_t pararnn_scan(int32_t state_size, const pararnn_shape_t *shape,
                              const float *const *Am, const float *const *bv,
                              const float *const *x0, float *const *x, int32_t reverse,
                              const pararnn_newton_t *opt, void *ws, size_t ws_bytes, void *stream)
{
    Plan pl;
    pararnn_status_t st = make_scan_plan(state_size, shape, opt, pl);
    if (st != PARARNN_OK) return st;
    const int S = state_size;
    const ScanStage sg = scan_stage_layout(S, shape, scan_ws_layout(S, pl).total);
    bool staged = sg.total > 0 && ws && ws_bytes >= sg.total && aligned16(ws) && Am && bv && x &&
                  (reverse == 0 || reverse == 1);
    for (int i = 0; i < S * S && staged; ++i) staged = Am[i] != nullptr;
    for (int c = 0; c < S && staged; ++c) staged = bv[c] && x[c];
    if (!staged) return scan_core(S, shape, Am, bv, x0, x, reverse, opt, ws, ws_bytes, stream);

    hipStream_t strm = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    const int64_t dT = shape->T, dDT = shape->D * shape->T;
    pararnn_shape_t sh2 = *shape;
    const float *A2[4] = {}, *b2[2] = {};
    float *x2[2] = {};
    const auto stage_in = [&](const float *src, int k) -> const float * {
        float *dst = reinterpret_cast<float *>(base + sg.in_off + (size_t)k * sg.plane);
        const TransArgs t = plane_copy(src, shape, shape->u_stride_b, shape->u_stride_d,
                                       shape->u_stride_t, dst, dDT, dT, 1);
        return launch_transpose(4, t, strm) == hipSuccess ? dst : nullptr;
    };
    for (int i = 0; i < S * S; ++i) {
        A2[i] = sg.in ? stage_in(Am[i], i) : Am[i];
        if (!A2[i]) return PARARNN_ERR_HIP;
    }
    for (int c = 0; c < S; ++c) {
        b2[c] = sg.in ? stage_in(bv[c], S * S + c) : bv[c];
        if (!b2[c]) return PARARNN_ERR_HIP;
        x2[c] = sg.out ? reinterpret_cast<float *>(base + sg.out_off + (size_t)c * sg.plane) : x[c];
    }
    if (sg.in) {
        sh2.u_stride_b = dDT;
        sh2.u_stride_d = dT;
        sh2.u_stride_t = 1;
    }
    if (sg.out) {
        sh2.s_stride_b = dDT;
        sh2.s_stride_d = dT;
        sh2.s_stride_t = 1;
    }
    st = scan_core(S, &sh2, A2, b2, x0, x2, reverse, opt, ws, ws_bytes, stream);
    if (st != PARARNN_OK) return st;
    for (int c = 0; c < S && sg.out; ++c) {
        const TransArgs t = plane_copy(x2[c], shape, dDT, dT, 1, x[c], shape->s_stride_b,
                                       shape->s_stride_d, shape->s_stride_t);
        if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
    }
    return PARARNN_OK;
}

}  // extern "C"

namespace {

pararnn_status_t scan_core(int32_t state_size, const pararnn_shape_t *shape,
                           const float *const *Am, const float *const *bv, const float *const *x0,
                           float *const *x, int32_t reverse, const pararnn_newton_t *opt, void *ws,
                           size_t ws_bytes, void *stream)
{
    Plan pl;
    pararnn_status_t st = make_scan_plan(state_size, shape, opt, pl);
    if (st != PARARNN_OK) return st;
    if (reverse != 0 && reverse != 1) return PARARNN_ERR_INVALID;
    const int S = state_size;
    const bool work = pl.channels > 0 && shape->T > 0;
    if (!work) return PARARNN_OK;
    if (!Am || !bv || !x) return PARARNN_ERR_INVALID;
    for (int i = 0; i < S * S; ++i)
        if (!Am[i]) return PARARNN_ERR_INVALID;
    for (int c = 0; c < S; ++c)
        if (!bv[c] || !x[c] || (x0 && !x0[c])) return PARARNN_ERR_INVALID;
    const ScanWs wl = scan_ws_layout(S, pl);
    if (wl.total > 0 && (!ws || ws_bytes < wl.total || !aligned16(ws))) return PARARNN_ERR_WORKSPACE;
    hipStream_t strm = static_cast<hipStream_t>(stream);

    ScanArgs A;
    std::memset(&A, 0, sizeof(A));
    for (int i = 0; i < S * S; ++i) A.A[i] = Am[i];
    for (int c = 0; c < S; ++c) {
        A.b[c] = bv[c];
        A.x[c] = x[c];
        A.x0[c] = x0 ? x0[c] : nullptr;
    }
    A.B = shape->B;
    A.T = shape->T;
    A.D = shape->D;
    A.isb = shape->u_stride_b;
    A.isd = shape->u_stride_d;
    A.osb = shape->s_stride_b;
    A.osd = shape->s_stride_d;
    A.ist = shape->u_stride_t;
    A.ost = shape->s_stride_t;
    A.channels = pl.channels;
    A.nb = (int32_t)pl.nb;
    bool iv = shape->u_stride_t == 1 && (shape->T % 4 == 0) && (shape->u_stride_b % 4 == 0) &&
              (shape->u_stride_d % 4 == 0);
    for (int i = 0; i < S * S; ++i) iv = iv && aligned16(Am[i]);
    for (int c = 0; c < S; ++c) iv = iv && aligned16(bv[c]);
    bool ov = shape->s_stride_t == 1 && (shape->T % 4 == 0) && (shape->s_stride_b % 4 == 0) &&
              (shape->s_stride_d % 4 == 0);
    for (int c = 0; c < S; ++c) ov = ov && aligned16(x[c]);
    A.in_vec = iv ? 1 : 0;
    A.out_vec = ov ? 1 : 0;
    if (wl.total > 0) {
        char *base = static_cast<char *>(ws);
        A.ticket = reinterpret_cast<uint32_t *>(base + wl.ticket);
        A.flags = reinterpret_cast<int32_t *>(base + wl.flags);
        A.records = reinterpret_cast<float *>(base + wl.records);
        const int tpb = 256;
        hipLaunchKernelGGL(scan_init_kernel, dim3((unsigned)((pl.units + tpb - 1) / tpb)), dim3(tpb),
                           0, strm, A, pl.units);
        if (hipGetLastError() != hipSuccess) return PARARNN_ERR_HIP;
    }
    const int64_t groups = ((pl.channels + 7) / 8) * 8 * pl.nb;
    return launch_scan(S, pl.K, pl.W, reverse != 0, groups, strm, A) == hipSuccess ? PARARNN_OK
                                                                                  : PARARNN_ERR_HIP;
}

}  // namespace

extern "C" {

pararnn_status_t pararnn_project(const pararnn_proj_shape_t *sh, const void *x, const void *w,
                                 const float *bias, void *u, pararnn_dtype_t u_dtype,
                                 void *stream)
{
    if (!sh) return PARARNN_ERR_INVALID;
    if (sh->B < 0 || sh->T < 0 || sh->I < 0 || sh->M < 0) return PARARNN_ERR_INVALID;
    if (u_dtype != PARARNN_F32 && u_dtype != PARARNN_BF16) return PARARNN_ERR_UNSUPPORTED;
    if (sh->B == 0 || sh->T == 0 || sh->M == 0) return PARARNN_OK;
    // rows must not overlap: x rows of I elements, W rows of I, u rows of T
    if (sh->x_stride_t < sh->I || sh->x_stride_b < sh->x_stride_t * sh->T) return PARARNN_ERR_INVALID;
    if (sh->w_stride_m < sh->I) return PARARNN_ERR_INVALID;
    if (sh->u_stride_m < sh->T || sh->u_stride_b < sh->u_stride_m * sh->M) return PARARNN_ERR_INVALID;
    if (!u || (sh->I > 0 && (!x || !w))) return PARARNN_ERR_INVALID;
    ProjArgs A;
    std::memset(&A, 0, sizeof(A));
    A.x = static_cast<const uint16_t *>(x);
    A.w = static_cast<const uint16_t *>(w);
    A.bias = bias;
    A.u = u;
    A.B = sh->B;
    A.T = sh->T;
    A.I = sh->I;
    A.M = sh->M;
    A.xsb = sh->x_stride_b;
    A.xst = sh->x_stride_t;
    A.wsm = sh->w_stride_m;
    A.usb = sh->u_stride_b;
    A.usm = sh->u_stride_m;
    A.out_bf16 = u_dtype == PARARNN_BF16 ? 1 : 0;
    // workgroup count with the narrowest tile any projection kernel uses
    const int64_t tm = (sh->M + proj::kBM - 1) / proj::kBM, tn = (sh->T + proj::kBN - 1) / proj::kBN;
    if (tm * tn * sh->B >= (int64_t(1) << 31)) return PARARNN_ERR_UNSUPPORTED;
    const hipError_t e = launch_project(static_cast<hipStream_t>(stream), A);
    return e == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
}

pararnn_status_t pararnn_sequential(pararnn_cell_t cell, const pararnn_shape_t *shape,
                                    const void *const *u, pararnn_dtype_t u_dtype,
                                    const float *a, const float *const *s0, float *const *s,
                                    void *stream)
{
    if (cell != PARARNN_GRU && cell != PARARNN_LSTM) return PARARNN_ERR_INVALID;
    pararnn_status_t st = check_shape(shape);
    if (st != PARARNN_OK) return st;
    if (u_dtype != PARARNN_F32 && u_dtype != PARARNN_BF16) return PARARNN_ERR_UNSUPPORTED;
    const int G = cell_G(cell), S = cell_S(cell);
    const int64_t channels = shape->B * shape->D;
    if (channels == 0 || shape->T == 0) return PARARNN_OK;
    if ((channels + kWave - 1) / kWave >= (int64_t(1) << 31)) return PARARNN_ERR_UNSUPPORTED;
    if (!u || !a || !s0 || !s) return PARARNN_ERR_INVALID;
    for (int g = 0; g < G; ++g)
        if (!u[g]) return PARARNN_ERR_INVALID;
    for (int c = 0; c < S; ++c)
        if (!s0[c] || !s[c]) return PARARNN_ERR_INVALID;
    SeqArgs A;
    std::memset(&A, 0, sizeof(A));
    for (int g = 0; g < G; ++g) A.u[g] = u[g];
    A.a = a;
    for (int c = 0; c < S; ++c) {
        A.s0[c] = s0[c];
        A.s[c] = s[c];
    }
    A.T = shape->T;
    A.D = shape->D;
    A.usb = shape->u_stride_b;
    A.usd = shape->u_stride_d;
    A.ssb = shape->s_stride_b;
    A.ssd = shape->s_stride_d;
    A.ust = shape->u_stride_t;
    A.sst = shape->s_stride_t;
    A.channels = channels;
    const int ve = u_dtype == PARARNN_BF16 ? 8 : 4;
    bool uv = shape->u_stride_t == 1 && (shape->T % ve == 0) && (shape->u_stride_b % ve == 0) &&
              (shape->u_stride_d % ve == 0);
    for (int g = 0; g < G; ++g) uv = uv && aligned16(u[g]);
    bool sv = shape->s_stride_t == 1 && (shape->T % 4 == 0) && (shape->s_stride_b % 4 == 0) &&
              (shape->s_stride_d % 4 == 0);
    for (int c = 0; c < S; ++c) sv = sv && aligned16(s[c]);
    A.u_vec = uv ? 1 : 0;
    A.s_vec = sv ? 1 : 0;
    const hipError_t e = launch_sequential(cell == PARARNN_LSTM, u_dtype == PARARNN_BF16,
                                           static_cast<hipStream_t>(stream), A);
    return e == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
}

const char *pararnn_status_string(pararnn_status_t s)
{
    switch (s) {
    case PARARNN_OK: return "ok";
    case PARARNN_ERR_INVALID: return "invalid argument";
    case PARARNN_ERR_UNSUPPORTED: return "unsupported argument combination";
    case PARARNN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PARARNN_ERR_HIP: return "HIP runtime error at launch";
    case PARARNN_ERR_SCRATCH:
        return "problem needs more scratch than the library's static array "
               "(PARARNN_STATIC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

pararnn_status_t pararnn_plan(pararnn_cell_t cell, const pararnn_shape_t *shape,
                              const pararnn_newton_t *opt, int adjoint, int32_t *K, int32_t *W,
                              int64_t *nb)
{
    if (cell != PARARNN_GRU && cell != PARARNN_LSTM) return PARARNN_ERR_INVALID;
    Plan pl;
    pararnn_status_t st = make_plan(cell, shape, opt, adjoint ? 1 : 0, pl);
    if (st != PARARNN_OK) return st;
    if (K) *K = pl.K;
    if (W) *W = pl.W;
    if (nb) *nb = pl.nb;
    return PARARNN_OK;
}

size_t pararnn_workspace_bytes(pararnn_cell_t cell, const pararnn_shape_t *shape,
                               const pararnn_newton_t *opt, int adjoint)
{
    if (cell != PARARNN_GRU && cell != PARARNN_LSTM) return 0;
    Plan pl;
    if (make_plan(cell, shape, opt, adjoint ? 1 : 0, pl) != PARARNN_OK) return 0;
    if (adjoint) {
        const size_t base = adj_ws_layout(cell, pl).total;
        const AdjStage sg = adj_stage_layout(cell, shape, 4, base);
        return sg.total > 0 ? sg.total : base;
    }
    if (opt && (opt->max_iters < 0 || opt->max_iters > kMaxIters)) return 0;
    // staging room for planes that are not time-contiguous (projections
    // counted at 4 bytes, enough for either dtype)
    const size_t base = solve_ws_layout(cell, pl, opt).total;
    const Stage sg = stage_layout(cell, shape, 4, base);
    return sg.total > 0 ? sg.total : base;
}

pararnn_status_t pararnn_solve_gru(const pararnn_shape_t *shape, const void *const u[3],
                                   pararnn_dtype_t u_dtype, const float *a, const float *h0,
                                   float *h, const pararnn_newton_t *opt, pararnn_info_t *info,
                                   void *ws, size_t ws_bytes, void *stream)
{
    const float *s0[1] = {h0};
    float *s[1] = {h};
    return solve_common(PARARNN_GRU, shape, u, u_dtype, a, s0, s, opt, info, ws, ws_bytes, stream);
}

pararnn_status_t pararnn_solve_lstm(const pararnn_shape_t *shape, const void *const u[4],
                                    pararnn_dtype_t u_dtype, const float *a, const float *c0,
                                    const float *h0, float *c, float *h,
                                    const pararnn_newton_t *opt, pararnn_info_t *info, void *ws,
                                    size_t ws_bytes, void *stream)
{
    const float *s0[2] = {c0, h0};
    float *s[2] = {c, h};
    return solve_common(PARARNN_LSTM, shape, u, u_dtype, a, s0, s, opt, info, ws, ws_bytes, stream);
}

pararnn_status_t pararnn_adjoint(pararnn_cell_t cell, const pararnn_shape_t *shape,
                                 const void *const *u, pararnn_dtype_t u_dtype, const float *a,
                                 const float *const *s0, const float *const *s,
                                 const float *const *gs, const float *const *gs_end,
                                 float *const *du, float *da, int32_t da_accumulate,
                                 float *const *ds0, float *const *lam, const pararnn_newton_t *opt,
                                 void *ws, size_t ws_bytes, void *stream)
{
    if (cell != PARARNN_GRU && cell != PARARNN_LSTM) return PARARNN_ERR_INVALID;
    if (u_dtype != PARARNN_F32 && u_dtype != PARARNN_BF16) return PARARNN_ERR_UNSUPPORTED;
    Plan pl;
    pararnn_status_t st = make_plan(cell, shape, opt, 1, pl);
    if (st != PARARNN_OK) return st;
    const int G = cell_G(cell), S = cell_S(cell);
    const size_t esize = u_dtype == PARARNN_BF16 ? 2 : 4;
    const AdjStage sg = adj_stage_layout(cell, shape, esize, adj_ws_layout(cell, pl).total);
    bool staged = sg.total > 0 && ws && ws_bytes >= sg.total && aligned16(ws) && u && s && gs &&
                  du;
    for (int g = 0; g < G && staged; ++g) staged = u[g] && du[g];
    for (int c = 0; c < S && staged; ++c) staged = s[c] && (!lam || lam[c]);
    if (!staged)
        return adjoint_core(cell, shape, u, u_dtype, a, s0, s, gs, gs_end, du, da, da_accumulate,
                            ds0, lam, opt, ws, ws_bytes, stream);

    hipStream_t strm = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    const int64_t dT = shape->T, dDT = shape->D * shape->T;
    pararnn_shape_t sh2 = *shape;
    const void *u2[4] = {};
    float *du2[4] = {};
    const float *s2[2] = {}, *gs2[2] = {};
    float *lam2[2] = {};
    for (int g = 0; g < G; ++g) {
        u2[g] = u[g];
        du2[g] = du[g];
        if (!sg.u) continue;
        u2[g] = base + sg.u_off + (size_t)g * sg.u_plane;
        du2[g] = reinterpret_cast<float *>(base + sg.du_off + (size_t)g * sg.f_plane);
        const TransArgs t = plane_copy(u[g], shape, shape->u_stride_b, shape->u_stride_d,
                                       shape->u_stride_t, const_cast<void *>(u2[g]), dDT, dT, 1);
        if (launch_transpose((int)esize, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
    }
    if (sg.u) {
        sh2.u_stride_b = dDT;
        sh2.u_stride_d = dT;
        sh2.u_stride_t = 1;
    }
    for (int c = 0; c < S; ++c) {
        s2[c] = s[c];
        gs2[c] = gs[c];
        lam2[c] = lam ? lam[c] : nullptr;
        if (!sg.s) continue;
        float *sp = reinterpret_cast<float *>(base + sg.s_off + (size_t)c * sg.f_plane);
        TransArgs t = plane_copy(s[c], shape, shape->s_stride_b, shape->s_stride_d,
                                 shape->s_stride_t, sp, dDT, dT, 1);
        if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
        s2[c] = sp;
        if (gs[c]) {
            float *gp = reinterpret_cast<float *>(base + sg.gs_off + (size_t)c * sg.f_plane);
            t = plane_copy(gs[c], shape, shape->s_stride_b, shape->s_stride_d, shape->s_stride_t,
                           gp, dDT, dT, 1);
            if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
            gs2[c] = gp;
        }
        if (lam) lam2[c] = reinterpret_cast<float *>(base + sg.lam_off + (size_t)c * sg.f_plane);
    }
    if (sg.s) {
        sh2.s_stride_b = dDT;
        sh2.s_stride_d = dT;
        sh2.s_stride_t = 1;
    }
    st = adjoint_core(cell, &sh2, u2, u_dtype, a, s0, s2, gs2, gs_end, du2, da, da_accumulate,
                      ds0, lam ? lam2 : nullptr, opt, ws, ws_bytes, stream);
    if (st != PARARNN_OK) return st;
    for (int g = 0; g < G && sg.u; ++g) {
        const TransArgs t = plane_copy(du2[g], shape, dDT, dT, 1, du[g], shape->u_stride_b,
                                       shape->u_stride_d, shape->u_stride_t);
        if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
    }
    for (int c = 0; c < S && sg.s && lam; ++c) {
        const TransArgs t = plane_copy(lam2[c], shape, dDT, dT, 1, lam[c], shape->s_stride_b,
                                       shape->s_stride_d, shape->s_stride_t);
        if (launch_transpose(4, t, strm) != hipSuccess) return PARARNN_ERR_HIP;
    }
    return PARARNN_OK;
}

}  // extern "C"

namespace {

pararnn_status_t adjoint_core(pararnn_cell_t cell, const pararnn_shape_t *shape,
                              const void *const *u, pararnn_dtype_t u_dtype, const float *a,
                              const float *const *s0, const float *const *s,
                              const float *const *gs, const float *const *gs_end,
                              float *const *du, float *da, int32_t da_accumulate,
                              float *const *ds0, float *const *lam, const pararnn_newton_t *opt,
                              void *ws, size_t ws_bytes, void *stream)
{
    if (cell != PARARNN_GRU && cell != PARARNN_LSTM) return PARARNN_ERR_INVALID;
    if (u_dtype != PARARNN_F32 && u_dtype != PARARNN_BF16) return PARARNN_ERR_UNSUPPORTED;
    if (da_accumulate != 0 && da_accumulate != 1) return PARARNN_ERR_INVALID;
    Plan pl;
    pararnn_status_t st = make_plan(cell, shape, opt, 1, pl);
    if (st != PARARNN_OK) return st;
    const int G = cell_G(cell), S = cell_S(cell);
    if (!da && shape->D > 0) return PARARNN_ERR_INVALID;
    const bool work = pl.channels > 0 && shape->T > 0;
    if (pl.channels > 0) {
        if (!u || !s0 || !s || !gs || !du || !ds0 || !a) return PARARNN_ERR_INVALID;
        for (int c = 0; c < S; ++c)
            if (!s0[c] || !ds0[c] || (work && !s[c]) || (lam && !lam[c])) return PARARNN_ERR_INVALID;
        for (int g = 0; g < G; ++g)
            if (work && (!u[g] || !du[g])) return PARARNN_ERR_INVALID;
    }
    const AdjWs wl = adj_ws_layout(cell, pl);
    if (!ws || ws_bytes < wl.total || !aligned16(ws)) return PARARNN_ERR_WORKSPACE;
    hipStream_t strm = static_cast<hipStream_t>(stream);

    AdjArgs A;
    std::memset(&A, 0, sizeof(A));
    for (int g = 0; g < G && pl.channels > 0; ++g) {
        A.u[g] = work ? u[g] : nullptr;
        A.du[g] = work ? du[g] : nullptr;
    }
    for (int c = 0; c < S && pl.channels > 0; ++c) {
        A.s0[c] = s0[c];
        A.s[c] = work ? s[c] : nullptr;
        A.gs[c] = gs[c];
        A.gend[c] = gs_end ? gs_end[c] : nullptr;
        A.ds0[c] = ds0[c];
        A.lam[c] = lam ? lam[c] : nullptr;
    }
    A.a = a;
    A.da = da;
    A.da_acc = da_accumulate;
    A.B = shape->B;
    A.T = shape->T;
    A.D = shape->D;
    A.usb = shape->u_stride_b;
    A.usd = shape->u_stride_d;
    A.ssb = shape->s_stride_b;
    A.ssd = shape->s_stride_d;
    A.ust = shape->u_stride_t;
    A.sst = shape->s_stride_t;
    A.channels = pl.channels;
    A.nb = (int32_t)pl.nb;
    const int ve = u_dtype == PARARNN_BF16 ? 8 : 4;
    bool uv = shape->u_stride_t == 1 && (shape->T % ve == 0) && (shape->u_stride_b % ve == 0) &&
              (shape->u_stride_d % ve == 0);
    bool dv = shape->u_stride_t == 1 && (shape->T % 4 == 0) && (shape->u_stride_b % 4 == 0) &&
              (shape->u_stride_d % 4 == 0);
    for (int g = 0; g < G && work; ++g) {
        uv = uv && aligned16(u[g]);
        dv = dv && aligned16(du[g]);
    }
    bool sv = shape->s_stride_t == 1 && (shape->T % 4 == 0) && (shape->s_stride_b % 4 == 0) &&
              (shape->s_stride_d % 4 == 0);
    for (int c = 0; c < S && work; ++c) {
        sv = sv && aligned16(s[c]);
        if (gs[c]) sv = sv && aligned16(gs[c]);
        if (lam) sv = sv && aligned16(lam[c]);
    }
    A.u_vec = uv ? 1 : 0;
    A.du_vec = dv ? 1 : 0;
    A.s_vec = sv ? 1 : 0;
    char *base = static_cast<char *>(ws);
    A.ticket = reinterpret_cast<uint32_t *>(base + wl.ticket);
    A.flags = reinterpret_cast<int32_t *>(base + wl.flags);
    A.records = reinterpret_cast<float *>(base + wl.records);
    A.da_part = reinterpret_cast<float *>(base + wl.da_part);

    const int tpb = 256;
    if (pl.channels == 0) {
        // no batch rows (or no channels): da is a sum of no terms
        if (shape->D == 0) return PARARNN_OK;
        const int64_t n = (int64_t)G * shape->D;
        hipLaunchKernelGGL(da_reduce_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0,
                           strm, A, G);
        return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
    }
    {
        const int64_t n = pl.units;
        hipLaunchKernelGGL(adjoint_init_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0,
                           strm, A, S, G, pl.units);
        if (hipGetLastError() != hipSuccess) return PARARNN_ERR_HIP;
    }
    if (work) {
        const int64_t groups = ((pl.channels + 7) / 8) * 8 * pl.nb;
        hipError_t e;
        if (cell == PARARNN_GRU)
            e = u_dtype == PARARNN_BF16 ? launch_adjoint_gru_bf16(pl.K, pl.W, groups, strm, A)
                                        : launch_adjoint_gru_f32(pl.K, pl.W, groups, strm, A);
        else
            e = u_dtype == PARARNN_BF16 ? launch_adjoint_lstm_bf16(pl.K, pl.W, groups, strm, A)
                                        : launch_adjoint_lstm_f32(pl.K, pl.W, groups, strm, A);
        if (e != hipSuccess) return PARARNN_ERR_HIP;
    }
    {
        const int64_t n = (int64_t)G * shape->D;
        hipLaunchKernelGGL(da_reduce_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0, strm,
                           A, G);
        if (hipGetLastError() != hipSuccess) return PARARNN_ERR_HIP;
    }
    return PARARNN_OK;
}

}  // namespace

// ------------------------------------------------ static scratch solve ---
// For callers that cannot allocate device memory: the workspace of
// pararnn_solve_gru_noalloc is this file-scope array.  Every GPU the library
// runs on holds its own copy (at its own address) until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so
// the device address is looked up once per device with hipGetSymbolAddress
// and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[PARARNN_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array; looked up on the first
// call on a device (with that device current, which is the device of the
// caller's stream) and kept.
pararnn_status_t device_scratch(void *stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PARARNN_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return PARARNN_ERR_HIP;
        if (sdev != dev) return PARARNN_ERR_INVALID;  // the stream's device must be current
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return PARARNN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PARARNN_OK;
}

}  // namespace

extern "C" {

pararnn_status_t pararnn_solve_gru_noalloc(const pararnn_shape_t *shape, const void *const u[3],
                                           pararnn_dtype_t u_dtype, const float *a,
                                           const float *h0, float *h,
                                           const pararnn_newton_t *opt, pararnn_info_t *info,
                                           void *stream)
{
    // every size check before any HIP call: what the solve needs beyond
    // its inputs and outputs must fit the static array
    pararnn_status_t st = check_newton(opt);
    if (st != PARARNN_OK) return st;
    Plan pl;
    st = make_plan(PARARNN_GRU, shape, opt, 0, pl);
    if (st != PARARNN_OK) return st;
    const SolveWs wl = solve_ws_layout(PARARNN_GRU, pl, opt);
    const size_t need = info ? wl.total : wl.multi;
    if (need > (size_t)PARARNN_STATIC_SCRATCH_BYTES) return PARARNN_ERR_SCRATCH;
    void *ws = nullptr;
    st = device_scratch(stream, &ws);
    if (st != PARARNN_OK) return st;
    // planes that are not time-contiguous are staged through the scratch
    // when they fit there and gathered step by step otherwise
    return pararnn_solve_gru(shape, u, u_dtype, a, h0, h, opt, info, ws,
                             (size_t)PARARNN_STATIC_SCRATCH_BYTES, stream);
}

}  // extern "C"
