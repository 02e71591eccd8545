// Standalone parallel scan of a first-order linear recurrence, per channel:
//     forward:  x_t = A_t x_{t-1} + b_t,  t = 1..T,  x_0 given
//     reverse:  x_t = A_t x_{t+1} + b_t,  t = T..1,  x_{T+1} given
// with A_t a scalar (state size 1) or a 2x2 block (state size 2).  This is the
// linear system each Newton iteration solves ("Параллельность RNN?",
// forpes.ru, §1.3, levels 1-2) exposed on its own, the "parallel reduction"
// tier of the voguetech.ru ParaRNN article ("Три уровня производительности",
// item 2), for callers that assemble (A, b) themselves.
//
// Same decomposition as the fused solve, in one pass: K steps per lane
// composed serially, a DPP scan over the wave, a fold over the workgroup's
// waves through LDS, and a fold of the preceding time blocks' published
// aggregates.  Scan order = time order (forward) or reversed time (reverse):
// "rank" counts time blocks, lanes and steps in scan order.
#pragma once

#include "solve.hpp"

namespace pararnn {

struct ScanArgs {
    const float *A[4];   // S*S planes, row-major blocks (a00, a01, a10, a11)
    const float *b[2];   // S planes
    const float *x0[2];  // S planes [B][D] (boundary value), or null = 0
    float *x[2];         // S planes out
    int64_t B, T, D;
    int64_t isb, isd, osb, osd;
    int64_t ist, ost;  // time strides (1 = channel-major)
    int64_t channels;
    int32_t nb;
    int32_t in_vec, out_vec;
    uint32_t *ticket;
    int32_t *flags;
    float *records;
};

template <class M>
struct ScanIo;
template <>
struct ScanIo<Map1> {
    using V = Vec1;
    static constexpr int S = 1;
    // `inside`: the workgroup's block lies inside [0, T) and the planes are
    // in 16-byte vectors
    template <int K>
    static __device__ __forceinline__ void load(const ScanArgs &A, int64_t off, int64_t t0,
                                                bool inside, Map1 (&m)[K])
    {
        float a[K], b[K];
        bool done = false;
        if constexpr (K % 4 == 0) {
            if (inside) {
                load_steps_inside<K>(A.A[0] + off + t0, a);
                load_steps_inside<K>(A.b[0] + off + t0, b);
                done = true;
            }
        }
        if (!done) {
            load_steps<K, false>(A.A[0], off, t0, A.T, A.ist, A.in_vec != 0, a);
            load_steps<K, false>(A.b[0], off, t0, A.T, A.ist, A.in_vec != 0, b);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) m[k] = {a[k], b[k]};
    }
};
template <>
struct ScanIo<Map2> {
    using V = Vec2;
    static constexpr int S = 2;
    template <int K>
    static __device__ __forceinline__ void load(const ScanArgs &A, int64_t off, int64_t t0,
                                                bool inside, Map2 (&m)[K])
    {
        float a00[K], a01[K], a10[K], a11[K], b0[K], b1[K];
        bool done = false;
        if constexpr (K % 4 == 0) {
            if (inside) {
                const int64_t o = off + t0;
                load_steps_inside<K>(A.A[0] + o, a00);
                load_steps_inside<K>(A.A[1] + o, a01);
                load_steps_inside<K>(A.A[2] + o, a10);
                load_steps_inside<K>(A.A[3] + o, a11);
                load_steps_inside<K>(A.b[0] + o, b0);
                load_steps_inside<K>(A.b[1] + o, b1);
                done = true;
            }
        }
        if (!done) {
            const bool v = A.in_vec != 0;
            load_steps<K, false>(A.A[0], off, t0, A.T, A.ist, v, a00);
            load_steps<K, false>(A.A[1], off, t0, A.T, A.ist, v, a01);
            load_steps<K, false>(A.A[2], off, t0, A.T, A.ist, v, a10);
            load_steps<K, false>(A.A[3], off, t0, A.T, A.ist, v, a11);
            load_steps<K, false>(A.b[0], off, t0, A.T, A.ist, v, b0);
            load_steps<K, false>(A.b[1], off, t0, A.T, A.ist, v, b1);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) m[k] = {a00[k], a01[k], a10[k], a11[k], b0[k], b1[k]};
    }
};

template <class M, int K, int W, bool REV>
__global__ void __launch_bounds__(W * kWave) scan_kernel(ScanArgs A)
{
    using V = typename ScanIo<M>::V;
    constexpr int S = ScanIo<M>::S;
    constexpr int P = W * kWave * K;
    constexpr int RF = MapRec<M>::kFloats;

    __shared__ M s_agg[W];
    __shared__ int64_t s_ticket;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    int64_t ch;
    int32_t r;  // rank of this time block in scan order
    if (A.nb > 1) {
        take_unit(A.ticket, A.channels, A.nb, s_ticket, ch, r);
    } else {
        ch = xcd_channel(blockIdx.x, A.channels);
        r = 0;
    }
    if (ch >= A.channels) return;
    const int32_t k = REV ? A.nb - 1 - r : r;
    const int64_t b = ch / A.D, d = ch - b * A.D;
    const int64_t T = A.T;
    const int64_t pos = wave * kWave + lane;  // position in scan order
    const int64_t chunk = REV ? (int64_t)(W * kWave - 1) - pos : pos;
    const int64_t t0 = (int64_t)k * P + chunk * K;
    const int64_t ioff = b * A.isb + d * A.isd;
    const int64_t ooff = b * A.osb + d * A.osd;

    // maps in time order, identity past T; composed in scan order
    M m[K];
    const bool inside = A.in_vec && (int64_t)(k + 1) * P <= T;
    ScanIo<M>::template load<K>(A, ioff, t0, inside, m);
#pragma unroll
    for (int kk = 0; kk < K; ++kk) m[kk] = keep_or_identity(m[kk], t0 + kk < T);
    M agg = identity_map(M{});
#pragma unroll
    for (int q = 0; q < K; ++q) {
        const int kk = REV ? K - 1 - q : q;
        agg = q == 0 ? m[kk] : compose(m[kk], agg);
        m[kk] = agg;  // running composition up to this step, in scan order
    }
    const M inc = wave_scan_inclusive(agg);
    const M exc = wave_shift_up(inc);
    if (lane == kWave - 1) s_agg[wave] = inc;
    __syncthreads();
    M blk = s_agg[0];
#pragma unroll
    for (int j = 1; j < W; ++j) blk = compose(s_agg[j], blk);

    // carry into this time block: the boundary value, through every block
    // earlier in scan order
    V din = vzero<V>();
    if (A.x0[0]) {
#pragma unroll
        for (int c = 0; c < S; ++c) vset(din, c, A.x0[c][b * A.D + d]);
    }
    if (A.nb > 1) {
        const int64_t unit = ch * A.nb + r;
        if (threadIdx.x == 0) {
            rec_store(A.records + unit * RF, blk, 0u);
            publish_flag(A.flags + unit, 1);
        }
        const int32_t *flags = A.flags + ch * A.nb;
        for (int32_t lo = 0; lo < r; lo += kWave) {
            const int32_t hi = r - lo > kWave ? lo + kWave : r;
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
            for (int32_t q = 0; q < hi - lo; ++q) din = apply(readlane_map(mj, q), din);
        }
    }
    V dw = din;
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        if (j < wave) dw = apply(s_agg[j], dw);
    const V dl = apply(exc, dw);

    float xo[S][K];
#pragma unroll
    for (int kk = 0; kk < K; ++kk) {
        const V xv = apply(m[kk], dl);
#pragma unroll
        for (int c = 0; c < S; ++c) xo[c][kk] = vget(xv, c);
    }
#pragma unroll
    for (int c = 0; c < S; ++c) store_steps<K>(A.x[c] + ooff, t0, T, A.ost, A.out_vec != 0, xo[c]);
}

#ifdef PARARNN_DEFINE_AUX_KERNELS
__global__ void scan_init_kernel(ScanArgs A, int64_t units)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) *A.ticket = 0u;
    if (i < units) A.flags[i] = 0;
}
#endif

}  // namespace pararnn
