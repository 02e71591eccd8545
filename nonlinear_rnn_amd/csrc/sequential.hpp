// Step-by-step application of the recurrence, one lane per channel:
// s_t = f(s_{t-1}, u_t), t = 1..T, from the given s_0.  This is the
// sequential evaluation the parallel Newton solve replaces ("Параллельность
// RNN?", forpes.ru, §1.1: the true trajectory is the unique zero of the
// residual), and the baseline the pages measure their speed-up against (the
// voguetech.ru ParaRNN article, "Что именно сделали технически").  Its time
// is T times the latency of one step's dependency chain, whatever the number
// of channels up to the device's width, so with enough channels it is the
// faster way to the same trajectory; with few channels and long sequences
// the Newton solve wins.
//
// A lane streams its channel's projections in chunks of K steps, loading
// chunk c + 1 while it computes chunk c, and writes the states of a chunk
// with 16-byte stores.
#pragma once

#include "cells.hpp"
#include "solve.hpp"

namespace pararnn {

struct SeqArgs {
    const void *u[4];
    const float *a;
    const float *s0[2];
    float *s[2];
    int64_t T, D;
    int64_t usb, usd, ssb, ssd;
    int64_t ust, sst;  // time strides (1 = channel-major)
    int64_t channels;
    int32_t u_vec, s_vec;
};

template <class Cell, int K, bool BF16>
__device__ __forceinline__ void seq_load_chunk(const SeqArgs &A, int64_t uoff, int64_t t0,
                                               float (&u)[Cell::G][K])
{
#pragma unroll
    for (int g = 0; g < Cell::G; ++g) {
        load_steps<K, BF16>(A.u[g], uoff, t0, A.T, A.ust, A.u_vec != 0, u[g]);
        const float sc = Cell::uscale(g);
#pragma unroll
        for (int k = 0; k < K; ++k) u[g][k] *= sc;
    }
}

template <class Cell, int K, bool BF16>
__global__ void __launch_bounds__(kWave) sequential_kernel(SeqArgs A)
{
    using V = typename Cell::Vec;
    constexpr int G = Cell::G, S = Cell::S;
    const int64_t ch = (int64_t)blockIdx.x * kWave + threadIdx.x;
    if (ch >= A.channels) return;
    const int64_t b = ch / A.D, d = ch - b * A.D;
    const typename Cell::Coef cf = Cell::coef(A.a, A.D, d);
    const int64_t uoff = b * A.usb + d * A.usd, soff = b * A.ssb + d * A.ssd;
    V st;
#pragma unroll
    for (int c = 0; c < S; ++c) vset(st, c, A.s0[c][b * A.D + d]);

    float cur[G][K], nxt[G][K];
    seq_load_chunk<Cell, K, BF16>(A, uoff, 0, cur);
    for (int64_t t0 = 0; t0 < A.T; t0 += K) {
        if (t0 + K < A.T) seq_load_chunk<Cell, K, BF16>(A, uoff, t0 + K, nxt);
        float out[S][K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float uk[G];
#pragma unroll
            for (int g = 0; g < G; ++g) uk[g] = cur[g][k];
            st = Cell::next(cf, uk, st);
#pragma unroll
            for (int c = 0; c < S; ++c) out[c][k] = vget(st, c);
        }
#pragma unroll
        for (int c = 0; c < S; ++c) store_steps<K>(A.s[c] + soff, t0, A.T, A.sst, A.s_vec != 0, out[c]);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int k = 0; k < K; ++k) cur[g][k] = nxt[g][k];
    }
}

}  // namespace pararnn
