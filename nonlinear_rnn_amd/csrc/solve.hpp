// Fused DEER Newton solve: one kernel runs, for every channel, the whole
// Newton loop — residual and local Jacobian of the cell, parallel scan of the
// resulting affine maps, state update and convergence test — with the
// states, projections and per-step maps held in registers across iterations.
// Only the projections are read from HBM (once) and only the converged
// states are written (once).
//
// Method: "Параллельность RNN?" (forpes.ru), section 1.  Newton on the
// residual r_t = s_t - f(s_{t-1}) (§1.1-1.2); each Newton system is the
// block-bidiagonal forward substitution ds_t = A_t ds_{t-1} - r_t with
// ds_1 = -r_1 (§1.3, level 1), solved as an associative scan of affine maps
// (§1.3, level 2).  The fused single-kernel form is the "fully fused" tier
// of the voguetech.ru ParaRNN article ("Три уровня производительности").
//
// Work decomposition for one channel (b, d) of length T:
//   lane   : K consecutive steps, composed serially (up-sweep), later
//            re-applied serially from the lane's carry-in (down-sweep);
//   wave   : 64 lanes, inclusive scan of the lane aggregates via DPP;
//   block  : W waves (P = 64 W K steps); wave aggregates go through LDS
//            (double-buffered by iteration parity, one barrier/iteration);
//   channel: ceil(T / P) time blocks; block k folds the aggregates its
//            predecessors publish in global memory for the same iteration
//            (decoupled: it waits only for their local work, not for a
//            chain of prefixes).
//
// Every carry is applied with the same apply() on the same operands
// wherever it is needed, so a lane's copy of its predecessor's last state
// (h_{t0-1}) stays bitwise identical to the predecessor's own: no state
// exchange between lanes, waves or blocks is ever needed.
//
// Stopping (per time block, causal): block k stops at iteration i iff its
// max |r| < tol and every earlier block of the channel has stopped at or
// before i; at the iteration cap every block stops.  With one block per
// channel this is plain per-channel convergence.
#pragma once

#include "cells.hpp"
#include "pararnn.h"

namespace pararnn {

constexpr int32_t kStopBase = 1 << 24;

#ifndef PARARNN_GRU_MAPS_IN_LDS
#define PARARNN_GRU_MAPS_IN_LDS 1
#endif
// Occupancy target (waves per SIMD) of the unmasked K = 16 ParaGRU loop with
// up to 4 waves per workgroup: 4 (128 VGPRs) or 5 (96 VGPRs).
#ifndef PARARNN_GRU_K16_WAVES
#define PARARNN_GRU_K16_WAVES 4
#endif
#ifndef PARARNN_LSTM_GATES_IN_LDS
#define PARARNN_LSTM_GATES_IN_LDS 3
#endif

struct SolveArgs {
    const void *u[4];
    const float *a;
    const float *s0[2];
    float *s[2];
    int64_t B, T, D;
    int64_t usb, usd, ssb, ssd;
    int64_t ust, sst;  // time strides (1 = channel-major)
    int64_t channels;
    float tol;
    float guess_tol;  // max|r| below which the next evaluation is guessed to be the last (0 = never)
    int32_t cap;
    int32_t nb;
    int32_t init_from_output;
    int32_t u_vec, s_vec;
    uint32_t *ticket;
    int32_t *flags;
    float *records;
    float *hin0;
    uint32_t *unit_info;  // per work unit: (max|r| bits, updates), or null
};

template <class M>
struct MapRec;
template <>
struct MapRec<Map1> {
    static constexpr int kFloats = 4;  // a, b, cbit, pad
};
template <>
struct MapRec<Map2> {
    static constexpr int kFloats = 8;  // a00 a01 a10 a11 b0 b1 cbit pad
};

__device__ __forceinline__ void rec_store(float *r, const Map1 &m, uint32_t cbit)
{
    store_relaxed(r + 0, m.a);
    store_relaxed(r + 1, m.b);
    store_relaxed(r + 2, __uint_as_float(cbit));
}
__device__ __forceinline__ void rec_store(float *r, const Map2 &m, uint32_t cbit)
{
    store_relaxed(r + 0, m.a00);
    store_relaxed(r + 1, m.a01);
    store_relaxed(r + 2, m.a10);
    store_relaxed(r + 3, m.a11);
    store_relaxed(r + 4, m.b0);
    store_relaxed(r + 5, m.b1);
    store_relaxed(r + 6, __uint_as_float(cbit));
}
__device__ __forceinline__ void rec_load(const float *r, Map1 &m) { m = {load_relaxed(r), load_relaxed(r + 1)}; }
__device__ __forceinline__ void rec_load(const float *r, Map2 &m)
{
    m = {load_relaxed(r),     load_relaxed(r + 1), load_relaxed(r + 2),
         load_relaxed(r + 3), load_relaxed(r + 4), load_relaxed(r + 5)};
}
__device__ __forceinline__ uint32_t rec_cbit(const float *r, int n)
{
    return __float_as_uint(load_relaxed(r + n - 2));
}

// ------------------------------------------------------ vector plumbing ---

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// K consecutive steps t0..t0+K-1 of one plane (steps `st` elements apart),
// zero beyond T.  `vec` (uniform) means st = 1 and T, the row strides and the
// base are multiples of 16 bytes, so 16-byte vectors never straddle T;
// otherwise every step is its own load.
template <int K, bool BF16>
__device__ __forceinline__ void load_steps(const void *base, int64_t off, int64_t t0, int64_t T,
                                           int64_t st, bool vec, float (&out)[K])
{
    if constexpr (BF16) {
        const uint16_t *p = static_cast<const uint16_t *>(base) + off;
        if constexpr (K % 8 == 0) {
            if (vec) {
#pragma unroll
                for (int q = 0; q < K / 8; ++q) {
                    uint4 v = make_uint4(0u, 0u, 0u, 0u);
                    if (t0 + 8 * q < T) v = *reinterpret_cast<const uint4 *>(p + t0 + 8 * q);
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        out[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
                        out[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                    }
                }
                return;
            }
        }
        const uint16_t *q = p + t0 * st;
#pragma unroll
        for (int k = 0; k < K; ++k) out[k] = (t0 + k < T) ? bf16_to_f32(q[k * st]) : 0.0f;
    } else {
        const float *p = static_cast<const float *>(base) + off;
        if constexpr (K % 4 == 0) {
            if (vec) {
#pragma unroll
                for (int q = 0; q < K / 4; ++q) {
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (t0 + 4 * q < T) v = *reinterpret_cast<const float4 *>(p + t0 + 4 * q);
                    out[4 * q] = v.x;
                    out[4 * q + 1] = v.y;
                    out[4 * q + 2] = v.z;
                    out[4 * q + 3] = v.w;
                }
                return;
            }
        }
        const float *q = p + t0 * st;
#pragma unroll
        for (int k = 0; k < K; ++k) out[k] = (t0 + k < T) ? q[k * st] : 0.0f;
    }
}

// K consecutive float32 steps of a plane known to lie inside [0, T) in
// 16-byte vectors (p at the first step): plain loads with no bounds test, so
// that several planes' loads are in flight together (a bounds test per
// vector puts each load in a block of its own, and the compiler waits for
// one before issuing the next).
template <int K>
__device__ __forceinline__ void load_steps_inside(const float *p, float (&out)[K])
{
    static_assert(K % 4 == 0, "16-byte vectors");
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
        const float4 v = reinterpret_cast<const float4 *>(p)[q];
        out[4 * q] = v.x;
        out[4 * q + 1] = v.y;
        out[4 * q + 2] = v.z;
        out[4 * q + 3] = v.w;
    }
}

template <int K>
__device__ __forceinline__ void store_steps(float *p, int64_t t0, int64_t T, int64_t st, bool vec,
                                            const float (&v)[K])
{
    if constexpr (K % 4 == 0) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < K / 4; ++q)
                if (t0 + 4 * q < T)
                    *reinterpret_cast<float4 *>(p + t0 + 4 * q) =
                        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            return;
        }
    }
    float *q = p + t0 * st;
#pragma unroll
    for (int k = 0; k < K; ++k)
        if (t0 + k < T) q[k * st] = v[k];
}

// Channel of workgroup `blk` when every channel is one work unit and the
// grid is 8 * ceil(n / 8): workgroups are dispatched round-robin over the 8
// XCDs, and each XCD gets a contiguous range of channels, so channels that
// share cache lines (time-major planes) share an L2 and run close in time.
// Returns a value >= n for the padding workgroups.
__device__ __forceinline__ int64_t xcd_channel(int64_t blk, int64_t n)
{
    const int64_t per = (n + 7) >> 3;
    return (blk & 7) * per + (blk >> 3);
}

template <class V>
__device__ __forceinline__ V vzero();
template <>
__device__ __forceinline__ Vec1 vzero<Vec1>() { return {0.0f}; }
template <>
__device__ __forceinline__ Vec2 vzero<Vec2>() { return {0.0f, 0.0f}; }
__device__ __forceinline__ Vec1 vadd(const Vec1 &a, const Vec1 &b) { return {a.x + b.x}; }
__device__ __forceinline__ Vec2 vadd(const Vec2 &a, const Vec2 &b) { return {a.x0 + b.x0, a.x1 + b.x1}; }
__device__ __forceinline__ float vget(const Vec1 &v, int) { return v.x; }
__device__ __forceinline__ float vget(const Vec2 &v, int i) { return i ? v.x1 : v.x0; }
__device__ __forceinline__ void vset(Vec1 &v, int, float x) { v.x = x; }
__device__ __forceinline__ void vset(Vec2 &v, int i, float x)
{
    if (i)
        v.x1 = x;
    else
        v.x0 = x;
}

// Dynamic work units of a multi-block launch (grid 8 * ceil(channels / 8) *
// nb, the channels past the last one are padding).  A workgroup takes the
// next ticket of one counter once it is resident.  Tickets run over groups
// of kTicketGroup channels, handing out time-block rank 0 of every channel
// in the group, then rank 1, and so on, so a channel's rank r-1 always
// holds a smaller ticket than its rank r: it is resident or done whenever
// rank r runs, and the waits on predecessors cannot deadlock.  Spacing a
// channel's blocks a group apart lets a predecessor run ahead of its
// successor instead of both spinning in step (adjacent tickets measured up
// to 29% slower on the adjoint, 7-11% on the solve and the scan).
constexpr int64_t kTicketGroup = 1024;

__device__ __forceinline__ void take_unit(uint32_t *ticket, int64_t channels, int32_t nb,
                                          int64_t &s_ticket, int64_t &ch, int32_t &r)
{
    if (threadIdx.x == 0) s_ticket = (int64_t)atomicAdd(ticket, 1u);
    __syncthreads();
    const int64_t t = s_ticket;
    const int64_t padded = (channels + 7) / 8 * 8;
    const int64_t g = t / (kTicketGroup * nb);
    const int64_t base = g * kTicketGroup;
    const int64_t size = padded - base < kTicketGroup ? padded - base : kTicketGroup;
    const int64_t within = t - base * nb;
    r = (int32_t)(within / size);
    ch = base + (within - (int64_t)r * size);
}

// Map held by lane `src` of the wave, read by every lane (wave-uniform).
__device__ __forceinline__ float readlane_f(float x, int src)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}
__device__ __forceinline__ Map1 readlane_map(const Map1 &m, int src)
{
    return {readlane_f(m.a, src), readlane_f(m.b, src)};
}
__device__ __forceinline__ Map2 readlane_map(const Map2 &m, int src)
{
    return {readlane_f(m.a00, src), readlane_f(m.a01, src), readlane_f(m.a10, src),
            readlane_f(m.a11, src), readlane_f(m.b0, src),  readlane_f(m.b1, src)};
}

// Look-back for time block k of channel `ch` at Newton iteration `it`:
// returns the carry ds at the step before the block, and whether every
// earlier block has stopped by `it`.  Lane j of the wave handles predecessor
// lo + j, so a window of up to 64 predecessors costs one flag load and one
// record load per lane instead of a chain of dependent loads.
template <class M, class V>
__device__ __forceinline__ void look_back(const SolveArgs &A, int64_t ch, int32_t k, int32_t it,
                                          V &din, bool &pred_stopped, int32_t &known)
{
    constexpr int RF = MapRec<M>::kFloats;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t *flags = A.flags + ch * A.nb;
    const float *rec = A.records + (ch * A.nb) * (int64_t)(A.cap + 1) * RF;
    const int64_t rstride = (int64_t)(A.cap + 1) * RF;
    // Pass 1: from k-1 downwards, find the nearest block that stopped at or
    // before `it` (every block before it stopped no later); wait until each
    // block above it has published its record of this iteration.
    // A stop flag never changes once set, so the nearest window's stop
    // values seen in earlier iterations (`known`, one per lane) are reused:
    // once every predecessor there has stopped, this pass issues no loads.
    // Records behind such a flag were complete when it was first seen.
    int32_t start = 0;
    for (int32_t hi = k; hi > 0; hi -= kWave) {
        const int32_t lo = hi > kWave ? hi - kWave : 0;
        const int32_t j = lo + lane;
        const bool mine = j < hi;
        const bool nearest = hi == k;
        int32_t v = kStopBase;
        if (mine) v = (nearest && known >= kStopBase) ? known : load_flag(flags + j);
        while (!__all(!mine || v >= it + 1)) {
            __builtin_amdgcn_s_sleep(1);
            if (mine && v < it + 1) v = load_flag(flags + j);
        }
        if (nearest && mine && v >= kStopBase) known = v;
        const unsigned long long stopped =
            __ballot(mine && v >= kStopBase && v - kStopBase <= it);
        if (stopped) {
            start = lo + (63 - __clzll(stopped)) + 1;
            break;
        }
    }
    after_flag();
    // Pass 2: the first block p in start..k-1 that does not report |r| < tol
    // at `it`; blocks start..p-1 stop now (their carry-out is zero) and the
    // carry is the ordered fold of p..k-1.  Each lane loads its block's whole
    // record (bit and map) at once, so finding p and folding from it take
    // one round trip per window of 64 blocks, not two.
    int32_t p = k;
    din = vzero<V>();
    for (int32_t lo = start; lo < k; lo += kWave) {
        const int32_t j = lo + lane;
        const bool mine = j < k;
        M mj = identity_map(M{});
        uint32_t cb = 1u;
        if (mine) {
            rec_load(rec + j * rstride + it * RF, mj);
            cb = rec_cbit(rec + j * rstride + it * RF, RF);
        }
        int32_t q0 = 0;
        if (p == k) {
            const unsigned long long open = __ballot(mine && cb == 0u);
            if (!open) continue;
            q0 = __ffsll((long long)open) - 1;
            p = lo + q0;
        }
        const int32_t n = (k - lo) < kWave ? (k - lo) : kWave;
        for (int32_t q = q0; q < n; ++q) din = apply(readlane_map(mj, q), din);
    }
    pred_stopped = (p == k);
}

// Carries of every iteration at once, for a time block whose predecessors
// have all stopped before it starts (the common case: tickets hand out a
// channel's blocks a group apart, so rank r-1 is usually done when rank r
// begins).  Their stop iterations j_p and their per-iteration records are
// then final, and the carry into block k at iteration q is the fold over
// p = 0..k-1 of block p's aggregate map at q, restarted from zero at every
// block stopped by q (a stopped block's carry-out is zero): the same carry
// look_back() returns at q.  Lane q holds the carry of iteration q, so the
// Newton loop reads it with readlane instead of one round trip to the
// predecessors' records per iteration.  `v` holds the predecessors' flags
// as preload_flags() loaded them when the block started (lane p: block p).
// Returns false (nothing loaded) when a predecessor was still running then,
// when there are more than kPreloadBlocks predecessors, or when iterations
// would not fit one lane each.
constexpr int32_t kPreloadBlocks = 8;

// The flags preload_carries() decides on, loaded as the block starts and
// first read at its first carry, so that the load overlaps the first Newton
// evaluation instead of delaying it; 0 everywhere when no preload is
// possible.
__device__ __forceinline__ int32_t preload_flags(const SolveArgs &A, int64_t ch, int32_t k)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (k > kPreloadBlocks || A.cap >= kWave) return 0;
    return lane < k ? load_flag(A.flags + ch * A.nb + lane) : kStopBase;
}

template <class M, class V>
__device__ __forceinline__ bool preload_carries(const SolveArgs &A, int64_t ch, int32_t k,
                                                int32_t v, V &carry, int32_t &j_last)
{
    constexpr int RF = MapRec<M>::kFloats;
    const int lane = threadIdx.x & (kWave - 1);
    if (!__all(v >= kStopBase)) return false;
    after_flag();
    const int64_t rstride = (int64_t)(A.cap + 1) * RF;
    const float *rec = A.records + (ch * A.nb) * rstride;
    V c = vzero<V>();
    for (int32_t p = 0; p < k; ++p) {
        const int32_t jp = __builtin_amdgcn_readlane(v, p) - kStopBase;
        if (jp <= lane) {
            c = vzero<V>();
        } else {
            M m;
            rec_load(rec + p * rstride + lane * RF, m);
            c = apply(m, c);
        }
    }
    carry = c;
    j_last = __builtin_amdgcn_readlane(v, k - 1) - kStopBase;
    return true;
}

__device__ __forceinline__ Vec1 readlane_vec(const Vec1 &v, int src) { return {readlane_f(v.x, src)}; }
__device__ __forceinline__ Vec2 readlane_vec(const Vec2 &v, int src)
{
    return {readlane_f(v.x0, src), readlane_f(v.x1, src)};
}

template <class M>
struct Slot {
    M agg;
    uint32_t mx;
};

// Where the lane's running compositions wait between up-sweep and down-sweep:
// in VGPRs, or the first kLdsMaps of them in LDS.  ParaGRU (2 floats per
// step) keeps all K - 1 in LDS, which frees 2K VGPRs: 30 KB per 4-wave
// workgroup at K = 16, so that 5 such workgroups (5 waves per SIMD) share a
// CU's 160 KB; the last step's composition is the lane aggregate itself and
// stays in registers.  ParaLSTM (6 floats per step) keeps them in VGPRs,
// except in time blocks at K = 16, whose cross-block code needs the room:
// 8 of the 15 go to LDS (48 KB per 4-wave workgroup, two workgroups per CU;
// 96 KB per 8-wave one), where at 256 VGPRs 24-36 registers spilled.
template <class Cell, int K, int W, bool FULL, bool SINGLE>
struct MapStore {
    static constexpr bool kGru = sizeof(typename Cell::Map) == 8;
    static constexpr int kLdsMaps =
        (kGru && PARARNN_GRU_MAPS_IN_LDS && K >= 8) ? K - 1
        : (!kGru && !SINGLE && K == 16) ? 8
                                                  : 0;
    // ParaLSTM with one block per channel (running compositions in VGPRs,
    // LDS otherwise unused): the projections of its last kLdsGates gates
    // wait in LDS between Newton evaluations (48 KB per 4-wave workgroup at
    // K = 16), which brings the loop to the 168 VGPRs of three waves per
    // SIMD.  With two gates there the loop spilled 21-25 registers; with
    // all four the LDS would allow only two workgroups per CU.
    static constexpr int kLdsGates =
        (!kGru && SINGLE && FULL && K == 16 && W <= 4) ? PARARNN_LSTM_GATES_IN_LDS : 0;
    // register budget of the unmasked ParaGRU loop and of the ParaLSTM loop
    // above (everything else: at most 256 VGPRs, two waves per SIMD; one
    // more register would halve the occupancy)
    static constexpr int kMinWavesPerEu =
        kLdsGates > 0                                ? 3
        : !(kGru && kLdsMaps > 0 && FULL && K <= 16) ? 2
        : (K == 16 && W <= 4)                        ? PARARNN_GRU_K16_WAVES
                                                     : 4;
};

// Projections of the last NG gates of every step in LDS, as 16-byte groups
// of four steps, one plane per (group, gate) so that a wave's accesses are
// consecutive 16-byte words.
template <int K, int NG, int N>
struct GateLds {
    float4 v[K / 4][NG][N];
};
template <int K, int N>
struct GateLds<K, 0, N> {
    float4 v[1][1][1];
};

// A running composition in LDS, one plane of floats per map component so
// that a lane's accesses are 8-byte words at an 8-byte stride (no bank
// conflicts for either map size).
template <class M, int NL, int N>
struct MapPlanes;
template <int NL, int N>
struct MapPlanes<Map1, NL, N> {
    float2 v[NL][N];
    __device__ __forceinline__ void put(int kk, int i, const Map1 &m) { v[kk][i] = make_float2(m.a, m.b); }
    __device__ __forceinline__ Map1 get(int kk, int i) const
    {
        const float2 x = v[kk][i];
        return {x.x, x.y};
    }
};
template <int NL, int N>
struct MapPlanes<Map2, NL, N> {
    float2 v[NL][3][N];
    __device__ __forceinline__ void put(int kk, int i, const Map2 &m)
    {
        v[kk][0][i] = make_float2(m.a00, m.a01);
        v[kk][1][i] = make_float2(m.a10, m.a11);
        v[kk][2][i] = make_float2(m.b0, m.b1);
    }
    __device__ __forceinline__ Map2 get(int kk, int i) const
    {
        const float2 x = v[kk][0][i], y = v[kk][1][i], z = v[kk][2][i];
        return {x.x, x.y, y.x, y.y, z.x, z.y};
    }
};

// LDS of the Newton loop: wave aggregates (double-buffered by iteration
// parity) and the running compositions of steps 0..NL-1.
template <class Cell, int K, int W, int NL>
struct LoopSmem {
    Slot<typename Cell::Map> slots[2][W];
    MapPlanes<typename Cell::Map, (NL > 0 ? NL : 1), (NL > 0 ? W * kWave : 1)> mlds;
};

// Lane's K steps of every gate, pre-scaled for the exp2-based gates.  In a
// block wholly inside [0, T) (FULL) on 16-byte vectors, every plane's loads
// are issued before any is used and without branches, so they are in flight
// together; guarded per vector, each plane's loads sat in blocks of their own
// and the compiler waited for one before issuing the next, a memory round
// trip per vector at every work unit's start.
template <class Cell, int K, bool BF16, bool FULL>
__device__ __forceinline__ void load_projections(const SolveArgs &A, int64_t uoff, int64_t t0,
                                                 float (&u)[K][Cell::G])
{
    constexpr int G = Cell::G;
    constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte vector
    if constexpr (FULL && K % E == 0) {
        if (A.u_vec) {
            uint4 raw[G][K / E];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint8_t *p = static_cast<const uint8_t *>(A.u[g]) + (uoff + t0) * (BF16 ? 2 : 4);
#pragma unroll
                for (int q = 0; q < K / E; ++q) raw[g][q] = reinterpret_cast<const uint4 *>(p)[q];
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float sc = Cell::uscale(g);
#pragma unroll
                for (int q = 0; q < K / E; ++q) {
                    const uint32_t w[4] = {raw[g][q].x, raw[g][q].y, raw[g][q].z, raw[g][q].w};
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
            return;
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float tmp[K];
        load_steps<K, BF16>(A.u[g], uoff, t0, A.T, A.ust, A.u_vec != 0, tmp);
        const float sc = Cell::uscale(g);
#pragma unroll
        for (int kk = 0; kk < K; ++kk) u[kk][g] = tmp[kk] * sc;
    }
}

// The whole Newton solve of one work unit — channel `ch`, time block `k` —
// from the lane's pre-scaled projections `u`, its copy `hin` of the state
// before its first step and the Newton start `s`; writes the converged states
// and folds the unit into the info record.
// SEQ: block-sequential time blocks (no carries; see newton_kernel).
template <class Cell, int K, int W, bool FULL, int NL, bool SINGLE, bool SEQ, int NG = 0>
__device__ __forceinline__ void solve_unit(const SolveArgs &A, int64_t ch, int32_t k,
                                           const typename Cell::Coef &cf,
                                           const float (&u)[K][Cell::G],
                                           typename Cell::Vec (&s)[K], typename Cell::Vec hin,
                                           LoopSmem<Cell, K, W, NL> &sm,
                                           const GateLds<K, NG, W * kWave> *ug = nullptr)
{
    using M = typename Cell::Map;
    using V = typename Cell::Vec;
    constexpr int S = Cell::S;
    constexpr int P = W * kWave * K;
    constexpr int RF = MapRec<M>::kFloats;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t unit = ch * A.nb + k;
    const int64_t b = ch / A.D, d = ch - b * A.D;
    const int64_t T = A.T;
    const int64_t tb0 = (int64_t)k * P;
    const int64_t t0 = tb0 + (int64_t)(wave * kWave + lane) * K;
    const bool multi = !SINGLE && !SEQ && A.nb > 1;
    const bool last_lane_of_block = (wave == W - 1) && (lane == kWave - 1);
    const bool full = FULL || tb0 + P <= T;  // uniform over the workgroup

    // step kk's projections: the first G - NG gates from registers, the
    // rest from LDS
    constexpr int G = Cell::G;
    struct Proj {
        float v[G];
    };
    const auto proj = [&](int kk) {
        Proj p;
#pragma unroll
        for (int g = 0; g < G - NG; ++g) p.v[g] = u[kk][g];
        if constexpr (NG > 0) {
#pragma unroll
            for (int g = G - NG; g < G; ++g) {
                const float4 q = ug->v[kk / 4][g - (G - NG)][threadIdx.x];
                p.v[g] = (kk % 4 == 0) ? q.x : (kk % 4 == 1) ? q.y : (kk % 4 == 2) ? q.z : q.w;
            }
        }
        return p;
    };

    const uint32_t tolb = __float_as_uint(A.tol);
    // Newton converges quadratically: once max|r| < sqrt(tol) (A.guess_tol)
    // the next residual is expected below tol, so that evaluation skips the
    // Jacobian and the scan.  A wrong guess only costs a second evaluation of
    // the same iterate.  A time block whose residual passes must still learn
    // whether its predecessors stop at this iteration: it looks back first
    // and stops (publishing only its stop flag) if they do; otherwise it
    // evaluates the iterate in full, publishes its map and reuses the carry
    // it already has.  The stopping iteration of every unit is the one the
    // full evaluation would give.
    const uint32_t predb = __float_as_uint(A.guess_tol);
    M m[K];  // running composition of the lane's steps 0..kk (kk >= NL)
    int32_t it = 0;
    uint32_t bmx = 0;
    bool carry_known = false;  // the probe of this iteration already looked back
    int32_t lb_known = 0;      // this lane's predecessor's stop flag, once seen
    V din_probe = vzero<V>();
    bool stopped_probe = true;
    // every predecessor already done when the block started: all
    // iterations' carries in one load, at the first carry
    V pre_carry = vzero<V>();
    int32_t pre_jlast = 0;
    const int32_t pre_flags = (multi && k > 0) ? preload_flags(A, ch, k) : 0;
    int pre = (multi && k > 0) ? -1 : 0;  // -1: not decided yet
    const auto carry_at = [&](int32_t i, V &din, bool &stopped) {
        if (pre < 0) pre = preload_carries<M, V>(A, ch, k, pre_flags, pre_carry, pre_jlast) ? 1 : 0;
        if (pre > 0 && i < kWave) {
            din = readlane_vec(pre_carry, i);
            stopped = pre_jlast <= i;
        } else {
            look_back<M, V>(A, ch, k, i, din, stopped, lb_known);
        }
    };
    bool ronly = false;  // this evaluation is the predicted last one
    int xp = 0;          // LDS exchange slot parity (alternates every exchange)
    for (;; ++it) {
        if (ronly) {
            // ---- predicted last evaluation: residual and its maximum only
            // The gates of this pass and of a full pass of the same iterate
            // after a wrong guess must not look alike to the compiler, or it
            // keeps all K steps' gate values live into the full pass.  One
            // side passes its states through an empty asm: the full pass, in
            // place (one workgroup per channel or block-sequential blocks:
            // fewer registers and moves), or this one (blocks exchanging
            // carries: measured faster there).
            float mxf = 0.0f;
            V prev = (SINGLE || SEQ) ? hin : opaque(hin);
#pragma unroll
            for (int kk = 0; kk < K; ++kk) {
                V rk = Cell::step_residual(cf, proj(kk).v, prev, s[kk]);
                if (!full) rk = keep_or_zero(rk, t0 + kk < T);
                mxf = resmax(mxf, rk);
                prev = (SINGLE || SEQ) ? s[kk] : opaque(s[kk]);
            }
            const uint32_t wmx = wave_max_to_last(__float_as_uint(mxf));
            if (lane == kWave - 1) sm.slots[xp][wave].mx = wmx;
            __syncthreads();
            bmx = sm.slots[xp][0].mx;
#pragma unroll
            for (int j = 1; j < W; ++j) bmx = max(bmx, sm.slots[xp][j].mx);
            xp ^= 1;
            if (it == A.cap) break;
            if (bmx < tolb) {
                if (!multi) break;
                if (k > 0) carry_at(it, din_probe, stopped_probe);
                if (k == 0 || stopped_probe) {
                    if (threadIdx.x == 0) publish_flag(A.flags + unit, kStopBase + it);
                    break;
                }
                carry_known = true;
            }
            // not yet: full evaluation of the same iterate
            if constexpr (SINGLE || SEQ) {
                hin = opaque(hin);
#pragma unroll
                for (int kk = 0; kk < K; ++kk) s[kk] = opaque(s[kk]);
            }
            ronly = false;
        }
        // ---- residual, Jacobian and lane up-sweep.  Blocks that lie wholly
        // inside [0, T) take a path without per-step masks; the ragged last
        // block turns steps past T into identity maps by selection.
        float mxf = 0.0f;
        M agg = identity_map(M{});
        V prev = hin;
        const auto up = [&](int kk, M mk) {
            if (!full) mk = keep_or_identity(mk, t0 + kk < T);
            mxf = resmax(mxf, mk);
            prev = s[kk];
            agg = kk == 0 ? mk : compose(mk, agg);
            if (kk < NL)
                sm.mlds.put(kk, threadIdx.x, agg);
            else
                m[kk] = agg;
        };
        const auto up_all = [&]() {
#pragma unroll
            for (int kk = 0; kk < K; ++kk) up(kk, Cell::step_map(cf, proj(kk).v, prev, s[kk]));
        };
        // (the carry-exchanging kernels would spill with the second loop)
        if constexpr (Cell::kZeroPass && (SINGLE || SEQ)) {
            if (it == 0 && !A.init_from_output) {
                // first evaluation from the zero start: every step but the
                // lane's first (whose predecessor may be a given state) sees
                // h_{t-1} = h_t = 0
                up(0, Cell::step_map(cf, proj(0).v, prev, s[0]));
#pragma unroll
                for (int kk = 1; kk < K; ++kk) up(kk, Cell::step_map_zero(cf, proj(kk).v));
            } else {
                up_all();
            }
        } else {
            up_all();
        }
        // ---- wave scan, then block exchange through LDS
        const M inc = wave_scan_inclusive(agg);
        const M exc = wave_shift_up(inc);
        // |r| bit patterns: unsigned order = float order, NaN above +inf
        const uint32_t wmx = wave_max_to_last(__float_as_uint(mxf));
        const int par = xp;
        xp ^= 1;
        if (lane == kWave - 1) {
            sm.slots[par][wave].agg = inc;
            sm.slots[par][wave].mx = wmx;
        }
        __syncthreads();
        bmx = sm.slots[par][0].mx;
        M blk = sm.slots[par][0].agg;
#pragma unroll
        for (int j = 1; j < W; ++j) {
            bmx = max(bmx, sm.slots[par][j].mx);
            blk = compose(sm.slots[par][j].agg, blk);
        }
        const uint32_t cbit = bmx < tolb ? 1u : 0u;
        const bool at_cap = (it == A.cap);
        // Each record is certified by a flag as soon as it is stored (the
        // flag store waits for the record's stores to complete).
        if (multi && threadIdx.x == 0) {
            rec_store(A.records + (unit * (int64_t)(A.cap + 1) + it) * RF, blk, cbit);
            publish_flag(A.flags + unit, it + 1);
        }
        if (at_cap) break;
        V din = carry_known ? din_probe : vzero<V>();
        bool pred_stopped = carry_known ? stopped_probe : true;
        if (multi && k > 0 && !carry_known) carry_at(it, din, pred_stopped);
        carry_known = false;
        if (cbit && pred_stopped) {
            if (multi && threadIdx.x == 0) publish_flag(A.flags + unit, kStopBase + it);
            break;
        }
        ronly = bmx < predb;
        // ---- down-sweep from the carries, Newton update
        V dw = din;
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
            if (j < wave) dw = apply(sm.slots[par][j].agg, dw);
        const V dl = apply(exc, dw);
        const V dout = (multi && last_lane_of_block) ? apply(blk, din) : apply(inc, dw);
        hin = vadd(hin, dl);
        // m[kk] holds the lane's running composition of steps 0..kk, so every
        // step's correction comes straight from the lane carry-in (no serial
        // chain); the last step takes the carry the next lane also sees.
#pragma unroll
        for (int kk = 0; kk < K - 1; ++kk) {
            if (kk < NL)
                s[kk] = vadd(s[kk], apply(sm.mlds.get(kk, threadIdx.x), dl));
            else
                s[kk] = vadd(s[kk], apply(m[kk], dl));
        }
        s[K - 1] = vadd(s[K - 1], dout);
    }

    // ---- converged states out
    const int64_t soff = b * A.ssb + d * A.ssd;
#pragma unroll
    for (int c = 0; c < S; ++c) {
        float tmp[K];
#pragma unroll
        for (int kk = 0; kk < K; ++kk) tmp[kk] = vget(s[kk], c);
        store_steps<K>(A.s[c] + soff, t0, T, A.sst, A.s_vec != 0, tmp);
    }
    // The unit's own convergence record, folded into the info record by a
    // separate pass: atomics on one shared record from every workgroup
    // serialise on a single address and stall the whole solve.
    if (A.unit_info && threadIdx.x == 0)
        *reinterpret_cast<uint2 *>(A.unit_info + 2 * unit) = make_uint2(bmx, (uint32_t)it);
}

// One work unit per workgroup, or (SEQ) every time block of one channel.
// Serves every case: several time blocks per channel (dynamic tickets),
// ragged T, warm starts.
// SEQ (time blocks of many channels): block-sequential.  The workgroup
// solves its channel's blocks one after the other, block k from the exact
// state before it — block k-1's converged last state, handed from the last
// lane to the first through LDS — with no per-iteration carries, look-back
// or waits on other workgroups.  Every block still stops only when its own
// max |r_t| < tol, the residual of its first step taken against that state,
// so the whole trajectory meets the stopping rule; the iterates differ from
// one Newton iteration over the whole sequence, the converged states agree
// with it to within the tolerance.  Block k+1's projection loads are issued
// as soon as block k's states are stored, so they overlap that store.
template <class Cell, int K, int W, bool BF16, bool FULL, bool SINGLE, bool SEQ = false>
__global__ void __launch_bounds__(W * kWave, (MapStore<Cell, K, W, FULL, SINGLE>::kMinWavesPerEu))
    newton_kernel(SolveArgs A)
{
    using V = typename Cell::Vec;
    constexpr int G = Cell::G, S = Cell::S;
    constexpr int P = W * kWave * K;
    constexpr int kLdsMaps = MapStore<Cell, K, W, FULL, SINGLE>::kLdsMaps;
    constexpr int NG = MapStore<Cell, K, W, FULL, SINGLE>::kLdsGates;

    __shared__ LoopSmem<Cell, K, W, kLdsMaps> sm;
    __shared__ int64_t s_ticket;
    __shared__ V s_carry;
    __shared__ GateLds<K, NG, W * kWave> ug;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    int64_t ch;
    int32_t k;
    if (!SINGLE && !SEQ && A.nb > 1) {
        take_unit(A.ticket, A.channels, A.nb, s_ticket, ch, k);
    } else {
        ch = xcd_channel(blockIdx.x, A.channels);
        k = 0;
    }
    if (ch >= A.channels) return;
    const int64_t b = ch / A.D, d = ch - b * A.D;
    const int64_t T = A.T;
    const typename Cell::Coef cf = Cell::coef(A.a, A.D, d);
    const int64_t soff = b * A.ssb + d * A.ssd;
    const int32_t k_end = SEQ ? A.nb : k + 1;
    V carry = vzero<V>();  // (SEQ) block k-1's last state, for block k's first lane

    for (; k < k_end; ++k) {
        const int64_t unit = ch * A.nb + k;
        const int64_t tb0 = (int64_t)k * P;
        const int64_t t0 = tb0 + (int64_t)(wave * kWave + lane) * K;

        float u[K][G];
        load_projections<Cell, K, BF16, FULL>(A, b * A.usb + d * A.usd, t0, u);
        if constexpr (NG > 0) {
            // (each lane reads back only its own words, so no barrier)
#pragma unroll
            for (int q = 0; q < K / 4; ++q)
#pragma unroll
                for (int g = G - NG; g < G; ++g)
                    ug.v[q][g - (G - NG)][threadIdx.x] =
                        make_float4(u[4 * q][g], u[4 * q + 1][g], u[4 * q + 2][g], u[4 * q + 3][g]);
        }

        // Newton start and the lane's copy of the state just before it.
        V s[K];
        V hin = vzero<V>();
        if (A.init_from_output) {
#pragma unroll
            for (int c = 0; c < S; ++c) {
                float tmp[K];
                load_steps<K, false>(A.s[c], soff, t0, T, A.sst, A.s_vec != 0, tmp);
#pragma unroll
                for (int kk = 0; kk < K; ++kk) vset(s[kk], c, tmp[kk]);
            }
#pragma unroll
            for (int c = 0; c < S; ++c) {
                float x = 0.0f;
                if (t0 == 0)
                    x = A.s0[c][b * A.D + d];
                else if (t0 == tb0)
                    x = SEQ ? vget(carry, c) : A.hin0[unit * S + c];
                else if (t0 - 1 < T)
                    x = A.s[c][soff + (t0 - 1) * A.sst];
                vset(hin, c, x);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < K; ++kk) s[kk] = vzero<V>();
            if (t0 == 0) {
#pragma unroll
                for (int c = 0; c < S; ++c) vset(hin, c, A.s0[c][b * A.D + d]);
            } else if (SEQ && t0 == tb0) {
                hin = carry;
            }
        }
        solve_unit<Cell, K, W, FULL, kLdsMaps, SINGLE, SEQ, NG>(A, ch, k, cf, u, s, hin, sm, &ug);
        if constexpr (SEQ) {
            if (k + 1 < k_end) {
                // the block's last state, from its last lane to every lane
                // (the next block's first lane takes it); the barrier also
                // orders this block's last LDS reads before the next block's
                // first writes
                if (wave == W - 1 && lane == kWave - 1) s_carry = s[K - 1];
                __syncthreads();
                carry = s_carry;
            }
        }
    }
}

#ifdef PARARNN_DEFINE_AUX_KERNELS  // compiled once, in the ABI translation unit
// Clears the per-launch state of a multi-block solve (ticket counter, block
// flags) and gathers the initial boundary states a warm start needs.
__global__ void solve_init_kernel(SolveArgs A, int32_t S, int64_t units, int32_t P)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0 && A.ticket) *A.ticket = 0u;
    if (i < units && A.flags) {
        A.flags[i] = 0;
        if (A.init_from_output && A.hin0) {
            const int64_t ch = i / A.nb;
            const int32_t k = (int32_t)(i - ch * A.nb);
            const int64_t b = ch / A.D, d = ch - b * A.D;
            for (int c = 0; c < S; ++c)
                A.hin0[i * S + c] =
                    k > 0 ? A.s[c][b * A.ssb + d * A.ssd + ((int64_t)k * P - 1) * A.sst] : 0.0f;
        }
    }
}

// The info record from the units' own records: max updates, max of the
// final max|r| (bit patterns of non-negative floats order like the floats,
// NaN above +inf), converged iff that maximum is below tol, and the sum of
// updates.  Every field is an exact integer or max fold, so the result does
// not depend on the order.  One workgroup; the records are 8 bytes a unit.
constexpr int kFoldThreads = 1024;
__global__ void __launch_bounds__(kFoldThreads)
    info_fold_kernel(const uint32_t *rec, int64_t units, uint32_t tolb, pararnn_info_t *info)
{
    uint32_t mx = 0u, itmax = 0u;
    unsigned long long sum = 0ull;
    const uint2 *r2 = reinterpret_cast<const uint2 *>(rec);
    // four independent loads in flight per thread
    constexpr int kU = 4;
    int64_t i = threadIdx.x;
    for (; i + (kU - 1) * kFoldThreads < units; i += kU * kFoldThreads) {
        uint2 r[kU];
#pragma unroll
        for (int j = 0; j < kU; ++j) r[j] = r2[i + j * kFoldThreads];
#pragma unroll
        for (int j = 0; j < kU; ++j) {
            mx = max(mx, r[j].x);
            itmax = max(itmax, r[j].y);
            sum += r[j].y;
        }
    }
    for (; i < units; i += kFoldThreads) {
        const uint2 r = r2[i];
        mx = max(mx, r.x);
        itmax = max(itmax, r.y);
        sum += r.y;
    }
    __shared__ uint32_t smx[kFoldThreads / kWave], sit[kFoldThreads / kWave];
    __shared__ unsigned long long ssum[kFoldThreads / kWave];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        itmax = max(itmax, (uint32_t)__shfl_xor((int)itmax, o));
        sum += (unsigned long long)__shfl_xor((long long)sum, o);
    }
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        smx[wave] = mx;
        sit[wave] = itmax;
        ssum[wave] = sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kFoldThreads / kWave; ++w) {
            mx = max(mx, smx[w]);
            itmax = max(itmax, sit[w]);
            sum += ssum[w];
        }
        info->iters = (int32_t)itmax;
        info->converged = (units == 0 || mx < tolb) ? 1 : 0;
        info->max_abs_res = __uint_as_float(mx);
        info->nan_seen = mx > 0x7f800000u ? 1 : 0;
        info->iters_sum = (int64_t)sum;
        info->units = units;
    }
}

#endif

}  // namespace pararnn
