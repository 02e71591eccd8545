// Kernel launchers, one set per (cell, projection dtype); each set is
// instantiated in its own translation unit (inst_*.hip) so the tiling
// variants compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "adjoint.hpp"
#include "project.hpp"
#include "scan_kernel.hpp"
#include "sequential.hpp"
#include "solve.hpp"
#include "transpose.hpp"

namespace pararnn {

// Tilings with kernels: steps per lane K and waves per workgroup W.
inline bool newton_tiling_built(bool lstm, int K, int W)
{
    const bool base = (K == 1 || K == 2 || K == 4 || K == 8 || K == 16) &&
                      (W == 1 || W == 2 || W == 4 || W == 8);
    return base || (!lstm && K == 32 && (W == 1 || W == 2));
}
inline bool adjoint_tiling_built(bool, int K, int W)
{
    return (K == 1 || K == 2 || K == 4 || K == 8 || K == 16) &&
           (W == 1 || W == 2 || W == 4 || W == 8);
}

#define PARARNN_DECLARE_LAUNCHERS(NAME)                                                          \
    hipError_t launch_newton_##NAME(int K, int W, int variant, int64_t groups, hipStream_t st,  \
                                    const SolveArgs &a);                                        \
    hipError_t launch_newton_seq_##NAME(int K, int W, int64_t groups, hipStream_t st,          \
                                        const SolveArgs &a);                                    \
    hipError_t launch_adjoint_##NAME(int K, int W, int64_t groups, hipStream_t st,              \
                                     const AdjArgs &a);
PARARNN_DECLARE_LAUNCHERS(gru_f32)
PARARNN_DECLARE_LAUNCHERS(gru_bf16)
PARARNN_DECLARE_LAUNCHERS(lstm_f32)
PARARNN_DECLARE_LAUNCHERS(lstm_bf16)
#undef PARARNN_DECLARE_LAUNCHERS

// Input projection u = W x + b (MFMA).
hipError_t launch_project(hipStream_t st, const ProjArgs &a);

// Step-by-step application, one lane per channel.
hipError_t launch_sequential(bool lstm, bool bf16, hipStream_t st, const SeqArgs &a);

// Standalone scan: state size 1 or 2, forward or reverse.
hipError_t launch_scan(int S, int K, int W, bool reverse, int64_t groups, hipStream_t st,
                       const ScanArgs &a);

#define PARARNN_BASE_KW(X)                                                                      \
    X(1, 1) X(1, 2) X(1, 4) X(1, 8) X(2, 1) X(2, 2) X(2, 4) X(2, 8) X(4, 1) X(4, 2) X(4, 4)    \
        X(4, 8) X(8, 1) X(8, 2) X(8, 4) X(8, 8) X(16, 1) X(16, 2) X(16, 4) X(16, 8)

// Newton kernel variants: 0 = any block (ragged T), 1 = blocks wholly inside
// [0, T), 2 = as 1 with one block per channel (no cross-block code); 3 and 4
// = 0 and 1 with block-sequential time blocks (built for K = 16, W = 4 only:
// the long-sequence default with many channels, each workgroup solving one
// channel's blocks in order).
enum {
    kNewtonAny = 0,
    kNewtonFull = 1,
    kNewtonFullSingle = 2,
    kNewtonAnySeq = 3,
    kNewtonFullSeq = 4
};
inline bool newton_seq_built(int K, int W) { return K == 16 && W == 4; }

#define PARARNN_NEWTON_CASE(CELL, BF16, KK, WW)                                                 \
    case KK * 100 + WW:                                                                         \
        if (variant == kNewtonFullSingle)                                                       \
            hipLaunchKernelGGL((newton_kernel<CELL, KK, WW, BF16, true, true>), grid, block, 0,  \
                               st, a);                                                          \
        else if (variant == kNewtonFull)                                                        \
            hipLaunchKernelGGL((newton_kernel<CELL, KK, WW, BF16, true, false>), grid, block, 0, \
                               st, a);                                                          \
        else                                                                                    \
            hipLaunchKernelGGL((newton_kernel<CELL, KK, WW, BF16, false, false>), grid, block,  \
                               0, st, a);                                                       \
        break;

#define PARARNN_ADJOINT_CASE(CELL, BF16, KK, WW)                                                \
    case KK * 100 + WW:                                                                         \
        hipLaunchKernelGGL((adjoint_kernel<CELL, KK, WW, BF16>), grid, block, 0, st, a);        \
        break;

// EXTRA(X) lists tilings beyond the base set for this cell.
#define PARARNN_DEFINE_LAUNCHERS(NAME, CELL, BF16, EXTRA)                                  \
    hipError_t launch_newton_##NAME(int K, int W, int variant, int64_t groups, hipStream_t st,  \
                                    const SolveArgs &a)                                         \
    {                                                                                           \
        const dim3 grid((unsigned)groups), block((unsigned)(kWave * W));                        \
        if (variant == kNewtonFullSeq) return launch_newton_seq_##NAME(K, W, groups, st, a);     \
        if (variant == kNewtonAnySeq) {                                                         \
            if (!newton_seq_built(K, W)) return hipErrorInvalidValue;                            \
            hipLaunchKernelGGL((newton_kernel<CELL, 16, 4, BF16, false, false, true>), grid,     \
                               block, 0, st, a);                                                \
            return hipGetLastError();                                                           \
        }                                                                                       \
        switch (K * 100 + W) {                                                                  \
            PARARNN_BASE_KW(PARARNN_NEWTON_CASE_##NAME)                                         \
            EXTRA(PARARNN_NEWTON_CASE_##NAME)                                                   \
        default:                                                                                \
            return hipErrorInvalidValue;                                                        \
        }                                                                                       \
        return hipGetLastError();                                                               \
    }                                                                                           \
    hipError_t launch_adjoint_##NAME(int K, int W, int64_t groups, hipStream_t st,              \
                                     const AdjArgs &a)                                          \
    {                                                                                           \
        const dim3 grid((unsigned)groups), block((unsigned)(kWave * W));                        \
        switch (K * 100 + W) {                                                                  \
            PARARNN_BASE_KW(PARARNN_ADJOINT_CASE_##NAME)                                        \
        default:                                                                                \
            return hipErrorInvalidValue;                                                        \
        }                                                                                       \
        return hipGetLastError();                                                               \
    }

// The block-sequential kernel on full blocks (K = 16, W = 4), in a
// translation unit of its own where a cell needs other compiler options for
// it (the ragged-T variant is launched with the other kernels).
#define PARARNN_DEFINE_SEQ_LAUNCHER(NAME, CELL, BF16)                                            \
    hipError_t launch_newton_seq_##NAME(int K, int W, int64_t groups, hipStream_t st,          \
                                        const SolveArgs &a)                                     \
    {                                                                                           \
        if (!newton_seq_built(K, W)) return hipErrorInvalidValue;                                \
        const dim3 grid((unsigned)groups), block((unsigned)(kWave * W));                        \
        hipLaunchKernelGGL((newton_kernel<CELL, 16, 4, BF16, true, false, true>), grid, block,   \
                           0, st, a);                                                           \
        return hipGetLastError();                                                               \
    }

#define PARARNN_NO_EXTRA(X)
#define PARARNN_GRU_EXTRA(X) X(32, 1) X(32, 2)

}  // namespace pararnn
