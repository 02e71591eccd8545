// Plane re-layout between any two strided (b, d, t) layouts, used to stage
// time-major planes ([B][T][D]-like, channels adjacent in memory) into the
// channel-major [B][D][T] layout the solve reads with 16-byte vectors, and
// to write the states back.  A 256-thread workgroup moves a 64 (d) x 64 (t)
// tile of one batch row through LDS: it reads along whichever of d or t is
// contiguous in the source and writes along whichever is contiguous in the
// destination, so both sides are coalesced.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace pararnn {

struct TransArgs {
    const void *src;
    void *dst;
    int64_t B, T, D;
    int64_t ssb, ssd, sst;  // source strides (elements)
    int64_t dsb, dsd, dstt; // destination strides (elements)
    int32_t src_t_fast;     // 1: source consecutive along t (else along d)
    int32_t dst_t_fast;
    int32_t vec;            // 4-byte elements, unit stride along the fast dimension
                            // of each side, other strides multiples of 4, bases
                            // 16-byte aligned: full tiles move 16 bytes per lane
};

constexpr int kTransTile = 64;

inline int64_t transpose_groups(int64_t B, int64_t T, int64_t D)
{
    return B * ((T + kTransTile - 1) / kTransTile) * ((D + kTransTile - 1) / kTransTile);
}

#ifdef PARARNN_DEFINE_AUX_KERNELS  // compiled once, in the ABI translation unit
template <int ES>
__global__ void __launch_bounds__(256) plane_transpose_kernel(TransArgs A)
{
    using E = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
    __shared__ E tile[kTransTile][kTransTile + 1];  // [d][t], padded against bank conflicts
    const int64_t nt = (A.T + kTransTile - 1) / kTransTile;
    const int64_t nd = (A.D + kTransTile - 1) / kTransTile;
    const int64_t g = blockIdx.x;
    const int64_t b = g / (nt * nd), r = g - b * nt * nd;
    const int64_t d0 = (r / nt) * kTransTile, t0 = (r % nt) * kTransTile;
    const E *src = static_cast<const E *>(A.src) + b * A.ssb;
    E *dst = static_cast<E *>(A.dst) + b * A.dsb;
    if constexpr (ES == 4) {
        if (A.vec && d0 + kTransTile <= A.D && t0 + kTransTile <= A.T) {
            // 16 lanes cover one 64-element line of the fast dimension
            const int x4 = (threadIdx.x & 15) * 4, y0 = threadIdx.x >> 4;
#pragma unroll
            for (int y = y0; y < kTransTile; y += 16) {
                const int64_t off = A.src_t_fast ? (d0 + y) * A.ssd + (t0 + x4)
                                                 : (t0 + y) * A.sst + (d0 + x4);
                const uint4 v = *reinterpret_cast<const uint4 *>(src + off);
                const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (A.src_t_fast)
                        tile[y][x4 + q] = e[q];
                    else
                        tile[x4 + q][y] = e[q];
                }
            }
            __syncthreads();
#pragma unroll
            for (int y = y0; y < kTransTile; y += 16) {
                uint32_t e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) e[q] = A.dst_t_fast ? tile[y][x4 + q] : tile[x4 + q][y];
                const int64_t off = A.dst_t_fast ? (d0 + y) * A.dsd + (t0 + x4)
                                                 : (t0 + y) * A.dstt + (d0 + x4);
                *reinterpret_cast<uint4 *>(dst + off) = make_uint4(e[0], e[1], e[2], e[3]);
            }
            return;
        }
    }
#pragma unroll 4
    for (int i = threadIdx.x; i < kTransTile * kTransTile; i += 256) {
        const int x = i & (kTransTile - 1), y = i / kTransTile;
        const int d = A.src_t_fast ? y : x, t = A.src_t_fast ? x : y;
        if (d0 + d < A.D && t0 + t < A.T) tile[d][t] = src[(d0 + d) * A.ssd + (t0 + t) * A.sst];
    }
    __syncthreads();
#pragma unroll 4
    for (int i = threadIdx.x; i < kTransTile * kTransTile; i += 256) {
        const int x = i & (kTransTile - 1), y = i / kTransTile;
        const int d = A.dst_t_fast ? y : x, t = A.dst_t_fast ? x : y;
        if (d0 + d < A.D && t0 + t < A.T) dst[(d0 + d) * A.dsd + (t0 + t) * A.dstt] = tile[d][t];
    }
}
#endif

}  // namespace pararnn
