// Input projection u = W x + b, the dense step before the recurrence: every
// gate's pre-activation input u_t = W x_t + b is computed once for the whole
// sequence before the Newton solve (the cells of the voguetech.ru ParaRNN
// article, "Что именно сделали технически", item 3, take u as precomputed
// projections; only the diagonal recurrent part stays inside the solve).
//
// Per batch row b it is one matrix product
//     u[b][m][t] = sum_k W[m][k] x[b][t][k] + bias[m],   m < M = G*D, t < T,
// with W [M][I] and x [B][T][I] both contiguous along k: the MFMA operand
// layout needs no transpose, and the output comes out channel-major with
// time contiguous — the [B][G*D][T] layout the solve reads (gate g's plane
// starts at row g*D).  bf16 operands, fp32 accumulation on the matrix cores
// (v_mfma_f32_32x32x16_bf16), fp32 or bf16 (round to nearest even) output.
//
// Tiling: a 256-thread workgroup computes a 256 (m) x 128 (t) tile; each of
// its 4 waves a 128 x 64 tile as 4 x 2 MFMA 32x32 blocks (128 accumulator
// VGPRs).  K advances 32 at a time through two LDS stages: while the waves
// multiply out of one stage, the next stage is in flight from memory into
// registers and is written to the other one afterwards (one barrier per
// step).  Tiles are ordered per XCD and in groups of m tiles so
// that the workgroups in flight on one XCD share their operands in its L2.  LDS rows are padded to 80 bytes so the 16-byte operand
// reads of 16 lanes cover all 64 banks once.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pararnn {

struct ProjArgs {
    const uint16_t *x;   // bf16 bits, x[b][t][k] at b*xsb + t*xst + k
    const uint16_t *w;   // bf16 bits, W[m][k] at m*wsm + k
    const float *bias;   // [M] or null
    void *u;             // u[b][m][t] at b*usb + m*usm + t
    int64_t B, T, I, M;
    int64_t xsb, xst, wsm, usb, usm;
    int32_t out_bf16;
    int32_t tiles_m, tiles_n;  // workgroup tiles along m and t
    int32_t group_m;           // m tiles that walk the t tiles together
};

namespace proj {

#ifndef PARARNN_PROJ_BK
#define PARARNN_PROJ_BK 32
#endif
constexpr int kBM = 256, kBN = 128, kBK = PARARNN_PROJ_BK;
constexpr int kRow = kBK + 8;   // padded LDS row, bf16 elements
constexpr int kCR = kBK / 8;    // 16-byte chunks per row
constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// One 16-byte chunk (8 k-values) of a row, zero beyond the matrix.
__device__ __forceinline__ uint4 load_chunk(const uint16_t *row, int64_t k, int64_t K,
                                            bool row_ok, bool vec)
{
    if (!row_ok) return make_uint4(0u, 0u, 0u, 0u);
    if (vec && k + 8 <= K) return *reinterpret_cast<const uint4 *>(row + k);
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (k + j < K) ? row[k + j] : (uint16_t)0;
    uint4 v;
    __builtin_memcpy(&v, e, 16);
    return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace proj

#ifdef PARARNN_DEFINE_PROJECT_KERNEL  // compiled once, in its own translation unit
// VEC: every row of x and W is 16-byte aligned and I % 32 == 0, so every
// chunk of every stage lies inside its row: unconditional vector loads (rows
// past M or T read a valid row whose results are not stored).
template <bool VEC>
__global__ void __launch_bounds__(proj::kThreads, 2) project_kernel(ProjArgs A)
{
    using namespace proj;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM][kRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN][kRow];

    // Workgroup -> tile.  Workgroups are dealt to the 8 XCDs round-robin, so
    // the hardware index is first turned into an index that runs
    // contiguously within one XCD (whose L2 the tiles then share).  Within a
    // batch row, groups of group_m m tiles walk the t tiles together: the
    // workgroups in flight on an XCD share a few W tiles and each x tile.
    const int64_t total = (int64_t)A.tiles_m * A.tiles_n * A.B;
    int64_t g = blockIdx.x;
    if (total % 8 == 0) g = (g % 8) * (total / 8) + g / 8;
    const int64_t per_b = (int64_t)A.tiles_m * A.tiles_n;
    const int64_t b = g / per_b;
    const int64_t r = g - b * per_b;
    const int64_t mg = r / ((int64_t)A.group_m * A.tiles_n);
    const int64_t gsz = (A.tiles_m - mg * A.group_m) < A.group_m ? (A.tiles_m - mg * A.group_m)
                                                                  : A.group_m;
    const int64_t rr = r - mg * A.group_m * A.tiles_n;
    const int64_t tn = rr / gsz;
    const int64_t tm = mg * A.group_m + (rr - tn * gsz);
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // wave tile: rows wm*128, cols wn*64
    const int64_t K = A.I;
    const uint16_t *xb = A.x + b * A.xsb;
    const bool wvec = (A.wsm % 8 == 0) && ((reinterpret_cast<uintptr_t>(A.w) & 15u) == 0);
    const bool xvec = (A.xst % 8 == 0) && (A.xsb % 8 == 0) &&
                      ((reinterpret_cast<uintptr_t>(A.x) & 15u) == 0);

    // staging registers: the A tile is 256 rows x kCR chunks, the B tile
    // 128 x kCR, spread over the 256 threads
    constexpr int kAC = kBM * kCR / kThreads, kBC = kBN * kCR / kThreads;
    uint4 ra[kAC], rb[kBC];
#define PARARNN_PROJ_FETCH(K0)                                                                  \
    do {                                                                                        \
        _Pragma("unroll") for (int j = 0; j < kAC; ++j)                                         \
        {                                                                                       \
            const int c = tid + j * kThreads;                                                   \
            const int64_t m = m0 + c / kCR, k = (K0) + (c % kCR) * 8;                           \
            if constexpr (VEC) {                                                                \
                ra[j] = *reinterpret_cast<const uint4 *>(A.w + (m < A.M ? m : A.M - 1) * A.wsm + \
                                                         k);                                    \
            } else {                                                                            \
                ra[j] = load_chunk(A.w + m * A.wsm, k, K, m < A.M, wvec);                       \
            }                                                                                   \
        }                                                                                       \
        _Pragma("unroll") for (int j = 0; j < kBC; ++j)                                         \
        {                                                                                       \
            const int c = tid + j * kThreads;                                                   \
            const int64_t t = n0 + c / kCR, k = (K0) + (c % kCR) * 8;                           \
            if constexpr (VEC) {                                                                \
                rb[j] = *reinterpret_cast<const uint4 *>(xb + (t < A.T ? t : A.T - 1) * A.xst + \
                                                         k);                                    \
            } else {                                                                            \
                rb[j] = load_chunk(xb + t * A.xst, k, K, t < A.T, xvec);                        \
            }                                                                                   \
        }                                                                                       \
    } while (0)
#define PARARNN_PROJ_STASH(BUF)                                                                 \
    do {                                                                                        \
        _Pragma("unroll") for (int j = 0; j < kAC; ++j)                                         \
        {                                                                                       \
            const int c = tid + j * kThreads;                                                   \
            *reinterpret_cast<uint4 *>(&As[BUF][c / kCR][(c % kCR) * 8]) = ra[j];               \
        }                                                                                       \
        _Pragma("unroll") for (int j = 0; j < kBC; ++j)                                         \
        {                                                                                       \
            const int c = tid + j * kThreads;                                                   \
            *reinterpret_cast<uint4 *>(&Bs[BUF][c / kCR][(c % kCR) * 8]) = rb[j];               \
        }                                                                                       \
    } while (0)

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t steps = (K + kBK - 1) / kBK;
    const int ar = lane & 31, ak = (lane >> 5) * 8;  // operand row and k offset of this lane
    auto mma = [&](int buf) {
#pragma unroll
        for (int h = 0; h < kBK / 16; ++h) {
            bf16x8 fa[4], fb[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &As[buf][wm * 128 + i * 32 + ar][h * 16 + ak]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &Bs[buf][wn * 64 + j * 32 + ar][h * 16 + ak]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };
    // step s multiplies LDS stage s % 2 while stage s + 1 is in flight into
    // the staging registers; it is written to the other stage afterwards.
    // In the VEC case the loads are unconditional (past the last stage they
    // reread it), so the compiler can count them instead of waiting for all.
    const int64_t last = steps > 0 ? (steps - 1) * kBK : 0;
    if (steps > 0) {
        PARARNN_PROJ_FETCH(0);
        PARARNN_PROJ_STASH(0);
    }
    __syncthreads();
    for (int64_t s = 0; s < steps; ++s) {
        const int64_t kn = (s + 1) * kBK < last ? (s + 1) * kBK : last;
        if (VEC || s + 1 < steps) PARARNN_PROJ_FETCH(kn);
        mma((int)(s & 1));
        if (s + 1 < steps) PARARNN_PROJ_STASH((int)((s + 1) & 1));
        __syncthreads();
    }
#undef PARARNN_PROJ_FETCH
#undef PARARNN_PROJ_STASH

    // epilogue: accumulator r of block (i, j) holds row
    // 8 (r / 4) + 4 (lane / 32) + r % 4 and column lane % 32 of that block
    const int64_t col_base = n0 + wn * 64 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m >= A.M) continue;
            const float bias = A.bias ? A.bias[m] : 0.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t t = col_base + j * 32;
                if (t >= A.T) continue;
                const float v = acc[i][j][r] + bias;
                const int64_t off = b * A.usb + m * A.usm + t;
                if (A.out_bf16)
                    static_cast<uint16_t *>(A.u)[off] = f32_to_bf16_rne(v);
                else
                    static_cast<float *>(A.u)[off] = v;
            }
        }
    }
}
#endif

}  // namespace pararnn
