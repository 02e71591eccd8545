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
// Two kernels.  Aligned operands (I % 64 == 0, 16-byte aligned rows) take
// the ring kernel: a 512-thread workgroup computes a 256 (m) x 256 (t) tile,
// each of its 8 waves a 128 x 64 tile as 4 x 2 MFMA 32x32 blocks; operand
// tiles stream from memory straight into LDS (16-byte global->LDS copies,
// whole 128-byte rows per k step of 64: the copy path runs at half rate on
// half lines) through a 2-stage ring, rows XOR-swizzled so the 16-byte
// operand reads are bank-conflict free.  Anything else takes the register-
// staged kernel: 256 x 128 tiles, k steps of 32 through two padded LDS
// stages, per-element checked loads.  Both order tiles per XCD and in groups
// of m tiles so that the workgroups in flight on one XCD share their
// operands in its L2.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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

#ifndef PARARNN_PROJ_BN
#define PARARNN_PROJ_BN 128
#endif
#ifndef PARARNN_PROJ_BK
#define PARARNN_PROJ_BK 32
#endif
#ifndef PARARNN_PROJ_OCC
#define PARARNN_PROJ_OCC 2
#endif
constexpr int kBM = 256, kBN = PARARNN_PROJ_BN, kBK = PARARNN_PROJ_BK;
constexpr int kWM = kBM / 2, kWN = kBN / 2;  // wave tile (2 x 2 waves)
constexpr int kMB = kWM / 32, kNB = kWN / 32;  // 32x32 MFMA blocks per wave
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

// ---- direct-to-LDS ring (aligned operands)
// A stage holds the A tile (kBM rows) then the B tile (kBN rows), each row
// kBK bf16 = kCR 16-byte chunks, unpadded; chunk c of row r sits at chunk
// position c ^ swz(r), so the 16-byte operand reads of 8 (or 16) consecutive
// lanes — 8 (16) consecutive rows at one chunk — fall on distinct banks.
#ifndef PARARNN_PROJ_RING_BN
#define PARARNN_PROJ_RING_BN 256
#endif
#ifndef PARARNN_PROJ_RING_BK
#define PARARNN_PROJ_RING_BK 64
#endif
#ifndef PARARNN_PROJ_RING_WAVES
#define PARARNN_PROJ_RING_WAVES 8
#endif
#ifndef PARARNN_PROJ_RING_WM
#define PARARNN_PROJ_RING_WM 2
#endif
#ifndef PARARNN_PROJ_RING_STAGES
#define PARARNN_PROJ_RING_STAGES 2
#endif
#ifndef PARARNN_PROJ_RING_OCC
#define PARARNN_PROJ_RING_OCC 2
#endif
constexpr int kRBN = PARARNN_PROJ_RING_BN, kRBK = PARARNN_PROJ_RING_BK;
constexpr int kRWaves = PARARNN_PROJ_RING_WAVES, kRThreads = 64 * kRWaves;
constexpr int kRWMw = PARARNN_PROJ_RING_WM, kRWNw = kRWaves / kRWMw;  // wave grid
constexpr int kRWM = kBM / kRWMw, kRWN = kRBN / kRWNw;              // wave tile
constexpr int kRMB = kRWM / 32, kRNB = kRWN / 32;                    // MFMA blocks
constexpr int kStages = PARARNN_PROJ_RING_STAGES;
constexpr int kRCR = kRBK / 8;                                        // chunks per row
constexpr int kRowBytes = kRBK * 2;
constexpr int kAStage = kBM * kRowBytes, kStageBytes = (kBM + kRBN) * kRowBytes;
constexpr int kAQ = kBM * kRCR / 64 / kRWaves, kBQ = kRBN * kRCR / 64 / kRWaves;  // copies per wave
constexpr int kPerStage = kAQ + kBQ;
static_assert(kAQ * 64 * kRWaves == kBM * kRCR && kBQ * 64 * kRWaves == kRBN * kRCR,
              "stage must split evenly into 1 KB copies");
static_assert(kRMB >= 1 && kRNB >= 1 && (kStages - 2) * kPerStage < 64, "ring shape");
// Chunk position of memory chunk c in tile row r: c ^ swz(r).  16-byte reads
// of 8 (or 16) consecutive rows at one chunk then hit distinct banks.
__device__ __forceinline__ int swz(int r)
{
    if constexpr (kRCR == 8)
        return (r ^ (r >> 3)) & 7;
    else
        return ((r >> 1) ^ (r >> 2)) & 3;
}

// A wave-uniform pointer, moved to scalar registers (the asm below takes its
// base address in an SGPR pair).
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void copy_to_lds(uint32_t voff, const void *sbase, uint32_t lds)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
}


}  // namespace proj

#ifdef PARARNN_DEFINE_PROJECT_KERNEL  // compiled once, in its own translation unit
// Epilogue rows: accumulator e of block (i, j) holds row
// 8 (e / 4) + 4 (lane / 32) + e % 4 and column lane % 32 of that block, so
// this lane writes rows mrow0 + 32 i + 8 g + r (g, r < 4) at columns
// tcol0 + 32 j.  FULL: the tile lies inside M x T (no per-element checks).
template <bool BF16OUT, bool FULL>
__device__ __forceinline__ void store_rows(const ProjArgs &A, int64_t b, int64_t mrow0,
                                           int64_t tcol0,
                                           const proj::f32x16 (&acc)[proj::kRMB][proj::kRNB],
                                           const float (&bias)[proj::kRMB][4][4])
{
    using namespace proj;
    using Out = typename std::conditional<BF16OUT, __bf16, float>::type;
    Out *u = static_cast<Out *>(A.u) + b * A.usb + tcol0;
#pragma unroll
    for (int i = 0; i < kRMB; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = mrow0 + i * 32 + 8 * g + r;
                if (!FULL && m >= A.M) continue;
                Out *row = u + m * A.usm;
#pragma unroll
                for (int j = 0; j < kRNB; ++j) {
                    if (!FULL && tcol0 + j * 32 >= A.T) continue;
                    row[j * 32] = (Out)(acc[i][j][4 * g + r] + bias[i][g][r]);
                }
            }
}

// Epilogue of both kernels (their waves hold the same 128 x 64 tile shape):
// bias, then fp32 or bf16 (the hardware's round-to-nearest-even conversion)
// stores.  full_m / full: the tile's rows / rows and columns all exist.
__device__ __forceinline__ void store_tile(const ProjArgs &A, int64_t b, int64_t mrow0,
                                           int64_t tcol0, bool full, bool full_m,
                                           const proj::f32x16 (&acc)[proj::kRMB][proj::kRNB])
{
    using namespace proj;
    // bias of this lane's rows: four consecutive rows per 16-byte load when
    // the tile's rows all exist and the bias array is 16-byte aligned
    float bias[kRMB][4][4];
    const bool bvec = full_m && (reinterpret_cast<uintptr_t>(A.bias) & 15u) == 0;
#pragma unroll
    for (int i = 0; i < kRMB; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t m = mrow0 + i * 32 + 8 * g;
            if (A.bias && bvec) {
                const float4 v = *reinterpret_cast<const float4 *>(A.bias + m);
                bias[i][g][0] = v.x;
                bias[i][g][1] = v.y;
                bias[i][g][2] = v.z;
                bias[i][g][3] = v.w;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    bias[i][g][r] = (A.bias && m + r < A.M) ? A.bias[m + r] : 0.0f;
            }
        }
    if (A.out_bf16) {
        if (full)
            store_rows<true, true>(A, b, mrow0, tcol0, acc, bias);
        else
            store_rows<true, false>(A, b, mrow0, tcol0, acc, bias);
    } else {
        if (full)
            store_rows<false, true>(A, b, mrow0, tcol0, acc, bias);
        else
            store_rows<false, false>(A, b, mrow0, tcol0, acc, bias);
    }
}

// VEC: every row of x and W is 16-byte aligned and I % 32 == 0, so every
// chunk of every stage lies inside its row: unconditional vector loads (rows
// past M or T read a valid row whose results are not stored).
template <bool VEC>
__global__ void __launch_bounds__(proj::kThreads, PARARNN_PROJ_OCC) project_kernel(ProjArgs A)
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
    const int wm = wave >> 1, wn = wave & 1;  // wave tile: rows wm*kWM, cols wn*kWN
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

    f32x16 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t steps = (K + kBK - 1) / kBK;
    const int ar = lane & 31, ak = (lane >> 5) * 8;  // operand row and k offset of this lane
    auto mma = [&](int buf) {
#pragma unroll
        for (int h = 0; h < kBK / 16; ++h) {
            bf16x8 fa[kMB], fb[kNB];
#pragma unroll
            for (int i = 0; i < kMB; ++i)
                fa[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &As[buf][wm * kWM + i * 32 + ar][h * 16 + ak]));
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                fb[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &Bs[buf][wn * kWN + j * 32 + ar][h * 16 + ak]));
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
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

    static_assert(kMB == kRMB && kNB == kRNB, "both kernels share the epilogue");
    store_tile(A, b, m0 + wm * 128 + 4 * (lane >> 5), n0 + wn * 64 + (lane & 31),
               m0 + kBM <= A.M && n0 + kBN <= A.T, m0 + kBM <= A.M, acc);
}

// Aligned operands (I % kRBK == 0, 16-byte aligned rows): tiles stream
// straight into a ring of kStages LDS stages; while stage s is multiplied,
// stages s + 1 .. s + kStages - 1 are in flight, one barrier per step.  Each
// copy moves whole 128-byte rows when kRBK = 64 (the load path runs at half
// rate on half lines).
__global__ void __launch_bounds__(proj::kRThreads, PARARNN_PROJ_RING_OCC)
    project_kernel_ring(ProjArgs A)
{
    using namespace proj;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][kStageBytes];

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
    const int64_t m0 = tm * kBM, n0 = tn * kRBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / kRWNw, wn = wave % kRWNw;
    const int64_t K = A.I;
    const int steps = (int)(K / kRBK);

    // copy plan: copy q of this wave fills 1 KB block q * kRWaves + wave of
    // the A (then B) tile; lane l of it takes chunk position p = 64 block + l,
    // i.e. tile row p / kRCR and memory chunk (p % kRCR) ^ swz(row).  Rows
    // past M or T read the last row (their results are not stored).
    const uint8_t *wbase = uniform_ptr(reinterpret_cast<const uint8_t *>(A.w + m0 * A.wsm));
    const uint8_t *xbase =
        uniform_ptr(reinterpret_cast<const uint8_t *>(A.x + b * A.xsb + n0 * A.xst));
    uint32_t voa[kAQ], vob[kBQ];
#pragma unroll
    for (int q = 0; q < kAQ; ++q) {
        const int p = (q * kRWaves + wave) * 64 + lane, row = p / kRCR;
        const int64_t m = m0 + row < A.M ? m0 + row : A.M - 1;
        voa[q] = (uint32_t)(((m - m0) * A.wsm + ((p % kRCR) ^ swz(row)) * 8) * 2);
    }
#pragma unroll
    for (int q = 0; q < kBQ; ++q) {
        const int p = (q * kRWaves + wave) * 64 + lane, row = p / kRCR;
        const int64_t t = n0 + row < A.T ? n0 + row : A.T - 1;
        vob[q] = (uint32_t)(((t - n0) * A.xst + ((p % kRCR) ^ swz(row)) * 8) * 2);
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>(&ring[0][0]) + wave * 1024);
    auto issue = [&](int s) {
        const uint32_t l = lds0 + (uint32_t)((s % kStages) * kStageBytes);
        const int64_t kb = (int64_t)s * kRowBytes;
#pragma unroll
        for (int q = 0; q < kAQ; ++q) copy_to_lds(voa[q], wbase + kb, l + q * kRWaves * 1024);
#pragma unroll
        for (int q = 0; q < kBQ; ++q)
            copy_to_lds(vob[q], xbase + kb, l + kAStage + q * kRWaves * 1024);
    };

    f32x16 acc[kRMB][kRNB];
#pragma unroll
    for (int i = 0; i < kRMB; ++i)
#pragma unroll
        for (int j = 0; j < kRNB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // operand row of this lane in block i (j): base + 32 i + lane % 32; the
    // k16 step h reads memory chunk 2 h + lane / 32 of it
    const int lr = lane & 31, lh = lane >> 5;
    auto a_off = [&](int i, int h) {
        const int row = wm * kRWM + i * 32 + lr;
        return row * kRowBytes + (((2 * h + lh) ^ swz(row)) * 16);
    };
    auto b_off = [&](int j, int h) {
        const int row = wn * kRWN + j * 32 + lr;
        return kAStage + row * kRowBytes + (((2 * h + lh) ^ swz(row)) * 16);
    };

    for (int s = 0; s < kStages - 1 && s < steps; ++s) issue(s);
    for (int s = 0; s < steps; ++s) {
        // this wave's copies of stage s have landed (later stages may fly)
        if (kStages > 2 && s + kStages - 2 < steps)
            __builtin_amdgcn_s_waitcnt(0x0F70 | ((kStages - 2) * kPerStage & 15) |
                                       (((kStages - 2) * kPerStage >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_s_barrier();  // all copies of stage s landed; stage s - 1 is free
        asm volatile("" ::: "memory");
        if (s + kStages - 1 < steps) issue(s + kStages - 1);
        const uint8_t *st = &ring[s % kStages][0];
#ifndef PARARNN_PROJ_RING_AHEAD
#define PARARNN_PROJ_RING_AHEAD 2
#endif
        // operand reads of PARARNN_PROJ_RING_AHEAD k16 steps first, then
        // their products: the first products wait only for their own operands
        constexpr int kAh = PARARNN_PROJ_RING_AHEAD;
#pragma unroll
        for (int h2 = 0; h2 < kRBK / 16 / kAh; ++h2) {
            bf16x8 fa[kAh][kRMB], fb[kAh][kRNB];
#pragma unroll
            for (int hh = 0; hh < kAh; ++hh) {
#pragma unroll
                for (int i = 0; i < kRMB; ++i)
                    fa[hh][i] = as_bf16x8(
                        *reinterpret_cast<const uint4 *>(st + a_off(i, kAh * h2 + hh)));
#pragma unroll
                for (int j = 0; j < kRNB; ++j)
                    fb[hh][j] = as_bf16x8(
                        *reinterpret_cast<const uint4 *>(st + b_off(j, kAh * h2 + hh)));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int hh = 0; hh < kAh; ++hh)
#pragma unroll
                for (int i = 0; i < kRMB; ++i)
#pragma unroll
                    for (int j = 0; j < kRNB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fa[hh][i], fb[hh][j], acc[i][j], 0, 0, 0);
        }
        asm volatile("" ::: "memory");
    }

    store_tile(A, b, m0 + wm * kRWM + 4 * (lane >> 5), n0 + wn * kRWN + (lane & 31),
               m0 + kBM <= A.M && n0 + kRBN <= A.T, m0 + kBM <= A.M, acc);
}
#endif

}  // namespace pararnn
