// Device primitives for the ParaRNN / DEER solve on gfx950 (CDNA4, wave64):
// fast transcendentals, the affine maps the Newton systems are made of, and
// wavefront-level scans built on DPP lane moves.
//
// Source of the scan structure: "Параллельность RNN?" (forpes.ru), §1.3,
// level 2 — the linear recurrence ds_t = A_t ds_{t-1} + b_t is associative
// because composing affine maps is; any bracketing of the composition gives
// the same prefixes, so each channel's length-T recurrence is split into
// per-lane serial chunks, a 64-lane wavefront scan, a scan over the waves of
// a workgroup and a carry across workgroups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pararnn {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------- arithmetic ---

__device__ __forceinline__ float fmaf_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
// v_exp_f32: 2^x.  v_rcp_f32: 1/x (1 ulp).  Both saturate cleanly:
// 2^(+big) = +inf, 1/inf = 0, so the sigmoid/tanh forms below need no
// clamping.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcpf_(float x) { return __builtin_amdgcn_rcpf(x); }

// sig(p) given q = -log2(e) * p.
__device__ __forceinline__ float sigmoid_q(float q) { return rcpf_(1.0f + ex2(q)); }
// tanh(p) given q = -2 log2(e) * p:  tanh p = 2 / (1 + e^{-2p}) - 1.
__device__ __forceinline__ float tanh_q(float q) { return fmaf_(2.0f, rcpf_(1.0f + ex2(q)), -1.0f); }

// |x| as an unsigned bit pattern.  For non-negative floats unsigned order is
// float order and every NaN pattern is larger than +inf, so an unsigned max
// over these never loses a NaN (IEEE fmax would).
__device__ __forceinline__ uint32_t absbits(float x) { return __float_as_uint(x) & 0x7fffffffu; }
// Running max of |x| that propagates NaN (IEEE 754-2019 maximum; CDNA4 has
// it as v_maximum3_f32 with |.| source modifiers, two new values per op).
__device__ __forceinline__ float max_abs(float m, float x)
{
    return __builtin_elementwise_maximum(m, __builtin_fabsf(x));
}

// ---------------------------------------------------------- affine maps ---
// A map x -> A x + b.  compose(L, E) applies E first, then L:
//   (A_L, b_L) o (A_E, b_E) = (A_L A_E, A_L b_E + b_L).
// apply() is the only place a map meets a vector: every carry in the
// library goes through it, so two places that apply the same map to the
// same vector get the same bits.

// 8-byte aligned so a map in LDS moves as one 64-bit access whose
// immediate offset reaches every step's slot from one base address.
struct alignas(8) Map1 {  // diagonal Jacobian (ParaGRU): 1x1 per channel
    float a, b;
};
__device__ __forceinline__ Map1 identity_map(Map1) { return {1.0f, 0.0f}; }
__device__ __forceinline__ Map1 compose(const Map1 &L, const Map1 &E)
{
    return {L.a * E.a, fmaf_(L.a, E.b, L.b)};
}
struct Vec1 {
    float x;
};
// running max of |b| (the residual part of a step map), NaN-propagating
__device__ __forceinline__ float resmax(float mx, const Map1 &m) { return max_abs(mx, m.b); }
// the identity where `keep` is false (select, no branch)
__device__ __forceinline__ Map1 keep_or_identity(const Map1 &m, bool keep)
{
    return {keep ? m.a : 1.0f, keep ? m.b : 0.0f};
}
__device__ __forceinline__ Vec1 apply(const Map1 &m, const Vec1 &v) { return {fmaf_(m.a, v.x, m.b)}; }
__device__ __forceinline__ float resmax(float mx, const Vec1 &r) { return max_abs(mx, r.x); }
// The same value, but one the compiler cannot prove equal to its source
// (an empty asm that claims to modify it).
__device__ __forceinline__ float opaque(float x)
{
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ Vec1 opaque(const Vec1 &v) { return {opaque(v.x)}; }
__device__ __forceinline__ Vec1 keep_or_zero(const Vec1 &v, bool keep) { return {keep ? v.x : 0.0f}; }

struct Map2 {  // 2x2 block Jacobian (ParaLSTM), state order (c, h)
    float a00, a01, a10, a11, b0, b1;
};
__device__ __forceinline__ Map2 identity_map(Map2) { return {1.0f, 0.0f, 0.0f, 1.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ Map2 compose(const Map2 &L, const Map2 &E)
{
    Map2 r;
    r.a00 = fmaf_(L.a00, E.a00, L.a01 * E.a10);
    r.a01 = fmaf_(L.a00, E.a01, L.a01 * E.a11);
    r.a10 = fmaf_(L.a10, E.a00, L.a11 * E.a10);
    r.a11 = fmaf_(L.a10, E.a01, L.a11 * E.a11);
    r.b0 = fmaf_(L.a00, E.b0, fmaf_(L.a01, E.b1, L.b0));
    r.b1 = fmaf_(L.a10, E.b0, fmaf_(L.a11, E.b1, L.b1));
    return r;
}
struct Vec2 {
    float x0, x1;
};
__device__ __forceinline__ float resmax(float mx, const Map2 &m)
{
    return max_abs(max_abs(mx, m.b0), m.b1);
}
__device__ __forceinline__ Map2 keep_or_identity(const Map2 &m, bool keep)
{
    return {keep ? m.a00 : 1.0f, keep ? m.a01 : 0.0f, keep ? m.a10 : 0.0f,
            keep ? m.a11 : 1.0f, keep ? m.b0 : 0.0f,  keep ? m.b1 : 0.0f};
}
__device__ __forceinline__ Vec2 apply(const Map2 &m, const Vec2 &v)
{
    return {fmaf_(m.a00, v.x0, fmaf_(m.a01, v.x1, m.b0)),
            fmaf_(m.a10, v.x0, fmaf_(m.a11, v.x1, m.b1))};
}
__device__ __forceinline__ float resmax(float mx, const Vec2 &r)
{
    return max_abs(max_abs(mx, r.x0), r.x1);
}
__device__ __forceinline__ Vec2 opaque(const Vec2 &v) { return {opaque(v.x0), opaque(v.x1)}; }
__device__ __forceinline__ Vec2 keep_or_zero(const Vec2 &v, bool keep)
{
    return {keep ? v.x0 : 0.0f, keep ? v.x1 : 0.0f};
}

// ------------------------------------------------------------ DPP moves ---
// update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl=false): lanes
// whose source lane is out of range, or whose row is masked off, keep `old`.
// GFX9 controls used: row_shr:n = 0x110+n, wave_shr:1 = 0x138,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ float dppf(float old, float src)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                      CTRL, RM, 0xF, false));
}
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint32_t dppu(uint32_t old, uint32_t src)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, RM, 0xF, false);
}

template <int CTRL, int RM = 0xF>
__device__ __forceinline__ Map1 dpp_map(const Map1 &x)
{
    return {dppf<CTRL, RM>(1.0f, x.a), dppf<CTRL, RM>(0.0f, x.b)};
}
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ Map2 dpp_map(const Map2 &x)
{
    return {dppf<CTRL, RM>(1.0f, x.a00), dppf<CTRL, RM>(0.0f, x.a01),
            dppf<CTRL, RM>(0.0f, x.a10), dppf<CTRL, RM>(1.0f, x.a11),
            dppf<CTRL, RM>(0.0f, x.b0),  dppf<CTRL, RM>(0.0f, x.b1)};
}

// Inclusive scan over the 64 lanes in lane order: lane l ends with
// x_l o x_{l-1} o ... o x_0.  Hillis-Steele inside each 16-lane row
// (row_shr 1, 2, 4, 8), then row 0's total into row 1 and row 2's into
// row 3 (row_bcast:15), then lanes 0..31's total into rows 2 and 3
// (row_bcast:31).  Lanes that receive nothing compose with the identity.
template <class M>
__device__ __forceinline__ M wave_scan_inclusive(M x)
{
    x = compose(x, dpp_map<0x111>(x));
    x = compose(x, dpp_map<0x112>(x));
    x = compose(x, dpp_map<0x114>(x));
    x = compose(x, dpp_map<0x118>(x));
    x = compose(x, dpp_map<0x142, 0xA>(x));
    x = compose(x, dpp_map<0x143, 0xC>(x));
    return x;
}

// One level of the 1x1 scan with the lane shift folded into the arithmetic
// (two DPP instructions instead of two moves, two identity fills and two
// products): b += a * b[src] with a missing source reading 0 (bound_ctrl),
// then a *= a[src] with a missing source leaving the lane as it is.  Same
// operations in the same order as compose(x, dpp_map(x)), so the same bits.
// A DPP read needs two wait states after the VALU write of its source.
#define PARARNN_SCAN1_LEVEL(DPP)                                                      \
    asm volatile("s_nop 1\n\t"                                                         \
                 "v_fmac_f32_dpp %1, %1, %0 " DPP " bound_ctrl:1\n\t"                   \
                 "s_nop 1\n\t"                                                         \
                 "v_mul_f32_dpp %0, %0, %0 " DPP "\n\t"                                 \
                 "s_nop 1"                                                               \
                 : "+v"(x.a), "+v"(x.b))
template <>
__device__ __forceinline__ Map1 wave_scan_inclusive<Map1>(Map1 x)
{
    PARARNN_SCAN1_LEVEL("row_shr:1 row_mask:0xf bank_mask:0xf");
    PARARNN_SCAN1_LEVEL("row_shr:2 row_mask:0xf bank_mask:0xf");
    PARARNN_SCAN1_LEVEL("row_shr:4 row_mask:0xf bank_mask:0xf");
    PARARNN_SCAN1_LEVEL("row_shr:8 row_mask:0xf bank_mask:0xf");
    PARARNN_SCAN1_LEVEL("row_bcast:15 row_mask:0xa bank_mask:0xf");
    PARARNN_SCAN1_LEVEL("row_bcast:31 row_mask:0xc bank_mask:0xf");
    return x;
}
#undef PARARNN_SCAN1_LEVEL

// Value of lane l-1 (identity at lane 0): turns the inclusive scan into the
// exclusive one.
template <class M>
__device__ __forceinline__ M wave_shift_up(const M &x) { return dpp_map<0x138>(x); }

// Max over the 64 lanes, valid in lane 63 (same data movement as the scan).
__device__ __forceinline__ uint32_t wave_max_to_last(uint32_t x)
{
    x = max(x, dppu<0x111>(0u, x));
    x = max(x, dppu<0x112>(0u, x));
    x = max(x, dppu<0x114>(0u, x));
    x = max(x, dppu<0x118>(0u, x));
    x = max(x, dppu<0x142, 0xA>(0u, x));
    x = max(x, dppu<0x143, 0xC>(0u, x));
    return x;
}

// Sum over the 64 lanes, valid in lane 63.
__device__ __forceinline__ float wave_sum_to_last(float x)
{
    x += dppf<0x111>(0.0f, x);
    x += dppf<0x112>(0.0f, x);
    x += dppf<0x114>(0.0f, x);
    x += dppf<0x118>(0.0f, x);
    x += dppf<0x142, 0xA>(0.0f, x);
    x += dppf<0x143, 0xC>(0.0f, x);
    return x;
}

// ------------------------------------------------ device-scope flag ops ---
// Cross-workgroup records are written and read only with device-coherent
// (agent-scope) atomic accesses, which go to the coherence point themselves;
// so publishing needs no cache maintenance, only ordering.  A release/acquire
// fence at agent scope would write back / invalidate the XCD's whole L2 on
// every publish, which costs far more than the exchange itself.
__device__ __forceinline__ float load_relaxed(const float *p)
{
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void store_relaxed(float *p, float v)
{
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_flag(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt through the builtin rather than inline asm, so the compiler's own
// wait insertion sees it and does not add a second, blanket vmcnt(0) later
// (it cannot look inside an asm block).  gfx9 immediate: vmcnt in bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]; all-ones = no wait.  The
// empty asm keeps the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("" ::: "memory");
}
// Flag store ordered after every earlier store of this lane: wait until those
// have completed (reached the coherence point), then write the flag.
__device__ __forceinline__ void publish_flag(int32_t *p, int32_t v)
{
    wait_vm();
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// After a flag read has returned the awaited value: keep the compiler from
// hoisting the payload loads above it (the hardware issues them after the
// flag value was consumed by the branch).
__device__ __forceinline__ void after_flag() { asm volatile("" ::: "memory"); }

}  // namespace pararnn
