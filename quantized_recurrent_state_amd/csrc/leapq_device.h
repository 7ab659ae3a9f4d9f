// Device-side building blocks shared by the libleapq kernels (gfx950).
//
// Arithmetic: IEEE binary32, no contraction (-ffp-contract=off; every fused
// multiply-add is an explicit __builtin_fmaf), correctly rounded '/' and
// sqrtf, subnormals kept.  Every sum that feeds a stored value follows one
// canonical order, the 128-term halving tree: level 0 combines element e
// with element e+64 (for a dot product fma(a_e, b_e, a_{e+64} * b_{e+64}),
// for a plain sum x_e + x_{e+64}), then levels h = 32, 16, ..., 1 add partial
// e and partial e+h.  The cross-lane steps below only move data; every sum is
// an ordinary fp32 add of exactly the tree's pair, and fp32 addition is
// commutative, so any lane order that pairs the same partials gives the same
// bits.
//
// Thread map of a 256-thread workgroup that owns one head: wave w (0..3),
// lane l (0..63),
//     i  = (l & 3) | (l >> 3) << 2      key rows  i + 32p,  p = 0..3
//     hb = (l >> 2) & 1,  j = w + 4 hb  value columns j + 8m, m = 0..15
// A column sum over the 128 rows therefore runs: levels 0 and 1 inside the
// thread (rows i, i+64 and i+32, i+96), then levels h = 16, 8, 4, 2, 1 on
// lane bits 5, 4, 3, 1, 0: a v_permlane32_swap, a v_permlane16_swap and three
// exact-xor DPP moves, all inside one wave.  A row sum over the 128 columns
// runs: levels 0..3 inside the thread (columns j+8m), level 4 on lane bit 2
// (DPP), levels 5 and 6 across waves w^2, w^1 through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "leapq_internal.h"

namespace leapq {
namespace dev {

constexpr int D = 128;
constexpr int NT = 256;

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// ---------------------------------------------------------------- thread map
struct AMap {
    int w, l, i, hb, j;
    __device__ __forceinline__ int row(int p) const { return i + 32 * p; }
    __device__ __forceinline__ int col(int m) const { return j + 8 * m; }
};

__device__ __forceinline__ AMap amap()
{
    AMap a;
    a.l = threadIdx.x & 63;
    a.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    a.i = (a.l & 3) | ((a.l >> 3) << 2);
    a.hb = (a.l >> 2) & 1;
    a.j = a.w + 4 * a.hb;
    return a;
}

// ---------------------------------------------------------------- layouts
// Record keys are stored with key row r at 4*(r % 32) + r / 32 (a thread's 4
// rows are one float4); record corrections with value column c at
// 16*(c % 8) + c / 8 (a thread's 16 columns are four float4s), the same
// interleave as the codes of a row.
__device__ __forceinline__ int kpos(int r) { return 4 * (r & 31) + (r >> 5); }
__device__ __forceinline__ int upos(int c) { return 16 * (c & 7) + (c >> 3); }

struct HeadState {
    int8_t *codes;
    float *rho, *sigma;
    int32_t *cidx;
    float *cvec;
    float *rgam, *rk, *ru;
};

__device__ __forceinline__ HeadState head_state(const StateView &sv, int h)
{
    HeadState s;
    s.codes = sv.codes + (size_t)h * D * D;
    s.rho = sv.rho + (size_t)h * D;
    s.sigma = sv.sigma + (size_t)h * D;
    s.cidx = sv.cidx + (size_t)h * sv.C;
    s.cvec = sv.cvec + (size_t)h * sv.C * D;
    s.rgam = sv.rgam + (size_t)h * sv.W;
    s.rk = sv.rk + (size_t)h * sv.W * D;
    s.ru = sv.ru + (size_t)h * sv.W * D;
    return s;
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x007fffffu)) return (uint16_t)((b >> 16) | 0x40);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

template <typename T>
__device__ __forceinline__ float ld_in(const T *p, int e);
template <>
__device__ __forceinline__ float ld_in<float>(const float *p, int e) { return p[e]; }
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t *p, int e) { return bf16_to_f32(p[e]); }

// int8 code b of a packed word, as fp32 (exact)
__device__ __forceinline__ float code_f(uint32_t word, int b) { return (float)(int8_t)(word >> (8 * b)); }

// ---------------------------------------------------------------- data movement
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                 false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int DPP_QREV = 0x1B;   // quad_perm [3,2,1,0]: lane ^ 3
constexpr int DPP_HMIR = 0x141;  // row_half_mirror: lane -> 7 - lane within 8
constexpr int DPP_ROR8 = 0x128;  // row_ror:8: lane ^ 8 within a 16-lane row
constexpr int DPP_ROR4 = 0x124;  // row_ror:4: lane ^ 4 once values agree across lane ^ 8

// lane ^ 4 exactly: half-mirror then quad reversal, (7 - l) ^ 3 == l ^ 4
__device__ __forceinline__ float xor4(float x) { return dpp<DPP_QREV>(dpp<DPP_HMIR>(x)); }
__device__ __forceinline__ int xor4i(int x) { return dppi<DPP_QREV>(dppi<DPP_HMIR>(x)); }

// v_permlane32_swap / v_permlane16_swap exchange the upper 32 lanes (odd
// 16-lane rows) of the first operand with the lower 32 lanes (even rows) of
// the second.  With (K, G) the lower lane of each pair ends with (own K,
// partner's K) and the upper lane with (partner's G, own G): the sum of the
// two results is the exchange-and-add of one tree level, the lower lane
// keeping K and the upper lane G.
__device__ __forceinline__ float xhalf32(float K, float G)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(K), __float_as_uint(G), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf16(float K, float G)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(K), __float_as_uint(G), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xmax32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax16(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int xmin32i(int x)
{
    auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return min((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int xmin16i(int x)
{
    auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return min((int)r[0], (int)r[1]);
}
// exchange-and-add over an exact-xor DPP pattern: lower lane keeps K, upper G
template <int CTRL>
__device__ __forceinline__ float xhalf_dpp(float K, float G, bool upper)
{
    const float send = upper ? K : G;
    return (upper ? G : K) + dpp<CTRL>(send);
}

// Canonical 128-term dot of (a0 = a[l], a1 = a[l+64]) and (b0, b1) over one
// wave: level 0 fma(a0, b0, a1*b1), then levels 32..1 as a butterfly; every
// lane ends with the same value.
__device__ __forceinline__ float wdot(float a0, float a1, float b0, float b1)
{
    float s = fma_(a0, b0, a1 * b1);
    s = xhalf32(s, s);
    s = xhalf16(s, s);
    s = s + dpp<DPP_ROR8>(s);
    s = s + dpp<DPP_ROR4>(s);
    s = s + dpp<DPP_XOR2>(s);
    s = s + dpp<DPP_XOR1>(s);
    return s;
}

// wave-wide max / min (order-free); every lane ends with the result
__device__ __forceinline__ float wave_max(float x)
{
    x = xmax32(x);
    x = xmax16(x);
    x = fmaxf(x, dpp<DPP_ROR8>(x));
    x = fmaxf(x, dpp<DPP_ROR4>(x));
    x = fmaxf(x, dpp<DPP_XOR2>(x));
    return fmaxf(x, dpp<DPP_XOR1>(x));
}
__device__ __forceinline__ int wave_min(int x)
{
    x = xmin32i(x);
    x = xmin16i(x);
    x = min(x, dppi<DPP_ROR8>(x));
    x = min(x, dppi<DPP_ROR4>(x));
    x = min(x, dppi<DPP_XOR2>(x));
    return min(x, dppi<DPP_XOR1>(x));
}

// Column sum over the 128 rows, from the 16 level-1 partials v[m] (column
// j+8m) of each thread.  Returns the sum of the lane's column
// j + 8 * colm(l), colm(l) = (l>>5&1)<<3 | (l>>4&1)<<2 | (l>>3&1)<<1 | (l>>1&1);
// lanes l and l^1 hold the same column.
__device__ __forceinline__ int colm_of(int l)
{
    return (((l >> 5) & 1) << 3) | (((l >> 4) & 1) << 2) | (((l >> 3) & 1) << 1) | ((l >> 1) & 1);
}
__device__ __forceinline__ float colsum16(const float (&v)[16], int l)
{
    float a8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a8[e] = xhalf32(v[e], v[e + 8]);
    float a4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a4[e] = xhalf16(a8[e], a8[e + 4]);
    float a2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) a2[e] = xhalf_dpp<DPP_ROR8>(a4[e], a4[e + 2], (l >> 3) & 1);
    const float a1 = xhalf_dpp<DPP_XOR2>(a2[0], a2[1], (l >> 1) & 1);
    return a1 + dpp<DPP_XOR1>(a1);
}

// Row partial over a thread's 16 columns of one row (levels 0..3 of the
// tree over columns), as a dot of the row with itself.
__device__ __forceinline__ float row_energy16(const float (&x)[16])
{
    float t[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) t[m] = fma_(x[m], x[m], x[m + 8] * x[m + 8]);
#pragma unroll
    for (int m = 0; m < 4; ++m) t[m] = t[m] + t[m + 4];
    t[0] = t[0] + t[2];
    t[1] = t[1] + t[3];
    return t[0] + t[1];
}

// ---------------------------------------------------------------- LDS-direct copies
__device__ __forceinline__ void lds_copy16(const void *g, float *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 4, 0, 0);
}
__device__ __forceinline__ float rdl(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(x), lane));
}

}  // namespace dev
}  // namespace leapq
