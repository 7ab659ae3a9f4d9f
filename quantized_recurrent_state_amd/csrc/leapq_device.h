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
// Thread map of the quantized-state kernels (init, append, fold, dequant):
// a 256-thread workgroup owns one head; wave w (0..3), lane l (0..63),
//     h = l >> 5,  jp = l & 31,  i = jp ^ (jp & 4 ? 3 : 0)
//     key rows      i + 32 p,         p = 0..3
//     value columns w + 4 h + 8 m,    m = 0..15
// This is the accumulator layout of v_mfma_f32_32x32x1_2b_f32 with the key
// on the B operand (B lane 32b + jp carries row i + 32 (2q + b) of matrix
// instruction q) and the value on the A operand (A lane a carries column
// w + 4 ((a >> 2) & 1) + 8 ((a & 3) | (a >> 3 & 3) << 2)), so the fold's
// rank-one record updates run on the matrix cores, one K = 1 step each, which
// rounds exactly like an fma.
// A column sum over the 128 rows runs levels 0 and h = 32 inside the thread
// (rows i, i+64 and i+32, i+96), then h = 16, 8, 4, 2, 1 on lane bits 4, 3,
// 2, 1, 0: a v_permlane16_swap, row_ror:8, row_half_mirror (lane ^ 7, which
// is row ^ 4 because of the xor in i), quad_perm ^2 and ^1.  A row sum over
// the 128 columns runs levels 0, 32, 16, 8 inside the thread (columns
// w + 4h + 8m), level 4 on lane bit 5 (v_permlane32_swap) and levels 2, 1
// across waves w ^ 2, w ^ 1 through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "leapq_internal.h"

namespace leapq {
namespace dev {

constexpr int D = 128;
constexpr int NT = 256;

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
// value select (kept as a function so selects between array elements stay
// selects of values, not of addresses)
__device__ __forceinline__ float sel(bool c, float a, float b) { return c ? a : b; }

// ---------------------------------------------------------------- thread map
struct MMap {
    int w, l, h, jp, i;
    __device__ __forceinline__ int row(int p) const { return i + 32 * p; }
    __device__ __forceinline__ int col(int m) const { return w + 4 * h + 8 * m; }
};

__host__ __device__ __forceinline__ int iperm(int x) { return x ^ ((x & 4) ? 3 : 0); }

__device__ __forceinline__ MMap mmap()
{
    MMap a;
    a.l = threadIdx.x & 63;
    a.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    a.h = a.l >> 5;
    a.jp = a.l & 31;
    a.i = iperm(a.jp);
    return a;
}

// Thread map of the dense baselines (leapq_dense.hip): rows i + 32p and
// contiguous columns 16 j + m, with i = (l & 3) | (l >> 3) << 2 and
// j = w + 4 ((l >> 2) & 1); column sums run on lane bits 5, 4, 3, 1, 0.
struct AMap {
    int w, l, i, hb, j;
    __device__ __forceinline__ int row(int p) const { return i + 32 * p; }
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
// Codes of a head (16384 bytes): the 16 codes of thread (w, l), row p, are
// the bytes code_off(w, l, p) + m, m = 0..15 (column w + 4h + 8m), so each
// 16-byte load of a wave reads 1 KB contiguous.
__host__ __device__ __forceinline__ int code_off(int w, int l, int p) { return w * 4096 + p * 1024 + l * 16; }

// Codes of the 6- and 4-bit options (state_bits).  CB = 4: 8192 bytes per
// head of nibbles; thread (w, l)'s rows p = 2j and 2j + 1 (j = 0, 1) sit in
// the 16 bytes at 2048 w + 1024 j + 16 l, two words per row, word t holding
// codes 8t .. 8t + 3 (columns w + 4h + 8m, m = code index) in the low
// nibbles of its bytes and codes 8t + 4 .. 8t + 7 in the high nibbles.
// CB = 6: the same low nibbles (bits 0-3 of each code), then 4096 bytes of
// bits 4-5: the word of row p at 8192 + 1024 w + 16 l + 4 p holds those of
// code 4k + b at bits 8b + 2k.  Every load and store of a wave covers 1 KB.
template <int CB>
struct CodeFmt;
template <>
struct CodeFmt<8> {
    static constexpr int loads = 4, bytes = D * D;
    static constexpr float levels = 127.0f;
};
template <>
struct CodeFmt<6> {
    static constexpr int loads = 3, bytes = D * D * 3 / 4;
    static constexpr float levels = 31.0f;
};
template <>
struct CodeFmt<4> {
    static constexpr int loads = 2, bytes = D * D / 2;
    static constexpr float levels = 7.0f;
};
// byte offset of the thread's j-th 16-byte piece of codes
template <int CB>
__host__ __device__ __forceinline__ int code_piece_off(int w, int l, int j)
{
    if constexpr (CB == 8)
        return code_off(w, l, j);
    else
        return j < 2 ? w * 2048 + j * 1024 + l * 16 : 8192 + w * 1024 + l * 16;
}
// 4 packed nibbles / 6-bit values (one per byte) sign-extended to int8 bytes
__device__ __forceinline__ uint32_t sext4x4(uint32_t x) { return x | ((x & 0x08080808u) * 0x1Eu); }
__device__ __forceinline__ uint32_t sext6x4(uint32_t x) { return x | ((x & 0x20202020u) * 0x06u); }
__device__ __forceinline__ uint32_t u4comp(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// The thread's stored pieces (raw[j], j < CodeFmt<CB>::loads) as int8 code
// bytes: cw[p][k] holds the codes 4k .. 4k + 3 of row block p.
template <int CB>
__device__ __forceinline__ void unpack_codes(const uint4 (&raw)[4], uint32_t (&cw)[4][4])
{
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if constexpr (CB == 8) {
#pragma unroll
            for (int k = 0; k < 4; ++k) cw[p][k] = u4comp(raw[p], k);
        } else {
            const uint32_t P0 = u4comp(raw[p >> 1], 2 * (p & 1)), P1 = u4comp(raw[p >> 1], 2 * (p & 1) + 1);
            const uint32_t lo[4] = {P0 & 0x0F0F0F0Fu, (P0 >> 4) & 0x0F0F0F0Fu, P1 & 0x0F0F0F0Fu,
                                    (P1 >> 4) & 0x0F0F0F0Fu};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (CB == 4) {
                    cw[p][k] = sext4x4(lo[k]);
                } else {
                    const uint32_t H = u4comp(raw[2], p);
                    cw[p][k] = sext6x4(lo[k] | (((H >> (2 * k)) & 0x03030303u) << 4));
                }
            }
        }
    }
}

// Stores the thread's codes, given as int8 bytes B[p][k] (codes 4k .. 4k +
// 3 of row block p), in the layout of CodeFmt<CB>.
template <int CB>
__device__ __forceinline__ void store_codes(int8_t *codes, int w, int l, const uint32_t (&B)[4][4])
{
    if constexpr (CB == 8) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint4 *>(codes + code_off(w, l, p)) = make_uint4(B[p][0], B[p][1], B[p][2], B[p][3]);
    } else {
        uint32_t P[4][2];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            P[p][0] = (B[p][0] & 0x0F0F0F0Fu) | ((B[p][1] & 0x0F0F0F0Fu) << 4);
            P[p][1] = (B[p][2] & 0x0F0F0F0Fu) | ((B[p][3] & 0x0F0F0F0Fu) << 4);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<uint4 *>(codes + code_piece_off<CB>(w, l, j)) =
                make_uint4(P[2 * j][0], P[2 * j][1], P[2 * j + 1][0], P[2 * j + 1][1]);
        if constexpr (CB == 6) {
            uint32_t H[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                H[p] = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) H[p] |= ((B[p][k] >> 4) & 0x03030303u) << (2 * k);
            }
            *reinterpret_cast<uint4 *>(codes + code_piece_off<CB>(w, l, 2)) = make_uint4(H[0], H[1], H[2], H[3]);
        }
    }
}
// Record corrections: column c at upos(c), the A operand order (lane a of
// wave w reads 32 w + (a & 31)).
__host__ __device__ __forceinline__ int upos(int c)
{
    return 32 * (c & 3) + 8 * (c >> 5) + 4 * ((c >> 2) & 1) + ((c >> 3) & 3);
}

struct HeadState {
    int8_t *codes;
    float *rho, *sigma;
    int32_t *cidx;
    float *cvec;
    float *rgam;
    char *rk;  // keys in the input dtype, row order
    char *ru;  // corrections (fp32, bf16, or fp8 codes then 4 scales), stored order
};

__device__ __forceinline__ HeadState head_state(const StateView &sv, int h)
{
    HeadState s;
    s.codes = sv.codes + (size_t)h * sv.code_bytes;
    s.rho = sv.rho + (size_t)h * D;
    s.sigma = sv.sigma + (size_t)h * D;
    s.cidx = sv.cidx + (size_t)h * sv.C;
    s.cvec = sv.cvec + (size_t)h * sv.C * D * (sv.r1 ? 2 : 1);
    s.rgam = sv.rgam + (size_t)h * sv.W * (sv.kda ? D : 1);
    s.rk = static_cast<char *>(sv.rk) + (size_t)h * sv.W * D * (sv.key_bf16 ? 2 : 4);
    s.ru = static_cast<char *>(sv.ru) + (size_t)h * sv.W * sv.u_rec_bytes;
    return s;
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// OCP 8-bit floating point E4M3 (sign, 4 exponent bits with bias 7, 3
// mantissa bits; exponent field 0 holds the subnormals m * 2^-9; largest
// finite value 448; no infinity).  The code of x, |x| <= 448, rounded to
// nearest, ties to even, in integer steps: a normal value keeps its top 3
// mantissa bits plus a carry (which may carry into the exponent field); a
// value below 2^-6 becomes rint(|x| * 2^9), exact before the rounding.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x)
{
    const uint32_t b = __float_as_uint(x);
    const uint32_t sign = (b >> 24) & 0x80u;
    const int e = (int)((b >> 23) & 0xffu) - 127;
    uint32_t mag;
    if (e >= -6) {
        const uint32_t f = b & 0x7fffffu, rem = f & 0xfffffu, m = f >> 20;
        mag = ((uint32_t)(e + 7) << 3) + m + ((rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ? 1u : 0u);
    } else {
        mag = (uint32_t)__builtin_rintf(__uint_as_float(b & 0x7fffffffu) * 512.0f);
    }
    return sign | mag;
}
// The value of code c (bits 0..7; every finite E4M3 value is an fp32 value):
// the hardware conversion v_cvt_f32_fp8 (one VALU instruction), which reads
// its byte as OCP E4M3 on this GPU and agrees with the definition (exponent
// field 0: m * 2^-9; else 1.m * 2^(E - 7)) on all 254 finite codes, checked
// bit for bit.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }
// The smallest power of two s >= 2^-126 with M <= 448 s (M >= 0 finite):
// M = 1.f * 2^(E - 127) needs s = 2^(E - 135), or 2^(E - 134) when 1.f > 1.75.
__device__ __forceinline__ float fp8_scale(float M)
{
    const uint32_t b = __float_as_uint(M);
    const int E = (int)(b >> 23);
    int e = E - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
    e = (E == 0 || e < -126) ? -126 : e;
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

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

// The canonical dots (a . x) and (a . y) in one butterfly: level 32
// exchanges halves, so lanes 0..31 end with a . x and lanes 32..63 with
// a . y, each bitwise equal to wdot.
__device__ __forceinline__ float wdot2(float a0, float a1, float x0, float x1, float y0, float y1)
{
    float s = xhalf32(fma_(a0, x0, a1 * x1), fma_(a0, y0, a1 * y1));
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
__device__ __forceinline__ int xmax32i(int x)
{
    auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int xmax16i(int x)
{
    auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return max((int)r[0], (int)r[1]);
}
// Largest int of the wave, in every lane.  On bit patterns of floats it is
// the float maximum when no value is NaN or -0 and every negative one is the
// same (non-negative floats order like their bits).
__device__ __forceinline__ int wave_max_i(int x)
{
    x = xmax32i(x);
    x = xmax16i(x);
    x = max(x, dppi<DPP_ROR8>(x));
    x = max(x, dppi<DPP_ROR4>(x));
    x = max(x, dppi<DPP_XOR2>(x));
    return max(x, dppi<DPP_XOR1>(x));
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

// AMap column sum over the 128 rows, from the 16 level-1 partials v[m]
// (column j+8m) of each thread.  Returns the sum of the lane's column
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

// MMap column sum over the 128 rows, from the 16 level-32 partials v[m]
// (column w + 4h + 8m, rows i, i+32, i+64, i+96 already combined) of each
// thread: exchange-and-add on lane bits 4 (permlane16 swap), 3 (row_ror:8),
// 2 (row_half_mirror: lane ^ 7, row ^ 4) and 1 (quad ^2), then a butterfly
// on bit 0.  Returns the sum of column w + 4h + 8 mcol(l), mcol(l) =
// (l >> 1) & 15; lanes l and l ^ 1 hold the same column.
__device__ __forceinline__ int mcol_of(int l) { return (l >> 1) & 15; }
__device__ __forceinline__ float mcolsum16(const float (&v)[16], int l)
{
    float a8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a8[e] = xhalf16(v[e], v[e + 8]);
    float a4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a4[e] = xhalf_dpp<DPP_ROR8>(a8[e], a8[e + 4], (l >> 3) & 1);
    float a2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) a2[e] = xhalf_dpp<DPP_HMIR>(a4[e], a4[e + 2], (l >> 2) & 1);
    const float a1 = xhalf_dpp<DPP_XOR2>(a2[0], a2[1], (l >> 1) & 1);
    return a1 + dpp<DPP_XOR1>(a1);
}

// Exchange-and-max on lane bit 5: the lower lane keeps max(K, partner K),
// the upper lane max(G, partner G).
__device__ __forceinline__ float xhalf32max(float K, float G)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(K), __float_as_uint(G), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Barrier between LDS phases of one workgroup: this wave's LDS writes are
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for the
// wave's outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited
    __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------- streaming access
// Loads and stores of data that no later access of the same launch reuses
// (the codes an append reads, the output and the record it writes), with the
// non-temporal cache hint.
__device__ __forceinline__ uint4 ld_stream(const int8_t *p)
{
    // four dword loads that combine into one 16-byte load (a vector-typed
    // load here costs the append some 20 VGPRs)
    const unsigned int *q = reinterpret_cast<const unsigned int *>(p);
    uint4 r;
    r.x = __builtin_nontemporal_load(q);
    r.y = __builtin_nontemporal_load(q + 1);
    r.z = __builtin_nontemporal_load(q + 2);
    r.w = __builtin_nontemporal_load(q + 3);
    return r;
}
__device__ __forceinline__ void st_stream(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_stream(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- LDS-direct copies
// Non-temporal (cache policy nt): a launch reads every copied operand once.
constexpr int kCopyPolicyNT = 2;
__device__ __forceinline__ void lds_copy16(const void *g, float *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, kCopyPolicyNT);
}
__device__ __forceinline__ void lds_copy4(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 4, 0, kCopyPolicyNT);
}
// A read-only fp32 value at a wave-uniform index, as a scalar load (constant
// address space): waited for by lgkmcnt, so it does not wait behind the
// wave's vector loads.
__device__ __forceinline__ float sload(const float *p, int i)
{
    typedef const __attribute__((address_space(4))) float *cptr;
    return ((cptr)(uintptr_t)p)[i];
}
__device__ __forceinline__ int sloadi(const int *p, int i)
{
    typedef const __attribute__((address_space(4))) int *cptr;
    return ((cptr)(uintptr_t)p)[i];
}

__device__ __forceinline__ float rdl(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(x), lane));
}

}  // namespace dev
}  // namespace leapq
