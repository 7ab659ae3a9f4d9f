// LeapQuant per-window int8 recurrent state for Gated DeltaNet heads:
// gfx950 kernels (init-quantize, append, fold, dequant, dense baselines).
//
// Method: "LeapQuant: Efficient Linear Attention with Accurate Recurrent
// State Quantization" (3.2 per-window quantization, 3.3 compensator tokens,
// 3.4 residual smoothing, B.2 window unrolling, B.3 readout with a smoothed
// quantized residual) and "Recurrent-state quantization for linear attention:
// a first GPU kernel" (Background: order of one token; What we built: append
// and fold).
//
// Arithmetic: IEEE binary32, no contraction (-ffp-contract=off; every fused
// multiply-add is an explicit __builtin_fmaf), correctly rounded '/' and
// sqrtf, subnormals kept.  Every sum that feeds a stored value follows one
// canonical order, the 128-term halving tree T128: level 0 combines element
// e with element e+64 (for a dot product: fma(a_e, b_e, a_{e+64}*b_{e+64})),
// then levels h = 32, 16, ..., 1 add partial e and partial e+h.  Any
// butterfly or exchange that adds exactly the tree's pairs gives the same
// bits, because fp32 addition is commutative.
//
// One workgroup of 256 threads (4 wave64s) owns one head.  Thread t = 64w+l
// (wave w, lane l) takes ib = l>>3, j = l&7, i = 4*ib + w and owns the 64
// entries at key rows i, i+32, i+64, i+96 (p = 0..3) and value columns
// j + 8m (m = 0..15).  With this map
//   - a column sum over rows is: level 0 and 1 in the thread; levels h=16, 8, 4
//     between lanes l^32, l^16, l^8 (ib^4, ib^2, ib^1); levels h=2, 1 between
//     waves w^2, w^1 through LDS;
//   - a row sum over columns is: levels 0..3 in the thread; levels h=4, 2, 1
//     between lanes l^4, l^2, l^1.
// Codes are stored column-interleaved (byte 16j+m of a row is column j+8m),
// so each thread's 16 columns of a row are one 16-byte load.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "leapq_internal.h"

namespace leapq {
namespace {

constexpr int D = 128;
constexpr int NT = 256;

struct Map {
    int w, l, ib, j, i;
};

__device__ __forceinline__ Map tmap()
{
    Map m;
    int t = threadIdx.x;
    m.w = t >> 6;
    m.l = t & 63;
    m.ib = m.l >> 3;
    m.j = m.l & 7;
    m.i = 4 * m.ib + m.w;
    return m;
}

__device__ __forceinline__ int row_of(const Map &mp, int p) { return mp.i + 32 * p; }
__device__ __forceinline__ int col_of(const Map &mp, int m) { return mp.j + 8 * m; }

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

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

// Exchange-and-add between lane pairs (l, l^mask): the lower lane returns
// keep_lo(own) + keep_lo(partner), the upper lane keep_hi(own) +
// keep_hi(partner).  Used to halve the set of partial sums a lane carries
// while adding exactly the tree's pairs.
__device__ __forceinline__ float xadd(float lo, float hi, int mask, bool upper)
{
    float send = upper ? lo : hi;
    float recv = __shfl_xor(send, mask);
    return (upper ? hi : lo) + recv;
}

// Column sums over key rows (levels h = 16 .. 1 of the tree) of 16 level-1
// partials v[m] (column j+8m) per thread; nv independent vectors are laid
// out as v[16*k + m].  Writes out[k*128 + c] (LDS) for every column c.
// part: LDS scratch of 4 * nv * 128 floats.  Ends with a barrier.
template <int NV>
__device__ __forceinline__ void col_reduce(const Map &mp, const float (&v)[16 * NV], float *part,
                                           float *out)
{
    constexpr int N0 = 16 * NV;
    const bool u32 = (mp.l & 32) != 0, u16 = (mp.l & 16) != 0, u8 = (mp.l & 8) != 0;
    float a[N0 / 2];
#pragma unroll
    for (int e = 0; e < N0 / 2; ++e) a[e] = xadd(v[e], v[e + N0 / 2], 32, u32);
    float b[N0 / 4];
#pragma unroll
    for (int e = 0; e < N0 / 4; ++e) b[e] = xadd(a[e], a[e + N0 / 4], 16, u16);
    float c[N0 / 8];
#pragma unroll
    for (int e = 0; e < N0 / 8; ++e) c[e] = xadd(b[e], b[e + N0 / 8], 8, u8);
    // lane (ib, j) now holds flat index f = (N0/8)*ib + e  (e < N0/8) of the
    // original 16*NV list, i.e. vector f/16, column j + 8*(f%16)
#pragma unroll
    for (int e = 0; e < N0 / 8; ++e) {
        int f = (N0 / 8) * mp.ib + e;
        part[(mp.w * NV + f / 16) * D + mp.j + 8 * (f % 16)] = c[e];
    }
    __syncthreads();
    for (int x = threadIdx.x; x < NV * D; x += NT) {
        int k = x / D, cc = x % D;
        float s0 = part[(0 * NV + k) * D + cc], s1 = part[(1 * NV + k) * D + cc];
        float s2 = part[(2 * NV + k) * D + cc], s3 = part[(3 * NV + k) * D + cc];
        out[x] = (s0 + s2) + (s1 + s3);
    }
    __syncthreads();
}

// Row sums over value columns of a thread's 16 values per row (levels 0..3
// of the tree in the thread, 4..6 between lanes l^4, l^2, l^1), as a dot of
// the row with itself (energy).  All 8 lanes of the row group get the sum.
__device__ __forceinline__ float row_energy(const float (&x)[16])
{
    float t[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) t[m] = fma_(x[m], x[m], x[m + 8] * x[m + 8]);
#pragma unroll
    for (int m = 0; m < 4; ++m) t[m] = t[m] + t[m + 4];
    t[0] = t[0] + t[2];
    t[1] = t[1] + t[3];
    float s = t[0] + t[1];
    s = s + __shfl_xor(s, 4);
    s = s + __shfl_xor(s, 2);
    s = s + __shfl_xor(s, 1);
    return s;
}

// Canonical dot product of two 128-vectors held as (a[l], a[l+64]) per lane
// of one wave; every lane gets the result.
__device__ __forceinline__ float wave_dot(float a0, float a1, float b0, float b1)
{
    float s = fma_(a0, b0, a1 * b1);
    s = s + __shfl_xor(s, 32);
    s = s + __shfl_xor(s, 16);
    s = s + __shfl_xor(s, 8);
    s = s + __shfl_xor(s, 4);
    s = s + __shfl_xor(s, 2);
    s = s + __shfl_xor(s, 1);
    return s;
}

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

// Unpacks a 16-byte chunk of codes into 16 floats (column j+8m at m).
__device__ __forceinline__ void unpack16(uint4 q, float (&f)[16])
{
    uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int b = 0; b < 4; ++b) f[4 * d + b] = (float)(int8_t)(w4[d] >> (8 * b));
}

// LDS staging of the boundary's small fields and of up to 16 records.
struct FoldSmem {
    float sig[D];
    float vec[8 * D];
    int32_t idx[8];
    float gam[64];
    float k[16 * D];
    float u[16 * D];
    float part[4 * D];
    float colv[D];
    float score[2 * D];
    unsigned long long red[4];
};

__device__ void stage_boundary(const HeadState &hs, int C, int n, FoldSmem &sm)
{
    const int t = threadIdx.x;
    if (t < D) sm.sig[t] = hs.sigma[t];
    for (int x = t; x < C * D; x += NT) sm.vec[x] = hs.cvec[x];
    if (t < C) sm.idx[t] = hs.cidx[t];
    if (t < n) sm.gam[t] = hs.rgam[t];
}

// Records base..base+cnt-1 (cnt <= 16): keys as k[i*128 + (r%32)*4 + r/32]
// (a thread's 4 rows are one float4), corrections as u[i*128 + j*16 + m]
// for column j+8m (a thread's 16 columns are 4 float4s).
__device__ void stage_records(const HeadState &hs, int base, int cnt, FoldSmem &sm)
{
    const int t = threadIdx.x;
    for (int x = t; x < cnt * D; x += NT) {
        const int i = x / D, e = x % D;
        sm.k[i * D + (e & 31) * 4 + (e >> 5)] = hs.rk[(size_t)base * D + x];
        sm.u[i * D + (e & 7) * 16 + (e >> 3)] = hs.ru[(size_t)base * D + x];
    }
}

// ---------------------------------------------------------------------------
// Shared by init, fold and dequant: the head's current state in registers.
// S[p][m] = entry (row i+32p, column j+8m).
//
// Residual (code * (gamma_n * rho_r)) * sigma_c; compensator lines in
// compensator order as S + gamma_n * line; records i = 0..n-1 in order as
// fma((gamma_n / gamma_i) * k_i[r], u_i[c], S).  With lines = false and
// n = 0 this is the residual alone, (code * rho_r) * sigma_c (gamma_0 = 1).
// Expects stage_boundary() done and visible; contains barriers (call from
// every thread).
// ---------------------------------------------------------------------------
__device__ void rebuild(const Map &mp, const HeadState &hs, int C, int n, bool lines, FoldSmem &sm,
                        float (&S)[4][16])
{
    const float gn = n > 0 ? sm.gam[n - 1] : 1.0f;
    float sig[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) sig[m] = sm.sig[col_of(mp, m)];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = row_of(mp, p);
        const float a = gn * hs.rho[r];
        uint4 q = *reinterpret_cast<const uint4 *>(hs.codes + r * D + 16 * mp.j);
        float f[16];
        unpack16(q, f);
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = (f[m] * a) * sig[m];
    }
    if (lines) {
        for (int jj = 0; jj < C; ++jj) {
            const int id = sm.idx[jj];
            const float *v = sm.vec + jj * D;
            if (id < 0) continue;
            if (id < D) {
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    if (row_of(mp, p) == id) {
#pragma unroll
                        for (int m = 0; m < 16; ++m) S[p][m] = S[p][m] + gn * v[col_of(mp, m)];
                    }
            } else {
                const int c = id - D;
                if ((c & 7) == mp.j) {
                    const int mm = c >> 3;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        if (m == mm) {
#pragma unroll
                            for (int p = 0; p < 4; ++p) S[p][m] = S[p][m] + gn * v[row_of(mp, p)];
                        }
                }
            }
        }
    }
    for (int base = 0; base < n; base += 16) {
        const int cnt = n - base < 16 ? n - base : 16;
        __syncthreads();  // the previous chunk is consumed
        stage_records(hs, base, cnt, sm);
        __syncthreads();
        for (int i = 0; i < cnt; ++i) {
            const float ci = gn / sm.gam[base + i];
            const float4 kk = *reinterpret_cast<const float4 *>(sm.k + i * D + 4 * mp.i);
            const float w[4] = {ci * kk.x, ci * kk.y, ci * kk.z, ci * kk.w};
            float u[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float4 uu = *reinterpret_cast<const float4 *>(sm.u + i * D + mp.j * 16 + 4 * d);
                u[4 * d] = uu.x;
                u[4 * d + 1] = uu.y;
                u[4 * d + 2] = uu.z;
                u[4 * d + 3] = uu.w;
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int m = 0; m < 16; ++m) S[p][m] = fma_(w[p], u[m], S[p][m]);
        }
    }
}

// Block-wide argmax over 256 candidates (one per thread) of the key
// (score bits, 255 - candidate): largest score, then lowest candidate.
__device__ __forceinline__ int block_pick(FoldSmem &sm)
{
    const int t = threadIdx.x;
    __syncthreads();  // every score of this round is written
    const float score = sm.score[t];
    unsigned long long key =
        ((unsigned long long)__float_as_uint(score) << 32) | (unsigned long long)(255 - t);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        unsigned long long o = __shfl_xor(key, mask);
        key = o > key ? o : key;
    }
    if ((t & 63) == 0) sm.red[t >> 6] = key;
    __syncthreads();
    unsigned long long best = sm.red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) best = sm.red[w] > best ? sm.red[w] : best;
    __syncthreads();
    if ((best >> 32) == 0ull) return -1;  // best score <= 0: nothing left to extract
    return 255 - (int)(best & 0xffull);
}

__device__ __forceinline__ void column_energies(const Map &mp, const float (&S)[4][16], FoldSmem &sm)
{
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        v[m] = fma_(S[0][m], S[0][m], S[2][m] * S[2][m]) + fma_(S[1][m], S[1][m], S[3][m] * S[3][m]);
    col_reduce<1>(mp, v, sm.part, sm.colv);
    if (threadIdx.x < D) sm.score[D + threadIdx.x] = sm.colv[threadIdx.x];
}

__device__ __forceinline__ void row_energies(const Map &mp, const float (&S)[4][16], FoldSmem &sm)
{
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float e = row_energy(S[p]);
        if (mp.j == 0) sm.score[row_of(mp, p)] = e;
    }
}

// Steps after the rebuild (shared by init and fold): compensator extraction,
// smoothing, per-row int8.  Writes the head's boundary state.
__device__ void quantize_state(const Map &mp, float (&S)[4][16], const HeadState &hs, int C,
                               int smoothing, float floor_, FoldSmem &sm)
{
    const int t = threadIdx.x;
    // --- compensator tokens: greedy whole-line extraction ("LeapQuant" 3.3)
    if (C > 0) {
        row_energies(mp, S, sm);
        column_energies(mp, S, sm);  // ends with a barrier; row scores visible too
        for (int jj = 0; jj < C; ++jj) {
            const int pick = block_pick(sm);
            float *vec = hs.cvec + jj * D;
            if (t == 0) hs.cidx[jj] = pick;
            if (pick < 0) {
                if (t < D) vec[t] = 0.0f;
                continue;
            }
            if (pick < D) {
                if ((pick & 31) == mp.i) {
                    const int pp = pick >> 5;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        if (p == pp) {
#pragma unroll
                            for (int m = 0; m < 16; ++m) {
                                vec[col_of(mp, m)] = S[p][m];
                                S[p][m] = 0.0f;
                            }
                        }
                }
            } else {
                const int c = pick - D;
                if ((c & 7) == mp.j) {
                    const int mm = c >> 3;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        if (m == mm) {
#pragma unroll
                            for (int p = 0; p < 4; ++p) {
                                vec[row_of(mp, p)] = S[p][m];
                                S[p][m] = 0.0f;
                            }
                        }
                }
            }
            if (jj + 1 < C) {
                if (t == pick) sm.score[pick] = 0.0f;
                __syncthreads();
                if (pick < D)
                    column_energies(mp, S, sm);
                else {
                    row_energies(mp, S, sm);
                    __syncthreads();
                }
            }
        }
    }
    // --- residual smoothing ("LeapQuant" 3.4): sigma_c = max(sqrt(mean_r |R|), floor)
    if (smoothing) {
        float v[16];
#pragma unroll
        for (int m = 0; m < 16; ++m)
            v[m] = (fabsf(S[0][m]) + fabsf(S[2][m])) + (fabsf(S[1][m]) + fabsf(S[3][m]));
        col_reduce<1>(mp, v, sm.part, sm.colv);
        if (t < D) {
            float s = sqrtf(sm.colv[t] * 0.0078125f);
            if (s < floor_) s = floor_;
            hs.sigma[t] = s;
            sm.sig[t] = 1.0f / s;
        }
    } else if (t < D) {
        hs.sigma[t] = 1.0f;
        sm.sig[t] = 1.0f;
    }
    __syncthreads();
    // --- per-row symmetric int8, round half to even
    float inv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) inv[m] = sm.sig[col_of(mp, m)];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float x[16];
        float M = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            x[m] = S[p][m] * inv[m];
            M = fmaxf(M, fabsf(x[m]));
        }
        M = fmaxf(M, __shfl_xor(M, 4));
        M = fmaxf(M, __shfl_xor(M, 2));
        M = fmaxf(M, __shfl_xor(M, 1));
        const int r = row_of(mp, p);
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        float rho = 0.0f;
        if (M >= 0x1p-120f) {
            rho = M / 127.0f;
            const float g = 127.0f / M;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                float y = rintf(x[m] * g);
                y = fminf(fmaxf(y, -127.0f), 127.0f);
                w4[m >> 2] |= ((uint32_t)(int32_t)y & 0xffu) << (8 * (m & 3));
            }
        }
        *reinterpret_cast<uint4 *>(hs.codes + r * D + 16 * mp.j) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        if (mp.j == 0) hs.rho[r] = rho;
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(NT) void k_init(StateView sv, const float *__restrict__ S0, int smoothing,
                                              float floor_)
{
    __shared__ FoldSmem sm;
    const Map mp = tmap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const float *src = S0 + (size_t)h * D * D;
    float S[4][16];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = src[row_of(mp, p) * D + col_of(mp, m)];
    quantize_state(mp, S, hs, sv.C, smoothing, floor_, sm);
}

__global__ __launch_bounds__(NT) void k_fold(StateView sv, int n, int smoothing, float floor_)
{
    __shared__ FoldSmem sm;
    const Map mp = tmap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    stage_boundary(hs, sv.C, n, sm);
    __syncthreads();
    float S[4][16];
    rebuild(mp, hs, sv.C, n, true, sm, S);
    __syncthreads();  // every thread has read the old rho, sigma, lines
    quantize_state(mp, S, hs, sv.C, smoothing, floor_, sm);
}

__global__ __launch_bounds__(NT) void k_dequant(StateView sv, int n, int what, float *__restrict__ out)
{
    __shared__ FoldSmem sm;
    const Map mp = tmap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const int nr = what == 2 ? n : 0;
    stage_boundary(hs, sv.C, nr, sm);
    __syncthreads();
    float S[4][16];
    rebuild(mp, hs, sv.C, nr, what >= 1, sm, S);
    float *dst = out + (size_t)h * D * D;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) dst[row_of(mp, p) * D + col_of(mp, m)] = S[p][m];
}

// Append: one token for one head ("Recurrent-state quantization for linear
// attention: a first GPU kernel", Background order; "LeapQuant" B.2-B.3).
//   gamma_t = gamma_n * alpha; c_i = gamma_t / gamma_i
//   Bx[c] = sigma_c * T128_r((x_r * rho_r) * code[r][c])  then, per
//           compensator in order: row token r: fma(x_r, line[c], Bx[c]);
//           column token c': Bx[c'] + T128(line . x)
//   r = gamma_t Bk, chained fma((c_i * (k_i . k)), u_i, r) over records
//   u = beta (v - r); o likewise from Bq, then fma((k . q), u, o)
struct AppendSmem {
    float part[4 * 2 * D];
    float red[2 * D];
    float kq[2 * D];  // k then q, fp32
    float dots[2 * 64 + 2 * 8 + 1];
};

template <typename T, int MAXW>
__global__ __launch_bounds__(NT) void k_append(StateView sv, int n, const T *__restrict__ qin,
                                                const T *__restrict__ kin, const T *__restrict__ vin,
                                                const float *__restrict__ alpha,
                                                const float *__restrict__ beta, float *__restrict__ o)
{
    __shared__ AppendSmem sm;
    const Map mp = tmap();
    const int t = threadIdx.x;
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const int C = sv.C;
    const T *qh = qin + (size_t)h * D;
    const T *kh = kin + (size_t)h * D;

    // ---- per-column operands for the tail, issued early (threads t < 128)
    float u_c[MAXW];
    float vcol = 0.0f, sigc = 0.0f;
    if (t < D) {
        vcol = ld_in<T>(vin + (size_t)h * D, t);
        sigc = hs.sigma[t];
#pragma unroll
        for (int i = 0; i < MAXW; ++i) u_c[i] = i < n ? hs.ru[i * D + t] : 0.0f;
        sm.kq[t] = ld_in<T>(kh, t);
        sm.kq[D + t] = ld_in<T>(qh, t);
    }

    // ---- residual read: both Sum_r (x_r rho_r) code[r][c] for x = k, q
    float v[32];
    {
        float wk[4], wq[4], f[4][16];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = row_of(mp, p);
            uint4 q = *reinterpret_cast<const uint4 *>(hs.codes + r * D + 16 * mp.j);
            unpack16(q, f[p]);
            const float rr = hs.rho[r];
            wk[p] = ld_in<T>(kh, r) * rr;
            wq[p] = ld_in<T>(qh, r) * rr;
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            v[m] = fma_(wk[0], f[0][m], wk[2] * f[2][m]) + fma_(wk[1], f[1][m], wk[3] * f[3][m]);
            v[16 + m] = fma_(wq[0], f[0][m], wq[2] * f[2][m]) + fma_(wq[1], f[1][m], wq[3] * f[3][m]);
        }
    }

    // ---- dot products of this token (one wave each, round robin):
    // job 2i, 2i+1: (k_i . k), (k_i . q); job 2n: (k . q);
    // job 2n+1+2jj, +1: (line_jj . k), (line_jj . q) for column tokens
    {
        const int l = mp.l;
        const float k0 = ld_in<T>(kh, l), k1 = ld_in<T>(kh, l + 64);
        const float q0 = ld_in<T>(qh, l), q1 = ld_in<T>(qh, l + 64);
        const int njobs = n + 1 + C;
        for (int job = mp.w; job < njobs; job += 4) {
            if (job < n) {
                const float a0 = hs.rk[job * D + l], a1 = hs.rk[job * D + l + 64];
                const float dk = wave_dot(a0, a1, k0, k1);
                const float dq = wave_dot(a0, a1, q0, q1);
                if (l == 0) {
                    sm.dots[2 * job] = dk;
                    sm.dots[2 * job + 1] = dq;
                }
            } else if (job == n) {
                const float d = wave_dot(k0, k1, q0, q1);
                if (l == 0) sm.dots[2 * n] = d;
            } else {
                const int jj = job - n - 1;
                const int id = hs.cidx[jj];
                if (id >= D) {
                    const float a0 = hs.cvec[jj * D + l], a1 = hs.cvec[jj * D + l + 64];
                    const float dk = wave_dot(a0, a1, k0, k1);
                    const float dq = wave_dot(a0, a1, q0, q1);
                    if (l == 0) {
                        sm.dots[2 * n + 1 + 2 * jj] = dk;
                        sm.dots[2 * n + 2 + 2 * jj] = dq;
                    }
                }
            }
        }
    }

    col_reduce<2>(mp, v, sm.part, sm.red);  // red[c] = k read, red[128 + c] = q read

    if (t < D) {
        const int c = t;
        const float gt = (n > 0 ? hs.rgam[n - 1] : 1.0f) * alpha[h];
        float bk = sigc * sm.red[c];
        float bq = sigc * sm.red[D + c];
        for (int jj = 0; jj < C; ++jj) {
            const int id = hs.cidx[jj];
            if (id < 0) continue;
            if (id < D) {
                const float lv = hs.cvec[jj * D + c];
                bk = fma_(sm.kq[id], lv, bk);
                bq = fma_(sm.kq[D + id], lv, bq);
            } else if (id - D == c) {
                bk = bk + sm.dots[2 * n + 1 + 2 * jj];
                bq = bq + sm.dots[2 * n + 2 + 2 * jj];
            }
        }
        float r = gt * bk;
        float oc = gt * bq;
#pragma unroll
        for (int i = 0; i < MAXW; ++i) {
            if (i < n) {
                const float ci = gt / hs.rgam[i];
                const float ak = ci * sm.dots[2 * i];
                const float aq = ci * sm.dots[2 * i + 1];
                r = fma_(ak, u_c[i], r);
                oc = fma_(aq, u_c[i], oc);
            }
        }
        const float u = beta[h] * (vcol - r);
        oc = fma_(sm.dots[2 * n], u, oc);
        o[(size_t)h * D + c] = oc;
        hs.ru[n * D + c] = u;
        hs.rk[n * D + c] = sm.kq[c];
        if (c == 0) hs.rgam[n] = gt;
    }
}

// Dense per-token GDN decode (the unquantized baselines), in place.  Thread
// map as above but with contiguous columns 16j + e, e < 16.
//   S = alpha S; r = T128-dot over rows of (S, k); u = beta (v - r);
//   S = fma(k_r, u_c, S); o = T128-dot over rows of (S, q).
template <typename TS, typename TI>
__global__ __launch_bounds__(NT) void k_gdn_decode(TS *__restrict__ Sg, const TI *__restrict__ qin,
                                                    const TI *__restrict__ kin, const TI *__restrict__ vin,
                                                    const float *__restrict__ alpha,
                                                    const float *__restrict__ beta, float *__restrict__ o)
{
    __shared__ float part[4 * D];
    __shared__ float red[D];
    __shared__ float uc[D];
    const Map mp = tmap();
    const int h = blockIdx.x;
    TS *Sh = Sg + (size_t)h * D * D;
    const TI *qh = qin + (size_t)h * D, *kh = kin + (size_t)h * D;
    const float a = alpha[h];
    float S[4][16];
    float kr[4], qr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = row_of(mp, p);
        kr[p] = ld_in<TI>(kh, r);
        qr[p] = ld_in<TI>(qh, r);
        if constexpr (sizeof(TS) == 4) {
            const float4 *src = reinterpret_cast<const float4 *>(Sh + r * D + 16 * mp.j);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float4 x = src[d];
                S[p][4 * d] = x.x;
                S[p][4 * d + 1] = x.y;
                S[p][4 * d + 2] = x.z;
                S[p][4 * d + 3] = x.w;
            }
        } else {
            const uint4 *src = reinterpret_cast<const uint4 *>(Sh + r * D + 16 * mp.j);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                uint4 x = src[d];
                uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    S[p][8 * d + 2 * b] = bf16_to_f32((uint16_t)(w4[b] & 0xffffu));
                    S[p][8 * d + 2 * b + 1] = bf16_to_f32((uint16_t)(w4[b] >> 16));
                }
            }
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = a * S[p][m];
    }
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        v[m] = fma_(S[0][m], kr[0], S[2][m] * kr[2]) + fma_(S[1][m], kr[1], S[3][m] * kr[3]);
    // col_reduce writes column j+8m for slot m; here slot m is column 16j+m,
    // so map through a permuted read afterwards.
    col_reduce<1>(mp, v, part, red);
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        // slot (j', m') written as column j'+8m' holds column 16j'+m'
        const float rc = red[(c >> 4) + 8 * (c & 15)];
        uc[c] = beta[h] * (ld_in<TI>(vin + (size_t)h * D, c) - rc);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = fma_(kr[p], uc[16 * mp.j + m], S[p][m]);
#pragma unroll
    for (int m = 0; m < 16; ++m)
        v[m] = fma_(S[0][m], qr[0], S[2][m] * qr[2]) + fma_(S[1][m], qr[1], S[3][m] * qr[3]);
    col_reduce<1>(mp, v, part, red);
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        o[(size_t)h * D + c] = red[(c >> 4) + 8 * (c & 15)];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = row_of(mp, p);
        if constexpr (sizeof(TS) == 4) {
            float4 *dst = reinterpret_cast<float4 *>(Sh + r * D + 16 * mp.j);
#pragma unroll
            for (int d = 0; d < 4; ++d)
                dst[d] = make_float4(S[p][4 * d], S[p][4 * d + 1], S[p][4 * d + 2], S[p][4 * d + 3]);
        } else {
            uint4 *dst = reinterpret_cast<uint4 *>(Sh + r * D + 16 * mp.j);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                uint32_t w4[4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    w4[b] = (uint32_t)f32_to_bf16_rne(S[p][8 * d + 2 * b]) |
                            ((uint32_t)f32_to_bf16_rne(S[p][8 * d + 2 * b + 1]) << 16);
                dst[d] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------

hipError_t launch_init(const StateView &sv, int heads, const float *S0, int smoothing, float floor_,
                       hipStream_t s)
{
    hipLaunchKernelGGL(k_init, dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
    return hipGetLastError();
}

hipError_t launch_fold(const StateView &sv, int heads, int n, int smoothing, float floor_, hipStream_t s)
{
    hipLaunchKernelGGL(k_fold, dim3(heads), dim3(NT), 0, s, sv, n, smoothing, floor_);
    return hipGetLastError();
}

hipError_t launch_dequant(const StateView &sv, int heads, int n, int what, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_dequant, dim3(heads), dim3(NT), 0, s, sv, n, what, out);
    return hipGetLastError();
}

hipError_t launch_append(const StateView &sv, int heads, int n, int bf16, const void *q, const void *k,
                         const void *v, const float *alpha, const float *beta, float *o, hipStream_t s)
{
    if (bf16) {
        using T = uint16_t;
        if (sv.W <= 16)
            hipLaunchKernelGGL((k_append<T, 16>), dim3(heads), dim3(NT), 0, s, sv, n, (const T *)q,
                               (const T *)k, (const T *)v, alpha, beta, o);
        else
            hipLaunchKernelGGL((k_append<T, 64>), dim3(heads), dim3(NT), 0, s, sv, n, (const T *)q,
                               (const T *)k, (const T *)v, alpha, beta, o);
    } else {
        using T = float;
        if (sv.W <= 16)
            hipLaunchKernelGGL((k_append<T, 16>), dim3(heads), dim3(NT), 0, s, sv, n, (const T *)q,
                               (const T *)k, (const T *)v, alpha, beta, o);
        else
            hipLaunchKernelGGL((k_append<T, 64>), dim3(heads), dim3(NT), 0, s, sv, n, (const T *)q,
                               (const T *)k, (const T *)v, alpha, beta, o);
    }
    return hipGetLastError();
}

hipError_t launch_gdn_decode(int heads, int state_bf16, int in_bf16, void *S, const void *q, const void *k,
                             const void *v, const float *alpha, const float *beta, float *o, hipStream_t s)
{
    if (state_bf16) {
        if (in_bf16)
            hipLaunchKernelGGL((k_gdn_decode<uint16_t, uint16_t>), dim3(heads), dim3(NT), 0, s,
                               (uint16_t *)S, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v,
                               alpha, beta, o);
        else
            hipLaunchKernelGGL((k_gdn_decode<uint16_t, float>), dim3(heads), dim3(NT), 0, s, (uint16_t *)S,
                               (const float *)q, (const float *)k, (const float *)v, alpha, beta, o);
    } else {
        if (in_bf16)
            hipLaunchKernelGGL((k_gdn_decode<float, uint16_t>), dim3(heads), dim3(NT), 0, s, (float *)S,
                               (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, beta,
                               o);
        else
            hipLaunchKernelGGL((k_gdn_decode<float, float>), dim3(heads), dim3(NT), 0, s, (float *)S,
                               (const float *)q, (const float *)k, (const float *)v, alpha, beta, o);
    }
    return hipGetLastError();
}

}  // namespace leapq
