// Fold, initial quantization and dequantization of the boundary state.
//
// Method: "Recurrent-state quantization for linear attention: a first GPU
// kernel" (What we built: the fold rebuilds the state, selects compensators,
// rescales, rounds and empties the buffer; Why rounding the state is
// difficult: rounded once per window, largest outliers set aside, the rest
// smoothed) and "LeapQuant: Efficient Linear Attention with Accurate
// Recurrent State Quantization" (3.3 compensator tokens; 3.4 residual
// smoothing by the square root of the mean absolute value with a positive
// floor; B.3 the state is rebuilt in original coordinates before the new
// factors and scales).  Steps, per head:
//   rebuild   S = (code * (gamma_n * rho_r)) * sigma_c; compensator lines
//             added as S + gamma_n * line; records i in order as
//             fma((gamma_n / gamma_i) * k_i[r], u_i[c], S)
//   extract   C greedy rounds: line energies (canonical dot of the line with
//             itself), pick the largest (rows 0..127 then columns 0..127,
//             lowest index on ties, none if no positive energy), store the
//             line, zero it; rescore the other axis
//   smooth    sigma_c = max(sqrt(T(|R[:,c]|) * 2^-7), floor), or 1
//   quantize  x = R * (1 / sigma_c); M_r = max |x|; rho_r = M_r / 127;
//             code = rint(x * (127 / M_r)) (rows with M_r < 2^-120: zeros)
// The clamp to +-127 of the plain statement is a no-op here: |x| <= M_r
// gives |x * RN(127 / M_r)| <= 127 (1 + 2^-23) < 127.5.
#include "leapq_device.h"

namespace leapq {
namespace {
using namespace dev;

struct FoldLds {
    float rec[16 * 256];  // a chunk of up to 16 records: keys | corrections (stored layouts)
    float lines[8 * 128];
    float rho[128];
    float sig[128];
    int idx[8];
    float gam[64];
    float part[4 * 128];  // cross-wave row partials / row maxima
    float score[256];     // row energies, then column energies
    float rowg[128];      // 127 / M_r per row (0 for zero rows)
    float sinv[128];      // 1 / sigma_c
    float redf[4];
    int redi[4];
};

// Copies boundary fields (lines, rho, sigma, indices) and n decays to LDS.
__device__ __forceinline__ void stage_small(const AMap &a, const HeadState &hs, int C, int n, FoldLds &sm)
{
    const int l = a.l, w = a.w;
    for (int pair = 2 * w; pair < C; pair += 8)
        if (pair + (l >> 5) < C) lds_copy16(hs.cvec + (pair + (l >> 5)) * D + 4 * (l & 31), sm.lines + pair * D);
    if (w == 0) {
        lds_copy16(l < 32 ? hs.rho + 4 * l : hs.sigma + 4 * (l - 32), sm.rho);
    } else if (w == 1) {
        if (l < C) lds_copy4(hs.cidx + l, sm.idx);
    } else if (w == 2) {
        if (l < n) lds_copy4(hs.rgam + l, sm.gam);
    }
}

__device__ __forceinline__ void stage_records(const AMap &a, const HeadState &hs, int base, int cnt, FoldLds &sm)
{
    const int l = a.l;
    for (int rr = a.w; rr < cnt; rr += 4) {
        const int g = base + rr;
        lds_copy16(l < 32 ? hs.rk + g * D + 4 * l : hs.ru + g * D + 4 * (l - 32), sm.rec + rr * 256);
    }
}

// Current state in registers: S[p][m] = entry (row i+32p, column j+8m).
// qc: the thread's 4 code chunks.  Expects stage_small() done and visible
// and, if n > 0, records 0..min(n,16)-1 staged and visible.  Contains
// barriers when n > 16.
__device__ __forceinline__ void rebuild(const AMap &a, const HeadState &hs, const uint4 (&qc)[4], int C, int n,
                                        bool lines, FoldLds &sm, float (&S)[4][16])
{
    const float gn = n > 0 ? sm.gam[n - 1] : 1.0f;
    float sg[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) sg[m] = sm.sig[a.col(m)];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float ap = gn * sm.rho[a.row(p)];
        const uint32_t cw[4] = {qc[p].x, qc[p].y, qc[p].z, qc[p].w};
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = (code_f(cw[m >> 2], m & 3) * ap) * sg[m];
    }
    if (lines) {
        for (int jj = 0; jj < C; ++jj) {
            const int id = sm.idx[jj];
            const float *v = sm.lines + jj * D;
            if (id < 0) continue;
            if (id < D) {
                const int pp = id >> 5;
                if (a.i == (id & 31)) {
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        if (p == pp) {
#pragma unroll
                            for (int m = 0; m < 16; ++m) S[p][m] = S[p][m] + gn * v[a.col(m)];
                        }
                }
            } else {
                const int c = id - D, mm = c >> 3;
                if (a.j == (c & 7)) {
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        if (m == mm) {
#pragma unroll
                            for (int p = 0; p < 4; ++p) S[p][m] = S[p][m] + gn * v[a.row(p)];
                        }
                }
            }
        }
    }
    const float ci_l = a.l < n ? gn / sm.gam[a.l] : 0.0f;  // c_i for record i = lane
    for (int base = 0; base < n; base += 16) {
        const int cnt = n - base < 16 ? n - base : 16;
        if (base > 0) {
            __syncthreads();  // the previous chunk is consumed
            stage_records(a, hs, base, cnt, sm);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        for (int r = 0; r < cnt; ++r) {
            const float ci = rdl(ci_l, base + r);
            const float4 kk = *reinterpret_cast<const float4 *>(sm.rec + r * 256 + 4 * a.i);
            const float wv[4] = {ci * kk.x, ci * kk.y, ci * kk.z, ci * kk.w};
            float u[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float4 uu = *reinterpret_cast<const float4 *>(sm.rec + r * 256 + 128 + 16 * a.j + 4 * d);
                u[4 * d] = uu.x;
                u[4 * d + 1] = uu.y;
                u[4 * d + 2] = uu.z;
                u[4 * d + 3] = uu.w;
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int m = 0; m < 16; ++m) S[p][m] = fma_(wv[p], u[m], S[p][m]);
        }
    }
}

// ---------------------------------------------------------------- energies
__device__ __forceinline__ void col_partials(const float (&S)[4][16], float (&cp)[16])
{
#pragma unroll
    for (int m = 0; m < 16; ++m)
        cp[m] = fma_(S[0][m], S[0][m], S[2][m] * S[2][m]) + fma_(S[1][m], S[1][m], S[3][m] * S[3][m]);
}

// Publishes the 128 column energies from the cached column partials.
__device__ __forceinline__ void publish_cols(const AMap &a, const float (&cp)[16], FoldLds &sm)
{
    const float e = colsum16(cp, a.l);
    if ((a.l & 1) == 0) sm.score[D + a.j + 8 * colm_of(a.l)] = e;
}

// Publishes the 128 row energies from the cached row partials (levels 0..3);
// level 4 across lane bit 2, levels 5 and 6 across waves.  Ends with a
// barrier after which score[0..127] is written (by threads < 128).
__device__ __forceinline__ void publish_rows(const AMap &a, const float (&rp)[4], FoldLds &sm)
{
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float s = rp[p] + xor4(rp[p]);
        if (a.hb == 0) sm.part[a.w * D + a.row(p)] = s;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < D) sm.score[t] = (sm.part[t] + sm.part[2 * D + t]) + (sm.part[D + t] + sm.part[3 * D + t]);
}

// Block argmax of score[0..255]: largest score, lowest candidate on ties;
// -1 when no score is positive.  Starts and ends with barriers.
__device__ __forceinline__ int pick_line(const AMap &a, FoldLds &sm)
{
    __syncthreads();
    const int t = threadIdx.x;
    const float s = sm.score[t];
    const float mw = wave_max(s);
    if (a.l == 0) sm.redf[a.w] = mw;
    __syncthreads();
    const float M = fmaxf(fmaxf(sm.redf[0], sm.redf[1]), fmaxf(sm.redf[2], sm.redf[3]));
    if (!(M > 0.0f)) return -1;  // uniform
    const int cw = wave_min(s == M ? t : 1 << 20);
    if (a.l == 0) sm.redi[a.w] = cw;
    __syncthreads();
    return min(min(sm.redi[0], sm.redi[1]), min(sm.redi[2], sm.redi[3]));
}

// Steps after the rebuild, shared by init and fold.  Writes the head's new
// boundary state (codes, rho, sigma, indices, lines).
__device__ void quantize_state(const AMap &a, float (&S)[4][16], const HeadState &hs, int C, int smoothing,
                               float floor_, FoldLds &sm)
{
    const int t = threadIdx.x, l = a.l;
    // ---- compensator tokens
    if (C > 0) {
        float cp[16], rp[4];
        col_partials(S, cp);
#pragma unroll
        for (int p = 0; p < 4; ++p) rp[p] = row_energy16(S[p]);
        publish_cols(a, cp, sm);
        publish_rows(a, rp, sm);
        for (int jj = 0; jj < C; ++jj) {
            const int pick = pick_line(a, sm);
            float *vec = hs.cvec + jj * D;
            if (t == 0) hs.cidx[jj] = pick;
            if (pick < 0) {
                if (t < D) vec[t] = 0.0f;
                continue;
            }
            if (pick < D) {
                const int pp = pick >> 5;
                const bool own = a.i == (pick & 31);
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    if (p == pp && own) {
#pragma unroll
                        for (int m = 0; m < 16; ++m) {
                            vec[a.col(m)] = S[p][m];
                            S[p][m] = 0.0f;
                        }
                        rp[p] = 0.0f;
                    }
                if (jj + 1 < C) {
                    if (own) col_partials(S, cp);
                    if (t == 0) sm.score[pick] = 0.0f;
                    publish_cols(a, cp, sm);
                }
            } else {
                const int cc = pick - D, mm = cc >> 3;
                const bool own = a.j == (cc & 7);
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    if (m == mm && own) {
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            vec[a.row(p)] = S[p][m];
                            S[p][m] = 0.0f;
                        }
                        cp[m] = 0.0f;
                    }
                if (jj + 1 < C) {
                    if (own) {
#pragma unroll
                        for (int p = 0; p < 4; ++p) rp[p] = row_energy16(S[p]);
                    }
                    if (t == 0) sm.score[pick] = 0.0f;
                    publish_rows(a, rp, sm);
                }
            }
        }
    }
    // ---- residual smoothing
    {
        float v[16];
#pragma unroll
        for (int m = 0; m < 16; ++m)
            v[m] = (fabsf(S[0][m]) + fabsf(S[2][m])) + (fabsf(S[1][m]) + fabsf(S[3][m]));
        const float msum = colsum16(v, l);
        if ((l & 1) == 0) {
            const int c = a.j + 8 * colm_of(l);
            float s = 1.0f;
            if (smoothing) {
                s = sqrtf(msum * 0.0078125f);
                if (s < floor_) s = floor_;
            }
            hs.sigma[c] = s;
            sm.sinv[c] = 1.0f / s;
        }
    }
    __syncthreads();
    // ---- per-row symmetric int8, round half to even
    float inv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) inv[m] = sm.sinv[a.col(m)];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float Mx = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            S[p][m] = S[p][m] * inv[m];
            Mx = fmaxf(Mx, fabsf(S[p][m]));
        }
        Mx = fmaxf(Mx, xor4(Mx));
        if (a.hb == 0) sm.part[a.w * D + a.row(p)] = Mx;
    }
    __syncthreads();
    if (t < D) {
        const float M = fmaxf(fmaxf(sm.part[t], sm.part[D + t]), fmaxf(sm.part[2 * D + t], sm.part[3 * D + t]));
        const bool live = M >= 0x1p-120f;
        hs.rho[t] = live ? M / 127.0f : 0.0f;
        sm.rowg[t] = live ? 127.0f / M : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float g = sm.rowg[a.row(p)];
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float y = rintf(S[p][m] * g);
            w4[m >> 2] |= ((uint32_t)(int32_t)y & 0xffu) << (8 * (m & 3));
        }
        *reinterpret_cast<uint4 *>(hs.codes + a.row(p) * D + 16 * a.j) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
}

__global__ __launch_bounds__(NT) void k_init(StateView sv, const float *__restrict__ S0, int smoothing,
                                              float floor_)
{
    __shared__ FoldLds sm;
    const AMap a = amap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const float *src = S0 + (size_t)h * D * D;
    float S[4][16];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = src[a.row(p) * D + a.col(m)];
    quantize_state(a, S, hs, sv.C, smoothing, floor_, sm);
}

__global__ __launch_bounds__(NT) void k_fold(StateView sv, int n, int smoothing, float floor_)
{
    __shared__ FoldLds sm;
    const AMap a = amap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    uint4 qc[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) qc[p] = *reinterpret_cast<const uint4 *>(hs.codes + a.row(p) * D + 16 * a.j);
    stage_small(a, hs, sv.C, n, sm);
    stage_records(a, hs, 0, n < 16 ? n : 16, sm);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float S[4][16];
    rebuild(a, hs, qc, sv.C, n, true, sm, S);
    __syncthreads();  // every thread has read the old boundary from LDS
    quantize_state(a, S, hs, sv.C, smoothing, floor_, sm);
}

__global__ __launch_bounds__(NT) void k_dequant(StateView sv, int n, int what, float *__restrict__ out)
{
    __shared__ FoldLds sm;
    const AMap a = amap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const int nr = what == 2 ? n : 0;
    uint4 qc[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) qc[p] = *reinterpret_cast<const uint4 *>(hs.codes + a.row(p) * D + 16 * a.j);
    stage_small(a, hs, sv.C, nr, sm);
    stage_records(a, hs, 0, nr < 16 ? nr : 16, sm);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float S[4][16];
    rebuild(a, hs, qc, sv.C, nr, what >= 1, sm, S);
    float *dst = out + (size_t)h * D * D;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) dst[a.row(p) * D + a.col(m)] = S[p][m];
}

}  // namespace

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

}  // namespace leapq
