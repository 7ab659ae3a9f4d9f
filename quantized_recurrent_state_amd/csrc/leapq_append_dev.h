// Device code of the append (one decode token per head), shared by the
// append kernel and the fused last-append-and-fold kernel.  See
// leapq_append.hip for the method and its sources.
#pragma once

#include <type_traits>

#include "leapq_device.h"

namespace leapq {
namespace {
using namespace dev;

template <typename T>
struct InLds;
template <>
struct InLds<float> {
    static constexpr int floats = 3 * 128;
    __device__ static float get(const float *base, int vecno, int e) { return base[vecno * 128 + e]; }
};
template <>
struct InLds<uint16_t> {
    static constexpr int floats = 3 * 64;
    __device__ static float get(const float *base, int vecno, int e)
    {
        return bf16_to_f32(reinterpret_cast<const uint16_t *>(base)[vecno * 128 + e]);
    }
};

// Record corrections kept as fp8 (an option): a record's 128 corrections in
// stored order are 128 E4M3 codes, then 4 fp32 scales, scale j serving
// stored positions 32 j .. 32 j + 31 (value columns c with c % 4 = j, the
// columns of wave j); the value is decode(code) * scale, exact.
struct Fp8 {};
template <>
struct InLds<Fp8> {
    __device__ static float get(const float *base, int vecno, int e)
    {
        (void)vecno;
        return e4m3_to_f32(reinterpret_cast<const uint8_t *>(base)[e]) * base[32 + (e >> 5)];
    }
};
template <typename U>
struct UBytes {
    static constexpr int value = D * (int)sizeof(U);
};
template <>
struct UBytes<Fp8> {
    static constexpr int value = D + 16;
};

// A record as stored and as staged in LDS: the key in dtype T (row order;
// the input dtype stores the token's k exactly unless the append normalizes
// it, which needs fp32), then the correction (fp32, stored order); keys take
// kbytes, a staged record stride floats.
// With per-channel decay (CH) a record also holds its cumulative decay as a
// 128-vector; the staged record is then [decay | correction | key].  U: the
// correction's storage (fp32, or bf16 or fp8 as lossy options).
template <typename T, bool CH = false, typename U = float>
struct Rec {
    static constexpr int kbytes = D * (int)sizeof(T);
    static constexpr int kf = kbytes / 4;
    static constexpr int ubytes = UBytes<U>::value;
    static constexpr int uf = ubytes / 4;
    static constexpr int goff = 0;                   // CH: the decay vector
    static constexpr int uoff = CH ? D : kf;         // the correction
    static constexpr int koff = CH ? D + uf : 0;     // the key
    static constexpr int stride = kf + uf + (CH ? D : 0);
    static constexpr int kpieces = kbytes / 16;
    static constexpr int upieces = ubytes / 16;
    __device__ static float key(const float *rec, int r) { return InLds<T>::get(rec + koff, 0, r); }
    __device__ static float u(const float *rec, int c) { return InLds<U>::get(rec + uoff, 0, c); }
};

// Copies record g of a head into LDS at dst (stride floats) with LDS-direct
// loads of 16 bytes per lane: without CH, the key's pieces then the
// correction's in one load; with CH, the decay's and the correction's in one
// load, then the key's.
template <typename T, bool CH = false, typename U = float>
__device__ __forceinline__ void copy_record(const HeadState &hs, int g, int l, float *dst)
{
    using R = Rec<T, CH, U>;
    constexpr int kp = R::kpieces, up = R::upieces;
    if constexpr (!CH) {
        if (kp + up >= 64 || l < kp + up)
            lds_copy16(l < kp ? static_cast<const void *>(hs.rk + g * R::kbytes + 16 * l)
                              : static_cast<const void *>(hs.ru + g * R::ubytes + 16 * (l - kp)),
                       dst);
    } else {
        if (32 + up >= 64 || l < 32 + up)
            lds_copy16(l < 32 ? static_cast<const void *>(hs.rgam + g * D + 4 * l)
                              : static_cast<const void *>(hs.ru + g * R::ubytes + 16 * (l - 32)),
                       dst);
        if (kp >= 64 || l < kp) lds_copy16(hs.rk + g * R::kbytes + 16 * l, dst + R::koff);
    }
}

// LDS of one head in floats: records [n][stride] (keys K), compensators
// ([C][128] lines, or with R1 [C][2][128] rank-one pairs), rho [128], sigma
// [128], inputs (k, q, v as T), indices [8], then the record decays [64] or,
// with CH, the token's decay vector [128]
template <typename T, typename K, bool CH = false, typename U = float, bool R1 = false>
__host__ __device__ constexpr int head_lds_floats(int n, int C)
{
    return n * Rec<K, CH, U>::stride + C * (R1 ? 256 : 128) + 256 + InLds<T>::floats + 8 + (CH ? 128 : 64);
}
// per-workgroup results of the dot jobs: coefficients [2][64], column-token
// dots [2][8], k.q [1], then the gated alpha and beta [2] (+1 pad)
constexpr int kDotFloats = 128 + 16 + 4;
constexpr int kGateSlot = 145;

template <typename T, typename K, bool CH = false, typename U = float, bool R1 = false>
struct HeadLds {
    float *rec, *cv, *srho, *ssig, *sin_, *sgam;
    int *sidx;
    __device__ HeadLds(float *rec_, float *cv_, float *rho_sigma, float *in_, int *idx_, float *gam_)
        : rec(rec_), cv(cv_), srho(rho_sigma), ssig(rho_sigma + D), sin_(in_), sgam(gam_), sidx(idx_)
    {
    }
    __device__ HeadLds(float *base, int n, int C)
    {
        rec = base;
        cv = rec + n * Rec<K, CH, U>::stride;
        srho = cv + C * D * (R1 ? 2 : 1);
        ssig = srho + D;
        sin_ = ssig + D;
        sidx = reinterpret_cast<int *>(sin_ + InLds<T>::floats);
        sgam = reinterpret_cast<float *>(sidx + 8);
    }
};

// Wait until at most NL vector loads of this wave are outstanding:
// with the codes issued last, every LDS-direct copy of append_issue() has
// landed (vector loads complete in issue order) while the codes may still be
// in flight.  Other waves' copies need a barrier after this.
// NL = CodeFmt<CB>::loads (4 for the int8 state, 3 or 2 for 6 or 4 bits).
template <int NL = 4>
__device__ __forceinline__ void wait_lds_copies()
{
    // vmcnt(NL) (bits 3:0 and 15:14), expcnt(7), lgkmcnt(15): not waited
    __builtin_amdgcn_s_waitcnt((NL & 15) | ((NL >> 4) << 14) | 0x70 | 0xF00);
}

// Issues every global load of head h: every operand other than the codes
// into the LDS buffer L by LDS-direct copies, then the thread's 64 codes into
// qc as the wave's last CodeFmt<CB>::loads vector loads.
template <typename T, typename K, bool CH = false, typename U = float, bool R1 = false, int CB = 8>
__device__ __forceinline__ void append_issue(const StateView &sv, int n, int h, const T *__restrict__ qin,
                                             const T *__restrict__ kin, const T *__restrict__ vin,
                                             const MMap &a, const HeadLds<T, K, CH, U, R1> &L, uint4 (&qc)[4],
                                             const float *__restrict__ alpha = nullptr)
{
    const int C = sv.C, l = a.l, w = a.w;
    const HeadState hs = head_state(sv, h);
    for (int rr = w; rr < n; rr += 4) copy_record<K, CH, U>(hs, rr, l, L.rec + rr * Rec<K, CH, U>::stride);
    const int nvec = R1 ? 2 * C : C;  // 128-vectors of the compensators
    for (int pair = 2 * w; pair < nvec; pair += 8)
        if (pair + (l >> 5) < nvec) lds_copy16(hs.cvec + (pair + (l >> 5)) * D + 4 * (l & 31), L.cv + pair * D);
    if (w == 0) {
        lds_copy16(l < 32 ? hs.rho + 4 * l : hs.sigma + 4 * (l - 32), L.srho);
    } else if (w == 1) {
        // inputs as 16-byte pieces of k, q, v in that order
        constexpr int per = (int)(128 * sizeof(T) / 16);
        if (l < 3 * per) {
            const int vecno = l / per, piece = l % per;
            const T *src = (vecno == 0 ? kin : vecno == 1 ? qin : vin) + (size_t)h * D;
            lds_copy16(reinterpret_cast<const char *>(src) + 16 * piece, L.sin_);
        }
        if (3 * per > 64 && l < 3 * per - 64) {
            const int f = 64 + l, vecno = f / per, piece = f % per;
            const T *src = (vecno == 0 ? kin : vecno == 1 ? qin : vin) + (size_t)h * D;
            lds_copy16(reinterpret_cast<const char *>(src) + 16 * piece, L.sin_ + 256);
        }
    } else if (w == 2) {
        if (l < C) lds_copy4(hs.cidx + l, L.sidx);
    } else if constexpr (CH) {
        // the token's decay vector (the records carry their own)
        if (l < 32) lds_copy16(alpha + (size_t)h * D + 4 * l, L.sgam);
    } else {
        if (l < n) lds_copy4(hs.rgam + l, L.sgam);
    }
    // the code loads stay behind every copy (wait_lds_copies counts on it)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < CodeFmt<CB>::loads; ++j) qc[j] = ld_stream(hs.codes + code_piece_off<CB>(w, l, j));
    __builtin_amdgcn_sched_barrier(0);
}

// Gate arithmetic of one head and token, in binary64 from the fp32
// arguments and rounded once to fp32: alpha = exp(-exp(A_log) softplus(a +
// dt_bias)) with softplus(x) = max(x, 0) + log1p(exp(-|x|)), beta =
// 1 / (1 + exp(-b)).  The pages time this step ("Recurrent-state
// quantization for linear attention: a first GPU kernel", Results: the
// column with gate arithmetic) without printing it; these are the gates of
// the Gated DeltaNet layer.
__device__ __forceinline__ void gate_eval(float a, float b, float A_log, float dt_bias, float &alpha, float &beta)
{
    const double x = (double)a + (double)dt_bias;
    const double sp = fmax(x, 0.0) + log1p(exp(-fabs(x)));
    alpha = (float)exp(-exp((double)A_log) * sp);
    beta = (float)(1.0 / (1.0 + exp(-(double)b)));
}

// The gates of head h by wave 0 alone, while the loads are in flight, into
// dots[kGateSlot..+1]; every wave reads them back after the next barrier
// (gate_read).  a_h, b_h: the raw projections.
__device__ __forceinline__ void gate_issue(const GateArgs &g, int h, const MMap &a, float a_h, float b_h, float *dots)
{
    if (a.w == 0) {
        const int j = h % g.heads;
        float al, be;
        gate_eval(a_h, b_h, sload(g.A_log, j), sload(g.dt_bias, j), al, be);
        if (a.l == 0) {
            dots[kGateSlot] = al;
            dots[kGateSlot + 1] = be;
        }
    }
}

// The token for head h from its staged operands (L, qc); writes o and the
// record.  NORM: q and k are L2-normalized first, k_r * (1 / sqrt(k . k +
// eps)) and (q_r * (1 / sqrt(q . q + eps))) * q_scale, with the canonical
// dot (the record key is then the normalized k in fp32).  Expects the LDS copies landed and visible (wait_lds_copies() and a
// barrier); the codes are waited for at their first use.  Contains one
// lds_barrier (dot jobs -> residual read and tail).
template <typename T, typename K, bool REC_LDS = false, bool NORM = false, bool CH = false, typename U = float,
          bool R1 = false, int CB = 8>
__device__ __forceinline__ void append_compute(const StateView &sv, int n, int h, const MMap &a,
                                               const HeadLds<T, K, CH, U, R1> &L, float *dots, const uint4 (&qc)[4],
                                               float a_h, float b_h, float *__restrict__ o, float q_scale = 1.0f,
                                               float eps = 0.0f, float *wout = nullptr)
{
    using R = Rec<K, CH, U>;
    const int C = sv.C, l = a.l, w = a.w;
    const HeadState hs = head_state(sv, h);
    const float *rec = L.rec, *cv = L.cv, *srho = L.srho, *ssig = L.ssig, *sin_ = L.sin_, *sgam = L.sgam;
    const int *sidx = L.sidx;
    float *coef = dots, *cdot = dots + 128, *kqd = dots + 144;
    // ---- operands from LDS; after the residual read lane l holds vector
    // vec = bit 4 of l (0: k, 1: q) of column w + 4h + 8 (l & 15)
    const int vec = (l >> 4) & 1;
    const int c = a.col(l & 15);
    float kn = 1.0f, qn = 1.0f;  // normalization factors (NORM)
    float k0 = InLds<T>::get(sin_, 0, l), k1 = InLds<T>::get(sin_, 0, l + 64);
    float q0 = InLds<T>::get(sin_, 1, l), q1 = InLds<T>::get(sin_, 1, l + 64);
    if constexpr (NORM) {
        kn = 1.0f / sqrtf(wdot(k0, k1, k0, k1) + eps);
        qn = 1.0f / sqrtf(wdot(q0, q1, q0, q1) + eps);
    }
    auto nk = [&](float x) { return NORM ? x * kn : x; };
    auto nq = [&](float x) { return NORM ? (x * qn) * q_scale : x; };
    k0 = nk(k0);
    k1 = nk(k1);
    q0 = nq(q0);
    q1 = nq(q1);
    // decay: the scalar gamma_t = gamma_{n-1} * alpha, or (CH) per row
    // gamma_t[r] = gamma_{n-1}[r] * alpha[r] from the staged previous record
    // and the token's staged alpha (sgam); with CH the boundary is read with
    // gamma_t (.) k and gamma_t (.) q
    const float *gprev = rec + (n > 0 ? n - 1 : 0) * R::stride + R::goff;
    auto gt_row = [&](int r) { return (n > 0 ? gprev[r] : 1.0f) * sgam[r]; };
    float rh[4], kr[4], qr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        rh[p] = srho[a.row(p)];
        kr[p] = nk(InLds<T>::get(sin_, 0, a.row(p)));
        qr[p] = nq(InLds<T>::get(sin_, 1, a.row(p)));
        if constexpr (CH) {
            const float g = gt_row(a.row(p));
            kr[p] = g * kr[p];
            qr[p] = g * qr[p];
        }
    }
    const float sig_c = ssig[c];
    const float v_c = InLds<T>::get(sin_, 2, c);
    float gt = 1.0f, ci_l = 0.0f, gt0 = 1.0f, gt1 = 1.0f;
    if constexpr (CH) {
        gt0 = gt_row(l);
        gt1 = gt_row(l + 64);
    } else {
        gt = (n > 0 ? sgam[n - 1] : 1.0f) * a_h;
        ci_l = l < n ? gt / sgam[l] : 0.0f;  // c_i of record i = lane, for the dot jobs
    }

    // ---- per-head dot products (operands in LDS; the codes may still be in
    // flight), one wave per job:
    // job r < n: c_r * (k_r . k), c_r * (k_r . q), or with CH
    //            (w_r . k), (w_r . q) with w_r = (gamma_t / gamma_r) (.) k_r;
    // job n: (k . q);
    // job n+1+jj: (line_jj . x), (line_jj . y) for column tokens, x = k and
    //            y = q, or with CH x = gamma_t (.) k and y = gamma_t (.) q;
    //            with R1 (a_jj . k), (a_jj . q) for every rank-one pair
    const int njobs = n + 1 + C;
    for (int job = w; job < njobs; job += 4) {
        if (job < n) {
            const float *kj = rec + job * R::stride;
            float a0 = R::key(kj, l), a1 = R::key(kj, l + 64);
            if constexpr (CH) {
                a0 = (gt0 / kj[R::goff + l]) * a0;
                a1 = (gt1 / kj[R::goff + l + 64]) * a1;
            }
            // lanes 0..31: the key dot, lanes 32..63: the query dot; lanes 0
            // and 32 store them at coef[job] and coef[64 + job]
            const float d = wdot2(a0, a1, k0, k1, q0, q1);
            const float ci = CH ? 1.0f : rdl(ci_l, job);
            if ((l & 31) == 0) coef[job + 2 * l] = CH ? d : ci * d;
            if constexpr (REC_LDS) {
                // the record's weighted key c_i k_i (with CH the weighted
                // key itself) for the fold's rebuild of this head
                wout[job * D + l] = CH ? a0 : ci * a0;
                wout[job * D + l + 64] = CH ? a1 : ci * a1;
            }
        } else if (job == n) {
            const float d = wdot(k0, k1, q0, q1);
            if (l == 0) kqd[0] = d;
        } else {
            const int jj = job - n - 1;
            if (R1 || sidx[jj] >= D) {
                const float *vj = cv + jj * D * (R1 ? 2 : 1);  // a line, or the pair's a
                const float a0 = vj[l], a1 = vj[l + 64];
                const float d = wdot2(a0, a1, CH ? gt0 * k0 : k0, CH ? gt1 * k1 : k1, CH ? gt0 * q0 : q0,
                                      CH ? gt1 * q1 : q1);
                if ((l & 31) == 0) cdot[jj + (l >> 2)] = d;  // lane 32: cdot[8 + jj]
            }
        }
    }
    lds_barrier();  // the coefficients of every wave's jobs

    // ---- residual read of column m for k and q: rows (i, i+64) and
    // (i+32, i+96) by fused level 0, then level 32; the next exchange (tree
    // level 16 on lane bit 4: k stays in lanes with bit 4 clear, q in the
    // others) follows at once so only 16 partials stay live.  Then levels 8,
    // 4, 2, 1 on lane bits 3, 2 (lane ^ 7 is row ^ 4), 1, 0, each keeping half
    // of the columns.
    float red;
    {
        float wk[4], wq[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            wk[p] = kr[p] * rh[p];
            wq[p] = qr[p] * rh[p];
        }
        uint32_t cw[4][4];
        unpack_codes<CB>(qc, cw);
        float a16[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            float f[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) f[p] = code_f(cw[p][m >> 2], m & 3);
            const float sk = fma_(wk[0], f[0], wk[2] * f[2]) + fma_(wk[1], f[1], wk[3] * f[3]);
            const float sq = fma_(wq[0], f[0], wq[2] * f[2]) + fma_(wq[1], f[1], wq[3] * f[3]);
            a16[m] = xhalf16(sk, sq);
        }
        float a8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = xhalf_dpp<DPP_ROR8>(a16[e], a16[e + 8], (l >> 3) & 1);
        float a4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = xhalf_dpp<DPP_HMIR>(a8[e], a8[e + 4], (l >> 2) & 1);
        float a2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) a2[e] = xhalf_dpp<DPP_XOR2>(a4[e], a4[e + 2], (l >> 1) & 1);
        red = xhalf_dpp<DPP_XOR1>(a2[0], a2[1], l & 1);
    }

    // ---- per-column tail: lane (vec, c)
    float b = sig_c * red;
    for (int jj = 0; jj < C; ++jj) {
        if constexpr (R1) {  // (a_jj . x) b_jj[c]
            b = fma_(cdot[vec * 8 + jj], cv[(2 * jj + 1) * D + c], b);
            continue;
        }
        const int id = sidx[jj];
        if (id < 0) continue;
        if (id < D) {
            const float x = InLds<T>::get(sin_, vec, id);
            float xr = vec ? nq(x) : nk(x);
            if constexpr (CH) xr = gt_row(id) * xr;
            b = fma_(xr, cv[jj * D + c], b);
        } else if (id - D == c) {
            b = b + cdot[vec * 8 + jj];
        }
    }
    float acc = CH ? b : gt * b;
    const int uc = upos(c);
    for (int r = 0; r < n; ++r) acc = fma_(coef[vec * 64 + r], R::u(rec + r * R::stride, uc), acc);
    // k lanes form u; q lanes receive it from lane l-16 and finish o
    const float u = b_h * (v_c - acc);
    // fp8 records: the scale of this wave's 32 corrections from their
    // largest magnitude (q lanes contribute 0)
    float s8 = 1.0f;
    if constexpr (std::is_same<U, Fp8>::value) s8 = fp8_scale(wave_max(vec == 0 ? fabsf(u) : 0.0f));
    auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(u), false, false);
    const float u_from_k = __uint_as_float(sw[0]);
    // the record goes to HBM, or (REC_LDS) into slot n of the staged records
    char *ru = REC_LDS ? reinterpret_cast<char *>(L.rec + n * R::stride + R::uoff) : hs.ru + n * R::ubytes;
    uint32_t *rk = REC_LDS ? reinterpret_cast<uint32_t *>(L.rec + n * R::stride + R::koff)
                           : reinterpret_cast<uint32_t *>(hs.rk + n * R::kbytes);
    if (vec == 0) {
        // the record's correction (rounded to nearest even with bf16 or fp8
        // U); this token's own output below uses the fp32 u
        if constexpr (std::is_same<U, float>::value) {
            if constexpr (REC_LDS)
                reinterpret_cast<float *>(ru)[uc] = u;
            else
                st_stream(reinterpret_cast<float *>(ru) + uc, u);
        } else if constexpr (std::is_same<U, Fp8>::value) {
            // u / s is exact (s is a power of two, 1 / s = 2^-e)
            const float inv = __uint_as_float((254u - (__float_as_uint(s8) >> 23)) << 23);
            reinterpret_cast<uint8_t *>(ru)[uc] = (uint8_t)f32_to_e4m3(u * inv);
            if (l == 0) reinterpret_cast<float *>(ru + D)[w] = s8;
        } else {
            reinterpret_cast<uint16_t *>(ru)[uc] = f32_to_bf16_rne(u);
        }
    } else {
        st_stream(o + (size_t)h * D + c, fma_(kqd[0], u_from_k, acc));
    }
    if (w == 0) {
        if constexpr (REC_LDS) {
            // this token's own record enters the rebuild with coefficient
            // gamma_t / gamma_t = 1
            wout[n * D + l] = k0;
            wout[n * D + l + 64] = k1;
        }
        if constexpr (std::is_same<K, T>::value && !NORM) {
            // the key is the token's k as staged (the first kbytes of the inputs)
            const uint32_t *kw = reinterpret_cast<const uint32_t *>(sin_);
            if constexpr (REC_LDS) {
                rk[l] = kw[l];
                if (R::kf > 64) rk[l + 64] = kw[l + 64];
            } else {
                st_stream(rk + l, kw[l]);
                if (R::kf > 64) st_stream(rk + l + 64, kw[l + 64]);
            }
        } else {
            static_assert(std::is_same<K, float>::value, "normalized or widened keys are fp32");
            rk[l] = __float_as_uint(k0);
            rk[l + 64] = __float_as_uint(k1);
        }
        if constexpr (CH) {
            float *rg = REC_LDS ? L.rec + n * R::stride + R::goff : hs.rgam + n * D;
            rg[l] = gt0;
            rg[l + 64] = gt1;
        } else {
            float *rg = REC_LDS ? L.sgam : hs.rgam;
            if (l == 0) rg[n] = gt;
        }
    }
}

}  // namespace
}  // namespace leapq
