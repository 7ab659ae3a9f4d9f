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
//
// The records are applied on the matrix cores: with the thread map of
// leapq_device.h a record is two v_mfma_f32_32x32x1_2b_f32 per wave (A = the
// correction over the wave's 32 columns, B = c_i k_i over 64 rows each), and
// a K = 1 matrix step rounds exactly like fma(c_i k_i[r], u_i[c], S), so the
// chain over the records is the same sequence of fused multiply-adds.
#include "leapq_append_dev.h"
#include "leapq_device.h"

namespace leapq {
namespace {
using namespace dev;

typedef float f32x32 __attribute__((ext_vector_type(32)));

// The thread's 64 entries S[p][m] = (row i + 32p, column w + 4h + 8m); in
// the matrix instructions' accumulators they are register 16 (p & 1) + m of
// accumulator p >> 1 (instruction q = p >> 1, block b = p & 1).
#define TS(T, p, m) ((T)[p][m])

// Operands of one head staged from HBM, and the work arrays of the steps
// after the rebuild.
template <int RS>
struct FoldStage {
    float rec[16 * RS];  // a chunk of up to 16 records (RS = Rec<K, CH, U>::stride floats each)
    float lines[8 * 128];
    float rho[128];
    float sig[128];
    int idx[8];
    float gam[64];   // record decays (scalar decay)
    float gW[128];   // the last record's decay vector (per-channel decay)
};
struct alignas(16) FoldWork {
    float colE[2][128];      // column energies (two buffers, see extraction)
    float rowP[2][4 * 128];  // per-wave row-energy partials (two buffers)
    float part[4 * 128];     // cross-wave row maxima
    float rowg[4][128];      // per wave: 127 / M_r per row (0 for zero rows)
    float sinv[128];         // 1 / sigma_c
    float spare[128];        // pads the area to the block fit's arrays
};
// The block fit's arrays, laid over FoldWork (the fit ends before the
// smoothing uses it).  z holds a slot's column dots in the thread-contiguous
// order zpos(c): thread (w, h) reads its 16 columns w + 4h + 8m as four
// 16-byte loads.
struct alignas(16) BlockWork {
    float P[4][128][4];  // per slot and row: the four waves' row-dot partials
    float z[4][128];     // per slot: column dots (z, finally b)
};
static_assert(sizeof(BlockWork) <= sizeof(FoldWork), "block fit arrays exceed the fold's work area");
static_assert(sizeof(FoldWork) >= 16 * 128 * sizeof(float), "the weighted keys of 16 records exceed the work area");
__device__ __forceinline__ int zpos(int c) { return (2 * (c & 3) + ((c >> 2) & 1)) * 16 + (c >> 3); }

constexpr int kBlockSweeps = 2;      // per fold, warm-started
constexpr int kBlockSweepsInit = 8;  // at init, from the longest rows

// Copies boundary fields (lines, rho, sigma, indices) and the decays to LDS:
// the n record decays, or with CH the last record's decay vector.
template <bool CH, typename Stage, bool R1 = false>
__device__ __forceinline__ void stage_small(const MMap &a, const HeadState &hs, int C, int n, Stage &sm)
{
    const int l = a.l, w = a.w;
    const int nvec = R1 ? 2 * C : C;  // 128-vectors of the compensators
    for (int pair = 2 * w; pair < nvec; pair += 8)
        if (pair + (l >> 5) < nvec) lds_copy16(hs.cvec + (pair + (l >> 5)) * D + 4 * (l & 31), sm.lines + pair * D);
    if (w == 0) {
        lds_copy16(l < 32 ? hs.rho + 4 * l : hs.sigma + 4 * (l - 32), sm.rho);
    } else if (w == 1) {
        if (l < C) lds_copy4(hs.cidx + l, sm.idx);
    } else if (w == 2) {
        if constexpr (CH) {
            if (n > 0 && l < 32) lds_copy16(hs.rgam + (size_t)(n - 1) * D + 4 * l, sm.gW);
        } else {
            if (l < n) lds_copy4(hs.rgam + l, sm.gam);
        }
    }
}

template <typename K, bool CH, typename U, typename Stage>
__device__ __forceinline__ void stage_records(const MMap &a, const HeadState &hs, int base, int cnt, Stage &sm)
{
    for (int rr = a.w; rr < cnt; rr += 4)
        copy_record<K, CH, U>(hs, base + rr, a.l, sm.rec + rr * Rec<K, CH, U>::stride);
}

template <int CB = 8>
__device__ __forceinline__ void load_codes(const MMap &a, const HeadState &hs, uint4 (&qc)[4])
{
#pragma unroll
    for (int j = 0; j < CodeFmt<CB>::loads; ++j)
        qc[j] = *reinterpret_cast<const uint4 *>(hs.codes + code_piece_off<CB>(a.w, a.l, j));
}

// Current state in the tile.  qc: the thread's 4 code chunks.  Expects
// stage_small() done and visible and, if n > 0, records 0..min(n,16)-1
// staged and visible.  Contains barriers when n > 16.  K: the key dtype.
// CH: per-channel decay, gamma_n[r] read from gW (the last record's decay
// vector), every scale and record coefficient taken per row.
// R1: the compensators are rank-one pairs [a | b] in sm.lines, applied as
// matrix-instruction steps fma(gamma_n a[r], b[c], S) before the records.
// wpre (n <= 16): the records' weighted keys c_i k_i (with CH, the per-row
// weighted keys) as [n][128] fp32 in LDS, formed by the append that shares
// the launch; the matrix steps then read their key operands from it.
template <typename K, bool CH, typename U, typename Stage, bool R1 = false, bool WPRE = false, int CB = 8>
__device__ __forceinline__ void rebuild(const MMap &a, const HeadState &hs, const uint4 (&qc)[4], int C, int n,
                                        bool lines, Stage &sm, float (&S)[4][16], const float *gW = nullptr,
                                        const float *wpre = nullptr)
{
    using R = Rec<K, CH, U>;
    const float gn = CH ? 1.0f : (n > 0 ? sm.gam[n - 1] : 1.0f);
    float gr[4];  // gamma_n of the thread's rows
#pragma unroll
    for (int p = 0; p < 4; ++p) gr[p] = CH ? (n > 0 ? gW[a.row(p)] : 1.0f) : gn;
    float sg[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) sg[m] = sm.sig[a.col(m)];
    uint32_t cw[4][4];
    unpack_codes<CB>(qc, cw);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float ap = gr[p] * sm.rho[a.row(p)];
#pragma unroll
        for (int m = 0; m < 16; ++m) TS(S, p, m) = (code_f(cw[p][m >> 2], m & 3) * ap) * sg[m];
    }
    if (!R1 && lines && C > 0) {
        // the line of each of the thread's row blocks and column entries, as
        // 1 + the line's slot in a nibble (0: none): rows in rpk (nibble p),
        // columns in cpk[0] (entries m < 8) and cpk[1] (m >= 8, nibble m - 8).
        // An entry on a row line and a column line is +0 in the line
        // extracted second (it was zeroed by the first), so adding the row
        // line and then the column line gives the bits of adding both in
        // extraction order.
        uint32_t rpk = 0u, cpk[2] = {0u, 0u};
        for (int jj = 0; jj < C; ++jj) {
            const int id = __builtin_amdgcn_readfirstlane(sm.idx[jj]);
            if (id >= 0 && id < D) {
                const uint32_t bits = (uint32_t)(jj + 1) << (4 * (id >> 5));
                rpk = a.i == (id & 31) ? rpk | bits : rpk;
            } else if (id >= D && a.w == ((id - D) & 3)) {
                const int c = id - D, mm = c >> 3;
                const uint32_t bits = (uint32_t)(jj + 1) << (4 * (mm & 7));
                const bool mine = a.h == ((c >> 2) & 1);
                if (mm < 8)
                    cpk[0] = mine ? cpk[0] | bits : cpk[0];
                else
                    cpk[1] = mine ? cpk[1] | bits : cpk[1];
            }
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t e = (rpk >> (4 * p)) & 15u;
            if (e != 0u) {
                const float *v = sm.lines + (e - 1u) * D;
#pragma unroll
                for (int m = 0; m < 16; ++m) TS(S, p, m) = TS(S, p, m) + gr[p] * v[a.col(m)];
            }
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const uint32_t e = (cpk[m >> 3] >> (4 * (m & 7))) & 15u;
            if (e != 0u) {
                const float *v = sm.lines + (e - 1u) * D;
#pragma unroll
                for (int p = 0; p < 4; ++p) TS(S, p, m) = TS(S, p, m) + gr[p] * v[a.row(p)];
            }
        }
    }
    // through the accumulators even when n == 0: one definition of S after
    // this point keeps it in one set of registers
    const float ci_l = !CH && a.l < n ? gn / sm.gam[a.l] : 0.0f;  // c_i for record i = lane (scalar decay)
    f32x32 acc[2];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[p >> 1][16 * (p & 1) + m] = S[p][m];
    if constexpr (R1) {
        if (lines) {
            // A lane (w, jp) carries column w + 4 ((jp >> 2) & 1) + 8 (jp & 3) + 32 (jp >> 3)
            const int ac = a.w + 4 * ((a.jp >> 2) & 1) + 8 * (a.jp & 3) + 32 * (a.jp >> 3);
            const int kr = a.i + 32 * a.h;
            for (int jj = 0; jj < C; ++jj) {
                const float *av = sm.lines + jj * 2 * D, *bv = av + D;
                const float b0 = gn * av[kr], b1 = gn * av[kr + 64];
                const float au = bv[ac];
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(au, b0, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x1f32(au, b1, acc[1], 0, 0, 0);
            }
        }
    }
    for (int base = 0; base < n; base += 16) {
        const int cnt = n - base < 16 ? n - base : 16;
        if (base > 0) {
            __syncthreads();  // the previous chunk is consumed
            stage_records<K, CH, U>(a, hs, base, cnt, sm);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // records r of the chunk in order; four per iteration, then the rest.
        // B lane l of instruction q carries key row a.i + 32 (a.h + 2q); with
        // CH its coefficient is gamma_n[row] / gamma_i[row].
        const int kr0 = a.i + 32 * a.h;
        const float gw0 = CH && n > 0 ? gW[kr0] : 1.0f, gw1 = CH && n > 0 ? gW[kr0 + 64] : 1.0f;
        int r = 0;
        for (; r + 4 <= cnt; r += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float *rr = sm.rec + (r + u) * R::stride;
                float b0, b1;
                if constexpr (WPRE) {
                    b0 = wpre[(r + u) * D + kr0];
                    b1 = wpre[(r + u) * D + kr0 + 64];
                } else if constexpr (CH) {
                    b0 = (gw0 / rr[R::goff + kr0]) * R::key(rr, kr0);
                    b1 = (gw1 / rr[R::goff + kr0 + 64]) * R::key(rr, kr0 + 64);
                } else {
                    const float ci = rdl(ci_l, base + r + u);
                    b0 = ci * R::key(rr, kr0);
                    b1 = ci * R::key(rr, kr0 + 64);
                }
                const float au = R::u(rr, 32 * a.w + a.jp);
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(au, b0, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x1f32(au, b1, acc[1], 0, 0, 0);
            }
        }
        for (; r < cnt; ++r) {
            const float *rr = sm.rec + r * R::stride;
            float b0, b1;
            if constexpr (WPRE) {
                b0 = wpre[r * D + kr0];
                b1 = wpre[r * D + kr0 + 64];
            } else if constexpr (CH) {
                b0 = (gw0 / rr[R::goff + kr0]) * R::key(rr, kr0);
                b1 = (gw1 / rr[R::goff + kr0 + 64]) * R::key(rr, kr0 + 64);
            } else {
                const float ci = rdl(ci_l, base + r);
                b0 = ci * R::key(rr, kr0);
                b1 = ci * R::key(rr, kr0 + 64);
            }
            const float au = R::u(rr, 32 * a.w + a.jp);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(au, b0, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x1f32(au, b1, acc[1], 0, 0, 0);
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = acc[p >> 1][16 * (p & 1) + m];
}

// ---------------------------------------------------------------- energies
__device__ __forceinline__ void col_partials(const float (&S)[4][16], float (&cp)[16])
{
#pragma unroll
    for (int m = 0; m < 16; ++m)
        cp[m] = fma_(TS(S, 0, m), TS(S, 0, m), TS(S, 2, m) * TS(S, 2, m)) +
                fma_(TS(S, 1, m), TS(S, 1, m), TS(S, 3, m) * TS(S, 3, m));
}

__device__ __forceinline__ float row_partial(const float (&S)[4][16], int p)
{
    float x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) x[m] = TS(S, p, m);
    return row_energy16(x);
}

// Column energies from the cached column partials (tree levels 16..1 across
// lanes); lane pairs (l, l ^ 1) hold one column, the even lane writes it.
__device__ __forceinline__ void put_cols(const MMap &a, const float (&cp)[16], float *colE)
{
    const float e = mcolsum16(cp, a.l);
    if ((a.l & 1) == 0) colE[a.col(mcol_of(a.l))] = e;
}

// Writes a per-row value pair to a per-wave row buffer [4][128]: the lower
// lane half holds rows i, i+32, the upper rows i+64, i+96.
__device__ __forceinline__ void put_rows(const MMap &a, float r0, float r1, float *buf)
{
    buf[a.w * D + a.i + 64 * a.h] = r0;
    buf[a.w * D + a.i + 64 * a.h + 32] = r1;
}

// This wave's row-energy partials: levels 0..3 cached in rp, level 4 across
// lane bit 5.  Levels 2 and 1 (across waves) are taken by the reader.
__device__ __forceinline__ void put_row_energies(const MMap &a, const float (&rp)[4], float *rowP)
{
    put_rows(a, xhalf32(rp[0], rp[2]), xhalf32(rp[1], rp[3]), rowP);
}

// Greedy pick over the 256 candidates (rows 0..127, then columns 128..255):
// largest energy, lowest candidate on ties, the candidates in pk[0..npk)
// (earlier picks) excluded; -1 when no energy is positive.  Every wave
// computes it from LDS; the row energy is the canonical sum of the four
// waves' partials (w, w ^ 2 first, then the two pairs).  Energies are sums
// of squares (+0 or positive, never -0), so they are compared as their bit
// patterns, with -1 for an excluded candidate; the pick is wave-uniform.
template <int NP>
__device__ __forceinline__ int pick_all(const MMap &a, const float *colE, const float *rowP, const int (&pk)[NP],
                                        int npk)
{
    const int l = a.l;
    int e[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = l + 64 * k;
        e[k] = __float_as_int((rowP[r] + rowP[2 * D + r]) + (rowP[D + r] + rowP[3 * D + r]));
        e[2 + k] = __float_as_int(colE[r]);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j)
        if (j < npk) {
#pragma unroll
            for (int k = 0; k < 4; ++k) e[k] = (pk[j] == 64 * k + l) ? -1 : e[k];
        }
    const int M = __builtin_amdgcn_readfirstlane(wave_max_i(max(max(e[0], e[1]), max(e[2], e[3]))));
    // the lowest candidate holding M: candidate 64 k + l is e[k] of lane l,
    // so the first k whose lane mask is not empty, then its lowest lane
    const uint64_t b0 = __builtin_amdgcn_ballot_w64(e[0] == M), b1 = __builtin_amdgcn_ballot_w64(e[1] == M);
    const uint64_t b2 = __builtin_amdgcn_ballot_w64(e[2] == M), b3 = __builtin_amdgcn_ballot_w64(e[3] == M);
    const int pick = b0 ? __builtin_ctzll(b0) : b1 ? 64 + __builtin_ctzll(b1) : b2 ? 128 + __builtin_ctzll(b2)
                                                                              : 192 + __builtin_ctzll(b3);
    return M > 0 ? pick : -1;
}

// Zeroing an extracted line in the register tile.  The line's position in
// the tile is wave-uniform (a row pick is block p = pick / 32 in the lanes
// with i = pick % 32; a column pick is entry m = c / 8 of the four blocks in
// lane half h of wave c % 4), but the tile is indexed statically.  One asm
// block walks a scalar branch tree on the block (p: 2 bits, m: 4 bits; -1
// skips) down to 16 (row) or 4 (column) lane-masked selects, in place of one
// select per entry (64).  The tree lives inside the asm: a C++ branch on the
// block made the compiler keep a copy of the tile on each side.
__device__ __forceinline__ void zero_line(const MMap &a, float (&S)[4][16], int pick)
{
    const bool isrow = pick >= 0 && pick < D, iscol = pick >= D;
    const int cc = pick - D;
    // -1 matches no block; the owning lanes as a lane mask
    const int pr = __builtin_amdgcn_readfirstlane(isrow ? pick >> 5 : -1);
    const int mm = __builtin_amdgcn_readfirstlane(iscol && a.w == (cc & 3) ? cc >> 3 : -1);
    const uint64_t rl = __builtin_amdgcn_ballot_w64(a.i == (pick & 31));
    const uint64_t cl = __builtin_amdgcn_ballot_w64(a.h == ((cc >> 2) & 1));
    asm volatile("s_cmp_lt_i32 %[pr], 0\n\ts_cbranch_scc1 10f\n\ts_bitcmp1_b32 %[pr], 1\n\ts_cbranch_scc1 11f\n\t"
                 "s_bitcmp1_b32 %[pr], 0\n\ts_cbranch_scc1 12f\n\tv_cndmask_b32_e64 %0, %0, 0, %[rl]\n\tv_cndmask_b32_e64 %1, %1, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %2, %2, 0, %[rl]\n\tv_cndmask_b32_e64 %3, %3, 0, %[rl]\n\tv_cndmask_b32_e64 %4, %4, 0, %[rl]\n\tv_cndmask_b32_e64 %5, %5, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %6, %6, 0, %[rl]\n\tv_cndmask_b32_e64 %7, %7, 0, %[rl]\n\tv_cndmask_b32_e64 %8, %8, 0, %[rl]\n\tv_cndmask_b32_e64 %9, %9, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %10, %10, 0, %[rl]\n\tv_cndmask_b32_e64 %11, %11, 0, %[rl]\n\tv_cndmask_b32_e64 %12, %12, 0, %[rl]\n\tv_cndmask_b32_e64 %13, %13, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %14, %14, 0, %[rl]\n\tv_cndmask_b32_e64 %15, %15, 0, %[rl]\n\ts_branch 10f\n\t12:\n\t"
                 "v_cndmask_b32_e64 %16, %16, 0, %[rl]\n\tv_cndmask_b32_e64 %17, %17, 0, %[rl]\n\tv_cndmask_b32_e64 %18, %18, 0, %[rl]\n\tv_cndmask_b32_e64 %19, %19, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %20, %20, 0, %[rl]\n\tv_cndmask_b32_e64 %21, %21, 0, %[rl]\n\tv_cndmask_b32_e64 %22, %22, 0, %[rl]\n\tv_cndmask_b32_e64 %23, %23, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %24, %24, 0, %[rl]\n\tv_cndmask_b32_e64 %25, %25, 0, %[rl]\n\tv_cndmask_b32_e64 %26, %26, 0, %[rl]\n\tv_cndmask_b32_e64 %27, %27, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %28, %28, 0, %[rl]\n\tv_cndmask_b32_e64 %29, %29, 0, %[rl]\n\tv_cndmask_b32_e64 %30, %30, 0, %[rl]\n\tv_cndmask_b32_e64 %31, %31, 0, %[rl]\n\t"
                 "s_branch 10f\n\t11:\n\ts_bitcmp1_b32 %[pr], 0\n\ts_cbranch_scc1 13f\n\t"
                 "v_cndmask_b32_e64 %32, %32, 0, %[rl]\n\tv_cndmask_b32_e64 %33, %33, 0, %[rl]\n\tv_cndmask_b32_e64 %34, %34, 0, %[rl]\n\tv_cndmask_b32_e64 %35, %35, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %36, %36, 0, %[rl]\n\tv_cndmask_b32_e64 %37, %37, 0, %[rl]\n\tv_cndmask_b32_e64 %38, %38, 0, %[rl]\n\tv_cndmask_b32_e64 %39, %39, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %40, %40, 0, %[rl]\n\tv_cndmask_b32_e64 %41, %41, 0, %[rl]\n\tv_cndmask_b32_e64 %42, %42, 0, %[rl]\n\tv_cndmask_b32_e64 %43, %43, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %44, %44, 0, %[rl]\n\tv_cndmask_b32_e64 %45, %45, 0, %[rl]\n\tv_cndmask_b32_e64 %46, %46, 0, %[rl]\n\tv_cndmask_b32_e64 %47, %47, 0, %[rl]\n\t"
                 "s_branch 10f\n\t13:\n\tv_cndmask_b32_e64 %48, %48, 0, %[rl]\n\tv_cndmask_b32_e64 %49, %49, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %50, %50, 0, %[rl]\n\tv_cndmask_b32_e64 %51, %51, 0, %[rl]\n\tv_cndmask_b32_e64 %52, %52, 0, %[rl]\n\tv_cndmask_b32_e64 %53, %53, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %54, %54, 0, %[rl]\n\tv_cndmask_b32_e64 %55, %55, 0, %[rl]\n\tv_cndmask_b32_e64 %56, %56, 0, %[rl]\n\tv_cndmask_b32_e64 %57, %57, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %58, %58, 0, %[rl]\n\tv_cndmask_b32_e64 %59, %59, 0, %[rl]\n\tv_cndmask_b32_e64 %60, %60, 0, %[rl]\n\tv_cndmask_b32_e64 %61, %61, 0, %[rl]\n\t"
                 "v_cndmask_b32_e64 %62, %62, 0, %[rl]\n\tv_cndmask_b32_e64 %63, %63, 0, %[rl]\n\t10:\n\ts_cmp_lt_i32 %[mm], 0\n\t"
                 "s_cbranch_scc1 14f\n\ts_bitcmp1_b32 %[mm], 3\n\ts_cbranch_scc1 15f\n\ts_bitcmp1_b32 %[mm], 2\n\t"
                 "s_cbranch_scc1 16f\n\ts_bitcmp1_b32 %[mm], 1\n\ts_cbranch_scc1 17f\n\ts_bitcmp1_b32 %[mm], 0\n\t"
                 "s_cbranch_scc1 18f\n\tv_cndmask_b32_e64 %0, %0, 0, %[cl]\n\tv_cndmask_b32_e64 %16, %16, 0, %[cl]\n\tv_cndmask_b32_e64 %32, %32, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %48, %48, 0, %[cl]\n\ts_branch 14f\n\t18:\n\tv_cndmask_b32_e64 %1, %1, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %17, %17, 0, %[cl]\n\tv_cndmask_b32_e64 %33, %33, 0, %[cl]\n\tv_cndmask_b32_e64 %49, %49, 0, %[cl]\n\ts_branch 14f\n\t"
                 "17:\n\ts_bitcmp1_b32 %[mm], 0\n\ts_cbranch_scc1 19f\n\tv_cndmask_b32_e64 %2, %2, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %18, %18, 0, %[cl]\n\tv_cndmask_b32_e64 %34, %34, 0, %[cl]\n\tv_cndmask_b32_e64 %50, %50, 0, %[cl]\n\ts_branch 14f\n\t"
                 "19:\n\tv_cndmask_b32_e64 %3, %3, 0, %[cl]\n\tv_cndmask_b32_e64 %19, %19, 0, %[cl]\n\tv_cndmask_b32_e64 %35, %35, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %51, %51, 0, %[cl]\n\ts_branch 14f\n\t16:\n\ts_bitcmp1_b32 %[mm], 1\n\t"
                 "s_cbranch_scc1 20f\n\ts_bitcmp1_b32 %[mm], 0\n\ts_cbranch_scc1 21f\n\tv_cndmask_b32_e64 %4, %4, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %20, %20, 0, %[cl]\n\tv_cndmask_b32_e64 %36, %36, 0, %[cl]\n\tv_cndmask_b32_e64 %52, %52, 0, %[cl]\n\ts_branch 14f\n\t"
                 "21:\n\tv_cndmask_b32_e64 %5, %5, 0, %[cl]\n\tv_cndmask_b32_e64 %21, %21, 0, %[cl]\n\tv_cndmask_b32_e64 %37, %37, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %53, %53, 0, %[cl]\n\ts_branch 14f\n\t20:\n\ts_bitcmp1_b32 %[mm], 0\n\t"
                 "s_cbranch_scc1 22f\n\tv_cndmask_b32_e64 %6, %6, 0, %[cl]\n\tv_cndmask_b32_e64 %22, %22, 0, %[cl]\n\tv_cndmask_b32_e64 %38, %38, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %54, %54, 0, %[cl]\n\ts_branch 14f\n\t22:\n\tv_cndmask_b32_e64 %7, %7, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %23, %23, 0, %[cl]\n\tv_cndmask_b32_e64 %39, %39, 0, %[cl]\n\tv_cndmask_b32_e64 %55, %55, 0, %[cl]\n\ts_branch 14f\n\t"
                 "15:\n\ts_bitcmp1_b32 %[mm], 2\n\ts_cbranch_scc1 23f\n\ts_bitcmp1_b32 %[mm], 1\n\t"
                 "s_cbranch_scc1 24f\n\ts_bitcmp1_b32 %[mm], 0\n\ts_cbranch_scc1 25f\n\tv_cndmask_b32_e64 %8, %8, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %24, %24, 0, %[cl]\n\tv_cndmask_b32_e64 %40, %40, 0, %[cl]\n\tv_cndmask_b32_e64 %56, %56, 0, %[cl]\n\ts_branch 14f\n\t"
                 "25:\n\tv_cndmask_b32_e64 %9, %9, 0, %[cl]\n\tv_cndmask_b32_e64 %25, %25, 0, %[cl]\n\tv_cndmask_b32_e64 %41, %41, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %57, %57, 0, %[cl]\n\ts_branch 14f\n\t24:\n\ts_bitcmp1_b32 %[mm], 0\n\t"
                 "s_cbranch_scc1 26f\n\tv_cndmask_b32_e64 %10, %10, 0, %[cl]\n\tv_cndmask_b32_e64 %26, %26, 0, %[cl]\n\tv_cndmask_b32_e64 %42, %42, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %58, %58, 0, %[cl]\n\ts_branch 14f\n\t26:\n\tv_cndmask_b32_e64 %11, %11, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %27, %27, 0, %[cl]\n\tv_cndmask_b32_e64 %43, %43, 0, %[cl]\n\tv_cndmask_b32_e64 %59, %59, 0, %[cl]\n\ts_branch 14f\n\t"
                 "23:\n\ts_bitcmp1_b32 %[mm], 1\n\ts_cbranch_scc1 27f\n\ts_bitcmp1_b32 %[mm], 0\n\t"
                 "s_cbranch_scc1 28f\n\tv_cndmask_b32_e64 %12, %12, 0, %[cl]\n\tv_cndmask_b32_e64 %28, %28, 0, %[cl]\n\tv_cndmask_b32_e64 %44, %44, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %60, %60, 0, %[cl]\n\ts_branch 14f\n\t28:\n\tv_cndmask_b32_e64 %13, %13, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %29, %29, 0, %[cl]\n\tv_cndmask_b32_e64 %45, %45, 0, %[cl]\n\tv_cndmask_b32_e64 %61, %61, 0, %[cl]\n\ts_branch 14f\n\t"
                 "27:\n\ts_bitcmp1_b32 %[mm], 0\n\ts_cbranch_scc1 29f\n\tv_cndmask_b32_e64 %14, %14, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %30, %30, 0, %[cl]\n\tv_cndmask_b32_e64 %46, %46, 0, %[cl]\n\tv_cndmask_b32_e64 %62, %62, 0, %[cl]\n\ts_branch 14f\n\t"
                 "29:\n\tv_cndmask_b32_e64 %15, %15, 0, %[cl]\n\tv_cndmask_b32_e64 %31, %31, 0, %[cl]\n\tv_cndmask_b32_e64 %47, %47, 0, %[cl]\n\t"
                 "v_cndmask_b32_e64 %63, %63, 0, %[cl]\n\ts_branch 14f\n\t14:\n\t"
                 : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[0][2]), "+v"(S[0][3]), "+v"(S[0][4]), "+v"(S[0][5]),
                   "+v"(S[0][6]), "+v"(S[0][7]), "+v"(S[0][8]), "+v"(S[0][9]), "+v"(S[0][10]),
                   "+v"(S[0][11]), "+v"(S[0][12]), "+v"(S[0][13]), "+v"(S[0][14]), "+v"(S[0][15]),
                   "+v"(S[1][0]), "+v"(S[1][1]), "+v"(S[1][2]), "+v"(S[1][3]), "+v"(S[1][4]),
                   "+v"(S[1][5]), "+v"(S[1][6]), "+v"(S[1][7]), "+v"(S[1][8]), "+v"(S[1][9]),
                   "+v"(S[1][10]), "+v"(S[1][11]), "+v"(S[1][12]), "+v"(S[1][13]), "+v"(S[1][14]),
                   "+v"(S[1][15]), "+v"(S[2][0]), "+v"(S[2][1]), "+v"(S[2][2]), "+v"(S[2][3]),
                   "+v"(S[2][4]), "+v"(S[2][5]), "+v"(S[2][6]), "+v"(S[2][7]), "+v"(S[2][8]),
                   "+v"(S[2][9]), "+v"(S[2][10]), "+v"(S[2][11]), "+v"(S[2][12]), "+v"(S[2][13]),
                   "+v"(S[2][14]), "+v"(S[2][15]), "+v"(S[3][0]), "+v"(S[3][1]), "+v"(S[3][2]),
                   "+v"(S[3][3]), "+v"(S[3][4]), "+v"(S[3][5]), "+v"(S[3][6]), "+v"(S[3][7]),
                   "+v"(S[3][8]), "+v"(S[3][9]), "+v"(S[3][10]), "+v"(S[3][11]), "+v"(S[3][12]),
                   "+v"(S[3][13]), "+v"(S[3][14]), "+v"(S[3][15])
                 : [pr] "s"(pr), [mm] "s"(mm), [rl] "s"(rl), [cl] "s"(cl)
                 : "scc");
}

// Low byte of the integer nearest to the exact product x * g (ties to even)
// for |x * g| < 2^22: the fused add of 1.5 * 2^23 rounds the product once,
// to an integer in the low mantissa bits.
__device__ __forceinline__ uint32_t rint_bits(float x, float g) { return __float_as_uint(fma_(x, g, 12582912.0f)); }
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3)
{
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Rank-one compensators by power sweeps (the rank-one fold option), in
// order: the row of largest canonical energy (lowest index on ties; none,
// with a zero pair and index -1, when no energy is positive); b = that row;
// eight sweeps a = S b (canonical row dots), a = a * (1 / sqrt(T(a . a))),
// b = S^T a (canonical column dots); the pair [a | b] is stored and S
// deflated by fma(-a_r, b_c, S).  The row dots reduce like the row energies
// (inside the thread, then lane bit 5, then across waves through LDS), the
// column dots like the column energies; two barriers per sweep.
template <int CT>
__device__ __forceinline__ void fit_rank1(const MMap &a, float (&S)[4][16], const HeadState &hs, int C, FoldWork &sm)
{
    const int t = threadIdx.x, l = a.l;
    constexpr int NR = CT >= 0 ? CT : 4;
    const int nrounds = CT >= 0 ? CT : C;
    float *bv = sm.colE[0];    // b, 128 values
    float *rowP = sm.rowP[0];  // per-wave row partials [4][128]
    auto combined = [&](int r) { return (rowP[r] + rowP[2 * D + r]) + (rowP[D + r] + rowP[3 * D + r]); };
#pragma unroll
    for (int jj = 0; jj < NR; ++jj) {
        if (jj >= nrounds) break;
        {
            float rp[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) rp[p] = row_partial(S, p);
            put_row_energies(a, rp, rowP);
        }
        lds_barrier();
        const float e0 = combined(l), e1 = combined(l + 64);
        const float M = wave_max(fmaxf(e0, e1));
        int pick = -1;
        if (M > 0.0f) {
            const int cand = e0 == M ? l : e1 == M ? 64 + l : 1 << 20;
            pick = __builtin_amdgcn_readfirstlane(wave_min(cand));
        }
        if (t == 0) hs.cidx[jj] = pick;
        float *aout = hs.cvec + jj * 2 * D, *bout = aout + D;
        if (pick < 0) {
            aout[t] = 0.0f;  // a and b: 256 values
            continue;
        }
        const int pr = pick >> 5;
        if (a.i == (pick & 31)) {
            // row pr of S by value selects (a branch per p becomes a runtime
            // index into S)
#pragma unroll
            for (int m = 0; m < 16; ++m)
                bv[a.col(m)] = sel((pr & 2) != 0, sel((pr & 1) != 0, TS(S, 3, m), TS(S, 2, m)),
                                   sel((pr & 1) != 0, TS(S, 1, m), TS(S, 0, m)));
        }
        lds_barrier();
        float bc[16], ar[4], a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m) bc[m] = bv[a.col(m)];
        bool dead = false;
        for (int s = 0; s < 8; ++s) {
            float rd[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float x[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = fma_(TS(S, p, m), bc[m], TS(S, p, m + 8) * bc[m + 8]);
#pragma unroll
                for (int m = 0; m < 4; ++m) x[m] = x[m] + x[m + 4];
                x[0] = x[0] + x[2];
                x[1] = x[1] + x[3];
                rd[p] = x[0] + x[1];
            }
            put_rows(a, xhalf32(rd[0], rd[2]), xhalf32(rd[1], rd[3]), rowP);
            lds_barrier();
#pragma unroll
            for (int p = 0; p < 4; ++p) ar[p] = combined(a.row(p));
            a0 = combined(l);
            a1 = combined(l + 64);
            const float na2 = wdot(a0, a1, a0, a1);
            if (!(na2 > 0.0f)) {
                dead = true;
                break;
            }
            const float inv = 1.0f / sqrtf(na2);
#pragma unroll
            for (int p = 0; p < 4; ++p) ar[p] = ar[p] * inv;
            a0 = a0 * inv;
            a1 = a1 * inv;
            float cp[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
                cp[m] = fma_(TS(S, 0, m), ar[0], TS(S, 2, m) * ar[2]) + fma_(TS(S, 1, m), ar[1], TS(S, 3, m) * ar[3]);
            const float bcol = mcolsum16(cp, l);
            if ((l & 1) == 0) bv[a.col(mcol_of(l))] = bcol;
            lds_barrier();
#pragma unroll
            for (int m = 0; m < 16; ++m) bc[m] = bv[a.col(m)];
        }
        if (dead) {
            aout[t] = 0.0f;
            continue;
        }
        if (a.w == 0) {
            aout[l] = a0;
            aout[l + 64] = a1;
        } else if (a.w == 1) {
            bout[l] = bv[l];
            bout[l + 64] = bv[l + 64];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int m = 0; m < 16; ++m) TS(S, p, m) = fma_(-ar[p], bc[m], TS(S, p, m));
    }
}

// Canonical 128-term dot of two vectors held in the row layout (rows
// i + 32p of the thread, p = 0..3, the same in both lane halves and in every
// wave): levels 0 (p, p + 2) and 32 (p = 0, 1) inside the thread, then
// levels 16, 8, 4, 2, 1 as butterflies on lane bit 4 (permlane16 swap), lane
// bit 3 (row_ror:8), lane ^ 7 (row_half_mirror: row ^ 4 through the xor in
// i), lane bits 1 and 0.  Every lane ends with the value.
__device__ __forceinline__ float rdot(const float (&x)[4], const float (&y)[4])
{
    float s = fma_(x[0], y[0], x[2] * y[2]) + fma_(x[1], y[1], x[3] * y[3]);
    s = xhalf16(s, s);
    s = s + dpp<DPP_ROR8>(s);
    s = s + dpp<DPP_HMIR>(s);
    s = s + dpp<DPP_XOR2>(s);
    return s + dpp<DPP_XOR1>(s);
}

// Block fit of the compensators (the block fold option): subspace iteration
// on the key side, fitting the pairs together.  Start: with WARM, a slot
// whose stored index is live starts from its stored a (prev, staged in LDS);
// every other slot, in slot order, from the unit vector of the next row by
// canonical energy (largest first, lowest index on ties, zero-energy rows
// never), else from zero.  Then A = MGS(start); per sweep z_j = S^T a_j
// (canonical column dots), y_j = S z_j (canonical row dots), A = MGS(Y);
// finally b_j = S^T a_j, index j (or -1 for an unused slot), and S deflated
// by fma(-a_j[r], b_j[c], S) in slot order.  MGS projects each earlier live
// slot out with fma(-T(a_i . y), a_i, y), then scales by 1 / sqrt(T(y . y))
// or leaves the slot unused (zero) when that norm is not positive.  A lives
// in the row layout (4 values per slot and thread), so its dots are rdot;
// two barriers per sweep.
template <int CT, bool WARM>
__device__ __forceinline__ void fit_block(const MMap &a, float (&S)[4][16], const HeadState &hs, int C,
                                          const float *prev, const int *prev_idx, int sweeps, FoldWork &fw)
{
    constexpr int NR = CT >= 0 ? CT : 4;
    const int nslot = CT >= 0 ? CT : C;
    BlockWork &bw = *reinterpret_cast<BlockWork *>(&fw);
    const int t = threadIdx.x, l = a.l;
    const int zb = (2 * a.w + a.h) * 16;
    float A[NR][4];
    bool live[NR];
    bool warm[NR];
    bool any_cold = false;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        warm[j] = WARM && j < nslot && prev_idx[j] >= 0;
        any_cold = any_cold || (j < nslot && !warm[j]);
    }
    // ---- start vectors
    float e0 = -1.0f, e1 = -1.0f;
    if (any_cold) {
        float rp[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) rp[p] = row_partial(S, p);
        put_row_energies(a, rp, fw.rowP[0]);
        lds_barrier();
        const float *rowP = fw.rowP[0];
        e0 = (rowP[l] + rowP[2 * D + l]) + (rowP[D + l] + rowP[3 * D + l]);
        e1 = (rowP[l + 64] + rowP[2 * D + l + 64]) + (rowP[D + l + 64] + rowP[3 * D + l + 64]);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        if (j >= nslot) break;
        if (warm[j]) {
#pragma unroll
            for (int p = 0; p < 4; ++p) A[j][p] = prev[2 * j * D + a.row(p)];
        } else {
            const float M = wave_max(fmaxf(e0, e1));
            int pick = -1;
            if (M > 0.0f) {
                const int cand = e0 == M ? l : e1 == M ? 64 + l : 1 << 20;
                pick = __builtin_amdgcn_readfirstlane(wave_min(cand));
                e0 = pick == l ? -1.0f : e0;
                e1 = pick == l + 64 ? -1.0f : e1;
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) A[j][p] = a.row(p) == pick ? 1.0f : 0.0f;
        }
    }
    auto mgs = [&]() {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            if (j >= nslot) break;
#pragma unroll
            for (int i = 0; i < j; ++i) {
                const float d = rdot(A[i], A[j]);
#pragma unroll
                for (int p = 0; p < 4; ++p) A[j][p] = live[i] ? fma_(-d, A[i][p], A[j][p]) : A[j][p];
            }
            const float n2 = rdot(A[j], A[j]);
            live[j] = n2 > 0.0f;
            const float inv = 1.0f / sqrtf(live[j] ? n2 : 1.0f);
#pragma unroll
            for (int p = 0; p < 4; ++p) A[j][p] = live[j] ? A[j][p] * inv : 0.0f;
        }
    };
    // z_j = S^T a_j over the wave's own columns (canonical column dots)
    auto col_dots = [&]() {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            if (j >= nslot) break;
            float cp[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
                cp[m] = fma_(TS(S, 0, m), A[j][0], TS(S, 2, m) * A[j][2]) +
                        fma_(TS(S, 1, m), A[j][1], TS(S, 3, m) * A[j][3]);
            const float z = mcolsum16(cp, l);
            if ((l & 1) == 0) bw.z[j][zb + mcol_of(l)] = z;
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    mgs();
    for (int s = 0; s < sweeps; ++s) {
        col_dots();
        lds_barrier();
        // y_j = S z_j: rows inside the thread, lane bit 5, then across waves
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            if (j >= nslot) break;
            float zc[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4 *>(&bw.z[j][zb + 4 * q]);
                zc[4 * q] = v.x;
                zc[4 * q + 1] = v.y;
                zc[4 * q + 2] = v.z;
                zc[4 * q + 3] = v.w;
            }
            float rd[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float x[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = fma_(TS(S, p, m), zc[m], TS(S, p, m + 8) * zc[m + 8]);
#pragma unroll
                for (int m = 0; m < 4; ++m) x[m] = x[m] + x[m + 4];
                x[0] = x[0] + x[2];
                x[1] = x[1] + x[3];
                rd[p] = x[0] + x[1];
            }
            const int r = a.i + 64 * a.h;
            bw.P[j][r][a.w] = xhalf32(rd[0], rd[2]);
            bw.P[j][r + 32][a.w] = xhalf32(rd[1], rd[3]);
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            if (j >= nslot) break;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float4 v = *reinterpret_cast<const float4 *>(&bw.P[j][a.row(p)][0]);
                A[j][p] = (v.x + v.z) + (v.y + v.w);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mgs();
    }
    col_dots();  // b_j = S^T a_j
    lds_barrier();
    // store the pairs, then deflate
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        if (j >= nslot) break;
        float *aout = hs.cvec + j * 2 * D, *bout = aout + D;
        if (t == 0) hs.cidx[j] = live[j] ? j : -1;
        if (a.w == 0 && a.h == 0) {
#pragma unroll
            for (int p = 0; p < 4; ++p) aout[a.row(p)] = A[j][p];
        } else if (a.w == 1) {
            bout[l] = bw.z[j][zpos(l)];
            bout[l + 64] = bw.z[j][zpos(l + 64)];
        }
        float bc[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(&bw.z[j][zb + 4 * q]);
            bc[4 * q] = v.x;
            bc[4 * q + 1] = v.y;
            bc[4 * q + 2] = v.z;
            bc[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int m = 0; m < 16; ++m) TS(S, p, m) = fma_(-A[j][p], bc[m], TS(S, p, m));
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Steps after the rebuild, shared by init and fold.  Writes the head's new
// boundary state (codes, rho, sigma, indices, compensators).  CT >= 0: the
// number of compensators as a compile-time constant (C == CT), unrolling the
// rounds.  R1: compensator pairs in place of lines, fitted by power sweeps,
// or with BLK by the block fit (WARM: from the pairs staged in prev and
// prev_idx, the window's own).
template <int CT, bool R1 = false, bool BLK = false, bool WARM = false, int CB = 8>
__device__ __forceinline__ void quantize_state(const MMap &a, float (&S)[4][16], const HeadState &hs, int C, int smoothing,
                                               float floor_, FoldWork &sm, const float *prev = nullptr,
                                               const int *prev_idx = nullptr)
{
    const int t = threadIdx.x, l = a.l;
    // ---- compensator tokens.  Lines: one greedy round per compensator (pick,
    // store and zero the line, rescore the other axis).  Every wave takes the
    // same pick from the energies in LDS, so a round needs one barrier: the
    // rescored axis is written to the other of its two buffers, which no wave
    // reads until that barrier.  The rounds are unrolled (C <= 8) and written
    // out here, not called, so S stays in registers.
    if (BLK && C > 0) {
        fit_block<CT, WARM>(a, S, hs, C, prev, prev_idx, WARM ? kBlockSweeps : kBlockSweepsInit, sm);
        lds_barrier();
    } else if (R1 && C > 0) {
        fit_rank1<CT>(a, S, hs, C, sm);
        lds_barrier();
    } else if (C > 0) {
        constexpr int NR = CT >= 0 ? CT : 8;
        const int nrounds = CT >= 0 ? CT : C;
        float rp[4];
        int pk[NR];
        int cb = 0, rb = 0;
        {
            float cp[16];
            col_partials(S, cp);
            put_cols(a, cp, sm.colE[0]);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) rp[p] = row_partial(S, p);
        put_row_energies(a, rp, sm.rowP[0]);
        lds_barrier();
        // Rescoring is lazy.  Removing a line only lowers the other axis's
        // energies (every square and every add of the canonical tree is
        // monotone), so after a row pick the stale column energies bound the
        // true ones from above, and likewise for rows after a column pick.
        // A pick made with stale energies on the other axis is therefore the
        // greedy pick whenever it falls on the fresh axis (a row beats every
        // column it ties, a column must beat the rows strictly); only a pick
        // on a stale axis rescores that axis (one barrier) and picks again.
        // At most one axis is stale at a time: a pick is only taken on a
        // fresh axis.
        bool staleR = false, staleC = false;
        bool dirty = false;  // this wave's row partials miss a zeroed column of its own
#pragma unroll
        for (int jj = 0; jj < NR; ++jj) {
            if (jj >= nrounds) break;
            int pick = pick_all(a, sm.colE[cb], sm.rowP[rb], pk, jj);
            if ((pick >= 0 && pick < D && staleR) || (pick >= D && staleC)) {
                if (pick >= D) {
                    // column energies from S (picked lines already zeroed)
                    float cp[16];
                    col_partials(S, cp);
                    put_cols(a, cp, sm.colE[cb ^ 1]);
                    cb ^= 1;
                    staleC = false;
                } else {
                    if (dirty) {
#pragma unroll
                        for (int p = 0; p < 4; ++p) rp[p] = row_partial(S, p);
                    }
                    dirty = false;
                    put_row_energies(a, rp, sm.rowP[rb ^ 1]);
                    rb ^= 1;
                    staleR = false;
                }
                lds_barrier();
                pick = pick_all(a, sm.colE[cb], sm.rowP[rb], pk, jj);
            }
            pk[jj] = pick;
            float *vec = hs.cvec + jj * D;
            if (t == 0) hs.cidx[jj] = pick;
            // a row pick is owned by the two lanes per wave with i == pick % 32
            // (row p = pick / 32); a column pick by lane half h of wave w
            // (m = c / 8).  One straight pass over S per round: S keeps its
            // registers across the rounds.
            const bool isrow = pick >= 0 && pick < D, iscol = pick >= D;
            const int pr = pick >> 5, cc = pick - D, mm = cc >> 3;
            const bool own_r = isrow && a.i == (pick & 31);
            const bool own_c = iscol && a.w == (cc & 3) && a.h == ((cc >> 2) & 1);
            if (pick < 0 && t < D) vec[t] = 0.0f;
            // the line's stores from its own registers, one uniform branch
            // per candidate block; the empty asm statements differ per
            // branch, so the compiler cannot merge the branches' stores into
            // one store of a selected (copied) block
            if (own_r) {
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    if (p == pr) {
#pragma unroll
                        for (int m = 0; m < 16; ++m) vec[a.col(m)] = TS(S, p, m);
                        asm volatile("; row line block %0" ::"n"(p) : "memory");
                    }
            }
            if (own_c) {
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    if (m == mm) {
#pragma unroll
                        for (int p = 0; p < 4; ++p) vec[a.row(p)] = TS(S, p, m);
                        asm volatile("; column line entry %0" ::"n"(m) : "memory");
                    }
            }
            zero_line(a, S, pick);
#pragma unroll
            for (int p = 0; p < 4; ++p) rp[p] = (own_r && p == pr) ? 0.0f : rp[p];
            staleC = staleC || isrow;
            staleR = staleR || iscol;
            dirty = dirty || (iscol && a.w == (cc & 3));
        }
    }
    // ---- residual smoothing
    {
        float v[16];
#pragma unroll
        for (int m = 0; m < 16; ++m)
            v[m] = (fabsf(TS(S, 0, m)) + fabsf(TS(S, 2, m))) + (fabsf(TS(S, 1, m)) + fabsf(TS(S, 3, m)));
        const float msum = mcolsum16(v, l);
        if ((l & 1) == 0) {
            const int c = a.col(mcol_of(l));
            float s = 1.0f;
            if (smoothing) {
                s = sqrtf(msum * 0.0078125f);
                if (s < floor_) s = floor_;
            }
            hs.sigma[c] = s;
            sm.sinv[c] = 1.0f / s;
        }
    }
    // the wave reads back only its own columns: LDS order within the wave
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    // ---- per-row symmetric codes (int8, or 6 / 4 bits), round half to even
    {
        float inv[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) inv[m] = sm.sinv[a.col(m)];
        float mx[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float Mx = 0.0f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                TS(S, p, m) = TS(S, p, m) * inv[m];
                Mx = fmaxf(Mx, fabsf(TS(S, p, m)));
            }
            mx[p] = Mx;
        }
        put_rows(a, xhalf32max(mx[0], mx[2]), xhalf32max(mx[1], mx[3]), sm.part);
    }
    lds_barrier();
    // every wave forms 127 / M_r for all rows (lane l: rows l, l + 64) in its
    // own buffer; wave 0 also stores rho
    {
        float *rg = sm.rowg[a.w];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = l + 64 * k;
            const float M = fmaxf(fmaxf(sm.part[r], sm.part[D + r]), fmaxf(sm.part[2 * D + r], sm.part[3 * D + r]));
            const bool live = M >= 0x1p-120f;
            if (a.w == 0) hs.rho[r] = live ? M / CodeFmt<CB>::levels : 0.0f;
            rg[r] = live ? CodeFmt<CB>::levels / M : 0.0f;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
    uint32_t B[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float g = sm.rowg[a.w][a.row(p)];
        uint32_t b[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) b[m] = rint_bits(TS(S, p, m), g);
#pragma unroll
        for (int k = 0; k < 4; ++k) B[p][k] = pack4(b[4 * k], b[4 * k + 1], b[4 * k + 2], b[4 * k + 3]);
    }
    store_codes<CB>(hs.codes, a.w, a.l, B);
}

template <int CT, bool R1, bool BLK = false, int CB = 8>
__global__ __launch_bounds__(NT) void k_init(StateView sv, const float *__restrict__ S0, int smoothing,
                                              float floor_)
{
    __shared__ FoldWork wk;
    const MMap a = mmap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const float *src = S0 + (size_t)h * D * D;
    float S[4][16];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) TS(S, p, m) = src[a.row(p) * D + a.col(m)];
    quantize_state<CT, R1, BLK, false, CB>(a, S, hs, sv.C, smoothing, floor_, wk);
}

template <typename K, int CT, bool CH, typename U, bool R1, bool BLK = false, int CB = 8>
__global__ __launch_bounds__(NT) void k_fold(StateView sv, int n, int smoothing, float floor_)
{
    __shared__ FoldStage<Rec<K, CH, U>::stride> st;
    __shared__ FoldWork wk;
    const MMap a = mmap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    uint4 qc[4];
    load_codes<CB>(a, hs, qc);
    stage_small<CH, decltype(st), R1>(a, hs, sv.C, n, st);
    stage_records<K, CH, U>(a, hs, 0, n < 16 ? n : 16, st);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float S[4][16];
    rebuild<K, CH, U, decltype(st), R1, false, CB>(a, hs, qc, sv.C, n, true, st, S, st.gW);
    // no barrier: the quantization writes only LDS arrays the rebuild does
    // not read, and each thread rewrites only the codes it loaded
    quantize_state<CT, R1, BLK, true, CB>(a, S, hs, sv.C, smoothing, floor_, wk, st.lines, st.idx);
}

// The last token of a full window and the fold, in one launch (W <= 16).
// The append's staging (codes in registers, records and the other operands
// in LDS) serves both steps: the token's output is written as by the append,
// its record goes into LDS slot n instead of HBM (the fold consumes it and
// empties the buffer), and the fold rebuilds from the same registers and LDS
// instead of reading the boundary and the records again.  The results are
// those of leapq_append followed by leapq_fold.
template <typename T, typename K, bool GATED, bool NORM, bool CH, typename U, bool R1, int CT, bool BLK = false,
          int CB = 8>
__global__ __launch_bounds__(NT) void k_append_fold(StateView sv, int n, const T *__restrict__ qin,
                                                     const T *__restrict__ kin, const T *__restrict__ vin,
                                                     const float *__restrict__ alpha,
                                                     const float *__restrict__ beta, float *__restrict__ o,
                                                     int smoothing, float floor_, GateArgs g)
{
    using R = Rec<K, CH, U>;
    __shared__ FoldStage<R::stride> st;
    __shared__ float sin_[InLds<T>::floats];
    __shared__ float dots[kDotFloats];
    __shared__ FoldWork wk;
    const MMap a = mmap();
    const int h = blockIdx.x;
    // with CH the token's decay vector is staged in gW (the fold then reads
    // gamma_n from the token's own record slot)
    const HeadLds<T, K, CH, U, R1> L(st.rec, st.lines, st.rho, sin_, st.idx, CH ? st.gW : st.gam);
    uint4 qc[4];
    append_issue<T, K, CH, U, R1, CB>(sv, n, h, qin, kin, vin, a, L, qc, alpha);
    float a_h = CH ? 1.0f : sload(alpha, h);
    float b_h = sload(beta, h);
    if constexpr (GATED) gate_issue(g, h, a, a_h, b_h, dots);
    wait_lds_copies<CodeFmt<CB>::loads>();
    lds_barrier();
    if constexpr (GATED) {
        a_h = dots[kGateSlot];
        b_h = dots[kGateSlot + 1];
    }
    // the records' weighted keys go to the work area, unused until the
    // rebuild has read them (barrier below)
    float *wkeys = reinterpret_cast<float *>(&wk);
    append_compute<T, K, true, NORM, CH, U, R1, CB>(sv, n, h, a, L, dots, qc, a_h, b_h, o, g.q_scale, g.eps, wkeys);
    lds_barrier();  // record n is in LDS for every wave
    const HeadState hs = head_state(sv, h);
    float S[4][16];
    rebuild<K, CH, U, decltype(st), R1, true, CB>(a, hs, qc, sv.C, n + 1, true, st, S,
                                                    st.rec + n * R::stride + R::goff, wkeys);
    lds_barrier();  // every wave is done with the weighted keys
    quantize_state<CT, R1, BLK, true, CB>(a, S, hs, sv.C, smoothing, floor_, wk, st.lines, st.idx);
}

// One decode token with a window phase per request (W <= 16).  The heads of
// request b (blocks b * heads_per_req ..) hold n = n_in[b] records: with
// n = W - 1 the head appends and folds in this launch (the steps of
// k_append_fold), with 0 <= n < W - 1 it appends (the steps of k_append,
// staged as in k_append_fold), and any other n takes no token: the head's
// state and output are left as they are.  Block 0 of each request writes the
// request's next count to n_out (when given): 0 after a fold, n + 1 after an
// append, n unchanged otherwise.  n is uniform per block, so the branches
// cost nothing, but every block is resourced for the fold.
template <typename T, typename K, bool GATED, bool NORM, bool CH, typename U, bool R1, int CT, bool BLK>
__global__ __launch_bounds__(NT) void k_step(StateView sv, int heads_per_req, const int *__restrict__ n_in,
                                              int *__restrict__ n_out, const T *__restrict__ qin,
                                              const T *__restrict__ kin, const T *__restrict__ vin,
                                              const float *__restrict__ alpha, const float *__restrict__ beta,
                                              float *__restrict__ o, int smoothing, float floor_, GateArgs g)
{
    using R = Rec<K, CH, U>;
    __shared__ FoldStage<R::stride> st;
    __shared__ float sin_[InLds<T>::floats];
    __shared__ float dots[kDotFloats];
    __shared__ FoldWork wk;
    const MMap a = mmap();
    const int h = blockIdx.x;
    const int req = h / heads_per_req;
    const int n = sloadi(n_in, req);
    const bool take = n >= 0 && n < sv.W;
    const bool last = n == sv.W - 1;
    if (n_out && h == req * heads_per_req && threadIdx.x == 0) n_out[req] = !take ? n : last ? 0 : n + 1;
    if (!take) return;
    const HeadLds<T, K, CH, U, R1> L(st.rec, st.lines, st.rho, sin_, st.idx, CH ? st.gW : st.gam);
    uint4 qc[4];
    append_issue<T, K, CH, U, R1>(sv, n, h, qin, kin, vin, a, L, qc, alpha);
    float a_h = CH ? 1.0f : sload(alpha, h);
    float b_h = sload(beta, h);
    if constexpr (GATED) gate_issue(g, h, a, a_h, b_h, dots);
    wait_lds_copies();
    lds_barrier();
    if constexpr (GATED) {
        a_h = dots[kGateSlot];
        b_h = dots[kGateSlot + 1];
    }
    if (!last) {
        append_compute<T, K, false, NORM, CH, U, R1>(sv, n, h, a, L, dots, qc, a_h, b_h, o, g.q_scale, g.eps);
        return;
    }
    // the records' weighted keys go to the work area, unused until the
    // rebuild has read them (barrier below)
    float *wkeys = reinterpret_cast<float *>(&wk);
    append_compute<T, K, true, NORM, CH, U, R1>(sv, n, h, a, L, dots, qc, a_h, b_h, o, g.q_scale, g.eps, wkeys);
    lds_barrier();  // record n is in LDS for every wave
    const HeadState hs = head_state(sv, h);
    float S[4][16];
    rebuild<K, CH, U, decltype(st), R1, true>(a, hs, qc, sv.C, n + 1, true, st, S, st.rec + n * R::stride + R::goff,
                                                wkeys);
    lds_barrier();  // every wave is done with the weighted keys
    quantize_state<CT, R1, BLK, true>(a, S, hs, sv.C, smoothing, floor_, wk, st.lines, st.idx);
}

template <typename K, bool CH, typename U, bool R1, int CB = 8>
__global__ __launch_bounds__(NT) void k_dequant(StateView sv, int n, int what, float *__restrict__ out)
{
    __shared__ FoldStage<Rec<K, CH, U>::stride> st;
    const MMap a = mmap();
    const int h = blockIdx.x;
    const HeadState hs = head_state(sv, h);
    const int nr = what == 2 ? n : 0;
    uint4 qc[4];
    load_codes<CB>(a, hs, qc);
    stage_small<CH, decltype(st), R1>(a, hs, sv.C, nr, st);
    stage_records<K, CH, U>(a, hs, 0, nr < 16 ? nr : 16, st);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float S[4][16];
    rebuild<K, CH, U, decltype(st), R1, false, CB>(a, hs, qc, sv.C, nr, what >= 1, st, S, st.gW);
    float *dst = out + (size_t)h * D * D;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) dst[a.row(p) * D + a.col(m)] = TS(S, p, m);
}

}  // namespace

template <int CB>
static void launch_init_bits(const StateView &sv, int heads, const float *S0, int smoothing, float floor_,
                             hipStream_t s)
{
    if (sv.C == 4)
        hipLaunchKernelGGL((k_init<4, false, false, CB>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
    else
        hipLaunchKernelGGL((k_init<-1, false, false, CB>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
}

hipError_t launch_init(const StateView &sv, int heads, const float *S0, int smoothing, float floor_,
                       hipStream_t s)
{
    if (sv.cbits == 6) {
        launch_init_bits<6>(sv, heads, S0, smoothing, floor_, s);
    } else if (sv.cbits == 4) {
        launch_init_bits<4>(sv, heads, S0, smoothing, floor_, s);
    } else if (sv.blk) {
        if (sv.C == 4)
            hipLaunchKernelGGL((k_init<4, true, true>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
        else
            hipLaunchKernelGGL((k_init<-1, true, true>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
    } else if (sv.r1) {
        if (sv.C == 4)
            hipLaunchKernelGGL((k_init<4, true>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
        else
            hipLaunchKernelGGL((k_init<-1, true>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
    } else if (sv.C == 4) {
        hipLaunchKernelGGL((k_init<4, false>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
    } else {
        hipLaunchKernelGGL((k_init<-1, false>), dim3(heads), dim3(NT), 0, s, sv, S0, smoothing, floor_);
    }
    return hipGetLastError();
}

template <typename K, bool CH, typename U = float, bool R1 = false, bool BLK = false, int CB = 8>
static void launch_fold_t(const StateView &sv, int heads, int n, int smoothing, float floor_, hipStream_t s)
{
    if (sv.C == 4)
        hipLaunchKernelGGL((k_fold<K, 4, CH, U, R1, BLK, CB>), dim3(heads), dim3(NT), 0, s, sv, n, smoothing,
                           floor_);
    else
        hipLaunchKernelGGL((k_fold<K, -1, CH, U, R1, BLK, CB>), dim3(heads), dim3(NT), 0, s, sv, n, smoothing,
                           floor_);
}

hipError_t launch_fold(const StateView &sv, int heads, int n, int smoothing, float floor_, hipStream_t s)
{
    if (sv.cbits != 8) {  // 6 or 4 bits: scalar decay, lines, fp32 corrections
        if (sv.cbits == 6) {
            if (sv.key_bf16)
                launch_fold_t<uint16_t, false, float, false, false, 6>(sv, heads, n, smoothing, floor_, s);
            else
                launch_fold_t<float, false, float, false, false, 6>(sv, heads, n, smoothing, floor_, s);
        } else {
            if (sv.key_bf16)
                launch_fold_t<uint16_t, false, float, false, false, 4>(sv, heads, n, smoothing, floor_, s);
            else
                launch_fold_t<float, false, float, false, false, 4>(sv, heads, n, smoothing, floor_, s);
        }
    } else if (sv.blk) {
        if (sv.key_bf16)
            launch_fold_t<uint16_t, false, float, true, true>(sv, heads, n, smoothing, floor_, s);
        else
            launch_fold_t<float, false, float, true, true>(sv, heads, n, smoothing, floor_, s);
    } else if (sv.r1) {
        if (sv.key_bf16)
            launch_fold_t<uint16_t, false, float, true>(sv, heads, n, smoothing, floor_, s);
        else
            launch_fold_t<float, false, float, true>(sv, heads, n, smoothing, floor_, s);
    } else if (sv.u_bf16) {
        if (sv.key_bf16)
            launch_fold_t<uint16_t, false, uint16_t>(sv, heads, n, smoothing, floor_, s);
        else
            launch_fold_t<float, false, uint16_t>(sv, heads, n, smoothing, floor_, s);
    } else if (sv.u_fp8) {
        if (sv.key_bf16)
            launch_fold_t<uint16_t, false, Fp8>(sv, heads, n, smoothing, floor_, s);
        else
            launch_fold_t<float, false, Fp8>(sv, heads, n, smoothing, floor_, s);
    } else if (sv.kda) {
        if (sv.key_bf16)
            launch_fold_t<uint16_t, true>(sv, heads, n, smoothing, floor_, s);
        else
            launch_fold_t<float, true>(sv, heads, n, smoothing, floor_, s);
    } else if (sv.key_bf16) {
        launch_fold_t<uint16_t, false>(sv, heads, n, smoothing, floor_, s);
    } else {
        launch_fold_t<float, false>(sv, heads, n, smoothing, floor_, s);
    }
    return hipGetLastError();
}

template <typename T, typename K, bool GATED, bool NORM, bool CH = false, typename U = float, bool R1 = false,
          bool BLK = false, int CB = 8>
static void launch_append_fold_t(const StateView &sv, int heads, int n, const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta, float *o, int smoothing, float floor_,
                                 const GateArgs &g, hipStream_t s)
{
    if (sv.C == 4)
        hipLaunchKernelGGL((k_append_fold<T, K, GATED, NORM, CH, U, R1, 4, BLK, CB>), dim3(heads), dim3(NT), 0, s, sv,
                           n, (const T *)q, (const T *)k, (const T *)v, alpha, beta, o, smoothing, floor_, g);
    else
        hipLaunchKernelGGL((k_append_fold<T, K, GATED, NORM, CH, U, R1, -1, BLK, CB>), dim3(heads), dim3(NT), 0, s,
                           sv, n, (const T *)q, (const T *)k, (const T *)v, alpha, beta, o, smoothing, floor_, g);
}

hipError_t launch_append_fold(const StateView &sv, int heads, int n, int bf16, const void *q, const void *k,
                              const void *v, const float *alpha, const float *beta, float *o, int smoothing,
                              float floor_, const GateArgs &g, hipStream_t s)
{
    // the (inputs, keys, gated, normalize) combinations of launch_append
    const bool kb = sv.key_bf16;
#define LQ_AF(T, K, G, N) launch_append_fold_t<T, K, G, N>(sv, heads, n, q, k, v, alpha, beta, o, smoothing, floor_, g, s)
#define LQ_AFB(T, CB)                                                                                               \
    launch_append_fold_t<T, T, false, false, false, float, false, false, CB>(sv, heads, n, q, k, v, alpha, beta, o, \
                                                                             smoothing, floor_, g, s)
    if (sv.cbits == 6) {
        if (!bf16)
            LQ_AFB(float, 6);
        else
            LQ_AFB(uint16_t, 6);
    } else if (sv.cbits == 4) {
        if (!bf16)
            LQ_AFB(float, 4);
        else
            LQ_AFB(uint16_t, 4);
    } else if (sv.blk) {
        if (!bf16)
            launch_append_fold_t<float, float, false, false, false, float, true, true>(sv, heads, n, q, k, v, alpha,
                                                                                     beta, o, smoothing, floor_, g, s);
        else
            launch_append_fold_t<uint16_t, uint16_t, false, false, false, float, true, true>(
                sv, heads, n, q, k, v, alpha, beta, o, smoothing, floor_, g, s);
    } else if (sv.r1) {
        if (!bf16)
            launch_append_fold_t<float, float, false, false, false, float, true>(sv, heads, n, q, k, v, alpha, beta, o,
                                                                               smoothing, floor_, g, s);
        else
            launch_append_fold_t<uint16_t, uint16_t, false, false, false, float, true>(
                sv, heads, n, q, k, v, alpha, beta, o, smoothing, floor_, g, s);
    } else if (sv.u_bf16) {
        if (!bf16)
            launch_append_fold_t<float, float, false, false, false, uint16_t>(sv, heads, n, q, k, v, alpha, beta, o,
                                                                            smoothing, floor_, g, s);
        else
            launch_append_fold_t<uint16_t, uint16_t, false, false, false, uint16_t>(
                sv, heads, n, q, k, v, alpha, beta, o, smoothing, floor_, g, s);
    } else if (sv.u_fp8) {
        if (!bf16)
            launch_append_fold_t<float, float, false, false, false, Fp8>(sv, heads, n, q, k, v, alpha, beta, o,
                                                                       smoothing, floor_, g, s);
        else
            launch_append_fold_t<uint16_t, uint16_t, false, false, false, Fp8>(sv, heads, n, q, k, v, alpha, beta,
                                                                             o, smoothing, floor_, g, s);
    } else if (sv.kda) {
        if (!bf16)
            launch_append_fold_t<float, float, false, false, true>(sv, heads, n, q, k, v, alpha, beta, o, smoothing,
                                                                 floor_, g, s);
        else
            launch_append_fold_t<uint16_t, uint16_t, false, false, true>(sv, heads, n, q, k, v, alpha, beta, o,
                                                                       smoothing, floor_, g, s);
    } else if (!g.gated) {
        if (!bf16)
            LQ_AF(float, float, false, false);
        else if (kb)
            LQ_AF(uint16_t, uint16_t, false, false);
        else
            LQ_AF(uint16_t, float, false, false);
    } else if (!bf16) {
        if (g.normalize)
            LQ_AF(float, float, true, true);
        else
            LQ_AF(float, float, true, false);
    } else if (kb) {
        LQ_AF(uint16_t, uint16_t, true, false);
    } else if (g.normalize) {
        LQ_AF(uint16_t, float, true, true);
    } else {
        LQ_AF(uint16_t, float, true, false);
    }
#undef LQ_AF
#undef LQ_AFB
    return hipGetLastError();
}

template <typename T, typename K, bool GATED, bool NORM, bool CH = false, typename U = float, bool R1 = false,
          bool BLK = false>
static void launch_step_t(const StateView &sv, int heads, int heads_per_req, const int *n_in, int *n_out,
                          const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                          float *o, int smoothing, float floor_, const GateArgs &g, hipStream_t s)
{
    if (sv.C == 4)
        hipLaunchKernelGGL((k_step<T, K, GATED, NORM, CH, U, R1, 4, BLK>), dim3(heads), dim3(NT), 0, s, sv,
                           heads_per_req, n_in, n_out, (const T *)q, (const T *)k, (const T *)v, alpha, beta, o,
                           smoothing, floor_, g);
    else
        hipLaunchKernelGGL((k_step<T, K, GATED, NORM, CH, U, R1, -1, BLK>), dim3(heads), dim3(NT), 0, s, sv,
                           heads_per_req, n_in, n_out, (const T *)q, (const T *)k, (const T *)v, alpha, beta, o,
                           smoothing, floor_, g);
}

hipError_t launch_step(const StateView &sv, int heads, int heads_per_req, const int *n_in, int *n_out, int bf16,
                       const void *q, const void *k, const void *v, const float *alpha, const float *beta, float *o,
                       int smoothing, float floor_, const GateArgs &g, hipStream_t s)
{
    // the variants of launch_append_fold
    const bool kb = sv.key_bf16;
#define LQ_ST(...) \
    launch_step_t<__VA_ARGS__>(sv, heads, heads_per_req, n_in, n_out, q, k, v, alpha, beta, o, smoothing, floor_, g, s)
    if (sv.blk) {
        if (!bf16)
            LQ_ST(float, float, false, false, false, float, true, true);
        else
            LQ_ST(uint16_t, uint16_t, false, false, false, float, true, true);
    } else if (sv.r1) {
        if (!bf16)
            LQ_ST(float, float, false, false, false, float, true);
        else
            LQ_ST(uint16_t, uint16_t, false, false, false, float, true);
    } else if (sv.u_bf16) {
        if (!bf16)
            LQ_ST(float, float, false, false, false, uint16_t);
        else
            LQ_ST(uint16_t, uint16_t, false, false, false, uint16_t);
    } else if (sv.u_fp8) {
        if (!bf16)
            LQ_ST(float, float, false, false, false, Fp8);
        else
            LQ_ST(uint16_t, uint16_t, false, false, false, Fp8);
    } else if (sv.kda) {
        if (!bf16)
            LQ_ST(float, float, false, false, true);
        else
            LQ_ST(uint16_t, uint16_t, false, false, true);
    } else if (!g.gated) {
        if (!bf16)
            LQ_ST(float, float, false, false);
        else if (kb)
            LQ_ST(uint16_t, uint16_t, false, false);
        else
            LQ_ST(uint16_t, float, false, false);
    } else if (!bf16) {
        if (g.normalize)
            LQ_ST(float, float, true, true);
        else
            LQ_ST(float, float, true, false);
    } else if (kb) {
        LQ_ST(uint16_t, uint16_t, true, false);
    } else if (g.normalize) {
        LQ_ST(uint16_t, float, true, true);
    } else {
        LQ_ST(uint16_t, float, true, false);
    }
#undef LQ_ST
    return hipGetLastError();
}

hipError_t launch_dequant(const StateView &sv, int heads, int n, int what, float *out, hipStream_t s)
{
#define LQ_DQ(K, CH, U, R1) hipLaunchKernelGGL((k_dequant<K, CH, U, R1>), dim3(heads), dim3(NT), 0, s, sv, n, what, out)
#define LQ_DQB(K, CB) \
    hipLaunchKernelGGL((k_dequant<K, false, float, false, CB>), dim3(heads), dim3(NT), 0, s, sv, n, what, out)
    if (sv.cbits == 6) {
        if (sv.key_bf16)
            LQ_DQB(uint16_t, 6);
        else
            LQ_DQB(float, 6);
    } else if (sv.cbits == 4) {
        if (sv.key_bf16)
            LQ_DQB(uint16_t, 4);
        else
            LQ_DQB(float, 4);
    } else if (sv.r1) {
        if (sv.key_bf16)
            LQ_DQ(uint16_t, false, float, true);
        else
            LQ_DQ(float, false, float, true);
    } else if (sv.u_bf16) {
        if (sv.key_bf16)
            LQ_DQ(uint16_t, false, uint16_t, false);
        else
            LQ_DQ(float, false, uint16_t, false);
    } else if (sv.u_fp8) {
        if (sv.key_bf16)
            LQ_DQ(uint16_t, false, Fp8, false);
        else
            LQ_DQ(float, false, Fp8, false);
    } else if (sv.kda) {
        if (sv.key_bf16)
            LQ_DQ(uint16_t, true, float, false);
        else
            LQ_DQ(float, true, float, false);
    } else if (sv.key_bf16) {
        LQ_DQ(uint16_t, false, float, false);
    } else {
        LQ_DQ(float, false, float, false);
    }
#undef LQ_DQ
#undef LQ_DQB
    return hipGetLastError();
}

}  // namespace leapq
