/*
 * LeapQuant per-window int8 recurrent state for Gated DeltaNet heads:
 * the ORACLE.  A plain, slow, single-threaded CPU statement of what the
 * decode path computes, one head at a time.
 *
 * This file is test infrastructure.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  The GPU library
 * shares no code, header, table or helper with it, and neither includes the
 * other.
 *
 * Sources (the method pages):
 *   [RN4]  "Recurrent-state quantization for linear attention: a first GPU
 *          kernel" (fastpathlabs.ai research note 4): Background (the order
 *          of one GDN token update), Why rounding the state is difficult
 *          (window of 16, records, fold, compensators, smoothing),
 *          What we built (append / fold split), Results.
 *   [LQ]   "LeapQuant: Efficient Linear Attention with Accurate Recurrent
 *          State Quantization" (paperlayer.ai summary of arXiv 2609.38166v1):
 *          abstract; 3.1 Preliminaries; 3.2 Per-window quantization;
 *          3.3 Compensator tokens; 3.4 Residual smoothing; App. A
 *          (general update, one rank-one record per GDN token); B.1
 *          (error only at window boundaries); B.2 (window unrolling and
 *          readout); B.3 (readout with a smoothed quantized residual);
 *          4.3 (1.19 bytes per element); 4.4 (window 16, four compensators).
 *
 * Arithmetic contract.  The pages fix the storage precisions (an 8-bit
 * residual, higher-precision records and compensators; fp32 for both here)
 * but not the arithmetic.  Because the int8 codes and the compensator choice
 * are integer decisions taken from fp32 values, the oracle computes in IEEE
 * binary32, round to nearest even, no flush of subnormals, no contraction
 * (a fused multiply-add appears only where fmaf() is written), correctly
 * rounded '/' and sqrtf, and a fixed summation order: the canonical
 * 128-term halving tree below.  Build with -ffp-contract=off and without
 * -ffast-math.
 *
 * State of one head (D = 128; rows are key coordinates, columns are value
 * coordinates, [LQ] 3.1):
 *   Q[r][c]   int8 residual codes (logical row-major order)
 *   rho[r]    fp32 per-row scale            sigma[c]  fp32 per-column smoothing
 *   idx[j]    compensator line, j < C: -1 unused, 0..127 row r, 128+c column c
 *   vec[j][]  fp32 copy of that line (128 values)
 *   n         records in the current window; gam[i], rk[i][], ru[i][] for
 *             i < n: cumulative decay since the window start, key, correction.
 *
 * Pins: every function here is pinned by the CPU tests (brute-force
 * recurrence in fp32 and fp64, closed-form special cases, exact scaling,
 * tree-automorphism equivariance, planted outliers, brute-force argmax,
 * textbook absmax int8, round-half-even fixtures, page figures).  The
 * compensator selection rule, the smoothing floor and the rounding mode are
 * readings of pages that leave them open; the tests fix them but no page
 * prints a worked fold to compare against.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define D 128

/* ------------------------------------------------------------------ */
/* Canonical sums                                                      */
/* ------------------------------------------------------------------ */

/* Sum of 128 terms by the canonical halving tree: level 0 adds term i and
 * term i+64 (i < 64); each further level adds partial i and partial i+h for
 * h = 32, 16, ..., 1.  The result is partial 0. */
float lqo_t128_sum(const float f[D])
{
    float s[64];
    for (int i = 0; i < 64; ++i) s[i] = f[i] + f[i + 64];
    for (int h = 32; h >= 1; h >>= 1)
        for (int i = 0; i < h; ++i) s[i] = s[i] + s[i + h];
    return s[0];
}

/* Dot product of two 128-vectors by the same tree; at level 0 the pair
 * (i, i+64) is formed with one fused multiply-add onto the rounded product
 * of the upper term. */
float lqo_t128_dot(const float a[D], const float b[D])
{
    float s[64];
    for (int i = 0; i < 64; ++i) s[i] = fmaf(a[i], b[i], a[i + 64] * b[i + 64]);
    for (int h = 32; h >= 1; h >>= 1)
        for (int i = 0; i < h; ++i) s[i] = s[i] + s[i + h];
    return s[0];
}

static float gamma_of(int n, const float *gam) { return n > 0 ? gam[n - 1] : 1.0f; }

/* ------------------------------------------------------------------ */
/* Dequantization ([LQ] B.3: scales apply to the residual only; the     */
/* compensator lines are added in full precision).                      */
/* ------------------------------------------------------------------ */

/* Residual in original coordinates: (code * rho_r) * sigma_c. */
void lqo_residual(const int8_t *Q, const float *rho, const float *sigma, float *out)
{
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c)
            out[r * D + c] = ((float)Q[r * D + c] * rho[r]) * sigma[c];
}

/* Adds scale * (compensator lines) to M, in compensator order.  A row token
 * r contributes its line to row r, a column token c to column c.  Extracted
 * lines were zero in the residual, so each entry receives at most one
 * nonzero term and these adds are exact. */
static void add_lines(float *M, int C, const int32_t *idx, const float *vec, float scale)
{
    for (int j = 0; j < C; ++j) {
        const float *v = vec + (size_t)j * D;
        if (idx[j] < 0) continue;
        if (idx[j] < D) {
            int r = idx[j];
            for (int c = 0; c < D; ++c) M[r * D + c] = M[r * D + c] + scale * v[c];
        } else {
            int c = idx[j] - D;
            for (int r = 0; r < D; ++r) M[r * D + c] = M[r * D + c] + scale * v[r];
        }
    }
}

/* Boundary state B = residual + compensator lines. */
void lqo_boundary(const int8_t *Q, const float *rho, const float *sigma, int C,
                  const int32_t *idx, const float *vec, float *out)
{
    lqo_residual(Q, rho, sigma, out);
    add_lines(out, C, idx, vec, 1.0f);
}

/* Current state after n records of the window ([LQ] B.2 unrolling; [RN4]
 * Why rounding: the fold applies the records):
 *   S = gamma_n * B + sum_i (gamma_n / gamma_i) k_i u_i^T.
 * Residual entries are formed as (code * (gamma_n * rho_r)) * sigma_c, the
 * compensator lines as gamma_n * line, then each record i = 0..n-1 in order
 * is applied to every entry with one fused multiply-add of
 * w_i[r] = (gamma_n / gamma_i) * k_i[r] and u_i[c]. */
static void add_rank1(float *M, int C, const float *ab, float g);

/* r1: the compensators are rank-one pairs (see the rank-one fit below). */
static void current_core(const int8_t *Q, const float *rho, const float *sigma, int C,
                         const int32_t *idx, const float *vec, int r1, int n, const float *gam,
                         const float *rk, const float *ru, float *out)
{
    float gn = gamma_of(n, gam);
    for (int r = 0; r < D; ++r) {
        float a = gn * rho[r];
        for (int c = 0; c < D; ++c) out[r * D + c] = ((float)Q[r * D + c] * a) * sigma[c];
    }
    if (r1)
        add_rank1(out, C, vec, gn);
    else
        add_lines(out, C, idx, vec, gn);
    for (int i = 0; i < n; ++i) {
        float ci = gn / gam[i];
        float w[D];
        for (int r = 0; r < D; ++r) w[r] = ci * rk[(size_t)i * D + r];
        for (int r = 0; r < D; ++r)
            for (int c = 0; c < D; ++c)
                out[r * D + c] = fmaf(w[r], ru[(size_t)i * D + c], out[r * D + c]);
    }
}

void lqo_current(const int8_t *Q, const float *rho, const float *sigma, int C,
                 const int32_t *idx, const float *vec, int n, const float *gam,
                 const float *rk, const float *ru, float *out)
{
    current_core(Q, rho, sigma, C, idx, vec, 0, n, gam, rk, ru, out);
}

/* ------------------------------------------------------------------ */
/* Quantization of a full fp32 matrix: compensator extraction, residual */
/* smoothing, per-row int8.  Used at init and at every fold.            */
/* ------------------------------------------------------------------ */

/* Largest row magnitude below which a row is stored as zeros: 127/M must
 * stay finite. */
#define LQO_TINY 0x1p-120f

/* R is consumed (extracted lines are zeroed in place). */
static void smooth_and_round(float *R, int smoothing, float sigma_floor, int8_t *Q, float *rho, float *sigma);

/* Greedy extraction of C compensator lines from R (zeroed in place). */
static void extract_lines(float *R, int C, int32_t *idx, float *vec)
{
    /* Compensator tokens ([LQ] 3.3; [RN4] Why rounding): greedy extraction
     * of whole rows or columns, largest energy first.  Energy of a line is
     * its canonical sum of squares.  Candidates are scanned rows 0..127 then
     * columns 0..127 and the first strict maximum wins; a line already taken
     * is not a candidate.  With no positive score left the slot is unused. */
    int taken[2 * D];
    memset(taken, 0, sizeof taken);
    for (int j = 0; j < C; ++j) {
        float score[2 * D];
        for (int r = 0; r < D; ++r) score[r] = lqo_t128_dot(R + r * D, R + r * D);
        for (int c = 0; c < D; ++c) {
            float col[D];
            for (int r = 0; r < D; ++r) col[r] = R[r * D + c];
            score[D + c] = lqo_t128_dot(col, col);
        }
        float best = 0.0f;
        int pick = -1;
        for (int cand = 0; cand < 2 * D; ++cand)
            if (!taken[cand] && score[cand] > best) { best = score[cand]; pick = cand; }
        float *v = vec + (size_t)j * D;
        idx[j] = pick;
        if (pick < 0) {
            for (int e = 0; e < D; ++e) v[e] = 0.0f;
            continue;
        }
        taken[pick] = 1;
        if (pick < D) {
            for (int c = 0; c < D; ++c) { v[c] = R[pick * D + c]; R[pick * D + c] = 0.0f; }
        } else {
            int c = pick - D;
            for (int r = 0; r < D; ++r) { v[r] = R[r * D + c]; R[r * D + c] = 0.0f; }
        }
    }
}

void lqo_quantize(float *R, int C, int smoothing, float sigma_floor,
                  int8_t *Q, float *rho, float *sigma, int32_t *idx, float *vec)
{
    extract_lines(R, C, idx, vec);
    smooth_and_round(R, smoothing, sigma_floor, Q, rho, sigma);
}

/* Smoothing and per-row int8 of the residual R (what remains after the
 * compensators), shared by both compensator fits. */
/* lv: the largest code; 127 for the int8 state, 31 or 7 for the 6- and
 * 4-bit options (symmetric codes -lv .. lv, scale absmax / lv). */
static void smooth_and_round_lv(float *R, int smoothing, float sigma_floor, float lv, int8_t *Q, float *rho,
                                float *sigma);

static void smooth_and_round(float *R, int smoothing, float sigma_floor, int8_t *Q, float *rho, float *sigma)
{
    smooth_and_round_lv(R, smoothing, sigma_floor, 127.0f, Q, rho, sigma);
}

static void smooth_and_round_lv(float *R, int smoothing, float sigma_floor, float lv, int8_t *Q, float *rho,
                                float *sigma)
{
    /* Residual smoothing ([LQ] 3.4): per value column, the square root of
     * the mean absolute value over the key rows, with a positive floor. */
    float inv_sigma[D];
    for (int c = 0; c < D; ++c) {
        float s = 1.0f;
        if (smoothing) {
            float col[D];
            for (int r = 0; r < D; ++r) col[r] = fabsf(R[r * D + c]);
            float m = lqo_t128_sum(col) * 0.0078125f;
            s = sqrtf(m);
            if (s < sigma_floor) s = sigma_floor;
        }
        sigma[c] = s;
        inv_sigma[c] = 1.0f / s;
    }

    /* Symmetric per-row codes (int8: lv = 127) with round half to even ([LQ] abstract: 8-bit
     * state; [RN4] Why rounding: rounded once per window).  A code is the
     * integer nearest to the exact product x * g, ties to even: one rounding
     * (the float64 product of two floats is exact). */
    for (int r = 0; r < D; ++r) {
        float x[D];
        float M = 0.0f;
        for (int c = 0; c < D; ++c) {
            x[c] = R[r * D + c] * inv_sigma[c];
            if (fabsf(x[c]) > M) M = fabsf(x[c]);
        }
        if (!(M >= LQO_TINY)) {
            rho[r] = 0.0f;
            for (int c = 0; c < D; ++c) Q[r * D + c] = 0;
            continue;
        }
        rho[r] = M / lv;
        float g = lv / M;
        for (int c = 0; c < D; ++c) {
            float y = (float)rint((double)x[c] * (double)g);
            if (y > lv) y = lv;
            if (y < -lv) y = -lv;
            Q[r * D + c] = (int8_t)y;
        }
    }
}

/* ------------------------------------------------------------------ */
/* The other smoothing axis (a study, CPU only).  "LeapQuant" 3.4      */
/* describes smoothing as a rescaling of the key rows whose inverse     */
/* restores the key coordinates; the path built here smooths per value  */
/* column with int8 scales per key row.  This variant exchanges the two */
/* axes: per key row, the square root of the row's mean absolute value  */
/* (floored) divides the row; the int8 scales are then per value column */
/* (absmax / 127, one rounding of the exact product, ties to even).     */
/* The compensators are extracted as in lqo_quantize.  On S it equals   */
/* lqo_quantize on the transpose of S, transposed (when no row ties a   */
/* column), which pins it.                                              */
/* ------------------------------------------------------------------ */
static void smooth_and_round_keyrow(float *R, int smoothing, float sigma_floor, int8_t *Q, float *rho_col,
                                    float *sigma_row)
{
    float inv_row[D];
    for (int r = 0; r < D; ++r) {
        float sr = 1.0f;
        if (smoothing) {
            float a[D];
            for (int c = 0; c < D; ++c) a[c] = fabsf(R[r * D + c]);
            sr = sqrtf(lqo_t128_sum(a) * (1.0f / 128.0f));
            if (sr < sigma_floor) sr = sigma_floor;
        }
        sigma_row[r] = sr;
        inv_row[r] = 1.0f / sr;
    }
    for (int c = 0; c < D; ++c) {
        float y[D];
        float Mc = 0.0f;
        for (int r = 0; r < D; ++r) {
            y[r] = R[r * D + c] * inv_row[r];
            if (fabsf(y[r]) > Mc) Mc = fabsf(y[r]);
        }
        if (!(Mc >= LQO_TINY)) {
            rho_col[c] = 0.0f;
            for (int r = 0; r < D; ++r) Q[r * D + c] = 0;
            continue;
        }
        rho_col[c] = Mc / 127.0f;
        float gc = 127.0f / Mc;
        for (int r = 0; r < D; ++r) {
            double z = rint((double)y[r] * (double)gc);
            if (z > 127.0) z = 127.0;
            if (z < -127.0) z = -127.0;
            Q[r * D + c] = (int8_t)z;
        }
    }
}

void lqo_quantize_keyrow(float *R, int C, int smoothing, float sigma_floor,
                         int8_t *Q, float *rho_col, float *sigma_row, int32_t *idx, float *vec)
{
    extract_lines(R, C, idx, vec);
    smooth_and_round_keyrow(R, smoothing, sigma_floor, Q, rho_col, sigma_row);
}

/* Boundary of the key-row variant: (code * rho_c) * sigma_r plus the lines. */
void lqo_boundary_keyrow(const int8_t *Q, const float *rho_col, const float *sigma_row, int C,
                         const int32_t *idx, const float *vec, float *out)
{
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) out[r * D + c] = ((float)Q[r * D + c] * rho_col[c]) * sigma_row[r];
    add_lines(out, C, idx, vec, 1.0f);
}

/* Initial quantization of a caller's fp32 state: the fold without records. */
void lqo_init(const float *S0, int C, int smoothing, float sigma_floor,
              int8_t *Q, float *rho, float *sigma, int32_t *idx, float *vec)
{
    float R[D * D];
    memcpy(R, S0, sizeof R);
    lqo_quantize(R, C, smoothing, sigma_floor, Q, rho, sigma, idx, vec);
}

/* Fold ([RN4] What we built: rebuild, select compensators, rescale, round,
 * empty the buffer; [LQ] B.3: rebuild in original coordinates before new
 * factors and scales).  Overwrites the boundary state; the caller sets n=0. */
void lqo_fold(int8_t *Q, float *rho, float *sigma, int C, int32_t *idx, float *vec,
              int n, const float *gam, const float *rk, const float *ru,
              int smoothing, float sigma_floor)
{
    float R[D * D];
    lqo_current(Q, rho, sigma, C, idx, vec, n, gam, rk, ru, R);
    lqo_quantize(R, C, smoothing, sigma_floor, Q, rho, sigma, idx, vec);
}

/* ------------------------------------------------------------------ */
/* 6- and 4-bit residual states (an option; [LQ] 4.2 reports LeapQuant  */
/* at 6 and 4 bits beside 8): the same fold with symmetric codes of     */
/* -31 .. 31 or -7 .. 7 (scale absmax / 31 or / 7).  bits = 8 is the    */
/* int8 state.  The codes keep their logical int8 array here; only the  */
/* GPU layout packs them.                                               */
/* ------------------------------------------------------------------ */
static float levels_of(int bits) { return bits == 4 ? 7.0f : bits == 6 ? 31.0f : 127.0f; }

void lqo_init_bits(const float *S0, int C, int smoothing, float sigma_floor, int bits,
                   int8_t *Q, float *rho, float *sigma, int32_t *idx, float *vec)
{
    float R[D * D];
    memcpy(R, S0, sizeof R);
    extract_lines(R, C, idx, vec);
    smooth_and_round_lv(R, smoothing, sigma_floor, levels_of(bits), Q, rho, sigma);
}

void lqo_fold_bits(int8_t *Q, float *rho, float *sigma, int C, int32_t *idx, float *vec,
                   int n, const float *gam, const float *rk, const float *ru,
                   int smoothing, float sigma_floor, int bits)
{
    float R[D * D];
    lqo_current(Q, rho, sigma, C, idx, vec, n, gam, rk, ru, R);
    extract_lines(R, C, idx, vec);
    smooth_and_round_lv(R, smoothing, sigma_floor, levels_of(bits), Q, rho, sigma);
}

/* ------------------------------------------------------------------ */
/* Rank-one compensators fitted by power sweeps (a fold option): [RN4]   */
/* Where the time goes describes four compensators found one at a time  */
/* with eight sweeps each, starting from the longest row of the matrix; */
/* [LQ] 3.3 keeps compensators as rank-one updates.  Compensator j is   */
/* the pair (a_j, b_j) with a_j of unit norm; it sets aside a_j b_j^T.  */
/* The pair sits in the line storage as [a_j | b_j] (2 x 128 values).  */
/* ------------------------------------------------------------------ */

#define LQO_SWEEPS 8

/* Fits C rank-one compensators to R in order and deflates R by each:
 *   r* = the row of largest canonical energy (lowest index on ties; none
 *        if no energy is positive: the pair is zero and idx_j = -1)
 *   b  = row r*;  then LQO_SWEEPS times:
 *        a_r = T(R[r,:] . b),  a = a * (1 / sqrt(T(a . a))),  b_c = T(R[:,c] . a)
 *   R[r][c] = fma(-a_r, b_c, R[r][c]);  idx_j = r*. */
static void fit_rank1(float *R, int C, int32_t *idx, float *ab)
{
    for (int j = 0; j < C; ++j) {
        float *a = ab + (size_t)j * 2 * D, *b = a + D;
        float best = 0.0f;
        int pick = -1;
        for (int r = 0; r < D; ++r) {
            float e = lqo_t128_dot(R + r * D, R + r * D);
            if (e > best) { best = e; pick = r; }
        }
        idx[j] = pick;
        for (int e = 0; e < D; ++e) { a[e] = 0.0f; b[e] = 0.0f; }
        if (pick < 0) continue;
        for (int c = 0; c < D; ++c) b[c] = R[pick * D + c];
        for (int s = 0; s < LQO_SWEEPS; ++s) {
            for (int r = 0; r < D; ++r) a[r] = lqo_t128_dot(R + r * D, b);
            float na2 = lqo_t128_dot(a, a);
            if (!(na2 > 0.0f)) {
                for (int e = 0; e < D; ++e) { a[e] = 0.0f; b[e] = 0.0f; }
                break;
            }
            float inv = 1.0f / sqrtf(na2);
            for (int r = 0; r < D; ++r) a[r] = a[r] * inv;
            for (int c = 0; c < D; ++c) {
                float col[D];
                for (int r = 0; r < D; ++r) col[r] = R[r * D + c];
                b[c] = lqo_t128_dot(col, a);
            }
        }
        for (int r = 0; r < D; ++r)
            for (int c = 0; c < D; ++c) R[r * D + c] = fmaf(-a[r], b[c], R[r * D + c]);
    }
}

/* Quantization with rank-one compensators: the fit, then the same smoothing
 * and rounding as with lines.  ab: [C][2][128]. */
void lqo_quantize_r1(float *R, int C, int smoothing, float sigma_floor,
                     int8_t *Q, float *rho, float *sigma, int32_t *idx, float *ab)
{
    fit_rank1(R, C, idx, ab);
    smooth_and_round(R, smoothing, sigma_floor, Q, rho, sigma);
}

/* Adds the compensators scaled by g: entry (r, c) gets fma(g a_j[r], b_j[c], .)
 * for j in order. */
static void add_rank1(float *M, int C, const float *ab, float g)
{
    for (int j = 0; j < C; ++j) {
        const float *a = ab + (size_t)j * 2 * D, *b = a + D;
        for (int r = 0; r < D; ++r) {
            float w = g * a[r];
            for (int c = 0; c < D; ++c) M[r * D + c] = fmaf(w, b[c], M[r * D + c]);
        }
    }
}

/* Current state with rank-one compensators: (code * (gamma_n rho_r)) *
 * sigma_c, then the compensators scaled by gamma_n, then the records. */
void lqo_current_r1(const int8_t *Q, const float *rho, const float *sigma, int C, const float *ab,
                    int n, const float *gam, const float *rk, const float *ru, float *out)
{
    current_core(Q, rho, sigma, C, NULL, ab, 1, n, gam, rk, ru, out);
}

void lqo_init_r1(const float *S0, int C, int smoothing, float sigma_floor,
                 int8_t *Q, float *rho, float *sigma, int32_t *idx, float *ab)
{
    float R[D * D];
    memcpy(R, S0, sizeof R);
    lqo_quantize_r1(R, C, smoothing, sigma_floor, Q, rho, sigma, idx, ab);
}

void lqo_fold_r1(int8_t *Q, float *rho, float *sigma, int C, int32_t *idx, float *ab,
                 int n, const float *gam, const float *rk, const float *ru, int smoothing, float sigma_floor)
{
    float R[D * D];
    lqo_current_r1(Q, rho, sigma, C, ab, n, gam, rk, ru, R);
    lqo_quantize_r1(R, C, smoothing, sigma_floor, Q, rho, sigma, idx, ab);
}

/* ------------------------------------------------------------------ */
/* Block fit of the compensators (a fold option): [RN4] Redesign plans   */
/* to fit the compensators together as one block, starting from the     */
/* previous window's compensators.  Read as subspace (block power)      */
/* iteration on the key side with modified Gram-Schmidt.  The pairs are */
/* stored and read exactly as the rank-one pairs above ([a | b], the    */
/* boundary is the residual plus sum_j a_j b_j^T); idx_j is j for a     */
/* live pair and -1 for an unused one.                                   */
/* ------------------------------------------------------------------ */

#define LQO_BLOCK_SWEEPS 2       /* per fold, warm-started */
#define LQO_BLOCK_SWEEPS_INIT 8  /* at init, from the longest rows */

/* Modified Gram-Schmidt over the slots in order: each earlier live vector
 * is projected out, y = fma(-T(a_i . y), a_i, y) per element; then a zero
 * norm T(y . y) leaves the slot unused (y = 0), otherwise y is scaled by
 * 1 / sqrt(T(y . y)). */
static void block_mgs(float A[][D], int C, int *live)
{
    for (int j = 0; j < C; ++j) {
        for (int i = 0; i < j; ++i) {
            if (!live[i]) continue;
            float d = lqo_t128_dot(A[i], A[j]);
            for (int r = 0; r < D; ++r) A[j][r] = fmaf(-d, A[i][r], A[j][r]);
        }
        float n2 = lqo_t128_dot(A[j], A[j]);
        live[j] = n2 > 0.0f;
        if (!live[j]) {
            for (int r = 0; r < D; ++r) A[j][r] = 0.0f;
            continue;
        }
        float inv = 1.0f / sqrtf(n2);
        for (int r = 0; r < D; ++r) A[j][r] = A[j][r] * inv;
    }
}

/* z[c] = T(R[:, c] . a) for every column. */
static void cols_dot(const float *R, const float *a, float *z)
{
    for (int c = 0; c < D; ++c) {
        float col[D];
        for (int r = 0; r < D; ++r) col[r] = R[r * D + c];
        z[c] = lqo_t128_dot(col, a);
    }
}

/* Fits C pairs to R and deflates R by them.
 *   start: with warm, a live pair j (idx_j >= 0) starts from its stored a_j;
 *          every other slot, in slot order, starts from the unit vector of
 *          the next row by canonical energy (largest first, lowest index on
 *          ties, rows of zero energy never), or from zero if none is left;
 *          then A = MGS(start).
 *   sweeps times: z_j = R^T a_j;  y_j[r] = T(R[r, :] . z_j);  A = MGS(Y).
 *   b_j = R^T a_j;  idx_j = j (or -1 if unused);
 *   R[r][c] = fma(-a_j[r], b_j[c], R[r][c]) for j in order. */
void lqo_fit_block(float *R, int C, int32_t *idx, float *ab, int warm, int sweeps)
{
    float A[8][D], Z[D];
    int live[8];
    float e[D];
    int used[D];
    for (int r = 0; r < D; ++r) {
        e[r] = lqo_t128_dot(R + r * D, R + r * D);
        used[r] = 0;
    }
    for (int j = 0; j < C; ++j) {
        if (warm && idx[j] >= 0) {
            for (int r = 0; r < D; ++r) A[j][r] = ab[(size_t)j * 2 * D + r];
            continue;
        }
        float best = 0.0f;
        int pick = -1;
        for (int r = 0; r < D; ++r)
            if (!used[r] && e[r] > best) { best = e[r]; pick = r; }
        for (int r = 0; r < D; ++r) A[j][r] = 0.0f;
        if (pick >= 0) {
            A[j][pick] = 1.0f;
            used[pick] = 1;
        }
    }
    block_mgs(A, C, live);
    for (int s = 0; s < sweeps; ++s) {
        for (int j = 0; j < C; ++j) {
            cols_dot(R, A[j], Z);
            for (int r = 0; r < D; ++r) A[j][r] = lqo_t128_dot(R + r * D, Z);
        }
        block_mgs(A, C, live);
    }
    for (int j = 0; j < C; ++j) {
        float *a = ab + (size_t)j * 2 * D, *b = a + D;
        for (int r = 0; r < D; ++r) a[r] = A[j][r];
        cols_dot(R, A[j], b);
        idx[j] = live[j] ? j : -1;
    }
    for (int j = 0; j < C; ++j) {
        const float *a = ab + (size_t)j * 2 * D, *b = a + D;
        for (int r = 0; r < D; ++r)
            for (int c = 0; c < D; ++c) R[r * D + c] = fmaf(-a[r], b[c], R[r * D + c]);
    }
}

/* Quantization with a block fit: the fit, then smoothing and rounding. */
void lqo_quantize_block(float *R, int C, int smoothing, float sigma_floor, int warm,
                        int8_t *Q, float *rho, float *sigma, int32_t *idx, float *ab)
{
    lqo_fit_block(R, C, idx, ab, warm, warm ? LQO_BLOCK_SWEEPS : LQO_BLOCK_SWEEPS_INIT);
    smooth_and_round(R, smoothing, sigma_floor, Q, rho, sigma);
}

void lqo_init_block(const float *S0, int C, int smoothing, float sigma_floor,
                    int8_t *Q, float *rho, float *sigma, int32_t *idx, float *ab)
{
    float R[D * D];
    memcpy(R, S0, sizeof R);
    lqo_quantize_block(R, C, smoothing, sigma_floor, 0, Q, rho, sigma, idx, ab);
}

/* Fold with a block fit: the current state (as with rank-one pairs), then
 * the fit warm-started from the window's own pairs. */
void lqo_fold_block(int8_t *Q, float *rho, float *sigma, int C, int32_t *idx, float *ab,
                    int n, const float *gam, const float *rk, const float *ru, int smoothing, float sigma_floor)
{
    float R[D * D];
    lqo_current_r1(Q, rho, sigma, C, ab, n, gam, rk, ru, R);
    lqo_quantize_block(R, C, smoothing, sigma_floor, 1, Q, rho, sigma, idx, ab);
}

/* ------------------------------------------------------------------ */
/* Append: one decode token against the fixed boundary plus the records */
/* ------------------------------------------------------------------ */

/* Read of the boundary with key x ([LQ] B.3): the residual scales act on
 * the residual's read only, sigma_c * sum_r (x_r * rho_r) * code[r][c];
 * each compensator then adds its read as a token: a row token r adds
 * x_r * line, a column token c adds (line . x) to column c. */
static void boundary_read(const int8_t *Q, const float *rho, const float *sigma, int C,
                          const int32_t *idx, const float *vec, const float *x, float *out);

/* The read with rank-one compensators: the residual's read as above, then
 * for each compensator in order (a_j . x) b_j, one fused multiply-add per
 * column. */
static void boundary_read_r1(const int8_t *Q, const float *rho, const float *sigma, int C, const float *ab,
                             const float *x, float *out)
{
    boundary_read(Q, rho, sigma, 0, NULL, NULL, x, out);
    for (int j = 0; j < C; ++j) {
        const float *a = ab + (size_t)j * 2 * D, *b = a + D;
        float d = lqo_t128_dot(a, x);
        for (int c = 0; c < D; ++c) out[c] = fmaf(d, b[c], out[c]);
    }
}

static void boundary_read(const int8_t *Q, const float *rho, const float *sigma, int C,
                          const int32_t *idx, const float *vec, const float *x, float *out)
{
    float w[D];
    for (int r = 0; r < D; ++r) w[r] = x[r] * rho[r];
    for (int c = 0; c < D; ++c) {
        float col[D];
        for (int r = 0; r < D; ++r) col[r] = (float)Q[r * D + c];
        out[c] = sigma[c] * lqo_t128_dot(w, col);
    }
    for (int j = 0; j < C; ++j) {
        const float *v = vec + (size_t)j * D;
        if (idx[j] < 0) continue;
        if (idx[j] < D) {
            float xr = x[idx[j]];
            for (int c = 0; c < D; ++c) out[c] = fmaf(xr, v[c], out[c]);
        } else {
            int c = idx[j] - D;
            out[c] = out[c] + lqo_t128_dot(v, x);
        }
    }
}

/* One token ([RN4] Background: decay, read with the key, correction,
 * rank-one write, read the output; [LQ] App. A: one record per GDN token;
 * [LQ] B.2: reads never form the dense state).  With n records present
 * (n < W), token t = n+1:
 *   gamma_t = gamma_n * alpha,   c_i = gamma_t / gamma_i
 *   r   = gamma_t * B^T k + sum_i (c_i * (k_i . k)) u_i     (read of alpha*S_{t-1})
 *   u_t = beta * (v - r)
 *   o   = gamma_t * B^T q + sum_i (c_i * (k_i . q)) u_i + (k . q) u_t  (read of S_t)
 * and the record (gamma_t, k, u_t) is stored at slot n. */
static void append_core(const int8_t *Q, const float *rho, const float *sigma, int C,
                        const int32_t *idx, const float *vec, int r1, int n, float *gam, float *rk,
                        float *ru, const float *q, const float *k, const float *v, float alpha,
                        float beta, float *o)
{
    float gt = gamma_of(n, gam) * alpha;
    float bk[D], bq[D], u[D];
    if (r1) {
        boundary_read_r1(Q, rho, sigma, C, vec, k, bk);
        boundary_read_r1(Q, rho, sigma, C, vec, q, bq);
    } else {
        boundary_read(Q, rho, sigma, C, idx, vec, k, bk);
        boundary_read(Q, rho, sigma, C, idx, vec, q, bq);
    }

    float r[D];
    for (int c = 0; c < D; ++c) { r[c] = gt * bk[c]; o[c] = gt * bq[c]; }
    for (int i = 0; i < n; ++i) {
        float ci = gt / gam[i];
        const float *ki = rk + (size_t)i * D, *ui = ru + (size_t)i * D;
        float ak = ci * lqo_t128_dot(ki, k);
        float aq = ci * lqo_t128_dot(ki, q);
        for (int c = 0; c < D; ++c) {
            r[c] = fmaf(ak, ui[c], r[c]);
            o[c] = fmaf(aq, ui[c], o[c]);
        }
    }
    for (int c = 0; c < D; ++c) u[c] = beta * (v[c] - r[c]);
    float kq = lqo_t128_dot(k, q);
    for (int c = 0; c < D; ++c) o[c] = fmaf(kq, u[c], o[c]);

    gam[n] = gt;
    memcpy(rk + (size_t)n * D, k, D * sizeof(float));
    memcpy(ru + (size_t)n * D, u, D * sizeof(float));
}

void lqo_append(const int8_t *Q, const float *rho, const float *sigma, int C,
                const int32_t *idx, const float *vec, int n, float *gam, float *rk,
                float *ru, const float *q, const float *k, const float *v, float alpha,
                float beta, float *o)
{
    append_core(Q, rho, sigma, C, idx, vec, 0, n, gam, rk, ru, q, k, v, alpha, beta, o);
}

/* The append with rank-one compensators (ab: [C][2][128] in the line
 * storage); everything else as lqo_append. */
void lqo_append_r1(const int8_t *Q, const float *rho, const float *sigma, int C,
                   const int32_t *idx, const float *ab, int n, float *gam, float *rk,
                   float *ru, const float *q, const float *k, const float *v, float alpha,
                   float beta, float *o)
{
    append_core(Q, rho, sigma, C, idx, ab, 1, n, gam, rk, ru, q, k, v, alpha, beta, o);
}

/* ------------------------------------------------------------------ */
/* Per-channel decay (KDA): [LQ] App. A writes the general update with   */
/* a diagonal decay D_t = Diag(alpha_t), alpha_t a d_k-vector for Kimi   */
/* Delta Attention, and one rank-one record per token as for GDN; [LQ]   */
/* B.2: cumulative diagonal decays are kept incrementally.  The state    */
/* rows are key coordinates, so the decay scales rows.  Records hold the */
/* cumulative decay as a vector, gam[i][r].                              */
/* ------------------------------------------------------------------ */

/* The cumulative decay after n records (all ones at n = 0) into g. */
static void gamma_vec_of(int n, const float *gam, float *g)
{
    for (int r = 0; r < D; ++r) g[r] = n > 0 ? gam[(size_t)(n - 1) * D + r] : 1.0f;
}

/* Compensator lines scaled per row: entry (r, c) of a line receives
 * g[r] * (its value). */
static void add_lines_rows(float *M, int C, const int32_t *idx, const float *vec, const float *g)
{
    for (int j = 0; j < C; ++j) {
        const float *v = vec + (size_t)j * D;
        if (idx[j] < 0) continue;
        if (idx[j] < D) {
            int r = idx[j];
            for (int c = 0; c < D; ++c) M[r * D + c] = M[r * D + c] + g[r] * v[c];
        } else {
            int c = idx[j] - D;
            for (int r = 0; r < D; ++r) M[r * D + c] = M[r * D + c] + g[r] * v[r];
        }
    }
}

/* Current state after n records with per-row cumulative decays:
 *   S = Diag(gamma_n) B + sum_i Diag(gamma_n / gamma_i) k_i u_i^T,
 * formed as for lqo_current with gamma_n[r] in place of the scalar:
 * (code * (gamma_n[r] * rho_r)) * sigma_c, lines gamma_n[r] * line, then
 * record i in order by fma((gamma_n[r] / gamma_i[r]) * k_i[r], u_i[c], S). */
void lqo_current_kda(const int8_t *Q, const float *rho, const float *sigma, int C,
                     const int32_t *idx, const float *vec, int n, const float *gam,
                     const float *rk, const float *ru, float *out)
{
    float gn[D];
    gamma_vec_of(n, gam, gn);
    for (int r = 0; r < D; ++r) {
        float a = gn[r] * rho[r];
        for (int c = 0; c < D; ++c) out[r * D + c] = ((float)Q[r * D + c] * a) * sigma[c];
    }
    add_lines_rows(out, C, idx, vec, gn);
    for (int i = 0; i < n; ++i) {
        float w[D];
        for (int r = 0; r < D; ++r) w[r] = (gn[r] / gam[(size_t)i * D + r]) * rk[(size_t)i * D + r];
        for (int r = 0; r < D; ++r)
            for (int c = 0; c < D; ++c)
                out[r * D + c] = fmaf(w[r], ru[(size_t)i * D + c], out[r * D + c]);
    }
}

/* Fold with per-channel decays: rebuild (lqo_current_kda), then the same
 * quantization as every fold.  The caller sets n = 0. */
void lqo_fold_kda(int8_t *Q, float *rho, float *sigma, int C, int32_t *idx, float *vec,
                  int n, const float *gam, const float *rk, const float *ru,
                  int smoothing, float sigma_floor)
{
    float R[D * D];
    lqo_current_kda(Q, rho, sigma, C, idx, vec, n, gam, rk, ru, R);
    lqo_quantize(R, C, smoothing, sigma_floor, Q, rho, sigma, idx, vec);
}

/* One token with per-channel decay alpha[r] (n records present, n < W):
 *   gamma_t[r] = gamma_n[r] * alpha[r],  x = gamma_t (.) k,  y = gamma_t (.) q
 *   w_i[r] = (gamma_t[r] / gamma_i[r]) * k_i[r]
 *   r   = B^T x + sum_i (w_i . k) u_i            (read of Diag(alpha) S_{t-1})
 *   u_t = beta * (v - r)
 *   o   = B^T y + sum_i (w_i . q) u_i + (k . q) u_t
 * with the boundary reads of lqo_append (residual scales on the residual
 * only, compensators as tokens) and the record (gamma_t, k, u_t) at slot n. */
void lqo_append_kda(const int8_t *Q, const float *rho, const float *sigma, int C,
                    const int32_t *idx, const float *vec, int n, float *gam, float *rk,
                    float *ru, const float *q, const float *k, const float *v, const float *alpha,
                    float beta, float *o)
{
    float gp[D], gt[D], x[D], y[D], r[D], u[D];
    gamma_vec_of(n, gam, gp);
    for (int e = 0; e < D; ++e) {
        gt[e] = gp[e] * alpha[e];
        x[e] = gt[e] * k[e];
        y[e] = gt[e] * q[e];
    }
    boundary_read(Q, rho, sigma, C, idx, vec, x, r);
    boundary_read(Q, rho, sigma, C, idx, vec, y, o);
    for (int i = 0; i < n; ++i) {
        const float *ki = rk + (size_t)i * D, *ui = ru + (size_t)i * D, *gi = gam + (size_t)i * D;
        float w[D];
        for (int e = 0; e < D; ++e) w[e] = (gt[e] / gi[e]) * ki[e];
        float ak = lqo_t128_dot(w, k);
        float aq = lqo_t128_dot(w, q);
        for (int c = 0; c < D; ++c) {
            r[c] = fmaf(ak, ui[c], r[c]);
            o[c] = fmaf(aq, ui[c], o[c]);
        }
    }
    for (int cc = 0; cc < D; ++cc) u[cc] = beta * (v[cc] - r[cc]);
    float kq = lqo_t128_dot(k, q);
    for (int cc = 0; cc < D; ++cc) o[cc] = fmaf(kq, u[cc], o[cc]);

    memcpy(gam + (size_t)n * D, gt, D * sizeof(float));
    memcpy(rk + (size_t)n * D, k, D * sizeof(float));
    memcpy(ru + (size_t)n * D, u, D * sizeof(float));
}

/* One KDA token on a dense fp32 state: S = Diag(alpha) S; r = S^T k;
 * u = beta (v - r); S += k u^T; o = S^T q.  Plain sequential sums. */
void lqo_kda_step_f32(float *S, const float *q, const float *k, const float *v,
                      const float *alpha, float beta, float *u_out, float *o)
{
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) S[r * D + c] = alpha[r] * S[r * D + c];
    float u[D];
    for (int c = 0; c < D; ++c) {
        float rc = 0.0f;
        for (int r = 0; r < D; ++r) rc = fmaf(S[r * D + c], k[r], rc);
        u[c] = beta * (v[c] - rc);
    }
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) S[r * D + c] = fmaf(k[r], u[c], S[r * D + c]);
    for (int c = 0; c < D; ++c) {
        float oc = 0.0f;
        for (int rr = 0; rr < D; ++rr) oc = fmaf(S[rr * D + c], q[rr], oc);
        o[c] = oc;
    }
    if (u_out) memcpy(u_out, u, sizeof u);
}

/* ------------------------------------------------------------------ */
/* Gate arithmetic: the per-token step in front of the path ([RN4]       */
/* Results: the column "with gate arithmetic").  The pages name the step */
/* but print no formula; these are the Gated DeltaNet layer's gates (the */
/* model family of [LQ] 3.1 and [RN4] Background).  Parity unpinned      */
/* against the pages: the tests pin them by closed forms instead.        */
/* ------------------------------------------------------------------ */

/* Decay and step size of one head and token from the raw projections a, b
 * and the head's parameters A_log, dt_bias:
 *   alpha = exp(-exp(A_log) * softplus(a + dt_bias)),  beta = 1 / (1 + exp(-b)),
 * softplus(x) = max(x, 0) + log1p(exp(-|x|)).  Evaluated in binary64 from
 * the fp32 arguments and rounded once to fp32, so that two correct libm's
 * agree on the fp32 result except where the binary64 value lies within a
 * few units of its last place from an fp32 rounding boundary. */
void lqo_gate(float a, float b, float A_log, float dt_bias, float *alpha, float *beta)
{
    double x = (double)a + (double)dt_bias;
    double sp = fmax(x, 0.0) + log1p(exp(-fabs(x)));
    *alpha = (float)exp(-exp((double)A_log) * sp);
    *beta = (float)(1.0 / (1.0 + exp(-(double)b)));
}

/* L2 normalization of a 128-vector in fp32 with a scale:
 *   s = T128(x . x),  inv = 1 / sqrt(s + eps),  out_r = (x_r * inv) * scale. */
void lqo_l2norm(const float *x, float eps, float scale, float *out)
{
    float s = lqo_t128_dot(x, x);
    float inv = 1.0f / sqrtf(s + eps);
    for (int r = 0; r < D; ++r) out[r] = (x[r] * inv) * scale;
}

/* ------------------------------------------------------------------ */
/* Dense per-token GDN recurrences: the brute-force checker of the       */
/* windowed path and the unquantized quality references.                */
/* ------------------------------------------------------------------ */

/* One GDN token on a dense fp32 state ([RN4] Background order; [LQ] App. A
 * with D_t = alpha I and b_t = beta): S = alpha S; r = S^T k;
 * u = beta (v - r); S += k u^T; o = S^T q.  Plain sequential sums. */
void lqo_gdn_step_f32(float *S, const float *q, const float *k, const float *v,
                      float alpha, float beta, float *u_out, float *o)
{
    for (int e = 0; e < D * D; ++e) S[e] = alpha * S[e];
    float u[D];
    for (int c = 0; c < D; ++c) {
        float rc = 0.0f;
        for (int r = 0; r < D; ++r) rc = fmaf(S[r * D + c], k[r], rc);
        u[c] = beta * (v[c] - rc);
    }
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) S[r * D + c] = fmaf(k[r], u[c], S[r * D + c]);
    for (int c = 0; c < D; ++c) {
        float oc = 0.0f;
        for (int r = 0; r < D; ++r) oc = fmaf(S[r * D + c], q[r], oc);
        o[c] = oc;
    }
    if (u_out) memcpy(u_out, u, sizeof u);
}

/* The same step in fp64, to attribute a disagreement to conditioning. */
void lqo_gdn_step_f64(double *S, const double *q, const double *k, const double *v,
                      double alpha, double beta, double *u_out, double *o)
{
    for (int e = 0; e < D * D; ++e) S[e] = alpha * S[e];
    double u[D];
    for (int c = 0; c < D; ++c) {
        double rc = 0.0;
        for (int r = 0; r < D; ++r) rc += S[r * D + c] * k[r];
        u[c] = beta * (v[c] - rc);
    }
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) S[r * D + c] += k[r] * u[c];
    for (int c = 0; c < D; ++c) {
        double oc = 0.0;
        for (int r = 0; r < D; ++r) oc += S[r * D + c] * q[r];
        o[c] = oc;
    }
    if (u_out) memcpy(u_out, u, sizeof u);
}

/* bf16 helpers: widening is exact; narrowing rounds to nearest even. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

uint16_t lqo_f32_to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x007fffffu)) return (uint16_t)((b >> 16) | 0x40);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7fffu + lsb;
    return (uint16_t)(b >> 16);
}

/* bf16 record corrections (a lower-precision record option: [LQ] keeps
 * records in higher precision than the state, [RN4] Why rounding the state
 * is difficult; storing them narrower trades record traffic for error):
 * rounds n values to bf16, nearest even, in place (the widened values). */
void lqo_round_bf16(float *x, int n)
{
    for (int e = 0; e < n; ++e) x[e] = bf16_to_f32(lqo_f32_to_bf16(x[e]));
}

/* ------------------------------------------------------------------ */
/* fp8 record corrections (an option; [RN4] Why rounding the state is   */
/* difficult keeps the records in higher precision, [LQ] 4.4 notes that */
/* record traffic grows with the window: a narrower record trades the   */
/* two).  Format: OCP 8-bit floating point E4M3 (sign, 4 exponent bits  */
/* with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals  */
/* m * 2^-9; the largest finite value is 1.75 * 2^8 = 448; no infinity). */
/* A record's 128 corrections form 4 groups, value columns c with c % 4 */
/* = j; group j is stored as E4M3 codes of u_c / s_j, where s_j is the  */
/* smallest power of two not below 2^-126 with max_c |u_c| <= 448 s_j,  */
/* rounded to nearest, ties to even.  The stored correction is         */
/* decode(code) * s_j (exact).                                          */
/* ------------------------------------------------------------------ */

/* The E4M3 code of x, |x| <= 448, rounded to nearest, ties to even. */
uint8_t lqo_f32_to_e4m3(float x)
{
    double a = fabs((double)x);
    unsigned sign = signbit(x) ? 0x80u : 0u;
    unsigned mag;
    if (a >= 0x1p-6) {
        int e;
        frexp(a, &e);                      /* a = f 2^e, f in [0.5, 1) */
        int E = e - 1;                     /* a = q 2^E, q in [1, 2) */
        double q = ldexp(a, -E);
        /* a mantissa that rounds up to 8 carries into the exponent field */
        mag = (unsigned)((E + 7) * 8) + (unsigned)rint((q - 1.0) * 8.0);
    } else {
        mag = (unsigned)rint(a * 512.0);   /* subnormal: a multiple of 2^-9 (8 carries to 2^-6) */
    }
    return (uint8_t)(sign | mag);
}

float lqo_e4m3_to_f32(uint8_t c)
{
    int E = (c >> 3) & 15, m = c & 7;
    double v = E == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    return (float)((c & 0x80) ? -v : v);
}

/* In place: a record correction u[128] (value-column order) replaced by
 * its stored fp8 value. */
void lqo_round_fp8_record(float *u)
{
    for (int j = 0; j < 4; ++j) {
        float M = 0.0f;
        for (int c = j; c < D; c += 4)
            if (fabsf(u[c]) > M) M = fabsf(u[c]);
        double s = 0x1p-126;
        while ((double)M > 448.0 * s) s *= 2.0;
        float sf = (float)s, inv = 1.0f / sf;
        for (int c = j; c < D; c += 4) u[c] = lqo_e4m3_to_f32(lqo_f32_to_e4m3(u[c] * inv)) * sf;
    }
}

/* Per-token bf16 state ([RN4] Why rounding: a bf16 state rounded at every
 * token; [LQ] 4.2/4.4 per-step baselines): widen, take the fp32 step, keep
 * the output of the fp32 state, store the state rounded to bf16. */
void lqo_gdn_step_bf16(uint16_t *Sb, const float *q, const float *k, const float *v,
                       float alpha, float beta, float *u_out, float *o)
{
    float S[D * D];
    for (int e = 0; e < D * D; ++e) S[e] = bf16_to_f32(Sb[e]);
    lqo_gdn_step_f32(S, q, k, v, alpha, beta, u_out, o);
    for (int e = 0; e < D * D; ++e) Sb[e] = lqo_f32_to_bf16(S[e]);
}

int lqo_dim(void) { return D; }
