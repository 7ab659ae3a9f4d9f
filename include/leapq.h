/*
 * leapq.h - C ABI of the LeapQuant per-window int8 recurrent-state decode
 * path for Gated DeltaNet heads, on AMD Instinct MI355X (gfx950).
 *
 * The method ("LeapQuant: Efficient Linear Attention with Accurate Recurrent
 * State Quantization", sections 3.2-3.4 and appendix B; "Recurrent-state
 * quantization for linear attention: a first GPU kernel", Background and
 * What we built): each head's 128 x 128 state (rows = key coordinates,
 * columns = value coordinates) is held as an int8 residual with per-row
 * scales rho and per-column smoothing scales sigma, plus C fp32 compensator
 * lines.  Each decode token runs an APPEND: the output is read from that
 * fixed boundary state plus the fp32 records of the current window, and a new
 * record (cumulative decay, correction u_t, key k_t) is added.  After W
 * tokens a FOLD rebuilds the state, extracts the largest rows or columns as
 * compensators, smooths the residual per column, rounds it to int8 per row
 * and empties the record buffer.
 *
 * Arithmetic: IEEE binary32 with a fixed order of operations (canonical
 * 128-term halving trees, explicit fused multiply-adds), so results are
 * reproducible bit for bit; see the kernel sources for the exact sequences.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses owned by the caller.  The
 *     library never allocates, frees or synchronizes; every call is enqueued
 *     on `stream` (a hipStream_t passed as void*, NULL = default stream) and
 *     returns without waiting.
 *   - Return value: LEAPQ_OK (0) or a negative status.  Every status except
 *     LEAPQ_ERR_HIP is decided on the host before any HIP call; on an error
 *     nothing is enqueued and no state (including n_records) changes.
 *     LEAPQ_ERR_HIP reports hipGetLastError() right after a launch.  Faults
 *     inside a kernel surface on the stream, not here.
 *   - Tensors are dense, row-major, contiguous; "heads" below means
 *     batch * heads, and head h's data starts at h * (per-head size).
 *   - A leapq_layer must not be used from two streams at once.
 *   - Inputs and states must be finite.  With a NaN or an infinity in S0,
 *     q, k, v, alpha, beta or the gate arguments the results are unspecified
 *     (no error is reported); in particular the compensator picks, which
 *     compare line energies, need not follow the tie rule.
 */
#ifndef LEAPQ_H
#define LEAPQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LEAPQ_OK 0
#define LEAPQ_ERR_NULL (-1)        /* a required pointer is NULL */
#define LEAPQ_ERR_SHAPE (-2)       /* dk or dv is not 128 */
#define LEAPQ_ERR_RANGE (-3)       /* batch/heads < 1, window not in [1,64], n_comp not in [0,8],
                                      smoothing or qk_norm not 0/1, sigma_floor not > 0, what not
                                      in {0,1,2}, heads*batch too large, n_records out of
                                      [0, window], state_bits not 0/8/6/4, an option combined
                                      with one it excludes, reserved fields not zero */
#define LEAPQ_ERR_ALIGN (-4)       /* state not 256-byte aligned, or a tensor not 16-byte aligned */
#define LEAPQ_ERR_WINDOW_FULL (-5) /* append with n_records == window: fold first */
#define LEAPQ_ERR_DTYPE (-6)       /* in_dtype / state_dtype not LEAPQ_F32 or LEAPQ_BF16, rec_dtype not
                                      LEAPQ_F32, LEAPQ_BF16 or LEAPQ_FP8 */
#define LEAPQ_ERR_HIP (-7)         /* the HIP launch failed */

/* element types of q, k, v (in_dtype) and of the dense baseline state */
#define LEAPQ_F32 0
#define LEAPQ_BF16 1
/* record corrections only (rec_dtype): OCP FP8 E4M3 codes with one
 * power-of-two scale per group of 32 value columns */
#define LEAPQ_FP8 2

/* decay of the recurrence ("LeapQuant" App. A: D_t = Diag(alpha_t)): one
 * scalar per head and token (Gated DeltaNet), or one value per key channel
 * (Kimi Delta Attention), which scales the state's rows */
#define LEAPQ_DECAY_SCALAR 0
#define LEAPQ_DECAY_CHANNEL 1

/* compensator fit at init and fold: greedy extraction of whole rows or
 * columns; rank-one pairs (a_j, b_j) by power sweeps from the longest row
 * ("Recurrent-state quantization for linear attention: a first GPU kernel",
 * Where the time goes: four compensators, eight sweeps each; "LeapQuant"
 * 3.3: compensators as rank-one updates); or the same pairs fitted together
 * as a block, warm-started from the window's own pairs (the same page,
 * Redesign): subspace iteration with modified Gram-Schmidt, 2 sweeps per
 * fold and 8 at init, where the start is the unit vectors of the rows of
 * largest energy */
#define LEAPQ_COMP_LINES 0
#define LEAPQ_COMP_RANK1 1
#define LEAPQ_COMP_BLOCK 2

/* what leapq_dequant writes */
#define LEAPQ_DEQ_RESIDUAL 0 /* (code * rho_r) * sigma_c, compensator lines left at zero */
#define LEAPQ_DEQ_BOUNDARY 1 /* residual + compensator lines: the window's fixed state B */
#define LEAPQ_DEQ_CURRENT 2  /* gamma_n * B + sum_i (gamma_n / gamma_i) k_i u_i^T: state after n records */

typedef struct leapq_config {
    int32_t batch;       /* requests (>= 1) */
    int32_t heads;       /* GDN heads per request (>= 1) */
    int32_t dk, dv;      /* state shape; must be 128, 128 */
    int32_t window;      /* W: tokens per window, [1, 64]; 16 in the pages' setting */
    int32_t n_comp;      /* C: compensator lines, [0, 8]; 4 in the pages' setting */
    int32_t smoothing;   /* 1: per-column residual smoothing; 0: sigma = 1 */
    float sigma_floor;   /* positive floor of the smoothing scale (1e-6) */
    int32_t in_dtype;    /* LEAPQ_F32 or LEAPQ_BF16 for q, k, v */
    int32_t qk_norm;     /* 1: the gated appends L2-normalize q and k (record keys are then fp32); 0 or 1 */
    int32_t decay;       /* LEAPQ_DECAY_SCALAR (GDN: alpha per head) or LEAPQ_DECAY_CHANNEL (KDA: alpha
                            per head and key channel); channel decay excludes qk_norm */
    int32_t rec_dtype;   /* LEAPQ_F32 (the method's records), LEAPQ_BF16: record corrections u kept in
                            bf16, rounded to nearest even on store, or LEAPQ_FP8: u kept as E4M3 (sign,
                            4 exponent bits, bias 7, 3 mantissa bits, largest 448) of u_c / s_j, where
                            group j holds the value columns c with c % 4 = j and s_j is the smallest
                            power of two >= 2^-126 with max_c |u_c| <= 448 s_j, rounded to nearest, ties
                            to even (lossy lower-precision options, "Recurrent-state quantization for
                            linear attention: a first GPU kernel", Why rounding the state is difficult:
                            records kept in higher precision, traded here for bytes; the token that makes
                            a record reads out with its fp32 u); both require scalar decay and
                            qk_norm = 0 and are not taken by the gated entry points */
    int32_t comp_fit;    /* LEAPQ_COMP_LINES (whole rows or columns), LEAPQ_COMP_RANK1 (rank-one pairs
                            fitted by power sweeps) or LEAPQ_COMP_BLOCK (the pairs fitted as a block);
                            the pair fits require n_comp <= 4, scalar decay, rec_dtype LEAPQ_F32, and
                            are not taken by the gated entry points */
    int32_t state_bits;  /* bits per residual code: 0 or 8 (int8, the method's state), 6 or 4 (symmetric
                            codes -31..31 or -7..7 with scale absmax / 31 or / 7, "LeapQuant" 4.2: the
                            method at 6 and 4 bits); 6 and 4 require scalar decay, line compensators,
                            rec_dtype LEAPQ_F32 and qk_norm = 0, and are not taken by the gated entry
                            points or leapq_step */
    int32_t reserved[2]; /* must be zero */
} leapq_config;

/* Byte layout of one layer's state buffer ("LeapQuant" 4.3: the boundary
 * state with its scales and compensators costs about 1.19 bytes per state
 * element, against 4 for fp32).  Sections are "structure of arrays" over
 * heads; each section starts on a 256-byte boundary and head h's
 * slice starts at off_X + h * (per-head size of X).  With
 * iperm(x) = x ^ (x & 4 ? 3 : 0) for x < 32:
 *   codes     int8  [heads][16384]     the code of (key row r, value column c)
 *                                      is byte 4096 (c % 4) + 1024 (r / 32)
 *                                      + 16 (iperm(r % 32) + 32 ((c / 4) % 2))
 *                                      + c / 8 of the head's block;
 *             state_bits 4: [heads][8192], with w = c % 4, p = r / 32,
 *                                      l = iperm(r % 32) + 32 ((c / 4) % 2),
 *                                      m = c / 8: the nibble of byte 2048 w
 *                                      + 1024 (p / 2) + 16 l + 8 (p % 2)
 *                                      + 4 (m / 8) + m % 4, low nibble for
 *                                      m % 8 < 4, else high (two's complement);
 *             state_bits 6: [heads][12288], bits 0-3 as for 4 bits in the
 *                                      first 8192 bytes, bits 4-5 at bit
 *                                      2 (m / 4) of byte 8192 + 1024 w + 16 l
 *                                      + 4 p + m % 4
 *   row_scale fp32  [heads][128]       rho_r
 *   col_scale fp32  [heads][128]       sigma_c
 *   comp_idx  int32 [heads][C]         -1 unused, 0..127 row r, 128+c column c
 *   comp_vec  fp32  [heads][C][128]    the line's values (over c for a row,
 *                                      over r for a column), natural order;
 *                   [heads][C][2][128] with LEAPQ_COMP_RANK1 or _BLOCK:
 *                                      a_j (unit norm, over rows) then b_j
 *                                      (over columns); comp_idx holds the
 *                                      start row (rank-one) or j (block),
 *                                      -1 for an unused pair
 *   rec_gamma fp32  [heads][W]         cumulative decay since the window start
 *                   ([heads][W][128] per key row with LEAPQ_DECAY_CHANNEL)
 *   rec_k     e     [heads][W][128]    record keys in key-row order, in the
 *                                      input dtype (a record's key is the
 *                                      token's k as given, so bf16 storage
 *                                      of bf16 inputs is exact), or fp32
 *                                      when qk_norm = 1
 *   rec_u     fp32 or bf16 (rec_dtype) [heads][W][128]  record corrections; value column c is
 *                                      stored at 32 (c % 4) + 8 (c / 32)
 *                                      + 4 ((c / 4) % 2) + (c / 8) % 4;
 *             with LEAPQ_FP8 [heads][W][144 bytes]: the 128 E4M3 codes
 *                                      in that order, then the 4 fp32 scales
 *                                      (scale j serves positions 32 j .. 32 j
 *                                      + 31, the columns with c % 4 = j)
 * These orders are the thread map of the kernels (each thread's 64 codes are
 * four 16-byte loads, each wave's loads 1 KB contiguous; the record keys and
 * corrections are the A operand order of the fold's matrix instructions).
 * boundary_bytes_per_head = 16384 + 512 + 512 + 4C + 512C (19,472 at C = 4:
 * 1.19 bytes per state element; 12,288 or 8,192 code bytes at 6 or 4 bits); record_bytes_per_head = W * (4 g + 128 e + f)
 * with e = 2 for bf16 inputs and qk_norm = 0, else 4, g = 1 (scalar decay)
 * or 128 (channel decay), and f = 512, 256 with rec_dtype = LEAPQ_BF16, or
 * 144 with LEAPQ_FP8. */
typedef struct leapq_layout {
    uint64_t total_bytes;
    uint64_t off_codes, off_row_scale, off_col_scale, off_comp_idx, off_comp_vec;
    uint64_t off_rec_gamma, off_rec_k, off_rec_u;
    uint64_t boundary_bytes_per_head;
    uint64_t record_bytes_per_head;
} leapq_layout;

/* One layer: its configuration, its state buffer (device, caller-owned,
 * total_bytes long, 256-byte aligned) and the host-side count of records in
 * the current window.  All heads of a layer share the window phase. */
typedef struct leapq_layer {
    leapq_config cfg;
    void *state;
    int32_t n_records;
    int32_t reserved;
} leapq_layer;

/* Fills *out with the layout for cfg ("LeapQuant" 4.3: int8 codes with
 * per-row and per-column scales and fp32 compensators, 19,472 bytes per
 * 128 x 128 head at C = 4, the 1.19 bytes per element it reports; plus the
 * window's records, "Recurrent-state quantization for linear attention: a
 * first GPU kernel", Why rounding the state is difficult: recent updates
 * kept in higher precision).  Host only; touches no device.  Returns
 * LEAPQ_ERR_NULL for a NULL argument and the configuration statuses above
 * for an invalid cfg. */
int32_t leapq_query_layout(const leapq_config *cfg, leapq_layout *out);

/* Quantizes the caller's fp32 states S0 [heads][128][128] (device) into the
 * layer's boundary state: compensator extraction, smoothing and per-row int8
 * exactly as a fold does ("LeapQuant" 3.3-3.4), then empties the window
 * (n_records := 0).  S0 is read only. */
int32_t leapq_init_state(leapq_layer *layer, const float *S0, void *stream);

/* One decode token for every head of the layer ("Recurrent-state
 * quantization for linear attention: a first GPU kernel", Background: decay,
 * read with the key, correction, rank-one write, read the output; "LeapQuant"
 * B.2-B.3: read from the fixed boundary plus the records).
 *   q, k [heads][128], v [heads][128] in cfg.in_dtype (device);
 *   alpha [heads] fp32 (device; [heads][128], 16-byte aligned, with
 *   LEAPQ_DECAY_CHANNEL): decay of this token; beta [heads] fp32: step size;
 *   o [heads][128] fp32 (device, written): the output S_t^T q_t.
 * Writes record n_records (gamma_t = gamma_{t-1} * alpha, k_t, u_t =
 * beta (v_t - (D_t S_{t-1})^T k_t) with D_t = alpha or Diag(alpha)) and
 * increments n_records.  Requires n_records < window (else
 * LEAPQ_ERR_WINDOW_FULL).  With channel decay ("LeapQuant" App. A, B.2) the
 * read uses gamma_t (.) k against the boundary and (gamma_t / gamma_i) (.) k_i
 * for record i, per key row. */
int32_t leapq_append(leapq_layer *layer, const void *q, const void *k, const void *v,
                     const float *alpha, const float *beta, float *o, void *stream);

/* The window's last token and its fold in one call: exactly leapq_append
 * followed by leapq_fold ("Recurrent-state quantization for linear
 * attention: a first GPU kernel", What we built: the append adds the
 * token's record and computes its output; the fold then rebuilds, selects
 * compensators, rescales, rounds and empties the buffer).  Requires
 * n_records == window - 1 (else LEAPQ_ERR_RANGE); arguments as for
 * leapq_append.  With window <= 16 this is one launch in which the
 * boundary and the records are read once and the token's record never
 * reaches HBM; otherwise the two steps are launched in turn.  Sets
 * n_records := 0. */
int32_t leapq_append_fold(leapq_layer *layer, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, float *o, void *stream);

/* Gate arithmetic in front of the append: the decay and step size are
 * computed from the layer's raw projections per head and token, and q, k
 * are L2-normalized when the layer has qk_norm = 1 ("Recurrent-state
 * quantization for linear attention: a first GPU kernel", Results: the
 * column with gate arithmetic; the pages give no formula, these are the
 * Gated DeltaNet layer's gates):
 *   alpha = exp(-exp(A_log[j]) * softplus(a + dt_bias[j])),  beta = 1 / (1 + exp(-b)),
 *   softplus(x) = max(x, 0) + log1p(exp(-|x|)), evaluated in binary64 from the
 *   fp32 arguments and rounded once to fp32 (j = head index within a request);
 *   k <- k * (1 / sqrt(k . k + norm_eps)),
 *   q <- (q * (1 / sqrt(q . q + norm_eps))) * q_scale, in fp32 with the
 *   canonical 128-term dot. */
typedef struct leapq_gate {
    const float *A_log;   /* [cfg.heads] fp32 (device), per model head, shared by the batch */
    const float *dt_bias; /* [cfg.heads] fp32 (device) */
    float q_scale;        /* multiplies the normalized query (used when qk_norm = 1), e.g. 128^-1/2 */
    float norm_eps;       /* >= 0, added under the root of the L2 norm (used when qk_norm = 1) */
    int32_t reserved[2];  /* must be zero */
} leapq_gate;

/* leapq_append with the gate arithmetic fused in front ("Recurrent-state
 * quantization for linear attention: a first GPU kernel", Results: the
 * kernel timed with gate arithmetic): a, b [heads] fp32
 * (device) are the raw decay and step-size projections of this token, and q,
 * k are the raw projections (normalized in the kernel when qk_norm = 1).
 * Everything else, including the record written and the output, is as for
 * leapq_append with the gated alpha, beta, q and k.  gate must not be NULL
 * (LEAPQ_ERR_NULL), its pointers 4-byte aligned (LEAPQ_ERR_ALIGN), norm_eps
 * finite and >= 0, q_scale finite and reserved zero (LEAPQ_ERR_RANGE).  The
 * gates are the scalar-decay (GDN) ones: a layer with LEAPQ_DECAY_CHANNEL
 * gets LEAPQ_ERR_RANGE. */
int32_t leapq_append_gated(leapq_layer *layer, const leapq_gate *gate, const void *q, const void *k,
                           const void *v, const float *a, const float *b, float *o, void *stream);

/* leapq_append_fold with the gate arithmetic of leapq_append_gated
 * ("Recurrent-state quantization for linear attention: a first GPU kernel",
 * Results: gate arithmetic; What we built: the append, then the fold).
 * Arguments, requirements and statuses as for the two calls it joins. */
int32_t leapq_append_fold_gated(leapq_layer *layer, const leapq_gate *gate, const void *q, const void *k,
                                const void *v, const float *a, const float *b, float *o, void *stream);

/* One decode token with a window phase per request (staggered phases:
 * requests that joined at different times fold at different tokens; a
 * window still holds W tokens of each request, "Recurrent-state quantization
 * for linear attention: a first GPU kernel", Why rounding the state is
 * difficult; What we built).  n_in [batch] int32 (device) holds each
 * request's record count n: with n = window - 1 its heads append and fold in
 * this launch (as leapq_append_fold), with 0 <= n < window - 1 they append
 * (as leapq_append), and with any other n (negative: the request takes no
 * token this step) its heads' state and output rows are left untouched.
 * n_out [batch] int32 (device) or NULL receives each request's next count:
 * 0 after a fold, n + 1 after an append, n otherwise; it must not overlap
 * n_in (LEAPQ_ERR_RANGE).  gate NULL: alpha, beta are given as for
 * leapq_append; otherwise a, b are the raw projections and the gate
 * arithmetic of leapq_append_gated applies.  Requires window <= 16
 * (LEAPQ_ERR_RANGE).  The token arguments, layout and per-head results are
 * those of the entry points named above, bit for bit.  layer->n_records is
 * neither read nor changed: a layer driven by leapq_step keeps its phases in
 * the caller's array and must not be mixed with the single-phase calls
 * (leapq_append, leapq_append_fold, leapq_fold, and leapq_dequant of the
 * current state) unless every request has the phase n_records.  All blocks
 * are resourced for the fold (4 per compute unit). */
int32_t leapq_step(leapq_layer *layer, const leapq_gate *gate, const int32_t *n_in, int32_t *n_out,
                   const void *q, const void *k, const void *v, const float *alpha, const float *beta, float *o,
                   void *stream);

/* Closes the window ("Recurrent-state quantization for linear attention: a
 * first GPU kernel", What we built: rebuild, select compensators, rescale,
 * round, empty the buffer; "LeapQuant" B.3): rebuilds the current state from
 * the boundary and the n_records records, re-extracts the compensators,
 * recomputes smoothing and row scales, rounds to int8 in place, and sets
 * n_records := 0.  Valid for any n_records in [0, window]. */
int32_t leapq_fold(leapq_layer *layer, void *stream);

/* Writes an fp32 [heads][128][128] view of the layer's state to S_out
 * (device): what = LEAPQ_DEQ_RESIDUAL, LEAPQ_DEQ_BOUNDARY or LEAPQ_DEQ_CURRENT
 * (see above; "LeapQuant" B.3: the residual is rescaled in original
 * coordinates and the compensators added in full precision; B.2: the state
 * after n records of the window is the decayed boundary plus the records'
 * rank-one terms).  Reads the state only; what outside {0, 1, 2} gives
 * LEAPQ_ERR_RANGE.  The current view runs the fold's own rebuild. */
int32_t leapq_dequant(const leapq_layer *layer, int32_t what, float *S_out, void *stream);

/* Unquantized per-token GDN decode on a dense state, in place (the fp32-state
 * and bf16-state baselines: "Recurrent-state quantization for linear
 * attention: a first GPU kernel", Background: per token the state is decayed,
 * read with the key, corrected and written back as a rank-one update, and the
 * output read, and Results: the kernels timed with an fp32 state;
 * "LeapQuant" 3.1 and App. A: the delta-rule recurrence with a scalar or
 * diagonal decay).  S [heads][128][128] in state_dtype (device,
 * natural row-major layout); q, k, v in cfg->in_dtype; alpha, beta fp32;
 * o fp32.  Per token: S = alpha S (row r scaled by alpha[r] with cfg->decay
 * = LEAPQ_DECAY_CHANNEL, alpha then [heads][128]); u = beta (v - S^T k);
 * S += k u^T; o = S^T q; a bf16 state is widened, updated in fp32 and
 * rounded to nearest even on store.  Uses batch, heads, dk, dv, in_dtype and
 * decay of cfg only. */
int32_t leapq_gdn_decode(const leapq_config *cfg, int32_t state_dtype, void *S, const void *q,
                         const void *k, const void *v, const float *alpha, const float *beta,
                         float *o, void *stream);

/* Static description of a status code (a utility with no passage behind
 * it; unknown codes give "unknown status"). */
const char *leapq_status_str(int32_t status);

/* Library version: major * 10000 + minor * 100 + patch (a utility with no
 * passage behind it). */
int32_t leapq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LEAPQ_H */
