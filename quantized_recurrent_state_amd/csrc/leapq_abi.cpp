// C ABI of libleapq: argument validation, state layout, kernel launches.
// Every check happens on the host before any HIP call; the library never
// allocates, frees or synchronizes.
#include "leapq.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "leapq_internal.h"

namespace {

constexpr int kD = 128;
constexpr uint64_t kAlign = 256;
constexpr int64_t kMaxHeads = (int64_t)1 << 31;

uint64_t round_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int32_t check_config(const leapq_config *c)
{
    if (!c) return LEAPQ_ERR_NULL;
    if (c->dk != kD || c->dv != kD) return LEAPQ_ERR_SHAPE;
    if (c->batch < 1 || c->heads < 1) return LEAPQ_ERR_RANGE;
    if ((int64_t)c->batch * c->heads >= kMaxHeads) return LEAPQ_ERR_RANGE;
    if (c->in_dtype != LEAPQ_F32 && c->in_dtype != LEAPQ_BF16) return LEAPQ_ERR_DTYPE;
    if (c->decay != LEAPQ_DECAY_SCALAR && c->decay != LEAPQ_DECAY_CHANNEL) return LEAPQ_ERR_RANGE;
    return LEAPQ_OK;
}

int32_t check_method_config(const leapq_config *c)
{
    int32_t st = check_config(c);
    if (st != LEAPQ_OK) return st;
    if (c->window < 1 || c->window > 64) return LEAPQ_ERR_RANGE;
    if (c->n_comp < 0 || c->n_comp > 8) return LEAPQ_ERR_RANGE;
    if (c->smoothing != 0 && c->smoothing != 1) return LEAPQ_ERR_RANGE;
    if (!(c->sigma_floor > 0.0f) || c->sigma_floor > 3.0e38f) return LEAPQ_ERR_RANGE;
    if (c->qk_norm != 0 && c->qk_norm != 1) return LEAPQ_ERR_RANGE;
    if (c->decay == LEAPQ_DECAY_CHANNEL && c->qk_norm) return LEAPQ_ERR_RANGE;
    if (c->rec_dtype != LEAPQ_F32 && c->rec_dtype != LEAPQ_BF16 && c->rec_dtype != LEAPQ_FP8)
        return LEAPQ_ERR_DTYPE;
    if (c->rec_dtype != LEAPQ_F32 && (c->decay != LEAPQ_DECAY_SCALAR || c->qk_norm)) return LEAPQ_ERR_RANGE;
    if (c->comp_fit != LEAPQ_COMP_LINES && c->comp_fit != LEAPQ_COMP_RANK1 && c->comp_fit != LEAPQ_COMP_BLOCK)
        return LEAPQ_ERR_RANGE;
    if (c->comp_fit != LEAPQ_COMP_LINES &&
        (c->n_comp > 4 || c->decay != LEAPQ_DECAY_SCALAR || c->rec_dtype != LEAPQ_F32))
        return LEAPQ_ERR_RANGE;
    if (c->state_bits != 0 && c->state_bits != 8 && c->state_bits != 6 && c->state_bits != 4) return LEAPQ_ERR_RANGE;
    if (c->state_bits == 6 || c->state_bits == 4) {
        // the 6- and 4-bit options: scalar decay, line compensators, fp32 records, no normalizing appends
        if (c->decay != LEAPQ_DECAY_SCALAR || c->comp_fit != LEAPQ_COMP_LINES || c->rec_dtype != LEAPQ_F32 ||
            c->qk_norm)
            return LEAPQ_ERR_RANGE;
    }
    if (c->reserved[0] || c->reserved[1]) return LEAPQ_ERR_RANGE;
    return LEAPQ_OK;
}

// Record keys are stored in the input dtype, which holds the token's k
// exactly, unless the layer's gated appends normalize k (then fp32).
bool key_bf16(const leapq_config *c) { return c->in_dtype == LEAPQ_BF16 && !c->qk_norm; }

// bits per residual code (8 when the field is 0) and bytes of a head's codes
int code_bits(const leapq_config *c) { return c->state_bits == 6 || c->state_bits == 4 ? c->state_bits : 8; }
uint64_t code_bytes(const leapq_config *c) { return (uint64_t)kD * kD * code_bits(c) / 8; }

void compute_layout(const leapq_config *c, leapq_layout *L)
{
    const uint64_t H = (uint64_t)c->batch * (uint64_t)c->heads;
    const uint64_t C = (uint64_t)c->n_comp, W = (uint64_t)c->window;
    const uint64_t kb = key_bf16(c) ? 2 : 4;  // record key element
    const uint64_t gw = c->decay == LEAPQ_DECAY_CHANNEL ? kD : 1;  // record decay values
    // one record's corrections: 128 fp32 or bf16 values, or 128 fp8 codes and 4 fp32 scales
    const uint64_t ub = c->rec_dtype == LEAPQ_BF16 ? 2 * kD : c->rec_dtype == LEAPQ_FP8 ? kD + 16 : 4 * kD;
    const uint64_t cw = c->comp_fit != LEAPQ_COMP_LINES ? 2 : 1;   // compensator vectors (pairs: a, b)
    uint64_t off = 0;
    L->off_codes = off;
    off = round_up(off + H * code_bytes(c));
    L->off_row_scale = off;
    off = round_up(off + H * kD * 4);
    L->off_col_scale = off;
    off = round_up(off + H * kD * 4);
    L->off_comp_idx = off;
    off = round_up(off + H * C * 4);
    L->off_comp_vec = off;
    off = round_up(off + H * C * cw * kD * 4);
    L->off_rec_gamma = off;
    off = round_up(off + H * W * gw * 4);
    L->off_rec_k = off;
    off = round_up(off + H * W * kD * kb);
    L->off_rec_u = off;
    off = round_up(off + H * W * ub);
    L->total_bytes = off;
    L->boundary_bytes_per_head = code_bytes(c) + 2 * kD * 4 + C * 4 + C * cw * kD * 4;
    L->record_bytes_per_head = W * (4 * gw + kD * kb + ub);
}

int32_t view_of(const leapq_layer *layer, leapq::StateView *sv)
{
    if (!layer) return LEAPQ_ERR_NULL;
    int32_t st = check_method_config(&layer->cfg);
    if (st != LEAPQ_OK) return st;
    if (!layer->state) return LEAPQ_ERR_NULL;
    if (!aligned(layer->state, kAlign)) return LEAPQ_ERR_ALIGN;
    if (layer->n_records < 0 || layer->n_records > layer->cfg.window) return LEAPQ_ERR_RANGE;
    leapq_layout L;
    compute_layout(&layer->cfg, &L);
    char *b = (char *)layer->state;
    sv->codes = (int8_t *)(b + L.off_codes);
    sv->rho = (float *)(b + L.off_row_scale);
    sv->sigma = (float *)(b + L.off_col_scale);
    sv->cidx = (int32_t *)(b + L.off_comp_idx);
    sv->cvec = (float *)(b + L.off_comp_vec);
    sv->rgam = (float *)(b + L.off_rec_gamma);
    sv->rk = b + L.off_rec_k;
    sv->ru = b + L.off_rec_u;
    sv->C = layer->cfg.n_comp;
    sv->W = layer->cfg.window;
    sv->key_bf16 = key_bf16(&layer->cfg);
    sv->kda = layer->cfg.decay == LEAPQ_DECAY_CHANNEL;
    sv->u_bf16 = layer->cfg.rec_dtype == LEAPQ_BF16;
    sv->u_fp8 = layer->cfg.rec_dtype == LEAPQ_FP8;
    sv->u_rec_bytes = layer->cfg.rec_dtype == LEAPQ_BF16 ? 2 * kD : layer->cfg.rec_dtype == LEAPQ_FP8 ? kD + 16 : 4 * kD;
    sv->r1 = layer->cfg.comp_fit != LEAPQ_COMP_LINES;
    sv->blk = layer->cfg.comp_fit == LEAPQ_COMP_BLOCK;
    sv->cbits = code_bits(&layer->cfg);
    sv->code_bytes = (int)code_bytes(&layer->cfg);
    return LEAPQ_OK;
}

int heads_of(const leapq_config *c) { return c->batch * c->heads; }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? LEAPQ_OK : LEAPQ_ERR_HIP; }

}  // namespace

extern "C" {

int32_t leapq_query_layout(const leapq_config *cfg, leapq_layout *out)
{
    if (!out) return LEAPQ_ERR_NULL;
    int32_t st = check_method_config(cfg);
    if (st != LEAPQ_OK) return st;
    compute_layout(cfg, out);
    return LEAPQ_OK;
}

int32_t leapq_init_state(leapq_layer *layer, const float *S0, void *stream)
{
    leapq::StateView sv;
    int32_t st = view_of(layer, &sv);
    if (st != LEAPQ_OK) return st;
    if (!S0) return LEAPQ_ERR_NULL;
    if (!aligned(S0, 16)) return LEAPQ_ERR_ALIGN;
    st = hip_status(leapq::launch_init(sv, heads_of(&layer->cfg), S0, layer->cfg.smoothing,
                                       layer->cfg.sigma_floor, (hipStream_t)stream));
    if (st == LEAPQ_OK) layer->n_records = 0;
    return st;
}

}  // extern "C"

namespace {

leapq::GateArgs plain_gate(const leapq_config &c) { return {nullptr, nullptr, 1.0f, 0.0f, c.heads, 0, 0}; }

int32_t gate_of(const leapq_layer *layer, const leapq_gate *g, leapq::GateArgs *out)
{
    if (!g || !g->A_log || !g->dt_bias) return LEAPQ_ERR_NULL;
    if (layer->cfg.decay != LEAPQ_DECAY_SCALAR || layer->cfg.rec_dtype != LEAPQ_F32 ||
        layer->cfg.comp_fit != LEAPQ_COMP_LINES || code_bits(&layer->cfg) != 8)
        return LEAPQ_ERR_RANGE;
    if (!aligned(g->A_log, 4) || !aligned(g->dt_bias, 4)) return LEAPQ_ERR_ALIGN;
    if (g->reserved[0] || g->reserved[1]) return LEAPQ_ERR_RANGE;
    if (!(g->norm_eps >= 0.0f) || g->norm_eps > 3.0e38f) return LEAPQ_ERR_RANGE;
    if (!(g->q_scale == g->q_scale) || g->q_scale > 3.0e38f || g->q_scale < -3.0e38f) return LEAPQ_ERR_RANGE;
    *out = {g->A_log, g->dt_bias, g->q_scale, g->norm_eps, layer->cfg.heads, 1, layer->cfg.qk_norm};
    return LEAPQ_OK;
}

int32_t check_token(const void *q, const void *k, const void *v, const float *a, const float *b, const float *o,
                    bool kda)
{
    if (!q || !k || !v || !a || !b || !o) return LEAPQ_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(a, kda ? 16 : 4) ||
        !aligned(b, 4))
        return LEAPQ_ERR_ALIGN;
    return LEAPQ_OK;
}

int32_t append_impl(leapq_layer *layer, const leapq_gate *gate, const void *q, const void *k, const void *v,
                    const float *alpha, const float *beta, float *o, void *stream)
{
    leapq::StateView sv;
    int32_t st = view_of(layer, &sv);
    if (st != LEAPQ_OK) return st;
    leapq::GateArgs g = plain_gate(layer->cfg);
    if (gate && (st = gate_of(layer, gate, &g)) != LEAPQ_OK) return st;
    if ((st = check_token(q, k, v, alpha, beta, o, sv.kda)) != LEAPQ_OK) return st;
    if (layer->n_records >= layer->cfg.window) return LEAPQ_ERR_WINDOW_FULL;
    st = hip_status(leapq::launch_append(sv, heads_of(&layer->cfg), layer->n_records,
                                         layer->cfg.in_dtype == LEAPQ_BF16, q, k, v, alpha, beta, o, g,
                                         (hipStream_t)stream));
    if (st == LEAPQ_OK) layer->n_records += 1;
    return st;
}

int32_t append_fold_impl(leapq_layer *layer, const leapq_gate *gate, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *o, void *stream)
{
    leapq::StateView sv;
    int32_t st = view_of(layer, &sv);
    if (st != LEAPQ_OK) return st;
    leapq::GateArgs g = plain_gate(layer->cfg);
    if (gate && (st = gate_of(layer, gate, &g)) != LEAPQ_OK) return st;
    if ((st = check_token(q, k, v, alpha, beta, o, sv.kda)) != LEAPQ_OK) return st;
    if (layer->n_records != layer->cfg.window - 1) return LEAPQ_ERR_RANGE;
    const int heads = heads_of(&layer->cfg);
    const int bf16 = layer->cfg.in_dtype == LEAPQ_BF16;
    hipStream_t s = (hipStream_t)stream;
    if (layer->cfg.window <= 16) {
        st = hip_status(leapq::launch_append_fold(sv, heads, layer->n_records, bf16, q, k, v, alpha, beta, o,
                                                  layer->cfg.smoothing, layer->cfg.sigma_floor, g, s));
    } else {
        st = hip_status(leapq::launch_append(sv, heads, layer->n_records, bf16, q, k, v, alpha, beta, o, g, s));
        if (st == LEAPQ_OK)
            st = hip_status(leapq::launch_fold(sv, heads, layer->n_records + 1, layer->cfg.smoothing,
                                               layer->cfg.sigma_floor, s));
    }
    if (st == LEAPQ_OK) layer->n_records = 0;
    return st;
}

int32_t step_impl(leapq_layer *layer, const leapq_gate *gate, const int32_t *n_in, int32_t *n_out, const void *q,
                  const void *k, const void *v, const float *alpha, const float *beta, float *o, void *stream)
{
    leapq::StateView sv;
    int32_t st = view_of(layer, &sv);
    if (st != LEAPQ_OK) return st;
    leapq::GateArgs g = plain_gate(layer->cfg);
    if (gate && (st = gate_of(layer, gate, &g)) != LEAPQ_OK) return st;
    if ((st = check_token(q, k, v, alpha, beta, o, sv.kda)) != LEAPQ_OK) return st;
    if (!n_in) return LEAPQ_ERR_NULL;
    if (!aligned(n_in, 4) || (n_out && !aligned(n_out, 4))) return LEAPQ_ERR_ALIGN;
    if (layer->cfg.window > 16 || code_bits(&layer->cfg) != 8) return LEAPQ_ERR_RANGE;
    // every head of a request reads n_in while block 0 of the request writes n_out
    if (n_out) {
        const char *a0 = (const char *)n_in, *b0 = (const char *)n_out;
        const size_t bytes = sizeof(int32_t) * (size_t)layer->cfg.batch;
        if (a0 < b0 + bytes && b0 < a0 + bytes) return LEAPQ_ERR_RANGE;
    }
    return hip_status(leapq::launch_step(sv, heads_of(&layer->cfg), layer->cfg.heads, n_in, n_out,
                                         layer->cfg.in_dtype == LEAPQ_BF16, q, k, v, alpha, beta, o,
                                         layer->cfg.smoothing, layer->cfg.sigma_floor, g, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int32_t leapq_append(leapq_layer *layer, const void *q, const void *k, const void *v, const float *alpha,
                     const float *beta, float *o, void *stream)
{
    return append_impl(layer, nullptr, q, k, v, alpha, beta, o, stream);
}

int32_t leapq_append_fold(leapq_layer *layer, const void *q, const void *k, const void *v, const float *alpha,
                          const float *beta, float *o, void *stream)
{
    return append_fold_impl(layer, nullptr, q, k, v, alpha, beta, o, stream);
}

int32_t leapq_append_gated(leapq_layer *layer, const leapq_gate *gate, const void *q, const void *k, const void *v,
                           const float *a, const float *b, float *o, void *stream)
{
    if (!gate) return LEAPQ_ERR_NULL;
    return append_impl(layer, gate, q, k, v, a, b, o, stream);
}

int32_t leapq_append_fold_gated(leapq_layer *layer, const leapq_gate *gate, const void *q, const void *k,
                                const void *v, const float *a, const float *b, float *o, void *stream)
{
    if (!gate) return LEAPQ_ERR_NULL;
    return append_fold_impl(layer, gate, q, k, v, a, b, o, stream);
}

int32_t leapq_step(leapq_layer *layer, const leapq_gate *gate, const int32_t *n_in, int32_t *n_out, const void *q,
                   const void *k, const void *v, const float *alpha, const float *beta, float *o, void *stream)
{
    return step_impl(layer, gate, n_in, n_out, q, k, v, alpha, beta, o, stream);
}

int32_t leapq_fold(leapq_layer *layer, void *stream)
{
    leapq::StateView sv;
    int32_t st = view_of(layer, &sv);
    if (st != LEAPQ_OK) return st;
    st = hip_status(leapq::launch_fold(sv, heads_of(&layer->cfg), layer->n_records, layer->cfg.smoothing,
                                       layer->cfg.sigma_floor, (hipStream_t)stream));
    if (st == LEAPQ_OK) layer->n_records = 0;
    return st;
}

int32_t leapq_dequant(const leapq_layer *layer, int32_t what, float *S_out, void *stream)
{
    leapq::StateView sv;
    int32_t st = view_of(layer, &sv);
    if (st != LEAPQ_OK) return st;
    if (what < LEAPQ_DEQ_RESIDUAL || what > LEAPQ_DEQ_CURRENT) return LEAPQ_ERR_RANGE;
    if (!S_out) return LEAPQ_ERR_NULL;
    if (!aligned(S_out, 16)) return LEAPQ_ERR_ALIGN;
    return hip_status(leapq::launch_dequant(sv, heads_of(&layer->cfg), layer->n_records, what, S_out,
                                            (hipStream_t)stream));
}

int32_t leapq_gdn_decode(const leapq_config *cfg, int32_t state_dtype, void *S, const void *q, const void *k,
                         const void *v, const float *alpha, const float *beta, float *o, void *stream)
{
    int32_t st = check_config(cfg);
    if (st != LEAPQ_OK) return st;
    if (state_dtype != LEAPQ_F32 && state_dtype != LEAPQ_BF16) return LEAPQ_ERR_DTYPE;
    if (!S || !q || !k || !v || !alpha || !beta || !o) return LEAPQ_ERR_NULL;
    const int kda = cfg->decay == LEAPQ_DECAY_CHANNEL;
    if (!aligned(S, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(alpha, kda ? 16 : 4) || !aligned(beta, 4))
        return LEAPQ_ERR_ALIGN;
    return hip_status(leapq::launch_gdn_decode(heads_of(cfg), state_dtype == LEAPQ_BF16,
                                               cfg->in_dtype == LEAPQ_BF16, kda, S, q, k, v, alpha, beta, o,
                                               (hipStream_t)stream));
}

const char *leapq_status_str(int32_t status)
{
    switch (status) {
    case LEAPQ_OK: return "ok";
    case LEAPQ_ERR_NULL: return "a required pointer is NULL";
    case LEAPQ_ERR_SHAPE: return "dk and dv must be 128";
    case LEAPQ_ERR_RANGE: return "an argument is out of range";
    case LEAPQ_ERR_ALIGN: return "misaligned pointer (state: 256 bytes, tensors: 16 bytes)";
    case LEAPQ_ERR_WINDOW_FULL: return "window full: fold before the next append";
    case LEAPQ_ERR_DTYPE: return "unsupported element type";
    case LEAPQ_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

int32_t leapq_version(void) { return 100; }

}  // extern "C"
