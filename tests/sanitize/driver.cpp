// Sanitizer driver (CPU only): built with AddressSanitizer and
// UndefinedBehaviorSanitizer together with the C ABI's host code
// (quantized_recurrent_state_amd/csrc/leapq_abi.cpp, its launchers replaced
// by launch_stubs.cpp) and the oracle (oracle/leapq_oracle.c).
//
// Part 1 drives every entry point of include/leapq.h through valid and
// invalid arguments on a grid of configurations and checks the statuses and
// the record count.  Part 2 runs every oracle routine on small seeded inputs:
// two windows per variant (lines, rank-one pairs, block fit, per-channel
// decay, the key-row smoothing study), gates, norms, dense steps and bf16
// conversions.  Exit status 0 means every check held; the sanitizers abort
// the process on any error they find.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "leapq.h"

namespace leapq {
extern int stub_calls, stub_heads, stub_n;
}

extern "C" {
void lqo_init(const float *, int, int, float, int8_t *, float *, float *, int32_t *, float *);
void lqo_append(const int8_t *, const float *, const float *, int, const int32_t *, const float *, int, float *,
                float *, float *, const float *, const float *, const float *, float, float, float *);
void lqo_fold(int8_t *, float *, float *, int, int32_t *, float *, int, const float *, const float *, const float *,
              int, float);
void lqo_current(const int8_t *, const float *, const float *, int, const int32_t *, const float *, int,
                 const float *, const float *, const float *, float *);
void lqo_boundary(const int8_t *, const float *, const float *, int, const int32_t *, const float *, float *);
void lqo_residual(const int8_t *, const float *, const float *, float *);
void lqo_init_r1(const float *, int, int, float, int8_t *, float *, float *, int32_t *, float *);
void lqo_append_r1(const int8_t *, const float *, const float *, int, const int32_t *, const float *, int, float *,
                   float *, float *, const float *, const float *, const float *, float, float, float *);
void lqo_fold_r1(int8_t *, float *, float *, int, int32_t *, float *, int, const float *, const float *,
                 const float *, int, float);
void lqo_current_r1(const int8_t *, const float *, const float *, int, const float *, int, const float *,
                    const float *, const float *, float *);
void lqo_init_block(const float *, int, int, float, int8_t *, float *, float *, int32_t *, float *);
void lqo_fold_block(int8_t *, float *, float *, int, int32_t *, float *, int, const float *, const float *,
                    const float *, int, float);
void lqo_append_kda(const int8_t *, const float *, const float *, int, const int32_t *, const float *, int, float *,
                    float *, float *, const float *, const float *, const float *, const float *, float, float *);
void lqo_fold_kda(int8_t *, float *, float *, int, int32_t *, float *, int, const float *, const float *,
                  const float *, int, float);
void lqo_current_kda(const int8_t *, const float *, const float *, int, const int32_t *, const float *, int,
                     const float *, const float *, const float *, float *);
void lqo_quantize_keyrow(float *, int, int, float, int8_t *, float *, float *, int32_t *, float *);
void lqo_boundary_keyrow(const int8_t *, const float *, const float *, int, const int32_t *, const float *, float *);
void lqo_gate(float, float, float, float, float *, float *);
void lqo_l2norm(const float *, float, float, float *);
void lqo_gdn_step_f32(float *, const float *, const float *, const float *, float, float, float *, float *);
void lqo_gdn_step_f64(double *, const double *, const double *, const double *, double, double, double *,
                      double *);
void lqo_gdn_step_bf16(uint16_t *, const float *, const float *, const float *, float, float, float *, float *);
void lqo_kda_step_f32(float *, const float *, const float *, const float *, const float *, float, float *, float *);
uint16_t lqo_f32_to_bf16(float);
void lqo_round_bf16(float *, int);
uint8_t lqo_f32_to_e4m3(float);
float lqo_e4m3_to_f32(uint8_t);
void lqo_round_fp8_record(float *);
float lqo_t128_sum(const float *);
float lqo_t128_dot(const float *, const float *);
}

static int failures = 0;
#define CHECK(cond)                                                           \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static const int D = 128;

// ------------------------------------------------------------------ inputs
static uint64_t rng_state = 0x243F6A8885A308D3ull;
static double unif()
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}
static float gauss()
{
    double u1 = unif(), u2 = unif();
    if (u1 < 1e-300) u1 = 1e-300;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}
static void unit(float *x)
{
    double s = 0;
    for (int i = 0; i < D; ++i) {
        x[i] = gauss();
        s += (double)x[i] * x[i];
    }
    for (int i = 0; i < D; ++i) x[i] = (float)(x[i] / sqrt(s));
}
static void state(float *S, int outliers)
{
    for (int e = 0; e < D * D; ++e) S[e] = 0.02f * gauss();
    for (int j = 0; j < outliers; ++j) {
        int r = (int)(unif() * D), c = (int)(unif() * D);
        for (int i = 0; i < D; ++i) {
            S[r * D + i] *= 50.0f;
            S[i * D + c] *= 50.0f;
        }
    }
}

// ------------------------------------------------------------------ part 1: the C ABI
struct Buf {
    void *p = nullptr;
    explicit Buf(size_t n) { p = aligned_alloc(256, (n + 255) / 256 * 256 + 256); }
    ~Buf() { free(p); }
};

static leapq_config cfg_of(int batch, int heads, int W, int C)
{
    leapq_config c;
    memset(&c, 0, sizeof c);
    c.batch = batch;
    c.heads = heads;
    c.dk = c.dv = D;
    c.window = W;
    c.n_comp = C;
    c.smoothing = 1;
    c.sigma_floor = 1e-6f;
    c.in_dtype = LEAPQ_F32;
    return c;
}

static void abi_layer(const leapq_config &cfg)
{
    leapq_layout lay;
    CHECK(leapq_query_layout(&cfg, &lay) == LEAPQ_OK);
    CHECK(lay.total_bytes > 0 && lay.off_codes == 0);
    CHECK(lay.off_row_scale % 256 == 0 && lay.off_rec_u % 256 == 0);
    Buf st(lay.total_bytes);
    const int H = cfg.batch * cfg.heads;
    Buf tok(8 * (size_t)H * D), out(4 * (size_t)H * D * D);
    float *t = (float *)tok.p;
    const void *q = t, *k = t + H * D, *v = t + 2 * H * D;
    const float *al = t + 3 * H * D, *be = t + 4 * H * D;
    float *o = t + 5 * H * D;
    leapq_layer L;
    memset(&L, 0, sizeof L);
    L.cfg = cfg;
    L.state = st.p;
    CHECK(leapq_init_state(&L, (const float *)out.p, nullptr) == LEAPQ_OK && L.n_records == 0);
    CHECK(leapq::stub_heads == H);
    CHECK(leapq_init_state(&L, nullptr, nullptr) == LEAPQ_ERR_NULL);
    int before = leapq::stub_calls;
    CHECK(leapq_append(&L, nullptr, k, v, al, be, o, nullptr) == LEAPQ_ERR_NULL);
    CHECK(leapq_append(&L, (const char *)q + 4, k, v, al, be, o, nullptr) == LEAPQ_ERR_ALIGN);
    CHECK(leapq_append(&L, q, k, v, al, be, nullptr, nullptr) == LEAPQ_ERR_NULL);
    CHECK(leapq::stub_calls == before && L.n_records == 0);
    for (int n = 0; n < cfg.window; ++n) {
        CHECK(leapq_append(&L, q, k, v, al, be, o, nullptr) == LEAPQ_OK);
        CHECK(L.n_records == n + 1 && leapq::stub_n == n);
    }
    before = leapq::stub_calls;
    CHECK(leapq_append(&L, q, k, v, al, be, o, nullptr) == LEAPQ_ERR_WINDOW_FULL);
    CHECK(leapq::stub_calls == before && L.n_records == cfg.window);
    CHECK(leapq_dequant(&L, 2, (float *)out.p, nullptr) == LEAPQ_OK);
    CHECK(leapq_dequant(&L, 3, (float *)out.p, nullptr) == LEAPQ_ERR_RANGE);
    CHECK(leapq_fold(&L, nullptr) == LEAPQ_OK && L.n_records == 0);
    for (int n = 0; n + 1 < cfg.window; ++n) CHECK(leapq_append(&L, q, k, v, al, be, o, nullptr) == LEAPQ_OK);
    if (cfg.window >= 2) CHECK(leapq_fold(&L, nullptr) == LEAPQ_OK && L.n_records == 0);
    CHECK(leapq_append_fold(&L, q, k, v, al, be, o, nullptr) == (cfg.window == 1 ? LEAPQ_OK : LEAPQ_ERR_RANGE));
    L.n_records = 0;
    for (int n = 0; n + 1 < cfg.window; ++n) CHECK(leapq_append(&L, q, k, v, al, be, o, nullptr) == LEAPQ_OK);
    CHECK(leapq_append_fold(&L, q, k, v, al, be, o, nullptr) == LEAPQ_OK && L.n_records == 0);
    // misaligned state, bad record count, reserved fields
    leapq_layer bad = L;
    bad.state = (char *)st.p + 16;
    CHECK(leapq_fold(&bad, nullptr) == LEAPQ_ERR_ALIGN);
    bad = L;
    bad.n_records = cfg.window + 1;
    CHECK(leapq_fold(&bad, nullptr) == LEAPQ_ERR_RANGE);
    bad = L;
    bad.cfg.reserved[1] = 7;
    CHECK(leapq_fold(&bad, nullptr) == LEAPQ_ERR_RANGE);
    // gated entry points
    leapq_gate g;
    memset(&g, 0, sizeof g);
    g.A_log = al;
    g.dt_bias = be;
    g.q_scale = 0.088f;
    g.norm_eps = 1e-6f;
    L.n_records = 0;
    const bool gated_ok = cfg.decay == LEAPQ_DECAY_SCALAR && cfg.comp_fit == LEAPQ_COMP_LINES &&
                          cfg.rec_dtype == LEAPQ_F32;
    CHECK(leapq_append_gated(&L, nullptr, q, k, v, al, be, o, nullptr) == LEAPQ_ERR_NULL);
    if (gated_ok) {
        g.norm_eps = -1.0f;
        CHECK(leapq_append_gated(&L, &g, q, k, v, al, be, o, nullptr) == LEAPQ_ERR_RANGE);
        g.norm_eps = 1e-6f;
        CHECK(leapq_append_gated(&L, &g, q, k, v, al, be, o, nullptr) == LEAPQ_OK && L.n_records == 1);
    } else {
        CHECK(leapq_append_gated(&L, &g, q, k, v, al, be, o, nullptr) == LEAPQ_ERR_RANGE && L.n_records == 0);
    }
    // per-request phases
    Buf nin(4 * (size_t)cfg.batch), nout(4 * (size_t)cfg.batch);
    memset(nin.p, 0, 4 * (size_t)cfg.batch);
    const int32_t st_ok = cfg.window <= 16 ? LEAPQ_OK : LEAPQ_ERR_RANGE;
    CHECK(leapq_step(&L, nullptr, (const int32_t *)nin.p, (int32_t *)nout.p, q, k, v, al, be, o, nullptr) == st_ok);
    CHECK(leapq_step(&L, nullptr, (const int32_t *)nin.p, (int32_t *)nin.p, q, k, v, al, be, o, nullptr) ==
          LEAPQ_ERR_RANGE || cfg.window > 16);
    // dense baselines
    CHECK(leapq_gdn_decode(&cfg, LEAPQ_F32, out.p, q, k, v, al, be, o, nullptr) == LEAPQ_OK);
    CHECK(leapq_gdn_decode(&cfg, 7, out.p, q, k, v, al, be, o, nullptr) == LEAPQ_ERR_DTYPE);
    CHECK(leapq_gdn_decode(&cfg, LEAPQ_BF16, nullptr, q, k, v, al, be, o, nullptr) == LEAPQ_ERR_NULL);
}

static void part_abi()
{
    const int Ws[] = {1, 5, 16, 20, 64};
    const int Cs[] = {0, 1, 4, 8};
    for (int W : Ws)
        for (int C : Cs) {
            leapq_config c = cfg_of(2, 3, W, C);
            abi_layer(c);
            c.in_dtype = LEAPQ_BF16;
            abi_layer(c);
            if (C <= 4) {
                c.comp_fit = LEAPQ_COMP_RANK1;
                abi_layer(c);
                c.comp_fit = LEAPQ_COMP_BLOCK;
                abi_layer(c);
                c.comp_fit = LEAPQ_COMP_LINES;
            }
            c.in_dtype = LEAPQ_F32;
            c.decay = LEAPQ_DECAY_CHANNEL;
            abi_layer(c);
            c.decay = LEAPQ_DECAY_SCALAR;
            c.rec_dtype = LEAPQ_BF16;
            abi_layer(c);
            c.rec_dtype = LEAPQ_FP8;
            abi_layer(c);
        }
    // invalid configurations
    leapq_layout lay;
    leapq_config c = cfg_of(1, 1, 16, 4);
    CHECK(leapq_query_layout(nullptr, &lay) == LEAPQ_ERR_NULL);
    CHECK(leapq_query_layout(&c, nullptr) == LEAPQ_ERR_NULL);
    const struct {
        int field, value;
        int32_t status;
    } bad[] = {{0, 0, LEAPQ_ERR_RANGE}, {1, -1, LEAPQ_ERR_RANGE}, {2, 64, LEAPQ_ERR_SHAPE},
               {4, 0, LEAPQ_ERR_RANGE}, {4, 65, LEAPQ_ERR_RANGE}, {5, 9, LEAPQ_ERR_RANGE},
               {5, -1, LEAPQ_ERR_RANGE}, {6, 2, LEAPQ_ERR_RANGE}, {8, 3, LEAPQ_ERR_DTYPE}};
    for (const auto &b : bad) {
        leapq_config x = c;
        int32_t *f = (int32_t *)&x;
        f[b.field] = b.value;
        CHECK(leapq_query_layout(&x, &lay) == b.status);
    }
    c.sigma_floor = 0.0f;
    CHECK(leapq_query_layout(&c, &lay) == LEAPQ_ERR_RANGE);
    c.sigma_floor = NAN;
    CHECK(leapq_query_layout(&c, &lay) == LEAPQ_ERR_RANGE);
    c = cfg_of(65536, 32768, 16, 4);
    CHECK(leapq_query_layout(&c, &lay) == LEAPQ_ERR_RANGE);
    for (int s = -8; s <= 1; ++s) CHECK(leapq_status_str(s) != nullptr);
    CHECK(leapq_version() > 0);
}

// ------------------------------------------------------------------ part 2: the oracle
struct Head {
    int C, W;
    std::vector<int8_t> Q = std::vector<int8_t>(D * D);
    std::vector<float> rho = std::vector<float>(D), sig = std::vector<float>(D);
    std::vector<int32_t> idx;
    std::vector<float> vec, gam, rk, ru;
    Head(int C_, int W_, int vw, int gw) : C(C_), W(W_), idx(C_ > 0 ? C_ : 1), vec((C_ > 0 ? C_ : 1) * vw * D),
                                           gam(W_ * gw), rk(W_ * D), ru(W_ * D) {}
};

static bool finite(const float *x, int n)
{
    for (int i = 0; i < n; ++i)
        if (!isfinite(x[i])) return false;
    return true;
}

static void window_tokens(int T, std::vector<float> &tq, std::vector<float> &tk, std::vector<float> &tv,
                          std::vector<float> &ta, std::vector<float> &tb, bool channel)
{
    tq.resize(T * D);
    tk.resize(T * D);
    tv.resize(T * D);
    ta.resize(T * (channel ? D : 1));
    tb.resize(T);
    for (int t = 0; t < T; ++t) {
        unit(&tq[t * D]);
        unit(&tk[t * D]);
        for (int i = 0; i < D; ++i) tv[t * D + i] = gauss();
        for (int i = 0; i < (channel ? D : 1); ++i) {
            double z = gauss() - 3.0;
            ta[t * (channel ? D : 1) + i] = (float)exp(-(z > 0 ? z + log1p(exp(-z)) : log1p(exp(z))));
        }
        tb[t] = (float)(1.0 / (1.0 + exp(-gauss())));
    }
}

static void part_oracle()
{
    std::vector<float> S(D * D), out(D * D), o(D), u(D);
    std::vector<float> tq, tk, tv, ta, tb;
    const int W = 16, T = 2 * W;
    for (int variant = 0; variant < 4; ++variant) {  // lines C = 8, lines C = 0, rank-one, block
        const int C = variant == 0 ? 8 : variant == 1 ? 0 : 4;
        const bool pairs = variant >= 2;
        Head h(C, W, pairs ? 2 : 1, 1);
        state(S.data(), 3);
        if (variant == 2)
            lqo_init_r1(S.data(), C, 1, 1e-6f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(), h.vec.data());
        else if (variant == 3)
            lqo_init_block(S.data(), C, 1, 1e-6f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(),
                           h.vec.data());
        else
            lqo_init(S.data(), C, variant == 0, 1e-6f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(),
                     h.vec.data());
        window_tokens(T, tq, tk, tv, ta, tb, false);
        int n = 0;
        for (int t = 0; t < T; ++t) {
            if (pairs)
                lqo_append_r1(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), n,
                              h.gam.data(), h.rk.data(), h.ru.data(), &tq[t * D], &tk[t * D], &tv[t * D], ta[t],
                              tb[t], o.data());
            else
                lqo_append(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), n,
                           h.gam.data(), h.rk.data(), h.ru.data(), &tq[t * D], &tk[t * D], &tv[t * D], ta[t], tb[t],
                           o.data());
            ++n;
            CHECK(finite(o.data(), D));
            if (n == W) {
                if (pairs)
                    lqo_current_r1(h.Q.data(), h.rho.data(), h.sig.data(), C, h.vec.data(), n, h.gam.data(),
                                   h.rk.data(), h.ru.data(), out.data());
                else
                    lqo_current(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), n,
                                h.gam.data(), h.rk.data(), h.ru.data(), out.data());
                CHECK(finite(out.data(), D * D));
                if (variant == 2)
                    lqo_fold_r1(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), n,
                                h.gam.data(), h.rk.data(), h.ru.data(), 1, 1e-6f);
                else if (variant == 3)
                    lqo_fold_block(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), n,
                                   h.gam.data(), h.rk.data(), h.ru.data(), 1, 1e-6f);
                else
                    lqo_fold(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), n,
                             h.gam.data(), h.rk.data(), h.ru.data(), variant == 0, 1e-6f);
                n = 0;
            }
        }
        if (!pairs) {
            lqo_boundary(h.Q.data(), h.rho.data(), h.sig.data(), C, h.idx.data(), h.vec.data(), out.data());
            lqo_residual(h.Q.data(), h.rho.data(), h.sig.data(), out.data());
            CHECK(finite(out.data(), D * D));
        }
    }
    {  // per-channel decay
        Head h(4, W, 1, D);
        state(S.data(), 2);
        lqo_init(S.data(), 4, 1, 1e-6f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(), h.vec.data());
        window_tokens(T, tq, tk, tv, ta, tb, true);
        int n = 0;
        for (int t = 0; t < T; ++t) {
            lqo_append_kda(h.Q.data(), h.rho.data(), h.sig.data(), 4, h.idx.data(), h.vec.data(), n, h.gam.data(),
                           h.rk.data(), h.ru.data(), &tq[t * D], &tk[t * D], &tv[t * D], &ta[t * D], tb[t], o.data());
            CHECK(finite(o.data(), D));
            if (++n == W) {
                lqo_current_kda(h.Q.data(), h.rho.data(), h.sig.data(), 4, h.idx.data(), h.vec.data(), n,
                                h.gam.data(), h.rk.data(), h.ru.data(), out.data());
                lqo_fold_kda(h.Q.data(), h.rho.data(), h.sig.data(), 4, h.idx.data(), h.vec.data(), n,
                             h.gam.data(), h.rk.data(), h.ru.data(), 1, 1e-6f);
                n = 0;
            }
        }
        std::vector<float> Sk(D * D), al(D);
        state(Sk.data(), 1);
        for (int i = 0; i < D; ++i) al[i] = 0.9f + 0.1f * (float)unif();
        lqo_kda_step_f32(Sk.data(), &tq[0], &tk[0], &tv[0], al.data(), 0.5f, u.data(), o.data());
        CHECK(finite(o.data(), D));
    }
    {  // key-row smoothing study, zero and tiny states
        Head h(4, W, 1, 1);
        state(S.data(), 3);
        std::vector<float> R = S;
        lqo_quantize_keyrow(R.data(), 4, 1, 1e-6f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(),
                            h.vec.data());
        lqo_boundary_keyrow(h.Q.data(), h.rho.data(), h.sig.data(), 4, h.idx.data(), h.vec.data(), out.data());
        CHECK(finite(out.data(), D * D));
        std::fill(S.begin(), S.end(), 0.0f);
        lqo_init(S.data(), 4, 1, 1e-6f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(), h.vec.data());
        CHECK(h.idx[0] == -1 && h.rho[0] == 0.0f);
        for (int e = 0; e < D * D; ++e) S[e] = ldexpf(gauss(), -130);
        lqo_init(S.data(), 4, 1, 1e-30f, h.Q.data(), h.rho.data(), h.sig.data(), h.idx.data(), h.vec.data());
        CHECK(finite(h.sig.data(), D));
    }
    {  // gates, norms, dense steps, bf16
        float a, b;
        lqo_gate(0.3f, -0.2f, 1.5f, -4.0f, &a, &b);
        CHECK(a > 0.0f && a < 1.0f && b > 0.0f && b < 1.0f);
        lqo_gate(80.0f, 80.0f, 2.7f, 10.0f, &a, &b);
        CHECK(a >= 0.0f && b <= 1.0f);
        std::vector<float> x(D), y(D);
        unit(x.data());
        lqo_l2norm(x.data(), 1e-6f, 0.088f, y.data());
        CHECK(finite(y.data(), D));
        state(S.data(), 0);
        lqo_gdn_step_f32(S.data(), x.data(), y.data(), x.data(), 0.9f, 0.5f, u.data(), o.data());
        std::vector<double> Sd(D * D), xd(D), od(D), ud(D);
        for (int i = 0; i < D; ++i) xd[i] = x[i];
        lqo_gdn_step_f64(Sd.data(), xd.data(), xd.data(), xd.data(), 0.9, 0.5, ud.data(), od.data());
        std::vector<uint16_t> Sb(D * D);
        for (int e = 0; e < D * D; ++e) Sb[e] = lqo_f32_to_bf16(S[e]);
        lqo_gdn_step_bf16(Sb.data(), x.data(), y.data(), x.data(), 0.9f, 0.5f, u.data(), o.data());
        CHECK(lqo_f32_to_bf16(1.0f) == 0x3f80 && lqo_f32_to_bf16(-0.0f) == 0x8000);
        lqo_round_bf16(x.data(), D);
        for (int c = 0; c < 256; ++c)
            if ((c & 0x7f) != 0x7f) CHECK(lqo_f32_to_e4m3(lqo_e4m3_to_f32((uint8_t)c)) == (uint8_t)c);
        std::vector<float> rec(D);
        for (int i = 0; i < D; ++i) rec[i] = ldexpf(gauss(), (i % 7) * 9 - 30);
        lqo_round_fp8_record(rec.data());
        CHECK(finite(rec.data(), D));
        const float sx = lqo_t128_sum(x.data()), dxy = lqo_t128_dot(x.data(), y.data());
        CHECK(isfinite(sx) && isfinite(dxy));
    }
}

int main()
{
    part_abi();
    part_oracle();
    printf("sanitizer driver: %d failed checks, %d launches reached the stubs\n", failures, leapq::stub_calls);
    return failures == 0 ? 0 : 1;
}
