// Private to libleapq: the per-layer view of a state buffer passed to the
// kernels, and the launchers the C ABI calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace leapq {

// Section base pointers of one layer's state buffer (see leapq_layout).
struct StateView {
    int8_t *codes;
    float *rho;
    float *sigma;
    int32_t *cidx;
    float *cvec;
    float *rgam;
    void *rk;  // record keys in the input dtype (fp32 or bf16)
    void *ru;  // record corrections (fp32, bf16 with u_bf16, fp8 codes and scales with u_fp8)
    int C;  // compensator lines per head
    int W;  // record slots per head
    int key_bf16;  // record keys (and inputs) are bf16
    int kda;       // per-channel decay: alpha [heads][128], record decays [W][128]
    int u_bf16;    // record corrections stored in bf16
    int u_fp8;     // record corrections stored as E4M3 codes with 4 power-of-two scales
    int u_rec_bytes;  // bytes of one record's corrections: 512 (fp32), 256 (bf16), 144 (fp8)
    int r1;        // compensator pairs [C][2][128] (a, b) in place of lines
    int blk;       // the pairs are fitted as a block (with r1)
    int cbits;       // bits per residual code: 8, 6 or 4
    int code_bytes;  // bytes of one head's codes: 16384, 12288 or 8192
};

// Gate arithmetic in front of the append (mode 0: alpha and beta are given;
// LEAPQ_GATE_*: they are computed from the raw projections, and q and k
// are L2-normalized when `normalize`).
struct GateArgs {
    const float *A_log;    // [heads] per model head
    const float *dt_bias;  // [heads]
    float q_scale;
    float eps;
    int heads;  // model heads per request: head h uses parameters h % heads
    int gated;
    int normalize;
};

hipError_t launch_init(const StateView &sv, int heads, const float *S0, int smoothing, float floor_,
                       hipStream_t s);
hipError_t launch_fold(const StateView &sv, int heads, int n, int smoothing, float floor_, hipStream_t s);
hipError_t launch_dequant(const StateView &sv, int heads, int n, int what, float *out, hipStream_t s);
hipError_t launch_append(const StateView &sv, int heads, int n, int bf16, const void *q, const void *k,
                         const void *v, const float *alpha, const float *beta, float *o, const GateArgs &g,
                         hipStream_t s);
// The window's last append and the fold in one launch; requires n + 1 == W
// and W <= 16 (the records fit one LDS chunk).
hipError_t launch_append_fold(const StateView &sv, int heads, int n, int bf16, const void *q, const void *k,
                              const void *v, const float *alpha, const float *beta, float *o, int smoothing,
                              float floor_, const GateArgs &g, hipStream_t s);
hipError_t launch_step(const StateView &sv, int heads, int heads_per_req, const int *n_in, int *n_out, int bf16,
                       const void *q, const void *k, const void *v, const float *alpha, const float *beta, float *o,
                       int smoothing, float floor_, const GateArgs &g, hipStream_t s);
hipError_t launch_gdn_decode(int heads, int state_bf16, int in_bf16, int kda, void *S, const void *q, const void *k,
                             const void *v, const float *alpha, const float *beta, float *o, hipStream_t s);

}  // namespace leapq
