// Append: one decode token for every head of a layer.
//
// Method: "Recurrent-state quantization for linear attention: a first GPU
// kernel" (Background: decay, read with the key, correction, rank-one write,
// read the output; What we built: the append adds one record and computes
// the output) and "LeapQuant: Efficient Linear Attention with Accurate
// Recurrent State Quantization" (B.2: reads never form the dense state; B.3:
// the residual's scales act on the residual read only, records and
// compensator tokens are added to it).  With n records in the window, token
// t = n+1:
//   gamma_t = gamma_n * alpha,  c_i = gamma_t / gamma_i
//   Bx[c] = sigma_c * T(sum_r (x_r * rho_r) * code[r][c])   (x = k, q)
//           then, per compensator in order: a row token r adds fma(x_r,
//           line[c], .), a column token c' adds T(line . x) to column c'
//   r = gamma_t * Bk, then fma(c_i * T(k_i . k), u_i, r) over the records
//   u_t = beta * (v - r)
//   o = gamma_t * Bq, then fma(c_i * T(k_i . q), u_i, o), then fma(T(k . q), u_t, o)
// (T = the canonical 128-term tree) and the record (gamma_t, k, u_t) is
// stored at slot n.
//
// Memory: every per-head operand but the codes (records, compensator lines,
// rho and sigma, k, q, v, the compensator indices and the record decays) is
// copied straight into LDS by a few LDS-direct loads per wave; then each
// thread loads its 64 codes as four 16-byte loads (1 KB contiguous per wave
// and load).  Once the copies have landed the per-head dot products run
// while the codes are still in flight; the residual read is then reduced
// inside each wave (thread map of leapq_device.h) and finished per column.
#include "leapq_append_dev.h"

namespace leapq {
namespace {
using namespace dev;

template <typename T, typename K, bool GATED, bool NORM, bool CH, typename U, bool R1, int CB = 8>
__global__ __launch_bounds__(NT) void k_append(StateView sv, int n, const T *__restrict__ qin,
                                                const T *__restrict__ kin, const T *__restrict__ vin,
                                                const float *__restrict__ alpha, const float *__restrict__ beta,
                                                float *__restrict__ o, GateArgs g)
{
    extern __shared__ float dsm[];
    const MMap a = mmap();
    const int h = blockIdx.x;
    const HeadLds<T, K, CH, U, R1> L(dsm, n, sv.C);
    float *dots = dsm + head_lds_floats<T, K, CH, U, R1>(n, sv.C);
    uint4 qc[4];
    append_issue<T, K, CH, U, R1, CB>(sv, n, h, qin, kin, vin, a, L, qc, alpha);
    float a_h = CH ? 1.0f : sload(alpha, h);  // with CH the decay vector is staged in LDS
    float b_h = sload(beta, h);
    if constexpr (GATED) gate_issue(g, h, a, a_h, b_h, dots);
    wait_lds_copies<CodeFmt<CB>::loads>();
    lds_barrier();
    if constexpr (GATED) {
        a_h = dots[kGateSlot];
        b_h = dots[kGateSlot + 1];
    }
    append_compute<T, K, false, NORM, CH, U, R1, CB>(sv, n, h, a, L, dots, qc, a_h, b_h, o, g.q_scale, g.eps);
}

}  // namespace

template <typename T, typename K, bool GATED, bool NORM, bool CH = false, typename U = float, bool R1 = false,
          int CB = 8>
static void launch_append_t(const StateView &sv, int heads, int n, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, float *o, const GateArgs &g, hipStream_t s)
{
    const size_t lds = sizeof(float) * (head_lds_floats<T, K, CH, U, R1>(n, sv.C) + kDotFloats);
    hipLaunchKernelGGL((k_append<T, K, GATED, NORM, CH, U, R1, CB>), dim3(heads), dim3(NT), lds, s, sv, n,
                       (const T *)q, (const T *)k, (const T *)v, alpha, beta, o, g);
}

hipError_t launch_append(const StateView &sv, int heads, int n, int bf16, const void *q, const void *k,
                         const void *v, const float *alpha, const float *beta, float *o, const GateArgs &g,
                         hipStream_t s)
{
    // (inputs, keys): (fp32, fp32), (bf16, bf16), or (bf16, fp32) for a layer
    // whose keys are fp32 because its gated appends normalize k; per-channel
    // decay comes with keys in the input dtype and no gates
    const bool kb = sv.key_bf16;
    if (sv.cbits != 8) {  // 6- or 4-bit codes: scalar decay, lines, fp32 corrections, keys in the input dtype, no gates
        if (sv.cbits == 6) {
            if (!bf16)
                launch_append_t<float, float, false, false, false, float, false, 6>(sv, heads, n, q, k, v, alpha, beta,
                                                                                 o, g, s);
            else
                launch_append_t<uint16_t, uint16_t, false, false, false, float, false, 6>(sv, heads, n, q, k, v, alpha,
                                                                                       beta, o, g, s);
        } else {
            if (!bf16)
                launch_append_t<float, float, false, false, false, float, false, 4>(sv, heads, n, q, k, v, alpha, beta,
                                                                                 o, g, s);
            else
                launch_append_t<uint16_t, uint16_t, false, false, false, float, false, 4>(sv, heads, n, q, k, v, alpha,
                                                                                       beta, o, g, s);
        }
    } else if (sv.r1) {  // rank-one compensators: scalar decay, fp32 corrections, keys in the input dtype, no gates
        if (!bf16)
            launch_append_t<float, float, false, false, false, float, true>(sv, heads, n, q, k, v, alpha, beta, o, g,
                                                                          s);
        else
            launch_append_t<uint16_t, uint16_t, false, false, false, float, true>(sv, heads, n, q, k, v, alpha, beta,
                                                                                o, g, s);
    } else if (sv.u_bf16) {  // lossy bf16 corrections: scalar decay, keys in the input dtype, no gates
        if (!bf16)
            launch_append_t<float, float, false, false, false, uint16_t>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
        else
            launch_append_t<uint16_t, uint16_t, false, false, false, uint16_t>(sv, heads, n, q, k, v, alpha, beta, o,
                                                                             g, s);
    } else if (sv.u_fp8) {  // lossy fp8 corrections: as bf16 ones
        if (!bf16)
            launch_append_t<float, float, false, false, false, Fp8>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
        else
            launch_append_t<uint16_t, uint16_t, false, false, false, Fp8>(sv, heads, n, q, k, v, alpha, beta, o, g,
                                                                        s);
    } else if (sv.kda) {
        if (!bf16)
            launch_append_t<float, float, false, false, true>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
        else
            launch_append_t<uint16_t, uint16_t, false, false, true>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
    } else if (!g.gated) {
        if (!bf16)
            launch_append_t<float, float, false, false>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
        else if (kb)
            launch_append_t<uint16_t, uint16_t, false, false>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
        else
            launch_append_t<uint16_t, float, false, false>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
    } else if (!bf16) {
        if (g.normalize)
            launch_append_t<float, float, true, true>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
        else
            launch_append_t<float, float, true, false>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
    } else if (kb) {
        launch_append_t<uint16_t, uint16_t, true, false>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
    } else if (g.normalize) {
        launch_append_t<uint16_t, float, true, true>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
    } else {
        launch_append_t<uint16_t, float, true, false>(sv, heads, n, q, k, v, alpha, beta, o, g, s);
    }
    return hipGetLastError();
}

}  // namespace leapq
