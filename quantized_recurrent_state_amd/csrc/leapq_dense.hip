// Dense per-token Gated DeltaNet decode: the fp32-state and bf16-state
// baselines the quantized path is compared with, in place on the state.
//
// One token ("Recurrent-state quantization for linear attention: a first GPU
// kernel", Background; "LeapQuant: Efficient Linear Attention with Accurate
// Recurrent State Quantization", App. A with D_t = alpha I, or D_t =
// Diag(alpha) per key row for per-channel decay (CH), and b_t = beta):
//   S = D_t S;  r = S^T k;  u = beta (v - r);  S = S + k u^T;  o = S^T q
// with S[r][c] indexed (key row, value column).  A bf16 state is widened,
// updated in fp32 and rounded to nearest even on store.  The reads are
// canonical-tree dot products over the rows; the update is one fma per
// entry.  A bf16 state is stored with the hardware round-to-nearest-even
// conversion.
//
// Thread map: rows i + 32p as in leapq_device.h, but the 16 columns of a
// thread are contiguous (16 j + m) to match the natural state layout.
#include "leapq_device.h"

namespace leapq {
namespace {
using namespace dev;

template <typename TS>
__device__ __forceinline__ void load_row16(const TS *p, float (&x)[16]);
template <>
__device__ __forceinline__ void load_row16<float>(const float *p, float (&x)[16])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float4 v = reinterpret_cast<const float4 *>(p)[d];
        x[4 * d] = v.x;
        x[4 * d + 1] = v.y;
        x[4 * d + 2] = v.z;
        x[4 * d + 3] = v.w;
    }
}
template <>
__device__ __forceinline__ void load_row16<uint16_t>(const uint16_t *p, float (&x)[16])
{
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const uint4 v = reinterpret_cast<const uint4 *>(p)[d];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            x[8 * d + 2 * b] = bf16_to_f32((uint16_t)(w4[b] & 0xffffu));
            x[8 * d + 2 * b + 1] = bf16_to_f32((uint16_t)(w4[b] >> 16));
        }
    }
}
template <typename TS>
__device__ __forceinline__ void store_row16(TS *p, const float (&x)[16]);
template <>
__device__ __forceinline__ void store_row16<float>(float *p, const float (&x)[16])
{
#pragma unroll
    for (int d = 0; d < 4; ++d)
        reinterpret_cast<float4 *>(p)[d] = make_float4(x[4 * d], x[4 * d + 1], x[4 * d + 2], x[4 * d + 3]);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even as packed bf16 (one
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <>
__device__ __forceinline__ void store_row16<uint16_t>(uint16_t *p, const float (&x)[16])
{
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        uint32_t w4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) w4[b] = pack_bf16x2(x[8 * d + 2 * b], x[8 * d + 2 * b + 1]);
        reinterpret_cast<uint4 *>(p)[d] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
}

template <typename TS, typename TI, bool CH>
__global__ __launch_bounds__(NT) void k_gdn_decode(TS *__restrict__ Sg, const TI *__restrict__ qin,
                                                    const TI *__restrict__ kin, const TI *__restrict__ vin,
                                                    const float *__restrict__ alpha,
                                                    const float *__restrict__ beta, float *__restrict__ o)
{
    __shared__ float uc[D];
    const AMap a = amap();
    const int l = a.l;
    const int h = blockIdx.x;
    TS *Sh = Sg + (size_t)h * D * D;
    const TI *qh = qin + (size_t)h * D, *kh = kin + (size_t)h * D;
    float S[4][16], kr[4], qr[4], al[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        al[p] = CH ? alpha[(size_t)h * D + a.row(p)] : alpha[h];
        kr[p] = ld_in<TI>(kh, a.row(p));
        qr[p] = ld_in<TI>(qh, a.row(p));
        load_row16<TS>(Sh + a.row(p) * D + 16 * a.j, S[p]);
    }
    const int c = 16 * a.j + colm_of(l);
    const float vc = ld_in<TI>(vin + (size_t)h * D, c);
    const float bt = beta[h];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = al[p] * S[p][m];
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        v[m] = fma_(S[0][m], kr[0], S[2][m] * kr[2]) + fma_(S[1][m], kr[1], S[3][m] * kr[3]);
    const float rc = colsum16(v, l);
    if ((l & 1) == 0) uc[c] = bt * (vc - rc);
    __syncthreads();
    float u[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float4 uu = reinterpret_cast<const float4 *>(uc + 16 * a.j)[d];
        u[4 * d] = uu.x;
        u[4 * d + 1] = uu.y;
        u[4 * d + 2] = uu.z;
        u[4 * d + 3] = uu.w;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int m = 0; m < 16; ++m) S[p][m] = fma_(kr[p], u[m], S[p][m]);
#pragma unroll
    for (int m = 0; m < 16; ++m)
        v[m] = fma_(S[0][m], qr[0], S[2][m] * qr[2]) + fma_(S[1][m], qr[1], S[3][m] * qr[3]);
    const float oc = colsum16(v, l);
    if ((l & 1) == 0) o[(size_t)h * D + c] = oc;
#pragma unroll
    for (int p = 0; p < 4; ++p) store_row16<TS>(Sh + a.row(p) * D + 16 * a.j, S[p]);
}

}  // namespace

template <bool CH>
static void launch_gdn_t(int heads, int state_bf16, int in_bf16, void *S, const void *q, const void *k,
                         const void *v, const float *alpha, const float *beta, float *o, hipStream_t s)
{
    if (state_bf16) {
        if (in_bf16)
            hipLaunchKernelGGL((k_gdn_decode<uint16_t, uint16_t, CH>), dim3(heads), dim3(NT), 0, s, (uint16_t *)S,
                               (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, beta, o);
        else
            hipLaunchKernelGGL((k_gdn_decode<uint16_t, float, CH>), dim3(heads), dim3(NT), 0, s, (uint16_t *)S,
                               (const float *)q, (const float *)k, (const float *)v, alpha, beta, o);
    } else {
        if (in_bf16)
            hipLaunchKernelGGL((k_gdn_decode<float, uint16_t, CH>), dim3(heads), dim3(NT), 0, s, (float *)S,
                               (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, beta, o);
        else
            hipLaunchKernelGGL((k_gdn_decode<float, float, CH>), dim3(heads), dim3(NT), 0, s, (float *)S,
                               (const float *)q, (const float *)k, (const float *)v, alpha, beta, o);
    }
}

hipError_t launch_gdn_decode(int heads, int state_bf16, int in_bf16, int kda, void *S, const void *q, const void *k,
                             const void *v, const float *alpha, const float *beta, float *o, hipStream_t s)
{
    if (kda)
        launch_gdn_t<true>(heads, state_bf16, in_bf16, S, q, k, v, alpha, beta, o, s);
    else
        launch_gdn_t<false>(heads, state_bf16, in_bf16, S, q, k, v, alpha, beta, o, s);
    return hipGetLastError();
}

}  // namespace leapq
