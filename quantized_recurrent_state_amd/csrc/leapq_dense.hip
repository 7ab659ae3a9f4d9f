// Dense per-token Gated DeltaNet decode: the fp32-state and bf16-state
// baselines the quantized path is compared with, in place on the state.
//
// One token ("Recurrent-state quantization for linear attention: a first GPU
// kernel", Background; "LeapQuant: Efficient Linear Attention with Accurate
// Recurrent State Quantization", App. A with D_t = alpha I, or D_t =
// Diag(alpha) per key row for per-channel decay (CH), and b_t = beta):
//   S = D_t S;  r = S^T k;  u = beta (v - r);  S = S + k u^T;  o = S^T q
// with S[r][c] indexed (key row, value column).  A bf16 state is widened,
// updated in fp32 and rounded to nearest even on store (the hardware's
// packed conversion).  The update is one fma per entry; the reads are sums
// over the rows in the order of the thread map below (these baselines are
// checked against the dense fp32 step to a tolerance, not bit for bit).
//
// Thread map: the head's state is read and written as 16-byte pieces, piece
// d * 256 + t by thread t (d = 0 .. 64 / VEC - 1), so every load and store
// instruction of a wave covers 1 KB of contiguous memory.  A piece holds VEC
// = 4 (fp32) or 8 (bf16) consecutive columns of one row: thread t owns the
// columns VEC (t % LPR) .. + VEC - 1 (LPR = 128 / VEC pieces per row) of the
// rows t / LPR + (256 / LPR) d.  Column sums run over the thread's rows,
// then across the lanes that share the column group (lane bits >= log2 LPR),
// then across the four waves through LDS.  The state is streamed with the
// non-temporal hint: each launch reads and writes every byte once.
#include "leapq_device.h"

namespace leapq {
namespace {
using namespace dev;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even as packed bf16 (one
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <typename TS>
struct Piece {
    static constexpr int VEC = 16 / (int)sizeof(TS);  // elements per 16-byte piece
    static constexpr int LPR = D / VEC;                // pieces per row
    static constexpr int RPT = 64 / VEC;               // pieces (rows) per thread
    static constexpr int RS = NT / LPR;                // row stride between a thread's pieces
};

__device__ __forceinline__ void unpack(u32x4 x, float (&f)[4])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
}
__device__ __forceinline__ void unpack(u32x4 x, float (&f)[8])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(x[e] << 16);
        f[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ u32x4 pack(const float (&f)[4])
{
    u32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __float_as_uint(f[e]);
    return x;
}
__device__ __forceinline__ u32x4 pack(const float (&f)[8])
{
    u32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
    return x;
}

// Sum of x over the lanes of the wave that share lane % LPR.
template <int LPR>
__device__ __forceinline__ float lanesum(float x)
{
#pragma unroll
    for (int s = LPR; s < 64; s <<= 1) x += __shfl_xor(x, s);
    return x;
}

template <typename TS, typename TI, bool CH>
__global__ __launch_bounds__(NT) void k_gdn_decode(TS *__restrict__ Sg, const TI *__restrict__ qin,
                                                    const TI *__restrict__ kin, const TI *__restrict__ vin,
                                                    const float *__restrict__ alpha,
                                                    const float *__restrict__ beta, float *__restrict__ o)
{
    using P = Piece<TS>;
    constexpr int VEC = P::VEC, LPR = P::LPR, RPT = P::RPT, RS = P::RS;
    __shared__ float red[2][4][D];  // per-wave column partials of S^T k and S^T q
    __shared__ float kq[3][D];      // k, q and (per-channel decay) alpha of the head
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = t % LPR, g = t / LPR;
    const int h = blockIdx.x;
    u32x4 *Sh = reinterpret_cast<u32x4 *>(Sg + (size_t)h * D * D);
    u32x4 raw[RPT];
#pragma unroll
    for (int d = 0; d < RPT; ++d) raw[d] = __builtin_nontemporal_load(Sh + d * NT + t);
    const TI *qh = qin + (size_t)h * D, *kh = kin + (size_t)h * D, *vh = vin + (size_t)h * D;
    if (t < D) {
        kq[0][t] = ld_in<TI>(kh, t);
        kq[1][t] = ld_in<TI>(qh, t);
        if (CH) kq[2][t] = alpha[(size_t)h * D + t];
    }
    float vc[VEC];
#pragma unroll
    for (int m = 0; m < VEC; ++m) vc[m] = ld_in<TI>(vh, cg * VEC + m);
    const float bt = beta[h];
    const float a0 = CH ? 0.0f : alpha[h];
    __syncthreads();
    float S[RPT][VEC], pr[VEC];
#pragma unroll
    for (int m = 0; m < VEC; ++m) pr[m] = 0.0f;
#pragma unroll
    for (int d = 0; d < RPT; ++d) {
        unpack(raw[d], S[d]);
        const float al = CH ? kq[2][d * RS + g] : a0;
        const float kr = kq[0][d * RS + g];
#pragma unroll
        for (int m = 0; m < VEC; ++m) {
            S[d][m] = al * S[d][m];
            pr[m] = fma_(S[d][m], kr, pr[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < VEC; ++m) pr[m] = lanesum<LPR>(pr[m]);
    if (l < LPR)
#pragma unroll
        for (int m = 0; m < VEC; ++m) red[0][w][cg * VEC + m] = pr[m];
    __syncthreads();
    float u[VEC], po[VEC];
#pragma unroll
    for (int m = 0; m < VEC; ++m) {
        const int c = cg * VEC + m;
        const float rc = (red[0][0][c] + red[0][1][c]) + (red[0][2][c] + red[0][3][c]);
        u[m] = bt * (vc[m] - rc);
        po[m] = 0.0f;
    }
#pragma unroll
    for (int d = 0; d < RPT; ++d) {
        const float kr = kq[0][d * RS + g], qr = kq[1][d * RS + g];
#pragma unroll
        for (int m = 0; m < VEC; ++m) {
            S[d][m] = fma_(kr, u[m], S[d][m]);
            po[m] = fma_(S[d][m], qr, po[m]);
        }
        __builtin_nontemporal_store(pack(S[d]), Sh + d * NT + t);
    }
#pragma unroll
    for (int m = 0; m < VEC; ++m) po[m] = lanesum<LPR>(po[m]);
    if (l < LPR)
#pragma unroll
        for (int m = 0; m < VEC; ++m) red[1][w][cg * VEC + m] = po[m];
    __syncthreads();
    if (t < LPR)
#pragma unroll
        for (int m = 0; m < VEC; ++m) {
            const int c = cg * VEC + m;
            o[(size_t)h * D + c] = (red[1][0][c] + red[1][1][c]) + (red[1][2][c] + red[1][3][c]);
        }
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
