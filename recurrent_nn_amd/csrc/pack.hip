// pack.hip -- weight packing and state initialisation kernels.
//
// The onemodel page ("Computation") transposes the weights once per plan when
// they are constant and otherwise on each run into scratch.  On the matrix
// cores both products want the reduction index contiguous, which is already
// how W [dirs, G*H, input] and R [dirs, G*H, H] are stored, so "packing" here
// is a row permutation instead of a transpose: the G gate rows of each block
// of U hidden units become adjacent, so that one workgroup of the recurrence
// finds its XW columns and its R rows contiguous.  W may be rounded to
// bfloat16 (round to nearest even) for the bf16 projection; R is padded with
// zero rows to whole 16-column tiles and with zero columns to Hp.
#include <hip/hip_runtime.h>

#include "common.h"

namespace rnnamd {

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);          // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Source row (in W's or R's natural gate-major order) of packed row r.
__device__ __forceinline__ int64_t packed_to_natural(int64_t r, int64_t G, int64_t H, int32_t U)
{
    const int64_t GH = G * H;
    const int64_t d = r / GH;
    const int64_t rl = r - d * GH;
    const int64_t ub = rl / (G * U);
    const int64_t rem = rl - ub * G * U;
    const int64_t u0 = ub * U;
    const int64_t uc = (H - u0) < U ? (H - u0) : U;
    const int64_t g = rem / uc;
    const int64_t u = rem - g * uc;
    return d * GH + g * H + u0 + u;
}

__global__ void pack_w_f32(const float *__restrict__ W, float *__restrict__ Wp, int64_t rows,
                           int64_t I, int64_t G, int64_t H, int32_t U)
{
    const int64_t r = blockIdx.x;
    if (r >= rows)
        return;
    const float *src = W + packed_to_natural(r, G, H, U) * I;
    float *dst = Wp + r * I;
    for (int64_t k = threadIdx.x; k < I; k += blockDim.x)
        dst[k] = src[k];
}

__global__ void pack_w_bf16(const float *__restrict__ W, uint16_t *__restrict__ Wp, int64_t rows,
                            int64_t I, int64_t G, int64_t H, int32_t U)
{
    const int64_t r = blockIdx.x;
    if (r >= rows)
        return;
    const float *src = W + packed_to_natural(r, G, H, U) * I;
    uint16_t *dst = Wp + r * I;
    for (int64_t k = threadIdx.x; k < I; k += blockDim.x)
        dst[k] = bf16_rne(src[k]);
}

// Rp [D][NUB][NT*16][Hp]: row c of unit block ub holds, for phase 0, gate g of
// unit u at c = g*uc + u (GRU lbr=0: only z and r), and for phase 1 (GRU
// lbr=0 candidate) unit u at c = NTA*16 + u.  Everything else is zero.
__global__ void pack_r(const float *__restrict__ R, float *__restrict__ Rp, int64_t D, int64_t G,
                       int64_t H, int64_t Hp, int32_t U, int32_t NUB, int32_t NTA, int32_t NTB,
                       int32_t phases)
{
    const int32_t NTC = (NTA + NTB) * 16;
    const int64_t row = blockIdx.x;                       // over D * NUB * NTC
    if (row >= D * NUB * NTC)
        return;
    const int64_t d = row / ((int64_t)NUB * NTC);
    const int64_t ub = (row / NTC) % NUB;
    const int32_t c = (int32_t)(row % NTC);
    const int64_t u0 = ub * U;
    const int32_t uc = (int32_t)((H - u0) < U ? (H - u0) : U);
    int64_t src = -1;
    if (phases == 2) {
        if (c < NTA * 16) {
            if (c < 2 * uc)
                src = d * G * H + (c / uc) * H + u0 + (c % uc);
        } else if (c - NTA * 16 < uc) {
            src = d * G * H + 2 * H + u0 + (c - NTA * 16);
        }
    } else if (c < G * uc) {
        src = d * G * H + (c / uc) * H + u0 + (c % uc);
    }
    float *dst = Rp + row * Hp;
    for (int64_t k = threadIdx.x; k < Hp; k += blockDim.x)
        dst[k] = (src >= 0 && k < H) ? R[src * H + k] : 0.0f;
}

int launch_pack(const PackArgs &a, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const int64_t rows = a.D * a.G * a.H;
    if (rows > 0 && a.I > 0) {
        if (a.bf16)
            hipLaunchKernelGGL(pack_w_bf16, dim3((unsigned)rows), dim3(256), 0, s, a.W,
                               (uint16_t *)a.Wp, rows, a.I, a.G, a.H, a.U);
        else
            hipLaunchKernelGGL(pack_w_f32, dim3((unsigned)rows), dim3(256), 0, s, a.W,
                               (float *)a.Wp, rows, a.I, a.G, a.H, a.U);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return (int)e;
    }
    const int64_t rrows = a.D * a.NUB * (int64_t)(a.NTA + a.NTB) * 16;
    hipLaunchKernelGGL(pack_r, dim3((unsigned)rrows), dim3(256), 0, s, a.R, a.Rp, a.D, a.G, a.H,
                       a.Hp, a.U, a.NUB, a.NTA, a.NTB, a.phases);
    return (int)hipGetLastError();
}

// X -> bf16 (round to nearest even); kept for callers that want a separate
// cast (the projection kernel otherwise rounds X while staging it).
// States before the first step: plane 0 of the H history holds initial_h
// (zero when absent, and zero in the padding rows and columns), cbuf holds
// initial_c, and the step flags and the error word are cleared.  Later planes
// are written by the steps themselves.
__global__ void init_kernel(InitArgs a)
{
    const int64_t plane = a.D * a.Btp * a.Hp;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = tid; i < plane; i += stride) {
        float v = 0.0f;
        if (a.h0) {
            const int64_t k = i % a.Hp;
            const int64_t s = (i / a.Hp) % a.Btp;    // position; batch row order[s]
            const int64_t d = i / (a.Hp * a.Btp);
            if (s < a.Bt && k < a.H) {
                const int64_t b = a.order ? a.order[s] : s;
                v = a.layout == 0 ? a.h0[(d * a.Bt + b) * a.H + k] : a.h0[(b * a.D + d) * a.H + k];
            }
        }
        a.hbuf[i] = v;
    }
    if (a.cbuf) {
        const int64_t n = a.D * a.Bt * a.H;
        for (int64_t i = tid; i < n; i += stride) {
            float v = 0.0f;
            if (a.c0) {
                const int64_t k = i % a.H;
                const int64_t s = (i / a.H) % a.Bt;
                const int64_t b = a.order ? a.order[s] : s;
                const int64_t d = i / (a.H * a.Bt);
                v = a.layout == 0 ? a.c0[(d * a.Bt + b) * a.H + k] : a.c0[(b * a.D + d) * a.H + k];
            }
            a.cbuf[i] = v;
        }
    }
    if (a.fill_lens >= 0)
        for (int64_t b = tid; b < a.Bt; b += stride)
            a.lens_dev[b] = a.fill_lens;
    for (int64_t i = tid; i <= a.n_bar; i += stride)
        a.bar[i] = 0u;          // step flags, then the error word
}

int launch_init(const InitArgs &a, void *stream)
{
    const int64_t work = a.D * a.Btp * a.Hp;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(init_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

__global__ void lens_inline_kernel(InlineLens l, int32_t *dst)
{
    for (int i = threadIdx.x; i < l.n; i += blockDim.x) {
        dst[i] = l.lens[i];
        dst[l.n + i] = l.order[i];
        dst[2 * l.n + i] = l.rank_pos[i];
    }
}

int launch_lens_inline(const InlineLens &l, int32_t *dst, void *stream)
{
    if (l.n < 1 || l.n > kInlineRows)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(lens_inline_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, l, dst);
    return (int)hipGetLastError();
}

__device__ __forceinline__ float canon0(float v)
{
    return v != v ? __uint_as_float(0x7FC00000u) : v;
}

// seq = 0 or batch = 0: nothing runs; Y_h / Y_c are the initial states or 0.
__global__ void zero_size_states(FinalArgs a)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (a.Yh)
            a.Yh[i] = a.h0 ? canon0(a.h0[i]) : 0.0f;
        if (a.Yc)
            a.Yc[i] = a.c0 ? canon0(a.c0[i]) : 0.0f;
    }
}

// The cell convention's single summed bias B (OpenVINO "RNNCell-3", section
// "Inputs": the sum of the W and R biases) as an ONNX B: Wb = B, Rb = +0.
// Adding +0 after it is exact: no pre-activation is -0 at that point (both
// products' sums start at +0).
__global__ void cell_bias_kernel(const float *__restrict__ Bs, float *__restrict__ dst, int64_t D,
                                 int64_t GH)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < D * 2 * GH;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t d = i / (2 * GH), k = i - d * 2 * GH;
        dst[i] = k < GH ? Bs[d * GH + k] : 0.0f;
    }
}

int launch_cell_bias(const float *B_sum, float *dst, int64_t D, int64_t GH, void *stream)
{
    const int64_t n = D * 2 * GH;
    if (n <= 0)
        return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024)
        blocks = 1024;
    hipLaunchKernelGGL(cell_bias_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       B_sum, dst, D, GH);
    return (int)hipGetLastError();
}

int launch_zero_size_states(const FinalArgs &a, void *stream)
{
    if (a.n <= 0)
        return 0;
    int64_t blocks = (a.n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(zero_size_states, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace rnnamd
