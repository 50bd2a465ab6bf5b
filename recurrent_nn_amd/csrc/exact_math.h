// exact_math.h -- exact-mode elementary functions and activations.
//
// The onemodel page "Recurrent operators: RNN, GRU, LSTM" (section "Exact
// mode") asks for results that are the same bits on every machine, with the
// transcendental activations taken from a polynomial document that is not
// available.  Exact mode here evaluates Sigmoid, Tanh, ScaledTanh, Elu and
// Softplus in binary64 from the binary32 argument and rounds once to
// binary32, with every binary64 function computed by one fixed sequence of
// IEEE operations (round to nearest, no fused multiply-add -- the
// __d*_rn intrinsics make each step explicit):
//   e^x     NaN -> NaN; x > 708 -> +inf; x < -708 -> +0; else k = rint(x/ln2)
//           taken as rint(x * INV_LN2), r = (x - k*LN2_HI) - k*LN2_LO (ln 2
//           split in a head with 32 trailing zero bits and a tail: Cody and
//           Waite), p = sum_{i<=13} r^i/i! by Horner from i = 13, p * 2^k.
//   e^x - 1 |x| < 1/2: x * sum_{i=1..17} x^(i-1)/i! by Horner from i = 17;
//           else e^x - 1.
//   tanh x  NaN -> NaN; |x| > 22 -> +-1; else m = e^(2|x|) - 1 and
//           copysign(m / (m + 2), x).
//   log(1+u), 0 <= u <= 1: s = u / (2 + u), q = s*s,
//           2 * s * sum_{n<=20} q^n / (2n+1) by Horner from n = 20.
// The other activations are the written binary32 operations, as in fast mode.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace rnnamd {
namespace xm {

constexpr double kLn2Hi = 0x1.62e42feep-1;       // head of ln 2 (low 32 bits zero)
constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;  // ln 2 - kLn2Hi
constexpr double kInvLn2 = 0x1.71547652b82fep+0;  // 1 / ln 2

// 1 / i!, rounded once (i! is exact in binary64 for i <= 18)
__host__ __device__ constexpr double recip_factorial(int i)
{
    double f = 1.0;
    for (int j = 2; j <= i; ++j)
        f = f * (double)j;
    return 1.0 / f;
}

__device__ inline double exp_d(double x)
{
    if (x != x)
        return x;
    if (x > 708.0)
        return __builtin_huge_val();
    if (x < -708.0)
        return 0.0;
    const double k = rint(__dmul_rn(x, kInvLn2));
    const double r = __dsub_rn(__dsub_rn(x, __dmul_rn(k, kLn2Hi)), __dmul_rn(k, kLn2Lo));
    double p = recip_factorial(13);
#pragma unroll
    for (int i = 12; i >= 0; --i)
        p = __dadd_rn(__dmul_rn(p, r), recip_factorial(i));
    return ldexp(p, (int)k);
}

__device__ inline double expm1_d(double x)
{
    if (fabs(x) < 0.5) {
        double p = recip_factorial(17);
#pragma unroll
        for (int i = 16; i >= 1; --i)
            p = __dadd_rn(__dmul_rn(p, x), recip_factorial(i));
        return __dmul_rn(x, p);
    }
    return __dsub_rn(exp_d(x), 1.0);
}

__device__ inline double tanh_d(double x)
{
    if (x != x)
        return x;
    const double ax = fabs(x);
    if (ax > 22.0)
        return copysign(1.0, x);
    const double m = expm1_d(__dmul_rn(2.0, ax));
    return copysign(__ddiv_rn(m, __dadd_rn(m, 2.0)), x);
}

__device__ inline double log1p_01(double u)        // 0 <= u <= 1
{
    const double s = __ddiv_rn(u, __dadd_rn(2.0, u));
    const double q = __dmul_rn(s, s);
    double p = 1.0 / 41.0;
#pragma unroll
    for (int n = 19; n >= 0; --n)
        p = __dadd_rn(__dmul_rn(p, q), 1.0 / (double)(2 * n + 1));
    return __dmul_rn(__dmul_rn(2.0, s), p);
}

// One activation in exact mode (kinds as ActKind).
__device__ inline float act_exact(int32_t kind, float alpha, float beta, float x)
{
    switch (kind) {
    case ACT_SIGMOID:
        return (float)__ddiv_rn(1.0, __dadd_rn(1.0, exp_d(-(double)x)));
    case ACT_TANH:
        return (float)tanh_d((double)x);
    case ACT_RELU:
        return x < 0.0f ? 0.0f : x;
    case ACT_AFFINE:
        return __fadd_rn(__fmul_rn(alpha, x), beta);
    case ACT_LEAKYRELU:
        return x < 0.0f ? __fmul_rn(alpha, x) : x;
    case ACT_THRESHOLDEDRELU:
        return x > alpha ? x : 0.0f;
    case ACT_SCALEDTANH:
        return (float)__dmul_rn((double)alpha, tanh_d(__dmul_rn((double)beta, (double)x)));
    case ACT_HARDSIGMOID: {
        float y = __fadd_rn(__fmul_rn(alpha, x), beta);
        y = y < 0.0f ? 0.0f : y;
        y = y > 1.0f ? 1.0f : y;
        return y;
    }
    case ACT_ELU:
        return x >= 0.0f ? x : (float)__dmul_rn((double)alpha, expm1_d((double)x));
    case ACT_SOFTSIGN:
        return __fdiv_rn(x, __fadd_rn(1.0f, fabsf(x)));
    case ACT_SOFTPLUS:
        if (x > 20.0f)
            return x;                                   // log(1 + e^x) rounds to x
        if (x > 0.0f)
            return (float)__dadd_rn((double)x, log1p_01(exp_d(-(double)x)));
        return (float)log1p_01(exp_d((double)x));
    default:
        return __builtin_nanf("");
    }
}

}  // namespace xm

// Functor form for the gate helpers.
struct ActExact {
    ActSpec s;
    __device__ float operator()(float x) const { return xm::act_exact(s.kind, s.alpha, s.beta, x); }
};

}  // namespace rnnamd
