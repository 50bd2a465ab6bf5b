// activations.h -- device activation functions of the ONNX recurrent
// operators (onemodel "Recurrent operators", section "Activations": the
// supported list and the definitions).  The files that include this are
// compiled with -ffp-contract=off, so every written operation is one IEEE
// binary32 operation, rounded on its own.  Compares and selects are written so
// that a NaN argument gives what the written definition gives (NaN for all but
// ThresholdedRelu, whose compare sends NaN to 0).  Sigmoid, Tanh and
// ScaledTanh use the fast exp2-based forms below, Elu and Softplus the device
// math library (the fast mode of that page allows fast elementwise functions).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace rnnamd {

// Fast-mode forms of the two default activations ("Fast mode": elementwise
// functions use fast approximations).  exp is the hardware base-2 exponential
// of x*log2(e) and 1/y the hardware reciprocal (v_rcp_f32, within 1 ulp; its
// argument here is >= 1, never subnormal); absolute error below 3e-7 on all
// of R.  NaN gives NaN; +-inf give the limits.
__device__ __forceinline__ float fast_rcp(float y) { return __builtin_amdgcn_rcpf(y); }

__device__ __forceinline__ float fast_sigmoid(float x)
{
    const float e = __expf(-x);          // inf for x << 0, 0 for x >> 0
    const float den = 1.0f + e;
    return fast_rcp(den);
}

__device__ __forceinline__ float fast_tanh(float x)
{
    // tanh|x| = 1 - 2 / (exp(2|x|) + 1), sign restored; saturates to 1.
    const float ax = fabsf(x);
    const float e = __expf(2.0f * ax);
    const float den = e + 1.0f;
    const float q = 2.0f * fast_rcp(den);
    const float t = 1.0f - q;
    return copysignf(t, x);
}

__device__ __forceinline__ float act_apply(int32_t kind, float alpha, float beta, float x)
{
    switch (kind) {
    case ACT_SIGMOID:
        return fast_sigmoid(x);
    case ACT_TANH:
        return fast_tanh(x);
    case ACT_RELU:
        return x < 0.0f ? 0.0f : x;
    case ACT_AFFINE: {
        float ax = alpha * x;
        return ax + beta;
    }
    case ACT_LEAKYRELU: {
        float ax = alpha * x;
        return x < 0.0f ? ax : x;
    }
    case ACT_THRESHOLDEDRELU:
        return x > alpha ? x : 0.0f;
    case ACT_SCALEDTANH: {
        float bx = beta * x;
        float t = fast_tanh(bx);
        return alpha * t;
    }
    case ACT_HARDSIGMOID: {
        float ax = alpha * x;
        float y = ax + beta;
        y = y < 0.0f ? 0.0f : y;
        y = y > 1.0f ? 1.0f : y;
        return y;
    }
    case ACT_ELU: {
        float em1 = expm1f(x);
        float v = alpha * em1;
        return x >= 0.0f ? x : v;
    }
    case ACT_SOFTSIGN: {
        float den = 1.0f + fabsf(x);
        return x / den;
    }
    case ACT_SOFTPLUS: {
        float sp = log1pf(expf(x));
        return x > 20.0f ? x : sp;
    }
    default:
        return __builtin_nanf("");
    }
}

// Activation functors: the specialised forms used when the activation set is
// known per kernel launch, and the run-time switch for every other set.
struct ActSigmoid {
    __device__ __forceinline__ float operator()(float x) const { return fast_sigmoid(x); }
};
struct ActTanh {
    __device__ __forceinline__ float operator()(float x) const { return fast_tanh(x); }
};
struct ActHardSigmoid {
    float alpha, beta;
    __device__ __forceinline__ float operator()(float x) const
    {
        float ax = alpha * x;
        float y = ax + beta;
        y = y < 0.0f ? 0.0f : y;
        y = y > 1.0f ? 1.0f : y;
        return y;
    }
};
struct ActAny {
    ActSpec s;
    __device__ __forceinline__ float operator()(float x) const { return act_apply(s.kind, s.alpha, s.beta, x); }
};

// clip, active only when given and positive: clamp to [-c, c]; a NaN passes through.
__device__ __forceinline__ float clip_pre(float x, int on, float c)
{
    if (!on)
        return x;
    float nc = -c;
    float y = x > c ? c : x;
    return y < nc ? nc : y;
}

// The outputs carry one NaN encoding only (onemodel "Recurrent operators",
// section "Exact mode"): any NaN becomes the quiet NaN with bit pattern
// 0x7FC00000 (positive sign, no payload) when Y, Y_h or Y_c is stored.
__device__ __forceinline__ float canon_nan(float v)
{
    return v != v ? __uint_as_float(0x7FC00000u) : v;
}

}  // namespace rnnamd
