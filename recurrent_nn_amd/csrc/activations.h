// activations.h -- device activation functions of the ONNX recurrent
// operators (onemodel "Recurrent operators", section "Activations": the
// supported list and the definitions).  The files that include this are
// compiled with -ffp-contract=off, so every written operation is one IEEE
// binary32 operation, rounded on its own.  Compares and selects are written so
// that a NaN argument gives what the written definition gives (NaN for all but
// ThresholdedRelu, whose compare sends NaN to 0).  Sigmoid, Tanh, ScaledTanh,
// Elu and Softplus use the device math library ("fast mode" on that page).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace rnnamd {

__device__ __forceinline__ float act_apply(int32_t kind, float alpha, float beta, float x)
{
    switch (kind) {
    case ACT_SIGMOID: {
        float e = expf(-x);
        float den = 1.0f + e;
        return 1.0f / den;
    }
    case ACT_TANH:
        return tanhf(x);
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
        float t = tanhf(bx);
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

// clip "when present and positive": clamp to [-c, c]; a NaN passes through.
__device__ __forceinline__ float clip_pre(float x, int on, float c)
{
    if (!on)
        return x;
    float nc = -c;
    float y = x > c ? c : x;
    return y < nc ? nc : y;
}

// Every NaN in Y, Y_h and Y_c is written as 0x7FC00000.
__device__ __forceinline__ float canon_nan(float v)
{
    return v != v ? __uint_as_float(0x7FC00000u) : v;
}

}  // namespace rnnamd
