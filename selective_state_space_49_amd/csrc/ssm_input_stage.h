// ssm_input_stage.h -- the MambaBlock's input stage, applied as values are loaded.
//
// Before its scan, the MambaBlock ("【大模型】- Jamba 混合 SSM-Transformer", section
// 4.1 "Mamba 层") sends x through a depthwise convolution over time and silu, and
// the dt projection's output through softplus. The convolution has one filter of K
// taps and one bias per channel, with K-1 zeros of padding in front, and its output
// is cut back to the first L steps: output t sees inputs t-K+1 .. t only (causal).
// As in deep-learning convolutions the taps are not flipped: tap k multiplies input
// t-(K-1)+k. The fused kernels call these on every loaded (x, dt) pair, so the
// recurrence sees (u, dt) = (silu(conv(x)), softplus(dt + bias)) without either
// ever being written to memory.
#pragma once

#include "ssm_device.h"

namespace ssm {

constexpr float kLn2 = 0.6931471805599453f;

// softplus(v) = log(1 + e^v), evaluated as max(v, 0) + log1p(e^-|v|) (equal forms:
// for v > 0, 1 + e^v = e^v (1 + e^-v)), so it neither overflows nor rounds small
// results away. log1p(e) for e in [0, 1] uses Goldberg's correction (Theorem 4 of
// "What Every Computer Scientist Should Know About Floating-Point Arithmetic"): with
// w = 1 + e rounded to fp32, log1p(e) = e when w == 1 and log(w) * e / (w - 1)
// otherwise; the factor e / (w - 1) cancels the rounding of w. log(w) is the hardware
// base-2 logarithm times ln 2. NaN stays NaN; softplus(+inf) = inf, softplus(-inf) = 0.
// Operation order: e = e2(-|v| * log2(e)); w = 1 + e;
//   l = (w == 1) ? e : (log2(w) * ln2) * (e * rcp(w - 1));  result = max(v, 0) + l.
__device__ __forceinline__ float softplus(float v) {
    const float e = e2(-__builtin_fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    const float l = w == 1.0f ? e : (__builtin_amdgcn_logf(w) * kLn2) * (e * rcp(w - 1.0f));
    return __builtin_fmaxf(v, 0.0f) + l;
}

// Causal depthwise convolution of KC taps (1..4) followed by silu, for one channel
// walked forward in time. hist holds the KC-1 previous inputs, oldest first.
// Operation order: acc = bias; acc = fma(w[k], input t-(KC-1)+k, acc) for k = 0 ..
// KC-1; u = silu(acc).
template <int KC>
struct ConvSilu {
    static_assert(KC >= 1 && KC <= 4, "1 to 4 taps");
    float w[KC];
    float bias;
    float hist[KC > 1 ? KC - 1 : 1];

    // Output for the next input v; v becomes the newest history entry.
    __device__ __forceinline__ float operator()(float v) {
        float acc = bias;
#pragma unroll
        for (int k = 0; k < KC - 1; ++k) acc = __builtin_fmaf(w[k], hist[k], acc);
        acc = __builtin_fmaf(w[KC - 1], v, acc);
        if constexpr (KC > 1) {
#pragma unroll
            for (int k = 0; k + 1 < KC - 1; ++k) hist[k] = hist[k + 1];
            hist[KC - 2] = v;
        }
        return silu(acc);
    }
};

}  // namespace ssm
