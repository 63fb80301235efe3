// input_bwd.hip -- gradients through the MambaBlock's input stage, for training (gfx950).
//
// The fused prefill evaluates u = silu(conv(x_in)) and dt = softplus(dt_raw + bias)
// inside the scan's load stage: the depthwise causal convolution over time (K taps and
// a bias per channel) and silu on x, softplus on the dt projection's output
// ("【大模型】- Jamba 混合 SSM-Transformer", section 4.1 "Mamba 层"). Its backward,
// ssm_scan_bwd_fused, runs in three parts on one stream:
//   1. k_input_fwd writes u and dt (the scan's inputs) to the workspace, with the
//      fused prefill's own fp32 operations (ConvSilu, softplus);
//   2. the scan's backward (ssm_scan_bwd) gives du = dLoss/du and ddt = dLoss/ddt,
//      together with dz, dA, dB, dC, dD, dh0;
//   3. k_input_bwd takes du and ddt back through the input stage by the chain rule.
//      With xe the K-1 carried inputs followed by x_in and a_t = cb + sum_k w[k]
//      xe_{t-(K-1)+k} (the value silu is applied to),
//          da_t = du_t silu'(a_t),  silu'(a) = s (1 + a (1 - s)),  s = 1 / (1 + e^-a)
//          dx_in_s = sum_k w[k] da_{s+(K-1)-k}  (da past the last step is 0)
//          dw[k] = sum_t da_t xe_{t-(K-1)+k},  dcb = sum_t da_t
//          ddt_raw_t = ddt_t / (1 + e^-(dt_raw_t + bias)),  dbias = sum_t ddt_raw_t
//      and the carried state's gradient dxe_s for s = -(K-1) .. -1. One lane per
//      channel walks its chunk of steps backwards, keeping the window of K inputs the
//      step's a_t needs and the K-1 values da_{t+1} .. da_{t+K-1} its dx_in_t needs;
//      the first K-1 steps after the chunk are evaluated once at its start. The sums
//      over steps go to per-chunk partials, summed by k_input_bwd_reduce over chunks
//      and batch rows in a fixed order.
// Both kernels stream [rows][Dn] arrays with one lane per channel (coalesced across
// the wave) and 64-bit element indices.
#include "ssm_device.h"
#include "ssm_input_stage.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

struct Lane {
    int64_t b, d, t0, t1;
    bool live;
};

__device__ __forceinline__ Lane lane_of(const InBwdArgs &a) {
    const int64_t dblocks = (a.Dn + 255) / 256;
    Lane l;
    l.b = (int64_t)blockIdx.x / dblocks;
    l.d = ((int64_t)blockIdx.x % dblocks) * 256 + threadIdx.x;
    l.live = l.d < a.Dn;
    l.t0 = (int64_t)blockIdx.y * a.T;
    l.t1 = min(a.L, l.t0 + a.T);
    return l;
}

// Input xe_s of channel d in batch row b: x_in for s >= 0, else the carried state (or 0).
template <typename IO, int KC>
__device__ __forceinline__ float xe(const InBwdArgs &a, int64_t b, int64_t d, int64_t s) {
    if (s >= 0) return Io<IO>::ld((const IO *)a.x_in + (b * a.L + s) * a.Dn + d);
    if (!a.conv_state0) return 0.0f;
    return Io<IO>::ld((const IO *)a.conv_state0 + (b * (KC - 1) + (KC - 1 + s)) * a.Dn + d);
}

// ---------------------------------------------------------------- forward recompute
template <typename IO, int KC>
__global__ __launch_bounds__(256) void k_input_fwd(InBwdArgs a) {
    const Lane ln = lane_of(a);
    if (!ln.live) return;
    const int64_t b = ln.b, d = ln.d;
    const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
    ConvSilu<(KC > 0 ? KC : 1)> conv;
    if constexpr (KC > 0) {
#pragma unroll
        for (int k = 0; k < KC; ++k) conv.w[k] = a.conv_w[d * KC + k];
        conv.bias = a.conv_b ? a.conv_b[d] : 0.0f;
#pragma unroll
        for (int j = 0; j < KC - 1; ++j) conv.hist[j] = xe<IO, KC>(a, b, d, ln.t0 - (KC - 1) + j);
    }
    for (int64_t t = ln.t0; t < ln.t1; ++t) {
        const int64_t e = (b * a.L + t) * a.Dn + d;
        const float v = Io<IO>::ld((const IO *)a.x_in + e);
        float u = v;
        if constexpr (KC > 0) u = conv(v);
        Io<IO>::st((IO *)a.u + e, u);
        Io<IO>::st((IO *)a.dt + e, softplus(Io<IO>::ld((const IO *)a.dt_raw + e) + bias));
    }
}

// ---------------------------------------------------------------- chain rule
// a_t from the window win[k] = xe_{t-(KC-1)+k}, in the fused prefill's order (bias,
// then one fma per tap, oldest first).
template <int KC>
__device__ __forceinline__ float pre_act(const float (&w)[KC], float cb, const float (&win)[KC]) {
    float acc = cb;
#pragma unroll
    for (int k = 0; k < KC; ++k) acc = __builtin_fmaf(w[k], win[k], acc);
    return acc;
}

__device__ __forceinline__ float silu_grad(float du, float pre) {
    const float s = rcp(1.0f + e2(-pre * kLog2e));
    return du * (s * __builtin_fmaf(pre, 1.0f - s, 1.0f));
}

template <typename IO, int KC>
__global__ __launch_bounds__(256) void k_input_bwd(InBwdArgs a) {
    constexpr int P = KC + 2;  // partials per (chunk, batch row, channel): dw[KC], dcb, dbias
    const Lane ln = lane_of(a);
    if (!ln.live) return;
    const int64_t b = ln.b, d = ln.d, row = b * a.L;
    const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
    float dbias = 0.0f;
    constexpr int W = KC > 0 ? KC : 1;
    float w[W], win[W], dw[W], fut[KC > 1 ? KC - 1 : 1];
    float cb = 0.0f, dcb = 0.0f;
    if constexpr (KC > 0) {
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            w[k] = a.conv_w[d * KC + k];
            dw[k] = 0.0f;
        }
        cb = a.conv_b ? a.conv_b[d] : 0.0f;
        // da at the KC-1 steps after the chunk (0 past the sequence)
#pragma unroll
        for (int j = 0; j < KC - 1; ++j) {
            const int64_t s = ln.t1 + j;
            fut[j] = 0.0f;
            if (s < a.L) {
                float ws[KC];
#pragma unroll
                for (int k = 0; k < KC; ++k) ws[k] = xe<IO, KC>(a, b, d, s - (KC - 1) + k);
                fut[j] = silu_grad(Io<IO>::ld((const IO *)a.du + (row + s) * a.Dn + d), pre_act<KC>(w, cb, ws));
            }
        }
        // window of the chunk's last step
#pragma unroll
        for (int k = 0; k < KC; ++k) win[k] = ln.t1 > ln.t0 ? xe<IO, KC>(a, b, d, ln.t1 - 1 - (KC - 1) + k) : 0.0f;
    }
    for (int64_t t = ln.t1 - 1; t >= ln.t0; --t) {
        const int64_t e = (row + t) * a.Dn + d;
        const float du = Io<IO>::ld((const IO *)a.du + e);
        float dx = du;
        if constexpr (KC > 0) {
            const float da = silu_grad(du, pre_act<KC>(w, cb, win));
            // dx_in_t = sum_k w[k] da_{t+(KC-1)-k}: da_t with w[KC-1], da_{t+j} = fut[j-1]
            dx = w[KC - 1] * da;
#pragma unroll
            for (int j = 1; j < KC; ++j) dx = __builtin_fmaf(w[KC - 1 - j], fut[j - 1], dx);
#pragma unroll
            for (int k = 0; k < KC; ++k) dw[k] = __builtin_fmaf(da, win[k], dw[k]);
            dcb += da;
#pragma unroll
            for (int j = KC - 2; j >= 1; --j) fut[j] = fut[j - 1];
            if constexpr (KC > 1) fut[0] = da;
            // slide the window one step back
#pragma unroll
            for (int k = KC - 1; k >= 1; --k) win[k] = win[k - 1];
            if (t > ln.t0) win[0] = xe<IO, KC>(a, b, d, t - 1 - (KC - 1));
        }
        Io<IO>::st((IO *)a.dx_in + e, dx);
        const float r = Io<IO>::ld((const IO *)a.dt_raw + e) + bias;
        const float dr = Io<IO>::ld((const IO *)a.ddt + e) * rcp(1.0f + e2(-r * kLog2e));
        Io<IO>::st((IO *)a.ddt_raw + e, dr);
        dbias += dr;
    }
    if constexpr (KC > 1) {
        // the carried inputs before step 0: dxe_s, s = j - (KC-1), from da_0 .. da_{KC-2}
        // (fut now holds da_{t0} .. da_{t0+KC-2})
        if (ln.t0 == 0 && a.dconv_state0) {
#pragma unroll
            for (int j = 0; j < KC - 1; ++j) {
                float g = 0.0f;
#pragma unroll
                for (int k = 0; k <= j; ++k) g = __builtin_fmaf(w[k], fut[j - k], g);
                Io<IO>::st((IO *)a.dconv_state0 + (b * (KC - 1) + j) * a.Dn + d, g);
            }
        }
    }
    float *pp = a.part + (((int64_t)blockIdx.y * a.batch + b) * a.Dn + d) * P;
#pragma unroll
    for (int k = 0; k < KC; ++k) pp[k] = dw[k];
    pp[KC] = dcb;
    pp[KC + 1] = dbias;
}

// dconv_w [Dn][KC], dconv_b [Dn], ddt_bias [Dn]: sums of the partials over chunks, then
// batch rows (that fixed order), for the outputs given.
template <int KC>
__global__ __launch_bounds__(256) void k_input_bwd_reduce(InBwdArgs a) {
    constexpr int P = KC + 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over Dn * P
    if (i >= a.Dn * P) return;
    const int64_t d = i / P;
    const int k = (int)(i % P);
    float *out = k < KC ? a.dconv_w : k == KC ? a.dconv_b : a.ddt_bias;
    if (!out) return;
    float s = 0.0f;
    for (int64_t bb = 0; bb < a.batch; ++bb)
        for (int64_t c = 0; c < a.n_chunks; ++c) s += a.part[((c * a.batch + bb) * a.Dn + d) * P + k];
    out[k < KC ? d * KC + k : d] = s;
}

template <typename IO, int KC>
hipError_t launch_t(const InBwdArgs &a, bool fwd, hipStream_t s) {
    const dim3 grid((unsigned)(a.batch * ((a.Dn + 255) / 256)), (unsigned)a.n_chunks);
    if (fwd) {
        hipLaunchKernelGGL((k_input_fwd<IO, KC>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_input_bwd<IO, KC>), grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = a.Dn * (KC + 2);
    hipLaunchKernelGGL((k_input_bwd_reduce<KC>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_k(const InBwdArgs &a, bool fwd, hipStream_t s) {
    switch (a.conv_k) {
        case 0: return launch_t<IO, 0>(a, fwd, s);
        case 1: return launch_t<IO, 1>(a, fwd, s);
        case 2: return launch_t<IO, 2>(a, fwd, s);
        case 3: return launch_t<IO, 3>(a, fwd, s);
        case 4: return launch_t<IO, 4>(a, fwd, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_input_fwd(const InBwdArgs &a, int io, hipStream_t s) {
    return io == 0 ? launch_k<float>(a, true, s) : launch_k<bf16_bits>(a, true, s);
}

hipError_t launch_input_bwd(const InBwdArgs &a, int io, hipStream_t s) {
    return io == 0 ? launch_k<float>(a, false, s) : launch_k<bf16_bits>(a, false, s);
}

}  // namespace ssm
