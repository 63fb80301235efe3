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
// Both kernels stream [rows][Dn] arrays with 64-bit element indices, each lane taking
// V consecutive channels with one 8-byte access per row and stream (V = 4 for bf16, 2
// for fp32; one channel per lane when the sizes or pointers do not allow it).
#include "ssm_device.h"
#include "ssm_input_stage.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// V consecutive channels of one row: one access of V elements (8 bytes when V > 1).
template <typename IO, int V>
__device__ __forceinline__ void ldv(const IO *p, float (&v)[V]) {
    if constexpr (V == 1) {
        v[0] = Io<IO>::ld(p);
    } else if constexpr (sizeof(IO) == 2) {
        static_assert(V == 4, "bf16: 4 channels per lane");
        const u32x2v t = *(const u32x2v *)p;
        v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
        v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
    } else {
        static_assert(V == 2, "fp32: 2 channels per lane");
        const u32x2v t = *(const u32x2v *)p;
        v[0] = __uint_as_float(t.x); v[1] = __uint_as_float(t.y);
    }
}
template <typename IO, int V>
__device__ __forceinline__ void stv(IO *p, const float (&v)[V]) {
    if constexpr (V == 1) {
        Io<IO>::st(p, v[0]);
    } else if constexpr (sizeof(IO) == 2) {
        const u32x2v t = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                          (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
        *(u32x2v *)p = t;
    } else {
        const u32x2v t = {__float_as_uint(v[0]), __float_as_uint(v[1])};
        *(u32x2v *)p = t;
    }
}

// A lane's batch row, first channel d (it owns d .. d+V-1) and chunk.
struct Lane {
    int64_t b, d, t0, t1;
    bool live;
};

template <int V>
__device__ __forceinline__ Lane lane_of(const InBwdArgs &a) {
    const int64_t per_block = 256 * V;
    const int64_t dblocks = (a.Dn + per_block - 1) / per_block;
    Lane l;
    l.b = (int64_t)blockIdx.x / dblocks;
    l.d = ((int64_t)blockIdx.x % dblocks) * per_block + (int64_t)threadIdx.x * V;
    l.live = l.d < a.Dn;  // V > 1 only when V divides Dn
    l.t0 = (int64_t)blockIdx.y * a.T;
    l.t1 = min(a.L, l.t0 + a.T);
    return l;
}

// Steps per block of loads (both kernels walk a lane's steps one after the other; the
// block keeps kBlk rows of every stream in flight).
constexpr int kBlk = 8;

// Inputs xe_s of channels d .. d+V-1 in batch row b: x_in for s >= 0, else the carried
// state (or 0).
template <typename IO, int KC, int V>
__device__ __forceinline__ void xe(const InBwdArgs &a, int64_t b, int64_t d, int64_t s, float (&v)[V]) {
    if (s >= 0) {
        ldv<IO, V>((const IO *)a.x_in + (b * a.L + s) * a.Dn + d, v);
    } else if (!a.conv_state0) {
#pragma unroll
        for (int c = 0; c < V; ++c) v[c] = 0.0f;
    } else {
        ldv<IO, V>((const IO *)a.conv_state0 + (b * (KC - 1) + (KC - 1 + s)) * a.Dn + d, v);
    }
}

// ---------------------------------------------------------------- forward recompute
template <typename IO, int KC, int V>
__global__ __launch_bounds__(256) void k_input_fwd(InBwdArgs a) {
    const Lane ln = lane_of<V>(a);
    if (!ln.live) return;
    const int64_t b = ln.b, d = ln.d;
    float bias[V];
    ConvSilu<(KC > 0 ? KC : 1)> conv[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
        bias[c] = a.dt_bias ? a.dt_bias[d + c] : 0.0f;
        if constexpr (KC > 0) {
#pragma unroll
            for (int k = 0; k < KC; ++k) conv[c].w[k] = a.conv_w[(d + c) * KC + k];
            conv[c].bias = a.conv_b ? a.conv_b[d + c] : 0.0f;
        }
    }
    if constexpr (KC > 1) {
#pragma unroll
        for (int j = 0; j < KC - 1; ++j) {
            float h[V];
            xe<IO, KC, V>(a, b, d, ln.t0 - (KC - 1) + j, h);
#pragma unroll
            for (int c = 0; c < V; ++c) conv[c].hist[j] = h[c];
        }
    }
    // blocks of kBlk steps: every load of a block is issued before its arithmetic
    for (int64_t tb = ln.t0; tb < ln.t1; tb += kBlk) {
        float xv[kBlk][V], rv[kBlk][V];
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            if (tb + j < ln.t1) {
                const int64_t e = (b * a.L + tb + j) * a.Dn + d;
                ldv<IO, V>((const IO *)a.x_in + e, xv[j]);
                ldv<IO, V>((const IO *)a.dt_raw + e, rv[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            if (tb + j >= ln.t1) break;
            const int64_t e = (b * a.L + tb + j) * a.Dn + d;
            float u[V], dt[V];
#pragma unroll
            for (int c = 0; c < V; ++c) {
                u[c] = xv[j][c];
                if constexpr (KC > 0) u[c] = conv[c](xv[j][c]);
                dt[c] = softplus(rv[j][c] + bias[c]);
            }
            stv<IO, V>((IO *)a.u + e, u);
            stv<IO, V>((IO *)a.dt + e, dt);
        }
    }
}

// ---------------------------------------------------------------- chain rule
// a_t from the window win[k] = xe_{t-(KC-1)+k}, in the fused prefill's order (bias,
// then one fma per tap, oldest first).
template <int KC>
__device__ __forceinline__ float pre_act(const float *w, float cb, const float *win) {
    float acc = cb;
#pragma unroll
    for (int k = 0; k < KC; ++k) acc = __builtin_fmaf(w[k], win[k], acc);
    return acc;
}

__device__ __forceinline__ float silu_grad(float du, float pre) {
    const float s = rcp(1.0f + e2(-pre * kLog2e));
    return du * (s * __builtin_fmaf(pre, 1.0f - s, 1.0f));
}

template <typename IO, int KC, int V>
__global__ __launch_bounds__(256) void k_input_bwd(InBwdArgs a) {
    constexpr int P = KC + 2;  // partials per (chunk, batch row, channel): dw[KC], dcb, dbias
    constexpr int W = KC > 0 ? KC : 1;
    constexpr int F = KC > 1 ? KC - 1 : 1;
    const Lane ln = lane_of<V>(a);
    if (!ln.live) return;
    const int64_t b = ln.b, d = ln.d, row = b * a.L;
    float bias[V], dbias[V], w[V][W], dw[V][W], fut[V][F], cb[V], dcb[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
        bias[c] = a.dt_bias ? a.dt_bias[d + c] : 0.0f;
        dbias[c] = 0.0f;
        cb[c] = 0.0f;
        dcb[c] = 0.0f;
        if constexpr (KC > 0) {
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                w[c][k] = a.conv_w[(d + c) * KC + k];
                dw[c][k] = 0.0f;
            }
            cb[c] = a.conv_b ? a.conv_b[d + c] : 0.0f;
        }
    }
    if constexpr (KC > 1) {
        // da at the KC-1 steps after the chunk (0 past the sequence)
#pragma unroll
        for (int j = 0; j < KC - 1; ++j) {
            const int64_t s = ln.t1 + j;
#pragma unroll
            for (int c = 0; c < V; ++c) fut[c][j] = 0.0f;
            if (s < a.L) {
                float ws[KC][V], du[V];
#pragma unroll
                for (int k = 0; k < KC; ++k) xe<IO, KC, V>(a, b, d, s - (KC - 1) + k, ws[k]);
                ldv<IO, V>((const IO *)a.du + (row + s) * a.Dn + d, du);
#pragma unroll
                for (int c = 0; c < V; ++c) {
                    float win[KC];
#pragma unroll
                    for (int k = 0; k < KC; ++k) win[k] = ws[k][c];
                    fut[c][j] = silu_grad(du[c], pre_act<KC>(w[c], cb[c], win));
                }
            }
        }
    }
    // One step t (descending): du, dd, raw the step's values; win(k, c) = xe_{t-(KC-1)+k}.
    auto step = [&](int64_t t, const float (&du)[V], const float (&dd)[V], const float (&raw)[V],
                    auto win) {
        const int64_t e = (row + t) * a.Dn + d;
        float dx[V], dr[V];
#pragma unroll
        for (int c = 0; c < V; ++c) {
            dx[c] = du[c];
            if constexpr (KC > 0) {
                float acc = cb[c];
#pragma unroll
                for (int k = 0; k < KC; ++k) acc = __builtin_fmaf(w[c][k], win(k, c), acc);
                const float da = silu_grad(du[c], acc);
                // dx_in_t = sum_k w[k] da_{t+(KC-1)-k}: da_t with w[KC-1], da_{t+j} = fut[j-1]
                dx[c] = w[c][KC - 1] * da;
#pragma unroll
                for (int j = 1; j < KC; ++j) dx[c] = __builtin_fmaf(w[c][KC - 1 - j], fut[c][j - 1], dx[c]);
#pragma unroll
                for (int k = 0; k < KC; ++k) dw[c][k] = __builtin_fmaf(da, win(k, c), dw[c][k]);
                dcb[c] += da;
#pragma unroll
                for (int j = KC - 2; j >= 1; --j) fut[c][j] = fut[c][j - 1];
                if constexpr (KC > 1) fut[c][0] = da;
            }
            dr[c] = dd[c] * rcp(1.0f + e2(-(raw[c] + bias[c]) * kLog2e));
            dbias[c] += dr[c];
        }
        stv<IO, V>((IO *)a.dx_in + e, dx);
        stv<IO, V>((IO *)a.ddt_raw + e, dr);
    };
    constexpr int XW = kBlk + (KC > 0 ? KC - 1 : 0);  // inputs a block's windows span
    int64_t t = ln.t1 - 1;
    // whole blocks of kBlk steps, t - kBlk + 1 .. t, with every load issued first. A
    // block's windows span inputs tl-(KC-1) .. t; its top KC-1 (after the first block)
    // are the previous block's lowest ones, carried over instead of read again.
    float carry[F][V];
    bool have = false;
    for (; t - (kBlk - 1) >= ln.t0; t -= kBlk) {
        const int64_t tl = t - (kBlk - 1);
        float duv[kBlk][V], ddv[kBlk][V], rv[kBlk][V], xw[XW][V];
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int64_t e = (row + tl + j) * a.Dn + d;
            ldv<IO, V>((const IO *)a.du + e, duv[j]);
            ldv<IO, V>((const IO *)a.ddt + e, ddv[j]);
            ldv<IO, V>((const IO *)a.dt_raw + e, rv[j]);
        }
        if constexpr (KC > 0) {
#pragma unroll
            for (int i = 0; i < kBlk; ++i) xe<IO, KC, V>(a, b, d, tl - (KC - 1) + i, xw[i]);
#pragma unroll
            for (int i = 0; i < KC - 1; ++i) {
                if (have) {
#pragma unroll
                    for (int c = 0; c < V; ++c) xw[kBlk + i][c] = carry[i][c];
                } else {
                    xe<IO, KC, V>(a, b, d, tl - (KC - 1) + kBlk + i, xw[kBlk + i]);
                }
            }
        }
#pragma unroll
        for (int j = kBlk - 1; j >= 0; --j)
            step(tl + j, duv[j], ddv[j], rv[j], [&](int k, int c) { return xw[j + k][c]; });
        if constexpr (KC > 1) {
#pragma unroll
            for (int i = 0; i < KC - 1; ++i)
#pragma unroll
                for (int c = 0; c < V; ++c) carry[i][c] = xw[i][c];
            have = true;
        }
    }
    // the rest (fewer than kBlk steps), one at a time
    for (; t >= ln.t0; --t) {
        const int64_t e = (row + t) * a.Dn + d;
        float du[V], dd[V], raw[V], win[W][V];
        ldv<IO, V>((const IO *)a.du + e, du);
        ldv<IO, V>((const IO *)a.ddt + e, dd);
        ldv<IO, V>((const IO *)a.dt_raw + e, raw);
        if constexpr (KC > 0) {
#pragma unroll
            for (int k = 0; k < KC; ++k) xe<IO, KC, V>(a, b, d, t - (KC - 1) + k, win[k]);
        }
        step(t, du, dd, raw, [&](int k, int c) { return win[k][c]; });
    }
    if constexpr (KC > 1) {
        // the carried inputs before step 0: dxe_s, s = j - (KC-1), from da_0 .. da_{KC-2}
        // (fut now holds da_{t0} .. da_{t0+KC-2})
        if (ln.t0 == 0 && a.dconv_state0) {
#pragma unroll
            for (int j = 0; j < KC - 1; ++j) {
                float g[V];
#pragma unroll
                for (int c = 0; c < V; ++c) {
                    g[c] = 0.0f;
#pragma unroll
                    for (int k = 0; k <= j; ++k) g[c] = __builtin_fmaf(w[c][k], fut[c][j - k], g[c]);
                }
                stv<IO, V>((IO *)a.dconv_state0 + (b * (KC - 1) + j) * a.Dn + d, g);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < V; ++c) {
        float *pp = a.part + (((int64_t)blockIdx.y * a.batch + b) * a.Dn + d + c) * P;
#pragma unroll
        for (int k = 0; k < KC; ++k) pp[k] = dw[c][k];
        pp[KC] = dcb[c];
        pp[KC + 1] = dbias[c];
    }
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

template <typename IO, int KC, int V>
hipError_t launch_t(const InBwdArgs &a, bool fwd, hipStream_t s) {
    const dim3 grid((unsigned)(a.batch * ((a.Dn + 256 * V - 1) / (256 * V))), (unsigned)a.n_chunks);
    if (fwd) {
        hipLaunchKernelGGL((k_input_fwd<IO, KC, V>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_input_bwd<IO, KC, V>), grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = a.Dn * (KC + 2);
    hipLaunchKernelGGL((k_input_bwd_reduce<KC>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// 8-byte accesses (V channels per lane) when every [rows][Dn] array allows them: Dn a
// multiple of V and every base 8-byte aligned; else one channel per lane.
template <typename IO, int KC>
hipError_t launch_v(const InBwdArgs &a, bool fwd, hipStream_t s) {
    constexpr int V = sizeof(IO) == 2 ? 4 : 2;
    const void *ptrs[] = {a.x_in, a.dt_raw, a.conv_state0, a.u, a.dt, a.du, a.ddt, a.dx_in,
                          a.ddt_raw, a.dconv_state0};
    bool wide = a.Dn % V == 0;
    for (const void *p : ptrs) wide = wide && ((uintptr_t)p % 8 == 0);
    return wide ? launch_t<IO, KC, V>(a, fwd, s) : launch_t<IO, KC, 1>(a, fwd, s);
}

template <typename IO>
hipError_t launch_k(const InBwdArgs &a, bool fwd, hipStream_t s) {
    switch (a.conv_k) {
        case 0: return launch_v<IO, 0>(a, fwd, s);
        case 1: return launch_v<IO, 1>(a, fwd, s);
        case 2: return launch_v<IO, 2>(a, fwd, s);
        case 3: return launch_v<IO, 3>(a, fwd, s);
        case 4: return launch_v<IO, 4>(a, fwd, s);
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
