// step.hip -- single-token decode for many (layer, sequence) states (gfx950).
//
// A state-space layer needs only its previous state and the new token to emit the
// next output, so decoding keeps one fixed-size state per layer instead of a
// growing cache ("Jamba — SSM-Transformer Híbrido", section "Um SSM em uma
// página"; the same section of the zh lesson page). One call advances every
// (layer, sequence, channel) by one token, in place.
//
// The work is bound by HBM: per channel the 16-state fp32 state is read and
// written (128 of the 136 bytes moved). G lanes share one channel, each owning
// K = N / G consecutive states, so a wave reads and writes the state with fully
// coalesced 16-byte accesses; the G partial outputs are combined with lane
// shuffles in a fixed pairwise tree.
//
// The replay kernels run one thread per channel with plain loops and perform the
// same fp32 operations in the same order (the tree included), so that the decode
// kernels can be checked bit for bit against them. The library is built with
// floating-point contraction off; every fused multiply-add below is explicit.
//
// The fused entry point adds the MambaBlock input stage (ssm_input_stage.h): x_t is
// the convolution's new input and dt_t the raw dt projection output. One lane per
// channel computes u = silu(conv) from the carried convolution state and
// dt = softplus(dt + bias), hands both to the G lanes of the channel's state update
// (k_step), and writes the shifted conv state back; the replay performs the same
// operations, so the two agree bit for bit.
#include "ssm_device.h"
#include "ssm_input_stage.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// Grid: x = blocks of 256 threads over channels (the real-state kernels) or over
// (channel, group lane) pairs (the complex-state kernel), y = sequence q, z = layer l.
// Channel index ch = (l * n_seq + q) * Dn + d; lq = l * n_seq + q.
struct Chan {
    int64_t ch, lq;
    int64_t l, d;
};

template <int G>
__device__ __forceinline__ bool chan_of(const StepArgs &a, Chan &c, int &g) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    c.d = t / G;  // G is a power of two
    g = (int)(t % G);
    if (c.d >= a.Dn) return false;
    c.l = blockIdx.z;
    c.lq = (int64_t)blockIdx.z * a.n_seq + blockIdx.y;
    c.ch = c.lq * a.Dn + c.d;
    return true;
}

// Input stage of one decode token: apply() maps the loaded (x, dt) of a channel to the
// values the recurrence uses; store() writes what the next token needs. store() is
// called after the channel's output, so its stores wait on nothing.
struct NoStepInput {
    static constexpr bool kTrap = false;
    template <typename Chan>
    __device__ __forceinline__ void apply(const StepArgs &, const Chan &, float &, float &) {}
    __device__ __forceinline__ void store(const StepArgs &) const {}
};

// Ordered as in ssm_input_stage.h: dt = softplus(dt + bias); u = silu(conv over the
// KC-1 carried inputs and x) (KC = 0: u = x). store() puts the KC-1 newest inputs,
// x included, in place of the old state.
template <typename IO, int KC>
struct StepMamba {
    static constexpr bool kTrap = false;
    ConvSilu<(KC > 0 ? KC : 1)> conv;
    IO *st;  // the channel's conv state: row j at st + j * Dn

    template <typename Chan>
    __device__ __forceinline__ void apply(const StepArgs &a, const Chan &c, float &xv, float &dv) {
        const int64_t pd = c.l * a.Dn + c.d;  // (layer, channel) parameter index
        dv = softplus(dv + (a.dt_bias ? a.dt_bias[pd] : 0.0f));
        if constexpr (KC > 0) {
#pragma unroll
            for (int k = 0; k < KC; ++k) conv.w[k] = a.conv_w[pd * KC + k];
            conv.bias = a.conv_b ? a.conv_b[pd] : 0.0f;
            st = (IO *)a.conv_state + c.lq * (KC - 1) * a.Dn + c.d;
            if constexpr (KC > 1) {
#pragma unroll
                for (int j = 0; j < KC - 1; ++j) conv.hist[j] = Io<IO>::ld(st + j * a.Dn);
            }
            xv = conv(xv);
        }
    }
    __device__ __forceinline__ void store(const StepArgs &a) const {
        if constexpr (KC > 1) {
#pragma unroll
            for (int j = 0; j < KC - 1; ++j) Io<IO>::st(st + j * a.Dn, conv.hist[j]);
        }
    }
};

// The exponential-trapezoidal step (see scan_real.hip): x and dt as given, plus the
// previous token's x (x_prev, per channel) and B (B_prev, per sequence); null x_prev
// and B_prev (the entry point accepts both or neither) mean no previous input; lam is
// the token's weight per channel (null: 1/2). The update of state n is
//     h = a (h + up B_prev[n]) + uc B[n],   a = exp(dt A[n]),
//     up = (dt (1 - lam)) x_prev,   uc = (dt lam) x.
template <typename IO>
struct StepTrap {
    static constexpr bool kTrap = true;
    float xprev, lam;
    template <typename Chan>
    __device__ __forceinline__ void apply(const StepArgs &a, const Chan &c, float &, float &) {
        xprev = a.x_prev ? Io<IO>::ld((const IO *)a.x_prev + c.ch) : 0.0f;
        lam = a.lam ? Io<IO>::ld((const IO *)a.lam + c.ch) : 0.5f;
    }
    // The two input weights times their inputs, in the order both decode kernels use.
    __device__ __forceinline__ void taps(float dv, float xv, float &up, float &uc) const {
        const float wc = dv * lam, wp = dv * (1.0f - lam);
        up = wp * xprev;
        uc = wc * xv;
    }
    __device__ __forceinline__ void store(const StepArgs &) const {}
};

// The state is read once and written once per call: non-temporal (streaming) 16-byte
// accesses keep it from displacing the reused A, B, C rows in the caches.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void ld_state4(const float *p, float *v) {
    const f4v q = __builtin_nontemporal_load((const f4v *)p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void st_state4(float *p, const float *v) {
    f4v q;
    q.x = v[0]; q.y = v[1]; q.z = v[2]; q.w = v[3];
    __builtin_nontemporal_store(q, (f4v *)p);
}

// Vector load of K consecutive elements (K = 1, 2 or 4; 4-byte aligned for K >= 2
// with bf16 and 8/16-byte aligned for f32, which the layouts guarantee).
template <typename IO, int K> struct VecLd;
template <int K> struct VecLd<float, K> {
    static __device__ __forceinline__ void ld(const float *p, float (&v)[K]) {
        if constexpr (K == 4) {
            const float4 q = *(const float4 *)p;
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else if constexpr (K == 2) {
            const float2 q = *(const float2 *)p;
            v[0] = q.x; v[1] = q.y;
        } else {
            v[0] = *p;
        }
    }
};
template <int K> struct VecLd<bf16_bits, K> {
    static __device__ __forceinline__ void ld(const bf16_bits *p, float (&v)[K]) {
        if constexpr (K == 4) {
            const uint2 q = *(const uint2 *)p;
            v[0] = bf16_to_f32(q.x & 0xffffu); v[1] = __uint_as_float(q.x & 0xffff0000u);
            v[2] = bf16_to_f32(q.y & 0xffffu); v[3] = __uint_as_float(q.y & 0xffff0000u);
        } else if constexpr (K == 2) {
            const uint32_t q = *(const uint32_t *)p;
            v[0] = bf16_to_f32(q & 0xffffu); v[1] = __uint_as_float(q & 0xffff0000u);
        } else {
            v[0] = bf16_to_f32(*p);
        }
    }
};

template <int G>
__device__ __forceinline__ float group_sum(float p) {
    // Pairwise tree over the G lanes of a group: after the xor-1 step lanes hold
    // p0+p1, p2+p3, ...; after xor-2, (p0+p1)+(p2+p3), ... Addition is commutative,
    // so both lanes of a pair compute the same bits.
#pragma unroll
    for (int m = 1; m < G; m <<= 1) p = p + __shfl_xor(p, m, 64);
    return p;
}

template <int G>
__device__ __forceinline__ float tree_sum(float (&p)[G]) {
#pragma unroll
    for (int s = 1; s < G; s <<= 1)
#pragma unroll
        for (int i = 0; i < G; i += 2 * s) p[i] = p[i] + p[i + s];
    return p[0];
}

// ---------------------------------------------------------------- real state
template <int N> struct RealGroups {
    static constexpr int G = N >= 8 ? N / 4 : 1;
    static constexpr int K = N / G;
};

// A wave owns 64 consecutive channels. Each lane first loads (and, with an input
// stage, transforms) x and dt of its "home" channel (wave base + lane), so per-channel
// work is done once, not once per lane of the channel. The state update then takes
// G rounds, in which lane t works on channel r * 64/G + t/G, states (t % G) * K ..;
// it fetches that channel's (x, dt) from the home lane with a lane permute, and the
// round's output sum goes back to the home lane the same way. The home lane finishes
// y (and writes the conv state). Each wave has 4G state loads in flight before its
// first arithmetic. Every operation and its order are those of the replay, so the
// results agree bit for bit. Lanes past the last channel are clamped to it for
// their loads and store nothing; no lane leaves early, since its home and round
// channels differ.
template <typename IO, int N, bool GATED, typename In>
__global__ __launch_bounds__(256) void k_step(StepArgs a) {
    constexpr int G = RealGroups<N>::G, K = RealGroups<N>::K;
    constexpr int CPR = 64 / G;  // channels per round
    const int lane = (int)(threadIdx.x & 63u);
    const int64_t d0 = (int64_t)blockIdx.x * 256 + (threadIdx.x & ~63u);
    const int g = lane % G;
    Chan hc;
    hc.l = blockIdx.z;
    hc.lq = (int64_t)blockIdx.z * a.n_seq + blockIdx.y;
    const bool home_ok = d0 + lane < a.Dn;
    hc.d = home_ok ? d0 + lane : a.Dn - 1;
    hc.ch = hc.lq * a.Dn + hc.d;

    // Every load first: the state and A of each round's channel, the token's B and C
    // (one row per (layer, sequence), the same in every round), the home channel's
    // x, dt, z, D and (in apply) the input-stage parameters and conv state.
    float hv[G][K], av[G][K], bv[K], cv[K];
    bool rok[G];
    int64_t rch[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const int64_t d = d0 + r * CPR + lane / G;
        rok[r] = d < a.Dn;
        const int64_t dc = rok[r] ? d : a.Dn - 1;
        rch[r] = hc.lq * a.Dn + dc;
        const float *hp = a.h + rch[r] * N + g * K;
        if constexpr (K == 4) ld_state4(hp, hv[r]);
        else VecLd<float, K>::ld(hp, hv[r]);
        VecLd<float, K>::ld(a.A + (hc.l * a.Dn + dc) * N + g * K, av[r]);
    }
    VecLd<IO, K>::ld((const IO *)a.B + hc.lq * N + g * K, bv);
    VecLd<IO, K>::ld((const IO *)a.C + hc.lq * N + g * K, cv);
    float pv[K];  // exponential-trapezoidal step: the previous token's B
    if constexpr (In::kTrap) {
        if (a.B_prev) {
            VecLd<IO, K>::ld((const IO *)a.B_prev + hc.lq * N + g * K, pv);
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) pv[k] = 0.0f;
        }
    }
    float xv = Io<IO>::ld((const IO *)a.x + hc.ch);
    float dv = Io<IO>::ld((const IO *)a.dt + hc.ch);
    const float zv = GATED ? Io<IO>::ld((const IO *)a.z + hc.ch) : 0.0f;
    const float Dd = a.D[hc.l * a.Dn + hc.d];
    In in;
    in.apply(a, hc, xv, dv);
    float uph = 0.0f, uch = 0.0f;  // exponential-trapezoidal step: the home channel's taps
    if constexpr (In::kTrap) in.taps(dv, xv, uph, uch);

    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const int src = r * CPR + lane / G;
        const float dr = G == 1 ? dv : __shfl(dv, src, 64);
        float p = 0.0f;
        if constexpr (In::kTrap) {
            const float up = G == 1 ? uph : __shfl(uph, src, 64);
            const float uc = G == 1 ? uch : __shfl(uch, src, 64);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float a2 = av[r][k] * kLog2e;
                hv[r][k] = __builtin_fmaf(e2(dr * a2), __builtin_fmaf(up, pv[k], hv[r][k]), uc * bv[k]);
                p = __builtin_fmaf(cv[k], hv[r][k], p);
            }
        } else {
            const float xr = G == 1 ? xv : __shfl(xv, src, 64);
            const float u = dr * xr;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float a2 = av[r][k] * kLog2e;
                hv[r][k] = __builtin_fmaf(e2(dr * a2), hv[r][k], u * bv[k]);
                p = __builtin_fmaf(cv[k], hv[r][k], p);
            }
        }
        const float s = group_sum<G>(p);
        if (rok[r]) {
            float *hp = a.h + rch[r] * N + g * K;
            if constexpr (K == 4) {
                st_state4(hp, hv[r]);
            } else if constexpr (K == 2) {
                *(float2 *)hp = make_float2(hv[r][0], hv[r][1]);
            } else {
                hp[0] = hv[r][0];
            }
        }
        if constexpr (G == 1) {
            acc = s;
        } else {
            const float sh = __shfl(s, (lane % CPR) * G, 64);
            if (lane / CPR == r) acc = sh;
        }
    }
    if (home_ok) {
        float yv = __builtin_fmaf(Dd, xv, acc);
        if (GATED) yv = yv * silu(zv);
        Io<IO>::st((IO *)a.y + hc.ch, yv);
        in.store(a);
    }
}

template <typename IO, int N, bool GATED, typename In>
__global__ __launch_bounds__(256) void k_step_replay(StepArgs a) {
    constexpr int G = RealGroups<N>::G, K = RealGroups<N>::K;
    Chan c;
    int g0;
    if (!chan_of<1>(a, c, g0)) return;
    const int64_t ch = c.ch;
    float *hp = a.h + ch * N;
    const float *Ap = a.A + (c.l * a.Dn + c.d) * N;
    const IO *Bp = (const IO *)a.B + c.lq * N;
    const IO *Cp = (const IO *)a.C + c.lq * N;
    float xv = Io<IO>::ld((const IO *)a.x + ch);
    float dv = Io<IO>::ld((const IO *)a.dt + ch);
    In in;
    in.apply(a, c, xv, dv);
    float p[G];
    if constexpr (In::kTrap) {
        const IO *Pp = a.B_prev ? (const IO *)a.B_prev + c.lq * N : nullptr;
        float up, uc;
        in.taps(dv, xv, up, uc);
        for (int g = 0; g < G; ++g) {
            p[g] = 0.0f;
            for (int k = 0; k < K; ++k) {
                const int n = g * K + k;
                const float a2 = Ap[n] * kLog2e;
                const float pb = Pp ? Io<IO>::ld(Pp + n) : 0.0f;
                hp[n] = __builtin_fmaf(e2(dv * a2), __builtin_fmaf(up, pb, hp[n]), uc * Io<IO>::ld(Bp + n));
                p[g] = __builtin_fmaf(Io<IO>::ld(Cp + n), hp[n], p[g]);
            }
        }
    } else {
        const float u = dv * xv;
        for (int g = 0; g < G; ++g) {
            p[g] = 0.0f;
            for (int k = 0; k < K; ++k) {
                const int n = g * K + k;
                const float a2 = Ap[n] * kLog2e;
                hp[n] = __builtin_fmaf(e2(dv * a2), hp[n], u * Io<IO>::ld(Bp + n));
                p[g] = __builtin_fmaf(Io<IO>::ld(Cp + n), hp[n], p[g]);
            }
        }
    }
    float yv = __builtin_fmaf(a.D[c.l * a.Dn + c.d], xv, tree_sum<G>(p));
    if (GATED) yv = yv * silu(Io<IO>::ld((const IO *)a.z + ch));
    Io<IO>::st((IO *)a.y + ch, yv);
    in.store(a);
}

// ---------------------------------------------------------------- complex state
template <int N> struct CplxGroups {
    static constexpr int G = N >= 2 ? N / 2 : 1;
    static constexpr int K = N / G;
};

// One complex state update: h <- exp(dt A) h + dt x B.
__device__ __forceinline__ void cstep(float dv, float u, float are, float aim, float br, float bi,
                                      float &hr, float &hi) {
    const float mag = e2(dv * (are * kLog2e));
    const float r = fract(dv * (aim * kInv2Pi));
    const float pr = mag * cos_rev(r), pi = mag * sin_rev(r);
    const float nr = __builtin_fmaf(pr, hr, __builtin_fmaf(-pi, hi, u * br));
    const float ni = __builtin_fmaf(pr, hi, __builtin_fmaf(pi, hr, u * bi));
    hr = nr;
    hi = ni;
}

template <typename IO, int N, bool GATED>
__global__ __launch_bounds__(256) void k_step_c(StepArgs a) {
    constexpr int G = CplxGroups<N>::G, K = CplxGroups<N>::K;
    Chan c;
    int g;
    if (!chan_of<G>(a, c, g)) return;
    const int64_t ch = c.ch;
    float *hp = a.h + (ch * N + g * K) * 2;
    const float *Ap = a.A + ((c.l * a.Dn + c.d) * N + g * K) * 2;
    const IO *Bp = (const IO *)a.B + (c.lq * N + g * K) * 2;
    const IO *Cp = (const IO *)a.C + (c.lq * N + g * K) * 2;
    float hv[2 * K], av[2 * K];
    if constexpr (K == 2) {
        ld_state4(hp, hv);
        const float4 a4 = *(const float4 *)Ap;
        av[0] = a4.x; av[1] = a4.y; av[2] = a4.z; av[3] = a4.w;
    } else {
#pragma unroll
        for (int k = 0; k < 2 * K; ++k) { hv[k] = hp[k]; av[k] = Ap[k]; }
    }
    const float xv = Io<IO>::ld((const IO *)a.x + ch);
    const float dv = Io<IO>::ld((const IO *)a.dt + ch);
    const float u = dv * xv;
    float p = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        cstep(dv, u, av[2 * k], av[2 * k + 1], Io<IO>::ld(Bp + 2 * k), Io<IO>::ld(Bp + 2 * k + 1),
              hv[2 * k], hv[2 * k + 1]);
        p = __builtin_fmaf(Io<IO>::ld(Cp + 2 * k), hv[2 * k], p);
        p = __builtin_fmaf(-Io<IO>::ld(Cp + 2 * k + 1), hv[2 * k + 1], p);
    }
    const float acc = group_sum<G>(p);
    if constexpr (K == 2) {
        st_state4(hp, hv);
    } else {
#pragma unroll
        for (int k = 0; k < 2 * K; ++k) hp[k] = hv[k];
    }
    if (g == 0) {
        float yv = __builtin_fmaf(a.D[c.l * a.Dn + c.d], xv, acc);
        if (GATED) yv = yv * silu(Io<IO>::ld((const IO *)a.z + ch));
        Io<IO>::st((IO *)a.y + ch, yv);
    }
}

template <typename IO, int N, bool GATED>
__global__ __launch_bounds__(256) void k_step_c_replay(StepArgs a) {
    constexpr int G = CplxGroups<N>::G, K = CplxGroups<N>::K;
    Chan c;
    int g0;
    if (!chan_of<1>(a, c, g0)) return;
    const int64_t ch = c.ch;
    float *hp = a.h + ch * N * 2;
    const float *Ap = a.A + (c.l * a.Dn + c.d) * N * 2;
    const IO *Bp = (const IO *)a.B + c.lq * N * 2;
    const IO *Cp = (const IO *)a.C + c.lq * N * 2;
    const float xv = Io<IO>::ld((const IO *)a.x + ch);
    const float dv = Io<IO>::ld((const IO *)a.dt + ch);
    const float u = dv * xv;
    float p[G];
    for (int g = 0; g < G; ++g) {
        p[g] = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int n = g * K + k;
            float hr = hp[2 * n], hi = hp[2 * n + 1];
            cstep(dv, u, Ap[2 * n], Ap[2 * n + 1], Io<IO>::ld(Bp + 2 * n),
                  Io<IO>::ld(Bp + 2 * n + 1), hr, hi);
            hp[2 * n] = hr;
            hp[2 * n + 1] = hi;
            p[g] = __builtin_fmaf(Io<IO>::ld(Cp + 2 * n), hr, p[g]);
            p[g] = __builtin_fmaf(-Io<IO>::ld(Cp + 2 * n + 1), hi, p[g]);
        }
    }
    float yv = __builtin_fmaf(a.D[c.l * a.Dn + c.d], xv, tree_sum<G>(p));
    if (GATED) yv = yv * silu(Io<IO>::ld((const IO *)a.z + ch));
    Io<IO>::st((IO *)a.y + ch, yv);
}

// ---------------------------------------------------------------- launch
inline dim3 grid_for(const StepArgs &a, int lanes_per_ch) {
    return dim3((unsigned)((a.Dn * lanes_per_ch + 255) / 256), (unsigned)a.n_seq,
                (unsigned)a.n_layers);
}

template <typename IO, int N, typename In = NoStepInput>
hipError_t launch_real_n(const StepArgs &a, bool gated, bool replay, hipStream_t s) {
    const dim3 blk(256), grid(grid_for(a, 1));  // both kernels: 256 channels per block
    if (replay) {
        if (gated) hipLaunchKernelGGL((k_step_replay<IO, N, true, In>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_step_replay<IO, N, false, In>), grid, blk, 0, s, a);
    } else {
        if (gated) hipLaunchKernelGGL((k_step<IO, N, true, In>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_step<IO, N, false, In>), grid, blk, 0, s, a);
    }
    return hipGetLastError();
}

template <typename IO, typename In>
hipError_t launch_fused_n(const StepArgs &a, int d_state, bool gated, bool replay, hipStream_t s) {
    switch (d_state) {
        case 1: return launch_real_n<IO, 1, In>(a, gated, replay, s);
        case 2: return launch_real_n<IO, 2, In>(a, gated, replay, s);
        case 4: return launch_real_n<IO, 4, In>(a, gated, replay, s);
        case 8: return launch_real_n<IO, 8, In>(a, gated, replay, s);
        case 16: return launch_real_n<IO, 16, In>(a, gated, replay, s);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_fused_io(const StepArgs &a, int d_state, bool gated, bool replay, hipStream_t s) {
    switch (a.conv_k) {
        case 0: return launch_fused_n<IO, StepMamba<IO, 0>>(a, d_state, gated, replay, s);
        case 1: return launch_fused_n<IO, StepMamba<IO, 1>>(a, d_state, gated, replay, s);
        case 2: return launch_fused_n<IO, StepMamba<IO, 2>>(a, d_state, gated, replay, s);
        case 3: return launch_fused_n<IO, StepMamba<IO, 3>>(a, d_state, gated, replay, s);
        case 4: return launch_fused_n<IO, StepMamba<IO, 4>>(a, d_state, gated, replay, s);
    }
    return hipErrorInvalidValue;
}

template <typename IO, int N>
hipError_t launch_cplx_n(const StepArgs &a, bool gated, bool replay, hipStream_t s) {
    const dim3 blk(256), grid(grid_for(a, replay ? 1 : CplxGroups<N>::G));
    if (replay) {
        if (gated) hipLaunchKernelGGL((k_step_c_replay<IO, N, true>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_step_c_replay<IO, N, false>), grid, blk, 0, s, a);
    } else {
        if (gated) hipLaunchKernelGGL((k_step_c<IO, N, true>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_step_c<IO, N, false>), grid, blk, 0, s, a);
    }
    return hipGetLastError();
}

template <typename IO, bool CPLX>
hipError_t launch_io(const StepArgs &a, int d_state, bool gated, bool replay, hipStream_t s) {
    switch (d_state) {
        case 1: return CPLX ? launch_cplx_n<IO, 1>(a, gated, replay, s) : launch_real_n<IO, 1>(a, gated, replay, s);
        case 2: return CPLX ? launch_cplx_n<IO, 2>(a, gated, replay, s) : launch_real_n<IO, 2>(a, gated, replay, s);
        case 4: return CPLX ? launch_cplx_n<IO, 4>(a, gated, replay, s) : launch_real_n<IO, 4>(a, gated, replay, s);
        case 8: return CPLX ? launch_cplx_n<IO, 8>(a, gated, replay, s) : launch_real_n<IO, 8>(a, gated, replay, s);
        case 16: return CPLX ? launch_cplx_n<IO, 16>(a, gated, replay, s) : launch_real_n<IO, 16>(a, gated, replay, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_step_real(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                            hipStream_t s) {
    return io == 0 ? launch_io<float, false>(a, d_state, gated, replay, s)
                   : launch_io<bf16_bits, false>(a, d_state, gated, replay, s);
}

hipError_t launch_step_complex(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                               hipStream_t s) {
    return io == 0 ? launch_io<float, true>(a, d_state, gated, replay, s)
                   : launch_io<bf16_bits, true>(a, d_state, gated, replay, s);
}

hipError_t launch_step_trap(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                            hipStream_t s) {
    return io == 0 ? launch_fused_n<float, StepTrap<float>>(a, d_state, gated, replay, s)
                   : launch_fused_n<bf16_bits, StepTrap<bf16_bits>>(a, d_state, gated, replay, s);
}

hipError_t launch_step_fused(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                             hipStream_t s) {
    return io == 0 ? launch_fused_io<float>(a, d_state, gated, replay, s)
                   : launch_fused_io<bf16_bits>(a, d_state, gated, replay, s);
}

}  // namespace ssm
