// scan_complex.hip -- prefill with a complex diagonal state (gfx950).
//
// The Mamba-3 item on complex-valued state updates of "Jamba — SSM-Transformer
// Híbrido" (ai-engineering.academy) equates a complex diagonal state with a
// data-dependent rotary embedding on the state. Per channel d and state n, with
// A = -a + i theta:
//     Abar_t = exp(dt_t A) = exp(-dt_t a) (cos(dt_t theta) + i sin(dt_t theta))
//     h_t    = Abar_t h_{t-1} + dt_t B_t x_t              (B_t complex)
//     y_t    = Re(sum_n C_t[n] h_t[n]) + D x_t, then the optional silu(z) gate.
// The work split is that of the real-state scan: one lane per channel with the
// state (2N floats) in VGPRs, B/C through scalar loads, chunks + carry scan +
// rescan. The rotation angle is kept in revolutions (theta / 2 pi) so that the
// hardware sine/cosine (which take revolutions) get an exactly range-reduced
// argument from fract().
#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_stream.h"

namespace ssm {
namespace {

struct LaneId {
    int64_t b, d;
};

__device__ __forceinline__ LaneId lane_id(const ScanArgs &a) {
    LaneId r;
    r.b = (int64_t)blockIdx.x / a.dblocks;
    r.d = ((int64_t)blockIdx.x % a.dblocks) * a.threads + threadIdx.x;
    return r;
}

// exp(dt * (are + i aim)) with are2 = are log2 e and arev = aim / 2 pi.
__device__ __forceinline__ void decay_rotation(float dv, float are2, float arev, float &pr,
                                               float &pi) {
    const float mag = e2(dv * are2);
    const float r = fract(dv * arev);
    pr = mag * cos_rev(r);
    pi = mag * sin_rev(r);
}

// Chunk summary as in the real-state scan. The rotation has modulus one, so only the
// real part of A decays and the decay horizon is computed from Re A.
template <typename IO, int N>
__global__ __launch_bounds__(256) void k_chunk_summary_c(ScanArgs a) {
    const LaneId ln = lane_id(a);
    if (ln.d >= a.Dn) return;
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const int64_t t1 = t0 + a.T;
    const int64_t Dn = a.Dn;
    float Ar2[N], Arev[N], hr[N], hi[N];
    float amax = -INFINITY;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        Ar2[n] = a.A[(ln.d * N + n) * 2 + 0] * kLog2e;
        Arev[n] = a.A[(ln.d * N + n) * 2 + 1] * kInv2Pi;
        amax = fmaxf(amax, Ar2[n]);
        hr[n] = 0.0f;
        hi[n] = 0.0f;
    }
    const int64_t row0 = (ln.b * a.L + t0) * Dn;
    const uint32_t T = (uint32_t)a.T;
    const uint32_t rb = (uint32_t)(Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const RowStream<IO> dts((const IO *)a.dt + row0);
    const uint32_t ts = horizon_start<IO>(dts, voff, rb, T, amax);
    const IO *Bp = (const IO *)a.B + ln.b * a.L * N * 2;
    const int64_t rw = row0 + (int64_t)ts * Dn;
    const RowStream<IO> xs((const IO *)a.x + rw), dws((const IO *)a.dt + rw);
    double S = 0.0;
    stream_steps<IO, false, 2>(xs, dws, dws, voff, rb, T - ts, kSummaryPrioScale, [&](uint32_t i, float xv, float dv, float) {
        const int64_t t = t0 + ts + i;
        const float u = dv * xv;
        S += (double)dv;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float br = Uniform<IO>::ld(Bp, (t * N + n) * 2 + 0);
            const float bi = Uniform<IO>::ld(Bp, (t * N + n) * 2 + 1);
            float pr, pi;
            decay_rotation(dv, Ar2[n], Arev[n], pr, pi);
            const float nr = __builtin_fmaf(pr, hr[n], __builtin_fmaf(-pi, hi[n], u * br));
            const float ni = __builtin_fmaf(pr, hi[n], __builtin_fmaf(pi, hr[n], u * bi));
            hr[n] = nr;
            hi[n] = ni;
        }
    });
    const size_t o = (((size_t)c * a.batch + ln.b) * a.Dn + ln.d) * N * 2;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float pr = 0.0f, pi = 0.0f;
        if (ts == 0) {
            // total decay and rotation of the chunk: exp(S * A); the angle in double
            const double aim = (double)a.A[(ln.d * N + n) * 2 + 1];
            const double rev = aim * kInv2PiD * S;
            const float r = (float)(rev - floor(rev));
            const float mag = e2(Ar2[n] * (float)S);
            pr = mag * cos_rev(r);
            pi = mag * sin_rev(r);
        }
        a.sumP[o + 2 * n + 0] = pr;
        a.sumP[o + 2 * n + 1] = pi;
        a.sumH[o + 2 * n + 0] = hr[n];
        a.sumH[o + 2 * n + 1] = hi[n];
    }
}

// ---------------------------------------------------------------- carry scan
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xf, false));
}

// Segment (p, h) maps an incoming state s to p*s + h (complex). Combine with the
// earlier segment (pe, he): (p pe, p he + h); missing sources read (1, 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_step(float &pr, float &pi, float &hr, float &hi) {
    const float per = dpp<CTRL, ROW_MASK>(1.0f, pr), pei = dpp<CTRL, ROW_MASK>(0.0f, pi);
    const float her = dpp<CTRL, ROW_MASK>(0.0f, hr), hei = dpp<CTRL, ROW_MASK>(0.0f, hi);
    const float nhr = __builtin_fmaf(pr, her, __builtin_fmaf(-pi, hei, hr));
    const float nhi = __builtin_fmaf(pr, hei, __builtin_fmaf(pi, her, hi));
    const float npr = __builtin_fmaf(pr, per, -(pi * pei));
    const float npi = __builtin_fmaf(pr, pei, pi * per);
    pr = npr; pi = npi; hr = nhr; hi = nhi;
}

__device__ __forceinline__ void wave_scan(float &pr, float &pi, float &hr, float &hi) {
    scan_step<0x111, 0xf>(pr, pi, hr, hi);
    scan_step<0x112, 0xf>(pr, pi, hr, hi);
    scan_step<0x114, 0xf>(pr, pi, hr, hi);
    scan_step<0x118, 0xf>(pr, pi, hr, hi);
    scan_step<0x142, 0xa>(pr, pi, hr, hi);
    scan_step<0x143, 0xc>(pr, pi, hr, hi);
}

// M = batch * Dn * N complex columns, stored as (re, im) pairs.
__global__ __launch_bounds__(256) void k_carry_c(ScanArgs a, int64_t M) {
    __shared__ float2 sP[64][65];
    __shared__ float2 sH[64][65];
    __shared__ float2 sCarry[64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * 64;
    const int64_t col = col0 + lane;
    const int nsum = a.n_chunks - 1;
    const float2 *P2 = (const float2 *)a.sumP;
    float2 *H2 = (float2 *)a.sumH;
    if (threadIdx.x < 64)
        sCarry[lane] = (col < M && a.h0) ? ((const float2 *)a.h0)[col] : make_float2(0.0f, 0.0f);
    for (int k0 = 0; k0 < nsum; k0 += 64) {
        const int rows = min(64, nsum - k0);
        __syncthreads();
        for (int r = w; r < rows; r += 4) {
            if (col < M) {
                sP[r][lane] = P2[(size_t)(k0 + r) * M + col];
                sH[r][lane] = H2[(size_t)(k0 + r) * M + col];
            }
        }
        __syncthreads();
        for (int jj = 0; jj < 16; ++jj) {
            const int j = w * 16 + jj;
            if (col0 + j >= M) break;
            float2 p = lane < rows ? sP[lane][j] : make_float2(1.0f, 0.0f);
            float2 h = lane < rows ? sH[lane][j] : make_float2(0.0f, 0.0f);
            wave_scan(p.x, p.y, h.x, h.y);
            const float2 cs = sCarry[j];
            float2 out;
            out.x = __builtin_fmaf(p.x, cs.x, __builtin_fmaf(-p.y, cs.y, h.x));
            out.y = __builtin_fmaf(p.x, cs.y, __builtin_fmaf(p.y, cs.x, h.y));
            if (lane < rows) sH[lane][j] = out;
            float2 next;
            next.x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(out.x), rows - 1));
            next.y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(out.y), rows - 1));
            if (lane == 0) sCarry[j] = next;
        }
        __syncthreads();
        for (int r = w; r < rows; r += 4)
            if (col < M) H2[(size_t)(k0 + r) * M + col] = sH[r][lane];
    }
}

// ---------------------------------------------------------------- rescan + epilogue
template <typename IO, int N, bool GATED>
__global__ __launch_bounds__(256) void k_chunk_scan_c(ScanArgs a) {
    const LaneId ln = lane_id(a);
    if (ln.d >= a.Dn) return;
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const int64_t t1 = min(a.L, t0 + a.T);
    const size_t col = (size_t)(ln.b * a.Dn + ln.d) * N * 2;
    const float *hin = c == 0 ? (a.h0 ? a.h0 + col : nullptr)
                              : a.sumH + (size_t)(c - 1) * a.batch * a.Dn * N * 2 + col;
    float Ar2[N], Arev[N], hr[N], hi[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        Ar2[n] = a.A[(ln.d * N + n) * 2 + 0] * kLog2e;
        Arev[n] = a.A[(ln.d * N + n) * 2 + 1] * kInv2Pi;
        hr[n] = hin ? hin[2 * n + 0] : 0.0f;
        hi[n] = hin ? hin[2 * n + 1] : 0.0f;
    }
    const float Dd = a.D[ln.d];
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> xs((const IO *)a.x + row0), dts((const IO *)a.dt + row0),
        zs(GATED ? (const IO *)a.z + row0 : (const IO *)a.x + row0), ys((IO *)a.y + row0);
    const IO *Bp = (const IO *)a.B + ln.b * a.L * N * 2;
    const IO *Cp = (const IO *)a.C + ln.b * a.L * N * 2;
    stream_steps<IO, GATED, 2>(xs, dts, zs, voff, rb, (uint32_t)(t1 - t0),
                            (uint32_t)(t1 - t0), [&](uint32_t i, float xv, float dv, float zv) {
        const int64_t t = t0 + i;
        const float u = dv * xv;
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float br = Uniform<IO>::ld(Bp, (t * N + n) * 2 + 0);
            const float bi = Uniform<IO>::ld(Bp, (t * N + n) * 2 + 1);
            const float cr = Uniform<IO>::ld(Cp, (t * N + n) * 2 + 0);
            const float ci = Uniform<IO>::ld(Cp, (t * N + n) * 2 + 1);
            float pr, pi;
            decay_rotation(dv, Ar2[n], Arev[n], pr, pi);
            const float nr = __builtin_fmaf(pr, hr[n], __builtin_fmaf(-pi, hi[n], u * br));
            const float ni = __builtin_fmaf(pr, hi[n], __builtin_fmaf(pi, hr[n], u * bi));
            hr[n] = nr;
            hi[n] = ni;
            acc = __builtin_fmaf(cr, nr, acc);
            acc = __builtin_fmaf(-ci, ni, acc);
        }
        float yv = __builtin_fmaf(Dd, xv, acc);
        if (GATED) yv = yv * silu(zv);
        ys.st(voff, i * rb, yv);
    });
    if (c == a.n_chunks - 1 && a.h_final) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            a.h_final[col + 2 * n + 0] = hr[n];
            a.h_final[col + 2 * n + 1] = hi[n];
        }
    }
}

inline void mark(hipEvent_t const *ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

template <typename IO, int N>
hipError_t launch_t(const ScanArgs &a, bool gated, hipStream_t s, hipEvent_t const *ev) {
    const dim3 blk(a.threads);
    const unsigned gx = (unsigned)(a.batch * a.dblocks);
    mark(ev, 0, s);
    if (a.n_chunks > 1)
        hipLaunchKernelGGL((k_chunk_summary_c<IO, N>), dim3(gx, a.n_chunks - 1), blk, 0, s, a);
    mark(ev, 1, s);
    if (a.n_chunks > 1) {
        const int64_t M = a.batch * a.Dn * N;
        hipLaunchKernelGGL(k_carry_c, dim3((unsigned)((M + 63) / 64)), dim3(256), 0, s, a, M);
    }
    mark(ev, 2, s);
    if (gated)
        hipLaunchKernelGGL((k_chunk_scan_c<IO, N, true>), dim3(gx, a.n_chunks), blk, 0, s, a);
    else
        hipLaunchKernelGGL((k_chunk_scan_c<IO, N, false>), dim3(gx, a.n_chunks), blk, 0, s, a);
    mark(ev, 3, s);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const ScanArgs &a, int d_state, bool gated, hipStream_t s,
                     hipEvent_t const *ev) {
    switch (d_state) {
        case 1: return launch_t<IO, 1>(a, gated, s, ev);
        case 2: return launch_t<IO, 2>(a, gated, s, ev);
        case 4: return launch_t<IO, 4>(a, gated, s, ev);
        case 8: return launch_t<IO, 8>(a, gated, s, ev);
        case 16: return launch_t<IO, 16>(a, gated, s, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_complex(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev) {
    return io == 0 ? launch_io<float>(a, d_state, gated, s, ev)
                   : launch_io<bf16_bits>(a, d_state, gated, s, ev);
}

}  // namespace ssm
