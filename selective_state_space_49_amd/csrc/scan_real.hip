// scan_real.hip -- prefill of the selective scan with a real diagonal state (gfx950).
//
// Recurrence ("Jamba — SSM-Transformer Híbrido", section "Um SSM em uma página";
// discretisation and gate of the MambaBlock in "【大模型】- Jamba 混合
// SSM-Transformer", section 4.1 "Mamba 层"), per batch row b and channel d:
//     h_t[n] = exp(dt_t A[n]) h_{t-1}[n] + dt_t B_t[n] x_t
//     y_t    = (sum_n C_t[n] h_t[n] + D x_t) * silu(z_t)
//
// Work split. One lane owns one channel and keeps its N-wide fp32 state in VGPRs;
// B_t and C_t are wave-uniform and come in through scalar loads. The sequence is cut
// into chunks of T steps so that there are enough waves to fill 256 CUs:
//   1. k_chunk_summary: for every chunk but the last, the end state from a zero
//      start, H_c, and the chunk's total decay P_c = exp(A * sum of dt over the chunk),
//      walking only the steps that can still reach the chunk's end (decay horizon).
//   2. k_carry: per state column, an exclusive associative scan over chunks with
//      (P1, H1) then (P2, H2) = (P2 P1, P2 H1 + H2), seeded with h0. Lanes hold
//      chunks; the prefix uses DPP row shifts and row broadcasts; a block walks
//      chunk tiles of 64 in order, carrying the running state between tiles.
//   3. k_chunk_scan: re-walks every chunk from its true incoming state with the
//      fused epilogue (C.h + D x, silu gate, rounding to the output type) and
//      writes y once; the last chunk writes h_final.
// With one chunk only step 3 runs. Steps 1-2 re-associate the recurrence exactly;
// results differ from a sequential loop only by rounding.
//
// exp(v) is evaluated as 2^(v log2 e) with the hardware exponential: log2 e is
// folded into A once per lane, so each state update costs one multiply, one
// exponential, one multiply (dt x times B) and two fused multiply-adds.
//
// The same kernels, instantiated with the MambaBlock input stage (MambaInput below),
// take the convolution's input in place of x and the raw dt projection output in
// place of dt, and apply the causal convolution + silu and softplus to each value as
// it is loaded (ssm_input_stage.h). Every lane then walks its chunk with the last
// KC-1 convolution inputs in registers, starting from the rows just before the
// chunk (or the carried convolution state before step 0).
#include <type_traits>

#include "ssm_device.h"
#include "ssm_input_stage.h"
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

// ---------------------------------------------------------------- input stage
// The kernels read x and dt as given.
struct NoInput {
    static constexpr bool kSave = false;  // store the state every kStateEvery steps
    static constexpr bool kSaveIn = false;  // store the scan's inputs u and dt
    static constexpr bool kTrap = false;
    static constexpr bool kW = false;  // no weight stream
    static constexpr int kWavesPerSimd = 5;
    static constexpr int kKU = 4;               // rows prefetched per block
    static constexpr bool kRawPrefetch = true;  // see StepIn (ssm_stream.h)
    __device__ __forceinline__ void params(const ScanArgs &, int64_t) {}
    __device__ __forceinline__ void history(const ScanArgs &, int64_t, int64_t, int64_t) {}
    __device__ __forceinline__ float x(float v) { return v; }
    __device__ __forceinline__ float dt(float v) const { return v; }
    __device__ __forceinline__ void store_state(const ScanArgs &, int64_t, int64_t) const {}
};

// The training forward: the plain scan that also stores the state entering every
// kStateEvery-th step for the backward (ScanArgs::states).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
struct SaveInput : NoInput {
    static constexpr bool kSave = true;
};

// The MambaBlock input stage: u = silu(causal conv of KC taps over x) (KC = 0: x as
// is) and dt = softplus(dt + dt_bias).
template <typename IO, int KC>
struct MambaInput {
    static constexpr bool kSave = false;
    static constexpr bool kSaveIn = false;
    static constexpr bool kTrap = false;
    static constexpr bool kW = false;
    static constexpr int kWavesPerSimd = 4;  // at five (prefetching 2 rows per block to fit)
    static constexpr int kKU = 4;            // the extra summary windows cost more than it gains
    static constexpr bool kRawPrefetch = false;
    ConvSilu<(KC > 0 ? KC : 1)> conv;
    float dbias;

    __device__ __forceinline__ void params(const ScanArgs &a, int64_t d) {
        dbias = a.dt_bias ? a.dt_bias[d] : 0.0f;
        if constexpr (KC > 0) {
#pragma unroll
            for (int k = 0; k < KC; ++k) conv.w[k] = a.conv_w[d * KC + k];
            conv.bias = a.conv_b ? a.conv_b[d] : 0.0f;
        }
    }
    // The KC-1 inputs before step t: rows of x, or of the carried state before step 0.
    __device__ __forceinline__ void history(const ScanArgs &a, int64_t b, int64_t d, int64_t t) {
        if constexpr (KC > 1) {
#pragma unroll
            for (int j = 0; j < KC - 1; ++j) {
                const int64_t r = t - (KC - 1) + j;
                if (r >= 0)
                    conv.hist[j] = Io<IO>::ld((const IO *)a.x + (b * a.L + r) * a.Dn + d);
                else if (a.conv_state0)
                    conv.hist[j] = Io<IO>::ld((const IO *)a.conv_state0 +
                                              (b * (KC - 1) + (KC - 1 + r)) * a.Dn + d);
                else
                    conv.hist[j] = 0.0f;
            }
        }
    }
    __device__ __forceinline__ float x(float v) {
        if constexpr (KC > 0) return conv(v);
        else return v;
    }
    __device__ __forceinline__ float dt(float v) const { return softplus(v + dbias); }
    // After the last step: the last KC-1 inputs, for the next call.
    __device__ __forceinline__ void store_state(const ScanArgs &a, int64_t b, int64_t d) const {
        if constexpr (KC > 1) {
            if (a.conv_state_out) {
#pragma unroll
                for (int j = 0; j < KC - 1; ++j)
                    Io<IO>::st((IO *)a.conv_state_out + (b * (KC - 1) + j) * a.Dn + d, conv.hist[j]);
            }
        }
    }
};

// The fused training forward: MambaInput's prefill that also stores the state entering
// every kStateEvery-th step (ScanArgs::states), as SaveInput does for the plain scan, and
// the scan's inputs u and dt as it makes them (ScanArgs::u_out, dt_out), so that the
// backward need not make them again.
template <typename IO, int KC>
struct MambaSave : MambaInput<IO, KC> {
    static constexpr bool kSave = true;
    static constexpr bool kSaveIn = true;
};

// The exponential-trapezoidal discretisation (the Mamba-3 item of "Jamba —
// SSM-Transformer Híbrido", section "Mamba-3: a linha de base de SSM puro em 2026",
// which names the rule, and the key-terms rows of the zh and hi lessons, which say it
// subsumes Euler's; no page gives a formula): the step's input integral is taken by a
// two-point rule over its ends, the current input weighted lam_t, the older one (decayed
// across the step) 1 - lam_t,
//     h_t = a_t h_{t-1} + dt_t ((1 - lam_t) a_t B_{t-1} x_{t-1} + lam_t B_t x_t),
// evaluated as a_t (h_{t-1} + wp x_{t-1} B_{t-1}) + wc x_t B_t with wc = dt_t lam_t and
// wp = dt_t (1 - lam_t). lam = 1 is Euler's step, lam = 1/2 (LAM = false: no weight
// stream) the trapezoid rule. The recurrence stays linear in h with a known input term,
// so chunk summaries, the carry and the rescan are unchanged apart from that term; each
// walk starts with the input before its first row (the row before, or x_prev / B_prev
// before step 0). x and dt are read as given; lam is a fourth stream laid out like dt.
template <typename IO, bool LAM>
struct TrapInput {
    static constexpr bool kSave = false;
    static constexpr bool kSaveIn = false;
    static constexpr bool kTrap = true;
    static constexpr bool kW = LAM;
    static constexpr int kWavesPerSimd = 5;
    static constexpr int kKU = LAM ? 2 : 4;  // the weight stream's blocks of 4 rows would spill
    static constexpr bool kRawPrefetch = false;
    float xprev;  // x of the step before the current one
    // The weights of the older and the current input for a step of length dv.
    __device__ __forceinline__ static void weights(float dv, float lr, float &wp, float &wc) {
        const float lv = LAM ? lr : 0.5f;
        wc = dv * lv;
        wp = dv * (1.0f - lv);
    }
    __device__ __forceinline__ void params(const ScanArgs &, int64_t) {}
    __device__ __forceinline__ void history(const ScanArgs &a, int64_t b, int64_t d, int64_t t) {
        if (t > 0) xprev = Io<IO>::ld((const IO *)a.x + (b * a.L + t - 1) * a.Dn + d);
        else xprev = a.x_prev ? Io<IO>::ld((const IO *)a.x_prev + b * a.Dn + d) : 0.0f;
    }
    __device__ __forceinline__ float x(float v) { return v; }
    __device__ __forceinline__ float dt(float v) const { return v; }
    __device__ __forceinline__ void store_state(const ScanArgs &, int64_t, int64_t) const {}
    // B of the step before step t (wave-uniform t): the start of a walk.
    template <int N, typename Row>
    __device__ __forceinline__ void prev_row(const ScanArgs &a, const Row &Bp, int64_t b, int64_t t,
                                             float (&bp)[N]) const {
        if (t > 0) {
#pragma unroll
            for (int n = 0; n < N; ++n) bp[n] = Bp.ld((t - 1) * N + n);
        } else if (a.B_prev) {
            const UniRow<IO, N> P(a.B_prev, b * N);
#pragma unroll
            for (int n = 0; n < N; ++n) bp[n] = P.ld(n);
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) bp[n] = 0.0f;
        }
    }
};

// ---------------------------------------------------------------- carry scan
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xf, false));
}

// Lane i holds the segment ending at i as (p, h): state_after = p * state_before + h.
// Combine with the earlier segment read over DPP; lanes without a source read the
// identity (1, 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_step(float &p, float &h) {
    const float pe = dpp<CTRL, ROW_MASK>(1.0f, p);
    const float he = dpp<CTRL, ROW_MASK>(0.0f, h);
    h = __builtin_fmaf(p, he, h);
    p = p * pe;
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ void wave_scan(float &p, float &h) {
    scan_step<0x111, 0xf>(p, h);  // row_shr:1
    scan_step<0x112, 0xf>(p, h);  // row_shr:2
    scan_step<0x114, 0xf>(p, h);  // row_shr:4
    scan_step<0x118, 0xf>(p, h);  // row_shr:8
    scan_step<0x142, 0xa>(p, h);  // row_bcast:15 into rows 1 and 3
    scan_step<0x143, 0xc>(p, h);  // row_bcast:31 into rows 2 and 3
}

// M = batch * Dn * N state columns; block = 4 waves, 64 columns; LDS tiles are
// [64 chunks][64 columns], loaded and stored row by row (coalesced), scanned
// column by column with lanes = chunks.
__global__ __launch_bounds__(256) void k_carry(ScanArgs a, int64_t M) {
    __shared__ float sP[64][65];
    __shared__ float sH[64][65];
    __shared__ float sCarry[64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * 64;
    const int64_t col = col0 + lane;
    const int nsum = a.n_chunks - 1;
    if (threadIdx.x < 64) sCarry[lane] = (col < M && a.h0) ? a.h0[col] : 0.0f;
    for (int k0 = 0; k0 < nsum; k0 += 64) {
        const int rows = min(64, nsum - k0);
        __syncthreads();
        for (int r = w; r < rows; r += 4) {
            if (col < M) {
                sP[r][lane] = a.sumP[(size_t)(k0 + r) * M + col];
                sH[r][lane] = a.sumH[(size_t)(k0 + r) * M + col];
            }
        }
        __syncthreads();
        for (int jj = 0; jj < 16; ++jj) {
            const int j = w * 16 + jj;
            if (col0 + j >= M) break;  // uniform over the wave
            float p = lane < rows ? sP[lane][j] : 1.0f;
            float h = lane < rows ? sH[lane][j] : 0.0f;
            wave_scan(p, h);
            const float out = __builtin_fmaf(p, sCarry[j], h);
            if (lane < rows) sH[lane][j] = out;
            const float next = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(out), rows - 1));
            if (lane == 0) sCarry[j] = next;
        }
        __syncthreads();
        for (int r = w; r < rows; r += 4)
            if (col < M) a.sumH[(size_t)(k0 + r) * M + col] = sH[r][lane];
    }
}

// With few chunks the wave-wide scan above mostly runs on empty lanes. Then one lane
// per state column walks the chunks in order, carry = P_c carry + H_c, with the loads of
// kCarryBatch chunks issued before their multiply-adds; the carries are written over H_c
// as above. The same result up to rounding (a sequential rather than a tree association).
constexpr int kCarrySeqMax = 64;  // chunk summaries handled by the sequential walk
constexpr int kCarryBatch = 8;

__global__ __launch_bounds__(256) void k_carry_seq(ScanArgs a, int64_t M) {
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= M) return;
    const int nsum = a.n_chunks - 1;
    float carry = a.h0 ? a.h0[col] : 0.0f;
    for (int c0 = 0; c0 < nsum; c0 += kCarryBatch) {
        float p[kCarryBatch], h[kCarryBatch];
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            if (c0 + k < nsum) {
                p[k] = a.sumP[(size_t)(c0 + k) * M + col];
                h[k] = a.sumH[(size_t)(c0 + k) * M + col];
            }
        }
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            if (c0 + k < nsum) {
                carry = __builtin_fmaf(p[k], carry, h[k]);
                a.sumH[(size_t)(c0 + k) * M + col] = carry;
            }
        }
    }
}

// The carry over the chunk summaries of M state columns: sequential for up to
// kCarrySeqMax summaries, else the tiled wave scan.
inline void carry_launch(const ScanArgs &a, int64_t M, hipStream_t s) {
    if (a.n_chunks - 1 <= kCarrySeqMax)
        hipLaunchKernelGGL(k_carry_seq, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, a, M);
    else
        hipLaunchKernelGGL(k_carry, dim3((unsigned)((M + 63) / 64)), dim3(256), 0, s, a, M);
}

// ---------------------------------------------------------------- chunk summary
// Chunk summary: end state from a zero start and total decay, walking only the
// window back to the decay horizon (see horizon_start). Issue priority follows the
// window's remaining steps on a scale of kSummaryPrioScale steps, so that longer windows
// go first, or of the chunk's length when that is shorter: windows that span whole short
// chunks (all of one length) then step down like the rescan's waves, where on the longer
// scale every wave fell to the lowest level within a few steps and the waves finished one
// after another (Jamba layer, 205-step chunks: summary 0.216 -> 0.194-0.200 ms on one
// MI355X).
template <typename IO, int N, typename In>
__global__ __launch_bounds__(256) void k_chunk_summary(ScanArgs a) {
    const LaneId ln = lane_id(a);
    if (ln.d >= a.Dn) return;
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t T = (uint32_t)a.T;  // every chunk that has a summary is full length
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    float A2[N], h[N];
    float amax = -INFINITY;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[ln.d * N + n] * kLog2e;
        amax = fmaxf(amax, A2[n]);
        h[n] = 0.0f;
    }
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> dts((const IO *)a.dt + row0);
    In in;
    in.params(a, ln.d);
    // 1. window start ts (chunk-relative): walk dt backwards from the chunk end
    const uint32_t ts = horizon_start<IO>(dts, voff, rb, T, amax, [&](float v) { return in.dt(v); });
    in.history(a, ln.b, ln.d, t0 + ts);
    // 2. end state from zero over rows [ts, T) of the chunk
    const UniRow<IO, N> Bp(a.B, ln.b * a.L * N);
    const int64_t rw = row0 + (int64_t)ts * a.Dn;
    const RowStream<IO> xs((const IO *)a.x + rw), dws((const IO *)a.dt + rw),
        lws(In::kW ? (const IO *)a.lam + rw : (const IO *)a.x + rw);
    double S = 0.0;  // sum of dt, needed only when the window is the whole chunk
    float bp[N];     // trapezoidal rule: B of the step before, carried from step to step
    if constexpr (In::kTrap) in.template prev_row<N>(a, Bp, ln.b, t0 + ts, bp);
    stream_steps_w<IO, false, 4, In::kRawPrefetch, In::kW>(xs, dws, dws, lws, voff, rb, T - ts, min(T, kSummaryPrioScale), [&](uint32_t i, float xr, float dr, float, float lr) {
        const float xv = in.x(xr), dv = in.dt(dr);
        const int64_t t = t0 + ts + i;
        S += (double)dv;
        if constexpr (In::kTrap) {
            float wp, wc;
            In::weights(dv, lr, wp, wc);
            const float up = wp * in.xprev, uc = wc * xv;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float bn = Bp.ld(t * N + n);
                h[n] = __builtin_fmaf(e2(dv * A2[n]), __builtin_fmaf(up, bp[n], h[n]), uc * bn);
                bp[n] = bn;
            }
            in.xprev = xv;
        } else {
            const float u = dv * xv;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float bn = Bp.ld(t * N + n);
                h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], u * bn);
            }
        }
    });
    const float Sf = (float)S;
    const size_t o = (((size_t)c * a.batch + ln.b) * a.Dn + ln.d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a.sumP[o + n] = ts == 0 ? e2(A2[n] * Sf) : 0.0f;
        a.sumH[o + n] = h[n];
    }
}

// ---------------------------------------------------------------- rescan + epilogue
// Compiled for at least In::kWavesPerSimd waves per SIMD, and the planner cuts the
// sequence into enough chunks to give every SIMD that many: 5 for the plain and the
// trapezoidal rescans (5 against 4: 6.25 -> 5.88 ms on the 256k rescan; with the weight
// stream, blocks of 2 rows instead of 4 keep it from spilling), 4 with the input stage.
template <typename IO, int N, bool GATED, typename In>
__global__ __launch_bounds__(256, In::kWavesPerSimd) void k_chunk_scan(ScanArgs a) {
    const LaneId ln = lane_id(a);
    if (ln.d >= a.Dn) return;
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t steps = (uint32_t)(min(a.L, t0 + a.T) - t0);
    const size_t col = (size_t)(ln.b * a.Dn + ln.d) * N;
    const float *hin = c == 0 ? (a.h0 ? a.h0 + col : nullptr)
                              : a.sumH + (size_t)(c - 1) * a.batch * a.Dn * N + col;
    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[ln.d * N + n] * kLog2e;
        h[n] = hin ? hin[n] : 0.0f;
    }
    const float Dd = a.D[ln.d];
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> xs((const IO *)a.x + row0), dts((const IO *)a.dt + row0),
        zs(GATED ? (const IO *)a.z + row0 : (const IO *)a.x + row0), ys((IO *)a.y + row0),
        lws(In::kW ? (const IO *)a.lam + row0 : (const IO *)a.x + row0),
        uos(In::kSaveIn ? (IO *)a.u_out + row0 : (IO *)a.y + row0),
        dtos(In::kSaveIn ? (IO *)a.dt_out + row0 : (IO *)a.y + row0);
    const UniRow<IO, N> Bp(a.B, ln.b * a.L * N);
    const UniRow<IO, N> Cp(a.C, ln.b * a.L * N);
    In in;
    in.params(a, ln.d);
    in.history(a, ln.b, ln.d, t0);
    float bp[N];  // trapezoidal rule: B of the step before, carried from step to step
    if constexpr (In::kTrap) in.template prev_row<N>(a, Bp, ln.b, t0, bp);
    // training forward: the lane's byte offset in a stored-state row, and between pieces
    const uint32_t sv_off = In::kSave ? (uint32_t)(state_at<N>(ln.b, ln.d, 0, a.Dn) * 4) : 0u;
    const uint32_t sv_qstride = (uint32_t)(a.Dn * 16);
    stream_steps_w<IO, GATED, In::kKU, In::kRawPrefetch, In::kW>(xs, dts, zs, lws, voff, rb, steps, steps, [&](uint32_t i, float xr, float dr, float zv, float lr) {
        const float xv = in.x(xr), dv = in.dt(dr);
        if constexpr (In::kSaveIn) {  // read back by the backward only: streaming stores
            uos.st_stream(voff, i * rb, xv);  // (the fused training forward 10.8-10.9 ->
            dtos.st_stream(voff, i * rb, dv);  // 10.5-10.6 ms at 256k on one MI355X)
        }
        const int64_t t = t0 + i;
        float acc = 0.0f;
        if constexpr (In::kTrap) {
            float wp, wc;
            In::weights(dv, lr, wp, wc);
            const float up = wp * in.xprev, uc = wc * xv;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float bn = Bp.ld(t * N + n);
                const float cn = Cp.ld(t * N + n);
                h[n] = __builtin_fmaf(e2(dv * A2[n]), __builtin_fmaf(up, bp[n], h[n]), uc * bn);
                acc = __builtin_fmaf(cn, h[n], acc);
                bp[n] = bn;
            }
            in.xprev = xv;
        } else {
            if constexpr (In::kSave) {
                // the state entering step t (chunks start at multiples of kStateEvery),
                // through a buffer resource based at its row (a row is below 2 GiB);
                // streaming stores (glc slc), as the compiler's nontemporal stores are:
                // 7.74-7.93 -> 7.51-7.59 ms for the 256k forward on one MI355X
                if (i % kStateEvery == 0) {
                    const auto r = __builtin_amdgcn_make_buffer_rsrc(
                        a.states + (size_t)(t / kStateEvery) * a.batch * a.Dn * N, 0, -1, kRsrcWord3);
                    if constexpr (N % 4 == 0) {
#pragma unroll
                        for (int q = 0; q < N / 4; ++q) {
                            const u32x4 v = {__float_as_uint(h[4 * q]), __float_as_uint(h[4 * q + 1]),
                                             __float_as_uint(h[4 * q + 2]), __float_as_uint(h[4 * q + 3])};
                            __builtin_amdgcn_raw_buffer_store_b128(v, r, sv_off, q * sv_qstride, 3);
                        }
                    } else {
#pragma unroll
                        for (int n = 0; n < N; ++n)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h[n]), r, sv_off + 4u * n, 0, 3);
                    }
                }
            }
            const float u = dv * xv;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float bn = Bp.ld(t * N + n);
                const float cn = Cp.ld(t * N + n);
                h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], u * bn);
                acc = __builtin_fmaf(cn, h[n], acc);
            }
        }
        float yv = __builtin_fmaf(Dd, xv, acc);
        if (GATED) yv = yv * silu(zv);
        // y is written once and read only by the caller's next step: streaming stores,
        // as for the stored states (256k: 6.48 -> 6.44 ms per step, the fused training
        // forward 10.5-10.6 -> 10.2-10.4 ms on one MI355X)
        ys.st_stream(voff, i * rb, yv);
    });
    if (c == a.n_chunks - 1) {
        if (a.h_final) {
#pragma unroll
            for (int n = 0; n < N; ++n) a.h_final[col + n] = h[n];
        }
        in.store_state(a, ln.b, ln.d);
    }
}

__global__ void k_state_fill(float *dst, const float *src, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) dst[i] = src ? src[i] : 0.0f;
}

__global__ void k_fill16(uint16_t *dst, const uint16_t *src, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) dst[i] = src ? src[i] : (uint16_t)0;
}

inline void mark(hipEvent_t const *ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

template <typename IO, int N, typename In>
hipError_t launch_t(const ScanArgs &a, bool gated, hipStream_t s, hipEvent_t const *ev) {
    const dim3 blk(a.threads);
    const unsigned gx = (unsigned)(a.batch * a.dblocks);
    mark(ev, 0, s);
    if (a.n_chunks > 1)
        hipLaunchKernelGGL((k_chunk_summary<IO, N, In>), dim3(gx, a.n_chunks - 1), blk, 0, s, a);
    mark(ev, 1, s);
    if (a.n_chunks > 1) {
        const int64_t M = a.batch * a.Dn * N;
        carry_launch(a, M, s);
    }
    mark(ev, 2, s);
    if (gated)
        hipLaunchKernelGGL((k_chunk_scan<IO, N, true, In>), dim3(gx, a.n_chunks), blk, 0, s, a);
    else
        hipLaunchKernelGGL((k_chunk_scan<IO, N, false, In>), dim3(gx, a.n_chunks), blk, 0, s, a);
    mark(ev, 3, s);
    return hipGetLastError();
}

template <typename IO, typename In>
hipError_t launch_io(const ScanArgs &a, int d_state, bool gated, hipStream_t s,
                     hipEvent_t const *ev) {
    switch (d_state) {
        case 1: return launch_t<IO, 1, In>(a, gated, s, ev);
        case 2: return launch_t<IO, 2, In>(a, gated, s, ev);
        case 4: return launch_t<IO, 4, In>(a, gated, s, ev);
        case 8: return launch_t<IO, 8, In>(a, gated, s, ev);
        case 16: return launch_t<IO, 16, In>(a, gated, s, ev);
    }
    return hipErrorInvalidValue;
}

template <typename IO, int KC, bool SAVE>
using FusedIn = typename std::conditional<SAVE, MambaSave<IO, KC>, MambaInput<IO, KC>>::type;

template <typename IO, bool SAVE>
hipError_t launch_fused_io(const ScanArgs &a, int d_state, bool gated, hipStream_t s,
                           hipEvent_t const *ev) {
    switch (a.conv_k) {
        case 0: return launch_io<IO, FusedIn<IO, 0, SAVE>>(a, d_state, gated, s, ev);
        case 1: return launch_io<IO, FusedIn<IO, 1, SAVE>>(a, d_state, gated, s, ev);
        case 2: return launch_io<IO, FusedIn<IO, 2, SAVE>>(a, d_state, gated, s, ev);
        case 3: return launch_io<IO, FusedIn<IO, 3, SAVE>>(a, d_state, gated, s, ev);
        case 4: return launch_io<IO, FusedIn<IO, 4, SAVE>>(a, d_state, gated, s, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_real(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev) {
    return io == 0 ? launch_io<float, NoInput>(a, d_state, gated, s, ev)
                   : launch_io<bf16_bits, NoInput>(a, d_state, gated, s, ev);
}

hipError_t launch_scan_save(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev) {
    return io == 0 ? launch_io<float, SaveInput>(a, d_state, gated, s, ev)
                   : launch_io<bf16_bits, SaveInput>(a, d_state, gated, s, ev);
}

hipError_t launch_scan_trap(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev) {
    if (a.lam)
        return io == 0 ? launch_io<float, TrapInput<float, true>>(a, d_state, gated, s, ev)
                       : launch_io<bf16_bits, TrapInput<bf16_bits, true>>(a, d_state, gated, s, ev);
    return io == 0 ? launch_io<float, TrapInput<float, false>>(a, d_state, gated, s, ev)
                   : launch_io<bf16_bits, TrapInput<bf16_bits, false>>(a, d_state, gated, s, ev);
}

hipError_t launch_scan_fused(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                             hipEvent_t const *ev) {
    if (a.states)
        return io == 0 ? launch_fused_io<float, true>(a, d_state, gated, s, ev)
                       : launch_fused_io<bf16_bits, true>(a, d_state, gated, s, ev);
    return io == 0 ? launch_fused_io<float, false>(a, d_state, gated, s, ev)
                   : launch_fused_io<bf16_bits, false>(a, d_state, gated, s, ev);
}

namespace {
template <typename IO>
hipError_t launch_summary_carry_io(const ScanArgs &a, int d_state, hipStream_t s) {
    if (a.n_chunks <= 1) return hipSuccess;
    const unsigned gx = (unsigned)(a.batch * a.dblocks);
    const dim3 grid(gx, a.n_chunks - 1), blk(a.threads);
    switch (d_state) {
        case 1: hipLaunchKernelGGL((k_chunk_summary<IO, 1, NoInput>), grid, blk, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_chunk_summary<IO, 2, NoInput>), grid, blk, 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_chunk_summary<IO, 4, NoInput>), grid, blk, 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_chunk_summary<IO, 8, NoInput>), grid, blk, 0, s, a); break;
        case 16: hipLaunchKernelGGL((k_chunk_summary<IO, 16, NoInput>), grid, blk, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    const int64_t M = a.batch * a.Dn * d_state;
    carry_launch(a, M, s);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_summary_carry(const ScanArgs &a, int io, int d_state, hipStream_t s) {
    return io == 0 ? launch_summary_carry_io<float>(a, d_state, s)
                   : launch_summary_carry_io<bf16_bits>(a, d_state, s);
}

hipError_t launch_carry(const ScanArgs &a, int d_state, hipStream_t s) {
    if (a.n_chunks <= 1) return hipSuccess;
    const int64_t M = a.batch * a.Dn * d_state;
    carry_launch(a, M, s);
    return hipGetLastError();
}

hipError_t launch_elem_fill(void *dst, const void *src, int64_t count, int elem_bytes,
                            hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const dim3 grid((unsigned)((count + 255) / 256));
    if (elem_bytes == 4)
        hipLaunchKernelGGL(k_state_fill, grid, dim3(256), 0, s, (float *)dst, (const float *)src, count);
    else
        hipLaunchKernelGGL(k_fill16, grid, dim3(256), 0, s, (uint16_t *)dst, (const uint16_t *)src, count);
    return hipGetLastError();
}

hipError_t launch_state_fill(float *dst, const float *src, int64_t count, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_state_fill, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, dst,
                       src, count);
    return hipGetLastError();
}

}  // namespace ssm
