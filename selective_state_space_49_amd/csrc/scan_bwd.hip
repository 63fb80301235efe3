// scan_bwd.hip -- gradients of the real-state prefill (gfx950).
//
// Training differentiates the scan ("Jamba — SSM-Transformer Híbrido", section "Um
// SSM em uma página", on evaluating the SSM at training time; the recurrence and the
// MambaBlock's gate from "【大模型】- Jamba 混合 SSM-Transformer", section 4.1). With
//     h_t = a_t h_{t-1} + dt_t x_t B_t,  a_t = exp(dt_t A),  o_t = C_t.h_t + D x_t,
//     y_t = o_t silu(z_t),
// and the upstream dy (and dh_final), the adjoint lam_t = dLoss/dh_t runs backwards:
//     lam_t = do_t C_t + a_{t+1} lam_{t+1},   do_t = dy_t silu(z_t),
// and per step
//     dx_t = do_t D + dt_t sum_n lam_t[n] B_t[n]
//     ddt_t = x_t sum_n lam_t[n] B_t[n] + sum_n A[n] lam_t[n] w_t[n]
//     dA[n] += dt_t lam_t[n] w_t[n],  dB_t[n] += lam_t[n] dt_t x_t,  dC_t[n] += do_t h_t[n]
// where w_t = a_t h_{t-1} = h_t - dt_t x_t B_t, so only h_t is needed at step t.
//
// The state runs forwards and the adjoint backwards, and neither recurrence can be
// inverted stably (a_t may be tiny), so states are recomputed. Phases, one lane per
// channel as in the forward kernels:
//   1. the forward's chunk summaries and carry: the state entering every chunk;
//   2. k_bwd_summary: per chunk c >= 1 the adjoint it passes to chunk c-1 from a zero
//      carry-in, G_c, and its total decay Q_c, over a window that ends where the
//      decay reaches the forward's horizon (horizon_bits), mirrored;
//   3. the forward's carry kernel over the chunks in reverse order, seeded with
//      dh_final: the adjoint entering every chunk from the right;
//   4. k_bwd_walk: per chunk, a forward walk from the incoming state that stores the
//      state every kSub steps; k_bwd_chunk: per chunk, a backward walk by sub-chunks:
//      each sub-chunk's kSub states are recomputed into registers from its stored start
//      and the gradients of its steps emitted. dB_t and dC_t, summed over channels, are reduced
//      across the 64 lanes of the wave (a transposing butterfly of lane permutations:
//      2N values over 64 lanes in 2N - 1 exchanges plus the final levels) and stored
//      per wave;
//   5. k_bwd_reduce_*: dA and dD summed over chunks and batch rows, dB and dC over waves.
// Every sum is over a fixed order: results are deterministic.
#include "ssm_device.h"
#include "ssm_input_stage.h"
#include "ssm_internal.h"
#include "ssm_stream.h"

namespace ssm {
namespace {

struct Lane {
    int64_t b, d;    // batch row, channel (d clamped to a valid channel)
    bool valid;      // false for the padding lanes of the last channel block
    int32_t w;       // channel wave within the batch row
};

__device__ __forceinline__ Lane lane_of(const BwdArgs &a) {
    Lane r;
    r.b = (int64_t)blockIdx.x / a.dblocks;
    const int64_t d = ((int64_t)blockIdx.x % a.dblocks) * a.threads + threadIdx.x;
    r.valid = d < a.Dn;
    r.d = r.valid ? d : a.Dn - 1;
    r.w = (int32_t)(((int64_t)blockIdx.x % a.dblocks) * (a.threads / 64) + threadIdx.x / 64);
    return r;
}

// Sum over the 64 lanes of a wave of each of V values. At each level of a butterfly
// over lane bits 32, 16, .., 1, a lane keeps the half of its values selected by its
// lane bit and adds the partner's copy of that half; once one value is left the
// remaining levels add it to the partner's. On return lane l holds the total of value
// l >> (6 - log2 V) (the lanes sharing that index hold the same total).
// Partners: lane bits 5 and 4 through v_permlane32_swap / v_permlane16_swap, whose two
// results already pair (own kept value, partner's) for both lanes, so a pair costs the
// swap and an add; bits 3 .. 0 through DPP row mirror (lane i with 15 - i), half-row
// mirror (i with 7 - i) and quad permutations (xor 2, xor 1), with a select of the half
// to send and to keep. The mirrors also flip lower bits, which only reorders partners
// within a group: the masks 15, 7, 2, 1 are independent, so every lane enters every
// total once.
__device__ __forceinline__ float swap32_sum(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_sum(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int S> struct Partner;
template <> struct Partner<8> { static constexpr int ctrl = 0x140; };  // row_mirror
template <> struct Partner<4> { static constexpr int ctrl = 0x141; };  // row_half_mirror
template <> struct Partner<2> { static constexpr int ctrl = 0x4E; };   // quad_perm [2,3,0,1]
template <> struct Partner<1> { static constexpr int ctrl = 0xB1; };   // quad_perm [1,0,3,2]

template <int K, int S, int V>
struct Butterfly {
    static __device__ __forceinline__ void run(float (&v)[V], int lane) {
        if constexpr (S > 0) {
            constexpr int half = K > 1 ? K / 2 : 1;
            if constexpr (S >= 16) {
#pragma unroll
                for (int i = 0; i < half; ++i) {
                    const float lo = v[i], hi = K > 1 ? v[i + half] : v[i];
                    v[i] = S == 32 ? swap32_sum(lo, hi) : swap16_sum(lo, hi);
                }
            } else if constexpr (K > 1) {
                const bool up = (lane & S) != 0;
#pragma unroll
                for (int i = 0; i < half; ++i) {
                    const float send = up ? v[i] : v[i + half];
                    const float keep = up ? v[i + half] : v[i];
                    v[i] = keep + dpp<Partner<S>::ctrl>(send);
                }
            } else {
                v[0] = v[0] + dpp<Partner<S>::ctrl>(v[0]);
            }
            Butterfly<half, S / 2, V>::run(v, lane);
        }
    }
};

template <int V>
__device__ __forceinline__ float wave_reduce_transpose(float (&v)[V]) {
    Butterfly<V, 32, V>::run(v, threadIdx.x & 63);
    return v[0];
}

template <int V> struct Log2;
template <> struct Log2<2> { static constexpr int v = 1; };
template <> struct Log2<4> { static constexpr int v = 2; };
template <> struct Log2<8> { static constexpr int v = 3; };
template <> struct Log2<16> { static constexpr int v = 4; };
template <> struct Log2<32> { static constexpr int v = 5; };

// Walks rows steps-1 .. 0 of up to three streams (s2 only if THREE), fetching the
// block of KU rows below the current one while the current one is computed; calls
// body(i, v0, v1, v2). prio_scale: issue priority by remaining rows (set_priority).
template <typename IO, bool THREE, int KU, typename Body>
__device__ __forceinline__ void stream_rev(const RowStream<IO> &s0, const RowStream<IO> &s1,
                                           const RowStream<IO> &s2, uint32_t voff, uint32_t rb,
                                           uint32_t steps, uint32_t prio_scale, Body &&body) {
    const uint32_t full = steps / KU;
    for (uint32_t i = steps; i > full * KU;) {  // ragged top rows first, one at a time
        --i;
        body(i, s0.ld(voff, i * rb), s1.ld(voff, i * rb), THREE ? s2.ld(voff, i * rb) : 0.0f);
    }
    if (full == 0) return;
    float a0[KU], a1[KU], a2[KU], b0[KU], b1[KU], b2[KU];
    auto load = [&](float(&v0)[KU], float(&v1)[KU], float(&v2)[KU], uint32_t blk) {
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const uint32_t r = blk * KU + k;
            v0[k] = s0.ld(voff, r * rb);
            v1[k] = s1.ld(voff, r * rb);
            if (THREE) v2[k] = s2.ld(voff, r * rb);
        }
    };
    load(a0, a1, a2, full - 1);
    for (uint32_t blk = full; blk > 0;) {
        --blk;  // block blk is in a*: fetch blk-1 into b*, compute blk
        set_priority((blk + 1) * KU, prio_scale);
        if (blk > 0) load(b0, b1, b2, blk - 1);
#pragma unroll
        for (int k = KU - 1; k >= 0; --k) {
            __builtin_amdgcn_sched_barrier(0);
            body(blk * KU + k, a0[k], a1[k], THREE ? a2[k] : 0.0f);
        }
        if (blk == 0) break;
        --blk;  // block blk is in b*: fetch blk-1 into a*, compute blk
        set_priority((blk + 1) * KU, prio_scale);
        if (blk > 0) load(a0, a1, a2, blk - 1);
#pragma unroll
        for (int k = KU - 1; k >= 0; --k) {
            __builtin_amdgcn_sched_barrier(0);
            body(blk * KU + k, b0[k], b1[k], THREE ? b2[k] : 0.0f);
        }
        if (blk == 0) break;
    }
    __builtin_amdgcn_s_setprio(0);
}

// First row (chunk-relative) from which the decay back to row 0 is below 2^-H (H =
// horizon_bits(T), as for the forward's windows) for every state of every lane of the
// wave, walking dt forward in whole blocks of kB rows: rows at or beyond it reach row 0
// with weight below 2^-H. Returns T when the horizon is not reached within the whole
// blocks (A >= 0, dt = 0, NaN, short T).
template <typename IO>
__device__ __forceinline__ uint32_t horizon_end(const RowStream<IO> &dt, uint32_t voff,
                                                uint32_t rb, uint32_t T, float amax) {
    if (!__any(amax < 0.0f) || T < (uint32_t)kB) return T;
    const float H = horizon_bits(T);
    float S = 0.0f;
    float cur[kB];
    uint32_t nxt[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) cur[k] = dt.ld(voff, k * rb);
    uint32_t tb = 0;
    while (true) {
        const uint32_t tn = tb + kB;  // rows [tb, tn) are in cur
        const bool more = tn + kB <= T;
        if (more) {
#pragma unroll
            for (int k = 0; k < kB; ++k) nxt[k] = dt.ldraw(voff, (tn + k) * rb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kB; ++k) S += cur[k];
        if (__all(amax * S <= -H)) return tn;
        if (!more) return T;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kB; ++k) cur[k] = RowStream<IO>::widen(nxt[k]);
        tb = tn;
    }
}

// d(output) of one step: dy times the gate, and the gate's derivative factor.
template <bool GATED>
__device__ __forceinline__ float gate_grad(float dy, float z, float &gp) {
    if (!GATED) {
        gp = 0.0f;
        return dy;
    }
    const float s = rcp(1.0f + e2(-z * kLog2e));  // sigmoid(z)
    gp = s * __builtin_fmaf(z, 1.0f - s, 1.0f);   // silu'(z) = s (1 + z (1 - s))
    return dy * (z * s);
}

// ---------------------------------------------------------------- reverse summary
// Chunks c = 1 .. n_chunks-1: G_c = sum over the chunk's steps t of
// (prod_{r = t0}^{t} a_r) do_t C_t and Q_c = prod of a_t over the chunk, stored at
// entry n_chunks-1-c of revG / revQ.
template <typename IO, int N, bool GATED>
__global__ __launch_bounds__(256) void k_bwd_summary(BwdArgs a) {
    const Lane ln = lane_of(a);
    if (!ln.valid) return;  // no cross-lane work here
    const int c = blockIdx.y + 1;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t T = (uint32_t)(min(a.L, t0 + a.T) - t0);
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    float A2[N], lam[N];
    float amax = -INFINITY;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[ln.d * N + n] * kLog2e;
        amax = fmaxf(amax, A2[n]);
        lam[n] = 0.0f;
    }
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> dts((const IO *)a.dt + row0), dys((const IO *)a.dy + row0),
        zs(GATED ? (const IO *)a.z + row0 : (const IO *)a.dt + row0);
    const uint32_t te = horizon_end<IO>(dts, voff, rb, T, amax);
    const UniRow<IO, N> Cp(a.C, ln.b * a.L * N);
    double S = 0.0;
    // issue priority as the forward summaries take it: windows on a 2048-step scale (longer
    // ones first), or the chunk's length when shorter
    stream_rev<IO, GATED, 4>(dts, dys, zs, voff, rb, te, min(T, kSummaryPrioScale), [&](uint32_t i, float dv, float dy, float zv) {
        const int64_t t = t0 + i;
        float gp;
        const float dout = gate_grad<GATED>(dy, zv, gp);
        S += (double)dv;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float lt = __builtin_fmaf(dout, Cp.ld(t * N + n), lam[n]);
            lam[n] = e2(dv * A2[n]) * lt;
        }
    });
    const float Sf = (float)S;
    const size_t M = (size_t)a.batch * a.Dn * N;
    const size_t o = (size_t)(a.n_chunks - 1 - c) * M + (size_t)(ln.b * a.Dn + ln.d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a.revQ[o + n] = te == T ? e2(A2[n] * Sf) : 0.0f;
        a.revG[o + n] = lam[n];
    }
}

// ---------------------------------------------------------------- sub-chunk staging
// At the start of each sub-chunk the backward walk needs its kSub rows of x, dt, dy
// (and z) and the state stored at its start. Loading them there would expose the HBM
// latency once per sub-chunk, with only two waves per SIMD to cover it. Instead they
// are copied into LDS by direct-to-LDS loads (no registers held while in flight) one
// sub-chunk ahead, while the current one is computed. Per wave, in dwords:
//   rows[s][j][lane]  stream s (x, dt, dy, z), row j of the sub-chunk; a 2-byte
//                     element lands zero-extended in its lane's dword;
//   st[q][lane][4]    the stored state in 16-byte pieces (N % 4 == 0), or st[n][lane].
// The compiler does not order these loads against LDS reads, so the kernel waits
// explicitly: vmcnt(0) before the LDS is read, lgkmcnt(0) before it is refilled.
#define SSM_LDS __attribute__((address_space(3)))
constexpr int kPair = 2 * kSub;               // rows staged at a time: two pieces
constexpr int kStageRows = 4 * kPair * 64;
template <int N> struct Stage { static constexpr int dwords = kStageRows + N * 64; };

typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kWaitVm0 = 0x0F70;    // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0)

template <typename IO>
__device__ __forceinline__ void row_to_lds(const RowStream<IO> &s, SSM_LDS uint32_t *dst,
                                           uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(IO) == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s.r, (SSM_LDS void *)dst, 2, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s.r, (SSM_LDS void *)dst, 4, voff, soff, 0, 0);
}

// Stage the rows j0 .. j0 + kPair - 1 of a pair of pieces (rows past the chunk's ns
// read row j0) and the lane's state entering the pair from the stored states' row st
// (null: a zero state), in the layout of ckpt_at: at byte st_voff, and for N % 4 == 0
// its 16-byte pieces st_qstride bytes apart. Both use buffer loads: the compiler then leaves their
// waits to the kernel (a global-address load to LDS makes it wait for every store in
// flight before the next LDS read).
template <typename IO, int N, bool GATED>
__device__ __forceinline__ void stage_sub(SSM_LDS uint32_t *stg, const RowStream<IO> &xs,
                                          const RowStream<IO> &dts, const RowStream<IO> &dys,
                                          const RowStream<IO> &zs, uint32_t voff, uint32_t rb,
                                          uint32_t j0, uint32_t ns, const float *st,
                                          uint32_t st_voff, uint32_t st_qstride, int lane) {
#pragma unroll
    for (int j = 0; j < kPair; ++j) {
        const uint32_t r = (j0 + (j < (int)ns ? j : 0)) * rb;
        row_to_lds<IO>(xs, stg + (0 * kPair + j) * 64, voff, r);
        row_to_lds<IO>(dts, stg + (1 * kPair + j) * 64, voff, r);
        row_to_lds<IO>(dys, stg + (2 * kPair + j) * 64, voff, r);
        if (GATED) row_to_lds<IO>(zs, stg + (3 * kPair + j) * 64, voff, r);
    }
    if (!st) {
#pragma unroll
        for (int n = 0; n < N; ++n) stg[kStageRows + n * 64 + lane] = 0u;  // either layout
    } else {
        const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(st), 0, -1, kRsrcWord3);
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SSM_LDS void *)(stg + kStageRows + q * 256), 16,
                                                         st_voff, q * st_qstride, 0, 0);
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SSM_LDS void *)(stg + kStageRows + n * 64), 4,
                                                         st_voff + 4 * n, 0, 0, 0);
        }
    }
}

// ---------------------------------------------------------------- stored states
// Row c R + p of ckpt (R = ck_rows rows per chunk) holds the state entering step
// kStateEvery p of chunk c, in the layout of state_at: every second piece's start is
// stored, and the other piece's start is recomputed from it (half the stored bytes, for
// one more 4-step walk per two pieces in the gradient kernel). With the training
// forward's states (saved) chunks start at multiples of kStateEvery and R = T / 8, so
// that row is the global row t / kStateEvery the forward wrote.
static_assert(kStateEvery == 2 * kSub, "a stored state starts every pair of pieces");

// ---------------------------------------------------------------- forward walk
// Per chunk, a forward walk from the state entering it that stores the state entering
// every pair of pieces (ckpt), the chunk's own incoming state included. A kernel of its own: inside the gradient
// kernel, at that kernel's two waves per SIMD, the walk took a third of the backward;
// alone it keeps many more waves resident. Waves get issue priority by remaining work.
template <typename IO, int N>
__global__ __launch_bounds__(256) void k_bwd_walk(BwdArgs a) {
    const Lane ln = lane_of(a);
    if (!ln.valid) return;  // no cross-lane work here
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t steps = (uint32_t)(min(a.L, t0 + a.T) - t0);
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const size_t M = (size_t)a.batch * a.Dn * N;
    const size_t col = (size_t)(ln.b * a.Dn + ln.d) * N;
    const float *hin_row = c == 0 ? a.h0 : a.sumH + (size_t)(c - 1) * M;
    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[ln.d * N + n] * kLog2e;
        h[n] = hin_row ? hin_row[col + n] : 0.0f;
    }
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> xs((const IO *)a.x + row0), dts((const IO *)a.dt + row0);
    const UniRow<IO, N> Bp(a.B, ln.b * a.L * N);
    const size_t row0c = (size_t)c * a.ck_rows;  // the chunk's first row of stored states
    stream_steps<IO, false, 4, false>(xs, dts, dts, voff, rb, steps, steps, [&](uint32_t i, float xv, float dv, float) {
        if (i % kPair == 0) {  // the chunk's incoming state too
            float *row = a.ckpt + (row0c + i / kPair) * M;
            if constexpr (N % 4 == 0) {
#pragma unroll
                for (int q = 0; q < N / 4; ++q) {
                    const f4v v = {h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
                    *(f4v *)(row + state_at<N>(ln.b, ln.d, q, a.Dn)) = v;
                }
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) row[state_at<N>(ln.b, ln.d, 0, a.Dn) + n] = h[n];
            }
        }
        const int64_t t = t0 + i;
        const float u = dv * xv;
#pragma unroll
        for (int n = 0; n < N; ++n)
            h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], u * Bp.ld(t * N + n));
    });
}

// ---------------------------------------------------------------- gradients
template <typename IO, int N, bool GATED>
__global__ __launch_bounds__(256) void k_bwd_chunk(BwdArgs a) {
    constexpr int V = 2 * N;
    const Lane ln = lane_of(a);
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t steps = (uint32_t)(min(a.L, t0 + a.T) - t0);
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const size_t M = (size_t)a.batch * a.Dn * N;
    const size_t col = (size_t)(ln.b * a.Dn + ln.d) * N;
    // the lane's stored states (< 2 GiB per row: checked on the host)
    const uint32_t st_voff = (uint32_t)(state_at<N>(ln.b, ln.d, 0, a.Dn) * sizeof(float));
    const uint32_t st_qstride = (uint32_t)(a.Dn * 16);
    float A2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        // padding lanes: no decay, so nothing of the clamped channel's A reaches them
        A2[n] = ln.valid ? a.A[ln.d * N + n] * kLog2e : 0.0f;
    }
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> xs((const IO *)a.x + row0), dts((const IO *)a.dt + row0),
        dys((const IO *)a.dy + row0), zs(GATED ? (const IO *)a.z + row0 : (const IO *)a.x + row0);
    const size_t row0c = (size_t)c * a.ck_rows;  // the chunk's first row of stored states
    // The states entering every second piece were stored by k_bwd_walk. The walk by
    // pieces goes backwards; each pair of pieces is staged in LDS during the pair after it.
    __shared__ uint32_t stage_mem[4 * Stage<N>::dwords];  // blocks have at most 4 waves
    SSM_LDS uint32_t *stg = (SSM_LDS uint32_t *)stage_mem + (threadIdx.x / 64) * Stage<N>::dwords;
    const int lane = threadIdx.x & 63;
    const bool pad_wave = __builtin_amdgcn_ballot_w64(!ln.valid) != 0;  // uniform
    const uint32_t nsub = (steps + kSub - 1) / kSub;
    if (nsub > 0) {
        const uint32_t pp = (nsub - 1) / 2;
        stage_sub<IO, N, GATED>(stg, xs, dts, dys, zs, voff, rb, pp * kPair, steps - pp * kPair,
                                a.ckpt + (row0c + pp) * M, st_voff, st_qstride, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    const int64_t mu_entry = (int64_t)a.n_chunks - 2 - c;  // adjoint entering from the right
    const float *mu = mu_entry < 0 ? (a.dh_final ? a.dh_final + col : nullptr)
                                   : a.revG + (size_t)mu_entry * M + col;
    float lam[N], dA[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        lam[n] = (mu && ln.valid) ? mu[n] : 0.0f;
        dA[n] = 0.0f;
    }
    float dD = 0.0f;
    const float Dd = a.D[ln.d];
    const RowStream<IO> dxs((IO *)a.dx + row0), ddts((IO *)a.ddt + row0),
        dzs((GATED && a.dz) ? (IO *)a.dz + row0 : (IO *)a.dx + row0);
    const bool want_dz = GATED && a.dz != nullptr;
    float *pbc = a.partBC + (size_t)ln.w * V;
    const size_t pbc_step = (size_t)a.waves * V;  // floats per (b, t) row of partials
    for (uint32_t k = nsub; k > 0;) {
        --k;
        set_priority(k + 1, nsub);
        const uint32_t j0 = k * kSub;
        const uint32_t ns = min((uint32_t)kSub, steps - j0);
        const int half = (int)(k & 1u);  // the piece's place in its staged pair
        // The staged rows and state (complete: the last wait on vmcnt came after their
        // loads were issued). Padding lanes stage their clamped channel's rows and
        // states, so they replace every staged value by 0: x = dt = dy = z = 0 and a zero
        // start state (and a zero adjoint, above) make every term of theirs exactly 0,
        // whatever the staged bits hold, and the channel sums need no mask. Their own
        // outputs are not stored. The reads are unconditional and the replacement is
        // taken only by a wave that holds padding lanes (a uniform branch).
        float xv[kSub], dv[kSub], yv[kSub], zv[kSub], start[N];
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            const int row = half * kSub + j;
            xv[j] = RowStream<IO>::widen(stg[(0 * kPair + row) * 64 + lane]);
            dv[j] = RowStream<IO>::widen(stg[(1 * kPair + row) * 64 + lane]);
            yv[j] = RowStream<IO>::widen(stg[(2 * kPair + row) * 64 + lane]);
            zv[j] = GATED ? RowStream<IO>::widen(stg[(3 * kPair + row) * 64 + lane]) : 0.0f;
        }
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const f4v v = *(const SSM_LDS f4v *)(stg + kStageRows + q * 256 + lane * 4);
                start[4 * q] = v.x; start[4 * q + 1] = v.y; start[4 * q + 2] = v.z; start[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) start[n] = __uint_as_float(stg[kStageRows + n * 64 + lane]);
        }
        if (pad_wave) {
#pragma unroll
            for (int j = 0; j < kSub; ++j) {
                xv[j] = ln.valid ? xv[j] : 0.0f;
                dv[j] = ln.valid ? dv[j] : 0.0f;
                yv[j] = ln.valid ? yv[j] : 0.0f;
                zv[j] = ln.valid ? zv[j] : 0.0f;
            }
#pragma unroll
            for (int n = 0; n < N; ++n) start[n] = ln.valid ? start[n] : 0.0f;
        }
        if (half) {
            // The second piece of a pair starts where the first ends: walk the first
            // piece (whole, since a later one exists) from the pair's stored state.
            const UniRow<IO, N> Bw(a.B, (ln.b * a.L + t0 + j0 - kSub) * N);
#pragma unroll
            for (int j = 0; j < kSub; ++j) {
                float x0 = RowStream<IO>::widen(stg[(0 * kPair + j) * 64 + lane]);
                float d0 = RowStream<IO>::widen(stg[(1 * kPair + j) * 64 + lane]);
                if (pad_wave) {
                    x0 = ln.valid ? x0 : 0.0f;
                    d0 = ln.valid ? d0 : 0.0f;
                }
                const float u0 = d0 * x0;
#pragma unroll
                for (int n = 0; n < N; ++n)
                    start[n] = __builtin_fmaf(e2(d0 * A2[n]), start[n], u0 * Bw.ld(j * N + n));
            }
        } else if (k > 0) {
            // the pair's last reads are done: stage the pair before it
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            const uint32_t pp = k / 2 - 1;
            stage_sub<IO, N, GATED>(stg, xs, dts, dys, zs, voff, rb, pp * kPair, kPair,
                                    a.ckpt + (row0c + pp) * M, st_voff, st_qstride, lane);
        }
        // The sub-chunk's rows of B and C, and of the dB/dC partials, from bases set here
        // once: the per-step offsets are then constants.
        const int64_t e_sub = (ln.b * a.L + t0 + j0) * N;
        const UniRow<IO, N> Bk(a.B, e_sub), Ck(a.C, e_sub);
        float *pk = pbc + (size_t)(ln.b * a.L + t0 + j0) * pbc_step;
        float hs[kSub][N];
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            const int jr = j < (int)ns ? j : 0;
            const float u = dv[j] * xv[j];
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float prev = j == 0 ? start[n] : hs[j - 1][n];
                hs[j][n] = __builtin_fmaf(e2(dv[j] * A2[n]), prev, u * Bk.ld(jr * N + n));
            }
        }
#pragma unroll
        for (int j = kSub - 1; j >= 0; --j) {
            if (j >= (int)ns) continue;  // uniform: every lane of the block has the same ns
            // The next pair's staging loads were issued before any store still in flight
            // here but this step's: wait for them before its stores.
            if (j == 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);
            float acc = 0.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) acc = __builtin_fmaf(Ck.ld(j * N + n), hs[j][n], acc);
            const float o = __builtin_fmaf(Dd, xv[j], acc);
            float gp;
            const float dout = gate_grad<GATED>(yv[j], zv[j], gp);
            dD = __builtin_fmaf(dout, xv[j], dD);
            const float u = dv[j] * xv[j];
            float gx = 0.0f, gA = 0.0f;
            float vals[V];
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float bn = Bk.ld(j * N + n);
                const float lt = __builtin_fmaf(dout, Ck.ld(j * N + n), lam[n]);
                const float w = __builtin_fmaf(-u, bn, hs[j][n]);  // a_t h_{t-1}
                const float q = lt * w;
                vals[n] = lt * u;                // dB_t[n] term
                vals[N + n] = dout * hs[j][n];   // dC_t[n] term
                gx = __builtin_fmaf(lt, bn, gx);
                gA = __builtin_fmaf(A2[n], q, gA);
                dA[n] = __builtin_fmaf(dv[j], q, dA[n]);
                lam[n] = e2(dv[j] * A2[n]) * lt;
            }
            if (ln.valid) {
                const uint32_t r = (j0 + j) * rb;
                dxs.st(voff, r, __builtin_fmaf(dout, Dd, dv[j] * gx));
                ddts.st(voff, r, __builtin_fmaf(xv[j], gx, gA * kLn2));
                if (want_dz) dzs.st(voff, r, yv[j] * o * gp);
            }
            const float tot = wave_reduce_transpose<V>(vals);
            constexpr int sh = 6 - Log2<V>::v;
            if ((lane & ((1 << sh) - 1)) == 0)
                pk[(size_t)j * pbc_step + (lane >> sh)] = tot;
        }
    }
    if (ln.valid) {
        const size_t pa = ((size_t)c * a.batch + ln.b) * a.Dn + ln.d;
#pragma unroll
        for (int n = 0; n < N; ++n) a.partA[pa * N + n] = dA[n];
        a.partD[pa] = dD;
        if (c == 0 && a.dh0) {
#pragma unroll
            for (int n = 0; n < N; ++n) a.dh0[col + n] = lam[n];
        }
    }
}

// ---------------------------------------------------------------- reductions
// dA[d][n] and dD[d]: sums over chunks and batch rows, in that fixed order.
__global__ void k_bwd_reduce_AD(BwdArgs a, int N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over Dn * (N + 1)
    const int64_t DN = a.Dn * N;
    if (i >= DN + a.Dn) return;
    const int64_t rows = (int64_t)a.n_chunks * a.batch;
    float s = 0.0f;
    if (i < DN) {
        for (int64_t r = 0; r < rows; ++r) s += a.partA[r * DN + i];
        a.dA[i] = s;
    } else {
        const int64_t d = i - DN;
        for (int64_t r = 0; r < rows; ++r) s += a.partD[r * a.Dn + d];
        a.dD[d] = s;
    }
}

// dB[b][t][n] and dC[b][t][n]: sums over the channel waves. A thread sums 4 adjacent
// values (16-byte loads; 2N is a multiple of 4 for N >= 2) with four running sums over
// the waves w = 0, 1, 2, 3 mod 4, added as (s0 + s1) + (s2 + s3): a fixed order.
__global__ void k_bwd_reduce_BC(BwdArgs a, int N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over batch * L * 2N / 4
    const int64_t V = 2 * N, Q = V / 4;
    if (i >= a.batch * a.L * Q) return;
    const int64_t bt = i / Q, j = (i % Q) * 4;
    const float4 *p = (const float4 *)(a.partBC + bt * a.waves * V + j);
    const int64_t step = V / 4;  // float4s per wave
    float4 s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int w = 0;
    for (; w + 4 <= a.waves; w += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 v = p[(int64_t)(w + r) * step];
            s[r].x += v.x; s[r].y += v.y; s[r].z += v.z; s[r].w += v.w;
        }
    }
    for (int r = 0; w < a.waves; ++w, ++r) {
        const float4 v = p[(int64_t)w * step];
        s[r].x += v.x; s[r].y += v.y; s[r].z += v.z; s[r].w += v.w;
    }
    const float o[4] = {(s[0].x + s[1].x) + (s[2].x + s[3].x), (s[0].y + s[1].y) + (s[2].y + s[3].y),
                        (s[0].z + s[1].z) + (s[2].z + s[3].z), (s[0].w + s[1].w) + (s[2].w + s[3].w)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t jj = j + k;
        if (jj < N) a.dB[bt * N + jj] = o[k];
        else a.dC[bt * N + (jj - N)] = o[k];
    }
}

// The same for N = 1 (2 values per row), one value per thread.
__global__ void k_bwd_reduce_BC1(BwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over batch * L * 2
    if (i >= a.batch * a.L * 2) return;
    const int64_t bt = i / 2, j = i % 2;
    const float *p = a.partBC + bt * a.waves * 2 + j;
    float s = 0.0f;
    for (int w = 0; w < a.waves; ++w) s += p[(int64_t)w * 2];
    if (j == 0) a.dB[bt] = s;
    else a.dC[bt] = s;
}

template <typename IO, int N>
hipError_t launch_n(const BwdArgs &a, const ScanArgs &fwd, int io, bool gated, hipStream_t s) {
    // the states entering the chunks, for the walk (not needed with the forward's states)
    hipError_t e = a.saved ? hipSuccess : launch_summary_carry(fwd, io, N, s);
    if (e != hipSuccess) return e;
    const unsigned gx = (unsigned)(a.batch * a.dblocks);
    const dim3 blk(a.threads);
    if (a.n_chunks > 1) {
        if (gated) hipLaunchKernelGGL((k_bwd_summary<IO, N, true>), dim3(gx, a.n_chunks - 1), blk, 0, s, a);
        else hipLaunchKernelGGL((k_bwd_summary<IO, N, false>), dim3(gx, a.n_chunks - 1), blk, 0, s, a);
        ScanArgs r = fwd;
        r.sumP = a.revQ;
        r.sumH = a.revG;
        r.h0 = a.dh_final;
        e = launch_carry(r, N, s);
        if (e != hipSuccess) return e;
    }
    if (!a.saved) hipLaunchKernelGGL((k_bwd_walk<IO, N>), dim3(gx, a.n_chunks), blk, 0, s, a);
    if (gated) hipLaunchKernelGGL((k_bwd_chunk<IO, N, true>), dim3(gx, a.n_chunks), blk, 0, s, a);
    else hipLaunchKernelGGL((k_bwd_chunk<IO, N, false>), dim3(gx, a.n_chunks), blk, 0, s, a);
    const int64_t nad = a.Dn * (N + 1);
    hipLaunchKernelGGL(k_bwd_reduce_AD, dim3((unsigned)((nad + 255) / 256)), dim3(256), 0, s, a, N);
    if constexpr (N >= 2) {
        const int64_t nbc = a.batch * a.L * 2 * N / 4;
        hipLaunchKernelGGL(k_bwd_reduce_BC, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, s, a, N);
    } else {
        const int64_t nbc = a.batch * a.L * 2;
        hipLaunchKernelGGL(k_bwd_reduce_BC1, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const BwdArgs &a, const ScanArgs &fwd, int io, int d_state, bool gated,
                     hipStream_t s) {
    switch (d_state) {
        case 1: return launch_n<IO, 1>(a, fwd, io, gated, s);
        case 2: return launch_n<IO, 2>(a, fwd, io, gated, s);
        case 4: return launch_n<IO, 4>(a, fwd, io, gated, s);
        case 8: return launch_n<IO, 8>(a, fwd, io, gated, s);
        case 16: return launch_n<IO, 16>(a, fwd, io, gated, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs &a, const ScanArgs &fwd, int io, int d_state, bool gated,
                           hipStream_t s) {
    return io == 0 ? launch_io<float>(a, fwd, io, d_state, gated, s)
                   : launch_io<bf16_bits>(a, fwd, io, d_state, gated, s);
}

}  // namespace ssm
