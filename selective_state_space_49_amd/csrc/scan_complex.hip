// scan_complex.hip -- prefill with a complex diagonal state (gfx950).
//
// The Mamba-3 item on complex-valued state updates of "Jamba — SSM-Transformer
// Híbrido" (ai-engineering.academy) equates a complex diagonal state with a
// data-dependent rotary embedding on the state. Per channel d and state n, with
// A = -a + i theta:
//     Abar_t = exp(dt_t A) = exp(-dt_t a) (cos(dt_t theta) + i sin(dt_t theta))
//     h_t    = Abar_t h_{t-1} + dt_t B_t x_t              (B_t complex)
//     y_t    = Re(sum_n C_t[n] h_t[n]) + D x_t, then the optional silu(z) gate.
// Work split: chunks + carry scan + rescan as in the real-state scan, but a channel's
// N complex states are spread over P = 4 adjacent lanes (K = N / P each; N < 4: one
// lane per state), so a wave covers 64 / P channels. Each state update costs ~19 issue
// slots (exp, sin, cos and 13 more), so P times the waves lets the plan cut the
// sequence into P times longer chunks at the same occupancy, and the chunk summaries
// then walk a smaller share of each chunk (their decay horizon is a few hundred steps).
// The channel's output is summed over its P lanes with DPP. B_t and C_t differ between
// the P lanes of a channel, so they cannot come through the scalar unit: each block of
// rows is loaded once per wave (one complex value per lane), widened to fp32 once, and
// staged in LDS, from where each lane reads its K values per step. The rotation angle
// is kept in revolutions (theta / 2 pi) so that the hardware sine/cosine (which take
// revolutions) get an exactly range-reduced argument from fract().
#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_stream.h"

#include <type_traits>

namespace ssm {
namespace {

#define SSM_LDS __attribute__((address_space(3)))
typedef float f2v __attribute__((ext_vector_type(2)));  // a complex value (re, im) in LDS

template <int N> struct CSplit {
    static constexpr int P = N >= 4 ? 4 : N;  // lanes per channel
    static constexpr int K = N / P;           // complex states per lane
    static constexpr int CPB = 256 / P;       // channels per block of 256 lanes
    static constexpr int KU = 4;              // steps per block of rows
    static constexpr int kWaves = 5;          // waves per SIMD the kernels are compiled for
};

// Lane (channel d, state group q) of a block of 256 lanes; a.dblocks blocks per batch
// row. Lanes past the last channel work on it too (the B/C staging needs every lane)
// and store nothing.
struct CLane {
    int64_t b, d;
    int q;
    bool valid;
};

template <int P, int CPB>
__device__ __forceinline__ CLane clane(const ScanArgs &a) {
    CLane r;
    r.b = (int64_t)blockIdx.x / a.dblocks;
    const int64_t d = ((int64_t)blockIdx.x % a.dblocks) * CPB + threadIdx.x / P;
    r.q = (int)(threadIdx.x % P);
    r.valid = d < a.Dn;
    r.d = r.valid ? d : a.Dn - 1;
    return r;
}

// Sum over the P lanes of a channel (adjacent lanes: quad permutations). Addition is
// commutative, so every lane of the group gets the same bits.
template <int P>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (P >= 2)
        v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
    if constexpr (P >= 4)
        v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
    return v;
}

// One block of KU rows of a [rows][N][2] array of complex values (B or C) staged in
// LDS as fp32 pairs, [KU][N]: lane l (l < KU N) loads value l of the block (4 bytes
// for bf16, 8 for fp32) one block ahead and writes it widened at the block's start.
template <typename IO, int N, int KU>
struct CStage {
    static constexpr int kVals = KU * N;
    static_assert(kVals <= 64, "one value per lane");
    typedef typename std::conditional<sizeof(IO) == 2, uint32_t, uint2>::type Raw;
    __amdgpu_buffer_rsrc_t r;  // the walk's first row on
    uint32_t voff;             // the lane's value, clamped into the block
    bool on;
    __device__ __forceinline__ void init(const IO *row0) {
        r = __builtin_amdgcn_make_buffer_rsrc(const_cast<IO *>(row0), 0, -1, kRsrcWord3);
        const uint32_t l = threadIdx.x & 63u;
        on = l < (uint32_t)kVals;
        voff = (on ? l : (uint32_t)kVals - 1) * 2u * (uint32_t)sizeof(IO);
    }
    __device__ __forceinline__ Raw load(uint32_t row) const {
        const uint32_t so = row * (uint32_t)(N * 2 * sizeof(IO));
        if constexpr (sizeof(IO) == 2) {
            return __builtin_amdgcn_raw_buffer_load_b32(r, voff, so, 0);
        } else {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, so, 0);
            return make_uint2(t[0], t[1]);
        }
    }
    __device__ __forceinline__ void put(SSM_LDS f2v *slot, const Raw &w) const {
        if (!on) return;
        f2v v;
        if constexpr (sizeof(IO) == 2) {
            v.x = __uint_as_float(w << 16);
            v.y = __uint_as_float(w & 0xffff0000u);
        } else {
            v.x = __uint_as_float(w.x);
            v.y = __uint_as_float(w.y);
        }
        slot[threadIdx.x & 63u] = v;
    }
};

// exp(dt * (are + i aim)) with are2 = are log2 e and arev = aim / 2 pi.
__device__ __forceinline__ void decay_rotation(float dv, float are2, float arev, float &pr,
                                               float &pi) {
    const float mag = e2(dv * are2);
    const float r = fract(dv * arev);
    pr = mag * cos_rev(r);
    pi = mag * sin_rev(r);
}

// Walks the rows [0, steps) of a chunk part in blocks of KU rows: x and dt (and z) one
// block ahead in registers (raw bits, widened at use), B (and C) rows one block ahead,
// staged in the wave's LDS slots at the block's start; body(i, x, dt, z, bslot, cslot)
// with bslot / cslot the step's row of the staged block (LDS), or null in the ragged
// tail, where the step reads its values from global memory (brow, crow: the walk's
// first rows).
template <typename IO, int N, bool GATED, bool WITH_C, typename Body>
__device__ __forceinline__ void csteps(const RowStream<IO> &xs, const RowStream<IO> &dts,
                                       const RowStream<IO> &zs, uint32_t voff, uint32_t rb,
                                       const CStage<IO, N, CSplit<N>::KU> &bst,
                                       const CStage<IO, N, CSplit<N>::KU> &cst,
                                       SSM_LDS f2v *bslot, SSM_LDS f2v *cslot, uint32_t steps,
                                       uint32_t prio_scale, Body &&body) {
    constexpr int KU = CSplit<N>::KU;
    typedef typename CStage<IO, N, KU>::Raw Raw;
    const uint32_t full = steps / KU;
    uint32_t i = 0;
    StepIn<KU, true> bufA, bufB;
    Raw bA{}, cA{}, bB{}, cB{};
    if (full > 0) {
        bA = bst.load(0);
        if constexpr (WITH_C) cA = cst.load(0);
        load_block<IO, GATED, KU, true, false>(bufA, xs, dts, zs, zs, voff, 0, rb);
    }
    for (uint32_t k = 0; k < full; k += 2) {
        if (prio_scale) set_priority(steps - i, prio_scale);
        // block k: its B/C rows into LDS, then fetch block k+1, then compute block k
        bst.put(bslot, bA);
        if constexpr (WITH_C) cst.put(cslot, cA);
        if (k + 1 < full) {
            bB = bst.load(i + KU);
            if constexpr (WITH_C) cB = cst.load(i + KU);
            load_block<IO, GATED, KU, true, false>(bufB, xs, dts, zs, zs, voff, i + KU, rb);
        }
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            body(i + j, RowStream<IO>::widen(bufA.x[j]), RowStream<IO>::widen(bufA.dt[j]),
                 GATED ? RowStream<IO>::widen(bufA.z[j]) : 0.0f, bslot + j * N, cslot + j * N);
        }
        i += KU;
        if (k + 1 >= full) break;
        bst.put(bslot, bB);
        if constexpr (WITH_C) cst.put(cslot, cB);
        if (k + 2 < full) {
            bA = bst.load(i + KU);
            if constexpr (WITH_C) cA = cst.load(i + KU);
            load_block<IO, GATED, KU, true, false>(bufA, xs, dts, zs, zs, voff, i + KU, rb);
        }
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            body(i + j, RowStream<IO>::widen(bufB.x[j]), RowStream<IO>::widen(bufB.dt[j]),
                 GATED ? RowStream<IO>::widen(bufB.z[j]) : 0.0f, bslot + j * N, cslot + j * N);
        }
        i += KU;
    }
    if (prio_scale) __builtin_amdgcn_s_setprio(0);
    for (; i < steps; ++i) {  // ragged tail, one step at a time
        const float xv = xs.ld(voff, i * rb), dv = dts.ld(voff, i * rb);
        const float zv = GATED ? zs.ld(voff, i * rb) : 0.0f;
        body(i, xv, dv, zv, (SSM_LDS f2v *)nullptr, (SSM_LDS f2v *)nullptr);
    }
}

// The lane's K complex values of a step's row: from the staged block, or (ragged tail)
// from global memory.
template <typename IO, int N, int K>
__device__ __forceinline__ void row_vals(const SSM_LDS f2v *slot, const IO *grow, int q,
                                         float (&re)[K], float (&im)[K]) {
    if (slot) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const f2v v = slot[q * K + k];
            re[k] = v.x;
            im[k] = v.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            re[k] = Io<IO>::ld(grow + (q * K + k) * 2 + 0);
            im[k] = Io<IO>::ld(grow + (q * K + k) * 2 + 1);
        }
    }
}

// Chunk summary as in the real-state scan. The rotation has modulus one, so only the
// real part of A decays and the decay horizon is computed from Re A (over the wave's
// lanes, each with its K states).
template <typename IO, int N>
__global__ __launch_bounds__(256, CSplit<N>::kWaves) void k_chunk_summary_c(ScanArgs a) {
    constexpr int P = CSplit<N>::P, K = CSplit<N>::K, KU = CSplit<N>::KU;
    const CLane ln = clane<P, CSplit<N>::CPB>(a);
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const int64_t Dn = a.Dn;
    float Ar2[K], Arev[K], hr[K], hi[K];
    float amax = -INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t n = ln.q * K + k;
        Ar2[k] = a.A[(ln.d * N + n) * 2 + 0] * kLog2e;
        Arev[k] = a.A[(ln.d * N + n) * 2 + 1] * kInv2Pi;
        amax = fmaxf(amax, Ar2[k]);
        hr[k] = 0.0f;
        hi[k] = 0.0f;
    }
    const int64_t row0 = (ln.b * a.L + t0) * Dn;
    const uint32_t T = (uint32_t)a.T;
    const uint32_t rb = (uint32_t)(Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const RowStream<IO> dts((const IO *)a.dt + row0);
    const uint32_t ts = horizon_start<IO>(dts, voff, rb, T, amax);
    const int64_t rw = row0 + (int64_t)ts * Dn;
    const RowStream<IO> xs((const IO *)a.x + rw), dws((const IO *)a.dt + rw);
    const IO *B0 = (const IO *)a.B + ((ln.b * a.L + t0 + ts) * N) * 2;  // the walk's first B row
    __shared__ __attribute__((aligned(16))) f2v stage_mem[4 * KU * N];
    SSM_LDS f2v *bslot = (SSM_LDS f2v *)stage_mem + (threadIdx.x / 64) * KU * N;
    CStage<IO, N, KU> bst;
    bst.init(B0);
    double S = 0.0;
    csteps<IO, N, false, false>(xs, dws, dws, voff, rb, bst, bst, bslot, bslot, T - ts, min(T, kSummaryPrioScale),
                                [&](uint32_t i, float xv, float dv, float, const SSM_LDS f2v *bs,
                                    const SSM_LDS f2v *) {
        const float u = dv * xv;
        S += (double)dv;
        float br[K], bi[K];
        row_vals<IO, N, K>(bs, B0 + (size_t)i * N * 2, ln.q, br, bi);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float pr, pi;
            decay_rotation(dv, Ar2[k], Arev[k], pr, pi);
            const float nr = __builtin_fmaf(pr, hr[k], __builtin_fmaf(-pi, hi[k], u * br[k]));
            const float ni = __builtin_fmaf(pr, hi[k], __builtin_fmaf(pi, hr[k], u * bi[k]));
            hr[k] = nr;
            hi[k] = ni;
        }
    });
    if (!ln.valid) return;
    const size_t o = (((size_t)c * a.batch + ln.b) * a.Dn + ln.d) * N * 2;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t n = ln.q * K + k;
        float pr = 0.0f, pi = 0.0f;
        if (ts == 0) {
            // total decay and rotation of the chunk: exp(S * A); the angle in double
            const double aim = (double)a.A[(ln.d * N + n) * 2 + 1];
            const double rev = aim * kInv2PiD * S;
            const float r = (float)(rev - floor(rev));
            const float mag = e2(Ar2[k] * (float)S);
            pr = mag * cos_rev(r);
            pi = mag * sin_rev(r);
        }
        a.sumP[o + 2 * n + 0] = pr;
        a.sumP[o + 2 * n + 1] = pi;
        a.sumH[o + 2 * n + 0] = hr[k];
        a.sumH[o + 2 * n + 1] = hi[k];
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

// With few chunks, one lane per complex state column walks the chunks in order (as
// k_carry_seq of the real-state scan does): carry = P_c carry + H_c.
constexpr int kCarrySeqMax = 64;
constexpr int kCarryBatch = 8;

__global__ __launch_bounds__(256) void k_carry_seq_c(ScanArgs a, int64_t M) {
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= M) return;
    const int nsum = a.n_chunks - 1;
    const float2 *P2 = (const float2 *)a.sumP;
    float2 *H2 = (float2 *)a.sumH;
    float2 carry = a.h0 ? ((const float2 *)a.h0)[col] : make_float2(0.0f, 0.0f);
    for (int c0 = 0; c0 < nsum; c0 += kCarryBatch) {
        float2 p[kCarryBatch], h[kCarryBatch];
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            if (c0 + k < nsum) {
                p[k] = P2[(size_t)(c0 + k) * M + col];
                h[k] = H2[(size_t)(c0 + k) * M + col];
            }
        }
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            if (c0 + k < nsum) {
                float2 n;
                n.x = __builtin_fmaf(p[k].x, carry.x, __builtin_fmaf(-p[k].y, carry.y, h[k].x));
                n.y = __builtin_fmaf(p[k].x, carry.y, __builtin_fmaf(p[k].y, carry.x, h[k].y));
                carry = n;
                H2[(size_t)(c0 + k) * M + col] = carry;
            }
        }
    }
}

// ---------------------------------------------------------------- rescan + epilogue
template <typename IO, int N, bool GATED>
__global__ __launch_bounds__(256, CSplit<N>::kWaves) void k_chunk_scan_c(ScanArgs a) {
    constexpr int P = CSplit<N>::P, K = CSplit<N>::K, KU = CSplit<N>::KU;
    const CLane ln = clane<P, CSplit<N>::CPB>(a);
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const int64_t t1 = min(a.L, t0 + a.T);
    const size_t col = (size_t)(ln.b * a.Dn + ln.d) * N * 2;
    const float *hin = c == 0 ? (a.h0 ? a.h0 + col : nullptr)
                              : a.sumH + (size_t)(c - 1) * a.batch * a.Dn * N * 2 + col;
    float Ar2[K], Arev[K], hr[K], hi[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t n = ln.q * K + k;
        Ar2[k] = a.A[(ln.d * N + n) * 2 + 0] * kLog2e;
        Arev[k] = a.A[(ln.d * N + n) * 2 + 1] * kInv2Pi;
        hr[k] = hin ? hin[2 * n + 0] : 0.0f;
        hi[k] = hin ? hin[2 * n + 1] : 0.0f;
    }
    const float Dd = a.D[ln.d];
    const uint32_t rb = (uint32_t)(a.Dn * sizeof(IO));
    const uint32_t voff = (uint32_t)ln.d * (uint32_t)sizeof(IO);
    const int64_t row0 = (ln.b * a.L + t0) * a.Dn;
    const RowStream<IO> xs((const IO *)a.x + row0), dts((const IO *)a.dt + row0),
        zs(GATED ? (const IO *)a.z + row0 : (const IO *)a.x + row0), ys((IO *)a.y + row0);
    const IO *B0 = (const IO *)a.B + ((ln.b * a.L + t0) * N) * 2;
    const IO *C0 = (const IO *)a.C + ((ln.b * a.L + t0) * N) * 2;
    __shared__ __attribute__((aligned(16))) f2v stage_mem[2 * 4 * KU * N];
    SSM_LDS f2v *bslot = (SSM_LDS f2v *)stage_mem + (threadIdx.x / 64) * 2 * KU * N;
    SSM_LDS f2v *cslot = bslot + KU * N;
    CStage<IO, N, KU> bst, cst;
    bst.init(B0);
    cst.init(C0);
    const bool store = ln.valid && ln.q == 0;
    csteps<IO, N, GATED, true>(xs, dts, zs, voff, rb, bst, cst, bslot, cslot, (uint32_t)(t1 - t0),
                               (uint32_t)(t1 - t0), [&](uint32_t i, float xv, float dv, float zv,
                                                        const SSM_LDS f2v *bs, const SSM_LDS f2v *cs) {
        const float u = dv * xv;
        float br[K], bi[K], cr[K], ci[K];
        row_vals<IO, N, K>(bs, B0 + (size_t)i * N * 2, ln.q, br, bi);
        row_vals<IO, N, K>(cs, C0 + (size_t)i * N * 2, ln.q, cr, ci);
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float pr, pi;
            decay_rotation(dv, Ar2[k], Arev[k], pr, pi);
            const float nr = __builtin_fmaf(pr, hr[k], __builtin_fmaf(-pi, hi[k], u * br[k]));
            const float ni = __builtin_fmaf(pr, hi[k], __builtin_fmaf(pi, hr[k], u * bi[k]));
            hr[k] = nr;
            hi[k] = ni;
            acc = __builtin_fmaf(cr[k], nr, acc);
            acc = __builtin_fmaf(-ci[k], ni, acc);
        }
        acc = group_sum<P>(acc);
        float yv = __builtin_fmaf(Dd, xv, acc);
        if (GATED) yv = yv * silu(zv);
        if (store) ys.st(voff, i * rb, yv);
    });
    if (c == a.n_chunks - 1 && a.h_final && ln.valid) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t n = ln.q * K + k;
            a.h_final[col + 2 * n + 0] = hr[k];
            a.h_final[col + 2 * n + 1] = hi[k];
        }
    }
}

inline void mark(hipEvent_t const *ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

template <typename IO, int N>
hipError_t launch_t(const ScanArgs &a0, bool gated, hipStream_t s, hipEvent_t const *ev) {
    // blocks of 256 lanes, CPB channels each
    ScanArgs a = a0;
    a.threads = 256;
    a.dblocks = (int32_t)((a.Dn + CSplit<N>::CPB - 1) / CSplit<N>::CPB);
    const dim3 blk(256);
    const unsigned gx = (unsigned)(a.batch * a.dblocks);
    mark(ev, 0, s);
    if (a.n_chunks > 1)
        hipLaunchKernelGGL((k_chunk_summary_c<IO, N>), dim3(gx, a.n_chunks - 1), blk, 0, s, a);
    mark(ev, 1, s);
    if (a.n_chunks > 1) {
        const int64_t M = a.batch * a.Dn * N;
        if (a.n_chunks - 1 <= kCarrySeqMax)
            hipLaunchKernelGGL(k_carry_seq_c, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, a, M);
        else
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
