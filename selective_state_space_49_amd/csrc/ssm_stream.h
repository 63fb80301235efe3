// ssm_stream.h -- walking [rows][Dn] arrays row by row in the prefill kernels.
//
// Each stream (x, dt, z, y) is addressed through a buffer resource based at the
// first row of the chunk: the lane's byte offset sits in a VGPR for the whole
// kernel and the row's byte offset is a wave-uniform SGPR, so a load or store is
// one buffer instruction with no vector address arithmetic. A chunk spans less
// than 2 GiB of any stream (the planner guarantees it), so 32-bit offsets suffice.
// The resource's record count is the maximum; the kernels keep every access in
// bounds by construction.
#pragma once

#include <type_traits>

#include "ssm_device.h"

namespace ssm {

// Word 3 of a gfx9-family buffer resource (raw byte addressing, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

template <typename IO> struct RowStream;

template <> struct RowStream<bf16_bits> {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit RowStream(const void *base)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, kRsrcWord3)) {}
    __device__ __forceinline__ float ld(uint32_t voff, uint32_t soff) const {
        return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
    }
    // The element's raw bits, to be widened later with widen().
    __device__ __forceinline__ uint32_t ldraw(uint32_t voff, uint32_t soff) const {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
    }
    static __device__ __forceinline__ float widen(uint32_t raw) { return bf16_to_f32(raw); }
    __device__ __forceinline__ void st(uint32_t voff, uint32_t soff, float v) const {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, voff, soff, 0);
    }
    // A streaming store (glc slc): for rows read back only long after.
    __device__ __forceinline__ void st_stream(uint32_t voff, uint32_t soff, float v) const {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, voff, soff, 3);
    }
};

template <> struct RowStream<float> {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit RowStream(const void *base)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, kRsrcWord3)) {}
    __device__ __forceinline__ float ld(uint32_t voff, uint32_t soff) const {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
    __device__ __forceinline__ uint32_t ldraw(uint32_t voff, uint32_t soff) const {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw); }
    __device__ __forceinline__ void st(uint32_t voff, uint32_t soff, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
    }
    __device__ __forceinline__ void st_stream(uint32_t voff, uint32_t soff, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 3);
    }
};

// Steps are visited in blocks of KU. The x, dt (and z) values of the next block are
// loaded into registers while the current block is computed (ping-pong buffers), so
// the HBM latency of one block hides behind the arithmetic of the previous one. A
// scheduling barrier between steps keeps each step's scalar B/C loads next to their
// use instead of hoisting a whole block's worth of them into SGPRs. KU is 4 for the
// real state and 2 for the complex state, whose larger state would otherwise push
// the kernel past 128 VGPRs (below four waves per SIMD).
//
// RAW: the buffers hold the bits as loaded (a bf16 value zero-extended in its dword) and
// the values are widened in the step that uses them. Widening at load time makes the
// compiler wait for the loads right after issuing them, which leaves the prefetch
// nothing to overlap (256k rescan 5.90-6.03 -> 5.84 ms, complex 1.08 -> 1.01 ms). It
// keeps each raw value live until its step, though, and the kernels with the most
// registers in use (the exponential-trapezoidal and input-stage rescans) then spill
// (6.9 -> 19.7 ms): they widen at load time (RAW = false).
// W: a fourth stream (the exponential-trapezoidal weight) is streamed alongside.
template <int KU, bool RAW, bool W = false>
struct StepIn {
    // raw bits (RAW), else the widened values
    typedef typename std::conditional<RAW, uint32_t, float>::type T;
    T x[KU], dt[KU], z[KU];
    T w[W ? KU : 1];
};

// Issue priority by remaining work. The SIMD arbiter favours the oldest of the waves
// that share a SIMD, so waves that start together with equal work finish one after
// another, and the last one runs alone at the end of the kernel. Lowering a wave's
// priority (s_setprio, 3 = highest) as its remaining steps fall below fractions of a
// scale lets the lagging waves catch up, so the waves of a SIMD finish close
// together. scale = the wave's own step count gives thresholds at 24/64, 44/64 and
// 58/64 of the work done (measured best on the 256k prefill: rescan 7.31 -> 6.33 ms);
// a fixed scale makes waves with more remaining work go first.
__device__ __forceinline__ void set_priority(uint32_t remaining, uint32_t scale) {
    const uint64_t r = (uint64_t)remaining * 64u, sc = scale;
    if (r > sc * 40u) __builtin_amdgcn_s_setprio(3);
    else if (r > sc * 20u) __builtin_amdgcn_s_setprio(2);
    else if (r > sc * 6u) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

template <typename IO, bool GATED, int KU, bool RAW, bool W>
__device__ __forceinline__ void load_block(StepIn<KU, RAW, W> &s, const RowStream<IO> &x,
                                           const RowStream<IO> &dt, const RowStream<IO> &z,
                                           const RowStream<IO> &w, uint32_t voff, uint32_t row,
                                           uint32_t rb) {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
        if constexpr (RAW) {
            s.x[k] = x.ldraw(voff, (row + k) * rb);
            s.dt[k] = dt.ldraw(voff, (row + k) * rb);
            if (GATED) s.z[k] = z.ldraw(voff, (row + k) * rb);
            if constexpr (W) s.w[k] = w.ldraw(voff, (row + k) * rb);
        } else {
            s.x[k] = x.ld(voff, (row + k) * rb);
            s.dt[k] = dt.ld(voff, (row + k) * rb);
            if (GATED) s.z[k] = z.ld(voff, (row + k) * rb);
            if constexpr (W) s.w[k] = w.ld(voff, (row + k) * rb);
        }
    }
}

template <typename IO, bool RAW, typename T>
__device__ __forceinline__ float use_value(T v) {
    if constexpr (RAW) return RowStream<IO>::widen(v);
    else return v;
}

// Calls body(i, x_i, dt_i, z_i, w_i) for i = 0 .. steps-1 (rows of the streams; w_i is
// 0 unless W); voff is the lane's byte offset in a row and rb the bytes per row.
// prio_scale: see set_priority (0 = leave the priority alone).
template <typename IO, bool GATED, int KU, bool RAW, bool W, typename Body>
__device__ __forceinline__ void stream_steps_w(const RowStream<IO> &x, const RowStream<IO> &dt,
                                               const RowStream<IO> &z, const RowStream<IO> &w,
                                               uint32_t voff, uint32_t rb, uint32_t steps,
                                               uint32_t prio_scale, Body &&body) {
    const uint32_t full = steps / KU;
    uint32_t i = 0;
    StepIn<KU, RAW, W> bufA, bufB;
    if (full > 0) load_block<IO, GATED, KU, RAW, W>(bufA, x, dt, z, w, voff, 0, rb);
    for (uint32_t k = 0; k < full; k += 2) {
        if (prio_scale) set_priority(steps - i, prio_scale);
        // block k is in bufA: fetch block k+1 into bufB, then compute block k
        if (k + 1 < full) load_block<IO, GATED, KU, RAW, W>(bufB, x, dt, z, w, voff, i + KU, rb);
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            body(i + j, use_value<IO, RAW>(bufA.x[j]), use_value<IO, RAW>(bufA.dt[j]),
                 GATED ? use_value<IO, RAW>(bufA.z[j]) : 0.0f,
                 W ? use_value<IO, RAW>(bufA.w[W ? j : 0]) : 0.0f);
        }
        i += KU;
        if (k + 1 >= full) break;
        // block k+1 is in bufB: fetch block k+2 into bufA, then compute block k+1
        if (k + 2 < full) load_block<IO, GATED, KU, RAW, W>(bufA, x, dt, z, w, voff, i + KU, rb);
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            body(i + j, use_value<IO, RAW>(bufB.x[j]), use_value<IO, RAW>(bufB.dt[j]),
                 GATED ? use_value<IO, RAW>(bufB.z[j]) : 0.0f,
                 W ? use_value<IO, RAW>(bufB.w[W ? j : 0]) : 0.0f);
        }
        i += KU;
    }
    if (prio_scale) __builtin_amdgcn_s_setprio(0);
    for (; i < steps; ++i) {  // ragged tail, one step at a time
        const float xv = x.ld(voff, i * rb), dv = dt.ld(voff, i * rb);
        const float zv = GATED ? z.ld(voff, i * rb) : 0.0f;
        const float wv = W ? w.ld(voff, i * rb) : 0.0f;
        body(i, xv, dv, zv, wv);
    }
}

// The same over x, dt (and z) only: body(i, x_i, dt_i, z_i).
template <typename IO, bool GATED, int KU, bool RAW = true, typename Body>
__device__ __forceinline__ void stream_steps(const RowStream<IO> &x, const RowStream<IO> &dt,
                                             const RowStream<IO> &z, uint32_t voff, uint32_t rb,
                                             uint32_t steps, uint32_t prio_scale, Body &&body) {
    stream_steps_w<IO, GATED, KU, RAW, false>(
        x, dt, z, z, voff, rb, steps, prio_scale,
        [&](uint32_t i, float xv, float dv, float zv, float) { body(i, xv, dv, zv); });
}

// ---------------------------------------------------------------- decay horizon
// The end state of a chunk from a zero start is sum_s W_s[n] dt_s x_s B_s[n] with
// W_s[n] = exp(A[n] * sum of dt after s). With dt >= 0 and Re A < 0 the weights only
// shrink going back in time. Once log2(e) * Re A[n] * (sum of dt over the last rows)
// <= -H for every state of every lane of a wave, everything older enters the end state
// with weight below 2^-H. The chunk's total transfer factor exp(A * sum dt) is then
// below 2^-H in modulus and is dropped the same way. Dropping both changes a carried
// state by at most 2^-H * (T * max|dt x B| + |incoming state|). H = 28 + the bit length
// of the chunk length T makes that at most 2^-28 of the input scale (T + 1 <= 2^bits),
// 16 times below fp32 resolution (2^-24), for every chunk length: 41 for the 256k
// prefill's chunks of 6554 steps, 48 for chunks just below 2^20 steps.
__device__ __forceinline__ float horizon_bits(uint32_t T) {
    return (float)(28 + 32 - __clz(T));
}
// Priority scale of the summary windows (steps): longer windows go first.
constexpr uint32_t kSummaryPrioScale = 2048;
constexpr int kB = 32;  // rows per block of the backward walk

// First row (chunk-relative) of the window that covers the horizon, walking dt back
// from row T-1 in whole blocks of kB rows; the next block is loaded while the
// current one is summed, and every load of a block is issued before any is waited
// on. amax = max over the lane's states of log2(e) * Re A; dtf maps a loaded value to
// the step (the identity, or softplus when the kernel applies the input stage).
// Returns 0 (the whole chunk) when some lane does not reach the horizon within the
// whole blocks (A >= 0, dt = 0, NaN, or simply a short chunk).
struct Identity {
    __device__ __forceinline__ float operator()(float v) const { return v; }
};

template <typename IO, typename DtF = Identity>
__device__ __forceinline__ uint32_t horizon_start(const RowStream<IO> &dt, uint32_t voff,
                                                  uint32_t rb, uint32_t T, float amax,
                                                  DtF dtf = DtF()) {
    if (!__any(amax < 0.0f) || T < (uint32_t)kB) return 0;
    const float H = horizon_bits(T);
    float S = 0.0f;
    float cur[kB];
    uint32_t nxt[kB];
    uint32_t tb = T;
#pragma unroll
    for (int k = 0; k < kB; ++k) cur[k] = dt.ld(voff, (tb - 1 - k) * rb);
    while (true) {
        const uint32_t tn = tb - kB;  // rows [tn, tb) are in cur
        const bool more = tn >= (uint32_t)kB;
        if (more) {
#pragma unroll
            for (int k = 0; k < kB; ++k) nxt[k] = dt.ldraw(voff, (tn - 1 - k) * rb);
        }
        __builtin_amdgcn_sched_barrier(0);  // sum the current block while nxt is in flight
#pragma unroll
        for (int k = 0; k < kB; ++k) S += dtf(cur[k]);
        if (__all(amax * S <= -H)) return tn;
        if (!more) return 0;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kB; ++k) cur[k] = RowStream<IO>::widen(nxt[k]);
        tb = tn;
    }
}

}  // namespace ssm
