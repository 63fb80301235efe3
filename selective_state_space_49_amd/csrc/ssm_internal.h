// ssm_internal.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// One prefill call, already validated. Pointers are device pointers.
struct ScanArgs {
    const void *x, *dt, *B, *C, *z;
    const float *A, *D, *h0;
    void *y;
    float *h_final;
    float *sumP;   // workspace: per-chunk decay over the chunk   [n_chunks-1][batch][Dn][N](x2 if complex)
    float *sumH;   // workspace: per-chunk end state from zero; the carry scan overwrites
                   // entry c with the state entering chunk c+1
    int64_t batch, L, Dn;
    int64_t T;         // steps per chunk
    int32_t n_chunks;  // ceil(L / T), >= 1
    int32_t dblocks;   // channel blocks per batch row (grid x = batch * dblocks)
    int32_t threads;   // threads per block (multiple of 64, <= 256)
    // Input stage (fused entry point only; conv_k = 0 and null pointers otherwise):
    // x is the convolution's input and dt the raw step before softplus.
    const float *conv_w;      // [Dn][conv_k], or null: x is used as is
    const float *conv_b;      // [Dn], or null: no bias
    const void *conv_state0;  // [batch][conv_k-1][Dn] of io, or null: zeros before step 0
    void *conv_state_out;     // [batch][conv_k-1][Dn] of io, or null
    const float *dt_bias;     // [Dn], or null
    int32_t conv_k;           // 0 (no convolution) or 1..4
    // Exponential-trapezoidal entry point only: the input before step 0.
    const void *x_prev;       // [batch][Dn] of io, or null (then B_prev is null too)
    const void *B_prev;       // [batch][N] of io, or null
    const void *lam;          // [batch][L][Dn] of io: weight of each step's current input,
                              // or null (1/2)
    // MIMO entry point only: inputs and outputs per channel (x, z, y are [batch][L][Dn][rank],
    // B and C [batch][L][N][rank]); 1 elsewhere.
    int32_t rank;
    // Training forward only: the state entering every kStateEvery-th step, in the
    // stored-state layout (state_at); null elsewhere. Chunks start at multiples of
    // kStateEvery.
    float *states;
    // Fused training forward only: the scan's inputs u and dt as the input stage makes
    // them, rounded to io, [batch][L][Dn]; null elsewhere.
    void *u_out, *dt_out;
};

// The backward's stored states: row r (batch Dn N floats) holds the state entering step
// kStateEvery r. For N % 4 == 0 a row is laid out [batch][N / 4][Dn][4], so the q-th
// 16-byte piece of the 64 channels of a wave is one contiguous 1 KB run and a wave's
// 16-byte stores and loads cover whole cache lines; otherwise [batch][Dn][N]. state_at
// gives the float index in a row of piece q (the first of its 4 states) of channel d.
constexpr int kStateEvery = 8;
template <int N>
__host__ __device__ inline size_t state_at(int64_t b, int64_t d, int q, int64_t Dn) {
    return N % 4 == 0 ? ((size_t)(b * (N / 4) + q) * Dn + d) * 4 : (size_t)(b * Dn + d) * N;
}

struct StepArgs {
    float *h;
    const void *x, *dt, *B, *C, *z;
    const float *A, *D;
    void *y;
    int64_t n_layers, n_seq, Dn;
    // Input stage (fused entry point only), as in ScanArgs with a leading layer index:
    const float *conv_w;  // [n_layers][Dn][conv_k], or null
    const float *conv_b;  // [n_layers][Dn], or null
    void *conv_state;     // [n_layers][n_seq][conv_k-1][Dn] of io, read and written
    const float *dt_bias; // [n_layers][Dn], or null
    int32_t conv_k;       // 0 or 1..4
    // Exponential-trapezoidal entry point only: the previous token's x and B.
    const void *x_prev;   // [n_layers][n_seq][Dn] of io, or null (then B_prev is null too)
    const void *B_prev;   // [n_layers][n_seq][N] of io, or null
    const void *lam;      // [n_layers][n_seq][Dn] of io: the token's weight, or null (1/2)
    // MIMO entry point only: rank (x, z, y are [n_layers][n_seq][Dn][rank], B and C
    // [n_layers][n_seq][N][rank]); 1 elsewhere.
    int32_t rank;
};

// Real diagonal state. io: 0 = f32, 1 = bf16. Returns hipSuccess or the launch error.
// ev: NULL, or 4 events recorded on s before the summary kernel, after it, after the
// carry kernel and after the rescan kernel (phases that do not run leave two
// consecutive records).
hipError_t launch_scan_save(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev);
hipError_t launch_scan_real(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev);
// The same with the exponential-trapezoidal discretisation (x_prev, B_prev, lam of a).
hipError_t launch_scan_trap(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev);
// The same with MIMO projections of rank a.rank (1, 2, 4 or 8).
hipError_t launch_scan_mimo(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev);
hipError_t launch_scan_complex(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                               hipEvent_t const *ev);
hipError_t launch_state_fill(float *dst, const float *src, int64_t count, hipStream_t s);
// Real state with the input stage: conv (a.conv_k in 0..4) and softplus on dt.
hipError_t launch_scan_fused(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                             hipEvent_t const *ev);
// The first two phases of the real prefill only (chunk summaries, carry scan): on
// return a.sumH[c] holds the state entering chunk c+1. Nothing when n_chunks == 1.
hipError_t launch_summary_carry(const ScanArgs &a, int io, int d_state, hipStream_t s);
// The carry scan alone over a.sumP / a.sumH seeded with a.h0 (a.n_chunks - 1 entries).
hipError_t launch_carry(const ScanArgs &a, int d_state, hipStream_t s);
// dst[i] = src ? src[i] : 0 for count elements of elem_bytes (2 or 4) bytes each.
hipError_t launch_elem_fill(void *dst, const void *src, int64_t count, int elem_bytes,
                            hipStream_t s);
// The device address and size of the current device's scratch array (scratch.hip),
// looked up once per device. Allocates nothing.
hipError_t scratch_buffer(void **ptr, size_t *bytes);

hipError_t launch_step_real(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                            hipStream_t s);
hipError_t launch_step_complex(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                               hipStream_t s);
hipError_t launch_step_fused(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                             hipStream_t s);
// MIMO decode of rank a.rank (1, 2, 4 or 8).
hipError_t launch_step_mimo(const StepArgs &a, int io, int d_state, bool gated, hipStream_t s);
// Exponential-trapezoidal decode (x_prev, B_prev, lam of a).
hipError_t launch_step_trap(const StepArgs &a, int io, int d_state, bool gated, bool replay,
                            hipStream_t s);

// ---------------------------------------------------------------- backward
// One backward call, already validated and planned. The forward phases use a ScanArgs
// built from the same pointers.
struct BwdArgs {
    const void *x, *dt, *B, *C, *z, *dy;
    const float *A, *D, *h0, *dh_final;
    void *dx, *ddt, *dz;          // [batch][L][Dn] of io (dz only when z is given)
    float *dA, *dB, *dC, *dD, *dh0;
    // workspace
    float *sumH;    // forward carry: entry c = state entering chunk c+1   [n_chunks-1][batch][Dn][N]
    float *revQ;    // reverse summaries, reversed chunk order: entry j is chunk n_chunks-1-j
    float *revG;    //   (decay over the chunk, adjoint passed left from a zero carry-in); after
                    //   the reverse carry revG[j] = adjoint entering chunk n_chunks-2-j from the right
    float *ckpt;    // states every kStateEvery = 2 kSub steps, [n_chunks][ck_rows] rows of
                    // batch Dn N floats (state_at); with saved, the training forward's
    float *partA;   // per-chunk dA              [n_chunks][batch][Dn][N]
    float *partD;   // per-chunk dD              [n_chunks][batch][Dn]
    float *partBC;  // per-wave dB, dC           [batch][L][waves][2N]
    int64_t batch, L, Dn;
    int64_t T;
    int32_t n_chunks, dblocks, threads, waves;  // waves = channel waves per batch row
    int64_t ck_rows;  // stored-state rows per chunk: ceil(min(T, L) / kStateEvery)
    bool saved;       // ckpt holds the training forward's states: no walk
};
constexpr int kSub = 4;  // steps per recomputed sub-chunk of the backward
hipError_t launch_scan_bwd(const BwdArgs &a, const ScanArgs &fwd, int io, int d_state, bool gated,
                           hipStream_t s);

// ---------------------------------------------------------------- input-stage backward
// The backward through the fused prefill's input stage (ssm_scan_bwd_fused). Arrays of
// [batch][L][Dn] are of io unless noted; chunks of T steps (n_chunks of them) are
// independent.
struct InBwdArgs {
    const void *x_in, *dt_raw;              // the fused prefill's inputs
    const float *conv_w, *conv_b, *dt_bias; // [Dn][conv_k], [Dn], [Dn] (conv_b, dt_bias nullable)
    const void *conv_state0;                // [batch][conv_k-1][Dn], or null: zeros
    void *u, *dt;                           // written by launch_input_fwd: silu(conv(x_in)), softplus
    const void *du, *ddt;                   // the scan's backward on (u, dt): dLoss/du, dLoss/ddt
    void *dx_in, *ddt_raw;                  // outputs
    void *dconv_state0;                     // [batch][conv_k-1][Dn], or null: not wanted
    float *part;                            // workspace: [n_chunks][batch][Dn][conv_k + 2] fp32
    float *dconv_w, *dconv_b, *ddt_bias;    // outputs, fp32 (null: not wanted)
    int64_t batch, L, Dn, T;
    int32_t n_chunks, conv_k;               // conv_k 0..4 (0: u = x_in)
};
// u and dt from x_in and dt_raw. io: 0 = f32, 1 = bf16.
hipError_t launch_input_fwd(const InBwdArgs &a, int io, hipStream_t s);
// dx_in, ddt_raw, the partials and their sums (dconv_w, dconv_b, ddt_bias), dconv_state0.
hipError_t launch_input_bwd(const InBwdArgs &a, int io, hipStream_t s);

}  // namespace ssm
